/*
 * jfa.h -- C ABI of the jagged flash attention library for AMD MI355X (gfx950).
 *
 * Exact softmax attention, forward and backward, computed directly on packed
 * variable-length ("jagged") Q/K/V whose sequence boundaries come from an offsets
 * (cu_seqlens) array; no padding is materialised at any step.
 *
 * Sources (page title, section):
 *  - "Using TLX to optimise jagged flash attention on Blackwell GPUs" (explore.n1n.ai),
 *    section on the performance defects of padded tensors: the jagged layout (valid
 *    tokens back to back) and the offsets array, e.g. lengths [128,4096,512,2048]
 *    -> offsets [0,128,4224,4736,6784].
 *  - "Jagged Flash Attention on TLX" (aixai.ru), "What is Jagged Flash Attention":
 *    the attention runs on packed Q, K, V plus offsets; the broadcast-Q production
 *    mode shares one dense Q across the batch and sums its gradient dQ over all
 *    sequences.
 *  - "TLX Block Attention" (bittide page), section 1: fixed 64-token groups that
 *    attend only within themselves (block-diagonal mode); section 2.1, Listing 1: the
 *    online-softmax forward and the log-sum-exp L = m + log(l) kept for the backward;
 *    section 4: the backward with Di = rowsum(dO * O) computed inline; section 5:
 *    persistent programs and host-side (CPU offsets) scheduling with no GPU sync.
 *
 * Conventions for every entry point:
 *  - All tensors are caller-allocated device buffers, contiguous, 16-byte aligned.
 *    Element types: bf16 for q, k, v, o, dout, dq, dk, dv; fp32 for lse; int32 for
 *    offsets.  Token-major layout [tokens, H, D] (row stride H*D elements).
 *  - Shapes by mode (T = offsets[B], Mq = shape->num_q):
 *        mode            q          k, v       o, dout       lse         dq
 *        SELF            [T,H,D]    [T,H,D]    [T,H,D]       [H,T]       [T,H,D]
 *        BROADCAST_Q     [Mq,H,D]   [T,H,D]    [B,Mq,H,D]    [B,H,Mq]    [Mq,H,D]
 *        BLOCK_DIAG      [T,H,D]    [T,H,D]    [T,H,D]       [H,T]       [T,H,D]
 *    k, v carry Hkv = shape->num_kv_heads heads where the table says H (forward only,
 *    see jfa_shape).  dk, dv always have the shape of k, v.  lse is the natural-log
 *    log-sum-exp of the scaled scores of each query row; a broadcast-Q sequence of
 *    length 0 gets o = 0 and lse = -inf and contributes no gradient.
 *  - offsets_dev / offsets_host: int32 [B+1], offsets[0] = 0, non-decreasing,
 *    offsets[B] = shape->total_tokens.  offsets_host may be NULL: the library then
 *    copies the device offsets to the host and synchronises the stream (slow path).
 *    With host offsets the call performs no device synchronisation.
 *  - workspace: caller-allocated device scratch of at least jfa_workspace_size()
 *    bytes (256-byte aligned); its contents are overwritten.
 *  - stream: a hipStream_t (NULL = the default stream).  Calls are asynchronous;
 *    outputs are valid once the stream has reached them.  Host arrays are consumed
 *    before the call returns.
 *  - Return value: 0 on success or a negative JFA_ERR_* code.  Every argument check
 *    runs before any device work is queued; a failed check queues nothing.
 *    jfa_last_error_detail() returns a thread-local message about the last failure.
 *    No C++ exception crosses this interface.
 */
#ifndef JFA_H_
#define JFA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define JFA_VERSION 160 /* 1.6.0 */

enum jfa_mode {
  JFA_MODE_SELF = 0,        /* each packed sequence attends to itself */
  JFA_MODE_BROADCAST_Q = 1, /* one shared Q [Mq,H,D] attends to every sequence's K/V */
  JFA_MODE_BLOCK_DIAG = 2   /* 64-token groups of each sequence attend within themselves */
};

enum jfa_pass {
  JFA_PASS_FWD = 0,
  JFA_PASS_BWD = 1,
  JFA_PASS_FWD_SPARSE = 2, /* jfa_fwd_block_sparse (self mode only) */
  JFA_PASS_FWD_MXFP8 = 3,  /* jfa_fwd_mxfp8 and jfa_mxfp8_quantize_v (self mode only) */
  JFA_PASS_BWD_MXFP8 = 4   /* jfa_bwd_mxfp8 (self mode only) */
};

enum jfa_status {
  JFA_OK = 0,
  JFA_ERR_NULL_POINTER = -1,    /* a required pointer argument is NULL */
  JFA_ERR_BAD_SHAPE = -2,       /* B < 0, H < 1, total_tokens < 0, Mq < 1 in broadcast-Q,
                                   H % Hkv != 0, Hkv != H in jfa_bwd ... */
  JFA_ERR_BAD_HEAD_DIM = -3,    /* head_dim not in {64, 128} */
  JFA_ERR_BAD_MODE = -4,        /* mode not a jfa_mode, or pass not a jfa_pass */
  JFA_ERR_BAD_OFFSETS = -5,     /* offsets[0] != 0, decreasing, or offsets[B] != T */
  JFA_ERR_MISALIGNED = -6,      /* a tensor is not 16-byte aligned (workspace: 256) */
  JFA_ERR_WORKSPACE = -7,       /* workspace smaller than jfa_workspace_size() */
  JFA_ERR_BAD_OPTION = -8,      /* an option field out of range */
  JFA_ERR_TOO_LARGE = -9,       /* sizes beyond the 32-bit tile / element indexing */
  JFA_ERR_HIP = -10,            /* a HIP runtime call or kernel launch failed */
  JFA_ERR_CAPACITY = -11        /* jfa_schedule: an output array is too small */
};

/* Problem sizes. */
typedef struct jfa_shape {
  int32_t num_seqs;     /* B >= 0 */
  int32_t num_heads;    /* H >= 1 query heads (and output heads) */
  int32_t head_dim;     /* D in {64, 128} */
  int32_t num_q;        /* Mq >= 1, broadcast-Q only (ignored otherwise) */
  int64_t total_tokens; /* T = offsets[B] */
  int32_t num_kv_heads; /* Hkv: key/value heads; 0 means H.  Grouped-query attention
                           when Hkv < H: H % Hkv == 0 and query head h reads key/value
                           head h / (H / Hkv) ("Jagged Flash Attention on TLX"
                           (aixai.ru), list of supported features: GQA in the forward,
                           the backward only with one query group per key/value head).
                           k, v (and dk, dv) then have Hkv heads; jfa_bwd requires
                           Hkv == H. */
  int32_t reserved;     /* must be 0 */
} jfa_shape;

/* Tuning options; pass NULL for the defaults (all zero). */
typedef struct jfa_opts {
  int32_t sched;        /* 0: static host schedule (sorted zigzag / head-pinned round robin /
                           contiguous ranges); 1: same order, tiles taken at run time from
                           atomic counters: one per XCD (8 groups of consecutive programs,
                           each serving the tiles the static deal gives them) when the
                           program count is a multiple of 8, else one; one per head in the
                           broadcast-Q dK/dV kernel (block-diagonal mode is always static) */
  int32_t dq_path;      /* broadcast-Q backward only. 0: one fused kernel, dQ by fp32
                           atomics into one [Mq,H,D] accumulator; 1: the fused kernel with
                           per-program fp32 partial slabs [P,Mq,D] reduced by a second kernel
                           (run-to-run deterministic); 2 (fastest): the self-attention
                           backward's two kernels -- a dQ kernel over tiles of the shared
                           queries against one chunk of one sequence's keys (long sequences
                           cut into chunks so that no tile walks far more keys than a
                           program's fair share), each chunk's fp32 dQ in a slab
                           [chunks,Mq,H,D], and a dK/dV kernel over head-pinned key tiles --
                           then a two-level reduce of the slabs (run-to-run deterministic) */
  int32_t num_programs; /* persistent workgroups; 0 = one per resident slot on the device */
  int32_t ds_budget_mib; /* self-mode backward only: MiB of workspace the backward may use
                           to keep dS (bf16) in HBM, >= 0.  0: recompute path (a dQ kernel
                           rebuilds S and dP, seven matrix products per query-key block).
                           > 0: when jfa_ds_bytes() of the call's lengths fits the budget,
                           the dK/dV kernel stores dS and dQ = scale dS K is read back from
                           it (five products plus two bytes of HBM traffic each way per
                           pair); otherwise the recompute path runs.  Both paths give the
                           same result up to fp32 summation order. */
} jfa_opts;

/* Bytes of workspace jfa_fwd (pass 0) or jfa_bwd (pass 1) needs for this shape and
 * mode.  Depends on (B, H, D, Mq, T) and the options only (a self-mode backward adds
 * opts->ds_budget_mib MiB), never on the individual lengths.  Returns 0 or an error
 * code; *bytes is written on success. */
int jfa_workspace_size(const jfa_shape* shape, int mode, int pass, const jfa_opts* opts,
                       size_t* bytes);

/* Bytes of dS storage the self-mode backward's stored-dS path needs for these lengths:
 * sum over sequences of H * ceil(L/128)*128 * ceil(L/64)*64 * 2 (dS of every
 * (query, key) pair of each sequence and head in bf16, keys padded to 128 and queries
 * to 64).  A budget of at least ceil(bytes / 2^20) MiB selects that path.  Host only;
 * offsets_host is required.  Returns 0 or an error code. */
int jfa_ds_bytes(const jfa_shape* shape, const int32_t* offsets_host, size_t* bytes);

/* Forward: o = softmax(scale * q k^T) v per sequence (per 64-token block in
 * BLOCK_DIAG mode) and the per-row lse.  See the header comment for shapes. */
int jfa_fwd(const jfa_shape* shape, int mode, float scale,
            const void* q, const void* k, const void* v,
            const int32_t* offsets_dev, const int32_t* offsets_host,
            void* o, float* lse,
            void* workspace, size_t workspace_bytes,
            const jfa_opts* opts, void* stream);

/* Backward of the forward above for upstream gradient dout: dq, dk, dv (bf16,
 * accumulated in fp32).  P is recomputed from q, k and lse; Di = rowsum(dout * o) is
 * computed inline (in a small row-term kernel on the stored-dS path).  `scale` must
 * equal the forward's.  In BROADCAST_Q mode dq is the sum over all sequences. */
int jfa_bwd(const jfa_shape* shape, int mode, float scale,
            const void* q, const void* k, const void* v,
            const void* o, const void* dout, const float* lse,
            const int32_t* offsets_dev, const int32_t* offsets_host,
            void* dq, void* dk, void* dv,
            void* workspace, size_t workspace_bytes,
            const jfa_opts* opts, void* stream);

/* Block-sparse top-k self attention, forward ("Jagged Flash Attention on TLX"
 * (aixai.ru), closing section on variants: a cheap first stage averages blocks of Q
 * and K and keeps the most relevant ones for the attention kernel).  Stage 1 pools
 * every 256-row query block and every 64-key block of each (sequence, head) to the
 * mean of its rows and keeps, per query block, the k = max(1, ceil(ratio * nkb)) key
 * blocks (nkb = ceil(L/64); ratio * nkb formed in double from the float ratio) whose
 * mean has the largest dot product with the query block's mean, ties going to the
 * lower block index.  Stage 2 is the forward of jfa_fwd restricted to the kept blocks
 * (an exact softmax over their keys).  ratio in (0, 1]; ratio 1 keeps every block and
 * gives exactly jfa_fwd's result.  Self mode only; grouped key/value heads allowed.
 * A sequence may have at most 2048 key blocks (131072 tokens): JFA_ERR_TOO_LARGE
 * otherwise.
 *
 * selection: device int32 array of at least jfa_block_sparse_entries() entries; the
 * call writes the kept block indices, for sequence b, head h and query block i at
 * [base_b + (h * nqb_b + i) * k_b, ... + k_b) in ascending order, where nqb_b =
 * ceil(L_b/256), k_b the count above and base_b the sum of H * nqb * k over earlier
 * sequences.  workspace: jfa_workspace_size(shape, JFA_MODE_SELF,
 * JFA_PASS_FWD_SPARSE, opts) bytes.  Other conventions as jfa_fwd. */
int jfa_block_sparse_entries(const jfa_shape* shape, const int32_t* offsets_host, float ratio, int64_t* entries);
int jfa_fwd_block_sparse(const jfa_shape* shape, float scale, float ratio,
                         const void* q, const void* k, const void* v,
                         const int32_t* offsets_dev, const int32_t* offsets_host,
                         void* o, float* lse, int32_t* selection, int64_t selection_entries,
                         void* workspace, size_t workspace_bytes,
                         const jfa_opts* opts, void* stream);

/* MXFP8 self-attention forward ("Jagged Flash Attention on TLX" (aixai.ru), closing
 * section on variants: MXFP8 inputs with block scales, P quantised on the fly, the
 * same pipeline).  MXFP8 is the OCP Microscaling format: 32 elements share an E8M0
 * scale 2^X (byte X + 127) and each element is FP8 E4M3 (OCP E4M3FN byte).  The
 * quantisers follow the OCP rule: X = floor(log2 max|x|) - 8 (0 for an all-zero
 * block), elements x / 2^X rounded to nearest E4M3, ties to even, clamped to +-448.
 *  - jfa_mxfp8_quantize_qk: q or k [T, H, D] bf16 -> codes [T, H, D] (16-byte aligned)
 *    and scales [T, H, D/32], blocks of 32 consecutive elements along D.
 *  - jfa_mxfp8_v_tokens: Tp, the token count of the transposed V layout: every
 *    sequence padded to a multiple of 64 keys (sequence b starts at the sum of its
 *    predecessors' padded lengths).
 *  - jfa_mxfp8_quantize_v: v [T, H, D] bf16 -> codes [H][D][Tp] (V transposed per
 *    head; zero past each sequence's end) and scales [H][D][Tp/32], blocks of 32 keys
 *    of one sequence from its start.  tokens must equal jfa_mxfp8_v_tokens().
 *  - jfa_fwd_mxfp8: o [T, H, D] bf16 and lse [H, T] (natural log) of self attention over
 *    the dequantised inputs, S and the softmax statistics in fp32, P quantised per 32
 *    keys of a row with the smallest power-of-two scale that keeps the block maximum
 *    at most 448 before the P V product.  D in {64, 128}; one key/value head per query
 *    head (JFA_ERR_BAD_SHAPE otherwise); static schedule of tiles of 256 query rows
 *    (D = 128) or 128 (D = 64).  At D = 128 the kernel is a two-group ping-pong whose
 *    per-lane copy offsets are 32-bit; past D * Tp >= 2^32, or with JFA_MX_GENERIC set
 *    to a value other than "0" in the environment (read at every call; for tests), the
 *    one-group kernel of D = 64 runs at D = 128 instead, with the same results' bound.
 * workspace (quantize_v and the forward): jfa_workspace_size(shape, JFA_MODE_SELF,
 * JFA_PASS_FWD_MXFP8, opts) bytes.  Other conventions as jfa_fwd. */
int jfa_mxfp8_v_tokens(const jfa_shape* shape, const int32_t* offsets_host, int64_t* tokens);
int jfa_mxfp8_quantize_qk(const jfa_shape* shape, const void* x, uint8_t* codes, uint8_t* scales, void* stream);
int jfa_mxfp8_quantize_v(const jfa_shape* shape, const void* v, const int32_t* offsets_dev,
                         const int32_t* offsets_host, uint8_t* codes, uint8_t* scales, int64_t tokens,
                         void* workspace, size_t workspace_bytes, void* stream);
int jfa_fwd_mxfp8(const jfa_shape* shape, float scale,
                  const uint8_t* q8, const uint8_t* q_scales, const uint8_t* k8, const uint8_t* k_scales,
                  const uint8_t* v8t, const uint8_t* v_scales, int64_t v_tokens,
                  const int32_t* offsets_dev, const int32_t* offsets_host,
                  void* o, float* lse,
                  void* workspace, size_t workspace_bytes,
                  const jfa_opts* opts, void* stream);

/* Backward of the MXFP8 self-attention forward (same section of the aixai.ru page, which
 * reports the MXFP8 backward at parity with bf16 on dense shapes without saying which of
 * its products run in FP8).  The MXFP8 inputs (the layouts above) are decoded once into
 * bf16 -- exact: an E4M3 value times 2^X keeps its four significant bits in bf16 for
 * X >= -117 -- and the self-attention backward (jfa_bwd's kernels, P and dS in bf16)
 * runs on them.  o and lse: jfa_fwd_mxfp8's outputs; dout [T, H, D] bf16.  dq, dk, dv
 * [T, H, D] bf16: the gradient of attention with respect to the decoded q, k, v (the
 * quantisation itself passes gradients straight through).  opts as jfa_bwd (stored-dS
 * path when ds_budget_mib holds dS).  workspace: jfa_workspace_size(shape,
 * JFA_MODE_SELF, JFA_PASS_BWD_MXFP8, opts) bytes (the three decoded tensors plus
 * jfa_bwd's workspace).  Argument errors as jfa_bwd and jfa_fwd_mxfp8, reported before
 * any device work. */
int jfa_bwd_mxfp8(const jfa_shape* shape, float scale,
                  const uint8_t* q8, const uint8_t* q_scales, const uint8_t* k8, const uint8_t* k_scales,
                  const uint8_t* v8t, const uint8_t* v_scales, int64_t v_tokens,
                  const void* o, const void* dout, const float* lse,
                  const int32_t* offsets_dev, const int32_t* offsets_host,
                  void* dq, void* dk, void* dv,
                  void* workspace, size_t workspace_bytes,
                  const jfa_opts* opts, void* stream);

/* Block-diagonal attention with a rotary position embedding fused in ("TLX Block
 * Attention" (bittide page), opening summary: the rotary embedding fused into the
 * attention kernel, attention plus rotary backward about 3.5x the unfused baseline).
 * The pages give no formula; this is RoFormer's rotation (Su et al.) in the
 * rotate-half pairing: for a token at position p inside its own sequence (0 .. L-1)
 * and i < D/2, the pair (x_i, x_{i+D/2}) of q and of k becomes
 * (x_i cos - x_{i+D/2} sin, x_{i+D/2} cos + x_i sin) with (cos, sin) =
 * rope_cos_sin[(p * D/2 + i) * 2 + {0, 1}] (fp32 device array, 16-byte aligned,
 * caller-owned; usually cos and sin of p * base^(-2i/D)).  The forward returns
 * attention(rope(q), rope(k), v) with lse; the backward returns the gradients with
 * respect to the un-rotated q and k (the rotation's transpose applied to dQ and dK in
 * the kernel) and v.  mode must be JFA_MODE_BLOCK_DIAG (JFA_ERR_BAD_MODE otherwise);
 * rope_positions (rows of the table) must be at least the longest sequence
 * (JFA_ERR_BAD_SHAPE).  Workspace and all other conventions as jfa_fwd / jfa_bwd. */
int jfa_fwd_rotary(const jfa_shape* shape, int mode, float scale,
                   const void* q, const void* k, const void* v,
                   const float* rope_cos_sin, int32_t rope_positions,
                   const int32_t* offsets_dev, const int32_t* offsets_host,
                   void* o, float* lse,
                   void* workspace, size_t workspace_bytes,
                   const jfa_opts* opts, void* stream);
int jfa_bwd_rotary(const jfa_shape* shape, int mode, float scale,
                   const void* q, const void* k, const void* v,
                   const void* o, const void* dout, const float* lse,
                   const float* rope_cos_sin, int32_t rope_positions,
                   const int32_t* offsets_dev, const int32_t* offsets_host,
                   void* dq, void* dk, void* dv,
                   void* workspace, size_t workspace_bytes,
                   const jfa_opts* opts, void* stream);

/* The cos / sin table jfa_fwd_rotary and jfa_bwd_rotary take, built on the device:
 * table[(p * D/2 + i) * 2 + {0, 1}] = cos, sin of p * base^(-2i/D) for p < positions,
 * i < D/2 (RoFormer's frequencies, usually base = 10000), formed in double precision
 * and rounded once to fp32.  table: caller-allocated fp32 device array of
 * positions * head_dim entries, 16-byte aligned; head_dim in {64, 128}; base > 1.
 * Asynchronous on stream like the other calls. */
int jfa_rope_table(float* table, int32_t positions, int32_t head_dim, float base, void* stream);

/* Block-sparse top-k self attention, backward: the gradient of sum(O * dout) for the
 * forward of jfa_fwd_block_sparse with its selection held fixed (the pooling and top-k
 * only choose which keys take part and carry no gradient): per (sequence, head, query
 * block) the exact-attention gradient over the kept keys, dK and dV summed over the
 * query blocks that kept them ("Jagged Flash Attention on TLX" (aixai.ru), closing
 * section on variants, names the variant for the forward; this is the plain reading of
 * its backward).  selection / selection_entries / ratio: exactly what the forward call
 * took and wrote (selection is read only; an entry outside [0, nkb) gives wrong
 * results but no access outside the sequence).  o, lse: that forward's outputs.
 * Recompute path (opts.ds_budget_mib is ignored).  H == Hkv required.  workspace:
 * jfa_bwd_block_sparse_workspace_size() bytes for these offsets (the recompute
 * backward's workspace plus a bitmap of ceil(L/128) * 2 * ceil(ceil(L/256)/32) words
 * per sequence and head).  dq, dk, dv: [T, H, D] bf16, fully written (keys no query
 * block kept get dK = dV = 0).  Other conventions as jfa_bwd. */
int jfa_bwd_block_sparse_workspace_size(const jfa_shape* shape, const int32_t* offsets_host,
                                        const jfa_opts* opts, size_t* bytes);
int jfa_bwd_block_sparse(const jfa_shape* shape, float scale, float ratio,
                         const void* q, const void* k, const void* v,
                         const void* o, const void* dout, const float* lse,
                         const int32_t* offsets_dev, const int32_t* offsets_host,
                         const int32_t* selection, int64_t selection_entries,
                         void* dq, void* dk, void* dv,
                         void* workspace, size_t workspace_bytes,
                         const jfa_opts* opts, void* stream);

/* Allocation-free forward, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, kernels and results as jfa_fwd without the workspace: the workspace is a
 * file-scope device array of JFA_NOALLOC_SCRATCH_BYTES that the library holds on every
 * GPU it runs on until the process ends (its address is looked up once per device, on
 * the first call there).  The call allocates no device or pinned host memory (no
 * hipMalloc, hipHostMalloc or hipFree; the host-side schedule is built in ordinary
 * heap memory and goes up by a pageable-memory copy, which the runtime has taken when
 * the call returns) and does not use the kernel timing hook.  Shapes whose jfa_fwd
 * workspace (jfa_workspace_size, pass JFA_PASS_FWD) exceeds the array return
 * JFA_ERR_TOO_LARGE before any device work.  Every call on one GPU shares that GPU's
 * array and each call overwrites it (counters included), so calls that overlap on one
 * GPU (other streams, other host threads) race: serialise them. */
#define JFA_NOALLOC_SCRATCH_BYTES (4u << 20)
int jfa_fwd_noalloc(const jfa_shape* shape, int mode, float scale,
                    const void* q, const void* k, const void* v,
                    const int32_t* offsets_dev, const int32_t* offsets_host,
                    void* o, float* lse, const jfa_opts* opts, void* stream);

/* Host-only view of the tile schedule the calls above would run (no device needed).
 * Tiles are (b, h, blk) triples: forward tiles are tile_rows query rows, backward
 * tiles tile_rows key rows, block-diagonal tiles one 64-token block.  Static
 * schedules list tiles program by program with one segment per program
 * (seg_ptr[P+1]); dynamic schedules list each counter group's tiles in sorted order,
 * one segment per group.  tiles (3*cap int32) and seg_ptr (seg_cap int32) may be NULL to
 * query the counts only; JFA_ERR_CAPACITY if an array is too small.
 *
 * Diagnostics: with JFA_LOG set to a value other than "0" in the environment (read once
 * per process), every schedule the library builds, here or inside the calls above,
 * prints one line on stderr: its tile and program counts, its segments (programs of a
 * static schedule, counter groups of a dynamic one), the summed tile cost (a tile costs
 * its sequence's or key chunk's length where tiles differ in cost, 1 where they cost the
 * same) and the largest segment cost against the mean. */
int jfa_schedule(const jfa_shape* shape, int mode, int pass, const int32_t* offsets_host,
                 const jfa_opts* opts, int32_t* tiles, int64_t cap, int32_t* seg_ptr,
                 int64_t seg_cap, int64_t* n_tiles, int32_t* n_segs, int32_t* n_programs,
                 int32_t* tile_rows);

/* Attention kernels timed by the measurement hook below. */
enum jfa_kernel {
  JFA_KERNEL_FWD = 0,    /* the forward attention kernel of jfa_fwd (and jfa_fwd_block_sparse) */
  JFA_KERNEL_BWD = 1,    /* the main backward kernel of jfa_bwd: the dK/dV kernel in self
                            mode, in broadcast-Q mode with dq_path 2 (and in
                            jfa_bwd_block_sparse), the fused kernel in broadcast-Q mode with
                            dq_path 0 or 1 and in block-diagonal mode */
  JFA_KERNEL_BWD_DQ = 2,  /* the dQ kernel of jfa_bwd in self mode (recompute or stored-dS) and
                             in broadcast-Q mode with dq_path 2, and of jfa_bwd_block_sparse */
  JFA_KERNEL_BWD_PREP = 3,    /* self mode: the row-term kernel (Di, lse) of the stored-dS
                                 path and of the side-by-side recompute path;
                                 jfa_bwd_block_sparse: the selection-bitmap (mark) kernel */
  JFA_KERNEL_SPARSE_SELECT = 4, /* jfa_fwd_block_sparse stage 1: the two pooling launches and the
                                  select launch (each recorded as one launch) */
  JFA_KERNEL_MX_QUANT = 5   /* the MXFP8 quantisation kernels (jfa_mxfp8_quantize_qk / _v) */
};

/* Measurement hook.  While enabled (enable != 0), every jfa_fwd / jfa_bwd /
 * jfa_fwd_block_sparse / jfa_bwd_block_sparse call records a
 * pair of HIP events on its stream immediately around each of its attention kernels
 * (not the schedule upload or the dQ fill / cast / reduce kernels).  jfa_kernel_times
 * waits for the events recorded so far for `kernel` (a jfa_kernel) and returns the
 * number of launches and their summed duration in milliseconds; reset != 0 then
 * forgets them.  Enabling or disabling also forgets them.  Events are created by the
 * library on the calling thread's current device and released when forgotten. */
int jfa_kernel_timing(int enable);
int jfa_kernel_times(int kernel, int64_t* launches, double* total_ms, int reset);

/* Which self-attention backward the calling thread's last jfa_bwd (or jfa_bwd_rotary /
 * jfa_bwd_mxfp8) call enqueued (JFA_BWD_PATH_OTHER for other modes, for a call that
 * failed before choosing, or before any call). */
enum jfa_bwd_path {
  JFA_BWD_PATH_OTHER = 0,
  JFA_BWD_PATH_RECOMPUTE = 1,       /* dQ kernel (also writing the row terms), then the
                                       dK/dV kernel, on the caller's stream */
  JFA_BWD_PATH_RECOMPUTE_SIDE = 2,  /* the two grids together fit the CUs: the row-term
                                       kernel, then the dQ kernel on a library-owned side
                                       stream (default priority) beside the dK/dV kernel;
                                       the caller's stream waits for both */
  JFA_BWD_PATH_STORED_DS = 3        /* row-term kernel, dK/dV kernel storing dS, dQ = dS K */
};
int jfa_last_bwd_path(void);

/* Debug hook: tile-visit counts, for checking that a schedule (static or run-time)
 * computes every tile exactly once.  counts: caller-allocated device int32 array of
 * 3 * stride entries that the caller zeroes; NULL turns counting off (the default).
 * While set, the tile kernels of every jfa_fwd / jfa_bwd / jfa_fwd_noalloc /
 * jfa_fwd_block_sparse / jfa_bwd_block_sparse / jfa_fwd_mxfp8 call (and the rotary
 * variants) add 1 to counts[kernel * stride + i] each time they take tile i of their
 * tile list, kernel = JFA_KERNEL_FWD (the forward kernel), JFA_KERNEL_BWD (the dK/dV
 * kernel, or the fused broadcast-Q / block-diagonal backward kernel) or
 * JFA_KERNEL_BWD_DQ (the dQ kernel); block-diagonal tiles are numbered (block, head)
 * in schedule order.  A call whose list is longer than stride fails with
 * JFA_ERR_CAPACITY before any device work.  jfa_debug_tile_list_size returns the
 * length of kernel's tile list in the last such call (0 if it launched no such
 * kernel).  Process-wide setting, one atomic add per tile; not for concurrent use. */
int jfa_debug_tile_visits(int32_t* counts, int64_t stride);
int jfa_debug_tile_list_size(int kernel, int64_t* tiles);

/* Static message for a status code. */
const char* jfa_error_string(int code);
/* Thread-local detail about the last failed call on this thread ("" if none). */
const char* jfa_last_error_detail(void);
/* JFA_VERSION of the built library. */
int jfa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* JFA_H_ */
