// Internal interface between the host runtime (jfa_api.cpp) and the kernels
// (jfa_*.hip): launch parameter blocks, tile sizes and launcher declarations.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jfa {

enum : int { kSelf = 0, kBroadcastQ = 1, kBlockDiag = 2, kSelfSparse = 3, kSelfChunks = 4 };

// Tile geometry.  A forward tile is kFwdRows query rows of one (sequence, head); its
// key/value loop streams kFwdKeys keys at a time.  A backward tile is kBwdKeys key
// rows of one (sequence, head); its loop streams kBwdRows query rows at a time.
// Block-diagonal tiles are one kBlock-token block of one head, one tile per wave.
constexpr int kFwdWaves = 8;      // waves per forward workgroup: two groups of four
constexpr int kFwdQPerWave = 32;  // query rows per wave (one 32-row MFMA block)
constexpr int kFwdRows = kFwdWaves * kFwdQPerWave;
constexpr int kFwdKeys = 64;
constexpr int kFwdStages = 3;     // K/V ring slots of the forward
constexpr int kDqWaves = 4;       // self-attention dQ kernel: 32 query rows per wave
constexpr int kDqRows = kDqWaves * 32;
constexpr int kDqKeys = 64;       // keys per step of the dQ kernel
constexpr int kBwdWaves = 4;      // waves per backward workgroup, 32 keys each
constexpr int kBwdKeys = kBwdWaves * 32;
constexpr int kBwdRows = 64;
constexpr int kBwdStages = 3;     // Q / dO ring slots of the dK/dV kernel
// Stored-dS self-attention backward: the dK/dV kernel writes dS in blocks of kBwdKeys
// keys x kBwdRows queries (bf16, 16 KB each) and a dQ = scale dS K kernel reads them
// back, kDsRows query rows per tile (kDsWaves waves of 32 rows, two per stored block
// column of 64 rows).
constexpr int kDsBlockBytes = kBwdKeys * kBwdRows * 2;
constexpr int kDsWaves = 8;
constexpr int kDsRows = kDsWaves * 32;
constexpr int kBlock = 64;
constexpr int kBdWaves = 4;
// Block-sparse variant: query blocks are forward tiles, key blocks forward key tiles;
// the select kernel ranks up to kSparseMaxKeyBlocks key blocks of a sequence in LDS.
constexpr int kSparseQBlock = kFwdRows;
constexpr int kSparseKBlock = kFwdKeys;
constexpr int kSparseMaxKeyBlocks = 2048;
// Block-sparse backward: a dK/dV tile's list of 64-row query steps holds at most this
// many entries (a sequence of kSparseMaxKeyBlocks key blocks).
constexpr int kSparseMaxSteps = kSparseMaxKeyBlocks * kSparseKBlock / kBwdRows;

// MXFP8 forward: mx_waves(D) waves of 32 query rows per workgroup (tiles of
// mx_rows(D) rows), mx_wg_per_cu(D) workgroups per CU (two waves per SIMD).
constexpr int mx_waves(int head_dim) { return head_dim == 128 ? 8 : 4; }
constexpr int mx_rows(int head_dim) { return mx_waves(head_dim) * 32; }
constexpr int mx_wg_per_cu(int head_dim) { return 8 / mx_waves(head_dim); }
constexpr int kMxMinRows = 128;  // smallest tile over the head dims (tile capacity)
// MXFP8 V layout: each sequence's keys padded to a multiple of this in the transposed codes.
constexpr int kMxVPad = 64;

// Persistent workgroups resident per CU (used for the default program count).
constexpr int kFwdWgPerCu = 1;    // one 8-wave workgroup: 2 waves per SIMD
constexpr int kBwdWgPerCu = 2;    // self-attention dK/dV kernel, upper bound over head dims
// Resident dK/dV workgroups per CU by head dim: D=64 fits 2 waves per SIMD in 256
// registers; D=128 needs the full 512 (1 wave per SIMD) to avoid spilling.
constexpr int dkdv_wg_per_cu(int head_dim) { return head_dim == 64 ? 2 : 1; }
constexpr int kBqWgPerCu = 1;     // broadcast-Q fused backward
constexpr int kDqWgPerCu = 2;     // self-attention dQ kernel
constexpr int kDsWgPerCu = 1;     // stored-dS dQ kernel (8 waves, three 48 KB LDS stages)
constexpr int kBdWgPerCu = 2;

constexpr float kLog2eHost = 1.4426950408889634f;

// Workspace run-time tile counters (zeroed by every schedule upload).  The dK/dV (and
// forward) kernels use counters 0 .. G-1, one per program group (G <= 127 heads); a dQ
// kernel that runs in the same call uses its own counter.
constexpr int kCounterSlots = 256;
constexpr int kDqCounter = 128;

// A scheduled tile: b = sequence, hb = (head << 24) | block index.
struct Tile {
  int32_t b;
  int32_t hb;
};

// Forward (self / broadcast-Q).  Pointers to bf16 data are typed as uint16_t here.
struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const int32_t* offsets;  // [B+1]
  const Tile* tiles;       // schedule
  const int32_t* seg_ptr;  // static: [P+1] per program; dynamic: [G+1] per counter group
  int32_t* counters;       // dynamic: one int32 per group (zeroed by the schedule upload)
  int32_t num_seqs, num_heads, num_q, num_programs;
  int64_t total_tokens;
  int32_t dynamic;
  int32_t num_kv_heads;  // key/value heads (divides num_heads)
  float scale_log2;  // scale * log2(e)
  // block-sparse self attention (kSelfSparse): tile (b, h, blk) attends to the key
  // tiles sel[sel_base[b] + (h * ceil(L_b / kSparseQBlock) + blk) * sel_k[b] + 0 ..
  // sel_k[b] - 1], ascending
  const int32_t* sel;
  const int64_t* sel_base;
  const int32_t* sel_k;
  // broadcast-Q key chunks: tile b field = chunk c; chunk c covers keys chunks[nc + c] ..
  // + chunks[2 nc + c] of sequence chunks[c] (nc = num_chunks).  chunks[3 nc + c] is -1
  // when the chunk is its sequence's only one (the tile writes o and lse) or a slot s
  // of part_o [S, Mq, H, D] / part_lse [S, H, Mq] (fp32: O normalised by the chunk's own
  // row sum, and the chunk's natural-log lse); then follow, per cut sequence i,
  // chunks[4 nc + 3 i + 0..2] = (b, first slot, slots), merged by launch_bq_combine.
  // Self-attention key chunks (kSelfChunks): the same [4, nc] table, with chunks[3 nc +
  // c] = -1 or the first part row r0 of the chunk: query row r of the tile's sequence
  // writes part row r0 + r of part_o [R, H, D] / part_lse [R, H]; then follows the cut
  // table of launch_self_combine.
  const int32_t* chunks;
  int32_t num_chunks;
  float* part_o;
  float* part_lse;
  int32_t* visits;  // debug (null: off): visits[i] += 1 each time tile i of the list is taken
};

// Block means of a bf16 [T, heads, D] tensor: out[h][blk][d] (fp32) over consecutive
// `block`-row groups of every sequence.
struct PoolParams {
  const uint16_t* x;
  float* out;
  const int32_t* offsets;     // [B+1]
  const int32_t* blk_prefix;  // [B+1]: blocks before sequence b
  int32_t num_seqs, heads, block, nblocks;
};

// Top-k key blocks per query block (block-sparse variant).
struct SelectParams {
  const float* qbar;          // [H][nqt][D] query-block means
  const float* kbar;          // [Hkv][nkb][D] key-block means
  const int32_t* offsets;     // [B+1]
  const int32_t* qt_prefix;   // [B+1]: query blocks before sequence b
  const int32_t* kb_prefix;   // [B+1]: key blocks before sequence b
  const int64_t* sel_base;    // [B+1]: first list entry of sequence b
  const int32_t* sel_k;       // [B]: kept key blocks per query block of sequence b
  int32_t* sel;               // out: ascending key-block lists
  int32_t num_seqs, num_heads, num_kv_heads, nqt, nkb;
};

// Block-sparse backward: marks, for every selection entry (b, h, query block i, key
// block kb), bit i of the bitmap of dK/dV tile kb / 2, half kb % 2 (BwdParams::sp_bits).
struct MarkParams {
  const int32_t* sel;
  const int64_t* sel_base;    // [B+1]
  const int32_t* sel_k;       // [B]
  const int32_t* offsets;     // [B+1]
  const int64_t* bits_base;   // [B+1]
  uint32_t* bits;             // zeroed by the caller
  int32_t num_seqs, num_heads;
  int64_t entries;            // sel_base[B]
};

// Backward (self / broadcast-Q).
struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;
  const int32_t* offsets;
  const Tile* tiles;
  const int32_t* seg_ptr;
  int32_t* counters;
  uint16_t* dk;
  uint16_t* dv;
  float* dq_acc;  // broadcast-Q atomics: [Mq,H,D] fp32; partials: [P,Mq,D] fp32
  uint16_t* dq;   // self: bf16 [T,H,D], written by the dQ kernel
  uint16_t* row_aug;         // self: [H,T,8] bf16 row terms (-lse log2 e, -Di as high/low pairs), written by the dQ (or row-term) kernel
  const Tile* dq_tiles;      // self: query-row tiles of the dQ kernel
  char* ds;                  // self, stored-dS path: dS blocks (null on the recompute path)
  const int64_t* ds_base;    // self, stored-dS path: [B+1] first dS block of each sequence
  // Block-sparse backward (sel non-null): the forward's selection lists (layout as in
  // FwdParams) for the dQ kernel, and per dK/dV tile (b, h, j) two bitmaps over the
  // query blocks of the sequence -- bit i of half x set when query block i kept key
  // block 2j + x -- at sp_bits[sp_bits_base[b] + ((h nj + j) 2 + x) nw + i / 32],
  // nj = ceil(L_b / kBwdKeys), nw = ceil(ceil(L_b / kSparseQBlock) / 32).
  const int32_t* sel;
  const int64_t* sel_base;
  const int32_t* sel_k;
  const uint32_t* sp_bits;
  const int64_t* sp_bits_base;
  int32_t sparse_narrow;     // block-sparse: 1 = 64-key dK/dV tiles of two waves (head_dim 128)
  const int32_t* dq_seg_ptr;
  int32_t dq_programs;
  int32_t num_seqs, num_heads, num_q, num_programs;
  int64_t total_tokens;
  int32_t dynamic;
  int32_t dq_partials;  // broadcast-Q: 1 = per-program slabs (plain read-modify-write)
  // Broadcast-Q through the dQ and dK/dV kernels (dq_path 2): the queries are the
  // shared q [Mq,H,D]; o, dout are [B,Mq,H,D]; lse and the row terms are [B,H,Mq(,8)].
  // The dQ kernel's tiles cover key chunks: chunk c is keys bq_chunks[NC + c] ..
  // + bq_chunks[2 NC + c] of sequence bq_chunks[c] (NC = num_chunks); the tile writes
  // the chunk's unscaled fp32 contribution to dq_acc [NC,Mq,H,D] (the chunk starting at
  // key 0 also writes the row terms) and a reduce kernel sums the chunks.
  int32_t bq;
  const int32_t* bq_chunks;
  int32_t num_chunks;
  int32_t programs_per_head;  // broadcast-Q head-pinned groups
  float scale;
  float scale_log2;
  int32_t* visits;     // debug (null: off): visit counts of the dK/dV (or fused) kernel's tiles
  int32_t* dq_visits;  // debug (null: off): visit counts of the dQ kernel's tiles
  int32_t rows_ready;  // self: 1 = the row-term kernel wrote row_aug, the dQ kernel leaves it alone
};

// Block-diagonal forward / backward.
struct BdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o_in;   // backward: forward output
  const uint16_t* dout;   // backward
  const float* lse_in;    // backward
  uint16_t* o;            // forward output / backward dq
  float* lse;             // forward
  uint16_t* dk;
  uint16_t* dv;
  const int32_t* offsets;      // [B+1]
  const int32_t* blk_prefix;   // [B+1]: blocks before sequence b
  int32_t num_seqs, num_heads, num_programs;
  int32_t num_kv_heads;  // forward: key/value heads (divides num_heads); backward: num_heads
  int64_t total_tokens;
  int64_t num_tiles;  // blocks * heads
  float scale;
  float scale_log2;
  // fused rotary embedding (null: none): cos, sin of p theta_i at rope[(p D/2 + i) 2 + {0, 1}],
  // p = position inside the sequence, i < D/2; q, k pairs (i, i + D/2) are rotated
  const float* rope;
  int32_t* visits;  // debug (null: off): visits[g] += 1 for every (block, head) tile g computed
};

// MXFP8 quantisation: Q / K rows (rows = T * heads, blocks along the head dimension),
// or V (transposed per head, blocks along each sequence's keys, vbase / tp / offsets).
struct MxQuantParams {
  const uint16_t* x;       // bf16 [T, H, D]
  uint8_t* codes;          // Q/K: [T, H, D]; V: [H][D][tp]
  uint8_t* scales;         // Q/K: [T, H, D/32]; V: [H][D][tp/32] (E8M0 codes)
  int64_t rows;            // Q/K: T * H
  int32_t num_heads, head_dim, num_seqs;
  const int32_t* offsets;  // V: [B+1]
  const int64_t* vbase;    // V: [B+1] padded start of each sequence
  const int32_t* group_seq;  // V: [tp / kMxVPad] sequence of each padded 64-key group
  int64_t tp;              // V: padded total (multiple of kMxVPad)
};

// MXFP8 decoding (the backward's inputs): codes + E8M0 exponents -> bf16.
struct MxDequantParams {
  const uint8_t* codes;      // Q/K: [T, H, D]; V: [H][D][tp]
  const uint8_t* scales;     // Q/K: [T, H, D/32]; V: [H][D][tp/32]
  uint16_t* out;             // bf16 [T, H, D]
  int64_t rows;              // Q/K: T * H
  int32_t num_heads, head_dim;
  const int32_t* offsets;    // V: [B+1]
  const int64_t* vbase;      // V: [B+1] padded start of each sequence
  const int32_t* group_seq;  // V: [tp / kMxVPad] sequence of each padded 64-key group
  int64_t tp;                // V: padded total
};

// MXFP8 forward (self attention; one key/value head per query head).
struct MxParams {
  const uint8_t* q8;
  const uint8_t* qsc;
  const uint8_t* k8;
  const uint8_t* ksc;
  const uint8_t* v8t;
  const uint8_t* vsc;
  const int64_t* vbase;
  int64_t tp;
  uint16_t* o;
  float* lse;
  const int32_t* offsets;
  const Tile* tiles;
  const int32_t* seg_ptr;
  int32_t num_heads, num_programs;
  int64_t total_tokens;
  float scale_log2;
  int32_t* visits;  // debug (null: off): visits[i] += 1 each time tile i of the list is taken
};

// Allocation-free forward (jfa_fwd_noalloc): bytes of the file-scope device scratch
// array that stands in for the workspace, and the calling device's address of it
// (looked up with hipGetSymbolAddress on the first call on each device).
constexpr size_t kNoAllocScratchBytes = size_t(4) << 20;
hipError_t noalloc_scratch(void** out);

// Launchers (defined next to their kernels).  head_dim selects the instantiation.
hipError_t launch_fwd(const FwdParams& p, int mode, int head_dim, hipStream_t s);
// Broadcast-Q forward: merge the chunk partials of the `cuts` cut sequences into o, lse.
hipError_t launch_bq_combine(const FwdParams& p, int cuts, int head_dim, hipStream_t s);
// Merge of cut self-attention sequences: `cuts` cuts covering `rows` query rows in all.
hipError_t launch_self_combine(const FwdParams& p, int cuts, int64_t rows, int head_dim, hipStream_t s);
hipError_t launch_bwd(const BwdParams& p, int mode, int head_dim, hipStream_t s);
// Self-attention backward: dQ kernel (query tiles; also writes the per-row stats the
// dK/dV kernel reads, so it runs first) and dK/dV kernel (key tiles).
hipError_t launch_bwd_self_dq(const BwdParams& p, int head_dim, hipStream_t s);
hipError_t launch_bwd_self_dkdv(const BwdParams& p, int head_dim, hipStream_t s);
// Stored-dS path: row terms (Di and lse per query row), then the dK/dV kernel with dS
// stores (p.ds non-null), then dQ from the stored dS.
hipError_t launch_bwd_self_prep(const BwdParams& p, int head_dim, hipStream_t s);
hipError_t launch_bwd_self_dq_ds(const BwdParams& p, int head_dim, hipStream_t s);
hipError_t launch_bd_fwd(const BdParams& p, int head_dim, hipStream_t s);
hipError_t launch_bd_bwd(const BdParams& p, int head_dim, hipStream_t s);
// Rotary table [positions][head_dim/2][2] fp32: cos, sin of pos * base^(-2i/D).
hipError_t launch_rope_table(float* table, int positions, int head_dim, double base, hipStream_t s);
hipError_t launch_fill_zero(float* x, int64_t n, hipStream_t s);
// Block-sparse variant, stage 1.
hipError_t launch_pool(const PoolParams& p, int head_dim, hipStream_t s);
hipError_t launch_select(const SelectParams& p, int head_dim, hipStream_t s);
hipError_t launch_mark(const MarkParams& p, hipStream_t s);
hipError_t launch_mx_quant_qk(const MxQuantParams& p, hipStream_t s);
hipError_t launch_mx_quant_v(const MxQuantParams& p, hipStream_t s);
hipError_t launch_mx_fwd(const MxParams& p, int head_dim, hipStream_t s);
hipError_t launch_mx_dequant_qk(const MxDequantParams& p, hipStream_t s);
hipError_t launch_mx_dequant_v(const MxDequantParams& p, hipStream_t s);
// dst[i] = bf16(scale * src[i]), i < n (n multiple of 8).
hipError_t launch_cast_scale(const float* src, uint16_t* dst, int64_t n, float scale, hipStream_t s);
// Broadcast-Q partial slabs [P, Mq, D] (programs h*ph .. h*ph+ph-1 hold head h) ->
// dq[Mq, H, D] = bf16(scale * sum).
hipError_t launch_dq_reduce(const float* partials, uint16_t* dq, int num_q, int num_heads,
                            int head_dim, int programs_per_head, float scale, hipStream_t s);
// Broadcast-Q key-chunk slabs [NC, Mq, H, D] -> dq[Mq, H, D] = bf16(scale * sum over the
// chunks), in a fixed (deterministic) order; the slabs are overwritten (0 slabs: dq = 0).
hipError_t launch_dq_seq_reduce(float* slabs, uint16_t* dq, int num_slabs, int64_t slab_elems,
                                float scale, hipStream_t s);
// Keys per broadcast-Q dQ chunk: at least kBqChunkMinSteps steps of kDqKeys.
constexpr int kBqChunkMinSteps = 4;

}  // namespace jfa
