// Self-attention backward for gfx950 as two persistent kernels with no dQ atomics.
//
// What it computes: the analytic gradient of sum(O * dO) per sequence and head, with
// P rebuilt from the forward's log-sum-exp, P = exp(scale * Q K^T - L) (the L kept for
// the backward, "TLX Block Attention", bittide page, section 2.1), and
// Di = rowsum(dO * O) formed inline in each kernel rather than in a preprocessing
// launch (same page, sections 2.1 and 4):
//   dV = P^T dO, dP = dO V^T, dS = P * (dP - Di), dK = scale dS^T Q, dQ = scale dS K.
//
// How it maps to CDNA4.  A fused kernel that owns a key/value block must hand its dQ
// contribution to every query row of the sequence; on MI355X coalesced fp32 atomics
// retire at roughly 3.4e11 per second device-wide, so for long jagged batches the
// dQ hand-off alone would outweigh the matrix work.  The self-attention backward is
// therefore split by ownership:
//  * dq_kernel (runs first): one workgroup = one tile of kDqRows query rows (32 per
//    wave) under the forward's sort + zigzag rule; the loop streams 64-key K and V
//    tiles through the same LDS ring as the forward.  Each lane owns one query row,
//    so Di = rowsum(dO * O) and lse are one scalar per lane; the kernel also stores
//    (lse * log2 e, Di) for its rows (8 bytes per row) for the second kernel.  Three
//    products per step: S^T = K Q^T and dP^T = V dO^T (C layout: lane = query), then
//    dQ^T += K^T dS^T with K^T read transposed from LDS and dS^T straight from
//    registers.  dQ is written once, by its owner.
//  * dkdv_kernel: one workgroup = one tile of kBwdKeys (128) keys of one (sequence,
//    head); wave w owns keys 32w..32w+31 with their K, V operands and fp32 dK^T, dV^T
//    accumulators in registers; 64 query rows stream through a three-slot ring of
//    swizzled LDS tiles (direct global->LDS copies issued two steps ahead) together
//    with their (lse * log2 e, Di) row terms.  Four products per step: S = Q K^T and
//    dP = dO V^T (C layout: lane = key), then dV^T += dO^T P and dK^T += Q^T dS with
//    dO^T, Q^T read transposed from LDS (ds_read_b64_tr_b16).  dK and dV are written
//    once, by their owner.
// The split recomputes S and dP once more (seven products per query-key block
// instead of five) in exchange for no atomics and no fp32 dQ accumulator in HBM.
//
// Stored-dS variant (when the caller grants the workspace): prep_kernel writes the row
// terms, the dK/dV kernel also stores dS (bf16, two bytes per query-key pair) and
// dq_ds_kernel forms dQ = scale dS K from it -- five products per block plus the dS
// round trip through HBM instead of seven products.
//
// Block-sparse variant (the backward of the block-sparse top-k forward with its
// selection held fixed): the dQ kernel walks its query block's kept key blocks instead
// of all of them; the dK/dV kernel walks only the query blocks that kept one of the
// tile's two 64-key blocks (from a bitmap built by the mark kernel), and where a query
// block kept only one of them, the waves of the other block turn P (hence dV, dS, dK)
// to zero through the row-term MFMA: every row term carries -1 in one extra k-slot,
// which those waves' B operand scales by 1e30.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "jfa_device.h"
#include "jfa_internal.h"
#include "jfa_sched.h"

namespace jfa {
namespace {

// ----------------------------------------------------------------------------- dQ

template <int D>
struct DqCfg {
  static constexpr int NW = kDqWaves;
  static constexpr int NT = NW * 64;
  static constexpr int BM = kDqRows;
  static constexpr int BN = kDqKeys;
  static constexpr int NKB = BN / 32;
  static constexpr int NKS = D / 16;
  static constexpr int NDB = D / 32;
  static constexpr int NT16 = BN / 16;
  static constexpr int RB = 2 * D;
  static constexpr int BUF = BN * RB;
};

// Per-lane constants of the dQ loop: LDS operand offsets and ring-copy offsets.
template <int D>
struct DqLane {
  RowOperands<DqCfg<D>::RB, DqCfg<D>::NKS> row;  // K, V rows as A operands of S^T, dP^T
  TrOperands<DqCfg<D>::RB, DqCfg<D>::NDB> ktr;   // K^T as the A operand of dQ^T
  TileCopy<DqCfg<D>::RB, DqCfg<D>::BN, DqCfg<D>::NW> copy;
};

// One key/value tile for this wave's 32 query rows.  MASK: keys >= keys_valid lie past
// the end of the sequence.
template <int D, bool MASK>
__device__ __forceinline__ void dq_step(const JFA_LDS char* kbuf, const JFA_LDS char* vbuf, const DqLane<D>& ln,
                                        const bf16x8 (&qf)[DqCfg<D>::NKS], const bf16x8 (&dof)[DqCfg<D>::NKS],
                                        f32x16 (&dq)[DqCfg<D>::NDB], float lse2, float di, int lane,
                                        int keys_valid, float c) {
  using C = DqCfg<D>;
  const int half = lane >> 5;
  f32x16 s[C::NKB], dp[C::NKB];
#pragma unroll
  for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) s[kb][i] = dp[kb][i] = 0.f;
#pragma unroll
  for (int ks = 0; ks < C::NKS; ++ks) {
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb) {
      s[kb] = mfma32(ln.row.read(kbuf, kb * 32, ks), qf[ks], s[kb]);
      dp[kb] = mfma32(ln.row.read(vbuf, kb * 32, ks), dof[ks], dp[kb]);
    }
  }
  // P^T = 2^(S^T c - lse2), dS^T = P^T (dP^T - Di); lane = query, register i <-> key.
#pragma unroll
  for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float pv = fast_exp2(fmaf(s[kb][i], c, -lse2));
      if (MASK) {
        const int key = kb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
        pv = key < keys_valid ? pv : 0.f;
      }
      dp[kb][i] = pv * (dp[kb][i] - di);
    }
  // dQ^T += K^T dS^T: A = K^T (transposed LDS read), B = dS^T from the C layout.
#pragma unroll
  for (int t = 0; t < C::NT16; ++t) {
    const f32x16& src = dp[t >> 1];
    const int r = 8 * (t & 1);
    const bf16x8 b = pack8(src[r], src[r + 1], src[r + 2], src[r + 3], src[r + 4], src[r + 5], src[r + 6], src[r + 7]);
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) dq[db] = mfma32(ln.ktr.read(kbuf, 16 * t, db), b, dq[db]);
  }
}

// SPARSE: the tile's rows lie in one block-sparse query block, whose kept key blocks
// (ascending, one 64-key step each) replace the full key range.
template <int D, bool SPARSE>
__device__ __forceinline__ void dq_tile(const BwdParams& p, Tile tile, JFA_LDS char* smem, const DqLane<D>& ln,
                                        int tid) {
  using C = DqCfg<D>;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int h = tile.hb >> 24, blk = tile.hb & 0xFFFFFF;
  // Self attention: the tile's rows are the sequence's own tokens and its keys all of
  // the sequence's keys.  Broadcast-Q: the rows are rows of the shared q (o, dO, lse
  // and the row terms per sequence) and the keys one chunk of the sequence's keys.
  const bool bq = p.bq != 0;
  const int chunk = tile.b;
  const int b = bq ? p.bq_chunks[chunk] : tile.b;
  const int64_t rs = (int64_t)p.num_heads * D;
  const int64_t s0 = p.offsets[b];
  const int kstart = bq ? p.bq_chunks[p.num_chunks + chunk] : 0;
  const int L = bq ? p.bq_chunks[2 * p.num_chunks + chunk] : (int)(p.offsets[b + 1] - s0);  // keys of the tile
  const int row = blk * C::BM + wave * 32 + l32;
  const int Lq = bq ? p.num_q : L;
  const bool row_ok = row < Lq;
  const int64_t qrow = bq ? (int64_t)row : s0 + row;
  const int64_t orow = bq ? (int64_t)b * p.num_q + row : s0 + row;
  const int64_t lrow = bq ? ((int64_t)b * p.num_heads + h) * p.num_q + row : (int64_t)h * p.total_tokens + s0 + row;
  const int64_t aug_rows = bq ? (int64_t)p.num_seqs * p.num_heads * p.num_q : (int64_t)p.num_heads * p.total_tokens;
  const float c = p.scale_log2;

  // Q and dO rows as B operands; Di = rowsum(dO * O) and lse2 for this lane's row.
  bf16x8 qf[C::NKS], dof[C::NKS];
  float di = 0.f;
  {
    const int64_t qbase = qrow * rs + (int64_t)h * D + 8 * half;
    const int64_t obase = orow * rs + (int64_t)h * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
      qf[ks] = as_bf16x8(row_ok ? ld16(p.q + qbase + 16 * ks) : zero16());
      dof[ks] = as_bf16x8(row_ok ? ld16(p.dout + obase + 16 * ks) : zero16());
      const bf16x8 o8 = as_bf16x8(row_ok ? ld16(p.o + obase + 16 * ks) : zero16());
#pragma unroll
      for (int e = 0; e < 8; ++e) di = fmaf((float)dof[ks][e], (float)o8[e], di);
    }
    di = half_sum(di);
  }
  const float lse = row_ok ? p.lse[lrow] : INFINITY;
  const float lse2 = lse * kLog2e;
  if (blockIdx.x == 0 && tid == 0 && !p.rows_ready) {
    // sentinel row term for query rows past the end of a sequence (P = dS = 0)
    const bf16 z = (bf16)0.0f;
    const bf16x8 t = {(bf16)(-1e30f), z, (bf16)(-1.0f), z, z, z, z, z};
    st16(p.row_aug + aug_rows * 8, __builtin_bit_cast(u32x4, t));
  }
  if (row_ok && half == 0 && kstart == 0 && !p.rows_ready) {
    // Row term for the dK/dV kernel: -lse log2 e and -Di as bf16 high + low parts
    // (c S - lse log2 e, c = scale log2 e, is the exponent of P in base 2), and the
    // constant -1 the block-sparse key mask multiplies.
    st16(p.row_aug + lrow * 8, __builtin_bit_cast(u32x4, row_term(lse, di)));
  }

  f32x16 dq[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dq[db][i] = 0.f;

  // Key steps: all of them, or (SPARSE) the kept blocks; only the last step can hold
  // the sequence's partial block (the kept list is ascending).  List entries are
  // clamped into [0, nkb) so that no copy leaves the sequence.
  int n_full = L / C::BN, tail = L % C::BN;
  int n_kv = n_full + (tail != 0);
  const int32_t* list = nullptr;
  const int nkb = (L + C::BN - 1) / C::BN;
  if constexpr (SPARSE) {
    static_assert(kSparseKBlock == C::BN && kSparseQBlock % C::BM == 0, "sparse blocks vs dQ tiles");
    const int nqb = (L + kSparseQBlock - 1) / kSparseQBlock;
    const int kk = p.sel_k[b];
    list = p.sel + p.sel_base[b] + ((int64_t)h * nqb + (blk * C::BM) / kSparseQBlock) * kk;
    const int last = min(max(list[kk - 1], 0), nkb - 1);
    const bool part = tail != 0 && last == nkb - 1;
    n_kv = kk;
    n_full = kk - (part ? 1 : 0);
    tail = part ? tail : 0;
  }
  auto key0_of = [&](int it) { return (SPARSE ? min(max(list[it], 0), nkb - 1) : it) * C::BN; };
  const uint16_t* kp = p.k + (s0 + kstart) * rs + (int64_t)h * D;
  const uint16_t* vp = p.v + (s0 + kstart) * rs + (int64_t)h * D;
  const uint32_t rsb = (uint32_t)(rs * 2);
  if (n_kv > 0) {  // (broadcast-Q tiles of an empty sequence have no keys: dQ = 0)
    const int k0 = key0_of(0);
    ln.copy.issue_rows(kp + (int64_t)k0 * rs, rsb, min(C::BN, L - k0), smem, wave, lane);
    ln.copy.issue_rows(vp + (int64_t)k0 * rs, rsb, min(C::BN, L - k0), smem + C::BUF, wave, lane);
  }
  wait_vmem();
  __syncthreads();
  for (int it = 0; it < n_full; ++it) {
    const int cur = it & 1;
    if (it + 1 < n_kv) {
      const int k1 = key0_of(it + 1);
      const int64_t nxt = (int64_t)k1 * rs;
      const int rv = min(C::BN, L - k1);
      JFA_LDS char* nbuf = smem + (cur ^ 1) * 2 * C::BUF;
      ln.copy.issue_rows(kp + nxt, rsb, rv, nbuf, wave, lane);
      ln.copy.issue_rows(vp + nxt, rsb, rv, nbuf + C::BUF, wave, lane);
    }
    JFA_LDS char* kbuf = smem + cur * 2 * C::BUF;
    dq_step<D, false>(kbuf, kbuf + C::BUF, ln, qf, dof, dq, lse2, di, lane, C::BN, c);
    wait_vmem();
    __syncthreads();
  }
  if (tail) {
    JFA_LDS char* kbuf = smem + (n_full & 1) * 2 * C::BUF;
    dq_step<D, true>(kbuf, kbuf + C::BUF, ln, qf, dof, dq, lse2, di, lane, tail, c);
    __syncthreads();
  }
  if (row_ok && bq) {
    // this sequence's unscaled contribution, summed over the sequences by a reduce kernel
    float* ap = p.dq_acc + ((int64_t)chunk * p.num_q + row) * rs + (int64_t)h * D + 4 * half;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<float4*>(ap + 32 * db + 8 * g4) =
            make_float4(dq[db][4 * g4], dq[db][4 * g4 + 1], dq[db][4 * g4 + 2], dq[db][4 * g4 + 3]);
  } else if (row_ok) {
    uint16_t* qp = p.dq + (s0 + row) * rs + (int64_t)h * D + 4 * half;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        st8(qp + 32 * db + 8 * g4, pack4(dq[db][4 * g4] * p.scale, dq[db][4 * g4 + 1] * p.scale,
                                        dq[db][4 * g4 + 2] * p.scale, dq[db][4 * g4 + 3] * p.scale));
  }
}

// ---------------------------------------------------------------------------- dK, dV

template <int D, int NW_ = kBwdWaves, int NS_ = kBwdStages>
struct KvCfg {
  static constexpr int NW = NW_;
  static constexpr int NT = NW * 64;
  static constexpr int BN = NW * 32;  // keys per tile
  static constexpr int QB = kBwdRows;
  static constexpr int NQB = QB / 32;
  static constexpr int NKS = D / 16;
  static constexpr int NDB = D / 32;
  static constexpr int RB = 2 * D;
  static constexpr int QBUF = QB * RB;
  static constexpr int ABUF = QB * 16;                 // one 16-byte row term per query row
  static constexpr int NS = NS_;
  static constexpr int OFF_Q = 0;                      // [NS][QBUF]
  static constexpr int OFF_DO = OFF_Q + NS * QBUF;     // [NS][QBUF]
  static constexpr int OFF_AUG = OFF_DO + NS * QBUF;   // [NS][ABUF]
  static constexpr int SMEM = OFF_AUG + NS * ABUF;
  static_assert(QB == 64, "one 64-lane copy moves a step's row terms");
};

// Per-lane constants of the dK/dV loop: LDS operand offsets, ring-copy offsets and the
// B operands of the row-term MFMAs.
template <int D, int NW = kBwdWaves>
struct KvLane {
  RowOperands<KvCfg<D>::RB, KvCfg<D>::NKS> row;  // Q, dO rows as A operands of S, dP
  TrOperands<KvCfg<D>::RB, KvCfg<D>::NDB> tr;    // Q^T, dO^T as A operands of dK^T, dV^T
  using Copy = TileCopy<KvCfg<D>::RB, KvCfg<D>::QB, NW>;
  Copy copy;
  bf16x8 pick_s, pick_dp;  // k-slots 0,1 (S) and 4,5 (dP) of the row term, lanes 0-31
  __device__ __forceinline__ void init_pick(int lane) {
    const bf16 one = (bf16)1.0f, zero = (bf16)0.0f;
    const bool lo = lane < 32;
    pick_s = bf16x8{lo ? one : zero, lo ? one : zero, zero, zero, zero, zero, zero, zero};
    pick_dp = bf16x8{zero, zero, zero, zero, lo ? one : zero, lo ? one : zero, zero, zero};
  }
};

// Issue the copies of a step: Q and dO rows (all waves; rows past rows_valid repeat the
// last valid row) and the 16-byte row terms (wave 0, one row per lane; rows past
// rows_valid take the sentinel term at index sentinel, whose -lse log2 e part is
// -1e30, so that their P and dS are exactly zero).
template <int D, int NW>
__device__ __forceinline__ void kv_issue(const KvLane<D, NW>& ln, const uint16_t* qb, const uint16_t* dob,
                                         const uint16_t* aug, int64_t rs, int64_t aug_row0, int64_t sentinel,
                                         int row0, int rows_valid, JFA_LDS char* qbuf, JFA_LDS char* dobuf,
                                         JFA_LDS char* augbuf, int wave, int lane) {
  const uint32_t rsb = (uint32_t)(rs * 2);
  ln.copy.issue_rows(qb + (int64_t)row0 * rs, rsb, rows_valid, qbuf, wave, lane);
  ln.copy.issue_rows(dob + (int64_t)row0 * rs, rsb, rows_valid, dobuf, wave, lane);
  if (wave == 0) {
    const int64_t r = lane < rows_valid ? aug_row0 + row0 + lane : sentinel;
    dma16(uniform_ptr(aug), (uint32_t)(r * 16), augbuf);
  }
}

// Stored dS (the stored-dS path).  dS of (sequence b, head h) is kept as blocks of 128
// keys (one dK/dV tile j) x 64 queries (one step it), NJ = ceil(L/128) x NQ = ceil(L/64)
// of them, block (j, it) at index ds_base[b] + (h NJ + j) NQ + it, 16 KB each.  Inside a
// block, dS[key 32w + r][query 32qq + 16x + 8y + 4e + i] (r < 32; x, y, e < 2; i < 4)
// sits at
//   byte w*4096 + qq*2048 + x*1024 + 16*(32e + (r ^ (8x + 4e))) + 8y + 2i.
// This is the order the dK/dV kernel produces it in: in wave w, lane (half e, key r)
// holds the packed dS of queries 32qq + 16x + 8y + 4e + i for y, i as one 16-byte
// register per (qq, x), so each of its four stores per step writes 1 KB contiguous.
// The XOR term makes the transposed LDS fetches of the dQ kernel (per half-wave: 4 keys
// x 8 query quads = 32 distinct 8-byte slots of a 256-byte bank line) conflict free.
__device__ __forceinline__ uint32_t ds_store_offset(int wave, int lane) {
  const int r = lane & 31, e = lane >> 5;
  return (uint32_t)(wave * 4096 + 512 * e + 16 * (r ^ (4 * e)));
}

// Store of register x of query block qq (unit offsets as above; x flips bit 7).
__device__ __forceinline__ void store_ds_unit(char* blk, uint32_t off, int qq, int x, const bf16x8& v) {
  st16_global_nt(blk, (off ^ (uint32_t)(x << 7)) + qq * 2048 + x * 1024, __builtin_bit_cast(u32x4, v));
}

// The four stores of one step.
template <int NQB>
__device__ __forceinline__ void store_ds(char* blk, uint32_t off, const bf16x8 (&keep)[NQB][2]) {
  char* b = (char*)uniform_ptr(blk);
#pragma unroll
  for (int qq = 0; qq < NQB; ++qq)
#pragma unroll
    for (int x = 0; x < 2; ++x) store_ds_unit(b, off, qq, x, keep[qq][x]);
}

// The row terms ride on one extra k-step of S and dP: each query row's 16-byte term
// holds -lse log2 e and -Di split into bf16 high and low parts, and the B operand picks
// the pair that belongs to each product, so that S' = Q (cK)^T - lse log2 e and
// dP' = dO V^T - Di come out of the MFMAs and P = 2^S', dS = P dP' need no per-row
// operands in the vector unit.  C layout of S', dP' ([queries x keys]): lane = key,
// register i <-> query 32*qq + 8*(i/4) + 4*half + i%4.
//
// Keys past the end of the sequence need no mask: their P and dS only feed their own
// dK, dV rows, which are never stored; query rows past the end carry the sentinel row
// term and get P = dS = 0.
//
// One 64-row step as a single stream of MFMAs.  Per 32-row query block (qq) the
// stream is
//   S' row term, S' k-steps | dP' row term, dP' k-steps | dV^T (u, db) | dK^T (u, db)
// and the two blocks follow each other.  Every operand that comes from LDS is read
// AHEAD (six) stream positions before its MFMA, across region and block boundaries, into a
// small register ring, so that no region starts by waiting for LDS.  The vector work
// is cut into slices placed between MFMAs: P = 2^S' (one slice per dP' k-step,
// from the first one after the dP' row term, when S' has left the pipeline) and
// dS = P dP' (during the dV products, from their third slot on).  The pack of P (dS) into B operands
// completes before the first dV (dK) MFMA that needs it.
template <int D, bool STORE, int NW = kBwdWaves>
struct KvStream {
  using C = KvCfg<D>;
  static constexpr int NKS = C::NKS, NDB = C::NDB;
  static constexpr int S0 = 0;                    // S' row term
  static constexpr int DP0 = NKS + 1;             // dP' row term
  static constexpr int DV0 = 2 * NKS + 2;         // first dV^T product
  static constexpr int DK0 = DV0 + 2 * NDB;       // first dK^T product
  static constexpr int PER = DK0 + 2 * NDB;       // MFMAs per query block
  static constexpr int N = C::NQB * PER;          // MFMAs per step
  static constexpr int AHEAD = 6, NBUF = AHEAD + 1;
  static constexpr int P_PER = 16 / NKS;          // P values per slice (one slice per dP' k-step)
  static constexpr int DS_SL = 2 * NDB - 2;       // dS slices (dV slots 2 .. 2*NDB-1)
  static constexpr int DS_PER = (16 + DS_SL - 1) / DS_SL;

  const JFA_LDS char *qt, *dot, *augt;
  const KvLane<D, NW>& ln;
  const bf16x8 (&kf)[NKS];
  const bf16x8 (&vf)[NKS];
  f32x16 (&dk)[NDB];
  f32x16 (&dv)[NDB];
  const int l32;
  const float c;
  const bf16x8 pick;  // B operand of the S' row-term MFMA (KvLane::pick_s, or the masking one)
  bf16x8 buf[NBUF];
  bf16x8 term;
  f32x16 s, dp;
  float pr[16], dsr[16];
  bf16x8 pf[2], dsf[2];
  // STORE: keep[qq] holds the packed dS of query block qq.  The previous step's values
  // are stored from inside this step's stream, spread over MFMA slots (block 0 before
  // slot DK0 - 1, where this step overwrites it; block 1 after), so that the stores
  // never queue behind the step's ring copies at the step start.
  bf16x8 (&keep)[C::NQB][2];
  char* sblk;       // wave-uniform: the stored block of the previous step
  uint32_t soff;    // this lane's store offset (ds_store_offset)
  static constexpr int ST0 = 6, ST0_STEP = (DK0 - 2 - ST0);       // block 0 stores: ST0 + x ST0_STEP
  static constexpr int ST1 = DK0 + 4, ST1_STEP = (PER + DK0 - 2 - ST1);
  static_assert(ST0_STEP >= 1 && ST0 + ST0_STEP < DK0 - 1 && ST1 + ST1_STEP < PER + DK0 - 1, "store slots");

  __device__ __forceinline__ KvStream(const JFA_LDS char* qt_, const JFA_LDS char* dot_, const JFA_LDS char* augt_,
                                      const KvLane<D, NW>& ln_, const bf16x8 (&kf_)[NKS], const bf16x8 (&vf_)[NKS],
                                      f32x16 (&dk_)[NDB], f32x16 (&dv_)[NDB], int l32_, float c_,
                                      bf16x8 (&keep_)[C::NQB][2], char* sblk_, uint32_t soff_,
                                      const bf16x8& pick_)
      : qt(qt_), dot(dot_), augt(augt_), ln(ln_), kf(kf_), vf(vf_), dk(dk_), dv(dv_), l32(l32_), c(c_),
        pick(pick_), keep(keep_), sblk(sblk_), soff(soff_) {}

  // Store slot of stream position K: query block (0 or 1) * 2 + register x, or -1.
  template <int K>
  static constexpr int store_slot() {
    if (!STORE) return -1;
    if (K == ST0 || K == ST0 + ST0_STEP) return (K - ST0) / ST0_STEP;
    if (K == ST1 || K == ST1 + ST1_STEP) return 2 + (K - ST1) / ST1_STEP;
    return -1;
  }
  template <int K>
  __device__ __forceinline__ void store() {
    constexpr int sl = store_slot<K>();
    if constexpr (sl >= 0) store_ds_unit(sblk, soff, sl >> 1, sl & 1, keep[sl >> 1][sl & 1]);
  }

  // LDS read(s) of stream position K (none for the dP' row term, which reuses the S'
  // one); reads<K>() counts them.
  template <int K>
  __device__ __forceinline__ void read() {
    constexpr int qq = K / PER, k = K % PER;
    if constexpr (k == S0) {
      buf[K % NBUF] = as_bf16x8(lds_ld16(augt, (qq * 32 + l32) * 16));
    } else if constexpr (k < DP0) {
      buf[K % NBUF] = ln.row.read(qt, qq * 32, k - 1);
    } else if constexpr (k == DP0) {
    } else if constexpr (k < DV0) {
      buf[K % NBUF] = ln.row.read(dot, qq * 32, k - DP0 - 1);
    } else if constexpr (k < DK0) {
      constexpr int u = (k - DV0) / NDB, db = (k - DV0) % NDB;
      buf[K % NBUF] = ln.tr.read(dot, 16 * (2 * qq + u), db);
    } else {
      constexpr int u = (k - DK0) / NDB, db = (k - DK0) % NDB;
      buf[K % NBUF] = ln.tr.read(qt, 16 * (2 * qq + u), db);
    }
  }
  template <int K>
  static constexpr int reads() {
    constexpr int k = K % PER;
    return k == DP0 ? 0 : (k < DV0 ? 1 : 2);
  }

  template <int K>
  __device__ __forceinline__ void mfma() {
    constexpr int k = K % PER;
    if constexpr (k == S0) {
      term = buf[K % NBUF];
      s = mfma32(term, pick, f32x16{});
    } else if constexpr (k < DP0) {
      s = mfma32(buf[K % NBUF], kf[k - 1], s);
    } else if constexpr (k == DP0) {
      dp = mfma32(term, ln.pick_dp, f32x16{});
    } else if constexpr (k < DV0) {
      dp = mfma32(buf[K % NBUF], vf[k - DP0 - 1], dp);
    } else if constexpr (k < DK0) {
      constexpr int u = (k - DV0) / NDB, db = (k - DV0) % NDB;
      dv[db] = mfma32(buf[K % NBUF], pf[u], dv[db]);
    } else {
      constexpr int u = (k - DK0) / NDB, db = (k - DK0) % NDB;
      dk[db] = mfma32(buf[K % NBUF], dsf[u], dk[db]);
    }
  }

  // Vector slice placed after MFMA K; valus<K>() is its VALU instruction count (for the
  // issue-order hints).
  template <int K>
  __device__ __forceinline__ void valu() {
    constexpr int k = K % PER;
    if constexpr (k >= DP0 + 1 && k < DV0) {
      constexpr int j = k - DP0 - 1;  // 0 .. NKS-1
#pragma unroll
      for (int e = 0; e < P_PER; ++e) pr[j * P_PER + e] = fast_exp2(s[j * P_PER + e]);
      if constexpr ((j + 1) * P_PER == 8) pf[0] = pack8(pr[0], pr[1], pr[2], pr[3], pr[4], pr[5], pr[6], pr[7]);
      if constexpr ((j + 1) * P_PER == 16)
        pf[1] = pack8(pr[8], pr[9], pr[10], pr[11], pr[12], pr[13], pr[14], pr[15]);
    } else if constexpr (k >= DV0 + 2 && k < DK0) {
      constexpr int j = k - DV0 - 2;  // 0 .. DS_SL-1
#pragma unroll
      for (int e = 0; e < DS_PER; ++e) {
        const int i = j * DS_PER + e;
        if (i < 16) dsr[i] = pr[i] * dp[i];
      }
      if constexpr ((j + 1) * DS_PER >= 8 && j * DS_PER < 8)
        dsf[0] = pack8(dsr[0], dsr[1], dsr[2], dsr[3], dsr[4], dsr[5], dsr[6], dsr[7]);
      if constexpr (j == DS_SL - 1) {
        dsf[1] = pack8(dsr[8], dsr[9], dsr[10], dsr[11], dsr[12], dsr[13], dsr[14], dsr[15]);
        if constexpr (STORE) {
          keep[K / PER][0] = dsf[0];
          keep[K / PER][1] = dsf[1];
        }
      }
    }
  }
  template <int K>
  static constexpr int valus() {
    constexpr int k = K % PER;
    if (k >= DP0 + 1 && k < DV0) return 2 * P_PER + ((k - DP0) * P_PER % 8 == 0 ? 4 : 0);
    if (k >= DV0 + 2 && k < DK0) return DS_PER + 2;
    return 0;
  }

  template <int K>
  __device__ __forceinline__ void order() {
    if constexpr (K == 0) __builtin_amdgcn_sched_group_barrier(0x100, AHEAD * 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (valus<K>() > 0) __builtin_amdgcn_sched_group_barrier(0x002, valus<K>(), 0);
    if constexpr (K + AHEAD < N && reads<K + AHEAD>() > 0)
      __builtin_amdgcn_sched_group_barrier(0x100, reads<K + AHEAD>(), 0);
    if constexpr (store_slot<K>() >= 0) __builtin_amdgcn_sched_group_barrier(0x040, 1, 0);
  }

  template <int K>
  __device__ __forceinline__ void step() {
    mfma<K>();
    valu<K>();
    if constexpr (K + AHEAD < N) read<K + AHEAD>();
    store<K>();
  }

  __device__ __forceinline__ void go() {
    prologue(std::make_integer_sequence<int, AHEAD>{});
    body(std::make_integer_sequence<int, N>{});
    orders(std::make_integer_sequence<int, N>{});
    __builtin_amdgcn_sched_barrier(0);
  }
  template <int... K>
  __device__ __forceinline__ void prologue(std::integer_sequence<int, K...>) { (read<K>(), ...); }
  template <int... K>
  __device__ __forceinline__ void body(std::integer_sequence<int, K...>) { (step<K>(), ...); }
  template <int... K>
  __device__ __forceinline__ void orders(std::integer_sequence<int, K...>) { (order<K>(), ...); }
};

// Block-sparse step list: wave 0 turns the tile's two query-block bitmaps into the
// ascending list of its 64-row query steps, entry = step | (halves kept) << 24, at
// steps[0 .. n) with n at steps[kSparseMaxSteps].  Returns n (all waves).
// TB = key blocks per tile: 2 (128-key tile j, both bitmaps) or 1 (64-key tile j: the
// bitmap of half j % 2 of 128-key tile j / 2; every listed step keeps the whole tile).
template <int QB, int TB>
__device__ __forceinline__ int sparse_steps(const BwdParams& p, int b, int h, int j, int L, int nq, JFA_LDS int* steps,
                                            int wave, int lane) {
  constexpr int SPQ = kSparseQBlock / QB;  // query steps per query block
  const int nqb = (L + kSparseQBlock - 1) / kSparseQBlock, nw = (nqb + 31) / 32;
  const int64_t nj = (L + kBwdKeys - 1) / kBwdKeys;
  const uint32_t* bm = p.sp_bits + p.sp_bits_base[b] + ((int64_t)h * nj + (TB == 2 ? j : j >> 1)) * 2 * nw;
  if (TB == 1) bm += (j & 1) * nw;
  __syncthreads();  // the previous tile's readers are done with the list
  if (wave == 0) {
    int count = 0;
    bool last_kept = false;
    for (int i0 = 0; i0 < nqb; i0 += 64) {
      const int i = i0 + lane;
      int m = 0;
      if (i < nqb) {
        m = (bm[i >> 5] >> (i & 31)) & 1;
        if (TB == 2) m |= ((bm[nw + (i >> 5)] >> (i & 31)) & 1) << 1;
      }
      const uint64_t kept = __ballot(m != 0);
      const int pos = count + __popcll(kept & ((1ull << lane) - 1));
      if (m != 0) {
#pragma unroll
        for (int t = 0; t < SPQ; ++t) {
          const int it = SPQ * i + t;
          if (it < nq && SPQ * pos + t < kSparseMaxSteps) steps[SPQ * pos + t] = it | (m << 24);
        }
      }
      count += __popcll(kept);
      last_kept = last_kept || __ballot(m != 0 && i == nqb - 1) != 0;
    }
    if (lane == 0) steps[kSparseMaxSteps] = min(SPQ * count - (last_kept ? SPQ * nqb - nq : 0), kSparseMaxSteps);
  }
  __syncthreads();
  return steps[kSparseMaxSteps];
}

// SPARSE: only the query steps of the block-sparse step list (see sparse_steps); the
// waves whose 64-key block a step's query block did not keep use the masking pick.
// NW waves of 32 keys (tile of NW*32 keys) and an NS-slot ring (NS = 3: copies two
// steps ahead; NS = 2: one step ahead).
template <int D, bool STORE, bool SPARSE, int NW = kBwdWaves, int NS = kBwdStages>
__device__ __forceinline__ void dkdv_tile(const BwdParams& p, Tile tile, char* smem_raw, const KvLane<D, NW>& ln,
                                          int tid) {
  static_assert(!(STORE && SPARSE), "the block-sparse backward recomputes dS");
  static_assert(NS == 2 || NS == 3, "ring of two or three slots");
  static_assert(!STORE || NW == kBwdWaves, "the stored-dS layout assumes the 128-key tile");
  using C = KvCfg<D, NW, NS>;
  JFA_LDS char* smem = (JFA_LDS char*)smem_raw;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int b = tile.b, h = tile.hb >> 24, j = tile.hb & 0xFFFFFF;
  const int64_t rs = (int64_t)p.num_heads * D;
  const int64_t s0 = p.offsets[b];
  const int L = (int)(p.offsets[b + 1] - s0);
  const int key0 = j * C::BN;
  const int my_key = wave * 32 + l32;
  const bool key_ok = my_key < L - key0;
  const float c = p.scale_log2;
  // Query rows: the sequence's own tokens, or (broadcast-Q) the shared q rows with this
  // sequence's dO and row terms.
  const bool bq = p.bq != 0;
  const int Lq = bq ? p.num_q : L;
  const uint16_t* qb = p.q + (bq ? 0 : s0 * rs) + (int64_t)h * D;
  const uint16_t* dob = p.dout + (bq ? (int64_t)b * p.num_q : s0) * rs + (int64_t)h * D;
  const int64_t aug_row0 = bq ? ((int64_t)b * p.num_heads + h) * p.num_q : (int64_t)h * p.total_tokens + s0;
  const int64_t sentinel = bq ? (int64_t)p.num_seqs * p.num_heads * p.num_q : (int64_t)p.num_heads * p.total_tokens;
  const int nq = (Lq + C::QB - 1) / C::QB;

  // Three-slot ring: step it+2 is copied while step it is computed, so each copy has two
  // steps to land.  The wait that closes a step leaves only the newest step's copies
  // outstanding (vector-memory loads return in issue order, so the older step's copies
  // have landed; dS stores that may still be in flight do not matter here).  Wave 0
  // issues one more copy (the row terms) than the others; waiting for all but 2J lets
  // it wait for one copy of the newest step as well, which is harmless.
  auto issue = [&](int it, int slot) {
    const int row0 = it * C::QB;
    kv_issue<D, NW>(ln, qb, dob, p.row_aug, rs, aug_row0, sentinel, row0, min(C::QB, Lq - row0),
                smem + C::OFF_Q + slot * C::QBUF, smem + C::OFF_DO + slot * C::QBUF,
                smem + C::OFF_AUG + slot * C::ABUF, wave, lane);
  };
  constexpr int COPIES = 2 * KvLane<D, NW>::Copy::J;
  int n = nq;
  JFA_LDS int* steps = (JFA_LDS int*)(smem + C::SMEM);
  bf16x8 pick_mask = ln.pick_s;
  if constexpr (SPARSE) {
    static_assert((kSparseKBlock * 2 == C::BN || kSparseKBlock == C::BN) && kSparseQBlock % C::QB == 0,
                  "sparse blocks vs dK/dV tiles");
    n = sparse_steps<C::QB, C::BN / kSparseKBlock>(p, b, h, j, L, nq, steps, wave, lane);
    // k-slot 2 (lanes 0-31) scales the row term's -1 by 1e30: S' -> -1e30, P = 0
    pick_mask[2] = lane < 32 ? (bf16)1e30f : (bf16)0.0f;
  }
  auto step_of = [&](int s) { return SPARSE ? (steps[s] & 0xFFFFFF) : s; };
  f32x16 dk[C::NDB], dv[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dk[db][i] = dv[db][i] = 0.f;
  // The ring's first copies go out before this wave's key rows are loaded, so that the
  // tile start waits out one memory round trip, not two.
  if (n > 0) {
    issue(step_of(0), 0);
    if constexpr (NS == 3) {
      if (n > 1) issue(step_of(1), 1);
    }
  }
  // This wave's keys as B operands, straight from global (rows past the end -> 0).
  bf16x8 kf[C::NKS], vf[C::NKS];
  {
    const int64_t base = (s0 + key0 + my_key) * rs + (int64_t)h * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
      // K pre-scaled by c = scale log2 e (rounded to bf16) so that S' = Q (cK)^T -
      // lse log2 e is already the base-2 exponent of P
      const bf16x8 kr = as_bf16x8(key_ok ? ld16(p.k + base + 16 * ks) : zero16());
#pragma unroll
      for (int e = 0; e < 8; ++e) kf[ks][e] = (bf16)((float)kr[e] * c);
      vf[ks] = as_bf16x8(key_ok ? ld16(p.v + base + 16 * ks) : zero16());
    }
  }
  if (n > 0) {
    // step 0 (and, with three slots, step 1) landed; older than the key-row loads
    wait_vmem();
    __syncthreads();
  }

  // Stored dS: this tile's blocks (j, 0 .. nq-1) and this lane's store offset.  A step's
  // dS is stored during the next step (see KvStream), the last one after the loop.  The
  // first step stores the zero-initialised registers into block 0, which the second
  // step (or the store after the loop) then overwrites -- stores of one lane to the
  // same address land in program order.
  bf16x8 keep[C::NQB][2];
  char* ds_row = nullptr;
  uint32_t ds_off = 0;
  if constexpr (STORE) {
    const int64_t nj = (L + C::BN - 1) / C::BN;
    ds_row = (char*)uniform_ptr(p.ds + (p.ds_base[b] + ((int64_t)h * nj + j) * nq) * kDsBlockBytes);
    ds_off = ds_store_offset(wave, lane);
#pragma unroll
    for (int qq = 0; qq < C::NQB; ++qq) keep[qq][0] = keep[qq][1] = as_bf16x8(zero16());
  }

  constexpr int AHEAD = NS - 1;  // steps a copy is issued ahead of its use
  for (int it = 0, cur = 0; it < n; ++it, cur = (cur == C::NS - 1 ? 0 : cur + 1)) {
    if (it + AHEAD < n) issue(step_of(it + AHEAD), cur == 0 ? C::NS - 1 : cur - 1);
    const JFA_LDS char* qt = smem + C::OFF_Q + cur * C::QBUF;
    const JFA_LDS char* dot = smem + C::OFF_DO + cur * C::QBUF;
    const JFA_LDS char* augt = smem + C::OFF_AUG + cur * C::ABUF;
    bool keep_keys = true;
    if constexpr (SPARSE && NW == kBwdWaves) keep_keys = ((steps[it] >> (24 + (wave >> 1))) & 1) != 0;
    KvStream<D, STORE, NW>(qt, dot, augt, ln, kf, vf, dk, dv, l32, c, keep,
                       ds_row + (int64_t)max(it - 1, 0) * kDsBlockBytes, ds_off, keep_keys ? ln.pick_s : pick_mask)
        .go();
    if constexpr (NS == 3) {
      if (it + 2 < n) wait_vmem_n<COPIES>();
      else wait_vmem();
    } else {
      wait_vmem();
    }
    __syncthreads();
  }
  if constexpr (STORE) store_ds(ds_row + (int64_t)(nq - 1) * kDsBlockBytes, ds_off, keep);

  if (key_ok) {
    const int64_t row = (s0 + key0 + my_key) * rs + (int64_t)h * D + 4 * half;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * db + 8 * g4;
        st8(p.dk + row + d, pack4(dk[db][4 * g4] * p.scale, dk[db][4 * g4 + 1] * p.scale,
                                  dk[db][4 * g4 + 2] * p.scale, dk[db][4 * g4 + 3] * p.scale));
        st8(p.dv + row + d, pack4(dv[db][4 * g4], dv[db][4 * g4 + 1], dv[db][4 * g4 + 2], dv[db][4 * g4 + 3]));
      }
  }
}

// Persistent tile loop shared by the kernels: static per-program lists, or (dynamic)
// groups of gsize consecutive programs, group g taking tiles seg_ptr[g] .. seg_ptr[g+1]
// first one each, then from its atomic counter counters[g].  xcd_gsize: the group size
// of a forward-rule schedule (one group per XCD, or one of all programs).
__device__ __forceinline__ int xcd_gsize() { return (int)gridDim.x / dynamic_groups((int)gridDim.x); }

template <class F>
__device__ __forceinline__ void tile_loop(const BwdParams& p, const Tile* tiles, const int32_t* seg_ptr,
                                          int32_t* counters, int gsize, int* next_tile, int32_t* visits, F&& body) {
  const int tid = threadIdx.x;
  const int prog = xcd_program_id(blockIdx.x, gridDim.x);
  const int grp = prog / gsize;
  int idx, end, base = 0;
  if (!p.dynamic) {
    idx = seg_ptr[prog];
    end = seg_ptr[prog + 1];
  } else {
    base = seg_ptr[grp];
    end = seg_ptr[grp + 1];
    idx = base + prog % gsize;
  }
  while (idx < end) {
    if (tid == 0) count_visit(visits, idx);
    body(tiles[idx]);
    if (!p.dynamic) {
      ++idx;
    } else {
      if (tid == 0) *next_tile = base + gsize + atomicAdd(counters + grp, 1);
      __syncthreads();
      idx = *next_tile;
      __syncthreads();
    }
  }
}

template <int D, bool SPARSE>
__global__ void __launch_bounds__(kDqWaves * 64)
    __attribute__((amdgpu_waves_per_eu(kDqWgPerCu * kDqWaves / 4, kDqWgPerCu * kDqWaves / 4)))
    dq_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(16))) char smem[4 * DqCfg<D>::BUF];
  __shared__ int next_tile;
  DqLane<D> ln;
  ln.row.init(threadIdx.x & 63);
  ln.ktr.init(threadIdx.x & 63);
  ln.copy.init((uint32_t)(p.num_heads * D * 2), threadIdx.x >> 6, threadIdx.x & 63);
  tile_loop(p, p.dq_tiles, p.dq_seg_ptr, p.counters + kDqCounter, xcd_gsize(), &next_tile, p.dq_visits,
            [&](Tile t) { dq_tile<D, SPARSE>(p, t, (JFA_LDS char*)smem, ln, threadIdx.x); });
}

// NW < kBwdWaves runs kBwdWaves / NW times as many workgroups per CU (same waves per SIMD).
template <int D, bool STORE, bool SPARSE, int NW = kBwdWaves, int NS = kBwdStages>
__global__ void __launch_bounds__(NW * 64)
    __attribute__((amdgpu_waves_per_eu(dkdv_wg_per_cu(D) * kBwdWaves / 4, dkdv_wg_per_cu(D) * kBwdWaves / 4)))
    dkdv_kernel(BwdParams p) {
  // SPARSE: the step list (kSparseMaxSteps entries + its length) follows the rings
  __shared__ __attribute__((aligned(16))) char smem[KvCfg<D, NW, NS>::SMEM + (SPARSE ? (kSparseMaxSteps + 1) * 4 : 0)];
  __shared__ int next_tile;
  KvLane<D, NW> ln;
  ln.row.init(threadIdx.x & 63);
  ln.tr.init(threadIdx.x & 63);
  ln.init_pick(threadIdx.x & 63);
  ln.copy.init((uint32_t)(p.num_heads * D * 2), threadIdx.x >> 6, threadIdx.x & 63);
  // broadcast-Q: head-pinned groups of programs_per_head programs
  tile_loop(p, p.tiles, p.seg_ptr, p.counters, p.bq ? p.programs_per_head : xcd_gsize(), &next_tile, p.visits,
            [&](Tile t) { dkdv_tile<D, STORE, SPARSE, NW, NS>(p, t, smem, ln, threadIdx.x); });
}

// ------------------------------- dK, dV: two waves per SIMD (self attention, head_dim 128)
//
// The products of dkdv_tile with two waves on every SIMD, so that one wave's waits on
// LDS data and matrix results are covered by the other's work.  A workgroup is 8 waves
// on one 128-key tile; waves w and w + 4 (one SIMD) own the same 32 keys, 32 (w & 3)
// .. + 31, and split every 64-row query step: wave group g = w / 4 takes rows
// 32 g .. 32 g + 31.  Each wave keeps fp32 dK^T, dV^T partials of its keys over its
// rows; at the end of the tile group 1 hands its partials to group 0 through LDS and
// group 0 stores the sums.  One wave's registers then hold only those partials, the
// scores and a few operands (no K, V rows): the K tile (pre-scaled by c = scale log2 e
// and rounded to bf16, as dkdv_tile does in registers) and the V tile stay in LDS for
// the whole tile and are read as the B operands of S' and dP'.  Q, dO and the row
// terms stream through a two-slot ring (copies one step ahead).  Per 32-row sub-step a
// wave runs one stream of 34 MFMAs
//   S' row term, S' k-steps | dP' row term, dP' k-steps | dV^T (u, db) | dK^T (u, db)
// with the LDS operands of each read AHEAD positions early, P = 2^S' formed during
// the dP' k-steps and dS = P dP' during the dV products (as KvStream).
template <int D>
struct Kv2Cfg {
  static constexpr int NW = 8;
  static constexpr int BN = 128;       // keys per tile (the backward schedule's kBwdKeys)
  static constexpr int QB = kBwdRows;  // query rows per step
  static constexpr int NKS = D / 16;
  static constexpr int NDB = D / 32;
  static constexpr int RB = 2 * D;
  static constexpr int KBUF = BN * RB;  // K or V tile
  static constexpr int QBUF = QB * RB;
  static constexpr int ABUF = QB * 16;
  // LDS: the two ring slots [Q | dO | row terms] first, so that every ring address is a
  // per-lane register plus an immediate below 64 KB; then the K and V tiles.
  static constexpr int SLOT = 2 * QBUF + ABUF;
  static constexpr int OFF_DO = QBUF, OFF_AUG = 2 * QBUF;
  static constexpr int OFF_K = 2 * SLOT, OFF_V = OFF_K + KBUF;
  static constexpr int SMEM = OFF_V + KBUF;
  // end of tile: group 1's partials, [dK | dV][key block][db][chunk][lane][4 floats]
  static constexpr int RED_ONE = 4 * NDB * 4 * 64 * 16;
  static_assert(BN == kBwdKeys && QB == 64, "tiles of the backward schedule, one 64-lane row-term copy");
  static_assert(2 * RED_ONE <= SMEM, "reduction buffer inside the tile's LDS");
  static_assert(SLOT + OFF_DO + 16 * RB + 256 <= 65536, "ring immediates (the largest: slot 1, dO, rows 16..) below 64 KB");
};

// Per-lane LDS byte offsets of one wave (its query rows 32 g .., its keys 32 kw ..
// folded in) and copy offsets.
template <int D>
struct Kv2Lane {
  using C = Kv2Cfg<D>;
  int qoff[C::NKS];        // row operand ks of the wave's 32 query rows (add a slot base, + OFF_DO for dO)
  int koff[C::NKS];        // row operand ks of the wave's 32 keys in the K tile (+ KBUF for V)
  int troff[C::NDB][2];    // transposed operand (db, half) of query rows 32 g .. (+ 16 u rows)
  int aoff;                // the row term of query row 32 g + l32
  TileCopy<C::RB, C::QB, 4> copy;   // a step's Q or dO rows (copied by the four waves of group 0)
  TileCopy<C::RB, C::BN, 8> kcopy;  // the tile's K or V rows
  bf16x8 pick_s, pick_dp;
  __device__ __forceinline__ void init(int wave, int lane, uint32_t row_stride_bytes) {
    const int g = wave >> 2, kw = wave & 3;
    RowOperands<C::RB, C::NKS> row;
    TrOperands<C::RB, C::NDB> tr;
    row.init(lane);
    tr.init(lane);
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
      qoff[ks] = 32 * g * C::RB + row.off[ks];
      koff[ks] = C::OFF_K + 32 * kw * C::RB + row.off[ks];
    }
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) troff[db][hi] = 32 * g * C::RB + tr.off[db][hi];
    aoff = C::OFF_AUG + (32 * g + (lane & 31)) * 16;
    copy.init(row_stride_bytes, wave & 3, lane);
    kcopy.init(row_stride_bytes, wave, lane);
    const bf16 one = (bf16)1.0f, zero = (bf16)0.0f;
    const bool lo = lane < 32;
    pick_s = bf16x8{lo ? one : zero, lo ? one : zero, zero, zero, zero, zero, zero, zero};
    pick_dp = bf16x8{zero, zero, zero, zero, lo ? one : zero, lo ? one : zero, zero, zero};
  }
};

// One 32-row sub-step of one wave, from ring slot SL, as a single MFMA stream
// (positions 0 .. N-1).
template <int D, bool STORE, int AHEAD, int SL>
struct Kv2Stream {
  using C = Kv2Cfg<D>;
  static constexpr int NKS = C::NKS, NDB = C::NDB;
  static constexpr int S0 = 0, DP0 = NKS + 1, DV0 = 2 * NKS + 2, DK0 = DV0 + 2 * NDB, N = DK0 + 2 * NDB;
  static constexpr int NBUF = AHEAD + 1;
  static constexpr int P_PER = 16 / NKS;          // P values per dP' k-step
  static constexpr int DS_SL = 2 * NDB - 2;       // dS slices: dV positions 2 .. 2 NDB - 1
  static constexpr int DS_PER = (16 + DS_SL - 1) / DS_SL;
  static constexpr int ST0 = DK0 + 1, ST1 = DK0 + 3;  // dS store positions (STORE)
  static constexpr int BASE = SL * C::SLOT;

  const JFA_LDS char* lds;
  const Kv2Lane<D>& ln;
  f32x16 (&dk)[NDB];
  f32x16 (&dv)[NDB];
  char* sblk;            // STORE: this step's dS block (wave-uniform)
  uint32_t soff;         // STORE: this lane's store offset
  const int qq;          // STORE: query block of the 64-row step (the wave group)
  bf16x8 a[NBUF], b[NBUF];
  bf16x8 term;
  f32x16 s, dp;
  float pr[16], dsr[16];
  bf16x8 pf[2], dsf[2];

  __device__ __forceinline__ Kv2Stream(const JFA_LDS char* lds_, const Kv2Lane<D>& ln_, f32x16 (&dk_)[NDB],
                                       f32x16 (&dv_)[NDB], char* sblk_, uint32_t soff_, int qq_)
      : lds(lds_), ln(ln_), dk(dk_), dv(dv_), sblk(sblk_), soff(soff_), qq(qq_) {}

  __device__ __forceinline__ bf16x8 rd(int reg_off, int imm) const { return as_bf16x8(lds_ld16(lds + imm, reg_off)); }
  __device__ __forceinline__ bf16x8 rd_tr(int db, int imm) const {
    return join_tr(lds_tr4(lds + imm, ln.troff[db][0]), lds_tr4(lds + imm, ln.troff[db][1]));
  }

  template <int K>
  __device__ __forceinline__ void read() {
    constexpr int i = K % NBUF;
    if constexpr (K == S0) {
      a[i] = rd(ln.aoff, BASE);
    } else if constexpr (K < DP0) {
      a[i] = rd(ln.qoff[K - 1], BASE);
      b[i] = rd(ln.koff[K - 1], 0);
    } else if constexpr (K == DP0) {
    } else if constexpr (K < DV0) {
      a[i] = rd(ln.qoff[K - DP0 - 1], BASE + C::OFF_DO);
      b[i] = rd(ln.koff[K - DP0 - 1], C::KBUF);
    } else if constexpr (K < DK0) {
      constexpr int u = (K - DV0) / NDB, db = (K - DV0) % NDB;
      a[i] = rd_tr(db, BASE + C::OFF_DO + 16 * u * C::RB);
    } else {
      constexpr int u = (K - DK0) / NDB, db = (K - DK0) % NDB;
      a[i] = rd_tr(db, BASE + 16 * u * C::RB);
    }
  }
  template <int K>
  static constexpr int reads() {
    return K == S0 ? 1 : (K < DP0 ? 2 : (K == DP0 ? 0 : 2));
  }

  template <int K>
  __device__ __forceinline__ void mfma() {
    constexpr int i = K % NBUF;
    if constexpr (K == S0) {
      term = a[i];
      s = mfma32(term, ln.pick_s, f32x16{});
    } else if constexpr (K < DP0) {
      s = mfma32(a[i], b[i], s);
    } else if constexpr (K == DP0) {
      dp = mfma32(term, ln.pick_dp, f32x16{});
    } else if constexpr (K < DV0) {
      dp = mfma32(a[i], b[i], dp);
    } else if constexpr (K < DK0) {
      constexpr int u = (K - DV0) / NDB, db = (K - DV0) % NDB;
      dv[db] = mfma32(a[i], pf[u], dv[db]);
    } else {
      constexpr int u = (K - DK0) / NDB, db = (K - DK0) % NDB;
      dk[db] = mfma32(a[i], dsf[u], dk[db]);
    }
  }

  template <int K>
  __device__ __forceinline__ void valu() {
    if constexpr (K >= DP0 + 1 && K < DV0) {
      constexpr int j = K - DP0 - 1;
#pragma unroll
      for (int e = 0; e < P_PER; ++e) pr[j * P_PER + e] = fast_exp2(s[j * P_PER + e]);
      if constexpr ((j + 1) * P_PER == 8) pf[0] = pack8(pr[0], pr[1], pr[2], pr[3], pr[4], pr[5], pr[6], pr[7]);
      if constexpr ((j + 1) * P_PER == 16)
        pf[1] = pack8(pr[8], pr[9], pr[10], pr[11], pr[12], pr[13], pr[14], pr[15]);
    } else if constexpr (K >= DV0 + 2 && K < DK0) {
      constexpr int j = K - DV0 - 2;
#pragma unroll
      for (int e = 0; e < DS_PER; ++e) {
        const int x = j * DS_PER + e;
        if (x < 16) dsr[x] = pr[x] * dp[x];
      }
      if constexpr ((j + 1) * DS_PER >= 8 && j * DS_PER < 8)
        dsf[0] = pack8(dsr[0], dsr[1], dsr[2], dsr[3], dsr[4], dsr[5], dsr[6], dsr[7]);
      if constexpr (j == DS_SL - 1) dsf[1] = pack8(dsr[8], dsr[9], dsr[10], dsr[11], dsr[12], dsr[13], dsr[14], dsr[15]);
    }
  }
  template <int K>
  static constexpr int valus() {
    if (K >= DP0 + 1 && K < DV0) return 2 * P_PER + ((K - DP0) * P_PER % 8 == 0 ? 4 : 0);
    if (K >= DV0 + 2 && K < DK0) return DS_PER + 2;
    return 0;
  }

  template <int K>
  __device__ __forceinline__ void store() {
    if constexpr (STORE && (K == ST0 || K == ST1)) store_ds_unit(sblk, soff, qq, K == ST0 ? 0 : 1, dsf[K == ST0 ? 0 : 1]);
  }

  template <int K>
  __device__ __forceinline__ void order() {
    if constexpr (K == 0) {
      constexpr int r0 = reads<0>() + (AHEAD > 1 ? reads<1>() : 0) + (AHEAD > 2 ? reads<2>() : 0) +
                         (AHEAD > 3 ? reads<3>() : 0);
      __builtin_amdgcn_sched_group_barrier(0x100, r0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (valus<K>() > 0) __builtin_amdgcn_sched_group_barrier(0x002, valus<K>(), 0);
    if constexpr (K + AHEAD < N && reads<K + AHEAD>() > 0)
      __builtin_amdgcn_sched_group_barrier(0x100, reads<K + AHEAD>(), 0);
    if constexpr (STORE && (K == ST0 || K == ST1)) __builtin_amdgcn_sched_group_barrier(0x040, 1, 0);
  }

  template <int K>
  __device__ __forceinline__ void step() {
    mfma<K>();
    valu<K>();
    if constexpr (K + AHEAD < N) read<K + AHEAD>();
    store<K>();
  }
  __device__ __forceinline__ void go() {
    static_assert(AHEAD >= 1 && AHEAD <= 4, "read-ahead window");
    prologue(std::make_integer_sequence<int, AHEAD>{});
    body(std::make_integer_sequence<int, N>{});
    orders(std::make_integer_sequence<int, N>{});
    __builtin_amdgcn_sched_barrier(0);
  }
  template <int... K>
  __device__ __forceinline__ void prologue(std::integer_sequence<int, K...>) { (read<K>(), ...); }
  template <int... K>
  __device__ __forceinline__ void body(std::integer_sequence<int, K...>) { (step<K>(), ...); }
  template <int... K>
  __device__ __forceinline__ void orders(std::integer_sequence<int, K...>) { (order<K>(), ...); }
};

// MFMA positions an LDS operand is read ahead of its use (the recompute variant, with
// no dS stores to keep, runs out of registers at 3).
template <bool STORE>
constexpr int kv2_ahead() { return STORE ? 3 : 2; }

// Row stores of one gradient per thread (a 128-key tile of 16-byte chunks over the
// eight waves) and per tile (dK, then dV), at the end of a dK/dV tile.
template <int D>
constexpr int kv2_store_passes() { return Kv2Cfg<D>::BN * Kv2Cfg<D>::RB / 16 / (Kv2Cfg<D>::NW * 64); }
template <int D>
constexpr int kv2_stores() { return 2 * kv2_store_passes<D>(); }

// Geometry of one dK/dV tile.
struct Kv2Tile {
  int h, j, L, key0, keys, n;
  int64_t s0, b;
};

// Tile idx (wave-uniform) of the list, through scalar loads: at the end of a tile a
// vector load would wait for the last step's dS stores.
template <int D>
__device__ __forceinline__ Kv2Tile kv2_tile_at(const BwdParams& p, int idx) {
  using C = Kv2Cfg<D>;
  const Tile t = ld_uniform(p.tiles, __builtin_amdgcn_readfirstlane(idx));
  Kv2Tile x;
  x.b = t.b;
  x.h = t.hb >> 24;
  x.j = t.hb & 0xFFFFFF;
  x.s0 = ld_uniform(p.offsets, t.b);
  x.L = ld_uniform(p.offsets, t.b + 1) - (int)x.s0;
  x.key0 = x.j * C::BN;
  x.keys = min(C::BN, x.L - x.key0);
  x.n = (x.L + C::QB - 1) / C::QB;
  return x;
}

// Copies of query step `it` of tile x into ring slot `slot`: Q and dO rows (the four
// waves of group 0; rows past the sequence repeat its last row) and the row terms
// (wave 0; rows past the sequence take the sentinel term, P = dS = 0).
template <int D>
__device__ __forceinline__ void kv2_issue_step(const BwdParams& p, const Kv2Lane<D>& ln, const Kv2Tile& x, int it,
                                               int slot, JFA_LDS char* smem, int wave, int lane) {
  using C = Kv2Cfg<D>;
  if (wave >= 4) return;
  const int64_t rs = (int64_t)p.num_heads * D;
  const uint32_t rsb = (uint32_t)(rs * 2);
  JFA_LDS char* base = smem + slot * C::SLOT;
  const int row0 = it * C::QB, rv = min(C::QB, x.L - row0);
  const int64_t first = (x.s0 + row0) * rs + (int64_t)x.h * D;
  ln.copy.issue_rows(p.q + first, rsb, rv, base, wave, lane);
  ln.copy.issue_rows(p.dout + first, rsb, rv, base + C::OFF_DO, wave, lane);
  if (wave == 0) {
    const int64_t r = lane < rv ? (int64_t)x.h * p.total_tokens + x.s0 + row0 + lane
                                : (int64_t)p.num_heads * p.total_tokens;
    dma16(uniform_ptr(p.row_aug), (uint32_t)(r * 16), base + C::OFF_AUG);
  }
}

// K, V rows of tile x (all eight waves; rows past the sequence repeat its last row:
// their dK, dV are not stored and their stored dS is masked by the dQ kernel).
template <int D>
__device__ __forceinline__ void kv2_issue_kv(const BwdParams& p, const Kv2Lane<D>& ln, const Kv2Tile& x,
                                             JFA_LDS char* smem, int wave, int lane) {
  using C = Kv2Cfg<D>;
  const int64_t rs = (int64_t)p.num_heads * D;
  const uint32_t rsb = (uint32_t)(rs * 2);
  const int64_t first = (x.s0 + x.key0) * rs + (int64_t)x.h * D;
  ln.kcopy.issue_rows(p.k + first, rsb, x.keys, smem + C::OFF_K, wave, lane);
  ln.kcopy.issue_rows(p.v + first, rsb, x.keys, smem + C::OFF_V, wave, lane);
}

// Persistent loop over the dK/dV tiles.  The next tile is reserved one tile ahead, so
// that its K, V rows and first query step are copied while the current tile sums its
// two groups' partials (which then use only ring slot 0; every tile starts its steps
// in slot 1).
template <int D, bool STORE>
__global__ void __launch_bounds__(Kv2Cfg<D>::NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
    dkdv2_kernel(BwdParams p) {
  using C = Kv2Cfg<D>;
  __shared__ __attribute__((aligned(16))) char smem_raw[C::SMEM];
  __shared__ int next_tile;
  JFA_LDS char* smem = (JFA_LDS char*)smem_raw;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = wave >> 2, kw = wave & 3;
  const int64_t rs = (int64_t)p.num_heads * D;
  const float c = p.scale_log2;
  Kv2Lane<D> ln;
  ln.init(wave, lane, (uint32_t)(rs * 2));

  const int prog = xcd_program_id(blockIdx.x, gridDim.x);
  const int gsize = xcd_gsize(), grp = prog / gsize;
  int idx, end, base = 0;
  if (!p.dynamic) {
    idx = p.seg_ptr[prog];
    end = p.seg_ptr[prog + 1];
  } else {
    base = p.seg_ptr[grp];
    end = p.seg_ptr[grp + 1];
    idx = base + prog % gsize;
  }
  if (idx >= end) return;
  Kv2Tile x = kv2_tile_at<D>(p, idx);
  kv2_issue_kv<D>(p, ln, x, smem, wave, lane);
  kv2_issue_step<D>(p, ln, x, 0, 1, smem, wave, lane);
  // set once a tile's dK, dV row stores were issued (kv2_stores() per wave, after the
  // next tile's copies)
  int stores = 0;
  while (true) {
    // reserve the next tile
    int nxt = idx + 1;
    if (p.dynamic) {
      if (tid == 0) next_tile = base + gsize + atomicAdd(p.counters + grp, 1);
      __syncthreads();
      nxt = next_tile;
    }
    if (tid == 0) count_visit(p.visits, idx);
    // this tile's K, V and first step have landed (the previous tile's dK, dV row
    // stores, issued after them, may still be in flight)
    if (stores) wait_vmem_upto<kv2_stores<D>()>();
    else wait_vmem();
    __syncthreads();
    {
      // K *= c, rounded to bf16 (elementwise, so the swizzle does not matter)
      constexpr int PASSES = C::KBUF / (C::NW * 64 * 16);
      JFA_LDS char* kt = smem + C::OFF_K;
#pragma unroll
      for (int ps = 0; ps < PASSES; ++ps) {
        const int off = ((ps * C::NW + wave) * 64 + lane) * 16;
        const bf16x8 xv = as_bf16x8(lds_ld16(kt, off));
        bf16x8 y;
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = (bf16)((float)xv[e] * c);
        lds_st16(kt, off, __builtin_bit_cast(u32x4, y));
      }
    }
    __syncthreads();

    f32x16 dk[C::NDB], dv[C::NDB];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) dk[db][i] = dv[db][i] = 0.f;
    char* ds_row = nullptr;
    uint32_t ds_off = 0;
    if constexpr (STORE) {
      const int64_t nj = (x.L + C::BN - 1) / C::BN;
      ds_row = (char*)uniform_ptr(p.ds + (p.ds_base[x.b] + ((int64_t)x.h * nj + x.j) * x.n) * kDsBlockBytes);
      ds_off = ds_store_offset(kw, lane);
    }
    // Step it reads slot (it + 1) & 1 (compile time, so that every LDS address is a lane
    // register plus an immediate); the next step's copies go to the other slot first.
    // A wave whose 32 keys all lie past the end (in a sequence's last key tile) runs the
    // same copies, waits and barriers without its streams: fewer LDS reads for the other
    // waves of the step.  (Its dS rows are not stored: the dQ kernel masks keys past the
    // end.)  Two instances of the step loop, so that no branch sits inside it.
    auto one_step = [&](auto slot_tag, auto active_tag, int it) {
      constexpr int SL = decltype(slot_tag)::value;
      constexpr bool ACTIVE = decltype(active_tag)::value;
      if (it + 1 < x.n) kv2_issue_step<D>(p, ln, x, it + 1, SL ^ 1, smem, wave, lane);
      if constexpr (ACTIVE)
        Kv2Stream<D, STORE, kv2_ahead<STORE>(), SL>(smem, ln, dk, dv, ds_row + (int64_t)it * kDsBlockBytes, ds_off, g)
            .go();
      // group 0's next-step copies were issued before this step's two dS stores; loads
      // and stores complete in issue order, so waiting for all but those two suffices
      if (STORE && ACTIVE) wait_vmem_n<2>();
      else wait_vmem();
      __syncthreads();
    };
    auto steps = [&](auto active_tag) {
      for (int it = 0; it < x.n; it += 2) {
        one_step(std::integral_constant<int, 1>{}, active_tag, it);
        if (it + 1 < x.n) one_step(std::integral_constant<int, 0>{}, active_tag, it + 1);
      }
    };
    if (32 * kw < x.keys) steps(std::true_type{});
    else steps(std::false_type{});

    // Prefetch the next tile (K, V tiles and ring slot 1 are free now).
    const bool more = nxt < end;
    Kv2Tile y = x;
    if (more) {
      y = kv2_tile_at<D>(p, nxt);
      kv2_issue_kv<D>(p, ln, y, smem, wave, lane);
      kv2_issue_step<D>(p, ln, y, 0, 1, smem, wave, lane);
    }
    // The groups swap partials through ring slot 0, a quarter at a time: group 1 hands
    // its dK partials to group 0 (parts 0, 1: head-dim blocks 0-1, 2-3) and group 0 its
    // dV partials to group 1 (parts 2, 3); group 0 then holds the tile's dK, group 1 dV.
    {
      JFA_LDS char* red = smem;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int giver = r < 2 ? 1 : 0;
        f32x16(&acc)[C::NDB] = r < 2 ? dk : dv;
        if (g == giver) {
#pragma unroll
          for (int dl = 0; dl < 2; ++dl)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const f32x16& a = acc[2 * (r & 1) + dl];
              lds_st16(red, ((kw * 2 + dl) * 4 + q4) * 1024 + lane * 16,
                       __builtin_bit_cast(u32x4, float4{a[4 * q4], a[4 * q4 + 1], a[4 * q4 + 2], a[4 * q4 + 3]}));
            }
        }
        __syncthreads();
        if (g != giver) {
#pragma unroll
          for (int dl = 0; dl < 2; ++dl)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              f32x16& a = acc[2 * (r & 1) + dl];
              const float4 v4 = __builtin_bit_cast(float4, lds_ld16(red, ((kw * 2 + dl) * 4 + q4) * 1024 + lane * 16));
              a[4 * q4] += v4.x;
              a[4 * q4 + 1] += v4.y;
              a[4 * q4 + 2] += v4.z;
              a[4 * q4 + 3] += v4.w;
            }
        }
        __syncthreads();
      }
    }
    // Stores: group 0's dK (times scale), then group 1's dV, go as bf16 rows through ring
    // slot 0 ([key][D], rows RB + 8 bytes apart, so that the 32 keys of one write land in
    // distinct banks), and all eight waves write whole rows with 16-byte stores (16 lanes
    // per 256-byte row) instead of every lane writing 8-byte pieces of its own key's row.
    // Rows past the tile's keys repeat its last row (same address, same value), so every
    // wave issues kv2_stores() stores.
    {
      constexpr int PITCH = C::RB + 8;
      static_assert(C::BN * PITCH <= C::SLOT, "staging rows inside ring slot 0");
      JFA_LDS char* stg = smem;
      // lane-dependent offsets from an opaque copy of the thread id, computed here: hoisted
      // out of the tile loop they would stay live through the steps and spill
      int tl = tid;
      asm volatile("" : "+v"(tl));
      const int wbase = (32 * ((tl >> 6) & 3) + (tl & 31)) * PITCH + 8 * ((tl >> 5) & 1);
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        if (g == r) {
          const f32x16(&a)[C::NDB] = r == 0 ? dk : dv;
          const float sc = r == 0 ? p.scale : 1.0f;
#pragma unroll
          for (int db = 0; db < C::NDB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4)
              lds_st8(stg + 64 * db + 16 * g4, wbase,
                      pack4(a[db][4 * g4] * sc, a[db][4 * g4 + 1] * sc, a[db][4 * g4 + 2] * sc, a[db][4 * g4 + 3] * sc));
        }
        __syncthreads();
        uint16_t* dst = (r == 0 ? p.dk : p.dv) + (x.s0 + x.key0) * rs + (int64_t)x.h * D;
#pragma unroll
        for (int k = 0; k < kv2_store_passes<D>(); ++k) {
          const int q = tl + C::NW * 64 * k;
          const int row = min(q / (C::RB / 16), x.keys - 1), cc = q % (C::RB / 16);
          const int ro = row * PITCH + 16 * cc;
          const u32x2 lo = lds_ld8(stg, ro), hi = lds_ld8(stg, ro + 8);
          st16(dst + (int64_t)row * rs + 8 * cc, u32x4{lo[0], lo[1], hi[0], hi[1]});
        }
        __syncthreads();
      }
    }
    stores = 1;
    if (!more) break;
    idx = nxt;
    x = y;
  }
}

// --------------------------------------------------------- stored-dS path: row terms

// Row terms for the dK/dV kernel when no dQ kernel runs before it: D/8 lanes per (token,
// head) row load 16 bytes each of O and dO, Di = rowsum(dO * O) in fp32, and the row's
// group leader writes (-lse log2 e, -Di) as bf16 high + low parts, the same 16-byte term
// as dq_tile.  Block 0 writes the sentinel term.
template <int D>
__global__ void __launch_bounds__(256) prep_kernel(BwdParams p) {
  constexpr int LPR = D / 8;
  constexpr int RPB = 256 / LPR;
  const int64_t H = p.num_heads, T = p.total_tokens;
  const int64_t rows = T * H;
  const int sub = threadIdx.x % LPR;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    const bf16 z = (bf16)0.0f;
    const bf16x8 t = {(bf16)(-1e30f), z, (bf16)(-1.0f), z, z, z, z, z};
    st16(p.row_aug + H * T * 8, __builtin_bit_cast(u32x4, t));
  }
  for (int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR; r < rows; r += (int64_t)gridDim.x * RPB) {
    const bf16x8 o8 = as_bf16x8(ld16_nt(p.o + r * D + 8 * sub));
    const bf16x8 d8 = as_bf16x8(ld16_nt(p.dout + r * D + 8 * sub));
    float di = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) di = fmaf((float)d8[e], (float)o8[e], di);
#pragma unroll
    for (int m = LPR / 2; m > 0; m >>= 1) di += __shfl_xor(di, m, LPR);
    if (sub == 0) {
      const int64_t t = r / H, h = r - t * H;
      st16(p.row_aug + (h * T + t) * 8, __builtin_bit_cast(u32x4, row_term(p.lse[h * T + t], di)));
    }
  }
}

// ---------------------------------------------------------- stored-dS path: dQ = dS K

// dQ = scale dS K from the stored dS: one workgroup = kDsRows (256) query rows of one
// (sequence, head).  Waves 2c and 2c+1 share stored block column it = 4 blk + c (64
// query rows) and each owns one 32-row column block of fp32 dQ^T accumulators; two
// waves per SIMD keep more copies in flight and hide the LDS latency (measured 4.6
// against 3.6 TB/s with one wave of 64 rows per SIMD).  The loop streams 64 keys at a
// time (half of a stored block) through a three-slot LDS ring: the K rows (swizzled
// tile, shared by the waves) and each block column's 8 KB dS slice (each wave copies
// the half with its column block).  Per 16-key k-step: dQ^T += K^T dS^T with A = K^T
// (transposed fetch of the K tile) and B = dS^T (transposed fetch of the slice, 4 keys
// x 16 queries per 16-lane group).  The kernel moves two bytes of dS per (query, key)
// pair for 2 D flops, so HBM, not the matrix unit, bounds it.
template <int D>
struct DsCfg {
  static constexpr int NW = kDsWaves;                    // two waves per stored block column
  static constexpr int BM = kDsRows;
  static constexpr int BK = 64;                          // keys per step
  static constexpr int NDB = D / 32;
  static constexpr int RB = 2 * D;
  static constexpr int KBUF = BK * RB;                   // K rows of a step
  static constexpr int SLICE = kDsBlockBytes / 2;        // one wave's dS: 64 keys x 64 queries
  static constexpr int STAGE = KBUF + (NW / 2) * SLICE;
  static constexpr int NS = 3;
  static constexpr int SMEM = NS * STAGE;
  using Copy = TileCopy<RB, BK, NW>;
  static constexpr int SLICE_COPIES = SLICE / 1024 / 2;  // each wave copies its column block's half
  static_assert(BK * 2 == kBwdKeys && kBwdRows == 64 && BM == (NW / 2) * kBwdRows, "slices are halves of stored blocks");
};

template <int D>
struct DsLane {
  TrOperands<DsCfg<D>::RB, DsCfg<D>::NDB> ktr;  // K^T as the A operand
  typename DsCfg<D>::Copy copy;
  int boff[2][2];  // dS^T fetch offsets by (k-step parity, upper 8 keys)
  __device__ __forceinline__ void init(int lane) {
    // Source lane (group g16, s16) of a transposed fetch points at key
    // 16t + 8hi + 4(g16 >> 1) + (s16 >> 2) and the query quad 16(g16 & 1) + 4(s16 & 3) of
    // column block cb; in stored-block terms that is row r = 16(t & 1) + 8hi +
    // 4(g16 >> 1) + (s16 >> 2) of key group w = t >> 1, quad x = g16 & 1,
    // y = (s16 >> 1) & 1, e = s16 & 1.
    const int g16 = lane >> 4, s16 = lane & 15;
    const int x = g16 & 1, y = (s16 >> 1) & 1, e = s16 & 1;
#pragma unroll
    for (int tl = 0; tl < 2; ++tl)
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const int r = 16 * tl + 8 * hi + 4 * (g16 >> 1) + (s16 >> 2);
        boff[tl][hi] = x * 1024 + 16 * (32 * e + (r ^ (8 * x + 4 * e))) + 8 * y;
      }
  }
  // B operand of k-step t (keys 16t .. 16t+15 of the step) for column block cb.
  __device__ __forceinline__ bf16x8 ds(const JFA_LDS char* slice, int t, int cb) const {
    const int c = 4096 * (t >> 1) + 2048 * cb;
    return join_tr(lds_tr4(slice, boff[t & 1][0] + c), lds_tr4(slice, boff[t & 1][1] + c));
  }
};

// Zero the B slots of keys >= keys_valid (the tail step of a sequence): slot j of a lane
// in half `half` is key 16t + 8(j/4) + 4 half + j%4; the stored dS of keys past the end
// is not meaningful (the dK/dV kernel computes it from zero K, V rows).
__device__ __forceinline__ bf16x8 mask_keys(const bf16x8& b, int t, int half, int keys_valid) {
  u32x4 u = __builtin_bit_cast(u32x4, b);
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int k0 = 16 * t + 8 * (m >> 1) + 4 * half + 2 * (m & 1);
    const uint32_t keep = (k0 < keys_valid ? 0x0000FFFFu : 0u) | (k0 + 1 < keys_valid ? 0xFFFF0000u : 0u);
    u[m] &= keep;
  }
  return __builtin_bit_cast(bf16x8, u);
}

// One 64-key step (MASK: the tail step of a sequence, keys past keys_valid zeroed).
template <int D, bool MASK>
__device__ __forceinline__ void dq_ds_step(const JFA_LDS char* kbuf, const JFA_LDS char* slice, const DsLane<D>& ln,
                                           f32x16 (&acc)[DsCfg<D>::NDB], int half, int keys_valid, int cb) {
  using C = DsCfg<D>;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    bf16x8 b0 = ln.ds(slice, t, cb);
    if (MASK) b0 = mask_keys(b0, t, half, keys_valid);
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) acc[db] = mfma32(ln.ktr.read(kbuf, 16 * t, db), b0, acc[db]);
  }
}

// Geometry of one dQ tile as one wave sees it (all wave-uniform), from scalar loads of
// the tile list and the sequence tables.
template <int D>
struct DsGeo {
  using C = DsCfg<D>;
  // (no padding bytes: a copy of a struct with padding kept those bytes in memory)
  int64_t s0;
  const uint16_t* kp;     // K rows of the sequence, head h
  const char* ds_col;     // block (j, it) of this (b, h) is at ds_col + j * nq blocks
  int L, nq, nkb, h, blk;
  int live;               // this wave's stored block column has rows (rows past the end only)
  __device__ __forceinline__ void init(const BwdParams& p, int idx, int wave) {
    const Tile t = ld_uniform(p.dq_tiles, __builtin_amdgcn_readfirstlane(idx));
    const int b = t.b;
    h = t.hb >> 24;
    blk = t.hb & 0xFFFFFF;
    s0 = ld_uniform(p.offsets, b);
    L = ld_uniform(p.offsets, b + 1) - (int)s0;
    nq = (L + kBwdRows - 1) / kBwdRows;
    const int nj = (L + kBwdKeys - 1) / kBwdKeys;
    const int it = blk * (C::BM / kBwdRows) + (wave >> 1);  // this wave's stored block column
    live = it < nq ? 1 : 0;
    nkb = (L + C::BK - 1) / C::BK;
    const int64_t rs = (int64_t)p.num_heads * D;
    kp = p.k + s0 * rs + (int64_t)h * D;
    ds_col = p.ds + (ld_uniform(p.ds_base, b) + (int64_t)h * nj * nq + it) * kDsBlockBytes;
  }
  // vector-memory instructions one wave issues for one step
  __device__ __forceinline__ int step_copies() const { return C::Copy::J + (live ? C::SLICE_COPIES : 0); }
};

// s_waitcnt vmcnt(m) for the largest even m <= n (n < 16): at most n of the wave's
// vector-memory instructions stay outstanding (fewer is never wrong).
__device__ __forceinline__ void wait_vmem_le(int n) {
  if (n >= 14) wait_vmem_n<14>();
  else if (n >= 12) wait_vmem_n<12>();
  else if (n >= 10) wait_vmem_n<10>();
  else if (n >= 8) wait_vmem_n<8>();
  else if (n >= 6) wait_vmem_n<6>();
  else if (n >= 4) wait_vmem_n<4>();
  else if (n >= 2) wait_vmem_n<2>();
  else wait_vmem();
}

// Persistent loop of the dQ-from-dS kernel.  The next tile is reserved one tile ahead
// (static list or run-time counter) and its first two steps are copied during the
// current tile's last two steps, into the ring slots that follow (the ring runs on
// across tiles), so a tile start waits for no memory round trip.  The tile's dQ rows go
// out through LDS (two halves of 128 rows, each in the ring slot the last step freed)
// as whole 16-byte row pieces, instead of each lane writing 8-byte pieces of its own
// row.  Waits count exactly the wave's vector-memory instructions issued after the step
// that must have landed (copies of later steps, the previous tile's dQ stores).
template <int D>
__global__ void __launch_bounds__(kDsWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
    dq_ds_kernel(BwdParams p) {
  using C = DsCfg<D>;
  __shared__ __attribute__((aligned(16))) char smem_raw[C::SMEM];
  __shared__ int next_tile;
  JFA_LDS char* smem = (JFA_LDS char*)smem_raw;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int pair = wave >> 1, cb = wave & 1;
  const int64_t rs = (int64_t)p.num_heads * D;
  const uint32_t rsb = (uint32_t)(rs * 2);
  DsLane<D> ln;
  ln.ktr.init(lane);
  ln.copy.init(rsb, wave, lane);
  ln.init(lane);

  const int prog = xcd_program_id(blockIdx.x, gridDim.x);
  const int gsize = xcd_gsize(), grp = prog / gsize;
  int idx, end, base = 0;
  if (!p.dynamic) {
    idx = p.dq_seg_ptr[prog];
    end = p.dq_seg_ptr[prog + 1];
  } else {
    base = p.dq_seg_ptr[grp];
    end = p.dq_seg_ptr[grp + 1];
    idx = base + prog % gsize;
  }
  if (idx >= end) return;

  constexpr int LAST = (C::NS - 1) * C::STAGE;
  auto adv = [](int off) { return off == LAST ? 0 : off + C::STAGE; };
  // Step kb of a tile (its K rows kp, L keys, dS column ds_col of nq blocks, live:
  // this wave copies dS) into the ring slot at byte offset off.  (Fields passed by value:
  // a reference chosen at run time between two tiles' geometries would put them in
  // scratch memory.)
  auto issue = [&](const uint16_t* kp, int L, int live, const char* ds_col, int nq, int kb, int off) {
    JFA_LDS char* st = smem + off;
    ln.copy.issue_rows(kp + (int64_t)kb * C::BK * rs, rsb, min(C::BK, L - kb * C::BK), st, wave, lane);
    if (live) {
      const void* src = uniform_ptr(ds_col + ((int64_t)(kb >> 1) * nq * kDsBlockBytes + (kb & 1) * C::SLICE));
      JFA_LDS char* dst = st + C::KBUF + pair * C::SLICE;
#pragma unroll
      for (int w2 = 0; w2 < 2; ++w2)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int o = w2 * 4096 + cb * 2048 + c * 1024;
          dma16_nt(src, (uint32_t)(o + lane * 16), dst + o);  // dS is read once
        }
    }
  };

  // Steps are numbered in one sequence across tiles: the current tile's steps 0 .. nkb - 1,
  // then the next tile's.  Position kb + 2 is copied at the start of step kb (ring slot
  // of position q: q mod NS); the next tile's steps from 2 on are copied by its own loop.
  DsGeo<D> cur;
  cur.init(p, idx, wave);
  if (p.dynamic && tid == 0) next_tile = base + gsize + atomicAdd(p.counters + kDqCounter + grp, 1);
  int cur_off = 0, iss_off = 0;
  int issued = 0;      // positions copied so far (relative to the current tile's step 0)
  int last_copies = 0; // the wave's copy instructions of position issued - 1
  int stores_at = -1;  // the previous tile's dQ stores were issued after position stores_at
  int stores = 0;      // ... and their number
  issue(cur.kp, cur.L, cur.live, cur.ds_col, cur.nq, 0, iss_off);
  iss_off = adv(iss_off);
  issued = 1;
  last_copies = cur.step_copies();
  if (cur.nkb > 1) {
    issue(cur.kp, cur.L, cur.live, cur.ds_col, cur.nq, 1, iss_off);
    iss_off = adv(iss_off);
    issued = 2;
  }
  wait_vmem_le(issued == 2 ? last_copies : 0);  // position 0 has landed
  __syncthreads();

  while (true) {
    if (tid == 0) count_visit(p.dq_visits, idx);
    const int nidx = p.dynamic ? next_tile : idx + 1;  // written before the barrier above
    const bool more = nidx < end;
    DsGeo<D> nx = cur;
    if (more) nx.init(p, nidx, wave);
    // reserve the tile after the next one now (every wave has read next_tile); its
    // number goes to next_tile before the tile's last barrier, so that the atomic's round
    // trip overlaps the whole tile
    // (the raw counter value, set and read under the same condition: no copy of it at
    // the branch join, which would wait for the atomic right away)
    const bool reserve = more && p.dynamic && tid == 0;
    int ticket;
    if (reserve) ticket = atomicAdd(p.counters + kDqCounter + grp, 1);
    const int limit = cur.nkb + (more ? min(2, nx.nkb) : 0);  // positions this tile's loop copies

    f32x16 acc[C::NDB];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

    // Full steps in the loop, the tail step (if any) after it: one instruction path per
    // loop body, so the accumulators stay in the same registers from step to step (a
    // full / tail branch inside the body made the compiler copy all 64 accumulator
    // registers out and back at every step).
    auto step = [&](int kb, auto mask) {
      // copy positions up to kb + 2 (two at a tile's first step when its predecessor
      // could copy only one)
      for (int rep = 0; rep < 2 && issued <= kb + 2 && issued < limit; ++rep) {
        const bool in_cur = issued < cur.nkb;
        issue(in_cur ? cur.kp : nx.kp, in_cur ? cur.L : nx.L, in_cur ? cur.live : nx.live,
              in_cur ? cur.ds_col : nx.ds_col, in_cur ? cur.nq : nx.nq, in_cur ? issued : issued - cur.nkb, iss_off);
        last_copies = in_cur ? cur.step_copies() : nx.step_copies();
        iss_off = adv(iss_off);
        ++issued;
      }
      const JFA_LDS char* st = smem + cur_off;
      if (cur.live)
        dq_ds_step<D, decltype(mask)::value>(st, st + C::KBUF + pair * C::SLICE, ln, acc, half, cur.L - kb * C::BK,
                                             cb);
      // position kb + 1 must have landed; issued after it: position kb + 2's copies (if
      // copied yet) and the previous tile's dQ stores (if issued after it)
      wait_vmem_le((issued - 1 == kb + 2 ? last_copies : 0) + (kb + 1 <= stores_at ? stores : 0));
      __syncthreads();
      cur_off = adv(cur_off);
    };
    const int nfull = cur.L / C::BK;
    for (int kb = 0; kb < nfull; ++kb) step(kb, std::false_type{});
    if (nfull < cur.nkb) step(nfull, std::true_type{});

    // dQ rows through the slot the last step used (the slot before cur_off): half r =
    // tile rows 128 r .. 128 r + 127 (waves 4 r .. 4 r + 3) as bf16 [row][D], rows RB + 8
    // bytes apart so that the 32 rows of one write land in distinct banks.  Rows past
    // the sequence repeat the half's last row (same address, same value).
    stores = 0;
    {
      constexpr int PITCH = C::RB + 8, HALF_ROWS = C::BM / 2;
      static_assert(HALF_ROWS * PITCH <= C::STAGE, "staging rows inside one ring slot");
      constexpr int PASSES = HALF_ROWS * (C::RB / 16) / (C::NW * 64);
      JFA_LDS char* stg = smem + (cur_off == 0 ? LAST : cur_off - C::STAGE);
      int tl = tid;
      asm volatile("" : "+v"(tl));  // computed here, not hoisted and kept live through the steps
      const int wrow = (tl >> 6 >> 1 & 1) * 64 + (tl >> 6 & 1) * 32 + (tl & 31);  // row within the half
      const int wbase = wrow * PITCH + 8 * ((tl >> 5) & 1);
      const int row0 = cur.blk * C::BM;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int valid = min(HALF_ROWS, cur.L - row0 - HALF_ROWS * r);  // rows of this half
        if (valid <= 0) break;                                         // workgroup-uniform
        if ((wave >> 2) == r) {
#pragma unroll
          for (int db = 0; db < C::NDB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4)
              lds_st8(stg + 64 * db + 16 * g4, wbase,
                      pack4(acc[db][4 * g4] * p.scale, acc[db][4 * g4 + 1] * p.scale, acc[db][4 * g4 + 2] * p.scale,
                            acc[db][4 * g4 + 3] * p.scale));
        }
        __syncthreads();
        uint16_t* dst = p.dq + (cur.s0 + row0 + HALF_ROWS * r) * rs + (int64_t)cur.h * D;
#pragma unroll
        for (int k = 0; k < PASSES; ++k) {
          const int q = tl + C::NW * 64 * k;
          const int row = min(q / (C::RB / 16), valid - 1), cc = q % (C::RB / 16);
          const int ro = row * PITCH + 16 * cc;
          const u32x2 lo = lds_ld8(stg, ro), hi = lds_ld8(stg, ro + 8);
          st16(dst + (int64_t)row * rs + 8 * cc, u32x4{lo[0], lo[1], hi[0], hi[1]});
        }
        stores += PASSES;
        if (r == 0 && reserve) next_tile = base + gsize + ticket;
        __syncthreads();
      }
    }
    if (!more) break;
    // renumber from the next tile's step 0 (landed: awaited at the last step)
    issued -= cur.nkb;
    stores_at = issued - 1;
    idx = nidx;
    cur = nx;
  }
}

}  // namespace

hipError_t launch_bwd_self_dq(const BwdParams& p, int head_dim, hipStream_t s) {
  if (p.dq_programs <= 0) return hipSuccess;
  const dim3 grid(p.dq_programs), block(kDqWaves * 64);
  if (head_dim == 64) {
    if (p.sel) hipLaunchKernelGGL((dq_kernel<64, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((dq_kernel<64, false>), grid, block, 0, s, p);
  } else {
    if (p.sel) hipLaunchKernelGGL((dq_kernel<128, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((dq_kernel<128, false>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_self_dkdv(const BwdParams& p, int head_dim, hipStream_t s) {
  if (p.num_programs <= 0) return hipSuccess;
  const dim3 grid(p.num_programs), block(kBwdWaves * 64);
  if (p.ds && p.sel) return hipErrorInvalidValue;  // stored dS and block sparsity do not combine
  if (p.sel && p.sparse_narrow) {
    // block-sparse, 64-key tiles of two waves (head_dim 128 only)
    if (head_dim != 128) return hipErrorInvalidValue;
    hipLaunchKernelGGL((dkdv_kernel<128, false, true, 2, 2>), grid, dim3(2 * 64), 0, s, p);
    return hipGetLastError();
  }
  if (head_dim == 64) {
    if (p.ds) hipLaunchKernelGGL((dkdv_kernel<64, true, false>), grid, block, 0, s, p);
    else if (p.sel) hipLaunchKernelGGL((dkdv_kernel<64, false, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((dkdv_kernel<64, false, false>), grid, block, 0, s, p);
  } else {
    // self attention: two waves per SIMD (dkdv2_kernel); broadcast-Q keys and
    // block-sparse 128-key tiles: one (dkdv_kernel)
    if (p.ds) hipLaunchKernelGGL((dkdv2_kernel<128, true>), grid, dim3(Kv2Cfg<128>::NW * 64), 0, s, p);
    else if (p.sel) hipLaunchKernelGGL((dkdv_kernel<128, false, true>), grid, block, 0, s, p);
    else if (!p.bq) hipLaunchKernelGGL((dkdv2_kernel<128, false>), grid, dim3(Kv2Cfg<128>::NW * 64), 0, s, p);
    else hipLaunchKernelGGL((dkdv_kernel<128, false, false>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_self_prep(const BwdParams& p, int head_dim, hipStream_t s) {
  const int64_t rows = p.total_tokens * p.num_heads;
  const int64_t rows_per_block = 256 / (head_dim / 8);
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>((rows + rows_per_block - 1) / rows_per_block, 4096));
  if (head_dim == 64)
    hipLaunchKernelGGL(prep_kernel<64>, dim3(grid), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(prep_kernel<128>, dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_bwd_self_dq_ds(const BwdParams& p, int head_dim, hipStream_t s) {
  if (p.dq_programs <= 0) return hipSuccess;
  if (head_dim == 64)
    hipLaunchKernelGGL(dq_ds_kernel<64>, dim3(p.dq_programs), dim3(kDsWaves * 64), 0, s, p);
  else
    hipLaunchKernelGGL(dq_ds_kernel<128>, dim3(p.dq_programs), dim3(kDsWaves * 64), 0, s, p);
  return hipGetLastError();
}

}  // namespace jfa
