// Block-diagonal jagged attention (fixed 64-token blocks) for gfx950, forward and
// backward.
//
// What it computes ("TLX Block Attention", bittide page, sections 1, 2.1 and 4): every
// sequence is cut into consecutive 64-token groups that attend only within
// themselves.  With one query tile matching exactly one key/value tile, the forward is
// a single S = Q K^T, a direct softmax (no running maximum, no correction factor, no
// loop) and a single O = P V; the backward rebuilds P for the one tile, forms
// Di = rowsum(dO * O) inline and finishes dQ, dK and dV of the block with no
// cross-tile accumulation.  A trailing partial block of a sequence attends within
// itself.
//
// How it maps to CDNA4: the work is memory bound (about 32 FLOP per byte at D=64, the
// same point the page makes for its own kernel in section 3.3), so one wave owns one
// (block, head) tile and the grid is persistent with balanced contiguous tile ranges
// computed in closed form from divmod (same page, section 5).  Tiles are numbered with
// the head fastest so the waves of a workgroup read one contiguous 64-token slab.
// A tile's sequence is found with a fixed-step binary search over the per-sequence
// block prefix sums.  Differences from the page's kernel: the backward reads the
// forward's lse (4 bytes per row, about 1% of the traffic) instead of recomputing the
// row maxima, because on this layout the keys of a row are spread across lanes.
//
// Fused rotary embedding (BdParams::rope non-null; the same page's opening summary
// reports the attention plus rotary backward fused into the attention kernel).  The
// rotation (RoFormer's: pair (x_i, x_{i+D/2}) turned by the angle p theta_i, p the
// token's index inside its sequence, cos and sin from the caller's table) is applied
// where q and k enter the kernel -- to the register fragments in the forward, to the
// Q and K LDS tiles in the backward (one lane per row, before any product reads them)
// -- and its transpose is applied to the dQ and dK accumulators before they are stored,
// so the caller receives the gradients with respect to the un-rotated q and k.  On
// both layouts a column c < D/2 and its partner c + D/2 sit in the same lane.
#include <type_traits>

#include "jfa_device.h"
#include "jfa_internal.h"

namespace jfa {
namespace {

template <int D>
struct BdCfg {
  static constexpr int NW = (D == 64) ? 4 : 2;  // waves per workgroup (LDS budget)
  static constexpr int RB = 2 * D;
  static constexpr int NKS = D / 16;
  static constexpr int NDB = D / 32;
  static constexpr int TBUF = kBlock * RB;       // one 64-row tile
  static constexpr int SRB = 2 * kBlock;         // dS^T row bytes
  static constexpr int SBUF = kBlock * SRB;
  // backward per-wave LDS: Q, K, dO tiles, dS^T, lse2[64], Di[64]
  static constexpr int W_Q = 0, W_K = TBUF, W_DO = 2 * TBUF, W_S = 3 * TBUF, W_LSE = 3 * TBUF + SBUF,
                       W_DI = W_LSE + 256, W_BWD = W_DI + 256;
};

struct BdTile {
  int64_t t0;  // first token of the block
  int n;       // rows in the block (1..64)
  int h;
  int pos0;    // position of the block's first token inside its sequence
};

// Tile g -> (block, head); block -> (sequence b, block j) by binary search over the
// per-sequence block prefix sums.
__device__ __forceinline__ BdTile locate(const BdParams& p, int64_t g) {
  const int H = p.num_heads;
  const int blk = (int)(g / H);
  BdTile t;
  t.h = (int)(g % H);
  int lo = 0, hi = p.num_seqs;  // prefix[lo] <= blk < prefix[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.blk_prefix[mid] <= blk) lo = mid; else hi = mid;
  }
  const int j = blk - p.blk_prefix[lo];
  const int64_t s0 = p.offsets[lo];
  const int L = (int)(p.offsets[lo + 1] - s0);
  t.t0 = s0 + (int64_t)j * kBlock;
  t.n = min(kBlock, L - j * kBlock);
  t.pos0 = j * kBlock;
  return t;
}

// A wave's walk over its tiles g, g + step, ... (increasing): the tile's (block, head)
// and the block's sequence follow from the previous tile's (the sequence index only
// grows), so that a step costs scalar loads only where a sequence ends.  Every field is
// uniform over the wave, and scalar loads do not wait for the wave's vector loads and
// stores in flight.
struct BdWalk {
  int blk, h, seq;
  int pfx0, pfx1;  // blk_prefix[seq], blk_prefix[seq + 1]
  int L;           // length of sequence seq
  int64_t s0;      // its first token
};

__device__ __forceinline__ void walk_seq(const BdParams& p, BdWalk& w) {
  w.pfx0 = ld_uniform(p.blk_prefix, w.seq);
  w.pfx1 = ld_uniform(p.blk_prefix, w.seq + 1);
  w.s0 = ld_uniform(p.offsets, w.seq);
  w.L = (int)(ld_uniform(p.offsets, w.seq + 1) - w.s0);
}

// g: a tile index below num_tiles, uniform over the wave.
__device__ __forceinline__ BdWalk walk_start(const BdParams& p, int64_t g) {
  BdWalk w;
  w.blk = (int)(g / p.num_heads);
  w.h = (int)(g % p.num_heads);
  int lo = 0, hi = p.num_seqs;  // prefix[lo] <= blk < prefix[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (ld_uniform(p.blk_prefix, mid) <= w.blk) lo = mid; else hi = mid;
  }
  w.seq = lo;
  walk_seq(p, w);
  return w;
}

// To tile g + step (which must be below num_tiles): empty sequences are passed over.
__device__ __forceinline__ void walk_advance(const BdParams& p, BdWalk& w, int step) {
  w.h += step;
  while (w.h >= p.num_heads) {
    w.h -= p.num_heads;
    ++w.blk;
  }
  if (w.blk >= w.pfx1) {
    do {
      ++w.seq;
      w.pfx1 = ld_uniform(p.blk_prefix, w.seq + 1);
    } while (w.blk >= w.pfx1);
    walk_seq(p, w);
  }
}

__device__ __forceinline__ BdTile walk_tile(const BdWalk& w) {
  const int j = w.blk - w.pfx0;
  BdTile t;
  t.h = w.h;
  t.t0 = w.s0 + (int64_t)j * kBlock;
  t.n = min(kBlock, w.L - j * kBlock);
  t.pos0 = j * kBlock;
  return t;
}

// (x1, x2) -> (x1 cos - x2 sin, x2 cos + x1 sin), and its transpose.
__device__ __forceinline__ void rot2(float& x1, float& x2, float c, float s) {
  const float y1 = fmaf(x1, c, -x2 * s), y2 = fmaf(x2, c, x1 * s);
  x1 = y1;
  x2 = y2;
}

// Eight (cos, sin) pairs of table row `tab` starting at pair i0.
__device__ __forceinline__ void rope_pairs8(const float* tab, int i0, float (&cs)[16]) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const float4 w = *reinterpret_cast<const float4*>(tab + 2 * i0 + 4 * u);
    cs[4 * u] = w.x;
    cs[4 * u + 1] = w.y;
    cs[4 * u + 2] = w.z;
    cs[4 * u + 3] = w.w;
  }
}

// Forward: the (cos, sin) pairs of this lane's columns of one row: pairs 16 ks + 8 half
// + e, ks < NKS/2.
template <int NKS>
__device__ __forceinline__ void rope_row_pairs(const float* tab, int half, float (&cs)[NKS / 2][16]) {
#pragma unroll
  for (int ks = 0; ks < NKS / 2; ++ks) rope_pairs8(tab, 16 * ks + 8 * half, cs[ks]);
}

// Forward: rotate this lane's q and k fragments of one row (columns 16 ks + 8 half + e;
// column c < D/2 is in fragment ks < NKS/2, its partner in fragment ks + NKS/2).
template <int NKS>
__device__ __forceinline__ void rope_fragments(bf16x8 (&a)[NKS], bf16x8 (&b)[NKS], const float (&pairs)[NKS / 2][16]) {
#pragma unroll
  for (int ks = 0; ks < NKS / 2; ++ks) {
    const float (&cs)[16] = pairs[ks];
    float a1[8], a2[8], b1[8], b2[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a1[e] = (float)a[ks][e];
      a2[e] = (float)a[ks + NKS / 2][e];
      b1[e] = (float)b[ks][e];
      b2[e] = (float)b[ks + NKS / 2][e];
      rot2(a1[e], a2[e], cs[2 * e], cs[2 * e + 1]);
      rot2(b1[e], b2[e], cs[2 * e], cs[2 * e + 1]);
    }
    a[ks] = pack8(a1[0], a1[1], a1[2], a1[3], a1[4], a1[5], a1[6], a1[7]);
    a[ks + NKS / 2] = pack8(a2[0], a2[1], a2[2], a2[3], a2[4], a2[5], a2[6], a2[7]);
    b[ks] = pack8(b1[0], b1[1], b1[2], b1[3], b1[4], b1[5], b1[6], b1[7]);
    b[ks + NKS / 2] = pack8(b2[0], b2[1], b2[2], b2[3], b2[4], b2[5], b2[6], b2[7]);
  }
}

// Backward: rotate row r of the swizzled Q and K LDS tiles in place (chunk c of 8
// columns pairs with chunk c + D/16).
// PRE: the row's pairs were loaded into `pre` beforehand; otherwise they are loaded
// from `tab` chunk by chunk.
template <int D, bool PRE>
__device__ __forceinline__ void rope_lds_row(JFA_LDS char* qt, JFA_LDS char* kt, const float* tab,
                                             const float (&pre)[PRE ? D / 16 : 1][16], int r) {
  constexpr int RB = 2 * D, NC = D / 16;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    float cs[16];
    if constexpr (PRE) {
#pragma unroll
      for (int u = 0; u < 16; ++u) cs[u] = pre[c][u];
    } else {
      rope_pairs8(tab, 8 * c, cs);
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      JFA_LDS char* tile = tt == 0 ? qt : kt;
      const bf16x8 x = as_bf16x8(lds_ld16(tile, swz_off<RB>(r, c)));
      const bf16x8 y = as_bf16x8(lds_ld16(tile, swz_off<RB>(r, c + NC)));
      float x1[8], x2[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x1[e] = (float)x[e];
        x2[e] = (float)y[e];
        rot2(x1[e], x2[e], cs[2 * e], cs[2 * e + 1]);
      }
      lds_st16(tile, swz_off<RB>(r, c),
               __builtin_bit_cast(u32x4, pack8(x1[0], x1[1], x1[2], x1[3], x1[4], x1[5], x1[6], x1[7])));
      lds_st16(tile, swz_off<RB>(r, c + NC),
               __builtin_bit_cast(u32x4, pack8(x2[0], x2[1], x2[2], x2[3], x2[4], x2[5], x2[6], x2[7])));
    }
  }
}

// Backward epilogue: the (cos, sin) pairs of a row's accumulator columns (register i of
// block db <-> column 32 db + 8 (i/4) + 4 half + i%4, db < NDB/2).
template <int NDB>
__device__ __forceinline__ void acc_pairs(const float* tab, int half, float (&cs)[NDB / 2][4][8]) {
#pragma unroll
  for (int db = 0; db < NDB / 2; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int c0 = 32 * db + 8 * g4 + 4 * half;
      const float4 w0 = *reinterpret_cast<const float4*>(tab + 2 * c0);
      const float4 w1 = *reinterpret_cast<const float4*>(tab + 2 * c0 + 4);
      const float v[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
      for (int u = 0; u < 8; ++u) cs[db][g4][u] = v[u];
    }
}

// The transpose rotation on dQ^T / dK^T accumulators (partner of block db is block
// db + NDB/2, same register).
template <int NDB>
__device__ __forceinline__ void unrope_acc(f32x16 (&g)[NDB], const float (&pairs)[NDB / 2][4][8]) {
#pragma unroll
  for (int db = 0; db < NDB / 2; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const float (&cs)[8] = pairs[db][g4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * g4 + e;
        float x1 = g[db][i], x2 = g[db + NDB / 2][i];
        rot2(x1, x2, cs[2 * e], -cs[2 * e + 1]);
        g[db][i] = x1;
        g[db + NDB / 2][i] = x2;
      }
    }
}

// Accumulator rows (block rb: rows 32 rb + l32, register i <-> column 32 db + 8 (i/4) +
// 4 half + i%4) times `mul`, bf16 -> a swizzled [64 rows][D] LDS tile.
template <int D>
__device__ __forceinline__ void bd_stage_rows(JFA_LDS char* tile, int rb, const f32x16 (&a)[D / 32], float mul,
                                              int lane) {
  using C = BdCfg<D>;
  const int row = rb * 32 + (lane & 31), half = lane >> 5;
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4)
      lds_st8(tile, swz_off<C::RB>(row, 4 * db + g4) + 8 * half,
              pack4(a[db][4 * g4] * mul, a[db][4 * g4 + 1] * mul, a[db][4 * g4 + 2] * mul, a[db][4 * g4 + 3] * mul));
}

// Row stores per lane of one staged 64-row tile (16-byte chunks).
template <int D>
constexpr int bd_tile_stores() { return kBlock * (2 * D / 16) / 64; }

// A staged tile's first n rows -> dst (row stride rs elements) as whole rows, 16-byte
// stores with a row's chunks from consecutive lanes.  Every lane issues exactly
// bd_tile_stores() stores: rows past the end repeat row n - 1 (same address, same value).
template <int D>
__device__ __forceinline__ void bd_store_rows(uint16_t* dst, int64_t rs, int n, JFA_LDS char* tile, int lane) {
  using C = BdCfg<D>;
  constexpr int CPR = C::RB / 16;
#pragma unroll
  for (int k = 0; k < bd_tile_stores<D>(); ++k) {
    const int q = lane + 64 * k;
    const int row = min(q / CPR, n - 1), cc = q % CPR;
    st16(dst + (int64_t)row * rs + 8 * cc, lds_ld16(tile, swz_off<C::RB>(row, cc)));
  }
}

// Inputs of one forward tile loaded ahead: Q and K row fragments in registers (rows
// past the block's end repeat its last row), with the rotary table at head_dim 64 the
// rows' (cos, sin) pairs; V goes to the wave's LDS tile by direct copies.
template <int D, bool ROPE>
struct BdFwdIn {
  using C = BdCfg<D>;
  static constexpr bool PRE = ROPE && D == 64;  // table pairs loaded with q, k
  bf16x8 qf[2][C::NKS], kf[2][C::NKS];
  float pre[PRE ? 2 : 1][C::NKS / 2][16];
};

template <int D, bool ROPE>
__device__ __forceinline__ void bd_fwd_load(const BdParams& p, const BdTile& t, JFA_LDS char* vt, int lane,
                                            BdFwdIn<D, ROPE>& in) {
  using C = BdCfg<D>;
  // lane-dependent offsets are recomputed at each call rather than kept live (in
  // registers the loop cannot spare) from the first
  asm volatile("" : "+v"(lane));
  const int l32 = lane & 31, half = lane >> 5;
  const int64_t rs = (int64_t)p.num_heads * D;                              // q, o row stride
  const int64_t base = t.t0 * rs + (int64_t)t.h * D;
  const int64_t rkv = (int64_t)p.num_kv_heads * D;                          // k, v row stride
  const int64_t kvbase = t.t0 * rkv + (int64_t)(t.h / (p.num_heads / p.num_kv_heads)) * D;
  const int n = t.n;
  dma_tile<C::RB, kBlock, 1>(p.v + kvbase, rkv, n, vt, 0, lane);
  if constexpr (BdFwdIn<D, ROPE>::PRE) {
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const int row = bb * 32 + l32;
      rope_row_pairs<C::NKS>(p.rope + (int64_t)(t.pos0 + min(row, n - 1)) * D, half, in.pre[bb]);
    }
  }
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
    // rows past the end repeat the block's last row: their keys are masked and their
    // query rows are not stored
    const int row = min(bb * 32 + l32, n - 1);
    const uint16_t* qp = p.q + base + row * rs + 8 * half;
    const uint16_t* kp = p.k + kvbase + row * rkv + 8 * half;
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
      in.qf[bb][ks] = as_bf16x8(ld16(qp + 16 * ks));
      in.kf[bb][ks] = as_bf16x8(ld16(kp + 16 * ks));
    }
  }
}

// One forward tile from its loaded inputs (V in `vt`).  PREV: the wave issued the
// previous tile's bd_tile_stores() O stores after this tile's loads (they may stay in
// flight).  Once O is in LDS, the next tile's inputs are loaded (has_next: tile `nx`,
// its V into `vt_next`) before this tile's O stores are issued, so that no tile
// waits for its predecessor's stores.
template <int D, bool ROPE, bool PREV>
__device__ __forceinline__ void bd_fwd_tile(const BdParams& p, const BdTile& t, JFA_LDS char* vt, int lane,
                                            BdFwdIn<D, ROPE>& in, bool has_next, BdTile nx,
                                            JFA_LDS char* vt_next) {
  using C = BdCfg<D>;
  asm volatile("" : "+v"(lane));  // lane-dependent offsets: recomputed per tile, not kept live
  const int l32 = lane & 31, half = lane >> 5;
  const int n = t.n;
  const float c = p.scale_log2;
  // This tile's V copies and Q, K loads have landed: every vector-memory instruction
  // but the previous tile's O stores (issued after them) is complete.
  if constexpr (PREV) wait_vmem_upto<bd_tile_stores<D>()>();
  else wait_vmem();
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
    // rows past the end hold the last row (see bd_fwd_load) and take its rotation
    const int row = min(bb * 32 + l32, n - 1);
    if constexpr (BdFwdIn<D, ROPE>::PRE) {
      rope_fragments<C::NKS>(in.qf[bb], in.kf[bb], in.pre[bb]);
    } else if constexpr (ROPE) {
      float cs[C::NKS / 2][16];
      rope_row_pairs<C::NKS>(p.rope + (int64_t)(t.pos0 + row) * D, half, cs);
      rope_fragments<C::NKS>(in.qf[bb], in.kf[bb], cs);
    }
  }
  // S^T = K Q^T, lane = query column.
  f32x16 s[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][qb][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < C::NKS; ++ks) s[kb][qb] = mfma32(in.kf[kb][ks], in.qf[qb][ks], s[kb][qb]);
    }
  // Direct softmax over the block's keys; the lse leaves now (before the next tile's
  // loads, so that the stores issued after those are exactly the O rows).
  float l[2];
  bf16x8 pf[2][4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
        if (key >= n) s[kb][qb][i] = -INFINITY;
        mx = fmaxf(mx, s[kb][qb][i]);
      }
    const float m = half_max(mx);
    const float mc = m * c;
    float sum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = fast_exp2(fmaf(s[kb][qb][i], c, -mc));
        s[kb][qb][i] = pv;
        sum += pv;
      }
    l[qb] = half_sum(sum);
    const int row = qb * 32 + l32;
    if (row < n && half == 0) p.lse[(int64_t)t.h * p.total_tokens + t.t0 + row] = (mc + fast_log2(l[qb])) * kLn2;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const f32x16& src = s[tt >> 1][qb];
      const int r = 8 * (tt & 1);
      pf[qb][tt] = pack8(src[r], src[r + 1], src[r + 2], src[r + 3], src[r + 4], src[r + 5], src[r + 6],
                         src[r + 7]);
    }
  }
  // O^T = V^T P^T for both 32-row blocks.
  f32x16 o[2][C::NDB];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
      for (int i = 0; i < 16; ++i) o[qb][db][i] = 0.f;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
        o[qb][db] = mfma32(tr_operand<C::RB>(vt, 16 * tt, 32 * db, lane), pf[qb][tt], o[qb][db]);
    }
  // The O rows go out through this tile's V tile (free once the products have read it;
  // one wave's LDS instructions execute in order, so its reads of V precede these
  // writes and the writes precede the reads below) as whole rows with 16-byte stores --
  // writing each lane's 8-byte pieces of its own row directly took about half the
  // kernel's time.
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) bd_stage_rows<D>(vt, qb, o[qb], 1.0f / l[qb], lane);
  // the next tile's loads go out between the LDS writes and reads of O
  if (has_next) bd_fwd_load<D, ROPE>(p, nx, vt_next, lane, in);
  const int64_t rs = (int64_t)p.num_heads * D;
  bd_store_rows<D>(p.o + t.t0 * rs + (int64_t)t.h * D, rs, n, vt, lane);
}

// Backward operands of one tile held in registers: the Q, K and dO rows (16-byte chunks,
// lane l holding chunks l, l + 64, ... of the row-major 64-row tile), this lane's V rows
// as the B operands of dP, its O rows for Di and its lse; rows past the block's end
// repeat its last row (their P and dS are zero, their results are not stored).  The
// kernel loads the next tile's into one of these while the current tile computes, so
// that the wave -- alone on its SIMD -- does not wait out a full memory round trip per
// tile.
template <int D>
struct BdBwdRegs {
  static constexpr int CPR = 2 * D / 16;       // 16-byte chunks per row
  static constexpr int CH = kBlock * CPR / 64;  // chunks per lane per tile
  u32x4 q[CH], k[CH], dout[CH];
  bf16x8 vf[2][D / 16];
  u32x4 o[2][D / 16];
  float lse;
};

// Every lane issues the same loads whatever the tile (a fixed count, which later waits
// rely on).
template <int D>
__device__ __forceinline__ void bd_bwd_load(const BdParams& p, const BdTile& t, BdBwdRegs<D>& x, int lane) {
  using R = BdBwdRegs<D>;
  asm volatile("" : "+v"(lane));  // lane-dependent offsets: recomputed per tile, not kept live
  const int l32 = lane & 31, half = lane >> 5;
  const int64_t rs = (int64_t)p.num_heads * D;
  const int64_t base = t.t0 * rs + (int64_t)t.h * D;
  const int n = t.n;
#pragma unroll
  for (int j = 0; j < R::CH; ++j) {
    const int idx = j * 64 + lane, r = min(idx / R::CPR, n - 1), c = idx % R::CPR;
    const int64_t off = base + r * rs + 8 * c;
    x.q[j] = ld16(p.q + off);
    x.k[j] = ld16(p.k + off);
    x.dout[j] = ld16(p.dout + off);
  }
#pragma unroll
  for (int b2 = 0; b2 < 2; ++b2) {
    const int r = min(b2 * 32 + l32, n - 1);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const int64_t off = base + r * rs + 16 * ks + 8 * half;
      x.vf[b2][ks] = as_bf16x8(ld16(p.v + off));
      x.o[b2][ks] = ld16(p.o_in + off);
    }
  }
  x.lse = p.lse_in[(int64_t)t.h * p.total_tokens + t.t0 + min(lane, n - 1)];
}

// Q, K, dO chunks -> this wave's swizzled LDS tiles.
template <int D>
__device__ __forceinline__ void bd_bwd_stage(const BdBwdRegs<D>& x, JFA_LDS char* qt, JFA_LDS char* kt,
                                             JFA_LDS char* dot, int lane) {
  using R = BdBwdRegs<D>;
#pragma unroll
  for (int j = 0; j < R::CH; ++j) {
    const int idx = j * 64 + lane, r = idx / R::CPR, c = idx % R::CPR;
    const int off = swz_off<2 * D>(r, c);
    lds_st16(qt, off, x.q[j]);
    lds_st16(kt, off, x.k[j]);
    lds_st16(dot, off, x.dout[j]);
  }
}

// Key block kb (keys 32 kb + l32) of one backward tile: S and dP of its keys against the
// tile's 64 queries, P and dS (zero for keys past the end and, through lse2 = +inf, for
// queries past it), dS^T rows -> LDS for the dQ product, and the dV^T, dK^T accumulators
// of these keys.  vf: this lane's key row of V as B operands.
template <int D>
__device__ __forceinline__ void bd_bwd_key_block(int kb, int n, float c, JFA_LDS char* qt, JFA_LDS char* kt,
                                                 JFA_LDS char* dot, JFA_LDS char* st, const float* lse2,
                                                 const float* di, const bf16x8 (&vf)[D / 16], int lane,
                                                 f32x16 (&dk)[D / 32], f32x16 (&dv)[D / 32]) {
  using C = BdCfg<D>;
  const int l32 = lane & 31, half = lane >> 5;
  const int key = kb * 32 + l32;
  const bool key_ok = key < n;
  bf16x8 kf[C::NKS];
#pragma unroll
  for (int ks = 0; ks < C::NKS; ++ks) kf[ks] = as_bf16x8(lds_ld16(kt, swz_off<C::RB>(key, 2 * ks + half)));
  f32x16 s[2], dp[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) s[qb][i] = dp[qb][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
      const int off = swz_off<C::RB>(qb * 32 + l32, 2 * ks + half);
      s[qb] = mfma32(as_bf16x8(lds_ld16(qt, off)), kf[ks], s[qb]);
      dp[qb] = mfma32(as_bf16x8(lds_ld16(dot, off)), vf[ks], dp[qb]);
    }
  }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int r4 = qb * 32 + 8 * g4 + 4 * half;
      const float4 la = *reinterpret_cast<const float4*>(lse2 + r4);
      const float4 da = *reinterpret_cast<const float4*>(di + r4);
      const float lz[4] = {la.x, la.y, la.z, la.w}, dz[4] = {da.x, da.y, da.z, da.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * g4 + e;
        float pv = fast_exp2(fmaf(s[qb][i], c, -lz[e]));
        pv = key_ok ? pv : 0.f;
        s[qb][i] = pv;
        dp[qb][i] = pv * (dp[qb][i] - dz[e]);
      }
    }
  bf16x8 pf[4], dsf[4];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const int qb = tt >> 1, r = 8 * (tt & 1);
    pf[tt] = pack8(s[qb][r], s[qb][r + 1], s[qb][r + 2], s[qb][r + 3], s[qb][r + 4], s[qb][r + 5], s[qb][r + 6],
                   s[qb][r + 7]);
    dsf[tt] = pack8(dp[qb][r], dp[qb][r + 1], dp[qb][r + 2], dp[qb][r + 3], dp[qb][r + 4], dp[qb][r + 5],
                    dp[qb][r + 6], dp[qb][r + 7]);
  }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int q = qb * 32 + 8 * g4 + 4 * half;
      lds_st8(st, swz_off<C::SRB>(key, q >> 3) + (q & 7) * 2,
              pack4(dp[qb][4 * g4], dp[qb][4 * g4 + 1], dp[qb][4 * g4 + 2], dp[qb][4 * g4 + 3]));
    }
  // dV^T = dO^T P and dK^T = Q^T dS for these 32 keys; complete after the single block.
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
    for (int i = 0; i < 16; ++i) dk[db][i] = dv[db][i] = 0.f;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      dv[db] = mfma32(tr_operand<C::RB>(dot, 16 * tt, 32 * db, lane), pf[tt], dv[db]);
      dk[db] = mfma32(tr_operand<C::RB>(qt, 16 * tt, 32 * db, lane), dsf[tt], dk[db]);
    }
  }
}

// dQ^T = K^T dS^T for query block qb: [head dim x queries], k = keys; lane = query column.
template <int D>
__device__ __forceinline__ void bd_bwd_dq(int qb, JFA_LDS char* kt, JFA_LDS char* st, int lane,
                                          f32x16 (&dq)[D / 32]) {
  using C = BdCfg<D>;
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
    for (int i = 0; i < 16; ++i) dq[db][i] = 0.f;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
      dq[db] = mfma32(tr_operand<C::RB>(kt, 16 * tt, 32 * db, lane), tr_operand<C::SRB>(st, 16 * tt, 32 * qb, lane),
                      dq[db]);
  }
}

// One backward tile whose Q, K, dO are in the wave's LDS tiles and whose V, O rows and
// lse come in `cur` (registers loaded one tile ahead); at head_dim 64 with the rotary
// table, `pre` holds this lane's row pairs for the in-place rotation of Q and K.
// dK, dV and dQ leave through the Q and dO tiles (free once the products have read
// them; one wave's LDS instructions execute in order) as 3 bd_tile_stores() row stores
// per lane: a fixed count issued at the tile's end, so that the next tile's wait for its
// operands (loaded before these stores) lets the stores stay in flight.
template <int D, bool ROPE>
__device__ __forceinline__ void bd_bwd_tile_pf(const BdParams& p, const BdTile& t, JFA_LDS char* w, float* wf,
                                               int lane, const BdBwdRegs<D>& cur,
                                               const float (&pre)[ROPE ? D / 16 : 1][16]) {
  using C = BdCfg<D>;
  static_assert(!ROPE || D == 64, "row pairs held in registers at head_dim 64 only");
  asm volatile("" : "+v"(lane));
  const int l32 = lane & 31, half = lane >> 5;
  const int64_t rs = (int64_t)p.num_heads * D;
  const int64_t base = t.t0 * rs + (int64_t)t.h * D;
  const int n = t.n;
  const float c = p.scale_log2;
  JFA_LDS char* qt = w + C::W_Q;
  JFA_LDS char* kt = w + C::W_K;
  JFA_LDS char* dot = w + C::W_DO;
  JFA_LDS char* st = w + C::W_S;
  float* lse2 = wf + C::W_LSE / 4;
  float* di = wf + C::W_DI / 4;
  if constexpr (ROPE) {
    // rows past the block's end stay as copied (their P and dS are zero)
    if (lane < n) rope_lds_row<D, true>(qt, kt, nullptr, pre, lane);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
  }
  // Di = rowsum(dO * O): lane = row of query block qb, half = which 8-column chunks.
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = qb * 32 + l32;
    float acc = 0.f;
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
      const bf16x8 d8 = as_bf16x8(lds_ld16(dot, swz_off<C::RB>(row, 2 * ks + half)));
      const bf16x8 o8 = as_bf16x8(cur.o[qb][ks]);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf((float)d8[e], (float)o8[e], acc);
    }
    acc = half_sum(acc);
    if (half == 0) di[row] = acc;
  }
  lse2[lane] = lane < n ? cur.lse * kLog2e : INFINITY;
  f32x16 dk[2][C::NDB], dv[2][C::NDB];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) bd_bwd_key_block<D>(kb, n, c, qt, kt, dot, st, lse2, di, cur.vf[kb], lane, dk[kb], dv[kb]);
  float epi[ROPE ? 2 : 1][C::NDB / 2][4][8];
  if constexpr (ROPE) {
    // the epilogue's pairs of rows l32 and 32 + l32 (key rows of key block kb, query
    // rows of query block qb); by now the loads issued before this tile have landed
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
      acc_pairs<C::NDB>(p.rope + (int64_t)(t.pos0 + min(rb * 32 + l32, n - 1)) * D, half, epi[rb]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) unrope_acc<C::NDB>(dk[kb], epi[kb]);
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    bd_stage_rows<D>(qt, kb, dk[kb], p.scale, lane);
    bd_stage_rows<D>(dot, kb, dv[kb], 1.0f, lane);
  }
  bd_store_rows<D>(p.dk + base, rs, n, qt, lane);
  bd_store_rows<D>(p.dv + base, rs, n, dot, lane);
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    f32x16 dq[C::NDB];
    bd_bwd_dq<D>(qb, kt, st, lane, dq);
    if constexpr (ROPE) unrope_acc<C::NDB>(dq, epi[qb]);
    bd_stage_rows<D>(qt, qb, dq, p.scale, lane);
  }
  bd_store_rows<D>(p.o + base, rs, n, qt, lane);
}

// One backward tile that loads its own operands (Q, K, dO by direct copies into the
// wave's LDS tiles; V, O rows and lse into registers).
template <int D, bool ROPE>
__device__ __forceinline__ void bd_bwd_tile(const BdParams& p, const BdTile& t, JFA_LDS char* w, float* wf,
                                            int lane) {
  using C = BdCfg<D>;
  const int l32 = lane & 31, half = lane >> 5;
  const int64_t rs = (int64_t)p.num_heads * D;
  const int64_t base = t.t0 * rs + (int64_t)t.h * D;
  const int n = t.n;
  const float c = p.scale_log2;
  JFA_LDS char* qt = w + C::W_Q;
  JFA_LDS char* kt = w + C::W_K;
  JFA_LDS char* dot = w + C::W_DO;
  JFA_LDS char* st = w + C::W_S;
  float* lse2 = wf + C::W_LSE / 4;
  float* di = wf + C::W_DI / 4;
  dma_tile<C::RB, kBlock, 1>(p.q + base, rs, n, qt, 0, lane);
  dma_tile<C::RB, kBlock, 1>(p.k + base, rs, n, kt, 0, lane);
  dma_tile<C::RB, kBlock, 1>(p.dout + base, rs, n, dot, 0, lane);
  const float lv = lane < n ? p.lse_in[(int64_t)t.h * p.total_tokens + t.t0 + lane] : 0.f;
  const float* tab_row = ROPE ? p.rope + (int64_t)(t.pos0 + min(lane, n - 1)) * D : nullptr;
  const float nopre[1][16] = {};
  wait_vmem();
  if constexpr (ROPE) {
    // rows past the block's end stay as copied (their P and dS are zero)
    if (lane < n) rope_lds_row<D, false>(qt, kt, tab_row, nopre, lane);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
  }
  // Di = rowsum(dO * O): lane = row of query block qb, half = which 8-column chunks.
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = qb * 32 + l32;
    float acc = 0.f;
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
      const bf16x8 d8 = as_bf16x8(lds_ld16(dot, swz_off<C::RB>(row, 2 * ks + half)));
      const bf16x8 o8 = as_bf16x8(row < n ? ld16(p.o_in + base + row * rs + 16 * ks + 8 * half) : zero16());
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf((float)d8[e], (float)o8[e], acc);
    }
    acc = half_sum(acc);
    if (half == 0) di[row] = acc;
  }
  lse2[lane] = lane < n ? lv * kLog2e : INFINITY;
  for (int kb = 0; kb < 2; ++kb) {
    const int key = kb * 32 + l32;
    bf16x8 vf[C::NKS];
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks)
      vf[ks] = as_bf16x8(key < n ? ld16(p.v + base + key * rs + 16 * ks + 8 * half) : zero16());
    f32x16 dk[C::NDB], dv[C::NDB];
    bd_bwd_key_block<D>(kb, n, c, qt, kt, dot, st, lse2, di, vf, lane, dk, dv);
    if (key < n) {
      if constexpr (ROPE) {
        float cs[C::NDB / 2][4][8];
        acc_pairs<C::NDB>(p.rope + (int64_t)(t.pos0 + key) * D, half, cs);
        unrope_acc<C::NDB>(dk, cs);
      }
      const int64_t row = base + key * rs + 4 * half;
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
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = qb * 32 + l32;
    f32x16 dq[C::NDB];
    bd_bwd_dq<D>(qb, kt, st, lane, dq);
    if (row < n) {
      if constexpr (ROPE) {
        float cs[C::NDB / 2][4][8];
        acc_pairs<C::NDB>(p.rope + (int64_t)(t.pos0 + row) * D, half, cs);
        unrope_acc<C::NDB>(dq, cs);
      }
      uint16_t* qp = p.o + base + row * rs + 4 * half;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          st8(qp + 32 * db + 8 * g4, pack4(dq[db][4 * g4] * p.scale, dq[db][4 * g4 + 1] * p.scale,
                                          dq[db][4 * g4 + 2] * p.scale, dq[db][4 * g4 + 3] * p.scale));
    }
  }
}

// Program p owns tiles [p*q + min(p, r), (p+1)*q + min(p+1, r)), (q, r) = divmod(N, P);
// its waves take every NW-th tile of the range.
// Two waves per SIMD at D = 64 (the rotary variant needs the cap to stay there).
template <int D, bool ROPE>
__global__ void __launch_bounds__(BdCfg<D>::NW * 64)
    __attribute__((amdgpu_waves_per_eu(D == 64 ? 2 : 1, D == 64 ? 2 : 1))) bd_fwd_kernel(BdParams p) {
  using C = BdCfg<D>;
  __shared__ __attribute__((aligned(16))) char smem[C::NW * 2 * C::TBUF];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int prog = xcd_program_id(blockIdx.x, gridDim.x);
  const int64_t P = gridDim.x, q = p.num_tiles / P, r = p.num_tiles % P;
  const int64_t start = prog * q + min((int64_t)prog, r), end = start + q + (prog < r ? 1 : 0);
  // Each wave walks its tiles g, g + NW, ... with two V tiles, loading the next tile's
  // inputs while the current one finishes (see bd_fwd_tile).
  JFA_LDS char* vt = (JFA_LDS char*)smem + wave * 2 * C::TBUF;
  JFA_LDS char* vt2 = vt + C::TBUF;
  int64_t g = start + wave;
  if (g >= end) return;
  int left = (int)((end - g + C::NW - 1) / C::NW);  // tiles left to this wave
  BdWalk wk = walk_start(p, g);
  BdTile t = walk_tile(wk);
  BdFwdIn<D, ROPE> in;
  bd_fwd_load<D, ROPE>(p, t, vt, lane, in);
  // The first tile has its own copy of the code, so that every entry to the loop has
  // issued the same stores after the same loads (the compiler's wait counts then need
  // not assume that the loads are the latest).
  auto step = [&](auto prev_tag) {
    if (lane == 0) count_visit(p.visits, g);
    --left;
    BdTile tn = t;
    if (left > 0) {
      walk_advance(p, wk, C::NW);
      tn = walk_tile(wk);
    }
    bd_fwd_tile<D, ROPE, decltype(prev_tag)::value>(p, t, vt, lane, in, left > 0, tn, vt2);
    if (left == 0) return false;
    g += C::NW;
    t = tn;
    JFA_LDS char* sw = vt;
    vt = vt2;
    vt2 = sw;
    return true;
  };
  if (!step(std::false_type{})) return;
  while (step(std::true_type{})) {
  }
}

template <int D, bool ROPE>
__global__ void __launch_bounds__(BdCfg<D>::NW * 64)
    __attribute__((amdgpu_waves_per_eu(1, 1))) bd_bwd_kernel(BdParams p) {
  using C = BdCfg<D>;
  __shared__ __attribute__((aligned(16))) char smem[C::NW * C::W_BWD];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int prog = xcd_program_id(blockIdx.x, gridDim.x);
  const int64_t P = gridDim.x, q = p.num_tiles / P, r = p.num_tiles % P;
  const int64_t start = prog * q + min((int64_t)prog, r), end = start + q + (prog < r ? 1 : 0);
  char* w = smem + wave * C::W_BWD;
  if constexpr (D == 64) {
    // Software pipeline over the wave's tiles: stage tile g's operands (loaded during
    // the previous tile), load the rotary pairs of its rows, issue the loads of the next
    // tile (the last tile loads itself again, so that every step issues the same loads),
    // then compute tile g.  The first tile has its own copy of the code, so that every
    // entry to the loop has issued the same stores after the same loads.
    int64_t g = start + wave;
    if (g >= end) return;
    int left = (int)((end - g + C::NW - 1) / C::NW);  // tiles left to this wave
    BdWalk wk = walk_start(p, g);
    BdTile t = walk_tile(wk);
    BdBwdRegs<D> nx;
    bd_bwd_load<D>(p, t, nx, lane);
    JFA_LDS char* lw = (JFA_LDS char*)w;
    auto step = [&](auto first_tag) {
      (void)first_tag;
      bd_bwd_stage<D>(nx, lw + C::W_Q, lw + C::W_K, lw + C::W_DO, lane);
      const BdBwdRegs<D> cur = nx;
      float pre[ROPE ? D / 16 : 1][16];
      if constexpr (ROPE) {
        const float* tab_row = p.rope + (int64_t)(t.pos0 + min(lane, t.n - 1)) * D;
#pragma unroll
        for (int c = 0; c < D / 16; ++c) rope_pairs8(tab_row, 8 * c, pre[c]);
      }
      --left;
      BdTile tn = t;
      if (left > 0) {
        walk_advance(p, wk, C::NW);
        tn = walk_tile(wk);
      }
      bd_bwd_load<D>(p, tn, nx, lane);
      if (lane == 0) count_visit(p.visits, g);
      bd_bwd_tile_pf<D, ROPE>(p, t, lw, (float*)w, lane, cur, pre);
      if (left == 0) return false;
      g += C::NW;
      t = tn;
      return true;
    };
    if (!step(std::true_type{})) return;
    while (step(std::false_type{})) {
    }
  } else {
    for (int64_t g = start + wave; g < end; g += C::NW) {
      if (lane == 0) count_visit(p.visits, g);
      bd_bwd_tile<D, ROPE>(p, locate(p, g), (JFA_LDS char*)w, (float*)w, lane);
    }
  }
}

int bd_programs(const BdParams& p, int nw) {
  const int64_t need = (p.num_tiles + nw - 1) / nw;
  return (int)(need < p.num_programs ? need : p.num_programs);
}

// cos / sin table of the fused rotary embedding: entry (pos, i) = (cos, sin) of
// pos * base^(-2i/D), i < D/2, formed in double precision and rounded once to fp32.
// One thread per (pos, i).
__global__ void rope_table_kernel(float* table, int positions, int head_dim, double base) {
  const int half = head_dim / 2;
  const int64_t n = (int64_t)positions * half;
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < n; t += (int64_t)gridDim.x * blockDim.x) {
    const int i = (int)(t % half);
    const double pos = (double)(t / half);
    const double ang = pos * pow(base, -2.0 * i / head_dim);
    double sn, cs;
    sincos(ang, &sn, &cs);
    *reinterpret_cast<float2*>(table + 2 * t) = make_float2((float)cs, (float)sn);
  }
}

}  // namespace

hipError_t launch_rope_table(float* table, int positions, int head_dim, double base, hipStream_t s) {
  const int64_t n = (int64_t)positions * (head_dim / 2);
  if (n <= 0) return hipSuccess;
  const int64_t g = (n + 255) / 256;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)(g < 8192 ? g : 8192)), dim3(256), 0, s, table, positions,
                     head_dim, base);
  return hipGetLastError();
}

hipError_t launch_bd_fwd(const BdParams& p, int head_dim, hipStream_t s) {
  if (p.num_tiles <= 0) return hipSuccess;
  const dim3 g64(bd_programs(p, BdCfg<64>::NW)), b64(BdCfg<64>::NW * 64);
  const dim3 g128(bd_programs(p, BdCfg<128>::NW)), b128(BdCfg<128>::NW * 64);
  if (head_dim == 64) {
    if (p.rope) hipLaunchKernelGGL((bd_fwd_kernel<64, true>), g64, b64, 0, s, p);
    else hipLaunchKernelGGL((bd_fwd_kernel<64, false>), g64, b64, 0, s, p);
  } else {
    if (p.rope) hipLaunchKernelGGL((bd_fwd_kernel<128, true>), g128, b128, 0, s, p);
    else hipLaunchKernelGGL((bd_fwd_kernel<128, false>), g128, b128, 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_bd_bwd(const BdParams& p, int head_dim, hipStream_t s) {
  if (p.num_tiles <= 0) return hipSuccess;
  const dim3 g64(bd_programs(p, BdCfg<64>::NW)), b64(BdCfg<64>::NW * 64);
  const dim3 g128(bd_programs(p, BdCfg<128>::NW)), b128(BdCfg<128>::NW * 64);
  if (head_dim == 64) {
    if (p.rope) hipLaunchKernelGGL((bd_bwd_kernel<64, true>), g64, b64, 0, s, p);
    else hipLaunchKernelGGL((bd_bwd_kernel<64, false>), g64, b64, 0, s, p);
  } else {
    if (p.rope) hipLaunchKernelGGL((bd_bwd_kernel<128, true>), g128, b128, 0, s, p);
    else hipLaunchKernelGGL((bd_bwd_kernel<128, false>), g128, b128, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace jfa
