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

template <int D, bool ROPE>
__device__ __forceinline__ void bd_fwd_tile(const BdParams& p, const BdTile& t, JFA_LDS char* vt, int lane) {
  using C = BdCfg<D>;
  const int l32 = lane & 31, half = lane >> 5;
  const int64_t rs = (int64_t)p.num_heads * D;                              // q, o row stride
  const int64_t base = t.t0 * rs + (int64_t)t.h * D;
  const int64_t rkv = (int64_t)p.num_kv_heads * D;                          // k, v row stride
  const int64_t kvbase = t.t0 * rkv + (int64_t)(t.h / (p.num_heads / p.num_kv_heads)) * D;
  const int n = t.n;
  const float c = p.scale_log2;
  dma_tile<C::RB, kBlock, 1>(p.v + kvbase, rkv, n, vt, 0, lane);

  // D = 64: the table pairs of both rows are loaded before q and k, so their latency
  // overlaps (at D = 128 the registers are not there; each row loads its own).
  constexpr bool PRE = ROPE && D == 64;
  float pre[PRE ? 2 : 1][C::NKS / 2][16];
  if constexpr (PRE) {
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const int row = bb * 32 + l32;
      rope_row_pairs<C::NKS>(p.rope + (int64_t)(t.pos0 + min(row, n - 1)) * D, half, pre[bb]);
    }
  }
  bf16x8 qf[2][C::NKS], kf[2][C::NKS];
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
    const int row = bb * 32 + l32;
    const uint16_t* qp = p.q + base + row * rs + 8 * half;
    const uint16_t* kp = p.k + kvbase + row * rkv + 8 * half;
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
      qf[bb][ks] = as_bf16x8(row < n ? ld16(qp + 16 * ks) : zero16());
      kf[bb][ks] = as_bf16x8(row < n ? ld16(kp + 16 * ks) : zero16());
    }
    if constexpr (PRE) {
      if (row < n) rope_fragments<C::NKS>(qf[bb], kf[bb], pre[bb]);
    } else if constexpr (ROPE) {
      if (row < n) {
        float cs[C::NKS / 2][16];
        rope_row_pairs<C::NKS>(p.rope + (int64_t)(t.pos0 + row) * D, half, cs);
        rope_fragments<C::NKS>(qf[bb], kf[bb], cs);
      }
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
      for (int ks = 0; ks < C::NKS; ++ks) s[kb][qb] = mfma32(kf[kb][ks], qf[qb][ks], s[kb][qb]);
    }
  // Direct softmax over the block's keys.
  float m[2], l[2];
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
    m[qb] = half_max(mx);
    const float mc = m[qb] * c;
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
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const f32x16& src = s[tt >> 1][qb];
      const int r = 8 * (tt & 1);
      pf[qb][tt] = pack8(src[r], src[r + 1], src[r + 2], src[r + 3], src[r + 4], src[r + 5], src[r + 6],
                         src[r + 7]);
    }
  }
  wait_vmem();
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
  // The O rows go out through the wave's V tile (free once the products have read it;
  // one wave's LDS instructions execute in order, so its reads of V precede these
  // writes and the writes precede the reads below): bf16 [row][D] with 16-byte chunks
  // swizzled by row, then whole rows with 16-byte stores (a row's chunks from
  // consecutive lanes) -- writing each lane's 8-byte pieces of its own row directly
  // took about half the kernel's time.
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = qb * 32 + l32;
    const float inv = 1.0f / l[qb];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        lds_st8(vt, swz_off<C::RB>(row, 4 * db + g4) + 8 * half,
                pack4(o[qb][db][4 * g4] * inv, o[qb][db][4 * g4 + 1] * inv, o[qb][db][4 * g4 + 2] * inv,
                      o[qb][db][4 * g4 + 3] * inv));
    if (row < n && half == 0) p.lse[(int64_t)t.h * p.total_tokens + t.t0 + row] = (m[qb] * c + fast_log2(l[qb])) * kLn2;
  }
  constexpr int CPR = C::RB / 16;  // 16-byte chunks per row
#pragma unroll
  for (int k = 0; k < kBlock * CPR / 64; ++k) {
    const int q = lane + 64 * k;
    const int row = q / CPR, cc = q % CPR;
    if (row < n) st16(p.o + base + row * rs + 8 * cc, lds_ld16(vt, swz_off<C::RB>(row, cc)));
  }
}

// Backward operands of one tile held in registers: the Q, K and dO rows (16-byte chunks,
// lane l holding chunks l, l + 64, ... of the row-major 64-row tile; rows past the
// block's end are zero), this lane's V rows as the B operands of dP, its O rows for Di
// and its lse.  The kernel loads the next tile's into one of these while the current
// tile computes, so that the wave -- alone on its SIMD -- does not wait out a full
// memory round trip per tile.
template <int D>
struct BdBwdRegs {
  static constexpr int CPR = 2 * D / 16;       // 16-byte chunks per row
  static constexpr int CH = kBlock * CPR / 64;  // chunks per lane per tile
  u32x4 q[CH], k[CH], dout[CH];
  bf16x8 vf[2][D / 16];
  u32x4 o[2][D / 16];
  float lse;
};

template <int D>
__device__ __forceinline__ void bd_bwd_load(const BdParams& p, const BdTile& t, BdBwdRegs<D>& x, int lane) {
  using R = BdBwdRegs<D>;
  const int l32 = lane & 31, half = lane >> 5;
  const int64_t rs = (int64_t)p.num_heads * D;
  const int64_t base = t.t0 * rs + (int64_t)t.h * D;
  const int n = t.n;
#pragma unroll
  for (int j = 0; j < R::CH; ++j) {
    const int idx = j * 64 + lane, r = idx / R::CPR, c = idx % R::CPR;
    const int64_t off = base + r * rs + 8 * c;
    x.q[j] = r < n ? ld16(p.q + off) : zero16();
    x.k[j] = r < n ? ld16(p.k + off) : zero16();
    x.dout[j] = r < n ? ld16(p.dout + off) : zero16();
  }
#pragma unroll
  for (int b2 = 0; b2 < 2; ++b2) {
    const int r = b2 * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const int64_t off = base + r * rs + 16 * ks + 8 * half;
      x.vf[b2][ks] = as_bf16x8(r < n ? ld16(p.v + off) : zero16());
      x.o[b2][ks] = r < n ? ld16(p.o_in + off) : zero16();
    }
  }
  x.lse = lane < n ? p.lse_in[(int64_t)t.h * p.total_tokens + t.t0 + lane] : 0.f;
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

// PF: the tile's Q, K, dO are already in the wave's LDS tiles and its V, O rows and lse
// come in `pf` (registers loaded one tile ahead); otherwise the tile loads them itself.
template <int D, bool ROPE, bool PF = false>
__device__ __forceinline__ void bd_bwd_tile(const BdParams& p, const BdTile& t, JFA_LDS char* w, float* wf,
                                            int lane, const BdBwdRegs<D>* pf = nullptr) {
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
  if constexpr (!PF) {
    dma_tile<C::RB, kBlock, 1>(p.q + base, rs, n, qt, 0, lane);
    dma_tile<C::RB, kBlock, 1>(p.k + base, rs, n, kt, 0, lane);
    dma_tile<C::RB, kBlock, 1>(p.dout + base, rs, n, dot, 0, lane);
  }
  const float lv = PF ? pf->lse : (lane < n ? p.lse_in[(int64_t)t.h * p.total_tokens + t.t0 + lane] : 0.f);
  // D = 64: this lane's table row is loaded while the tiles are in flight
  constexpr bool PRE = ROPE && D == 64;
  const float* tab_row = ROPE ? p.rope + (int64_t)(t.pos0 + min(lane, n - 1)) * D : nullptr;
  float pre[PRE ? D / 16 : 1][16];
  // and the epilogue's pairs of rows l32 and 32 + l32 (key rows of key block kb, query
  // rows of query block qb)
  float epi[PRE ? 2 : 1][C::NDB / 2][4][8];
  if constexpr (PRE) {
#pragma unroll
    for (int c = 0; c < D / 16; ++c) rope_pairs8(tab_row, 8 * c, pre[c]);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
      acc_pairs<C::NDB>(p.rope + (int64_t)(t.pos0 + min(rb * 32 + l32, n - 1)) * D, half, epi[rb]);
  }
  if constexpr (!PF) wait_vmem();
  if constexpr (ROPE) {
    // rows past the block's end stay as copied (their P and dS are zero)
    if (lane < n) rope_lds_row<D, PRE>(qt, kt, tab_row, pre, lane);
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
      const bf16x8 o8 =
          as_bf16x8(PF ? pf->o[qb][ks] : (row < n ? ld16(p.o_in + base + row * rs + 16 * ks + 8 * half) : zero16()));
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf((float)d8[e], (float)o8[e], acc);
    }
    acc = half_sum(acc);
    if (half == 0) di[row] = acc;
  }
  lse2[lane] = lane < n ? lv * kLog2e : INFINITY;

  for (int kb = 0; kb < 2; ++kb) {
    const int key = kb * 32 + l32;
    const bool key_ok = key < n;
    bf16x8 kf[C::NKS], vf[C::NKS];
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
      kf[ks] = as_bf16x8(lds_ld16(kt, swz_off<C::RB>(key, 2 * ks + half)));
      if constexpr (PF) vf[ks] = pf->vf[kb][ks];
      else vf[ks] = as_bf16x8(key_ok ? ld16(p.v + base + key * rs + 16 * ks + 8 * half) : zero16());
    }
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
    // dS^T rows of these keys -> LDS for the dQ product.
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int q = qb * 32 + 8 * g4 + 4 * half;
        lds_st8(st, swz_off<C::SRB>(key, q >> 3) + (q & 7) * 2,
                pack4(dp[qb][4 * g4], dp[qb][4 * g4 + 1], dp[qb][4 * g4 + 2], dp[qb][4 * g4 + 3]));
      }
    // dV^T = dO^T P and dK^T = Q^T dS for these 32 keys; complete after the single block.
    f32x16 dk[C::NDB], dv[C::NDB];
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
    if (key_ok) {
      if constexpr (PRE) {
        unrope_acc<C::NDB>(dk, epi[kb]);
      } else if constexpr (ROPE) {
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
  // dQ^T = K^T dS^T: [head dim x queries], k = keys; lane = query column.
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = qb * 32 + l32;
    f32x16 dq[C::NDB];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
      for (int i = 0; i < 16; ++i) dq[db][i] = 0.f;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
        dq[db] = mfma32(tr_operand<C::RB>(kt, 16 * tt, 32 * db, lane), tr_operand<C::SRB>(st, 16 * tt, 32 * qb, lane),
                        dq[db]);
    }
    if (row < n) {
      if constexpr (PRE) {
        unrope_acc<C::NDB>(dq, epi[qb]);
      } else if constexpr (ROPE) {
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
  __shared__ __attribute__((aligned(16))) char smem[C::NW * C::TBUF];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int prog = xcd_program_id(blockIdx.x, gridDim.x);
  const int64_t P = gridDim.x, q = p.num_tiles / P, r = p.num_tiles % P;
  const int64_t start = prog * q + min((int64_t)prog, r), end = start + q + (prog < r ? 1 : 0);
  JFA_LDS char* vt = (JFA_LDS char*)smem + wave * C::TBUF;
  for (int64_t g = start + wave; g < end; g += C::NW) {
    if (lane == 0) count_visit(p.visits, g);
    bd_fwd_tile<D, ROPE>(p, locate(p, g), vt, lane);
  }
}

template <int D, bool ROPE>
__global__ void __launch_bounds__(BdCfg<D>::NW * 64)
    __attribute__((amdgpu_waves_per_eu(1, 1))) bd_bwd_kernel(BdParams p) {
  using C = BdCfg<D>;
  __shared__ __attribute__((aligned(16))) char smem[C::NW * C::W_BWD];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int prog = xcd_program_id(blockIdx.x, gridDim.x);
  const int64_t P = gridDim.x, q = p.num_tiles / P, r = p.num_tiles % P;
  const int64_t start = prog * q + min((int64_t)prog, r), end = start + q + (prog < r ? 1 : 0);
  char* w = smem + wave * C::W_BWD;
  if constexpr (D == 64) {
    // software pipeline over the wave's tiles: stage tile g's operands (loaded during
    // the previous tile), issue the loads of tile g + NW, then compute tile g
    int64_t g = start + wave;
    if (g >= end) return;
    BdTile t = locate(p, g);
    BdBwdRegs<D> nx;
    bd_bwd_load<D>(p, t, nx, lane);
    JFA_LDS char* lw = (JFA_LDS char*)w;
    while (true) {
      bd_bwd_stage<D>(nx, lw + C::W_Q, lw + C::W_K, lw + C::W_DO, lane);
      const BdBwdRegs<D> cur = nx;
      const int64_t gn = g + C::NW;
      BdTile tn = t;
      if (gn < end) {
        tn = locate(p, gn);
        bd_bwd_load<D>(p, tn, nx, lane);
      }
      if (lane == 0) count_visit(p.visits, g);
      bd_bwd_tile<D, ROPE, true>(p, t, lw, (float*)w, lane, &cur);
      if (gn >= end) break;
      g = gn;
      t = tn;
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
