// Persistent jagged flash-attention forward for gfx950 (self and broadcast-Q modes).
//
// What it computes ("TLX Block Attention", bittide page, section 2.1, Listing 1):
// for each query row, a loop over key/value tiles keeping a running row maximum m and
// row sum l, rescaling the output accumulator by exp(m_old - m_new) when m grows, and
// finally O / l and the log-sum-exp L = m + log(l) for the backward.  The softmax is
// taken in base 2 (the forward pipeline's "exp2 / normalize" stage, same page, section
// 3.2, Fig. 1): scores are scaled by scale*log2(e) and v_exp_f32 (2^x) is used.
//
// How it maps to CDNA4:
//  * One workgroup = kFwdWaves waves = one tile of kFwdRows query rows of one
//    (sequence, head); each wave owns 64 query rows as two 32-column MFMA blocks.
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Q rows held in
//    registers for the whole tile).  In the C layout every lane then owns one query
//    column, so the row max / row sum are in-lane plus one permlane32 swap.
//  * O^T += V^T P^T: the probabilities leave the first product already in the B
//    operand layout (after a bf16 pack); V^T is fetched from the row-major V tile in
//    LDS with ds_read_b64_tr_b16.  The key order inside each 16-key step is the one
//    the C layout hands over, and the transposed fetch reads V rows in that order.
//  * K/V tiles of kFwdKeys keys are loaded with coalesced 16-byte global loads into a
//    2-slot LDS ring: the next tile's loads are in flight while the current tile
//    computes ("K/V multi-buffering", aixai.ru page, "Skeleton").
//  * Only the last key tile of a sequence is range-limited: full tiles run a
//    branch-free body, the tail runs a separately instantiated masked body (loop
//    peeling, aixai.ru page, "Loop splitting against register spills").
//  * The output is rescaled lazily: only when some row maximum grows by more than a
//    factor 2^8 (still exact: the final division uses the same stale maximum).
//  * Persistent grid: each workgroup walks its host-scheduled tile list, or takes
//    tiles from an atomic counter in dynamic mode (aixai.ru page, "Tile balancing and
//    Cluster Launch Control").
#include "jfa_device.h"
#include "jfa_internal.h"

namespace jfa {
namespace {

template <int D>
struct FwdCfg {
  static constexpr int NW = kFwdWaves;
  static constexpr int NT = NW * 64;
  static constexpr int QPW = kFwdQPerWave;
  static constexpr int NQB = QPW / 32;
  static constexpr int BM = kFwdRows;
  static constexpr int BN = kFwdKeys;
  static constexpr int NKB = BN / 32;        // 32-key blocks per tile
  static constexpr int NKS = D / 16;         // MFMA k-steps over the head dim
  static constexpr int NDB = D / 32;         // 32-wide head-dim blocks of O
  static constexpr int NT16 = BN / 16;       // 16-key k-steps of the PV product
  static constexpr int RB = D * 2;           // bytes per tile row
  static constexpr int CPR = D / 8;          // 16-byte chunks per row
  static constexpr int BUF = BN * RB;        // one K or V slot
  static_assert(NT16 == 2 * NKB, "key steps");
};

// Per-lane constants of the loop: LDS operand offsets and ring-copy offsets.
template <int D>
struct FwdLane {
  RowOperands<FwdCfg<D>::RB, FwdCfg<D>::NKS> krow;  // K rows as the A operand of S^T
  TrOperands<FwdCfg<D>::RB, FwdCfg<D>::NDB> vtr;     // V^T as the A operand of O^T
  TileCopy<FwdCfg<D>::RB, FwdCfg<D>::BN, FwdCfg<D>::NW> copy;
};

// One key/value tile for this wave's query rows.  MASK: keys >= keys_valid lie past
// the end of the sequence (tail tile only).
template <int D, bool MASK>
__device__ __forceinline__ void fwd_step(const JFA_LDS char* kbuf, const JFA_LDS char* vbuf, const FwdLane<D>& ln,
                                         const bf16x8 (&qf)[FwdCfg<D>::NQB][FwdCfg<D>::NKS],
                                         f32x16 (&o)[FwdCfg<D>::NDB][FwdCfg<D>::NQB],
                                         float (&m)[FwdCfg<D>::NQB], float (&l)[FwdCfg<D>::NQB],
                                         int lane, int keys_valid, float c) {
  using C = FwdCfg<D>;
  const int half = lane >> 5;

  // S^T = K Q^T : [keys x queries]; C layout -> lane = query column,
  // register i of key block kb <-> key 32*kb + 8*(i/4) + 4*half + i%4.
  f32x16 s[C::NKB][C::NQB];
#pragma unroll
  for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][qb][i] = 0.f;
#pragma unroll
  for (int ks = 0; ks < C::NKS; ++ks) {
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb) {
      const bf16x8 a = ln.krow.read(kbuf, kb * 32, ks);
#pragma unroll
      for (int qb = 0; qb < C::NQB; ++qb) s[kb][qb] = mfma32(a, qf[qb][ks], s[kb][qb]);
    }
  }

  if (MASK) {
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
        if (key >= keys_valid) {
#pragma unroll
          for (int qb = 0; qb < C::NQB; ++qb) s[kb][qb][i] = -INFINITY;
        }
      }
  }

  // Row maxima (raw scores; scale > 0 commutes with max) and the lazy rescale.
  float mnew[C::NQB];
  bool grow = false;
#pragma unroll
  for (int qb = 0; qb < C::NQB; ++qb) {
    float mx = s[0][qb][0];
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][qb][i]);
    mx = half_max(mx);
    mnew[qb] = fmaxf(m[qb], mx);
    grow |= (mnew[qb] - m[qb]) * c > 8.0f;
  }
  if (__ballot(grow)) {
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb) {
      const float alpha = fast_exp2((m[qb] - mnew[qb]) * c);
      m[qb] = mnew[qb];
      l[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][qb][i] *= alpha;
    }
  }

  // P = 2^(S*c - m*c); row sums; pack P into B operands of the PV product.
  bf16x8 pf[C::NQB][C::NT16];
#pragma unroll
  for (int qb = 0; qb < C::NQB; ++qb) {
    const float mc = m[qb] * c;
    float sum = 0.f;
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = fast_exp2(fmaf(s[kb][qb][i], c, -mc));
        s[kb][qb][i] = pv;
        sum += pv;
      }
    l[qb] += sum;
#pragma unroll
    for (int t = 0; t < C::NT16; ++t) {
      const f32x16& src = s[t >> 1][qb];
      const int r = 8 * (t & 1);
      pf[qb][t] = pack8(src[r], src[r + 1], src[r + 2], src[r + 3], src[r + 4], src[r + 5],
                        src[r + 6], src[r + 7]);
    }
  }

  // O^T += V^T P^T with V^T fetched transposed from the row-major V tile.
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
    for (int t = 0; t < C::NT16; ++t) {
      const bf16x8 a = ln.vtr.read(vbuf, 16 * t, db);
#pragma unroll
      for (int qb = 0; qb < C::NQB; ++qb) o[db][qb] = mfma32(a, pf[qb][t], o[db][qb]);
    }
  }
}

template <int D, int MODE>
__device__ __forceinline__ void fwd_tile(const FwdParams& p, Tile tile, JFA_LDS char* smem, const FwdLane<D>& ln,
                                         int tid) {
  using C = FwdCfg<D>;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int b = tile.b, h = tile.hb >> 24, blk = tile.hb & 0xFFFFFF;
  const int H = p.num_heads;
  const int64_t row_stride = (int64_t)H * D;
  const int64_t s0 = p.offsets[b];
  const int L = (int)(p.offsets[b + 1] - s0);
  const int Lq = (MODE == kSelf) ? L : p.num_q;
  const int row0 = blk * C::BM + wave * C::QPW;
  const float c = p.scale_log2;

  // Q rows of this wave as B operands, kept in registers for the whole tile.
  bf16x8 qf[C::NQB][C::NKS];
#pragma unroll
  for (int qb = 0; qb < C::NQB; ++qb) {
    const int row = row0 + qb * 32 + l32;
    const int64_t qrow = (MODE == kSelf) ? s0 + row : (int64_t)row;
    const uint16_t* qp = p.q + qrow * row_stride + (int64_t)h * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks)
      qf[qb][ks] = as_bf16x8(row < Lq ? ld16(qp + ks * 16) : zero16());
  }

  f32x16 o[C::NDB][C::NQB];
  float m[C::NQB], l[C::NQB];
#pragma unroll
  for (int qb = 0; qb < C::NQB; ++qb) {
    m[qb] = -INFINITY;
    l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][qb][i] = 0.f;
  }

  const int n_full = L / C::BN, tail = L % C::BN;
  const int n_kv = n_full + (tail != 0);
  if (n_kv > 0) {
    const uint32_t rsb = (uint32_t)(row_stride * 2);
    const uint16_t* kp = p.k + s0 * row_stride + (int64_t)h * D;
    const uint16_t* vp = p.v + s0 * row_stride + (int64_t)h * D;
    ln.copy.issue_rows(kp, rsb, min(C::BN, L), smem, wave, lane);
    ln.copy.issue_rows(vp, rsb, min(C::BN, L), smem + C::BUF, wave, lane);
    wait_vmem();
    __syncthreads();
    for (int it = 0; it < n_full; ++it) {
      const int cur = it & 1;
      if (it + 1 < n_kv) {
        const int64_t nxt = (int64_t)(it + 1) * C::BN * row_stride;
        const int rv = min(C::BN, L - (it + 1) * C::BN);
        JFA_LDS char* nbuf = smem + (cur ^ 1) * 2 * C::BUF;
        ln.copy.issue_rows(kp + nxt, rsb, rv, nbuf, wave, lane);
        ln.copy.issue_rows(vp + nxt, rsb, rv, nbuf + C::BUF, wave, lane);
      }
      JFA_LDS char* kbuf = smem + cur * 2 * C::BUF;
      fwd_step<D, false>(kbuf, kbuf + C::BUF, ln, qf, o, m, l, lane, C::BN, c);
      wait_vmem();
      __syncthreads();
    }
    if (tail) {
      JFA_LDS char* kbuf = smem + (n_full & 1) * 2 * C::BUF;
      fwd_step<D, true>(kbuf, kbuf + C::BUF, ln, qf, o, m, l, lane, tail, c);
      __syncthreads();
    }
  }

  // Epilogue: O / l in bf16, lse = ln 2 * (m*c + log2 l); empty rows give 0 and -inf.
#pragma unroll
  for (int qb = 0; qb < C::NQB; ++qb) {
    const float lt = half_sum(l[qb]);
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    const float lse = lt > 0.f ? (m[qb] * c + fast_log2(lt)) * kLn2 : -INFINITY;
    const int row = row0 + qb * 32 + l32;
    if (row < Lq) {
      const int64_t orow = (MODE == kSelf) ? s0 + row : (int64_t)b * p.num_q + row;
      uint16_t* op = p.o + orow * row_stride + (int64_t)h * D + 4 * half;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x16& a = o[db][qb];
          st8(op + 32 * db + 8 * g4,
              pack4(a[4 * g4] * inv, a[4 * g4 + 1] * inv, a[4 * g4 + 2] * inv, a[4 * g4 + 3] * inv));
        }
      if (half == 0) {
        const int64_t li = (MODE == kSelf) ? (int64_t)h * p.total_tokens + s0 + row
                                           : ((int64_t)b * H + h) * p.num_q + row;
        p.lse[li] = lse;
      }
    }
  }
}

template <int D, int MODE>
__global__ void __launch_bounds__(kFwdWaves * 64)
    __attribute__((amdgpu_waves_per_eu(kFwdWgPerCu * kFwdWaves / 4, kFwdWgPerCu * kFwdWaves / 4))) fwd_kernel(FwdParams p) {
  using C = FwdCfg<D>;
  __shared__ __attribute__((aligned(16))) char smem_raw[4 * C::BUF];
  __shared__ int next_tile;
  JFA_LDS char* smem = (JFA_LDS char*)smem_raw;
  const int tid = threadIdx.x;
  const int prog = xcd_program_id(blockIdx.x, gridDim.x);
  FwdLane<D> ln;
  ln.krow.init(tid & 63);
  ln.vtr.init(tid & 63);
  ln.copy.init((uint32_t)(p.num_heads * D * 2), tid >> 6, tid & 63);
  int idx, end;
  if (!p.dynamic) {
    idx = p.seg_ptr[prog];
    end = p.seg_ptr[prog + 1];
  } else {
    idx = prog;
    end = p.seg_ptr[1];
  }
  while (idx < end) {
    fwd_tile<D, MODE>(p, p.tiles[idx], smem, ln, tid);
    if (!p.dynamic) {
      ++idx;
    } else {
      if (tid == 0) next_tile = p.num_programs + atomicAdd(p.counters, 1);
      __syncthreads();
      idx = next_tile;
      __syncthreads();
    }
  }
}

template <int D, int MODE>
hipError_t launch(const FwdParams& p, hipStream_t s) {
  hipLaunchKernelGGL((fwd_kernel<D, MODE>), dim3(p.num_programs), dim3(kFwdWaves * 64), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p, int mode, int head_dim, hipStream_t s) {
  if (p.num_programs <= 0) return hipSuccess;
  if (mode == kSelf) return head_dim == 64 ? launch<64, kSelf>(p, s) : launch<128, kSelf>(p, s);
  return head_dim == 64 ? launch<64, kBroadcastQ>(p, s) : launch<128, kBroadcastQ>(p, s);
}

}  // namespace jfa
