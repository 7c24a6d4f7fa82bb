// Jagged flash-attention backward for gfx950 (self and broadcast-Q modes), plus the
// dQ accumulator kernels (zero fill, fp32 -> bf16 cast, broadcast-Q partial reduce).
//
// What it computes: the analytic gradient of sum(O * dO) with P rebuilt from the
// forward's log-sum-exp, P = exp(scale * Q K^T - L) (the L kept for the backward,
// "TLX Block Attention", bittide page, section 2.1), Di = rowsum(dO * O) computed inline
// instead of in a separate launch (same page, sections 2.1 and 4), and the five
// products per key/value block (aixai.ru page, "Paired CTAs"):
//   S = Q K^T, dP = dO V^T, dV += P^T dO, dS = P * (dP - Di), dK += scale dS^T Q,
//   dQ += scale dS K.
// In broadcast-Q mode dQ is summed over all sequences (aixai.ru page, "What is Jagged
// Flash Attention"; "dQ epilogue").
//
// How it maps to CDNA4:
//  * One workgroup = 4 waves = one tile of kBwdKeys (128) key rows of one
//    (sequence, head); wave w owns keys 32w..32w+31 and keeps their K, V operands and
//    the fp32 dK^T, dV^T accumulators in registers for the whole tile.
//  * The loop streams 64 query rows at a time: Q and dO land in double-buffered,
//    swizzled LDS tiles through direct global->LDS copies issued one step ahead; O and
//    lse for the next step are prefetched into registers and Di is formed from them.
//  * S and dP come out in the MFMA C layout with lane = key, which is already the B
//    operand layout of dV^T += dO^T P and dK^T += Q^T dS; dO^T and Q^T are read from
//    the row-major LDS tiles with ds_read_b64_tr_b16.
//  * dS^T goes to LDS once (bf16); after one barrier each wave computes a 64 x 32 (or
//    32 x 32) block of this tile's dQ contribution over all 128 keys (A = dS from
//    LDS, transposed read; B = K^T fragments read once per tile), so dQ leaves the
//    workgroup once per 128 keys.
//  * dQ hand-off: self mode and broadcast-Q path 0 add into an fp32 accumulator with
//    hardware float atomics; broadcast-Q path 1 gives every program its own fp32 slab
//    (plain read-modify-write: the head-pinned schedule keeps one head per program)
//    and a second kernel sums the slabs of each head.
#include "jfa_device.h"
#include "jfa_internal.h"
#include "jfa_sched.h"

namespace jfa {
namespace {

template <int D>
struct BwdCfg {
  static constexpr int NW = kBwdWaves;
  static constexpr int NT = NW * 64;
  static constexpr int BN = kBwdKeys;   // keys per tile
  static constexpr int QB = kBwdRows;   // query rows per step
  static constexpr int NQB = QB / 32;
  static constexpr int NKS = D / 16;
  static constexpr int NDB = D / 32;
  static constexpr int NT16 = QB / 16;  // 16-row k-steps of dV / dK products
  static constexpr int NK16 = BN / 16;  // 16-key k-steps of the dQ product
  static constexpr int RB = 2 * D;      // bytes per Q / dO / K tile row
  static constexpr int QBUF = QB * RB;
  static constexpr int KBUF = BN * RB;
  static constexpr int SRB = 2 * QB;    // bytes per dS^T row (one key, QB queries)
  static constexpr int SBUF = BN * SRB;
  // dQ product split over the waves: (query block, head-dim block) pairs.
  static constexpr int DQ_NQB = (NDB >= NW) ? NQB : 1;
  static constexpr int CPR = D / 8;              // 16-byte chunks per row
  static constexpr int DI_ROWS_PER_PASS = NT / CPR;
  static constexpr int DI_PASSES = QB / DI_ROWS_PER_PASS;
  // LDS map (bytes)
  static constexpr int OFF_Q = 0;                       // [2][QBUF]
  static constexpr int OFF_DO = OFF_Q + 2 * QBUF;       // [2][QBUF]
  static constexpr int OFF_K = OFF_DO + 2 * QBUF;       // [KBUF]
  static constexpr int OFF_S = OFF_K + KBUF;            // [SBUF]
  static constexpr int OFF_LSE = OFF_S + SBUF;          // float [2][QB]
  static constexpr int OFF_DI = OFF_LSE + 2 * QB * 4;   // float [2][QB]
  static constexpr int SMEM = OFF_DI + 2 * QB * 4;
  static_assert(NDB * NQB == NW * DQ_NQB, "dQ split");
};

template <int D>
struct StepPrefetch {
  u32x4 o[BwdCfg<D>::DI_PASSES];
  float lse;
};

// Issue the next step's copies (Q, dO -> LDS) and register loads (O rows for Di, lse).
template <int D>
__device__ __forceinline__ void prefetch_step(const uint16_t* qb, const uint16_t* dob, const uint16_t* ob,
                                              const float* lseb, int64_t rs, int row0, int rows_valid,
                                              JFA_LDS char* qbuf, JFA_LDS char* dobuf, StepPrefetch<D>& pf,
                                              int tid, int wave, int lane) {
  using C = BwdCfg<D>;
  dma_tile<C::RB, C::QB, C::NW>(qb + (int64_t)row0 * rs, rs, rows_valid, qbuf, wave, lane);
  dma_tile<C::RB, C::QB, C::NW>(dob + (int64_t)row0 * rs, rs, rows_valid, dobuf, wave, lane);
  const int c = tid % C::CPR;
#pragma unroll
  for (int j = 0; j < C::DI_PASSES; ++j) {
    const int r = tid / C::CPR + j * C::DI_ROWS_PER_PASS;
    pf.o[j] = r < rows_valid ? ld16(ob + (int64_t)(row0 + r) * rs + c * 8) : zero16();
  }
  pf.lse = (tid < C::QB && tid < rows_valid) ? lseb[row0 + tid] : 0.f;
}

// Di = rowsum(dO * O) for the prefetched step (dO from its LDS tile, O from registers)
// and lse in base 2 (+inf for rows past the end, which zeroes their probabilities).
template <int D>
__device__ __forceinline__ void finish_step(const StepPrefetch<D>& pf, const JFA_LDS char* dobuf,
                                            float* lse2, float* di, int rows_valid, int tid) {
  using C = BwdCfg<D>;
  const int c = tid % C::CPR;
#pragma unroll
  for (int j = 0; j < C::DI_PASSES; ++j) {
    const int r = tid / C::CPR + j * C::DI_ROWS_PER_PASS;
    const bf16x8 d8 = as_bf16x8(lds_ld16(dobuf, swz_off<C::RB>(r, c)));
    const bf16x8 o8 = as_bf16x8(pf.o[j]);
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf((float)d8[e], (float)o8[e], acc);
#pragma unroll
    for (int m = C::CPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
    if (c == 0) di[r] = acc;
  }
  if (tid < C::QB) lse2[tid] = tid < rows_valid ? pf.lse * kLog2e : INFINITY;
}

template <int D, int MODE>
__device__ __forceinline__ void bwd_tile(const BwdParams& p, Tile tile, int prog, char* smem_raw, int tid) {
  using C = BwdCfg<D>;
  JFA_LDS char* smem = (JFA_LDS char*)smem_raw;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int b = tile.b, h = tile.hb >> 24, j = tile.hb & 0xFFFFFF;
  const int H = p.num_heads;
  const int64_t rs = (int64_t)H * D;
  const int64_t s0 = p.offsets[b];
  const int L = (int)(p.offsets[b + 1] - s0);
  const int Lq = (MODE == kSelf) ? L : p.num_q;
  const int key0 = j * C::BN;
  const int keys_tile = min(C::BN, L - key0);
  const int my_key = wave * 32 + l32;  // key row within the tile (B-operand lane)
  const bool key_ok = my_key < keys_tile;
  const float c = p.scale_log2;

  const uint16_t* kb = p.k + (s0 + key0) * rs + (int64_t)h * D;
  const uint16_t* vb = p.v + (s0 + key0) * rs + (int64_t)h * D;
  const uint16_t *qb, *dob, *ob;
  const float* lseb;
  if (MODE == kSelf) {
    qb = p.q + s0 * rs + (int64_t)h * D;
    dob = p.dout + s0 * rs + (int64_t)h * D;
    ob = p.o + s0 * rs + (int64_t)h * D;
    lseb = p.lse + (int64_t)h * p.total_tokens + s0;
  } else {
    qb = p.q + (int64_t)h * D;
    dob = p.dout + (int64_t)b * p.num_q * rs + (int64_t)h * D;
    ob = p.o + (int64_t)b * p.num_q * rs + (int64_t)h * D;
    lseb = p.lse + ((int64_t)b * H + h) * p.num_q;
  }
  JFA_LDS char* kt = smem + C::OFF_K;
  JFA_LDS char* st = smem + C::OFF_S;
  float* lse2 = (float*)(smem_raw + C::OFF_LSE);
  float* di = (float*)(smem_raw + C::OFF_DI);
  const int nq = (Lq + C::QB - 1) / C::QB;

  // Prologue: K tile -> LDS, first Q / dO step, V operands straight from global.
  dma_tile<C::RB, C::BN, C::NW>(kb, rs, keys_tile, kt, wave, lane);
  StepPrefetch<D> pre;
  prefetch_step<D>(qb, dob, ob, lseb, rs, 0, min(C::QB, Lq), smem + C::OFF_Q, smem + C::OFF_DO, pre, tid,
                   wave, lane);
  bf16x8 vf[C::NKS];
#pragma unroll
  for (int ks = 0; ks < C::NKS; ++ks)
    vf[ks] = as_bf16x8(key_ok ? ld16(vb + (int64_t)my_key * rs + 16 * ks + 8 * half) : zero16());
  wait_vmem();
  __syncthreads();
  bf16x8 kf[C::NKS];
#pragma unroll
  for (int ks = 0; ks < C::NKS; ++ks) kf[ks] = as_bf16x8(lds_ld16(kt, swz_off<C::RB>(my_key, 2 * ks + half)));
  const int dq_db = (C::NDB >= C::NW) ? wave : (wave % C::NDB);
  const int dq_qb0 = (C::NDB >= C::NW) ? 0 : (wave / C::NDB);
  finish_step<D>(pre, smem + C::OFF_DO, lse2, di, min(C::QB, Lq), tid);
  __syncthreads();

  f32x16 dk[C::NDB], dv[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dk[db][i] = dv[db][i] = 0.f;

  for (int it = 0; it < nq; ++it) {
    const int cur = it & 1;
    const int row0 = it * C::QB;
    JFA_LDS char* qt = smem + C::OFF_Q + cur * C::QBUF;
    JFA_LDS char* dot = smem + C::OFF_DO + cur * C::QBUF;
    const bool has_next = it + 1 < nq;
    const int next_rows = min(C::QB, Lq - row0 - C::QB);
    if (has_next)
      prefetch_step<D>(qb, dob, ob, lseb, rs, row0 + C::QB, next_rows, smem + C::OFF_Q + (cur ^ 1) * C::QBUF,
                       smem + C::OFF_DO + (cur ^ 1) * C::QBUF, pre, tid, wave, lane);

    // One 32-row query block at a time: S = Q K^T and dP = dO V^T ([queries x keys],
    // C layout -> lane = key), P = 2^(S*c - lse2) (zero for keys past the end),
    // dS = P * (dP - Di), then dV^T += dO^T P and dK^T += Q^T dS ([head dim x keys],
    // k = query rows) and dS^T -> LDS.
    const float* l2 = lse2 + cur * C::QB;
    const float* dd = di + cur * C::QB;
#pragma unroll
    for (int qq = 0; qq < C::NQB; ++qq) {
      f32x16 s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < C::NKS; ++ks) {
        const int off = swz_off<C::RB>(qq * 32 + l32, 2 * ks + half);
        s = mfma32(as_bf16x8(lds_ld16(qt, off)), kf[ks], s);
        dp = mfma32(as_bf16x8(lds_ld16(dot, off)), vf[ks], dp);
      }
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int r4 = qq * 32 + 8 * g4 + 4 * half;
        const float4 lv = *reinterpret_cast<const float4*>(l2 + r4);
        const float4 dv4 = *reinterpret_cast<const float4*>(dd + r4);
        const float la[4] = {lv.x, lv.y, lv.z, lv.w};
        const float da[4] = {dv4.x, dv4.y, dv4.z, dv4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * g4 + e;
          float pv = fast_exp2(fmaf(s[i], c, -la[e]));
          pv = key_ok ? pv : 0.f;
          s[i] = pv;
          dp[i] = pv * (dp[i] - da[e]);
        }
      }
      bf16x8 pf[2], dsf[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int r = 8 * u;
        pf[u] = pack8(s[r], s[r + 1], s[r + 2], s[r + 3], s[r + 4], s[r + 5], s[r + 6], s[r + 7]);
        dsf[u] = pack8(dp[r], dp[r + 1], dp[r + 2], dp[r + 3], dp[r + 4], dp[r + 5], dp[r + 6], dp[r + 7]);
      }
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int t = 2 * qq + u;
          dv[db] = mfma32(tr_operand<C::RB>(dot, 16 * t, 32 * db, lane), pf[u], dv[db]);
          dk[db] = mfma32(tr_operand<C::RB>(qt, 16 * t, 32 * db, lane), dsf[u], dk[db]);
        }
      }
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int q = qq * 32 + 8 * g4 + 4 * half;
        lds_st8(st, swz_off<C::SRB>(my_key, q >> 3) + (q & 7) * 2,
                pack4(dp[4 * g4], dp[4 * g4 + 1], dp[4 * g4 + 2], dp[4 * g4 + 3]));
      }
    }
    wait_vmem();
    __syncthreads();

    // dQ block(s) of this wave: [queries x head dim] over all 128 keys of the tile;
    // the K^T operand comes from the K tile that stays in LDS for the whole tile.
    f32x16 dqa[C::DQ_NQB];
#pragma unroll
    for (int u = 0; u < C::DQ_NQB; ++u)
#pragma unroll
      for (int i = 0; i < 16; ++i) dqa[u][i] = 0.f;
#pragma unroll
    for (int t = 0; t < C::NK16; ++t) {
      const bf16x8 kt_op = tr_operand<C::RB>(kt, 16 * t, 32 * dq_db, lane);
#pragma unroll
      for (int u = 0; u < C::DQ_NQB; ++u)
        dqa[u] = mfma32(tr_operand<C::SRB>(st, 16 * t, 32 * (dq_qb0 + u), lane), kt_op, dqa[u]);
    }
#pragma unroll
    for (int u = 0; u < C::DQ_NQB; ++u) {
      const int qq = dq_qb0 + u;
      const f32x16& acc = dqa[u];
      const int d = 32 * dq_db + l32;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qrow = row0 + qq * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
        if (qrow < Lq) {
          if (MODE == kSelf) {
            unsafeAtomicAdd(p.dq_acc + (s0 + qrow) * rs + (int64_t)h * D + d, acc[i]);
          } else if (!p.dq_partials) {
            unsafeAtomicAdd(p.dq_acc + (int64_t)qrow * rs + (int64_t)h * D + d, acc[i]);
          } else {
            float* a = p.dq_acc + ((int64_t)prog * p.num_q + qrow) * D + d;
            *a += acc[i];
          }
        }
      }
    }

    if (has_next)
      finish_step<D>(pre, smem + C::OFF_DO + (cur ^ 1) * C::QBUF, lse2 + (cur ^ 1) * C::QB,
                     di + (cur ^ 1) * C::QB, next_rows, tid);
    __syncthreads();
  }

  // dK = scale * dK^T^T, dV: lane = key, 4 consecutive head-dim columns per store.
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

template <int D, int MODE>
__global__ void __launch_bounds__(kBwdWaves * 64)
    __attribute__((amdgpu_waves_per_eu(kBqWgPerCu, kBqWgPerCu))) bwd_kernel(BwdParams p) {
  using C = BwdCfg<D>;
  __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
  __shared__ int next_tile;
  const int tid = threadIdx.x;
  const int prog = xcd_program_id(blockIdx.x, gridDim.x);
  // Counter groups: one per head in broadcast-Q mode (head-pinned), one per XCD otherwise.
  const int gsize = (MODE == kBroadcastQ) ? p.programs_per_head : p.num_programs / dynamic_groups(p.num_programs);
  const int grp = prog / gsize, rank = prog % gsize;
  int idx, end, base = 0;
  if (!p.dynamic) {
    idx = p.seg_ptr[prog];
    end = p.seg_ptr[prog + 1];
  } else {
    base = p.seg_ptr[grp];
    end = p.seg_ptr[grp + 1];
    idx = base + rank;
  }
  while (idx < end) {
    if (tid == 0) count_visit(p.visits, idx);
    bwd_tile<D, MODE>(p, p.tiles[idx], prog, smem, tid);
    if (!p.dynamic) {
      ++idx;
    } else {
      if (tid == 0) next_tile = base + gsize + atomicAdd(p.counters + grp, 1);
      __syncthreads();
      idx = next_tile;
      __syncthreads();
    }
  }
}

template <int D, int MODE>
hipError_t launch(const BwdParams& p, hipStream_t s) {
  hipLaunchKernelGGL((bwd_kernel<D, MODE>), dim3(p.num_programs), dim3(kBwdWaves * 64), 0, s, p);
  return hipGetLastError();
}

__global__ void fill_zero_kernel(float* x, int64_t n) {
  const int64_t n4 = n / 4;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x)
    reinterpret_cast<float4*>(x)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int64_t i = n4 * 4 + blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    x[i] = 0.f;
}

__global__ void cast_scale_kernel(const float* src, uint16_t* dst, int64_t n, float scale) {
  const int64_t n8 = n / 8;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n8; i += (int64_t)gridDim.x * blockDim.x) {
    const float4 a = reinterpret_cast<const float4*>(src)[2 * i];
    const float4 b = reinterpret_cast<const float4*>(src)[2 * i + 1];
    const bf16x8 r = pack8(a.x * scale, a.y * scale, a.z * scale, a.w * scale, b.x * scale, b.y * scale,
                           b.z * scale, b.w * scale);
    st16(dst + 8 * i, __builtin_bit_cast(u32x4, r));
  }
}

// dq[q, h, d] = bf16(scale * sum over programs g of group h of partials[g, q, d]).
__global__ void dq_reduce_kernel(const float* part, uint16_t* dq, int num_q, int num_heads, int head_dim,
                                 int ph, float scale) {
  const int64_t n8 = (int64_t)num_q * num_heads * head_dim / 8;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n8; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = 8 * i;
    const int d = (int)(e % head_dim);
    const int h = (int)((e / head_dim) % num_heads);
    const int64_t q = e / ((int64_t)head_dim * num_heads);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int g = h * ph; g < (h + 1) * ph; ++g) {
      const float* src = part + ((int64_t)g * num_q + q) * head_dim + d;
      const float4 a = reinterpret_cast<const float4*>(src)[0];
      const float4 b = reinterpret_cast<const float4*>(src)[1];
      acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
      acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
    }
    const bf16x8 r = pack8(acc[0] * scale, acc[1] * scale, acc[2] * scale, acc[3] * scale, acc[4] * scale,
                           acc[5] * scale, acc[6] * scale, acc[7] * scale);
    st16(dq + e, __builtin_bit_cast(u32x4, r));
  }
}

// Chunk slabs [nc, E] (E = Mq * H * D, a multiple of 8), every one written in full by the
// dQ kernel, are summed in a fixed order (run-to-run deterministic): group g of
// kReduceGroups sums its contiguous range of slabs in order, then dq[e] = bf16(scale *
// sum of the group sums in group order).  One workgroup per 16 four-float columns: its
// 256 lanes are (group, column), each summing one group of one column; the group sums
// meet in LDS and 16 lanes add them up.
constexpr int kReduceGroups = 16;

__device__ __forceinline__ int64_t group_first(int g, int groups, int nc) { return (int64_t)g * nc / groups; }

__global__ void __launch_bounds__(256) dq_chunk_reduce_kernel(const float* __restrict__ slabs,
                                                              uint16_t* __restrict__ dq, int nc, int groups,
                                                              int64_t slab_elems, float scale) {
  __shared__ float4 part[kReduceGroups][16];
  const int64_t n4 = slab_elems / 4;
  const int c = threadIdx.x & 15, g = threadIdx.x >> 4;
  const float4* col = reinterpret_cast<const float4*>(slabs);
  for (int64_t c0 = (int64_t)blockIdx.x * 16; c0 < n4; c0 += (int64_t)gridDim.x * 16) {
    const int64_t i = c0 + c;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (g < groups && i < n4) {
      const int64_t first = group_first(g, groups, nc), last = group_first(g + 1, groups, nc);
      if (last > first) {
        acc = col[first * n4 + i];
        for (int64_t k = first + 1; k < last; ++k) {
          const float4 a = col[k * n4 + i];
          acc.x += a.x; acc.y += a.y; acc.z += a.z; acc.w += a.w;
        }
      }
    }
    part[g][c] = acc;
    __syncthreads();
    if (g == 0 && i < n4) {
      float4 tot = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int gg = 0; gg < groups; ++gg) {
        if (group_first(gg + 1, groups, nc) == group_first(gg, groups, nc)) continue;
        const float4 a = part[gg][c];
        tot.x += a.x; tot.y += a.y; tot.z += a.z; tot.w += a.w;
      }
      st8(dq + 4 * i, pack4(tot.x * scale, tot.y * scale, tot.z * scale, tot.w * scale));
    }
    __syncthreads();
  }
}

int grid_for(int64_t work, int block) {
  const int64_t g = (work + block - 1) / block;
  return (int)(g < 1 ? 1 : (g > 4096 ? 4096 : g));
}

}  // namespace

hipError_t launch_bwd(const BwdParams& p, int mode, int head_dim, hipStream_t s) {
  if (p.num_programs <= 0) return hipSuccess;
  if (mode != kBroadcastQ) return hipErrorInvalidValue;  // self mode: launch_bwd_self
  return head_dim == 64 ? launch<64, kBroadcastQ>(p, s) : launch<128, kBroadcastQ>(p, s);
}

hipError_t launch_fill_zero(float* x, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(n / 4 + 1, 256)), dim3(256), 0, s, x, n);
  return hipGetLastError();
}

hipError_t launch_cast_scale(const float* src, uint16_t* dst, int64_t n, float scale, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(cast_scale_kernel, dim3(grid_for(n / 8, 256)), dim3(256), 0, s, src, dst, n, scale);
  return hipGetLastError();
}

hipError_t launch_dq_reduce(const float* partials, uint16_t* dq, int num_q, int num_heads, int head_dim,
                            int programs_per_head, float scale, hipStream_t s) {
  const int64_t n8 = (int64_t)num_q * num_heads * head_dim / 8;
  if (n8 <= 0) return hipSuccess;
  hipLaunchKernelGGL(dq_reduce_kernel, dim3(grid_for(n8, 256)), dim3(256), 0, s, partials, dq, num_q, num_heads,
                     head_dim, programs_per_head, scale);
  return hipGetLastError();
}

hipError_t launch_dq_seq_reduce(float* slabs, uint16_t* dq, int num_slabs, int64_t slab_elems, float scale,
                                hipStream_t s) {
  if (slab_elems <= 0) return hipSuccess;
  const int groups = num_slabs < kReduceGroups ? num_slabs : kReduceGroups;
  hipLaunchKernelGGL(dq_chunk_reduce_kernel, dim3(grid_for(slab_elems / 4, 16)), dim3(256), 0, s, slabs, dq,
                     num_slabs, groups, slab_elems, scale);
  return hipGetLastError();
}

}  // namespace jfa
