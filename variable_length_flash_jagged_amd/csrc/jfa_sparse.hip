// Block-sparse top-k variant, stage 1, for gfx950: block means of Q and K and the
// top-k key blocks of every query block.
//
// What it computes ("Jagged Flash Attention on TLX", aixai.ru, closing section on
// variants: a cheap kernel averages blocks of Q and K and keeps the most relevant ones
// for the attention kernel).  Readings: query blocks are the forward's 256-row tiles,
// key blocks its 64-key tiles, a block is pooled to the mean of its rows, relevance is
// the dot product of the two means, each query block keeps
// k = max(1, ceil(ratio * nkb)) key blocks, ties going to the lower block index.  The
// kept lists are written in ascending block order, so a sequence's partial last key
// block, when kept, is the last entry -- the forward kernel's tail rule.
//
// How it maps to CDNA4: both kernels are memory bound and tiny next to the attention.
// pool_kernel gives one wave to one (block, head): every row is one 256-byte (D=128)
// or 128-byte (D=64) coalesced load, summed in fp32 in row order.  select_kernel gives
// one wave to one (query block, head): lane j forms the scores of key blocks
// j, j + 64, ... (fp32, head-dim order) into the wave's LDS row, then each lane ranks
// its blocks against all scores of the sequence (broadcast LDS reads) and a ballot
// turns the kept flags into ascending positions.  Grid-stride loops are per wave, so
// the only synchronisation is within a wave.
#include "jfa_device.h"
#include "jfa_internal.h"

namespace jfa {
namespace {

// Sequence of global block g: the b with prefix[b] <= g < prefix[b+1] (empty sequences
// are skipped because prefix[b] == prefix[b+1] for them).
__device__ __forceinline__ int find_seq(const int32_t* prefix, int num_seqs, int g) {
  int lo = 0, hi = num_seqs;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (prefix[mid] <= g) lo = mid;
    else hi = mid;
  }
  return lo;
}

template <int D>
__global__ void __launch_bounds__(256) pool_kernel(PoolParams p) {
  constexpr int CPL = D / 64;  // columns per lane
  const int lane = threadIdx.x & 63;
  const int64_t total = (int64_t)p.nblocks * p.heads;
  const int64_t stride = (int64_t)gridDim.x * 4;
  for (int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); g < total; g += stride) {
    const int blk = (int)(g / p.heads), h = (int)(g - (int64_t)blk * p.heads);
    const int b = find_seq(p.blk_prefix, p.num_seqs, blk);
    const int j = blk - p.blk_prefix[b];
    const int64_t s0 = p.offsets[b];
    const int L = (int)(p.offsets[b + 1] - s0);
    const int n = min(p.block, L - j * p.block);
    const uint16_t* x = p.x + ((s0 + (int64_t)j * p.block) * p.heads + h) * D + CPL * lane;
    const int64_t rs = (int64_t)p.heads * D;
    float acc[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
#pragma unroll 8
    for (int r = 0; r < n; ++r) {
      if (CPL == 2) {
        const uint32_t u = *reinterpret_cast<const uint32_t*>(x + r * rs);
        acc[0] += __uint_as_float(u << 16);
        acc[CPL - 1] += __uint_as_float(u & 0xFFFF0000u);
      } else {
        acc[0] += __uint_as_float((uint32_t)x[r * rs] << 16);
      }
    }
    float* out = p.out + ((int64_t)h * p.nblocks + blk) * D + CPL * lane;
    const float inv = 1.0f / (float)n;
#pragma unroll
    for (int c = 0; c < CPL; ++c) out[c] = acc[c] * inv;
  }
}

template <int D>
__global__ void __launch_bounds__(256) select_kernel(SelectParams p) {
  __shared__ float sc_all[4][kSparseMaxKeyBlocks];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float* sc = sc_all[wv];
  const int H = p.num_heads, group = H / p.num_kv_heads;
  const int64_t total = (int64_t)p.nqt * H;
  const int64_t stride = (int64_t)gridDim.x * 4;
  for (int64_t g = (int64_t)blockIdx.x * 4 + wv; g < total; g += stride) {
    const int qt = (int)(g / H), h = (int)(g - (int64_t)qt * H);
    const int b = find_seq(p.qt_prefix, p.num_seqs, qt);
    const int i = qt - p.qt_prefix[b];
    const int nqt_b = p.qt_prefix[b + 1] - p.qt_prefix[b];
    const int nkb_b = p.kb_prefix[b + 1] - p.kb_prefix[b];
    const int kk = p.sel_k[b];
    const float* qv = p.qbar + ((int64_t)h * p.nqt + qt) * D;
    const float* kv0 = p.kbar + ((int64_t)(h / group) * p.nkb + p.kb_prefix[b]) * D;
    for (int jb = lane; jb < nkb_b; jb += 64) {
      const float* kv = kv0 + (int64_t)jb * D;
      float s = 0.f;
#pragma unroll 8
      for (int d = 0; d < D; ++d) s = fmaf(qv[d], kv[d], s);
      sc[jb] = s == s ? s : -INFINITY;  // NaN ranks last, so exactly kk blocks are kept
    }
    // the scores of this wave's sequence are read by every lane of the wave
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
    int32_t* out = p.sel + p.sel_base[b] + ((int64_t)h * nqt_b + i) * kk;
    int base = 0;
    for (int c0 = 0; c0 < nkb_b; c0 += 64) {
      const int jb = c0 + lane;
      bool keep = false;
      if (jb < nkb_b) {
        const float si = sc[jb];
        int rank = 0;
        for (int j = 0; j < nkb_b; ++j) {
          const float sj = sc[j];
          rank += (sj > si) || (sj == si && j < jb);
        }
        keep = rank < kk;
      }
      const uint64_t m = __ballot(keep);
      if (keep) out[base + __popcll(m & ((1ull << lane) - 1ull))] = jb;
      base += __popcll(m);
    }
    // the LDS row is rewritten by the next tile of this wave
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
  }
}

// Block-sparse backward, inverse of the selection: one thread per selection entry sets
// the bit of its query block in the bitmap of the key block's dK/dV tile half.  Bits
// are only ever set (atomic OR), so the result does not depend on the order of the
// threads.  Entries outside [0, nkb) are ignored (they cannot come from the select
// kernel), so no write leaves the sequence's bitmaps.
__global__ void __launch_bounds__(256) mark_kernel(MarkParams p) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < p.entries; e += stride) {
    int lo = 0, hi = p.num_seqs;  // sequence b: sel_base[b] <= e < sel_base[b + 1]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.sel_base[mid] <= e) lo = mid;
      else hi = mid;
    }
    const int b = lo;
    const int L = p.offsets[b + 1] - p.offsets[b];
    const int nqb = (L + kSparseQBlock - 1) / kSparseQBlock, nkb = (L + kSparseKBlock - 1) / kSparseKBlock;
    const int nj = (L + kBwdKeys - 1) / kBwdKeys, nw = (nqb + 31) / 32;
    const int64_t r = e - p.sel_base[b];
    const int64_t list = r / p.sel_k[b];
    const int h = (int)(list / nqb), i = (int)(list - (int64_t)h * nqb);
    const int kb = p.sel[e];
    if (kb < 0 || kb >= nkb) continue;
    uint32_t* w = p.bits + p.bits_base[b] + (((int64_t)h * nj + (kb >> 1)) * 2 + (kb & 1)) * nw + (i >> 5);
    atomicOr(w, 1u << (i & 31));
  }
}

template <class K, class P>
hipError_t launch_grid(K kernel, const P& p, int64_t waves, hipStream_t s) {
  if (waves <= 0) return hipSuccess;
  const int grid = (int)std::min<int64_t>((waves + 3) / 4, 8192);
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pool(const PoolParams& p, int head_dim, hipStream_t s) {
  const int64_t waves = (int64_t)p.nblocks * p.heads;
  return head_dim == 64 ? launch_grid(pool_kernel<64>, p, waves, s) : launch_grid(pool_kernel<128>, p, waves, s);
}

hipError_t launch_select(const SelectParams& p, int head_dim, hipStream_t s) {
  const int64_t waves = (int64_t)p.nqt * p.num_heads;
  return head_dim == 64 ? launch_grid(select_kernel<64>, p, waves, s) : launch_grid(select_kernel<128>, p, waves, s);
}

hipError_t launch_mark(const MarkParams& p, hipStream_t s) {
  if (p.entries <= 0) return hipSuccess;
  const int grid = (int)std::min<int64_t>((p.entries + 255) / 256, 8192);
  hipLaunchKernelGGL(mark_kernel, dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace jfa
