// MXFP8 variant of the jagged self-attention forward for gfx950: OCP MX quantisation
// kernels and a forward kernel on the block-scaled FP8 matrix instruction.
//
// What it computes ("Jagged Flash Attention on TLX", aixai.ru, closing section on
// variants: MXFP8 inputs with block scales, P quantised on the fly, the same pipeline).
// MXFP8 is the OCP Microscaling format: 32 elements share one E8M0 scale 2^X and each
// element is FP8 E4M3.  Quantisation follows the OCP rule: X = floor(log2 max|x|) - 8,
// elements x / 2^X rounded to nearest E4M3 (ties to even) and clamped to +-448, X = 0
// for an all-zero block.  Q and K are blocked along the head dimension (the contraction
// of Q K^T), V along each sequence's keys (the contraction of P V), 32 keys from the
// sequence's start.  The forward keeps S, the running maximum and the row sums in fp32
// and quantises P per 32 keys of a row with the smallest power-of-two scale that keeps
// the block's largest value at most 448.
//
// How it maps to CDNA4.  v_mfma_scale_f32_32x32x64_f8f6f4 multiplies 32x64 by 64x32
// E4M3 operands with one E8M0 scale per lane: lane l holds 32 bytes of row (or column)
// l % 32, byte t being element k = 32 (t / 16) + 16 (l / 32) + t % 16 of the 64, and
// its scale applies to k-block l / 32 (k = 32 (l / 32) .. + 31) of that row -- so the
// 32 elements of one MX block are bytes 0-15 (or 16-31) of lanes r and r + 32 (measured
// with in-bounds probes).  S^T = K Q^T takes K rows as A in a permuted order, key
// 32 b + 16 h + 4 g + j for A row 8 g + 4 h + j of key block b, so that the C layout
// leaves, in lane (query n, half h), exactly the keys 32 b + 16 h + i (register i of
// block b) that P's B operand of O^T = V^T P^T needs in byte 16 b + i: P goes from the
// softmax to the second product without leaving registers, and a block's 32 values sit
// in lanes n and n + 32, whose maxima are combined with one lane swap.  V is stored
// transposed per head ([D][keys], each sequence padded to 64 keys), so V^T's A operand
// is two plain 16-byte reads of one LDS row.  One workgroup = 8 (D = 128) or 4 (D = 64)
// waves x 32 query rows, two waves per SIMD;
// each 64-key step's K tile, V^T tile and their scales are loaded into registers one
// step ahead and written to XOR-swizzled LDS tiles between two barriers.
#include <stdlib.h>
#include <algorithm>
#include <type_traits>

#include "jfa_device.h"
#include "jfa_internal.h"

namespace jfa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// OCP MX shared exponent of a block whose largest magnitude is amax.
__device__ __forceinline__ int mx_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  return min(max(ilogbf(amax) - 8, -127), 127);
}

// E4M3 byte of x (already divided by its block scale), ties to even, clamped to 448 (the
// conversion instruction turns values above 448 into NaN instead of saturating).
template <bool HI>
__device__ __forceinline__ uint32_t e4m3_pair(float a, float b, uint32_t old) {
  a = fminf(fmaxf(a, -448.f), 448.f);
  b = fminf(fmaxf(b, -448.f), 448.f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}

// Quantise 32 fp32 values with the block exponent x into 8 dwords.
__device__ __forceinline__ void quantise32(const float (&v)[32], int x, uint32_t (&out)[8]) {
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    uint32_t d = 0;
    d = e4m3_pair<false>(ldexpf(v[4 * w], -x), ldexpf(v[4 * w + 1], -x), d);
    d = e4m3_pair<true>(ldexpf(v[4 * w + 2], -x), ldexpf(v[4 * w + 3], -x), d);
    out[w] = d;
  }
}

// ---------------------------------------------------------------- quantisation

// Q or K [T, H, D] bf16 -> codes [T, H, D], exponents + 127 [T, H, D/32]: one thread
// per block of 32 consecutive elements of a row.
__global__ void __launch_bounds__(256) quant_qk_kernel(MxQuantParams p) {
  const int64_t nblk = p.rows * (p.head_dim / 32);
  for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < nblk; g += (int64_t)gridDim.x * 256) {
    const uint16_t* src = p.x + g * 32;
    float v[32];
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bf16x8 w = as_bf16x8(ld16(src + 8 * c));
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[8 * c + e] = (float)w[e];
        amax = fmaxf(amax, fabsf(v[8 * c + e]));
      }
    }
    const int x = mx_exponent(amax);
    uint32_t q[8];
    quantise32(v, x, q);
    u32x4* dst = reinterpret_cast<u32x4*>(p.codes + g * 32);
    dst[0] = u32x4{q[0], q[1], q[2], q[3]};
    dst[1] = u32x4{q[4], q[5], q[6], q[7]};
    p.scales[g] = (uint8_t)(x + 127);
  }
}

// V [T, H, D] bf16 -> codes [H][D][tp] (transposed per head) + exponents
// [H][D][tp/32]: one workgroup per (padded 64-key group, 256 / D heads).  The group's
// key rows of those heads (adjacent in a token row) are loaded 16 bytes per lane into an
// LDS tile [head][64 keys][D]; then lane (head, d) reads its dimension's 64 values down
// the tile, forms the two 32-key blocks' exponents and writes its 64 code bytes (one
// contiguous run of the transposed layout) and its two exponent bytes.  Keys past the
// sequence's end are zero.  A workgroup loads its next group's rows into registers
// before quantising the current one.
template <int D>
__global__ void __launch_bounds__(256) quant_v_kernel(MxQuantParams p) {
  constexpr int HPW = 256 / D;  // heads per workgroup
  constexpr int CPR = D / 8;    // 16-byte pieces per key row of one head
  constexpr int LOADS = (HPW * kMxVPad * CPR) / 256;
  __shared__ __attribute__((aligned(16))) uint16_t tile[HPW * kMxVPad * D];
  const int H = p.num_heads, t = threadIdx.x;
  const int hgroups = (H + HPW - 1) / HPW;
  const int64_t groups = p.tp / kMxVPad, work = groups * hgroups;
  // The next group's rows are loaded into registers while this group is quantised.
  u32x4 w[LOADS];
  auto load = [&](int64_t gh) {
    const int64_t grp = gh / hgroups;
    const int h0 = (int)(gh - grp * hgroups) * HPW;
    const int b = p.group_seq[grp];
    const int64_t s0 = p.offsets[b];
    const int64_t j0 = grp * kMxVPad - p.vbase[b];
    const int valid = (int)min<int64_t>(kMxVPad, p.offsets[b + 1] - s0 - j0);
#pragma unroll
    for (int r = 0; r < LOADS; ++r) {
      const int q = t + 256 * r;
      const int j = q / (HPW * CPR), rem = q % (HPW * CPR);
      const int hh = rem / CPR, c8 = rem % CPR;
      w[r] = (j < valid && h0 + hh < H) ? ld16(p.x + ((s0 + j0 + j) * H + h0 + hh) * D + 8 * c8) : zero16();
    }
  };
  if (blockIdx.x < work) load(blockIdx.x);
  for (int64_t gh = blockIdx.x; gh < work; gh += gridDim.x) {
    const int64_t grp = gh / hgroups;
    const int h0 = (int)(gh - grp * hgroups) * HPW;
    __syncthreads();  // the previous group's readers are done with the tile
#pragma unroll
    for (int r = 0; r < LOADS; ++r) {
      const int q = t + 256 * r;
      const int j = q / (HPW * CPR), rem = q % (HPW * CPR);
      const int hh = rem / CPR, c8 = rem % CPR;
      *reinterpret_cast<u32x4*>(&tile[(hh * kMxVPad + j) * D + 8 * c8]) = w[r];
    }
    __syncthreads();
    if (gh + gridDim.x < work) load(gh + gridDim.x);
    const int hh = t / D, d = t % D;
    if (h0 + hh < H) {
      const int64_t row = (int64_t)(h0 + hh) * D + d;
      uint32_t q[16];
      int xs[2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        float v[32];
        float amax = 0.f;
#pragma unroll
        for (int u = 0; u < 32; ++u) {
          v[u] = __uint_as_float((uint32_t)tile[(hh * kMxVPad + 32 * half + u) * D + d] << 16);
          amax = fmaxf(amax, fabsf(v[u]));
        }
        xs[half] = mx_exponent(amax);
        uint32_t qq[8];
        quantise32(v, xs[half], qq);
#pragma unroll
        for (int k = 0; k < 8; ++k) q[8 * half + k] = qq[k];
      }
      u32x4* dst = reinterpret_cast<u32x4*>(p.codes + row * p.tp + grp * kMxVPad);
#pragma unroll
      for (int k = 0; k < 4; ++k) dst[k] = u32x4{q[4 * k], q[4 * k + 1], q[4 * k + 2], q[4 * k + 3]};
      *reinterpret_cast<uint16_t*>(p.scales + row * (p.tp / 32) + 2 * grp) =
          (uint16_t)((xs[0] + 127) | ((xs[1] + 127) << 8));
    }
  }
}

// ---------------------------------------------------------------- decoding

// The four E4M3 bytes of a word (OCP E4M3FN, the encoding the quantisers write) times
// 2^x.  Exact, and exact again in bf16, for x >= -117: the at most four significant bits
// stay in the normal range.
__device__ __forceinline__ void mx_decode4(uint32_t word, int x, float* v) {
  v[0] = ldexpf(__builtin_amdgcn_cvt_f32_fp8((int)word, 0), x);
  v[1] = ldexpf(__builtin_amdgcn_cvt_f32_fp8((int)word, 1), x);
  v[2] = ldexpf(__builtin_amdgcn_cvt_f32_fp8((int)word, 2), x);
  v[3] = ldexpf(__builtin_amdgcn_cvt_f32_fp8((int)word, 3), x);
}

// Q or K codes [T, H, D] + exponents [T, H, D/32] -> bf16 [T, H, D]: one thread per 16
// codes (half of one 32-element block).
__global__ void __launch_bounds__(256) dequant_qk_kernel(MxDequantParams p) {
  const int64_t n16 = p.rows * (p.head_dim / 16);
  for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < n16; g += (int64_t)gridDim.x * 256) {
    const u32x4 c = ld16(p.codes + 16 * g);
    const int x = (int)p.scales[g >> 1] - 127;
    float v[16];
#pragma unroll
    for (int w = 0; w < 4; ++w) mx_decode4(c[w], x, v + 4 * w);
    uint16_t* dst = p.out + 16 * g;
    st16(dst, __builtin_bit_cast(u32x4, pack8(v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7])));
    st16(dst + 8, __builtin_bit_cast(u32x4, pack8(v[8], v[9], v[10], v[11], v[12], v[13], v[14], v[15])));
  }
}

// V codes [H][D][Tp] (transposed per head, sequences padded to 64 keys) + exponents
// [H][D][Tp/32] -> bf16 [T, H, D].  One workgroup per (padded 64-key group, head): four
// lanes read one dimension's 64 codes (64 contiguous bytes), decode them and write them
// into an LDS tile [64 keys][D]; then every lane copies 16-byte row pieces of the tile's
// valid keys to their token rows.
template <int D>
__global__ void __launch_bounds__(256) dequant_v_kernel(MxDequantParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kMxVPad * D];
  const int H = p.num_heads, t = threadIdx.x;
  const int64_t groups = p.tp / kMxVPad;
  for (int64_t gh = blockIdx.x; gh < groups * H; gh += gridDim.x) {
    const int64_t grp = gh / H;
    const int h = (int)(gh - grp * H);
    const int b = p.group_seq[grp];
    const int64_t s0 = p.offsets[b];
    const int64_t j0 = grp * kMxVPad - p.vbase[b];  // first key of the group in its sequence
    const int valid = (int)min<int64_t>(kMxVPad, p.offsets[b + 1] - s0 - j0);
    __syncthreads();  // the previous group's readers are done with the tile
#pragma unroll
    for (int r = 0; r < (4 * D) / 256; ++r) {
      const int ch = t + 256 * r;
      const int d = ch >> 2, c = ch & 3;  // 16 keys 16 c .. of dimension d
      const int64_t row = (int64_t)h * D + d;
      const u32x4 w = ld16(p.codes + row * p.tp + grp * kMxVPad + 16 * c);
      const int x = (int)p.scales[row * (p.tp / 32) + 2 * grp + (c >> 1)] - 127;
      float v[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) mx_decode4(w[q], x, v + 4 * q);
#pragma unroll
      for (int i = 0; i < 16; ++i) tile[(16 * c + i) * D + d] = __builtin_bit_cast(uint16_t, (bf16)v[i]);
    }
    __syncthreads();
    constexpr int CPR = D / 8;  // 16-byte pieces per key row
    for (int q = t; q < valid * CPR; q += 256) {
      const int j = q / CPR, c8 = q % CPR;
      st16(p.out + ((s0 + j0 + j) * H + h) * D + 8 * c8, *reinterpret_cast<const u32x4*>(&tile[j * D + 8 * c8]));
    }
  }
}

// ---------------------------------------------------------------- forward

template <int D>
struct MxCfg {
  static constexpr int NW = mx_waves(D);
  static constexpr int BM = NW * 32;   // query rows per tile
  static constexpr int BN = 64;        // keys per step
  static constexpr int KS = D / 64;    // k-steps of S
  static constexpr int NDB = D / 32;   // 32-row blocks of O^T
  static constexpr int KT = BN * D;    // K tile bytes: [64 keys][D]
  static constexpr int VT = D * BN;    // V^T tile bytes: [D][64 keys]
  static constexpr int KSC = BN * (D / 32);  // K scales: [64 keys][D/32]
  static constexpr int VSC = D * 2;          // V scales: [D][2]
  static constexpr int SMEM = KT + VT + KSC + VSC;
  static constexpr int KCH = KT / 16 / (NW * 64);  // 16-byte K chunks per thread
  static constexpr int VCH = VT / 16 / (NW * 64);
  static_assert(KCH >= 1 && VCH >= 1, "tile copy split");
};

// Byte offset of 16-byte chunk c of row r in a swizzled tile of RB-byte rows: the
// chunk index is XORed with (r / rows-per-256-byte-line) so that the rows one
// half-wave reads together land in different bank groups.
template <int RB>
__device__ __forceinline__ int mx_swz(int r, int c) {
  constexpr int RPL = 256 / RB, CPR = RB / 16;
  return r * RB + ((c ^ ((r / RPL) & (CPR - 1))) << 4);
}

template <int D>
struct MxStage {  // one step's global data, held in registers between the loads and the LDS stores
  u32x4 k[MxCfg<D>::KCH];
  u32x4 v[MxCfg<D>::VCH];
  uint32_t ksc, vsc;
};

template <int D>
__device__ __forceinline__ void mx_load(const MxParams& p, MxStage<D>& st, int64_t s0, int L, int h, int key0,
                                        int64_t vrow0, int tid) {
  using C = MxCfg<D>;
  const int H = p.num_heads;
  constexpr int CPR = D / 16;
#pragma unroll
  for (int u = 0; u < C::KCH; ++u) {
    const int ch = tid + u * C::NW * 64;
    const int r = ch / CPR, c = ch % CPR;
    const int key = min(key0 + r, L - 1);  // rows past the end repeat the last key (masked)
    st.k[u] = ld16(p.k8 + ((s0 + key) * H + h) * D + 16 * c);
  }
#pragma unroll
  for (int u = 0; u < C::VCH; ++u) {
    const int ch = tid + u * C::NW * 64;
    const int r = ch / 4, c = ch % 4;  // V^T row = dimension r, 64 keys = 4 chunks
    st.v[u] = ld16(p.v8t + ((int64_t)h * D + r) * p.tp + vrow0 + key0 + 16 * c);
  }
  if (tid < C::BN) {
    const int key = min(key0 + tid, L - 1);
    const uint8_t* ks = p.ksc + ((s0 + key) * H + h) * (D / 32);
    st.ksc = (D == 128) ? *reinterpret_cast<const uint32_t*>(ks) : (uint32_t)*reinterpret_cast<const uint16_t*>(ks);
  }
  if (tid < D) {
    st.vsc = *reinterpret_cast<const uint16_t*>(p.vsc + ((int64_t)h * D + tid) * (p.tp / 32) + (vrow0 + key0) / 32);
  }
}

template <int D>
__device__ __forceinline__ void mx_store(const MxStage<D>& st, JFA_LDS char* smem, int tid) {
  using C = MxCfg<D>;
  constexpr int CPR = D / 16;
#pragma unroll
  for (int u = 0; u < C::KCH; ++u) {
    const int ch = tid + u * C::NW * 64;
    lds_st16(smem, mx_swz<D>(ch / CPR, ch % CPR), st.k[u]);
  }
#pragma unroll
  for (int u = 0; u < C::VCH; ++u) {
    const int ch = tid + u * C::NW * 64;
    lds_st16(smem + C::KT, mx_swz<C::BN>(ch / 4, ch % 4), st.v[u]);
  }
  if (tid < C::BN) {
    if (D == 128) *reinterpret_cast<JFA_LDS uint32_t*>(smem + C::KT + C::VT + tid * 4) = st.ksc;
    else *reinterpret_cast<JFA_LDS uint16_t*>(smem + C::KT + C::VT + tid * 2) = (uint16_t)st.ksc;
  }
  if (tid < D) *reinterpret_cast<JFA_LDS uint16_t*>(smem + C::KT + C::VT + C::KSC + tid * 2) = (uint16_t)st.vsc;
}

__device__ __forceinline__ i32x8 lds_frag(const JFA_LDS char* tile, int off0, int off1) {
  const u32x4 a = lds_ld16(tile, off0), b = lds_ld16(tile, off1);
  return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

template <int D>
__device__ __forceinline__ void mx_tile(const MxParams& p, Tile tile, JFA_LDS char* smem, int tid) {
  using C = MxCfg<D>;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int b = tile.b, h = tile.hb >> 24, blk = tile.hb & 0xFFFFFF;
  const int H = p.num_heads;
  const int64_t s0 = p.offsets[b];
  const int L = (int)(p.offsets[b + 1] - s0);
  const int64_t vrow0 = p.vbase[b];
  const int row = blk * C::BM + wave * 32 + l32;  // this lane's query
  const bool row_ok = row < L;
  const float c = p.scale_log2;

  // Q^T as the B operand of S^T: lane (n, h') holds Q[n][64 s + 16 h' + 0..15] and
  // Q[n][64 s + 32 + 16 h' + 0..15]; its scale is that of block 2 s + h'.
  i32x8 qf[C::KS];
  int qsc[C::KS];
  {
    const uint8_t* qp = p.q8 + ((s0 + min(row, L - 1)) * H + h) * D;
    const uint8_t* qs = p.qsc + ((s0 + min(row, L - 1)) * H + h) * (D / 32);
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      const u32x4 a = ld16(qp + 64 * s + 16 * half), bq = ld16(qp + 64 * s + 32 + 16 * half);
      qf[s] = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)bq[0], (int)bq[1], (int)bq[2], (int)bq[3]};
      qsc[s] = qs[2 * s + half];
    }
  }

  f32x16 o[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  float m = -INFINITY, l = 0.f;

  // A rows of key block kb for this lane: key 32 kb + 16 ((m>>2)&1) + 4 (m>>3) + (m&3).
  const int pkey = 16 * ((l32 >> 2) & 1) + 4 * (l32 >> 3) + (l32 & 3);
  const int nsteps = (L + C::BN - 1) / C::BN;
  MxStage<D> st;
  mx_load<D>(p, st, s0, L, h, 0, vrow0, tid);
  for (int it = 0; it < nsteps; ++it) {
    __syncthreads();  // the previous step's readers are done with the tiles
    mx_store<D>(st, smem, tid);
    __syncthreads();
    if (it + 1 < nsteps) mx_load<D>(p, st, s0, L, h, (it + 1) * C::BN, vrow0, tid);
    const JFA_LDS char* kt = smem;
    const JFA_LDS char* vt = smem + C::KT;
    const JFA_LDS uint8_t* ksc = (const JFA_LDS uint8_t*)(smem + C::KT + C::VT);
    const JFA_LDS uint8_t* vsc = (const JFA_LDS uint8_t*)(smem + C::KT + C::VT + C::KSC);

    // S^T blocks: register i of block kb <-> key 32 kb + 16 half + i, lane n = query.
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
      const int kr = 32 * kb + pkey;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const i32x8 a = lds_frag(kt, mx_swz<D>(kr, 4 * ks + half), mx_swz<D>(kr, 4 * ks + 2 + half));
        const int as = ksc[kr * (D / 32) + 2 * ks + half];
        s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf[ks], s[kb], 0, 0, 0, as, 0, qsc[ks]);
      }
    }
    // Online softmax in base 2 with a lazily updated reference m (moved only when the
    // row maximum exceeds it by more than 2^8, so P <= 2^8 relative to m; exact).  The
    // block maxima of raw S (both halves, one lane swap) give the row maximum and each
    // 32-key block's P exponent X_b (smallest power of two keeping the block maximum at
    // most 448), so P is produced already divided by 2^X_b: exp2(S c - m - X_b).
    const int kv = L - it * C::BN;  // keys past the end of the sequence are masked
    float bm[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      bm[kb] = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (32 * kb + 16 * half + i >= kv) s[kb][i] = -INFINITY;
        bm[kb] = fmaxf(bm[kb], s[kb][i]);
      }
      bm[kb] = half_max(bm[kb]);
    }
    const float rmax = fmaxf(bm[0], bm[1]) * c;
    const bool grow = rmax > m + 8.f;
    if (__ballot(grow) != 0) {
      const float alpha = grow ? fast_exp2(m - rmax) : 1.f;
      m = grow ? rmax : m;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
    }
    int px[2];
    float sum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // log2(448) = 8.807...: X_b = ceil(log2(block max) - log2(448))
      px[kb] = bm[kb] == -INFINITY ? 0 : max((int)ceilf(fmaf(bm[kb], c, -m) - 8.807354922057604f), -127);
      const float off = m + (float)px[kb];
      float bs = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = fminf(fast_exp2(fmaf(s[kb][i], c, -off)), 448.f);
        s[kb][i] = pv;
        bs += pv;
      }
      sum += ldexpf(bs, px[kb]);
    }
    l += half_sum(sum);
    uint32_t pw[8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t d = 0;
        d = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(s[kb][4 * w], s[kb][4 * w + 1], (int)d, false);
        d = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(s[kb][4 * w + 2], s[kb][4 * w + 3], (int)d, true);
        pw[4 * kb + w] = d;
      }
    const i32x8 pf = i32x8{(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3], (int)pw[4], (int)pw[5], (int)pw[6], (int)pw[7]};
    const int ps = px[half] + 127;  // this lane's scale is that of key block `half`
    // O^T += V^T P^T: A lane (d, h') = V^T row d, keys 16 h' + 0..15 and 32 + 16 h' + 0..15
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      const int d = 32 * db + l32;
      const i32x8 a = lds_frag(vt, mx_swz<C::BN>(d, half), mx_swz<C::BN>(d, 2 + half));
      o[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pf, o[db], 0, 0, 0, vsc[2 * d + half], 0, ps);
    }
  }

  if (row_ok) {
    const float inv = 1.0f / l;
    uint16_t* op = p.o + ((s0 + row) * H + h) * D + 4 * half;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        st8(op + 32 * db + 8 * g4, pack4(o[db][4 * g4] * inv, o[db][4 * g4 + 1] * inv, o[db][4 * g4 + 2] * inv,
                                        o[db][4 * g4 + 3] * inv));
    if (half == 0) p.lse[(int64_t)h * p.total_tokens + s0 + row] = (m + fast_log2(l)) * kLn2;
  }
}

template <int D>
__global__ void __launch_bounds__(mx_waves(D) * 64)
    __attribute__((amdgpu_waves_per_eu(2, 2))) mx_fwd_kernel(MxParams p) {
  __shared__ __attribute__((aligned(16))) char smem[MxCfg<D>::SMEM];
  const int prog = xcd_program_id(blockIdx.x, gridDim.x);
  for (int idx = p.seg_ptr[prog]; idx < p.seg_ptr[prog + 1]; ++idx) {
    if (threadIdx.x == 0) count_visit(p.visits, idx);
    mx_tile<D>(p, p.tiles[idx], (JFA_LDS char*)smem, threadIdx.x);
  }
}

// ------------------------------------------------- forward, head_dim 128 (ping-pong)
//
// The same arithmetic per 64-key step as mx_tile, arranged like the bf16 forward: two
// groups of four 32-row waves (waves w and w + 4 share a SIMD) run the same phases one
// phase apart -- a matrix phase (O^T += V^T P^T of the previous step and S^T = K Q^T of
// this one, MFMAs alternating) and a vector phase (masking, block maxima, lazy rescale,
// P and its exponents, row sums) -- separated by workgroup barriers, so that on every
// SIMD one wave feeds the matrix core while the other runs the vector work.  Stage i =
// {K(i) and its scales, V^T(i-1) and its scales} reaches a 3-slot LDS ring by direct
// global -> LDS copies issued two stages ahead: every wave copies one 1 KB piece of the
// K tile and one of the V^T tile (each lane fetching the 16-byte chunk that the XOR
// swizzle puts at its LDS position), plus one scale copy (wave 0 and waves 3-7 the K
// scales, 4 bytes per key -- the same bytes to the same place --, waves 1 and 2 half of
// the V scales each, 2 bytes per dimension, one dword per lane in LDS), so that every
// wave issues the same three copies per stage and the waits count them exactly.  The
// next tile's Q rows and first two stages load during the current tile's last phases.
// Unlike the bf16 forward, the matrix phases keep the normal wave priority: here the
// vector phase is the longer one (equal priorities measured 1 % faster).
struct Mx2Cfg {
  static constexpr int D = 128, NW = 8, BM = 256, BN = 64, NS = 3;
  static constexpr int KS = D / 64, NDB = D / 32;
  static constexpr int KT = BN * D;                 // K tile [64 keys][D]
  static constexpr int VT = D * BN;                 // V^T tile [D][64 keys]
  static constexpr int KSC = BN * 4;                // K scales [64 keys][D/32]
  static constexpr int VSC = D * 4;                 // V scales [D][2 (+2 zero bytes)]
  static constexpr int OFF_V = KT, OFF_KS = KT + VT, OFF_VS = OFF_KS + KSC;
  static constexpr int STAGE = OFF_VS + VSC;
  static constexpr int DMA_PER_STAGE = 3;
  static constexpr int RB = 2 * D;                  // bf16 O row bytes
  static constexpr int PITCH = RB + 8;
  static constexpr int STG = (BM / 2) * PITCH;      // O staging: half a tile
  static_assert(KT == NW * 1024 && VT == NW * 1024, "one 1 KB copy per wave per tile");
  static_assert(KS * 64 == D && STAGE % 16 == 0, "layout");
};
static_assert(mx_rows(128) == Mx2Cfg::BM && mx_wg_per_cu(128) == 1, "the schedule's tiles and occupancy");

// Per-lane copy offsets (bytes from the stage's uniform bases) and operand constants.
struct Mx2Lane {
  uint32_t koff;   // K tile: this lane's chunk of row krow (unclamped)
  int krow, kch;   // K row and global chunk of that copy
  uint32_t voff;   // V^T tile: this lane's chunk of dimension row 16 wave + lane / 4
  uint32_t sofs;   // scales: K (4 bytes per key: lane = key) or V (2 bytes per dimension)
  int pkey;        // A row order of the S product (see mx_tile)
  __device__ __forceinline__ void init(const MxParams& p, int wave, int lane) {
    using C = Mx2Cfg;
    const uint32_t kstride = (uint32_t)p.num_heads * C::D;  // K bytes per token
    krow = 8 * wave + lane / 8;
    kch = (lane % 8) ^ ((krow / 2) & 7);
    koff = (uint32_t)krow * kstride + 16u * (uint32_t)kch;
    const int vr = 16 * wave + lane / 4;
    voff = (uint32_t)vr * (uint32_t)p.tp + 16u * (uint32_t)((lane % 4) ^ ((vr / 4) & 3));
    sofs = (wave == 1 || wave == 2) ? (uint32_t)(64 * (wave - 1) + lane) * (uint32_t)(p.tp / 32)
                                    : (uint32_t)lane * (uint32_t)p.num_heads * 4u;
    const int l32 = lane & 31;
    pkey = 16 * ((l32 >> 2) & 1) + 4 * (l32 >> 3) + (l32 & 3);
  }
};

// One wave's state: Q (B operands and their scales), O^T accumulators, the scores of
// the current step, its quantised probabilities with their exponent, the running
// reference maximum (scaled units) and sum.
struct Mx2Wave {
  i32x8 qf[Mx2Cfg::KS];
  int qsc[Mx2Cfg::KS];
  f32x16 o[Mx2Cfg::NDB];
  f32x16 s[2];
  i32x8 pf;
  int ps;
  float m, l;
};

__device__ __forceinline__ void mx2_issue(const MxParams& p, const Mx2Lane& ln, int64_t s0, int L, int h,
                                          int64_t vrow0, int n, int i, JFA_LDS char* slot, int wave, int lane) {
  using C = Mx2Cfg;
  const int H = p.num_heads;
  const int kt = min(i, n - 1), vt = max(i - 1, 0);
  const int rows_k = min(C::BN, L - C::BN * kt);
  const uint8_t* kb = p.k8 + ((s0 + (int64_t)C::BN * kt) * H + h) * C::D;
  const uint32_t ko = rows_k >= C::BN ? ln.koff
                                      : (uint32_t)min(ln.krow, rows_k - 1) * (uint32_t)(H * C::D) + 16u * (uint32_t)ln.kch;
  dma16(uniform_ptr(kb), ko, slot + wave * 1024);
  const uint8_t* vb = p.v8t + (int64_t)h * C::D * p.tp + vrow0 + (int64_t)C::BN * vt;
  dma16(uniform_ptr(vb), ln.voff, slot + C::OFF_V + wave * 1024);
  if (wave == 1 || wave == 2) {
    const uint8_t* vs = p.vsc + (int64_t)h * C::D * (p.tp / 32) + (vrow0 + (int64_t)C::BN * vt) / 32;
    dma2(uniform_ptr(vs), ln.sofs, slot + C::OFF_VS + (wave - 1) * 256);
  } else {
    const uint8_t* ks = p.ksc + ((s0 + (int64_t)C::BN * kt) * H + h) * 4;
    const uint32_t so = rows_k >= C::BN ? ln.sofs : (uint32_t)min(lane, rows_k - 1) * (uint32_t)H * 4u;
    dma4(uniform_ptr(ks), so, slot + C::OFF_KS);
  }
}

// S^T = K Q^T of one step into w.s (register i of block kb <-> key 32 kb + 16 half + i).
__device__ __forceinline__ void mx2_s_mfma(const JFA_LDS char* slot, const Mx2Lane& ln, Mx2Wave& w, int kb, int ks,
                                           int half) {
  using C = Mx2Cfg;
  const int kr = 32 * kb + ln.pkey;
  const i32x8 a = lds_frag(slot, mx_swz<C::D>(kr, 4 * ks + half), mx_swz<C::D>(kr, 4 * ks + 2 + half));
  const int as = ((const JFA_LDS uint8_t*)(slot + C::OFF_KS))[kr * 4 + 2 * ks + half];
  w.s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, w.qf[ks], w.s[kb], 0, 0, 0, as, 0, w.qsc[ks]);
}

// O^T += V^T P^T for head-dim block db.
__device__ __forceinline__ void mx2_pv_mfma(const JFA_LDS char* slot, Mx2Wave& w, int db, int l32, int half) {
  using C = Mx2Cfg;
  const int d = 32 * db + l32;
  const JFA_LDS char* vt = slot + C::OFF_V;
  const i32x8 a = lds_frag(vt, mx_swz<C::BN>(d, half), mx_swz<C::BN>(d, 2 + half));
  const int vs = ((const JFA_LDS uint8_t*)(slot + C::OFF_VS))[d * 4 + half];
  w.o[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, w.pf, w.o[db], 0, 0, 0, vs, 0, w.ps);
}

__device__ __forceinline__ void mx2_zero_s(Mx2Wave& w) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) w.s[kb][i] = 0.f;
}

// Matrix phase with S only (the tile's first step).
__device__ __forceinline__ void mx2_mma_s(const JFA_LDS char* slot, const Mx2Lane& ln, Mx2Wave& w, int half) {
  mx2_zero_s(w);
#pragma unroll
  for (int ks = 0; ks < Mx2Cfg::KS; ++ks)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) mx2_s_mfma(slot, ln, w, kb, ks, half);
}

// Steady matrix phase: PV of the previous step (V^T in this stage) and S of this one,
// their MFMAs alternating.
__device__ __forceinline__ void mx2_mma_pv_s(const JFA_LDS char* slot, const Mx2Lane& ln, Mx2Wave& w, int l32,
                                             int half) {
  using C = Mx2Cfg;
  static_assert(C::NDB == 2 * C::KS, "four PV and four S MFMAs");
  mx2_zero_s(w);
#pragma unroll
  for (int k = 0; k < C::NDB; ++k) {
    mx2_pv_mfma(slot, w, k, l32, half);
    mx2_s_mfma(slot, ln, w, k % 2, k / 2, half);
  }
}

// Last matrix phase: PV only.
__device__ __forceinline__ void mx2_mma_pv(const JFA_LDS char* slot, Mx2Wave& w, int l32, int half) {
#pragma unroll
  for (int db = 0; db < Mx2Cfg::NDB; ++db) mx2_pv_mfma(slot, w, db, l32, half);
}

__device__ __forceinline__ void mx2_pin_vector(Mx2Wave& w) {
  asm volatile("" : "+v"(w.pf));
#pragma unroll
  for (int db = 0; db < Mx2Cfg::NDB; ++db) pin(w.o[db]);
  pin(w.m);
  pin(w.l);
}
__device__ __forceinline__ void mx2_pin_matrix(Mx2Wave& w) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) pin(w.s[kb]);
#pragma unroll
  for (int db = 0; db < Mx2Cfg::NDB; ++db) pin(w.o[db]);
}

// Vector phase of one step (the arithmetic of mx_tile): keys at or past keys_valid
// masked, block maxima, lazy rescale, P / 2^X_b in E4M3 with its exponent, row sums.
__device__ __forceinline__ void mx2_softmax(Mx2Wave& w, int keys_valid, int half, float c) {
  using C = Mx2Cfg;
  if (keys_valid < C::BN) {
    asm volatile("" ::: "memory");
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (32 * kb + 16 * half + i >= keys_valid) w.s[kb][i] = -INFINITY;
  }
  float bm[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const f32x16& x = w.s[kb];
    float a0 = fmaxf(fmaxf(x[0], x[1]), x[2]), a1 = fmaxf(fmaxf(x[3], x[4]), x[5]);
    float a2 = fmaxf(fmaxf(x[6], x[7]), x[8]), a3 = fmaxf(fmaxf(x[9], x[10]), x[11]);
    float a4 = fmaxf(fmaxf(x[12], x[13]), x[14]);
    bm[kb] = half_max(fmaxf(fmaxf(fmaxf(a0, a1), a2), fmaxf(fmaxf(a3, a4), x[15])));
  }
  const float rmax = fmaxf(bm[0], bm[1]) * c;
  const bool grow = rmax > w.m + 8.f;
  if (__ballot(grow) != 0) {
    asm volatile("" ::: "memory");
    const float alpha = grow ? fast_exp2(w.m - rmax) : 1.f;
    w.m = grow ? rmax : w.m;
    w.l *= alpha;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) w.o[db][i] *= alpha;
  }
  int px[2];
  float sum = 0.f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    // log2(448) = 8.807...: X_b = ceil(log2(block max) - log2(448))
    px[kb] = bm[kb] == -INFINITY ? 0 : max((int)ceilf(fmaf(bm[kb], c, -w.m) - 8.807354922057604f), -127);
    const float off = w.m + (float)px[kb];
    float bs[4] = {0.f, 0.f, 0.f, 0.f};
    // (no clamp to 448: the block maximum's P exceeds 448 by rounding only, ~1e-6
    // relative, and the E4M3 conversion rounds everything below 464 to at most 448)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float pv = fast_exp2(fmaf(w.s[kb][i], c, -off));
      w.s[kb][i] = pv;
      bs[i & 3] += pv;
    }
    sum += ldexpf((bs[0] + bs[1]) + (bs[2] + bs[3]), px[kb]);
  }
  w.l += half_sum(sum);
  uint32_t pw[8];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t d = 0;
      d = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(w.s[kb][4 * q], w.s[kb][4 * q + 1], (int)d, false);
      d = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(w.s[kb][4 * q + 2], w.s[kb][4 * q + 3], (int)d, true);
      pw[4 * kb + q] = d;
    }
  w.pf = i32x8{(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3], (int)pw[4], (int)pw[5], (int)pw[6], (int)pw[7]};
  w.ps = px[half] + 127;  // this lane's scale is that of key block `half`
}

// Geometry of one tile (wave-uniform).
struct Mx2Geo {
  int h, blk, L, n;
  int64_t s0, vrow0;
  __device__ __forceinline__ void init(const MxParams& p, Tile tile) {
    const int b = tile.b;
    h = tile.hb >> 24;
    blk = tile.hb & 0xFFFFFF;
    s0 = p.offsets[b];
    L = (int)(p.offsets[b + 1] - s0);
    vrow0 = p.vbase[b];
    n = (L + Mx2Cfg::BN - 1) / Mx2Cfg::BN;
  }
  // This lane's Q row (query row0 + l32 of the tile, clamped to the sequence) as the B
  // operand of S^T: lane (n, h') holds Q[n][64 s + 16 h' + 0..15] and Q[n][64 s + 32 +
  // 16 h' + 0..15]; its scale is that of block 2 s + h'.
  __device__ __forceinline__ void load_q(const MxParams& p, int row, int half, Mx2Wave& w) const {
    using C = Mx2Cfg;
    const int H = p.num_heads;
    const uint8_t* qp = p.q8 + ((s0 + min(row, L - 1)) * H + h) * C::D;
    const uint8_t* qs = p.qsc + ((s0 + min(row, L - 1)) * H + h) * (C::D / 32);
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      const u32x4 a = ld16(qp + 64 * s + 16 * half), bq = ld16(qp + 64 * s + 32 + 16 * half);
      w.qf[s] = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)bq[0], (int)bq[1], (int)bq[2], (int)bq[3]};
      w.qsc[s] = qs[2 * s + half];
    }
  }
};

// One tile.  Stage i lives in ring slot (sb + i) % NS.  pre: the previous tile loaded
// this tile's Q rows into w and copied its stages 0 and 1, then issued prev_stores
// stores.  has_next: the next tile nx (with keys) starts loading after this tile's last
// vector phase -- its Q rows into w (dead after the last S product) and its stages 0, 1
// into the two slots after this tile's last stage.  Returns the number of epilogue
// stores this wave issued.
__device__ __forceinline__ int mx2_tile(const MxParams& p, const Mx2Geo& t, bool has_next, const Mx2Geo& nx,
                                        bool pre, int sb, int prev_stores, Mx2Wave& w, JFA_LDS char* smem,
                                        JFA_LDS char* stg, const Mx2Lane& ln, int tid) {
  using C = Mx2Cfg;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = wave >> 2;
  const int l32 = lane & 31, half = lane >> 5;
  const int H = p.num_heads;
  const int64_t s0 = t.s0;
  const int L = t.L, h = t.h, blk = t.blk, n = t.n;
  const int row = blk * C::BM + wave * 32 + l32;
  const float c = p.scale_log2;

  if (!pre) t.load_q(p, row, half, w);
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) w.o[db][i] = 0.f;
  w.m = -INFINITY;
  w.l = 0.f;

  if (n > 0) {
    constexpr int LAST = (C::NS - 1) * C::STAGE;
    auto adv = [](int off) { return off == LAST ? 0 : off + C::STAGE; };
    int mat_off = sb * C::STAGE;
    int iss_off = adv(adv(mat_off));
    auto issue = [&](int i, int off) { mx2_issue(p, ln, s0, L, h, t.vrow0, n, i, smem + off, wave, lane); };
    if (!pre) {
      issue(0, mat_off);
      issue(1, adv(mat_off));
    }
    // Q and stage 0 have landed (stage 1 and the previous tile's epilogue stores, issued
    // after them, may not have)
    wait_vmem_at_most(C::DMA_PER_STAGE + (pre ? prev_stores : 0));
    phase_barrier();
    int ph = 0;
    auto end_phase = [&]() {
      if ((ph & 1) && ph < 2 * n + 1) {
        if ((ph >> 1) + 2 <= n) wait_vmem_n<C::DMA_PER_STAGE>();
        else wait_vmem();
      }
      phase_barrier();
      ++ph;
      if (!(ph & 1) && (ph >> 1) + 2 <= n) {
        issue((ph >> 1) + 2, iss_off);
        iss_off = adv(iss_off);
      }
    };
    if (2 <= n) {
      issue(2, iss_off);
      iss_off = adv(iss_off);
    }
    // a wave whose 32 rows all lie past the end runs the phases without their work
    auto phases = [&](auto compute_tag) {
      constexpr bool COMP = decltype(compute_tag)::value;
      if (g) end_phase();
      if constexpr (COMP) {
        
        mx2_mma_s(smem + mat_off, ln, w, half);
        mx2_pin_matrix(w);
        
      }
      end_phase();
      for (int i = 1; i < n; ++i) {
        if constexpr (COMP) {
          mx2_softmax(w, C::BN, half, c);
          mx2_pin_vector(w);
        }
        end_phase();
        mat_off = adv(mat_off);
        if constexpr (COMP) {
          
          mx2_mma_pv_s(smem + mat_off, ln, w, l32, half);
          mx2_pin_matrix(w);
          
        }
        end_phase();
      }
      if constexpr (COMP) {
        mx2_softmax(w, L - C::BN * (n - 1), half, c);
        mx2_pin_vector(w);
      }
      end_phase();
      if (has_next) {
        // every stage 2 .. n has been issued: iss_off is the slot of stage n + 1
        nx.load_q(p, nx.blk * C::BM + wave * 32 + l32, half, w);
        mx2_issue(p, ln, nx.s0, nx.L, nx.h, nx.vrow0, nx.n, 0, smem + iss_off, wave, lane);
        mx2_issue(p, ln, nx.s0, nx.L, nx.h, nx.vrow0, nx.n, 1, smem + adv(iss_off), wave, lane);
      }
      if constexpr (COMP) {
        
        mx2_mma_pv(smem + adv(mat_off), w, l32, half);
        mx2_pin_matrix(w);
        
      }
      end_phase();
      if (!g) end_phase();
    };
    if ((row - l32) < L) phases(std::true_type{});
    else phases(std::false_type{});
  }

  // Epilogue: O / l in bf16 through LDS, half a tile (one wave group's rows) at a time,
  // then whole rows with 16-byte stores; lse = ln 2 (m + log2 l).  Rows past the end
  // repeat the half's last row.
  const float lt = w.l;
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  if (row < L && half == 0) p.lse[(int64_t)h * p.total_tokens + s0 + row] = (w.m + fast_log2(lt)) * kLn2;
  int stores = (row - l32) < L ? 1 : 0;  // the lse store (the wave's first row exists)
  const int64_t rs = (int64_t)H * C::D;
  constexpr int HR = C::BM / 2, CPR = C::RB / 16;
  constexpr int PASSES = HR * CPR / (C::NW * 64);
  int tl = tid;
  asm volatile("" : "+v"(tl));
  const int wbase = (((tl >> 6) & 3) * 32 + (tl & 31)) * C::PITCH + 8 * ((tl >> 5) & 1);
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int valid = min(HR, L - blk * C::BM - HR * r);  // workgroup-uniform
    if (valid <= 0) break;
    if (g == r) {
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x16& x = w.o[db];
          lds_st8(stg + 64 * db + 16 * g4, wbase,
                  pack4(x[4 * g4] * inv, x[4 * g4 + 1] * inv, x[4 * g4 + 2] * inv, x[4 * g4 + 3] * inv));
        }
    }
    __syncthreads();
    uint16_t* ob = p.o + (s0 + blk * C::BM + HR * r) * rs + (int64_t)h * C::D;
#pragma unroll
    for (int k = 0; k < PASSES; ++k) {
      const int q = tl + C::NW * 64 * k;
      const int rr = min(q / CPR, valid - 1), cc = q % CPR;
      const int ro = rr * C::PITCH + 16 * cc;
      const u32x2 lo = lds_ld8(stg, ro), hi = lds_ld8(stg, ro + 8);
      st16(ob + (int64_t)rr * rs + 8 * cc, u32x4{lo[0], lo[1], hi[0], hi[1]});
    }
    stores += PASSES;
    __syncthreads();
  }
  return stores;
}

__global__ void __launch_bounds__(Mx2Cfg::NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
    mx2_fwd_kernel(MxParams p) {
  using C = Mx2Cfg;
  __shared__ __attribute__((aligned(16))) char smem_raw[C::NS * C::STAGE];
  __shared__ __attribute__((aligned(16))) char stg_raw[C::STG];
  const int tid = threadIdx.x;
  Mx2Lane ln;
  ln.init(p, tid >> 6, tid & 63);
  const int prog = xcd_program_id(blockIdx.x, gridDim.x);
  int idx = p.seg_ptr[prog];
  const int end = p.seg_ptr[prog + 1];
  if (idx >= end) return;
  Mx2Wave w;
  bool pre = false;
  int sb = 0, stores = 0;
  Mx2Geo cur;
  cur.init(p, p.tiles[idx]);
  while (true) {
    if (tid == 0) count_visit(p.visits, idx);
    const bool more = idx + 1 < end;
    Mx2Geo nt = cur;
    if (more) nt.init(p, p.tiles[idx + 1]);
    const bool ahead = more && cur.n > 0 && nt.n > 0;
    stores = mx2_tile(p, cur, ahead, nt, pre, sb, stores, w, (JFA_LDS char*)smem_raw, (JFA_LDS char*)stg_raw, ln, tid);
    if (!more) break;
    if (cur.n > 0) sb = (sb + cur.n + 1) % C::NS;
    pre = ahead;
    ++idx;
    cur = nt;
  }
}

hipError_t grid_launch(void (*k)(MxQuantParams), const MxQuantParams& p, int64_t threads, hipStream_t s) {
  if (threads <= 0) return hipSuccess;
  const int grid = (int)std::min<int64_t>((threads + 255) / 256, 16384);
  hipLaunchKernelGGL(k, dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mx_quant_qk(const MxQuantParams& p, hipStream_t s) {
  return grid_launch(quant_qk_kernel, p, p.rows * (p.head_dim / 32), s);
}

hipError_t launch_mx_quant_v(const MxQuantParams& p, hipStream_t s) {
  const int hpw = 256 / p.head_dim;
  const int64_t work = (p.tp / kMxVPad) * ((p.num_heads + hpw - 1) / hpw);
  if (work <= 0) return hipSuccess;
  const dim3 grid((unsigned)std::min<int64_t>(work, 16384));
  if (p.head_dim == 64) hipLaunchKernelGGL(quant_v_kernel<64>, grid, dim3(256), 0, s, p);
  else hipLaunchKernelGGL(quant_v_kernel<128>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_mx_dequant_qk(const MxDequantParams& p, hipStream_t s) {
  const int64_t threads = p.rows * (p.head_dim / 16);
  if (threads <= 0) return hipSuccess;
  hipLaunchKernelGGL(dequant_qk_kernel, dim3((unsigned)std::min<int64_t>((threads + 255) / 256, 16384)), dim3(256), 0,
                     s, p);
  return hipGetLastError();
}

hipError_t launch_mx_dequant_v(const MxDequantParams& p, hipStream_t s) {
  const int64_t work = (p.tp / kMxVPad) * p.num_heads;
  if (work <= 0) return hipSuccess;
  const dim3 grid((unsigned)std::min<int64_t>(work, 16384));
  if (p.head_dim == 64) hipLaunchKernelGGL(dequant_v_kernel<64>, grid, dim3(256), 0, s, p);
  else hipLaunchKernelGGL(dequant_v_kernel<128>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

// JFA_MX_GENERIC set to a value other than "0" (read at every call) sends head_dim 128
// through mx_fwd_kernel, which otherwise serves only inputs past the ping-pong kernel's
// 32-bit copy offsets, so that tests can check it at small sizes.
bool mx_generic_forced() {
  const char* e = getenv("JFA_MX_GENERIC");
  return e && *e && *e != '0';
}

hipError_t launch_mx_fwd(const MxParams& p, int head_dim, hipStream_t s) {
  if (p.num_programs <= 0) return hipSuccess;
  // the ping-pong kernel's per-lane V^T copy offsets are 32-bit: D * Tp < 2^32
  if (head_dim == 128 && (uint64_t)p.tp * 128u < (uint64_t(1) << 32) && !mx_generic_forced()) {
    hipLaunchKernelGGL(mx2_fwd_kernel, dim3(p.num_programs), dim3(Mx2Cfg::NW * 64), 0, s, p);
    return hipGetLastError();
  }
  if (head_dim == 64)
    hipLaunchKernelGGL(mx_fwd_kernel<64>, dim3(p.num_programs), dim3(mx_waves(64) * 64), 0, s, p);
  else
    hipLaunchKernelGGL(mx_fwd_kernel<128>, dim3(p.num_programs), dim3(mx_waves(128) * 64), 0, s, p);
  return hipGetLastError();
}

}  // namespace jfa
