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
#include <algorithm>

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

hipError_t launch_mx_fwd(const MxParams& p, int head_dim, hipStream_t s) {
  if (p.num_programs <= 0) return hipSuccess;
  if (head_dim == 64)
    hipLaunchKernelGGL(mx_fwd_kernel<64>, dim3(p.num_programs), dim3(mx_waves(64) * 64), 0, s, p);
  else
    hipLaunchKernelGGL(mx_fwd_kernel<128>, dim3(p.num_programs), dim3(mx_waves(128) * 64), 0, s, p);
  return hipGetLastError();
}

}  // namespace jfa
