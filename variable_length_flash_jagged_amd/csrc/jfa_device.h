// Device-side building blocks for the gfx950 (CDNA4) kernels: MFMA operand types,
// LDS transposed reads, bf16 packing, wave-level exchanges and the XCD-aware
// program numbering.  Internal header; not part of the C ABI.
//
// Lane layouts (wave64) of the two matrix instructions used here, for A (m x k),
// B (k x n), C (m x n), with lane l, half = l / 32:
//   v_mfma_f32_32x32x16_bf16: A slot j -> (m = l % 32, k = 8*half + j), j < 8
//                             B slot j -> (k = 8*half + j, n = l % 32)
//                             C reg  i -> (m = 8*(i/4) + 4*half + i%4, n = l % 32), i < 16
// ds_read_b64_tr_b16 (per 16-lane group, source lane s reads 4 consecutive bf16 at its
// own address): result lane i, element j = element (i & 3) read by source lane
// (i >> 2) + 4*j.  With source lane s pointing at row r0 + (s >> 2), column c0 + 4*(s & 3)
// of a row-major tile, result lane i holds column c0 + i of rows r0 .. r0+3: a
// transposed fetch of a 4 x 16 block.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace jfa {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define JFA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// 16-byte global load / store.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ void st8(void* p, const u32x2& v) { *reinterpret_cast<u32x2*>(p) = v; }
__device__ __forceinline__ u32x4 zero16() { return u32x4{0u, 0u, 0u, 0u}; }

// 16-byte streaming (non-temporal) store at base + off, for data that is not read
// again soon, through a global (address space 1) pointer: a generic pointer whose
// origin the compiler cannot trace (e.g. one passed through readfirstlane) would become
// a flat store, which also counts against lgkmcnt, so that every later LDS wait would
// wait for the store to complete as well.
#define JFA_GLOBAL __attribute__((address_space(1)))
__device__ __forceinline__ void st16_global_nt(char* base, uint32_t off, const u32x4& v) {
  __builtin_nontemporal_store(v, reinterpret_cast<JFA_GLOBAL u32x4*>((JFA_GLOBAL char*)base + off));
}
// 16-byte load with the non-temporal hint (data read exactly once).
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const JFA_GLOBAL u32x4*>((const JFA_GLOBAL char*)p));
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& u) { return __builtin_bit_cast(bf16x8, u); }

// LDS 16-byte read / write (byte offsets into a __shared__ array).
__device__ __forceinline__ u32x4 lds_ld16(const JFA_LDS char* base, int byte_off) {
  return *reinterpret_cast<const JFA_LDS u32x4*>(base + byte_off);
}
__device__ __forceinline__ void lds_st16(JFA_LDS char* base, int byte_off, const u32x4& v) {
  *reinterpret_cast<JFA_LDS u32x4*>(base + byte_off) = v;
}
__device__ __forceinline__ void lds_st8(JFA_LDS char* base, int byte_off, const u32x2& v) {
  *reinterpret_cast<JFA_LDS u32x2*>(base + byte_off) = v;
}
__device__ __forceinline__ u32x2 lds_ld8(const JFA_LDS char* base, int byte_off) {
  return *reinterpret_cast<const JFA_LDS u32x2*>(base + byte_off);
}

// Element i (wave-uniform) of a read-only array through the scalar cache: a load from
// the constant address space, so that it becomes a scalar load, whose completion is
// counted by lgkmcnt and does not wait for the wave's outstanding vector-memory
// operations (a vector load's vmcnt wait would).  The array must not be written while
// the kernel runs.
template <typename T>
__device__ __forceinline__ T ld_uniform(const T* a, int64_t i) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "one or two dwords");
  using W = typename std::conditional<sizeof(T) == 4, uint32_t, uint64_t>::type;
  const W w = ((const __attribute__((address_space(4))) W*)a)[i];
  return __builtin_bit_cast(T, w);
}

// A pointer the whole wave agrees on, moved to scalar registers.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(((uint64_t)hi << 32) | lo);
}

// Direct global -> LDS copy (global_load_lds_dwordx4): every lane fetches 16 bytes at
// sbase + voff (sbase in scalar registers, voff a per-lane byte offset); the wave's 64
// results land contiguously at lds_base + 16 * lane.  sbase and lds_base must be the
// same for the whole wave (lds_base goes to M0, which the asm takes as an input operand
// so that the compiler sets it and knows it is in use).  Completion is tracked by vmcnt:
// wait_vmem() then a barrier before any wave reads the data.  The instruction is
// issued from inline assembly on purpose: the compiler cannot tell which LDS bytes the
// copy writes, and when it sees the copy it waits for it (vmcnt(0)) before the next LDS
// read of the other ring slot, which would serialise every prefetch with the compute
// it is meant to overlap.  The explicit wait_vmem() + barrier at the end of each ring
// step orders the copy against every read of its slot; copies the compiler does not
// see only make its own vmcnt waits more conservative, never less.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, JFA_LDS char* lds_base) {
  const uint32_t lds_addr = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  // The leading s_nop 4 provides the wait states the hardware needs between a VALU write
  // of an SGPR (the v_readfirstlane that makes sbase uniform, or M0's source) and a
  // memory instruction reading it.  The compiler inserts such waits for instructions it
  // knows but cannot see inside this asm; without them the copy may read the SGPR's old
  // value as its base address.
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "{m0}"(lds_addr) : "memory");
}
// The same copy with the non-temporal hint, for data read exactly once (measured on a
// plain 8 GiB stream: 7.1 TB/s against 6.3 TB/s without the hint).
__device__ __forceinline__ void dma16_nt(const void* sbase, uint32_t voff, JFA_LDS char* lds_base) {
  const uint32_t lds_addr = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1 nt" : : "v"(voff), "s"(sbase), "{m0}"(lds_addr) : "memory");
}
// Narrow forms of the same copy: each lane fetches 4 bytes (dma4) or 2 bytes (dma2) at
// sbase + voff; either way the lane's value lands as one dword at lds_base + 4 * lane
// (2-byte values zero-extended; measured with an in-bounds probe).
__device__ __forceinline__ void dma4(const void* sbase, uint32_t voff, JFA_LDS char* lds_base) {
  const uint32_t lds_addr = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile("s_nop 4\n\tglobal_load_lds_dword %0, %1" : : "v"(voff), "s"(sbase), "{m0}"(lds_addr) : "memory");
}
__device__ __forceinline__ void dma2(const void* sbase, uint32_t voff, JFA_LDS char* lds_base) {
  const uint32_t lds_addr = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile("s_nop 4\n\tglobal_load_lds_ushort %0, %1" : : "v"(voff), "s"(sbase), "{m0}"(lds_addr) : "memory");
}
// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left unconstrained).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// s_waitcnt vmcnt(N) with expcnt and lgkmcnt unconstrained.
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// s_waitcnt vmcnt(N) for N < 64 (the counter's high bits sit at [15:14]).
template <int N>
__device__ __forceinline__ void wait_vmem_upto() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// s_waitcnt vmcnt(n) for a run-time n (0 .. 31; larger counts wait for 31, which is
// never wrong: fewer outstanding instructions than allowed).
__device__ __forceinline__ void wait_vmem_at_most(int n) {
  switch (n < 0 ? 0 : (n > 31 ? 31 : n)) {
#define JFA_WAIT_CASE(k) \
  case k:                \
    wait_vmem_upto<k>(); \
    break;
    JFA_WAIT_CASE(0) JFA_WAIT_CASE(1) JFA_WAIT_CASE(2) JFA_WAIT_CASE(3) JFA_WAIT_CASE(4) JFA_WAIT_CASE(5)
    JFA_WAIT_CASE(6) JFA_WAIT_CASE(7) JFA_WAIT_CASE(8) JFA_WAIT_CASE(9) JFA_WAIT_CASE(10) JFA_WAIT_CASE(11)
    JFA_WAIT_CASE(12) JFA_WAIT_CASE(13) JFA_WAIT_CASE(14) JFA_WAIT_CASE(15) JFA_WAIT_CASE(16) JFA_WAIT_CASE(17)
    JFA_WAIT_CASE(18) JFA_WAIT_CASE(19) JFA_WAIT_CASE(20) JFA_WAIT_CASE(21) JFA_WAIT_CASE(22) JFA_WAIT_CASE(23)
    JFA_WAIT_CASE(24) JFA_WAIT_CASE(25) JFA_WAIT_CASE(26) JFA_WAIT_CASE(27) JFA_WAIT_CASE(28) JFA_WAIT_CASE(29)
    JFA_WAIT_CASE(30) default: wait_vmem_upto<31>();
#undef JFA_WAIT_CASE
  }
}

// Workgroup barrier between the phases of a two-group (ping-pong) kernel.  The LDS
// reads of a phase are consumed inside it; the lgkmcnt(0) makes sure none is still in
// flight when another wave's copy reuses its ring slot.  Copies are ordered explicitly
// with wait_vmem* before the barrier that publishes them.  The scheduling fences keep
// register-only work (MFMA, VALU) of one phase from being moved into the next.
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Pins a phase's results before its closing barrier: an empty asm that reads and
// writes them, so that no pass sinks their computation into the next phase (which
// would put one wave's vector and matrix work back into the same phase).
__device__ __forceinline__ void pin(f32x16& x) { asm volatile("" : "+v"(x)); }

// Row term of one query row for the dK/dV kernels' extra MFMA k-step: -lse log2 e and
// -Di as bf16 high + low parts, and the constant -1 the block-sparse key mask multiplies.
// One definition for every kernel that writes it (no multiply-add contraction, so the
// low parts are the same rounding of the same fp32 values everywhere).
__device__ __forceinline__ bf16x8 row_term(float lse, float di) {
#pragma clang fp contract(off)
  const float x = -lse * kLog2e, y = -di;
  const bf16 xh = (bf16)x, yh = (bf16)y;
  const bf16 xl = (bf16)(x - (float)xh), yl = (bf16)(y - (float)yh);
  const bf16 z = (bf16)0.0f;
  return bf16x8{xh, xl, (bf16)(-1.0f), z, yh, yl, z, z};
}
__device__ __forceinline__ void pin(bf16x8& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }

// Transposed 4 x 16 fetch (see the header comment); `byte_off` is this lane's source
// address.
__device__ __forceinline__ v4i16 lds_tr4(const JFA_LDS char* base, int byte_off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (JFA_LDS v4i16*)(const_cast<JFA_LDS char*>(base) + byte_off));
}

__device__ __forceinline__ bf16x8 join_tr(const v4i16& lo, const v4i16& hi) {
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  v8i16 r = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, r);
}

// Pack 8 fp32 values into a bf16x8 operand (round to nearest even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x8 pack8(float a0, float a1, float a2, float a3, float a4,
                                        float a5, float a6, float a7) {
  bf16x8 r = {(bf16)a0, (bf16)a1, (bf16)a2, (bf16)a3, (bf16)a4, (bf16)a5, (bf16)a6, (bf16)a7};
  return r;
}

__device__ __forceinline__ u32x2 pack4(float a0, float a1, float a2, float a3) {
  bf16x4 r = {(bf16)a0, (bf16)a1, (bf16)a2, (bf16)a3};
  return __builtin_bit_cast(u32x2, r);
}

// Combine a per-lane value with the same lane of the other wave half (lane ^ 32) via
// v_permlane32_swap: both halves get op(x[l], x[l ^ 32]).
__device__ __forceinline__ float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Swizzled row-major tiles in LDS: a tile row of RB bytes holds RB/16 chunks of 16
// bytes; chunk c of row r is stored at chunk position c ^ f(r).  f is chosen so that
// both access patterns of the kernels hit distinct banks (64 banks of 4 bytes):
//  * a row-wise operand fetch (ds_read_b128): 16 lanes read one chunk of 16
//    consecutive rows;
//  * a transposed fetch (ds_read_b64_tr_b16): 32 lanes read 4 consecutive chunks of 4
//    consecutive rows (row base a multiple of 4, chunk base a multiple of 4).
// For 256-byte rows (16 chunks) f(r) swaps the two low 2-bit fields of r; for 128-byte
// rows (8 chunks, two rows per 256-byte bank line) f acts on x = (r/2) mod 8 as
// (x mod 2) * 4 + x / 2.  (The plain f(r) = r mod 16 is conflict free for the first
// pattern but costs about six extra cycles per transposed fetch.)
template <int RB>
__device__ __forceinline__ int swz_f(int r) {
  static_assert(RB == 256 || RB == 128, "tile row must be 128 or 256 bytes");
  if (RB == 256) return ((r & 3) << 2) | ((r >> 2) & 3);
  const int x = (r >> 1) & 7;
  return ((x & 1) << 2) | (x >> 1);
}

template <int RB>
__device__ __forceinline__ int swz_off(int r, int c) {
  return r * RB + ((c ^ swz_f<RB>(r)) << 4);
}

// Copies of a ROWS x RB-byte tile (a row starts every row_stride_bytes in global memory)
// into a swizzled LDS tile with the 1 KB wave-wide direct copies, split over NW waves.
// init() precomputes this lane's byte offsets once per kernel, so a full-tile copy
// costs no vector ALU work; rows at or past rows_valid (tail tiles) repeat row
// rows_valid-1, so every read stays inside the caller's valid rows -- the caller masks
// their contribution.
template <int RB, int ROWS, int NW>
struct TileCopy {
  static constexpr int CPR = RB / 16;            // chunks per row
  static constexpr int RPC = 1024 / RB;          // rows per copy
  static constexpr int COPIES = ROWS * RB / 1024;
  static constexpr int J = COPIES / NW;          // copies per wave
  static_assert(COPIES % NW == 0, "copies must split evenly over the waves");
  uint32_t off[J];
  __device__ __forceinline__ static int row_of(int wave, int j, int lane) { return (wave * J + j) * RPC + lane / CPR; }
  __device__ __forceinline__ static int chunk_of(int r, int lane) { return (lane % CPR) ^ swz_f<RB>(r); }
  __device__ __forceinline__ void init(uint32_t row_stride_bytes, int wave, int lane) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int r = row_of(wave, j, lane);
      off[j] = (uint32_t)r * row_stride_bytes + (uint32_t)chunk_of(r, lane) * 16u;
    }
  }
  __device__ __forceinline__ void issue(const void* gbase, JFA_LDS char* lds, int wave) const {
    const void* b = uniform_ptr(gbase);
#pragma unroll
    for (int j = 0; j < J; ++j) dma16(b, off[j], lds + (wave * J + j) * 1024);
  }
  __device__ __forceinline__ static void issue_clamped(const void* gbase, uint32_t row_stride_bytes, int rows_valid,
                                                       JFA_LDS char* lds, int wave, int lane) {
    const void* b = uniform_ptr(gbase);
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int r = row_of(wave, j, lane);
      const uint32_t o = (uint32_t)min(r, rows_valid - 1) * row_stride_bytes + (uint32_t)chunk_of(r, lane) * 16u;
      dma16(b, o, lds + (wave * J + j) * 1024);
    }
  }
  __device__ __forceinline__ void issue_rows(const void* gbase, uint32_t row_stride_bytes, int rows_valid,
                                             JFA_LDS char* lds, int wave, int lane) const {
    if (rows_valid >= ROWS) issue(gbase, lds, wave);
    else issue_clamped(gbase, row_stride_bytes, rows_valid, lds, wave, lane);
  }
};

// Byte pointer arithmetic on bf16 data.
__device__ __forceinline__ const void* bf16_at(const uint16_t* base, int64_t elems) { return base + elems; }

// Row-wise MFMA operand fetch (A or B: lane = row l%32 of a 32-row block, slots =
// head-dim chunk 2*ks + half) from a swizzled tile; offsets precomputed per lane.  The
// swizzle of row rbase + l%32 equals that of l%32 because rbase is a multiple of 32.
template <int RB, int NKS>
struct RowOperands {
  int off[NKS];
  __device__ __forceinline__ void init(int lane) {
    const int l32 = lane & 31, half = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) off[ks] = l32 * RB + (((2 * ks + half) ^ swz_f<RB>(l32)) << 4);
  }
  __device__ __forceinline__ bf16x8 read(const JFA_LDS char* tile, int rbase, int ks) const {
    return as_bf16x8(lds_ld16(tile, rbase * RB + off[ks]));
  }
};

// Transposed MFMA operand (ds_read_b64_tr_b16) from a swizzled row-major bf16 tile:
// lane l of 16-lane group g gets column 32*cb + 16*(g & 1) + (l & 15) of rows
// row0 + 4*(g >> 1) + {0..3} (slots 0-3) and the same rows + 8 (slots 4-7) -- the
// operand whose k index runs over tile rows in the order a 32x32 C layout hands them
// over (register 8u+j <-> row 16u + 8*(j/4) + 4*half + j%4).  row0 is a multiple of
// 16, so the swizzle of each source row depends on the lane only.
template <int RB, int NCB>
struct TrOperands {
  int off[NCB][2];
  __device__ __forceinline__ void init(int lane) {
    const int g = lane >> 4, s16 = lane & 15;
    const int rr = 4 * (g >> 1) + (s16 >> 2);
    const int cc = 16 * (g & 1) + 4 * (s16 & 3);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const int r = rr + 8 * hi, col = 32 * cb + cc;
        off[cb][hi] = r * RB + (((col >> 3) ^ swz_f<RB>(r)) << 4) + (col & 7) * 2;
      }
  }
  __device__ __forceinline__ bf16x8 read(const JFA_LDS char* tile, int row0, int cb) const {
    return join_tr(lds_tr4(tile, row0 * RB + off[cb][0]), lds_tr4(tile, row0 * RB + off[cb][1]));
  }
};

// Generic forms (offsets computed per call) for the less hot kernels.
template <int RB, int ROWS, int NW>
__device__ __forceinline__ void dma_tile(const uint16_t* g, int64_t row_stride, int rows_valid,
                                         JFA_LDS char* lds, int wave, int lane) {
  TileCopy<RB, ROWS, NW>::issue_clamped(g, (uint32_t)(row_stride * 2), rows_valid, lds, wave, lane);
}

template <int RB>
__device__ __forceinline__ bf16x8 tr_operand(const JFA_LDS char* tile, int row0, int col0, int lane) {
  const int g = lane >> 4, s16 = lane & 15;
  const int r = row0 + 4 * (g >> 1) + (s16 >> 2);
  const int col = col0 + 16 * (g & 1) + 4 * (s16 & 3);
  const int w8 = (col & 7) * 2;
  return join_tr(lds_tr4(tile, swz_off<RB>(r, col >> 3) + w8), lds_tr4(tile, swz_off<RB>(r + 8, col >> 3) + w8));
}

// Debug tile-visit count (visits null: off): one atomic add per taken tile, issued by a
// single lane.
__device__ __forceinline__ void count_visit(int32_t* visits, int64_t idx) {
  if (visits) atomicAdd(visits + idx, 1);
}

// Workgroups are dealt to the 8 XCDs round robin by workgroup id; number the programs
// so that consecutive program ids share an XCD (and its L2).
__device__ __forceinline__ int xcd_program_id(int wg, int num_wg) {
  const int x = wg & 7, j = wg >> 3;
  const int q8 = num_wg >> 3, r8 = num_wg & 7;
  return x * q8 + min(x, r8) + j;
}

}  // namespace jfa
