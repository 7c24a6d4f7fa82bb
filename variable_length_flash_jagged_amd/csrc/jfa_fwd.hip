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
//  * One workgroup = 8 waves = one tile of kFwdRows (256) query rows of one
//    (sequence, head), 32 rows per wave, one workgroup per CU (2 waves per SIMD).
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Q rows held in
//    registers for the whole tile).  In the C layout every lane owns one query column,
//    so the row max / row sum are in-lane plus one permlane32 swap.
//  * O^T += V^T P^T: the probabilities leave the first product already in the B operand
//    layout (after a bf16 pack); V^T is fetched from the row-major V tile in LDS with
//    ds_read_b64_tr_b16, in the key order the C layout hands over.
//  * Ping-pong between the two waves of each SIMD.  Waves w and w+4 of a workgroup are
//    placed on the same SIMD; waves 0-3 (group A, rows 0-127) and 4-7 (group B, rows
//    128-255) run the same sequence of phases one phase apart: a matrix phase
//    (O += V(i-1) P(i-1) and S(i) = K(i) Q^T, their MFMAs alternating) and a vector
//    phase (row max, lazy rescale, P(i) = 2^(S(i) c - m c), row sums).  Workgroup
//    barriers between phases
//    keep the offset, so on every SIMD one wave feeds the matrix core while the other
//    keeps the vector unit busy (the producer / consumer overlap of matrix and softmax
//    work the TLX page describes for its forward pipeline, section 3.2, Fig. 1, mapped
//    onto SIMD pairs).
//  * Stage i = {K(i), V(i-1)} is needed by group A in phase 2i and by group B in phase
//    2i+1.  Stages reach LDS by direct global->LDS copies into a 3-slot ring, issued
//    four phases ahead ("K/V multi-buffering", aixai.ru page, "Skeleton").  Only the
//    last key tile of a sequence is range-limited; its scores past the end are masked
//    in a branch taken on that tile alone.
//  * The output is rescaled lazily: only when some row maximum grows by more than a
//    factor 2^8 (still exact: the final division uses the same stale maximum).
//  * Persistent grid: each workgroup walks its host-scheduled tile list, or takes
//    tiles from an atomic counter in dynamic mode (aixai.ru page, "Tile balancing and
//    Cluster Launch Control").
#include <type_traits>

#include "jfa_device.h"
#include "jfa_internal.h"
#include "jfa_sched.h"

namespace jfa {
namespace {

// Marks a rarely taken branch body as having side effects so that the compiler keeps
// the branch instead of executing the body unconditionally under a select.
#define JFA_KEEP_BRANCH() asm volatile("" ::: "memory")

template <int D>
struct FwdCfg {
  static constexpr int NW = kFwdWaves;
  static constexpr int BM = kFwdRows;
  static constexpr int BN = kFwdKeys;
  static constexpr int NS = kFwdStages;   // ring slots
  static constexpr int NKB = BN / 32;     // 32-key blocks per tile
  static constexpr int NKS = D / 16;      // MFMA k-steps over the head dim
  static constexpr int NDB = D / 32;      // 32-wide head-dim blocks of O
  static constexpr int NT16 = BN / 16;    // 16-key k-steps of the PV product
  static constexpr int RB = D * 2;        // bytes per tile row
  static constexpr int TILE = BN * RB;    // one K or V tile
  static constexpr int STAGE = 2 * TILE;  // ring slot: [K(i) | V(i-1)]
  using Copy = TileCopy<RB, BN, NW>;
  static constexpr int DMA_PER_STAGE = 2 * Copy::J;  // copies one wave issues per stage
  static_assert(NW == 8 && kFwdQPerWave == 32 && BM == 256, "two groups of four 32-row waves");
  static_assert(NT16 == 2 * NKB, "key steps");
  static_assert(DMA_PER_STAGE < 16, "vmcnt immediate");
};

// Per-lane constants: LDS operand offsets and ring-copy offsets.
template <int D>
struct FwdLane {
  RowOperands<FwdCfg<D>::RB, FwdCfg<D>::NKS> krow;  // K rows as the A operand of S^T
  TrOperands<FwdCfg<D>::RB, FwdCfg<D>::NDB> vtr;     // V^T as the A operand of O^T
  typename FwdCfg<D>::Copy copy;
};

// State of one wave's 32 query rows.
template <int D>
struct FwdWave {
  using C = FwdCfg<D>;
  bf16x8 (&qf)[C::NKS];  // Q rows (B operands), owned by the tile loop
  __device__ __forceinline__ explicit FwdWave(bf16x8 (&q)[C::NKS]) : qf(q) {}
  f32x16 o[C::NDB];      // O^T accumulators
  f32x16 s[C::NKB];      // scores of the current key tile, then its probabilities
  bf16x8 pf[C::NT16];    // probabilities as B operands of the PV product
  float m, l;            // running max (raw score units) and sum
};

template <int D>
__device__ __forceinline__ void pin_vector_phase(FwdWave<D>& w) {
#pragma unroll
  for (int t = 0; t < FwdCfg<D>::NT16; ++t) pin(w.pf[t]);
#pragma unroll
  for (int db = 0; db < FwdCfg<D>::NDB; ++db) pin(w.o[db]);
  pin(w.m);
  pin(w.l);
}

template <int D>
__device__ __forceinline__ void pin_matrix_phase(FwdWave<D>& w) {
#pragma unroll
  for (int kb = 0; kb < FwdCfg<D>::NKB; ++kb) pin(w.s[kb]);
#pragma unroll
  for (int db = 0; db < FwdCfg<D>::NDB; ++db) pin(w.o[db]);
}

// O^T += V^T P^T over one key tile (V tile row-major in LDS, fetched transposed).
template <int D>
__device__ __forceinline__ void mma_pv(const JFA_LDS char* vbuf, const FwdLane<D>& ln, FwdWave<D>& w) {
  using C = FwdCfg<D>;
#pragma unroll
  for (int t = 0; t < C::NT16; ++t)
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) w.o[db] = mfma32(ln.vtr.read(vbuf, 16 * t, db), w.pf[t], w.o[db]);
}

// S^T = K Q^T for one key tile ([keys x queries], C layout: lane = query column,
// register i of key block kb <-> key 32*kb + 8*(i/4) + 4*half + i%4).
template <int D>
__device__ __forceinline__ void mma_s(const JFA_LDS char* kbuf, const FwdLane<D>& ln, FwdWave<D>& w) {
  using C = FwdCfg<D>;
#pragma unroll
  for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) w.s[kb][i] = 0.f;
#pragma unroll
  for (int ks = 0; ks < C::NKS; ++ks)
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb) w.s[kb] = mfma32(ln.krow.read(kbuf, kb * 32, ks), w.qf[ks], w.s[kb]);
}

// Steady-state matrix phase: O^T += V^T P^T (previous tile) and S^T = K Q^T (this tile)
// with their MFMAs alternating, so that the LDS reads behind them (two transposed reads
// per PV operand, one row read per K operand) arrive at an even 1.5 per MFMA instead of
// two per MFMA through the first half of the phase.
template <int D>
__device__ __forceinline__ void mma_pv_s(const JFA_LDS char* kbuf, const JFA_LDS char* vbuf, const FwdLane<D>& ln,
                                         FwdWave<D>& w) {
  using C = FwdCfg<D>;
  constexpr int NPV = C::NT16 * C::NDB, NSK = C::NKS * C::NKB;
  static_assert(NPV == NSK, "PV and S products alternate one for one");
#pragma unroll
  for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) w.s[kb][i] = 0.f;
#pragma unroll
  for (int k = 0; k < NPV; ++k) {
    const int t = k / C::NDB, db = k % C::NDB;
    w.o[db] = mfma32(ln.vtr.read(vbuf, 16 * t, db), w.pf[t], w.o[db]);
    const int ks = k / C::NKB, kb = k % C::NKB;
    w.s[kb] = mfma32(ln.krow.read(kbuf, kb * 32, ks), w.qf[ks], w.s[kb]);
  }
}

// Issue order of mma_pv_s: operands of the first kAhead MFMAs, then each MFMA followed
// by the reads of the operand kAhead MFMAs later (even positions PV: two reads; odd: S).
template <int D>
__device__ __forceinline__ void order_mixed_phase() {
  using C = FwdCfg<D>;
  constexpr int kAhead = 4;
  constexpr int N = 2 * C::NT16 * C::NDB;
  __builtin_amdgcn_sched_group_barrier(0x100, 3 * kAhead / 2, 0);
#pragma unroll
  for (int k = 0; k < N; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (k + kAhead < N) {
      if ((k + kAhead) % 2 == 0) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      else __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  }
}

// Vector phase for one key tile: mask (tail tile only), row max, lazy rescale,
// probabilities, row sums, bf16 pack.
template <int D>
__device__ __forceinline__ void softmax_phase(FwdWave<D>& w, int keys_valid, int half, float c) {
  using C = FwdCfg<D>;
  if (keys_valid < C::BN) {
    JFA_KEEP_BRANCH();
    // key 32*kb + 8*(i/4) + 4*half + i%4 is past the end iff its lane-independent
    // part reaches keys_valid - 4*half (compared against immediates)
    const int kv = keys_valid - 4 * half;
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (kb * 32 + 8 * (i >> 2) + (i & 3) >= kv) w.s[kb][i] = -INFINITY;
  }
  // row max as a tree (short dependency chains: one wave issues this phase alone)
  float mk[C::NKB];
#pragma unroll
  for (int kb = 0; kb < C::NKB; ++kb) {
    const f32x16& x = w.s[kb];
    float a0 = fmaxf(fmaxf(x[0], x[1]), x[2]), a1 = fmaxf(fmaxf(x[3], x[4]), x[5]);
    float a2 = fmaxf(fmaxf(x[6], x[7]), x[8]), a3 = fmaxf(fmaxf(x[9], x[10]), x[11]);
    float a4 = fmaxf(fmaxf(x[12], x[13]), x[14]);
    mk[kb] = fmaxf(fmaxf(fmaxf(a0, a1), a2), fmaxf(fmaxf(a3, a4), x[15]));
  }
  float mx = mk[0];
#pragma unroll
  for (int kb = 1; kb < C::NKB; ++kb) mx = fmaxf(mx, mk[kb]);
  const float mnew = fmaxf(w.m, half_max(mx));  // raw scores: scale > 0 commutes with max
  if (__ballot((mnew - w.m) * c > 8.0f)) {
    JFA_KEEP_BRANCH();
    const float alpha = fast_exp2((w.m - mnew) * c);
    w.m = mnew;
    w.l *= alpha;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) w.o[db][i] *= alpha;
  }
  const float mc = w.m * c;
  float sum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float pv = fast_exp2(fmaf(w.s[kb][i], c, -mc));
      w.s[kb][i] = pv;
      sum[i & 3] += pv;
    }
  w.l += (sum[0] + sum[1]) + (sum[2] + sum[3]);
#pragma unroll
  for (int t = 0; t < C::NT16; ++t) {
    const f32x16& x = w.s[t >> 1];
    const int r = 8 * (t & 1);
    w.pf[t] = pack8(x[r], x[r + 1], x[r + 2], x[r + 3], x[r + 4], x[r + 5], x[r + 6], x[r + 7]);
  }
}

// Geometry of one forward tile (wave-uniform except `row`).
template <int D, int MODE>
struct FwdGeo {
  using C = FwdCfg<D>;
  static constexpr bool SELF = MODE != kBroadcastQ;  // queries are the sequence's own rows
  static constexpr bool CHUNKED = MODE == kBroadcastQ || MODE == kSelfChunks;  // tiles of key chunks
  int b, h, blk, kst, slot, L, Lq, row, n;
  int64_t s0;
  const int32_t* list;
  const uint16_t *kp, *vp;
  __device__ __forceinline__ void init(const FwdParams& p, Tile tile, int wave, int l32) {
    h = tile.hb >> 24;
    blk = tile.hb & 0xFFFFFF;
    const int hkv = h / (p.num_heads / p.num_kv_heads);  // key/value head of query head h
    // Key chunks (broadcast-Q, and self attention of few long sequences): the tile covers
    // keys kst .. kst + L - 1 of sequence b; slot >= 0 marks a chunk of a cut sequence,
    // whose partial O and lse go to the partial buffers.
    b = tile.b;
    kst = 0;
    slot = -1;
    if constexpr (CHUNKED) {
      const int ch = tile.b, nc = p.num_chunks;
      b = p.chunks[ch];
      kst = p.chunks[nc + ch];
      slot = p.chunks[3 * nc + ch];
    }
    s0 = p.offsets[b];
    const int Lseq = (int)(p.offsets[b + 1] - s0);
    L = CHUNKED ? p.chunks[2 * p.num_chunks + tile.b] : Lseq;  // keys visited
    Lq = SELF ? Lseq : p.num_q;
    row = blk * C::BM + wave * 32 + l32;
    // Key tiles visited: all ceil(L/BN) of the sequence, or (block sparse) the tile's
    // ascending list of kept key tiles.  Only a sequence's last key tile can be partial,
    // and in an ascending list it comes last, so the masking rule is unchanged.
    n = (L + C::BN - 1) / C::BN;  // key tiles; stages 0..n, phases 0..2n+1
    list = nullptr;
    if constexpr (MODE == kSelfSparse) {
      n = L > 0 ? p.sel_k[b] : 0;
      list = p.sel + p.sel_base[b] + ((int64_t)h * ((L + C::BM - 1) / C::BM) + blk) * n;
    }
    const int64_t rkv = (int64_t)p.num_kv_heads * D;
    kp = p.k + (s0 + kst) * rkv + (int64_t)hkv * D;
    vp = p.v + (s0 + kst) * rkv + (int64_t)hkv * D;
  }
  __device__ __forceinline__ int tile_of(int i) const { return MODE == kSelfSparse ? list[i] : i; }
  __device__ __forceinline__ int rows_of(int j) const { return min(C::BN, L - j * C::BN); }
  // Stage i (K(i), V(i-1)) into the ring slot at byte offset off.  Stage 0 has no V tile and stage n no K
  // tile; those halves repeat a neighbouring tile instead, so every stage is the same
  // number of copies and the counted waits stay exact.
  __device__ __forceinline__ void issue(const FwdParams& p, const FwdLane<D>& ln, int i, int off, JFA_LDS char* smem,
                                        int wave, int lane) const {
    const int64_t rkv = (int64_t)p.num_kv_heads * D;
    const uint32_t rkvb = (uint32_t)(rkv * 2);
    JFA_LDS char* slot_p = smem + off;
    const int kt = tile_of(min(i, n - 1)), vt = tile_of(max(i - 1, 0));
    ln.copy.issue_rows(kp + (int64_t)kt * C::BN * rkv, rkvb, rows_of(kt), slot_p, wave, lane);
    ln.copy.issue_rows(vp + (int64_t)vt * C::BN * rkv, rkvb, rows_of(vt), slot_p + C::TILE, wave, lane);
  }
  // This lane's Q row as B operands (rows past the tile's queries are zero).
  __device__ __forceinline__ void load_q(const FwdParams& p, bf16x8 (&qf)[C::NKS], int half) const {
    const int64_t qrow = SELF ? s0 + row : (int64_t)row;
    const uint16_t* qp = p.q + qrow * ((int64_t)p.num_heads * D) + (int64_t)h * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) qf[ks] = as_bf16x8(row < Lq ? ld16(qp + ks * 16) : zero16());
  }
};

// Key steps (K/V tiles) of a forward tile: n of its geometry, without building it.
template <int D, int MODE>
__device__ __forceinline__ int key_steps(const FwdParams& p, Tile tile) {
  if constexpr (MODE == kBroadcastQ || MODE == kSelfChunks) {
    const int L = p.chunks[2 * p.num_chunks + tile.b];
    return (L + kFwdKeys - 1) / kFwdKeys;
  } else {
    const int L = (int)(p.offsets[tile.b + 1] - p.offsets[tile.b]);
    if constexpr (MODE == kSelfSparse) return L > 0 ? p.sel_k[tile.b] : 0;
    return (L + kFwdKeys - 1) / kFwdKeys;
  }
}

// LDS of the epilogue's O staging: half a tile of bf16 rows, RB + 8 bytes apart.
template <int D>
constexpr int fwd_staging_bytes() { return (kFwdRows / 2) * (2 * D + 8); }

// One forward tile.  Stage i of the tile lives in ring slot (sb + i) % NS.  qf holds
// the tile's Q rows when pre (the previous tile loaded them and copied stages 0, 1).
// has_next: the next tile nx (with keys) starts loading after this tile's last softmax
// phase -- its Q rows into qf (dead after this tile's last S product) and its stages 0,
// 1 into the two slots after this tile's last stage (their stages n - 2, n - 1 are no
// longer read).  Returns the number of epilogue stores this wave issued.
template <int D, int MODE>
__device__ __forceinline__ int fwd_tile(const FwdParams& p, Tile tile, bool has_next, Tile nx, bool pre, int sb,
                                        int prev_stores, bf16x8 (&qf)[FwdCfg<D>::NKS], JFA_LDS char* smem,
                                        JFA_LDS char* stg, const FwdLane<D>& ln, int tid) {
  using C = FwdCfg<D>;
  constexpr bool SELF = FwdGeo<D, MODE>::SELF;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar control flow
  const int g = wave >> 2;  // 0: group A, 1: group B (same SIMD as wave - 4)
  const int half = lane >> 5;
  const int H = p.num_heads;
  const int64_t rs = (int64_t)H * D;                   // q, o row stride
  const float c = p.scale_log2;
  FwdGeo<D, MODE> t;
  t.init(p, tile, wave, lane & 31);
  const int n = t.n, row = t.row, Lq = t.Lq;

  FwdWave<D> w(qf);
  if (!pre) t.load_q(p, qf, half);
  w.m = -INFINITY;
  w.l = 0.f;
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) w.o[db][i] = 0.f;

  if (n > 0) {
    // Ring slots as byte offsets advanced one stage at a time (a scalar per use; a
    // modulo of the stage number would be folded into every lane's LDS address).
    constexpr int LAST = (C::NS - 1) * C::STAGE;
    auto adv = [](int off) { return off == LAST ? 0 : off + C::STAGE; };
    int mat_off = sb * C::STAGE;        // stage of the current matrix phase
    int iss_off = adv(adv(mat_off));    // slot of the next stage to copy (stage 2 first)
    auto issue = [&](int i, int off) { t.issue(p, ln, i, off, smem, wave, lane); };
    if (pre) {
      // Q and stage 0 landed (stage 1 and the previous tile's epilogue stores, issued
      // after them, may not have)
      wait_vmem_at_most(C::DMA_PER_STAGE + prev_stores);
    } else {
      issue(0, mat_off);
      wait_vmem();  // Q and stage 0
      issue(1, adv(mat_off));
    }
    phase_barrier();

    // Phase ph (0 .. 2n+1): group A runs matrix phase i in phase 2i and vector phase i
    // in phase 2i+1; group B runs the same one phase later.  Every wave passes 2n+2
    // barriers: group B idles through phase 0, group A through phase 2n+1.
    int ph = 0;
    auto end_phase = [&]() {
      if ((ph & 1) && ph < 2 * n + 1) {
        // stage ph/2 + 1 is read from the next phase on; stage ph/2 + 2 may still be in
        // flight (after the last phase nothing of this tile is waited for: the next
        // tile's loads stay in flight through the epilogue)
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
    // A wave whose 32 query rows all lie past the end (the last tile of a sequence) runs
    // the same phases -- copies, waits, barriers -- without the products and the softmax.
    auto phases = [&](auto compute_tag) {
      constexpr bool COMP = decltype(compute_tag)::value;
      if (g) end_phase();
      // matrix phase 0: S(0) only.  Matrix phases run at raised wave priority: when both
      // waves of a SIMD have an instruction ready, the one feeding the matrix core goes
      // first (measured: 1.7 % faster than equal priorities; raising the vector phase
      // instead changes nothing).
      if constexpr (COMP) {
        __builtin_amdgcn_s_setprio(2);
        mma_s<D>(smem + mat_off, ln, w);
        pin_matrix_phase<D>(w);
        __builtin_amdgcn_s_setprio(0);
      }
      end_phase();
      for (int i = 1; i < n; ++i) {
        if constexpr (COMP) {
          softmax_phase<D>(w, C::BN, half, c);  // tiles before the last are full
          pin_vector_phase<D>(w);
        }
        end_phase();
        mat_off = adv(mat_off);
        if constexpr (COMP) {
          const JFA_LDS char* slot_p = smem + mat_off;
          __builtin_amdgcn_s_setprio(2);
          mma_pv_s<D>(slot_p, slot_p + C::TILE, ln, w);
          order_mixed_phase<D>();
          pin_matrix_phase<D>(w);
          __builtin_amdgcn_s_setprio(0);
        }
        end_phase();
      }
      if constexpr (COMP) {
        softmax_phase<D>(w, t.rows_of(t.tile_of(n - 1)), half, c);
        pin_vector_phase<D>(w);
      }
      end_phase();
      if (has_next) {
        FwdGeo<D, MODE> t2;
        t2.init(p, nx, wave, lane & 31);
        t2.load_q(p, qf, half);
        // every stage 2 .. n has been issued: iss_off is the slot of stage n + 1
        t2.issue(p, ln, 0, iss_off, smem, wave, lane);
        t2.issue(p, ln, 1, adv(iss_off), smem, wave, lane);
      }
      // matrix phase n: O += V(n-1) P(n-1) only
      if constexpr (COMP) {
        __builtin_amdgcn_s_setprio(2);
        mma_pv<D>(smem + adv(mat_off) + C::TILE, ln, w);
        pin_matrix_phase<D>(w);
        __builtin_amdgcn_s_setprio(0);
      }
      end_phase();
      if (!g) end_phase();
    };
    if ((row - (lane & 31)) < Lq) phases(std::true_type{});
    else phases(std::false_type{});
  }

  // Epilogue: O / l in bf16, lse = ln 2 * (m*c + log2 l); empty rows give 0 and -inf.
  const bool any_row = (row - (lane & 31)) < Lq;  // wave-uniform: the wave's first row exists
  const float lt = half_sum(w.l);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  const float lse = lt > 0.f ? (w.m * c + fast_log2(lt)) * kLn2 : -INFINITY;
  constexpr bool CHUNKED = FwdGeo<D, MODE>::CHUNKED;
  int stores = 0;  // vector-memory stores this wave issues (counted by the next tile's first wait)
  if (CHUNKED && t.slot >= 0) {
    // chunk of a cut sequence: fp32 O / l and lse of this chunk, merged afterwards
    // (broadcast-Q: slot s of [S, Mq, H] rows; self: part row t.slot + row of [R, H])
    if (row < Lq) {
      const int64_t prow = SELF ? (int64_t)t.slot + row : (int64_t)t.slot * p.num_q + row;
      float* po = p.part_o + (prow * H + t.h) * D + 4 * half;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x16& x = w.o[db];
          *reinterpret_cast<float4*>(po + 32 * db + 8 * g4) =
              make_float4(x[4 * g4] * inv, x[4 * g4 + 1] * inv, x[4 * g4 + 2] * inv, x[4 * g4 + 3] * inv);
        }
      if (half == 0) {
        if constexpr (SELF) p.part_lse[prow * H + t.h] = lse;
        else p.part_lse[((int64_t)t.slot * H + t.h) * p.num_q + row] = lse;
      }
    }
    stores = any_row ? 4 * C::NDB + 1 : 0;
  } else {
    if (row < Lq && half == 0) {
      const int64_t li = SELF ? (int64_t)t.h * p.total_tokens + t.s0 + row : ((int64_t)t.b * H + t.h) * p.num_q + row;
      p.lse[li] = lse;
    }
    stores = any_row ? 1 : 0;
    // O rows through LDS, half a tile at a time (half r = rows 128 r .. 128 r + 127, the
    // rows of wave group r), as bf16 [row][D] with rows RB + 8 bytes apart (the 32 rows of
    // one write land in distinct banks); then all eight waves write whole rows with
    // 16-byte stores instead of each lane writing 8-byte pieces of its own row.  Rows past
    // the end repeat the half's last row (same address, same value).
    constexpr int PITCH = C::RB + 8, HR = C::BM / 2, CPR = C::RB / 16;
    constexpr int PASSES = HR * CPR / (C::NW * 64);
    int tl = tid;
    asm volatile("" : "+v"(tl));  // computed here, not hoisted and kept live through the phases
    const int wbase = (((tl >> 6) & 3) * 32 + (tl & 31)) * PITCH + 8 * ((tl >> 5) & 1);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int valid = min(HR, Lq - t.blk * C::BM - HR * r);  // workgroup-uniform
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
      const int row0 = t.blk * C::BM + HR * r;
      uint16_t* ob = p.o + (SELF ? t.s0 + row0 : (int64_t)t.b * p.num_q + row0) * rs + (int64_t)t.h * D;
#pragma unroll
      for (int k = 0; k < PASSES; ++k) {
        const int q = tl + C::NW * 64 * k;
        const int rr = min(q / CPR, valid - 1), cc = q % CPR;
        const int ro = rr * PITCH + 16 * cc;
        const u32x2 lo = lds_ld8(stg, ro), hi = lds_ld8(stg, ro + 8);
        st16(ob + (int64_t)rr * rs + 8 * cc, u32x4{lo[0], lo[1], hi[0], hi[1]});
      }
      stores += PASSES;
      __syncthreads();
    }
  }
  return stores;
}

template <int D, int MODE>
__global__ void __launch_bounds__(kFwdWaves * 64)
    __attribute__((amdgpu_waves_per_eu(kFwdWgPerCu * kFwdWaves / 4, kFwdWgPerCu * kFwdWaves / 4))) fwd_kernel(FwdParams p) {
  using C = FwdCfg<D>;
  __shared__ __attribute__((aligned(16))) char smem_raw[C::NS * C::STAGE];
  __shared__ __attribute__((aligned(16))) char stg_raw[fwd_staging_bytes<D>()];
  __shared__ int next_tile;
  JFA_LDS char* smem = (JFA_LDS char*)smem_raw;
  JFA_LDS char* stg = (JFA_LDS char*)stg_raw;
  const int tid = threadIdx.x;
  const int prog = xcd_program_id(blockIdx.x, gridDim.x);
  FwdLane<D> ln;
  ln.krow.init(tid & 63);
  ln.vtr.init(tid & 63);
  ln.copy.init((uint32_t)(p.num_kv_heads * D * 2), tid >> 6, tid & 63);  // k, v row stride
  // dynamic: counter group grp (one XCD's programs) takes its own tile segment
  const int gsize = gridDim.x / dynamic_groups(gridDim.x), grp = prog / gsize;
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
  // The next tile is reserved one tile ahead, so that its Q rows and first two stages
  // load during the current tile's last phases.
  bf16x8 qf[C::NKS];
  bool pre = false;
  int sb = 0, stores = 0;
  Tile cur = p.tiles[idx];
  int cur_n = key_steps<D, MODE>(p, cur);
  while (true) {
    int nxt = idx + 1;
    if (p.dynamic) {
      if (tid == 0) next_tile = base + gsize + atomicAdd(p.counters + grp, 1);
      __syncthreads();
      nxt = next_tile;
    }
    if (tid == 0) count_visit(p.visits, idx);
    const bool more = nxt < end;
    const Tile nt = more ? p.tiles[nxt] : cur;
    const int nt_n = more ? key_steps<D, MODE>(p, nt) : 0;
    const bool ahead = more && cur_n > 0 && nt_n > 0;
    stores = fwd_tile<D, MODE>(p, cur, ahead, nt, pre, sb, stores, qf, smem, stg, ln, tid);
    if (!more) break;
    if (cur_n > 0) sb = (sb + cur_n + 1) % C::NS;
    pre = ahead;
    idx = nxt;
    cur = nt;
    cur_n = nt_n;
    if (p.dynamic) __syncthreads();  // every wave has read next_tile before it is rewritten
  }
}

template <int D, int MODE>
hipError_t launch(const FwdParams& p, hipStream_t s) {
  hipLaunchKernelGGL((fwd_kernel<D, MODE>), dim3(p.num_programs), dim3(kFwdWaves * 64), 0, s, p);
  return hipGetLastError();
}

// One pass over the chunk partials of one (row, head) and 8 head-dim columns: with
// m the running maximum of the chunks' lse, s = sum_c exp(lse_c - m) and acc = sum_c
// exp(lse_c - m) O_c (each sum rescaled when m grows), so that O = acc / s and
// lse = m + ln s at the end; a chunk's loads do not wait on the previous chunk's sums.
struct LseMerge {
  float m = -INFINITY, s = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  __device__ __forceinline__ void add(float l, const float* o8) {
    const float4 a = reinterpret_cast<const float4*>(o8)[0];
    const float4 e = reinterpret_cast<const float4*>(o8)[1];
    if (!(l > -INFINITY)) return;  // a chunk with no keys for this row adds nothing
    if (l > m) {
      const float r = expf(m - l);  // 0 on the first chunk (m = -inf)
      s *= r;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] *= r;
      m = l;
    }
    const float w = expf(l - m);
    s += w;
    acc[0] += w * a.x; acc[1] += w * a.y; acc[2] += w * a.z; acc[3] += w * a.w;
    acc[4] += w * e.x; acc[5] += w * e.y; acc[6] += w * e.z; acc[7] += w * e.w;
  }
  // O (bf16, 8 columns) and, where lse_out is non-null, the row's lse
  __device__ __forceinline__ void store(uint16_t* o, float* lse_out) const {
    const float inv = s > 0.f ? 1.0f / s : 0.f;
    st16(o, __builtin_bit_cast(u32x4, pack8(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv, acc[4] * inv,
                                            acc[5] * inv, acc[6] * inv, acc[7] * inv)));
    if (lse_out) *lse_out = s > 0.f ? m + logf(s) : -INFINITY;
  }
};

// Merge of the chunk partials of cut broadcast-Q sequences: for cut sequence i with
// slots f .. f + n - 1 and each (query row, head), lse = log sum_c exp(lse_c) and
// O = sum_c exp(lse_c - lse) O_c (each O_c normalised by its own row sum, so the
// weights are the chunks' shares of the full row sum), in one pass (LseMerge).  One
// thread per 8 head-dim columns of a (cut sequence, row, head).
__global__ void bq_combine_kernel(FwdParams p, int cuts, int D) {
  const int nc = p.num_chunks, H = p.num_heads, Mq = p.num_q, nd8 = D / 8;
  const int64_t total = (int64_t)cuts * Mq * H * nd8;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int d8 = (int)(i % nd8);
    const int h = (int)((i / nd8) % H);
    const int row = (int)((i / ((int64_t)nd8 * H)) % Mq);
    const int cut = (int)(i / ((int64_t)nd8 * H * Mq));
    const int* t = p.chunks + 4 * nc + 3 * cut;
    const int b = t[0], first = t[1], n = t[2];
    LseMerge mg;
    for (int c = 0; c < n; ++c)
      mg.add(p.part_lse[((int64_t)(first + c) * H + h) * Mq + row],
             p.part_o + (((int64_t)(first + c) * Mq + row) * H + h) * D + 8 * d8);
    const int64_t orow = (int64_t)b * Mq + row;
    mg.store(p.o + (orow * H + h) * D + 8 * d8, d8 == 0 ? p.lse + ((int64_t)b * H + h) * Mq + row : nullptr);
  }
}

// Merge of the chunk partials of cut self-attention sequences (same weights as
// bq_combine_kernel).  Cut i (sequence b_i, n_i chunks of part rows f_i + c L_b ..,
// c < n_i) owns rows prefix[i] .. prefix[i + 1] - 1 of the merge's row space; one thread
// per 8 head-dim columns of a (row, head).  The table follows the 4 nc chunk entries:
// b[ncut] | first part row[ncut] | chunks[ncut] | row prefix[ncut + 1].
__global__ void self_combine_kernel(FwdParams p, int cuts, int D) {
  const int nc = p.num_chunks, H = p.num_heads, nd8 = D / 8;
  const int* cb = p.chunks + 4 * nc;
  const int* cf = cb + cuts;
  const int* cn = cf + cuts;
  const int* pre = cn + cuts;
  const int64_t total = (int64_t)pre[cuts] * H * nd8;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int d8 = (int)(i % nd8);
    const int h = (int)((i / nd8) % H);
    const int r = (int)(i / ((int64_t)nd8 * H));
    int lo = 0, hi = cuts - 1;  // the cut whose row range holds r
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre[mid] <= r) lo = mid;
      else hi = mid - 1;
    }
    const int b = cb[lo], n = cn[lo];
    const int row = r - pre[lo];
    const int64_t s0 = p.offsets[b];
    const int64_t len = p.offsets[b + 1] - s0;
    const int64_t first = cf[lo] + row;  // part row of chunk 0; chunk c is c * len further
    LseMerge mg;
    for (int c = 0; c < n; ++c) {
      const int64_t pr = first + c * len;
      mg.add(p.part_lse[pr * H + h], p.part_o + (pr * H + h) * D + 8 * d8);
    }
    mg.store(p.o + ((s0 + row) * H + h) * D + 8 * d8, d8 == 0 ? p.lse + (int64_t)h * p.total_tokens + s0 + row : nullptr);
  }
}

}  // namespace

hipError_t launch_bq_combine(const FwdParams& p, int cuts, int head_dim, hipStream_t s) {
  const int64_t total = (int64_t)cuts * p.num_q * p.num_heads * (head_dim / 8);
  if (total <= 0) return hipSuccess;
  const int64_t g = (total + 255) / 256;
  hipLaunchKernelGGL(bq_combine_kernel, dim3((unsigned)(g < 4096 ? g : 4096)), dim3(256), 0, s, p, cuts, head_dim);
  return hipGetLastError();
}

hipError_t launch_self_combine(const FwdParams& p, int cuts, int64_t rows, int head_dim, hipStream_t s) {
  const int64_t total = rows * p.num_heads * (head_dim / 8);
  if (cuts <= 0 || total <= 0) return hipSuccess;
  const int64_t g = (total + 255) / 256;
  hipLaunchKernelGGL(self_combine_kernel, dim3((unsigned)(g < 4096 ? g : 4096)), dim3(256), 0, s, p, cuts, head_dim);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdParams& p, int mode, int head_dim, hipStream_t s) {
  if (p.num_programs <= 0) return hipSuccess;
  if (mode == kSelf) return head_dim == 64 ? launch<64, kSelf>(p, s) : launch<128, kSelf>(p, s);
  if (mode == kSelfSparse) return head_dim == 64 ? launch<64, kSelfSparse>(p, s) : launch<128, kSelfSparse>(p, s);
  if (mode == kSelfChunks) return head_dim == 64 ? launch<64, kSelfChunks>(p, s) : launch<128, kSelfChunks>(p, s);
  return head_dim == 64 ? launch<64, kBroadcastQ>(p, s) : launch<128, kBroadcastQ>(p, s);
}

}  // namespace jfa
