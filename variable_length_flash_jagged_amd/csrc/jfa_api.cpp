// C ABI of the jagged flash attention library: argument checks, offsets intake, host
// scheduling, workspace layout, schedule upload and kernel launches.
//
// Offsets intake follows the jagged layout of the explore.n1n.ai page (section on the
// performance defects of padded tensors): offsets[0] = 0, non-decreasing, offsets[B]
// = T.  When the caller passes host offsets, every scalar of the schedule is computed
// on the host before launch with no device synchronisation (bittide page, section 5).
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <string>
#include <vector>

#include "jfa.h"
#include "jfa_internal.h"
#include "jfa_sched.h"

using namespace jfa;

static_assert(JFA_NOALLOC_SCRATCH_BYTES == kNoAllocScratchBytes, "scratch size in the header");

namespace {

thread_local std::string g_detail;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_detail = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(JFA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int kv_heads(const jfa_shape* s) { return s->num_kv_heads > 0 ? s->num_kv_heads : s->num_heads; }

// Compute units of the current device (256 if no device is visible: host-only use).
int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
      (void)hipGetLastError();
      n = 256;
    }
    cache[dev] = n;
  }
  return cache[dev];
}

struct Opts {
  int sched = 0, dq_path = 0, num_programs = 0;
  int64_t ds_budget = 0;  // bytes
};

int check_opts(const jfa_opts* o, Opts& out) {
  out = Opts();
  if (!o) return JFA_OK;
  if (o->sched != 0 && o->sched != 1) return fail(JFA_ERR_BAD_OPTION, "opts.sched must be 0 or 1");
  if (o->dq_path < 0 || o->dq_path > 2) return fail(JFA_ERR_BAD_OPTION, "opts.dq_path must be 0, 1 or 2");
  if (o->num_programs < 0 || o->num_programs > (1 << 20))
    return fail(JFA_ERR_BAD_OPTION, "opts.num_programs out of range");
  if (o->ds_budget_mib < 0 || o->ds_budget_mib > (1 << 20))
    return fail(JFA_ERR_BAD_OPTION, "opts.ds_budget_mib must be in [0, 2^20]");
  out.sched = o->sched;
  out.dq_path = o->dq_path;
  out.num_programs = o->num_programs;
  out.ds_budget = (int64_t)o->ds_budget_mib << 20;
  return JFA_OK;
}

int check_shape(const jfa_shape* s, int mode) {
  if (!s) return fail(JFA_ERR_NULL_POINTER, "shape is NULL");
  if (mode != JFA_MODE_SELF && mode != JFA_MODE_BROADCAST_Q && mode != JFA_MODE_BLOCK_DIAG)
    return fail(JFA_ERR_BAD_MODE, "mode %d is not a jfa_mode", mode);
  if (s->num_seqs < 0) return fail(JFA_ERR_BAD_SHAPE, "num_seqs < 0");
  if (s->num_heads < 1 || s->num_heads > 127) return fail(JFA_ERR_BAD_SHAPE, "num_heads must be in [1, 127]");
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(JFA_ERR_BAD_HEAD_DIM, "head_dim %d not in {64, 128}", s->head_dim);
  if (s->total_tokens < 0) return fail(JFA_ERR_BAD_SHAPE, "total_tokens < 0");
  if (s->reserved != 0) return fail(JFA_ERR_BAD_SHAPE, "shape.reserved must be 0");
  if (s->num_kv_heads < 0 || s->num_kv_heads > s->num_heads || (s->num_kv_heads > 0 && s->num_heads % s->num_kv_heads))
    return fail(JFA_ERR_BAD_SHAPE, "num_kv_heads %d must be 0 or divide num_heads %d", s->num_kv_heads, s->num_heads);
  if (mode == JFA_MODE_BROADCAST_Q && s->num_q < 1) return fail(JFA_ERR_BAD_SHAPE, "num_q < 1 in broadcast-Q mode");
  // 32-bit limits: block indices < 2^24 in the tile encoding, tile counts < 2^31.
  if (s->total_tokens >= (int64_t(1) << 30)) return fail(JFA_ERR_TOO_LARGE, "total_tokens >= 2^30");
  if (mode == JFA_MODE_BROADCAST_Q && s->num_q >= (1 << 24)) return fail(JFA_ERR_TOO_LARGE, "num_q >= 2^24");
  if (mode == JFA_MODE_BROADCAST_Q && (int64_t)s->num_seqs * s->num_q >= (int64_t(1) << 31))
    return fail(JFA_ERR_TOO_LARGE, "num_seqs * num_q >= 2^31");
  return JFA_OK;
}

int max_programs(const Opts& o, int wg_per_cu) {
  return o.num_programs > 0 ? o.num_programs : device_cus() * wg_per_cu;
}

// Resident workgroups per CU of the main (dK/dV or fused) backward kernel: the
// self-attention dK/dV kernel, which broadcast-Q dq_path 2 also runs, or the fused
// broadcast-Q kernel.  jfa_bwd and jfa_schedule both size the schedule with it.
int bwd_wg_per_cu(int mode, int dq_path, int head_dim) {
  return mode == JFA_MODE_SELF || (mode == JFA_MODE_BROADCAST_Q && dq_path == 2) ? dkdv_wg_per_cu(head_dim)
                                                                                 : kBqWgPerCu;
}

// Workspace layout (byte offsets, each region 256-byte aligned).
struct Layout {
  size_t counters = 0, seg = 0, tiles = 0, seg2 = 0, tiles2 = 0, ds_base = 0, stats = 0, ds = 0, prefix = 0, acc = 0,
         total = 0;
  // block-sparse forward: per-sequence arrays (uploaded with the schedule) and the
  // block means
  size_t sp_qt = 0, sp_kb = 0, sp_base = 0, sp_k = 0, sp_qbar = 0, sp_kbar = 0;
  int64_t sp_nqt_cap = 0, sp_nkb_cap = 0;
  int64_t seg_cap = 0, tile_cap = 0, seg2_cap = 0, tile2_cap = 0;
  // broadcast-Q key chunks (forward; split backward): chunk table and its capacity;
  // forward: partial-result slots of cut sequences (O [S,Mq,H,D], lse [S,H,Mq], fp32)
  size_t chunks = 0, part_o = 0, part_lse = 0;
  int64_t chunk_cap = 0, fwd_slot_cap = 0;
  // self-attention forward key chunks: partial rows x heads the buffers hold (0: the
  // layout has no room for them and the forward never cuts)
  int64_t self_part_cap = 0;
  int programs_cap = 0, programs2_cap = 0;
};

// Key chunks of broadcast-Q tiles (the forward's and the split backward's dQ kernel):
// a sequence longer than one program's fair share of key steps is cut into chunks of
// kKeyStep * max(kBqChunkMinSteps, share) keys, share = ceil(H * ceil(Mq / rows) *
// sum_b ceil(L_b / kKeyStep) / programs), so that no tile walks far more keys than the
// average program; each chunk is then a tile "sequence" of its own (cost key: its
// keys) and the chunks' partial results are merged afterwards.  Chunks are listed in
// sequence order; keep_empty gives an empty sequence one chunk of zero keys.
constexpr int kKeyStep = 64;
static_assert(kKeyStep == kFwdKeys && kKeyStep == kDqKeys, "one key step for both chunk rules");

struct KeyChunks {
  std::vector<int32_t> b, k0, len;
  int64_t keys = 0;  // chunk size
};

void bq_key_chunks(const std::vector<int32_t>& lengths, int64_t H, int64_t Mq, int rows, int programs,
                   bool keep_empty, KeyChunks& out) {
  int64_t steps = 0;
  for (int32_t len : lengths) steps += cdiv(len, kKeyStep);
  const int64_t share = cdiv(H * cdiv(Mq, rows) * steps, std::max(1, programs));
  out.keys = kKeyStep * std::max<int64_t>(kBqChunkMinSteps, share);
  out.b.clear();
  out.k0.clear();
  out.len.clear();
  for (int b = 0; b < (int)lengths.size(); ++b) {
    if (lengths[b] == 0 && keep_empty) {
      out.b.push_back(b);
      out.k0.push_back(0);
      out.len.push_back(0);
    }
    for (int64_t k0 = 0; k0 < lengths[b]; k0 += out.keys) {
      out.b.push_back(b);
      out.k0.push_back((int32_t)k0);
      out.len.push_back((int32_t)std::min<int64_t>(out.keys, lengths[b] - k0));
    }
  }
}

// Self-attention key chunks (forward): the broadcast-Q rule with each sequence's own
// query tiles, share = ceil(H * sum_b ceil(L_b / rows) * ceil(L_b / kKeyStep) /
// programs), and chunks of at least kSelfChunkMinSteps steps (a cut costs a merge
// launch, which a shorter chunk does not repay).  Only a batch of few long sequences is
// cut (a cut needs L_b > keys, and keys >= H sum_b L_b^2 / (rows P)); empty sequences
// have no chunk.
constexpr int kSelfChunkMinSteps = 8;
void self_key_chunks(const std::vector<int32_t>& lengths, int64_t H, int rows, int programs, KeyChunks& out) {
  int64_t steps = 0;
  for (int32_t len : lengths) steps += cdiv(len, rows) * cdiv(len, kKeyStep);
  const int64_t share = cdiv(H * steps, std::max(1, programs));
  out.keys = kKeyStep * std::max<int64_t>(kSelfChunkMinSteps, share);
  out.b.clear();
  out.k0.clear();
  out.len.clear();
  for (int b = 0; b < (int)lengths.size(); ++b)
    for (int64_t k0 = 0; k0 < lengths[b]; k0 += out.keys) {
      out.b.push_back(b);
      out.k0.push_back((int32_t)k0);
      out.len.push_back((int32_t)std::min<int64_t>(out.keys, lengths[b] - k0));
    }
}

// Partial rows x heads of cut self-attention sequences: a cut sequence has L_b > keys,
// so its n_b = ceil(L_b / keys) < 2 L_b / keys chunks of L_b rows each, and with keys >=
// H sum L^2 / (rows P) the sum over cut sequences of n_b L_b H stays below 2 rows P.
int64_t self_part_cap(int programs) { return 2 * (int64_t)kFwdRows * programs; }

// Self-attention forward key chunks of one call: when some sequence is cut, the chunk
// table [b | first key | keys | first part row (-1: uncut)] of nc chunks, then the cut
// table [b | first part row | chunks | row prefix (ncut + 1)] of launch_self_combine,
// and the schedule of (chunk, h, blk) tiles.  Returns false (and touches nothing) when
// no sequence is cut: the plain schedule applies.
struct SelfSplit {
  std::vector<int32_t> table;
  int nc = 0, ncut = 0;
  int64_t cut_rows = 0;   // query rows of the cut sequences (the merge's rows)
  int64_t part_rows = 0;  // partial rows (per head) the chunks write
};

bool self_split_plan(const std::vector<int32_t>& lengths, int H, int P, bool dynamic, Schedule& sc, SelfSplit& out) {
  KeyChunks kc;
  self_key_chunks(lengths, H, kFwdRows, P, kc);
  const int nc = (int)kc.b.size();
  if (nc == 0 || nc == (int)std::count_if(lengths.begin(), lengths.end(), [](int32_t l) { return l > 0; }))
    return false;
  std::vector<int32_t> r0(nc, -1), cb, cf, cn, pre{0};
  int64_t part = 0;
  for (int c = 0; c < nc;) {
    int e = c + 1;
    while (e < nc && kc.b[e] == kc.b[c]) ++e;
    if (e - c > 1) {
      const int64_t len = lengths[kc.b[c]];
      cb.push_back(kc.b[c]);
      cf.push_back((int32_t)part);
      cn.push_back(e - c);
      pre.push_back(pre.back() + (int32_t)len);
      for (int i = c; i < e; ++i, part += len) r0[i] = (int32_t)part;
    }
    c = e;
  }
  out.nc = nc;
  out.ncut = (int)cb.size();
  out.cut_rows = pre.back();
  out.part_rows = part;
  out.table = kc.b;
  for (const auto* v : {&kc.k0, &kc.len, &r0, &cb, &cf, &cn, &pre}) out.table.insert(out.table.end(), v->begin(), v->end());
  std::vector<int32_t> rows_of(nc);
  for (int c = 0; c < nc; ++c) rows_of[c] = lengths[kc.b[c]];
  schedule_fwd_chunks(kc.len, rows_of, H, kFwdRows, P, dynamic, sc);
  return true;
}

// Split backward: the most key chunks any lengths give.  A sequence that is not cut is
// one chunk; the chunks of cut sequences number fewer than 2 T / keys, with keys at
// least kBqChunkMinSteps * kKeyStep and at least H * ceil(Mq / kDqRows) * T / programs.
int64_t bq_chunk_cap(int64_t B, int64_t H, int64_t Mq, int64_t T, int programs) {
  return B + std::min<int64_t>(2 * (int64_t)programs / std::max<int64_t>(1, H * cdiv(Mq, kDqRows)),
                               2 * T / (kBqChunkMinSteps * kKeyStep)) + 1;
}

// Forward: the most partial-result slots (chunks of sequences cut into two or more):
// a cut sequence has L > keys >= max(256, H * ceil(Mq / rows) * T / P), so its
// ceil(L / keys) < 2 L / keys chunks sum to less than 2 T / keys.
int64_t bq_fwd_slot_cap(int64_t H, int64_t Mq, int64_t T, int programs) {
  return std::min<int64_t>(2 * (int64_t)programs / std::max<int64_t>(1, H * cdiv(Mq, kFwdRows)),
                           2 * T / (kBqChunkMinSteps * kKeyStep)) + 1;
}

// key_split: room for the self-attention forward's key chunks (jfa_fwd_noalloc, whose
// scratch array is small, runs without).
void layout_for(const jfa_shape* s, int mode, int pass, const Opts& o, Layout& L, bool key_split = true) {
  const int64_t B = s->num_seqs, H = s->num_heads, D = s->head_dim, T = s->total_tokens;
  const int64_t Mq = s->num_q;
  size_t at = 0;
  L.counters = at;
  at += align_up(kCounterSlots * sizeof(int32_t));
  if (mode == JFA_MODE_BLOCK_DIAG) {
    L.prefix = at;
    at += align_up((B + 1) * sizeof(int32_t));
    L.total = at;
    return;
  }
  const bool fwd = pass != JFA_PASS_BWD;
  const bool bq_split = pass == JFA_PASS_BWD && mode == JFA_MODE_BROADCAST_Q && o.dq_path == 2;
  const int wg = pass == JFA_PASS_FWD_MXFP8 ? mx_wg_per_cu(s->head_dim)
                 : fwd                       ? kFwdWgPerCu
                                             : (mode == JFA_MODE_SELF || bq_split ? kBwdWgPerCu : kBqWgPerCu);
  L.programs_cap = max_programs(o, wg);
  L.seg_cap = std::max<int64_t>(L.programs_cap, H) + 1;
  L.seg = at;
  at += align_up(L.seg_cap * sizeof(int32_t));
  if (fwd) {
    if (mode == JFA_MODE_BROADCAST_Q) {
      // key chunks: every sequence plus the extra chunks of cut sequences
      L.fwd_slot_cap = bq_fwd_slot_cap(H, Mq, T, L.programs_cap);
      L.chunk_cap = B + L.fwd_slot_cap;
      L.tile_cap = H * L.chunk_cap * cdiv(Mq, kFwdRows);
    } else {
      L.tile_cap = H * (T / kFwdRows + B + 1);
      if (pass == JFA_PASS_FWD && mode == JFA_MODE_SELF && key_split) {
        // chunks: every sequence plus fewer than 2 T / 256 extra; tiles of cut sequences:
        // n_b ceil(L_b / rows) H < (n_b L_b H) / rows + n_b H, summed < 2 P + H extra
        L.self_part_cap = self_part_cap(L.programs_cap);
        L.chunk_cap = B + 2 * T / (kBqChunkMinSteps * kKeyStep) + 1;
        L.tile_cap += 2 * (int64_t)L.programs_cap + H * L.chunk_cap;
      }
    }
  } else {
    L.tile_cap = H * (T / kBwdKeys + B + 1);
  }
  L.tiles = at;
  at += align_up(L.tile_cap * sizeof(Tile));
  if (pass == JFA_PASS_FWD_MXFP8) {
    // tiles of mx_rows(D) query rows and the padded V start of each sequence
    L.tile_cap = H * (T / kMxMinRows + B + 1);
    L.tiles = at;
    at += align_up(L.tile_cap * sizeof(Tile));
    L.ds_base = at;
    at += align_up((B + 1) * sizeof(int64_t));
    L.prefix = at;  // V quantiser: sequence of each padded 64-key group
    at += align_up((T / kMxVPad + B + 1) * sizeof(int32_t));
    L.total = at;
    return;
  }
  if (L.self_part_cap > 0) {
    L.chunks = at;  // [sequence | first key | keys | first part row] per chunk, then the cut table
    at += align_up((4 * L.chunk_cap + 4 * B + 1) * sizeof(int32_t));
    L.part_o = at;
    at += align_up((size_t)(L.self_part_cap * D) * sizeof(float));
    L.part_lse = at;
    at += align_up((size_t)L.self_part_cap * sizeof(float));
  }
  if (pass == JFA_PASS_FWD && mode == JFA_MODE_BROADCAST_Q) {
    L.chunks = at;  // [sequence | first key | keys | slot] per chunk, then (b, first slot, slots) per cut sequence
    at += align_up((4 * L.chunk_cap + 3 * B) * sizeof(int32_t));
    L.part_o = at;
    at += align_up((size_t)(L.fwd_slot_cap * Mq * H * D) * sizeof(float));
    L.part_lse = at;
    at += align_up((size_t)(L.fwd_slot_cap * H * Mq) * sizeof(float));
  }
  if (pass == JFA_PASS_FWD_SPARSE) {
    const int64_t Hkv = s->num_kv_heads > 0 ? s->num_kv_heads : H;
    L.sp_qt = at;
    at += align_up((B + 1) * sizeof(int32_t));
    L.sp_kb = at;
    at += align_up((B + 1) * sizeof(int32_t));
    L.sp_base = at;
    at += align_up((B + 1) * sizeof(int64_t));
    L.sp_k = at;
    at += align_up((B + 1) * sizeof(int32_t));
    L.sp_nqt_cap = T / kSparseQBlock + B + 1;
    L.sp_nkb_cap = T / kSparseKBlock + B + 1;
    L.sp_qbar = at;
    at += align_up((size_t)(H * L.sp_nqt_cap * D) * sizeof(float));
    L.sp_kbar = at;
    at += align_up((size_t)(Hkv * L.sp_nkb_cap * D) * sizeof(float));
  }
  if (pass == JFA_PASS_BWD && mode == JFA_MODE_SELF) {
    // second schedule: the dQ kernel's query-row tiles (kDqRows rows on the recompute
    // path, kDsRows on the stored-dS path; the capacities cover both)
    static_assert(kDqRows <= kDsRows && kDsWgPerCu <= kDqWgPerCu, "dQ schedule capacity");
    L.programs2_cap = max_programs(o, kDqWgPerCu);
    L.seg2_cap = L.programs2_cap + 1;
    L.seg2 = at;
    at += align_up(L.seg2_cap * sizeof(int32_t));
    L.tile2_cap = H * (T / kDqRows + B + 1);
    L.tiles2 = at;
    at += align_up(L.tile2_cap * sizeof(Tile));
    L.ds_base = at;  // stored-dS path: first dS block of each sequence, int64 [B+1]
    at += align_up((B + 1) * sizeof(int64_t));
    L.stats = at;  // per query row 16-byte term (-lse log2 e, -Di in bf16 high/low), [H, T, 8], + sentinel
    at += align_up((H * T + 1) * 16);
    if (o.ds_budget > 0) {
      L.ds = at;  // stored dS, up to the budget
      at += align_up((size_t)o.ds_budget);
    }
  } else if (bq_split) {
    // dQ kernel schedule (kDqRows-row tiles of the shared queries against one key chunk
    // each), the key-chunk table int32 [3, NC], the row terms [B, H, Mq, 8] + sentinel,
    // and the chunks' dQ slabs [NC, Mq, H, D] fp32 (NC <= B + T / minimum chunk)
    L.programs2_cap = max_programs(o, kDqWgPerCu);
    L.chunk_cap = bq_chunk_cap(B, H, Mq, T, L.programs2_cap);
    L.seg2_cap = L.programs2_cap + 1;
    L.seg2 = at;
    at += align_up(L.seg2_cap * sizeof(int32_t));
    L.tile2_cap = H * cdiv(Mq, kDqRows) * L.chunk_cap;
    L.tiles2 = at;
    at += align_up(L.tile2_cap * sizeof(Tile));
    L.chunks = at;
    at += align_up(3 * L.chunk_cap * sizeof(int32_t));
    L.stats = at;
    at += align_up((B * H * Mq + 1) * 16);
    L.acc = at;
    at += align_up((size_t)(L.chunk_cap * Mq * H * D) * sizeof(float));
  } else if (pass == JFA_PASS_BWD) {
    L.acc = at;
    const int64_t acc_elems = (o.dq_path == 0) ? Mq * H * D : (int64_t)std::max<int64_t>(L.programs_cap, H) * Mq * D;
    at += align_up(acc_elems * sizeof(float));
  }
  L.total = at;
}

// Lengths from host offsets (or the device copy on the slow path), validated.
int intake_offsets(const jfa_shape* s, const int32_t* off_dev, const int32_t* off_host,
                   hipStream_t stream, std::vector<int32_t>& lengths) {
  const int B = s->num_seqs;
  std::vector<int32_t> tmp;
  const int32_t* off = off_host;
  if (!off) {
    if (!off_dev) return fail(JFA_ERR_NULL_POINTER, "offsets_dev and offsets_host are both NULL");
    tmp.resize(B + 1);
    hipError_t e = hipMemcpyAsync(tmp.data(), off_dev, (B + 1) * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "copying device offsets to the host");
    off = tmp.data();
  }
  if (off[0] != 0) return fail(JFA_ERR_BAD_OFFSETS, "offsets[0] = %d, must be 0", off[0]);
  lengths.resize(B);
  for (int b = 0; b < B; ++b) {
    if (off[b + 1] < off[b]) return fail(JFA_ERR_BAD_OFFSETS, "offsets decrease at index %d", b + 1);
    lengths[b] = off[b + 1] - off[b];
  }
  if ((int64_t)off[B] != s->total_tokens)
    return fail(JFA_ERR_BAD_OFFSETS, "offsets[B] = %d differs from total_tokens = %lld", off[B],
                (long long)s->total_tokens);
  return JFA_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Stored-dS blocks (kBwdKeys keys x kBwdRows queries) of one head of a sequence of
// length len.
int64_t ds_blocks(int64_t len) { return cdiv(len, kBwdKeys) * cdiv(len, kBwdRows); }

// Pinned host staging ring for the asynchronous schedule upload.  A slot is reused
// only after the copy that last read it has completed (its event).
struct StagingRing {
  static constexpr int kSlots = 8;
  struct Slot {
    void* host = nullptr;
    size_t cap = 0;
    hipEvent_t ev = nullptr;
    bool pending = false;
  } slot[kSlots];
  int next = 0;
  std::mutex mu;
};
StagingRing g_ring[64];

// Copy `bytes` from `src` into the workspace at `dst` on `stream` via a pinned slot.
int upload(const void* src, size_t bytes, void* dst, hipStream_t stream) {
  if (bytes == 0) return JFA_OK;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= 64) return hip_fail(e, "hipGetDevice");
  StagingRing& ring = g_ring[dev];
  std::lock_guard<std::mutex> lock(ring.mu);
  StagingRing::Slot& s = ring.slot[ring.next];
  ring.next = (ring.next + 1) % StagingRing::kSlots;
  if (s.pending) {
    e = hipEventSynchronize(s.ev);
    if (e != hipSuccess) return hip_fail(e, "waiting for a staging slot");
    s.pending = false;
  }
  if (!s.ev) {
    e = hipEventCreateWithFlags(&s.ev, hipEventDisableTiming);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
  }
  if (s.cap < bytes) {
    if (s.host) (void)hipHostFree(s.host);
    s.host = nullptr;
    s.cap = 0;
    const size_t cap = std::max<size_t>(bytes, 1 << 16);
    e = hipHostMalloc(&s.host, cap, hipHostMallocDefault);
    if (e != hipSuccess) return hip_fail(e, "hipHostMalloc (staging)");
    s.cap = cap;
  }
  memcpy(s.host, src, bytes);
  e = hipMemcpyAsync(dst, s.host, bytes, hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return hip_fail(e, "uploading the schedule");
  e = hipEventRecord(s.ev, stream);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  s.pending = true;
  return JFA_OK;
}

thread_local int g_bwd_path = JFA_BWD_PATH_OTHER;  // jfa_last_bwd_path

// Per-device side stream (default priority) on which a latency-bound recompute
// backward runs its dQ kernel beside the dK/dV kernel, with the events that fork it from
// the caller's stream and join it back.  The mutex is held while a call enqueues the
// fork, the dQ launch and the join.
struct SideStream {
  std::mutex mu;
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
SideStream g_side[64];

// Locks and returns this device's side stream, creating it on first use.
int side_stream(SideStream** out, std::unique_lock<std::mutex>& lock) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= 64) return hip_fail(e, "hipGetDevice");
  SideStream& ss = g_side[dev];
  lock = std::unique_lock<std::mutex>(ss.mu);
  if (!ss.s) {
    e = hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking);
    if (e != hipSuccess) return hip_fail(e, "hipStreamCreate (side stream)");
  }
  if (!ss.fork) {
    e = hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreate (fork)");
  }
  if (!ss.join) {
    e = hipEventCreateWithFlags(&ss.join, hipEventDisableTiming);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreate (join)");
  }
  *out = &ss;
  return JFA_OK;
}

// Allocation-free variant of upload(): a plain copy from the caller's (pageable) host
// bytes.  The runtime stages pageable memory itself and returns once it has taken the
// bytes, so `src` may be reused as soon as this returns.  No pinned staging buffer is
// allocated.
int upload_pageable(const void* src, size_t bytes, void* dst, hipStream_t stream) {
  if (bytes == 0) return JFA_OK;
  hipError_t e = hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return hip_fail(e, "uploading the schedule");
  return JFA_OK;
}

// Serialise [counters | seg_ptr | tiles (| seg_ptr2 | tiles2)] of one or two schedules
// for the device (counters start at zero).
void put_schedule(const Schedule& sc, size_t seg_off, size_t tiles_off, std::vector<char>& buf) {
  memcpy(buf.data() + seg_off, sc.seg_ptr.data(), sc.seg_ptr.size() * sizeof(int32_t));
  Tile* t = reinterpret_cast<Tile*>(buf.data() + tiles_off);
  for (size_t i = 0; i < sc.tiles.size(); ++i)
    t[i] = Tile{sc.tiles[i].b, (sc.tiles[i].h << 24) | sc.tiles[i].blk};
}

void serialise(const Schedule& sc, const Layout& L, std::vector<char>& buf, const Schedule* sc2 = nullptr,
               const std::vector<int64_t>* ds_base = nullptr, const std::vector<int32_t>* chunks = nullptr) {
  size_t end = L.tiles + sc.tiles.size() * sizeof(Tile);
  if (sc2) end = L.tiles2 + sc2->tiles.size() * sizeof(Tile);
  if (ds_base) end = L.ds_base + ds_base->size() * sizeof(int64_t);
  if (chunks) end = L.chunks + chunks->size() * sizeof(int32_t);
  buf.assign(end, 0);
  put_schedule(sc, L.seg, L.tiles, buf);
  if (sc2) put_schedule(*sc2, L.seg2, L.tiles2, buf);
  if (ds_base) memcpy(buf.data() + L.ds_base, ds_base->data(), ds_base->size() * sizeof(int64_t));
  if (chunks) memcpy(buf.data() + L.chunks, chunks->data(), chunks->size() * sizeof(int32_t));
}

// Block-sparse forward: per-sequence query / key block prefixes, kept blocks per query
// block and the first selection entry of each sequence.
struct SparsePlan {
  std::vector<int32_t> qt_prefix, kb_prefix, sel_k;
  std::vector<int64_t> sel_base;
};

int sparse_plan(const jfa_shape* s, const std::vector<int32_t>& lengths, float ratio, SparsePlan& P) {
  if (!(ratio > 0.f && ratio <= 1.f)) return fail(JFA_ERR_BAD_OPTION, "ratio must be in (0, 1]");
  const size_t B = lengths.size();
  P.qt_prefix.assign(B + 1, 0);
  P.kb_prefix.assign(B + 1, 0);
  P.sel_base.assign(B + 1, 0);
  P.sel_k.assign(B + 1, 0);
  for (size_t b = 0; b < B; ++b) {
    const int64_t len = lengths[b];
    const int64_t nqt = cdiv(len, kSparseQBlock), nkb = cdiv(len, kSparseKBlock);
    if (nkb > kSparseMaxKeyBlocks)
      return fail(JFA_ERR_TOO_LARGE, "sequence %zu has %lld key blocks; the block-sparse forward takes at most %d", b,
                  (long long)nkb, kSparseMaxKeyBlocks);
    const int32_t k = len > 0 ? std::max<int32_t>(1, (int32_t)std::ceil((double)ratio * (double)nkb)) : 0;
    P.qt_prefix[b + 1] = P.qt_prefix[b] + (int32_t)nqt;
    P.kb_prefix[b + 1] = P.kb_prefix[b] + (int32_t)nkb;
    P.sel_k[b] = k;
    P.sel_base[b + 1] = P.sel_base[b] + (int64_t)s->num_heads * nqt * k;
  }
  return JFA_OK;
}

// Block-sparse backward: the recompute backward's workspace (no dS budget; its dQ
// schedule is used) followed by the selection plan (sel_base, sel_k), the dK/dV
// schedule (64-key tiles of two waves at head_dim 128, 128-key tiles otherwise) and the
// dK/dV tiles' query-block bitmaps.
struct SparseBwdLayout {
  Layout base;
  size_t sel_base = 0, sel_k = 0, bits_base = 0, kv_seg = 0, kv_tiles = 0, bits = 0, total = 0;
  int64_t kv_seg_cap = 0, kv_tile_cap = 0;
  int tile_keys = 0, programs = 0;
  std::vector<int64_t> bits_prefix;  // [B+1] first bitmap word of each sequence
};

void sparse_bwd_layout(const jfa_shape* s, const std::vector<int32_t>& lengths, const Opts& o, SparseBwdLayout& S) {
  Opts plain = o;
  plain.ds_budget = 0;
  layout_for(s, JFA_MODE_SELF, JFA_PASS_BWD, plain, S.base);
  const size_t B = lengths.size();
  const int64_t H = s->num_heads, T = s->total_tokens;
  const bool narrow = s->head_dim == 128;
  S.tile_keys = narrow ? kSparseKBlock : kBwdKeys;
  S.programs = max_programs(o, (narrow ? kBwdKeys / kSparseKBlock : 1) * dkdv_wg_per_cu(s->head_dim));
  S.kv_seg_cap = std::max<int64_t>(S.programs, H) + 1;
  S.kv_tile_cap = H * (T / S.tile_keys + (int64_t)B + 1);
  S.bits_prefix.assign(B + 1, 0);
  for (size_t b = 0; b < B; ++b) {
    const int64_t len = lengths[b];
    const int64_t words = cdiv(len, kBwdKeys) * 2 * cdiv(cdiv(len, kSparseQBlock), 32);
    S.bits_prefix[b + 1] = S.bits_prefix[b] + words * s->num_heads;
  }
  size_t at = S.base.total;
  S.sel_base = at;
  at += align_up((B + 1) * sizeof(int64_t));
  S.sel_k = at;
  at += align_up((B + 1) * sizeof(int32_t));
  S.bits_base = at;
  at += align_up((B + 1) * sizeof(int64_t));
  S.kv_seg = at;
  at += align_up(S.kv_seg_cap * sizeof(int32_t));
  S.kv_tiles = at;
  at += align_up(S.kv_tile_cap * sizeof(Tile));
  S.bits = at;
  at += align_up((size_t)S.bits_prefix.back() * sizeof(uint32_t));
  S.total = at;
}

// Fused rotary embedding: a [rope_positions][D/2][2] fp32 cos/sin table, 16-byte
// aligned, covering every position (0 .. L-1 of each sequence).
int check_rope(const float* rope, int32_t rope_positions, const std::vector<int32_t>& lengths) {
  if (!aligned(rope, 16)) return fail(JFA_ERR_MISALIGNED, "rope_cos_sin must be 16-byte aligned");
  int32_t max_len = 0;
  for (int32_t len : lengths) max_len = std::max(max_len, len);
  if (rope_positions < max_len)
    return fail(JFA_ERR_BAD_SHAPE, "rope_positions %d < longest sequence %d", rope_positions, max_len);
  return JFA_OK;
}

// MXFP8: padded start of each sequence in the transposed V codes.
std::vector<int64_t> mx_vbase(const std::vector<int32_t>& lengths) {
  std::vector<int64_t> vb(lengths.size() + 1, 0);
  for (size_t b = 0; b < lengths.size(); ++b) vb[b + 1] = vb[b] + cdiv(lengths[b], kMxVPad) * kMxVPad;
  return vb;
}

// Workspace of jfa_bwd_mxfp8: the decoded q, k, v (bf16 [T, H, D] each), the V layout
// tables (padded start of each sequence, sequence of each padded 64-key group), then the
// self-attention backward's own workspace.
struct MxBwdLayout {
  size_t q = 0, k = 0, v = 0, vbase = 0, groups = 0, bwd = 0, total = 0;
};

void mx_bwd_layout(const jfa_shape* s, const Opts& o, MxBwdLayout& M) {
  const int64_t B = s->num_seqs, T = s->total_tokens, H = s->num_heads, D = s->head_dim;
  const size_t tensor = align_up((size_t)(T * H * D) * 2);
  size_t at = 0;
  M.q = at;
  at += tensor;
  M.k = at;
  at += tensor;
  M.v = at;
  at += tensor;
  M.vbase = at;
  at += align_up((B + 1) * sizeof(int64_t));
  M.groups = at;  // sum_b ceil(L_b / 64) <= T / 64 + B padded groups
  at += align_up((T / kMxVPad + B + 1) * sizeof(int32_t));
  Layout L;
  layout_for(s, JFA_MODE_SELF, JFA_PASS_BWD, o, L);
  M.bwd = at;
  M.total = at + L.total;
}

int check_mx_shape(const jfa_shape* shape) {
  int rc = check_shape(shape, JFA_MODE_SELF);
  if (rc) return rc;
  if (kv_heads(shape) != shape->num_heads)
    return fail(JFA_ERR_BAD_SHAPE, "the MXFP8 path needs one query head per key/value head");
  return JFA_OK;
}

// Debug tile-visit counting (see jfa_debug_tile_visits in jfa.h).  Regions of the
// caller's count array per kernel role (forward, dK/dV or fused backward, dQ) and the
// tile-list lengths of the last call.
constexpr int kVisitRoles = 3;
struct VisitDebug {
  std::mutex mu;
  int32_t* counts = nullptr;
  int64_t stride = 0;
  int64_t last[kVisitRoles] = {0, 0, 0};
} g_visits;

void visits_begin() {
  std::lock_guard<std::mutex> lock(g_visits.mu);
  for (int64_t& n : g_visits.last) n = 0;
}

// Records that `kernel` walks a list of n tiles in this call and returns its count
// region (null when counting is off); a list longer than the region fails the call
// before any device work.
int visit_region(int kernel, int64_t n, int32_t** out) {
  std::lock_guard<std::mutex> lock(g_visits.mu);
  *out = nullptr;
  g_visits.last[kernel] = n;
  if (!g_visits.counts) return JFA_OK;
  if (n > g_visits.stride)
    return fail(JFA_ERR_CAPACITY, "tile-visit counts: %lld tiles > stride %lld", (long long)n,
                (long long)g_visits.stride);
  *out = g_visits.counts + kernel * g_visits.stride;
  return JFA_OK;
}

int launch_status(hipError_t e, const char* what) {
  return e == hipSuccess ? JFA_OK : hip_fail(e, what);
}

// Kernel timing hook (see jfa_kernel_timing in jfa.h).
struct KernelTimer {
  std::mutex mu;
  bool enabled = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> ev[6];
  void forget_locked() {
    for (auto& v : ev) {
      for (auto& pr : v) {
        (void)hipEventDestroy(pr.first);
        (void)hipEventDestroy(pr.second);
      }
      v.clear();
    }
  }
} g_timer;

// Launch `fn` (returning hipError_t) between two recorded events when timing is on.
template <class F>
hipError_t timed_launch(int pass, hipStream_t s, F fn) {
  hipEvent_t a = nullptr, b = nullptr;
  bool on;
  {
    std::lock_guard<std::mutex> lock(g_timer.mu);
    on = g_timer.enabled;
  }
  if (on) {
    hipError_t e = hipEventCreate(&a);
    if (e == hipSuccess) e = hipEventCreate(&b);
    if (e == hipSuccess) e = hipEventRecord(a, s);
    if (e != hipSuccess) return e;
  }
  hipError_t e = fn();
  if (on) {
    if (e == hipSuccess) e = hipEventRecord(b, s);
    std::lock_guard<std::mutex> lock(g_timer.mu);
    g_timer.ev[pass].push_back({a, b});
  }
  return e;
}

}  // namespace

extern "C" {

int jfa_version(void) { return JFA_VERSION; }

int jfa_last_bwd_path(void) { return g_bwd_path; }

int jfa_kernel_timing(int enable) {
  g_detail.clear();
  std::lock_guard<std::mutex> lock(g_timer.mu);
  g_timer.forget_locked();
  g_timer.enabled = enable != 0;
  return JFA_OK;
}

int jfa_kernel_times(int pass, int64_t* launches, double* total_ms, int reset) {
  g_detail.clear();
  if (pass != JFA_KERNEL_FWD && pass != JFA_KERNEL_BWD && pass != JFA_KERNEL_BWD_DQ && pass != JFA_KERNEL_BWD_PREP &&
      pass != JFA_KERNEL_SPARSE_SELECT && pass != JFA_KERNEL_MX_QUANT)
    return fail(JFA_ERR_BAD_MODE, "kernel must be a jfa_kernel");
  if (!launches || !total_ms) return fail(JFA_ERR_NULL_POINTER, "launches and total_ms must be non-NULL");
  std::lock_guard<std::mutex> lock(g_timer.mu);
  double sum = 0.0;
  for (auto& pr : g_timer.ev[pass]) {
    hipError_t e = hipEventSynchronize(pr.second);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, pr.first, pr.second);
    if (e != hipSuccess) return hip_fail(e, "reading kernel timing events");
    sum += ms;
  }
  *launches = (int64_t)g_timer.ev[pass].size();
  *total_ms = sum;
  if (reset) {
    for (auto& pr : g_timer.ev[pass]) {
      (void)hipEventDestroy(pr.first);
      (void)hipEventDestroy(pr.second);
    }
    g_timer.ev[pass].clear();
  }
  return JFA_OK;
}

int jfa_debug_tile_visits(int32_t* counts, int64_t stride) {
  g_detail.clear();
  if (counts && stride < 1) return fail(JFA_ERR_BAD_OPTION, "stride must be >= 1");
  if (counts && !aligned(counts, 4)) return fail(JFA_ERR_MISALIGNED, "counts must be 4-byte aligned");
  std::lock_guard<std::mutex> lock(g_visits.mu);
  g_visits.counts = counts;
  g_visits.stride = counts ? stride : 0;
  return JFA_OK;
}

int jfa_debug_tile_list_size(int kernel, int64_t* tiles) {
  g_detail.clear();
  if (kernel < 0 || kernel >= kVisitRoles) return fail(JFA_ERR_BAD_MODE, "kernel must be 0, 1 or 2");
  if (!tiles) return fail(JFA_ERR_NULL_POINTER, "tiles is NULL");
  std::lock_guard<std::mutex> lock(g_visits.mu);
  *tiles = g_visits.last[kernel];
  return JFA_OK;
}

const char* jfa_last_error_detail(void) { return g_detail.c_str(); }

const char* jfa_error_string(int code) {
  switch (code) {
    case JFA_OK: return "success";
    case JFA_ERR_NULL_POINTER: return "a required pointer argument is NULL";
    case JFA_ERR_BAD_SHAPE: return "invalid problem shape";
    case JFA_ERR_BAD_HEAD_DIM: return "head_dim must be 64 or 128";
    case JFA_ERR_BAD_MODE: return "invalid mode or pass";
    case JFA_ERR_BAD_OFFSETS: return "invalid offsets (offsets[0] != 0, decreasing, or offsets[B] != T)";
    case JFA_ERR_MISALIGNED: return "a tensor or the workspace is misaligned";
    case JFA_ERR_WORKSPACE: return "workspace too small";
    case JFA_ERR_BAD_OPTION: return "invalid option";
    case JFA_ERR_TOO_LARGE: return "problem exceeds the 32-bit tile indexing";
    case JFA_ERR_HIP: return "HIP runtime error";
    case JFA_ERR_CAPACITY: return "output array too small";
    default: return "unknown status code";
  }
}

int jfa_workspace_size(const jfa_shape* shape, int mode, int pass, const jfa_opts* opts, size_t* bytes) {
  g_detail.clear();
  int rc = check_shape(shape, mode);
  if (rc) return rc;
  if (pass != JFA_PASS_FWD && pass != JFA_PASS_BWD && pass != JFA_PASS_FWD_SPARSE && pass != JFA_PASS_FWD_MXFP8 &&
      pass != JFA_PASS_BWD_MXFP8)
    return fail(JFA_ERR_BAD_MODE, "pass must be a jfa_pass");
  if ((pass == JFA_PASS_FWD_SPARSE || pass == JFA_PASS_FWD_MXFP8 || pass == JFA_PASS_BWD_MXFP8) &&
      mode != JFA_MODE_SELF)
    return fail(JFA_ERR_BAD_MODE, "the block-sparse and MXFP8 variants are self mode only");
  if (!bytes) return fail(JFA_ERR_NULL_POINTER, "bytes is NULL");
  Opts o;
  if ((rc = check_opts(opts, o))) return rc;
  if (pass == JFA_PASS_BWD_MXFP8) {
    if ((rc = check_mx_shape(shape))) return rc;
    MxBwdLayout M;
    mx_bwd_layout(shape, o, M);
    *bytes = M.total;
    return JFA_OK;
  }
  Layout L;
  layout_for(shape, mode, pass, o, L);
  *bytes = L.total;
  return JFA_OK;
}

int jfa_ds_bytes(const jfa_shape* shape, const int32_t* offsets_host, size_t* bytes) {
  g_detail.clear();
  int rc = check_shape(shape, JFA_MODE_SELF);
  if (rc) return rc;
  if (!offsets_host || !bytes) return fail(JFA_ERR_NULL_POINTER, "offsets_host and bytes must be non-NULL");
  std::vector<int32_t> lengths;
  if ((rc = intake_offsets(shape, nullptr, offsets_host, nullptr, lengths))) return rc;
  int64_t blocks = 0;
  for (int32_t len : lengths) blocks += ds_blocks(len);
  *bytes = (size_t)blocks * shape->num_heads * kDsBlockBytes;
  return JFA_OK;
}

int jfa_block_sparse_entries(const jfa_shape* shape, const int32_t* offsets_host, float ratio, int64_t* entries) {
  g_detail.clear();
  int rc = check_shape(shape, JFA_MODE_SELF);
  if (rc) return rc;
  if (!offsets_host || !entries) return fail(JFA_ERR_NULL_POINTER, "offsets_host and entries must be non-NULL");
  std::vector<int32_t> lengths;
  if ((rc = intake_offsets(shape, nullptr, offsets_host, nullptr, lengths))) return rc;
  SparsePlan P;
  if ((rc = sparse_plan(shape, lengths, ratio, P))) return rc;
  *entries = P.sel_base.back();
  return JFA_OK;
}

int jfa_fwd_block_sparse(const jfa_shape* shape, float scale, float ratio, const void* q, const void* k, const void* v,
                         const int32_t* offsets_dev, const int32_t* offsets_host, void* o, float* lse,
                         int32_t* selection, int64_t selection_entries, void* workspace, size_t workspace_bytes,
                         const jfa_opts* opts, void* stream_) {
  g_detail.clear();
  visits_begin();
  hipStream_t stream = (hipStream_t)stream_;
  int rc = check_shape(shape, JFA_MODE_SELF);
  if (rc) return rc;
  Opts op;
  if ((rc = check_opts(opts, op))) return rc;
  if (!q || !k || !v || !o || !lse || !offsets_dev || !selection || !workspace)
    return fail(JFA_ERR_NULL_POINTER, "q, k, v, o, lse, offsets_dev, selection and workspace must be non-NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4) ||
      !aligned(selection, 4))
    return fail(JFA_ERR_MISALIGNED, "q, k, v, o must be 16-byte aligned, lse and selection 4-byte aligned");
  if (!aligned(workspace, kAlign)) return fail(JFA_ERR_MISALIGNED, "workspace must be 256-byte aligned");
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(JFA_ERR_BAD_SHAPE, "scale must be positive and finite");
  Layout L;
  layout_for(shape, JFA_MODE_SELF, JFA_PASS_FWD_SPARSE, op, L);
  if (workspace_bytes < L.total)
    return fail(JFA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, L.total);
  std::vector<int32_t> lengths;
  if ((rc = intake_offsets(shape, offsets_dev, offsets_host, stream, lengths))) return rc;
  SparsePlan P;
  if ((rc = sparse_plan(shape, lengths, ratio, P))) return rc;
  if (selection_entries < P.sel_base.back())
    return fail(JFA_ERR_CAPACITY, "selection holds %lld entries, %lld needed", (long long)selection_entries,
                (long long)P.sel_base.back());
  const int H = shape->num_heads, D = shape->head_dim, Hkv = kv_heads(shape);
  const int B = shape->num_seqs;
  Schedule sc;
  schedule_fwd(lengths, H, JFA_MODE_SELF, 0, kFwdRows, max_programs(op, kFwdWgPerCu), op.sched == 1, sc);
  if (sc.tiles.empty()) return JFA_OK;
  if ((int64_t)sc.tiles.size() > L.tile_cap) return fail(JFA_ERR_WORKSPACE, "internal: tile capacity");
  int32_t* visits = nullptr;
  if ((rc = visit_region(JFA_KERNEL_FWD, (int64_t)sc.tiles.size(), &visits))) return rc;
  if (P.qt_prefix.back() > L.sp_nqt_cap || P.kb_prefix.back() > L.sp_nkb_cap)
    return fail(JFA_ERR_WORKSPACE, "internal: block capacity");
  std::vector<char> buf;
  serialise(sc, L, buf);
  buf.resize(L.sp_k + (B + 1) * sizeof(int32_t), 0);
  memcpy(buf.data() + L.sp_qt, P.qt_prefix.data(), (B + 1) * sizeof(int32_t));
  memcpy(buf.data() + L.sp_kb, P.kb_prefix.data(), (B + 1) * sizeof(int32_t));
  memcpy(buf.data() + L.sp_base, P.sel_base.data(), (B + 1) * sizeof(int64_t));
  memcpy(buf.data() + L.sp_k, P.sel_k.data(), (B + 1) * sizeof(int32_t));
  char* ws = (char*)workspace;
  if ((rc = upload(buf.data(), buf.size(), ws, stream))) return rc;

  const int32_t* qt_prefix = (const int32_t*)(ws + L.sp_qt);
  const int32_t* kb_prefix = (const int32_t*)(ws + L.sp_kb);
  float* qbar = (float*)(ws + L.sp_qbar);
  float* kbar = (float*)(ws + L.sp_kbar);
  const PoolParams pq{(const uint16_t*)q, qbar, offsets_dev, qt_prefix, B, H, kSparseQBlock, P.qt_prefix.back()};
  const PoolParams pk{(const uint16_t*)k, kbar, offsets_dev, kb_prefix, B, Hkv, kSparseKBlock, P.kb_prefix.back()};
  SelectParams ps{};
  ps.qbar = qbar;
  ps.kbar = kbar;
  ps.offsets = offsets_dev;
  ps.qt_prefix = qt_prefix;
  ps.kb_prefix = kb_prefix;
  ps.sel_base = (const int64_t*)(ws + L.sp_base);
  ps.sel_k = (const int32_t*)(ws + L.sp_k);
  ps.sel = selection;
  ps.num_seqs = B;
  ps.num_heads = H;
  ps.num_kv_heads = Hkv;
  ps.nqt = P.qt_prefix.back();
  ps.nkb = P.kb_prefix.back();
  if ((rc = launch_status(timed_launch(JFA_KERNEL_SPARSE_SELECT, stream, [&] { return launch_pool(pq, D, stream); }),
                          "query-block pooling launch")))
    return rc;
  if ((rc = launch_status(timed_launch(JFA_KERNEL_SPARSE_SELECT, stream, [&] { return launch_pool(pk, D, stream); }),
                          "key-block pooling launch")))
    return rc;
  if ((rc = launch_status(timed_launch(JFA_KERNEL_SPARSE_SELECT, stream, [&] { return launch_select(ps, D, stream); }),
                          "block selection launch")))
    return rc;

  FwdParams p{};
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.o = (uint16_t*)o;
  p.lse = lse;
  p.offsets = offsets_dev;
  p.tiles = (const Tile*)(ws + L.tiles);
  p.seg_ptr = (const int32_t*)(ws + L.seg);
  p.counters = (int32_t*)(ws + L.counters);
  p.num_seqs = B;
  p.num_heads = H;
  p.num_kv_heads = Hkv;
  p.num_q = 0;
  p.num_programs = sc.programs;
  p.total_tokens = shape->total_tokens;
  p.dynamic = op.sched;
  p.scale_log2 = scale * kLog2eHost;
  p.sel = selection;
  p.sel_base = ps.sel_base;
  p.sel_k = ps.sel_k;
  p.visits = visits;
  return launch_status(timed_launch(JFA_KERNEL_FWD, stream, [&] { return launch_fwd(p, kSelfSparse, D, stream); }),
                       "block-sparse forward launch");
}

int jfa_bwd_block_sparse_workspace_size(const jfa_shape* shape, const int32_t* offsets_host, const jfa_opts* opts,
                                        size_t* bytes) {
  g_detail.clear();
  int rc = check_shape(shape, JFA_MODE_SELF);
  if (rc) return rc;
  if (!offsets_host || !bytes) return fail(JFA_ERR_NULL_POINTER, "offsets_host and bytes must be non-NULL");
  Opts op;
  if ((rc = check_opts(opts, op))) return rc;
  std::vector<int32_t> lengths;
  if ((rc = intake_offsets(shape, nullptr, offsets_host, nullptr, lengths))) return rc;
  SparseBwdLayout S;
  sparse_bwd_layout(shape, lengths, op, S);
  *bytes = S.total;
  return JFA_OK;
}

int jfa_bwd_block_sparse(const jfa_shape* shape, float scale, float ratio, const void* q, const void* k,
                         const void* v, const void* o, const void* dout, const float* lse,
                         const int32_t* offsets_dev, const int32_t* offsets_host, const int32_t* selection,
                         int64_t selection_entries, void* dq, void* dk, void* dv, void* workspace,
                         size_t workspace_bytes, const jfa_opts* opts, void* stream_) {
  g_detail.clear();
  visits_begin();
  hipStream_t stream = (hipStream_t)stream_;
  int rc = check_shape(shape, JFA_MODE_SELF);
  if (rc) return rc;
  Opts op;
  if ((rc = check_opts(opts, op))) return rc;
  if (!q || !k || !v || !o || !dout || !lse || !offsets_dev || !selection || !dq || !dk || !dv || !workspace)
    return fail(JFA_ERR_NULL_POINTER, "tensor, offsets_dev, selection and workspace pointers must be non-NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dout, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(lse, 4) || !aligned(selection, 4))
    return fail(JFA_ERR_MISALIGNED, "bf16 tensors must be 16-byte aligned, lse and selection 4-byte aligned");
  if (!aligned(workspace, kAlign)) return fail(JFA_ERR_MISALIGNED, "workspace must be 256-byte aligned");
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(JFA_ERR_BAD_SHAPE, "scale must be positive and finite");
  if (kv_heads(shape) != shape->num_heads)
    return fail(JFA_ERR_BAD_SHAPE, "the backward needs one query head per key/value head (num_kv_heads %d != num_heads %d)",
                shape->num_kv_heads, shape->num_heads);
  std::vector<int32_t> lengths;
  if ((rc = intake_offsets(shape, offsets_dev, offsets_host, stream, lengths))) return rc;
  SparsePlan P;
  if ((rc = sparse_plan(shape, lengths, ratio, P))) return rc;
  if (selection_entries < P.sel_base.back())
    return fail(JFA_ERR_CAPACITY, "selection holds %lld entries, %lld needed", (long long)selection_entries,
                (long long)P.sel_base.back());
  SparseBwdLayout S;
  sparse_bwd_layout(shape, lengths, op, S);
  if (workspace_bytes < S.total)
    return fail(JFA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, S.total);
  const Layout& L = S.base;
  const int H = shape->num_heads, D = shape->head_dim, B = shape->num_seqs;
  Schedule sc, sq;
  schedule_bwd(lengths, H, JFA_MODE_SELF, S.tile_keys, S.programs, op.sched == 1, sc);
  if (sc.tiles.empty()) return JFA_OK;
  schedule_fwd(lengths, H, JFA_MODE_SELF, 0, kDqRows, max_programs(op, kDqWgPerCu), op.sched == 1, sq);
  if ((int64_t)sc.tiles.size() > S.kv_tile_cap || (int64_t)sc.seg_ptr.size() > S.kv_seg_cap ||
      (int64_t)sq.tiles.size() > L.tile2_cap || (int64_t)sq.seg_ptr.size() > L.seg2_cap)
    return fail(JFA_ERR_WORKSPACE, "internal: tile capacity");
  int32_t *visits = nullptr, *dq_visits = nullptr;
  if ((rc = visit_region(JFA_KERNEL_BWD, (int64_t)sc.tiles.size(), &visits))) return rc;
  if ((rc = visit_region(JFA_KERNEL_BWD_DQ, (int64_t)sq.tiles.size(), &dq_visits))) return rc;
  char* ws = (char*)workspace;
  {
    // [counters (zero) .. dQ schedule]
    std::vector<char> buf(L.tiles2 + sq.tiles.size() * sizeof(Tile), 0);
    put_schedule(sq, L.seg2, L.tiles2, buf);
    if ((rc = upload(buf.data(), buf.size(), ws, stream))) return rc;
  }
  {
    // [sel_base | sel_k | bits_base | dK/dV schedule]
    std::vector<char> arr(S.kv_tiles + sc.tiles.size() * sizeof(Tile) - S.sel_base, 0);
    memcpy(arr.data(), P.sel_base.data(), (B + 1) * sizeof(int64_t));
    memcpy(arr.data() + (S.sel_k - S.sel_base), P.sel_k.data(), (B + 1) * sizeof(int32_t));
    memcpy(arr.data() + (S.bits_base - S.sel_base), S.bits_prefix.data(), (B + 1) * sizeof(int64_t));
    put_schedule(sc, S.kv_seg - S.sel_base, S.kv_tiles - S.sel_base, arr);
    if ((rc = upload(arr.data(), arr.size(), ws + S.sel_base, stream))) return rc;
  }
  uint32_t* bits = (uint32_t*)(ws + S.bits);
  if ((rc = launch_status(launch_fill_zero((float*)bits, S.bits_prefix.back(), stream), "bitmap fill"))) return rc;
  MarkParams mp{};
  mp.sel = selection;
  mp.sel_base = (const int64_t*)(ws + S.sel_base);
  mp.sel_k = (const int32_t*)(ws + S.sel_k);
  mp.offsets = offsets_dev;
  mp.bits_base = (const int64_t*)(ws + S.bits_base);
  mp.bits = bits;
  mp.num_seqs = B;
  mp.num_heads = H;
  mp.entries = P.sel_base.back();
  if ((rc = launch_status(timed_launch(JFA_KERNEL_BWD_PREP, stream, [&] { return launch_mark(mp, stream); }),
                          "block-sparse mark launch")))
    return rc;

  BwdParams p{};
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.o = (const uint16_t*)o;
  p.dout = (const uint16_t*)dout;
  p.lse = lse;
  p.offsets = offsets_dev;
  p.tiles = (const Tile*)(ws + S.kv_tiles);
  p.seg_ptr = (const int32_t*)(ws + S.kv_seg);
  p.counters = (int32_t*)(ws + L.counters);
  p.dk = (uint16_t*)dk;
  p.dv = (uint16_t*)dv;
  p.dq = (uint16_t*)dq;
  p.row_aug = (uint16_t*)(ws + L.stats);
  p.sparse_narrow = S.tile_keys == kSparseKBlock ? 1 : 0;
  p.dq_tiles = (const Tile*)(ws + L.tiles2);
  p.dq_seg_ptr = (const int32_t*)(ws + L.seg2);
  p.dq_programs = sq.programs;
  p.sel = selection;
  p.sel_base = mp.sel_base;
  p.sel_k = mp.sel_k;
  p.sp_bits = bits;
  p.sp_bits_base = mp.bits_base;
  p.visits = visits;
  p.dq_visits = dq_visits;
  p.num_seqs = B;
  p.num_heads = H;
  p.num_programs = sc.programs;
  p.total_tokens = shape->total_tokens;
  p.dynamic = op.sched;
  p.scale = scale;
  p.scale_log2 = scale * kLog2eHost;
  if ((rc = launch_status(timed_launch(JFA_KERNEL_BWD_DQ, stream, [&] { return launch_bwd_self_dq(p, D, stream); }),
                          "block-sparse dQ launch")))
    return rc;
  return launch_status(timed_launch(JFA_PASS_BWD, stream, [&] { return launch_bwd_self_dkdv(p, D, stream); }),
                       "block-sparse dK/dV launch");
}

int jfa_rope_table(float* table, int32_t positions, int32_t head_dim, float base, void* stream) {
  g_detail.clear();
  if (!table) return fail(JFA_ERR_NULL_POINTER, "table is NULL");
  if (!aligned(table, 16)) return fail(JFA_ERR_MISALIGNED, "table must be 16-byte aligned");
  if (head_dim != 64 && head_dim != 128) return fail(JFA_ERR_BAD_HEAD_DIM, "head_dim %d not in {64, 128}", head_dim);
  if (positions < 0) return fail(JFA_ERR_BAD_SHAPE, "positions < 0");
  if (!(base > 1.f) || !std::isfinite(base)) return fail(JFA_ERR_BAD_OPTION, "base must be finite and > 1");
  return launch_status(launch_rope_table(table, positions, head_dim, (double)base, (hipStream_t)stream),
                       "rotary table launch");
}

int jfa_mxfp8_v_tokens(const jfa_shape* shape, const int32_t* offsets_host, int64_t* tokens) {
  g_detail.clear();
  int rc = check_mx_shape(shape);
  if (rc) return rc;
  if (!offsets_host || !tokens) return fail(JFA_ERR_NULL_POINTER, "offsets_host and tokens must be non-NULL");
  std::vector<int32_t> lengths;
  if ((rc = intake_offsets(shape, nullptr, offsets_host, nullptr, lengths))) return rc;
  *tokens = mx_vbase(lengths).back();
  return JFA_OK;
}

int jfa_mxfp8_quantize_qk(const jfa_shape* shape, const void* x, uint8_t* codes, uint8_t* scales, void* stream) {
  g_detail.clear();
  int rc = check_mx_shape(shape);
  if (rc) return rc;
  if (!x || !codes || !scales) return fail(JFA_ERR_NULL_POINTER, "x, codes and scales must be non-NULL");
  if (!aligned(x, 16) || !aligned(codes, 16))
    return fail(JFA_ERR_MISALIGNED, "x and codes must be 16-byte aligned");
  MxQuantParams p{};
  p.x = (const uint16_t*)x;
  p.codes = codes;
  p.scales = scales;
  p.rows = shape->total_tokens * shape->num_heads;
  p.num_heads = shape->num_heads;
  p.head_dim = shape->head_dim;
  hipStream_t s = (hipStream_t)stream;
  return launch_status(timed_launch(JFA_KERNEL_MX_QUANT, s, [&] { return launch_mx_quant_qk(p, s); }),
                       "MXFP8 quantisation launch");
}

int jfa_mxfp8_quantize_v(const jfa_shape* shape, const void* v, const int32_t* offsets_dev,
                         const int32_t* offsets_host, uint8_t* codes, uint8_t* scales, int64_t tokens,
                         void* workspace, size_t workspace_bytes, void* stream_) {
  g_detail.clear();
  hipStream_t stream = (hipStream_t)stream_;
  int rc = check_mx_shape(shape);
  if (rc) return rc;
  if (!v || !offsets_dev || !codes || !scales || !workspace)
    return fail(JFA_ERR_NULL_POINTER, "v, offsets_dev, codes, scales and workspace must be non-NULL");
  if (!aligned(v, 2) || !aligned(codes, 16) || !aligned(scales, 2) || !aligned(workspace, kAlign))
    return fail(JFA_ERR_MISALIGNED, "codes must be 16-byte aligned, scales 2-byte, workspace 256-byte");
  Layout L;
  layout_for(shape, JFA_MODE_SELF, JFA_PASS_FWD_MXFP8, Opts(), L);
  if (workspace_bytes < L.total)
    return fail(JFA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, L.total);
  std::vector<int32_t> lengths;
  if ((rc = intake_offsets(shape, offsets_dev, offsets_host, stream, lengths))) return rc;
  const std::vector<int64_t> vb = mx_vbase(lengths);
  if (tokens != vb.back())
    return fail(JFA_ERR_BAD_SHAPE, "tokens %lld differs from jfa_mxfp8_v_tokens() = %lld", (long long)tokens,
                (long long)vb.back());
  if (vb.back() == 0) return JFA_OK;
  char* ws = (char*)workspace;
  std::vector<char> buf(L.prefix - L.ds_base + (size_t)(vb.back() / kMxVPad) * sizeof(int32_t), 0);
  memcpy(buf.data(), vb.data(), vb.size() * sizeof(int64_t));
  int32_t* gs = reinterpret_cast<int32_t*>(buf.data() + (L.prefix - L.ds_base));
  for (size_t b = 0; b < lengths.size(); ++b)
    for (int64_t g = vb[b] / kMxVPad; g < vb[b + 1] / kMxVPad; ++g) gs[g] = (int32_t)b;
  if ((rc = upload(buf.data(), buf.size(), ws + L.ds_base, stream))) return rc;
  MxQuantParams p{};
  p.x = (const uint16_t*)v;
  p.codes = codes;
  p.scales = scales;
  p.num_heads = shape->num_heads;
  p.head_dim = shape->head_dim;
  p.num_seqs = shape->num_seqs;
  p.offsets = offsets_dev;
  p.vbase = (const int64_t*)(ws + L.ds_base);
  p.group_seq = (const int32_t*)(ws + L.prefix);
  p.tp = vb.back();
  return launch_status(timed_launch(JFA_KERNEL_MX_QUANT, stream, [&] { return launch_mx_quant_v(p, stream); }),
                       "MXFP8 V quantisation launch");
}

int jfa_fwd_mxfp8(const jfa_shape* shape, float scale, const uint8_t* q8, const uint8_t* q_scales,
                  const uint8_t* k8, const uint8_t* k_scales, const uint8_t* v8t, const uint8_t* v_scales,
                  int64_t v_tokens, const int32_t* offsets_dev, const int32_t* offsets_host, void* o, float* lse,
                  void* workspace, size_t workspace_bytes, const jfa_opts* opts, void* stream_) {
  g_detail.clear();
  visits_begin();
  hipStream_t stream = (hipStream_t)stream_;
  int rc = check_mx_shape(shape);
  if (rc) return rc;
  Opts op;
  if ((rc = check_opts(opts, op))) return rc;
  if (!q8 || !q_scales || !k8 || !k_scales || !v8t || !v_scales || !offsets_dev || !o || !lse || !workspace)
    return fail(JFA_ERR_NULL_POINTER, "codes, scales, offsets_dev, o, lse and workspace must be non-NULL");
  if (!aligned(q8, 16) || !aligned(k8, 16) || !aligned(v8t, 16) || !aligned(k_scales, 4) || !aligned(v_scales, 2) ||
      !aligned(o, 16) || !aligned(lse, 4) || !aligned(workspace, kAlign))
    return fail(JFA_ERR_MISALIGNED, "codes and o 16-byte aligned, k_scales 4, v_scales 2, lse 4, workspace 256");
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(JFA_ERR_BAD_SHAPE, "scale must be positive and finite");
  Layout L;
  layout_for(shape, JFA_MODE_SELF, JFA_PASS_FWD_MXFP8, op, L);
  if (workspace_bytes < L.total)
    return fail(JFA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, L.total);
  std::vector<int32_t> lengths;
  if ((rc = intake_offsets(shape, offsets_dev, offsets_host, stream, lengths))) return rc;
  const std::vector<int64_t> vb = mx_vbase(lengths);
  if (v_tokens != vb.back())
    return fail(JFA_ERR_BAD_SHAPE, "v_tokens %lld differs from jfa_mxfp8_v_tokens() = %lld", (long long)v_tokens,
                (long long)vb.back());
  const int H = shape->num_heads, D = shape->head_dim;
  Schedule sc;
  schedule_fwd(lengths, H, JFA_MODE_SELF, 0, mx_rows(D), max_programs(op, mx_wg_per_cu(D)), false, sc);
  if (sc.tiles.empty()) return JFA_OK;
  if ((int64_t)sc.tiles.size() > L.tile_cap || (int64_t)sc.seg_ptr.size() > L.seg_cap)
    return fail(JFA_ERR_WORKSPACE, "internal: tile capacity");
  int32_t* visits = nullptr;
  if ((rc = visit_region(JFA_KERNEL_FWD, (int64_t)sc.tiles.size(), &visits))) return rc;
  std::vector<char> buf;
  serialise(sc, L, buf, nullptr, &vb);
  char* ws = (char*)workspace;
  if ((rc = upload(buf.data(), buf.size(), ws, stream))) return rc;
  MxParams p{};
  p.q8 = q8;
  p.qsc = q_scales;
  p.k8 = k8;
  p.ksc = k_scales;
  p.v8t = v8t;
  p.vsc = v_scales;
  p.vbase = (const int64_t*)(ws + L.ds_base);
  p.tp = vb.back();
  p.o = (uint16_t*)o;
  p.lse = lse;
  p.offsets = offsets_dev;
  p.tiles = (const Tile*)(ws + L.tiles);
  p.seg_ptr = (const int32_t*)(ws + L.seg);
  p.num_heads = H;
  p.num_programs = sc.programs;
  p.total_tokens = shape->total_tokens;
  p.scale_log2 = scale * kLog2eHost;
  p.visits = visits;
  return launch_status(timed_launch(JFA_KERNEL_FWD, stream, [&] { return launch_mx_fwd(p, D, stream); }),
                       "MXFP8 forward launch");
}

int jfa_schedule(const jfa_shape* shape, int mode, int pass, const int32_t* offsets_host,
                 const jfa_opts* opts, int32_t* tiles, int64_t cap, int32_t* seg_ptr, int64_t seg_cap,
                 int64_t* n_tiles, int32_t* n_segs, int32_t* n_programs, int32_t* tile_rows) {
  g_detail.clear();
  int rc = check_shape(shape, mode);
  if (rc) return rc;
  if (pass != JFA_PASS_FWD && pass != JFA_PASS_BWD) return fail(JFA_ERR_BAD_MODE, "pass must be 0 or 1");
  if (!offsets_host) return fail(JFA_ERR_NULL_POINTER, "jfa_schedule needs host offsets");
  Opts o;
  if ((rc = check_opts(opts, o))) return rc;
  std::vector<int32_t> lengths;
  if ((rc = intake_offsets(shape, nullptr, offsets_host, nullptr, lengths))) return rc;
  Schedule sc;
  const bool dyn = o.sched == 1;
  if (mode == JFA_MODE_BLOCK_DIAG)
    schedule_blockdiag(lengths, shape->num_heads, kBlock, max_programs(o, kBdWgPerCu), kBdWaves, sc);
  else if (pass == JFA_PASS_FWD && mode == JFA_MODE_BROADCAST_Q) {
    KeyChunks kc;
    bq_key_chunks(lengths, shape->num_heads, shape->num_q, kFwdRows, max_programs(o, kFwdWgPerCu), true, kc);
    schedule_fwd(kc.len, shape->num_heads, mode, shape->num_q, kFwdRows, max_programs(o, kFwdWgPerCu), dyn, sc);
  } else if (pass == JFA_PASS_FWD) {
    SelfSplit split;
    const int P = max_programs(o, kFwdWgPerCu);
    if (!(mode == JFA_MODE_SELF && self_split_plan(lengths, shape->num_heads, P, dyn, sc, split)))
      schedule_fwd(lengths, shape->num_heads, mode, shape->num_q, kFwdRows, P, dyn, sc);
  }
  else
    schedule_bwd(lengths, shape->num_heads, mode, kBwdKeys,
                 max_programs(o, bwd_wg_per_cu(mode, o.dq_path, shape->head_dim)), dyn, sc);
  if (n_tiles) *n_tiles = (int64_t)sc.tiles.size();
  if (n_segs) *n_segs = (int32_t)sc.seg_ptr.size();
  if (n_programs) *n_programs = sc.programs;
  if (tile_rows) *tile_rows = sc.tile_rows;
  if (tiles) {
    if (cap < (int64_t)sc.tiles.size()) return fail(JFA_ERR_CAPACITY, "tiles capacity %lld < %zu", (long long)cap, sc.tiles.size());
    for (size_t i = 0; i < sc.tiles.size(); ++i) {
      tiles[3 * i] = sc.tiles[i].b;
      tiles[3 * i + 1] = sc.tiles[i].h;
      tiles[3 * i + 2] = sc.tiles[i].blk;
    }
  }
  if (seg_ptr) {
    if (seg_cap < (int64_t)sc.seg_ptr.size()) return fail(JFA_ERR_CAPACITY, "seg_ptr capacity too small");
    memcpy(seg_ptr, sc.seg_ptr.data(), sc.seg_ptr.size() * sizeof(int32_t));
  }
  return JFA_OK;
}

// jfa_fwd, jfa_fwd_rotary with rope non-null (block-diagonal mode only), and
// jfa_fwd_noalloc (noalloc: the workspace is this device's file-scope scratch array,
// the schedule goes up by a pageable copy, and the timing hook is not used, so that
// nothing is allocated).
static int fwd_entry(const jfa_shape* shape, int mode, float scale, const void* q, const void* k, const void* v,
                     const float* rope, int32_t rope_positions, const int32_t* offsets_dev,
                     const int32_t* offsets_host, void* o, float* lse, void* workspace, size_t workspace_bytes,
                     const jfa_opts* opts, void* stream_, bool noalloc = false) {
  g_detail.clear();
  visits_begin();
  hipStream_t stream = (hipStream_t)stream_;
  int rc = check_shape(shape, mode);
  if (rc) return rc;
  if (rope && mode != JFA_MODE_BLOCK_DIAG)
    return fail(JFA_ERR_BAD_MODE, "the fused rotary embedding is built for the block-diagonal mode only");
  Opts op;
  if ((rc = check_opts(opts, op))) return rc;
  Layout L;
  layout_for(shape, mode, JFA_PASS_FWD, op, L, /*key_split=*/!noalloc);
  if (noalloc && L.total > kNoAllocScratchBytes)
    return fail(JFA_ERR_TOO_LARGE, "jfa_fwd_noalloc: this shape needs %zu bytes of scratch, more than its %zu",
                L.total, kNoAllocScratchBytes);
  if (!q || !k || !v || !o || !lse || !offsets_dev || (!noalloc && !workspace))
    return fail(JFA_ERR_NULL_POINTER, "q, k, v, o, lse, offsets_dev and workspace must be non-NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return fail(JFA_ERR_MISALIGNED, "q, k, v, o must be 16-byte aligned and lse 4-byte aligned");
  if (!noalloc && !aligned(workspace, kAlign)) return fail(JFA_ERR_MISALIGNED, "workspace must be 256-byte aligned");
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(JFA_ERR_BAD_SHAPE, "scale must be positive and finite");
  if (!noalloc && workspace_bytes < L.total)
    return fail(JFA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, L.total);
  std::vector<int32_t> lengths;
  if ((rc = intake_offsets(shape, offsets_dev, offsets_host, stream, lengths))) return rc;
  if (rope && (rc = check_rope(rope, rope_positions, lengths))) return rc;
  if (noalloc) {
    hipError_t e = noalloc_scratch(&workspace);
    if (e != hipSuccess) return hip_fail(e, "looking up the device scratch array");
  }
  char* ws = (char*)workspace;
  const int H = shape->num_heads, D = shape->head_dim;
  auto put = [&](const void* src, size_t bytes, void* dst) {
    return noalloc ? upload_pageable(src, bytes, dst, stream) : upload(src, bytes, dst, stream);
  };
  auto launch = [&](int kernel, auto fn) { return noalloc ? fn() : timed_launch(kernel, stream, fn); };

  if (mode == JFA_MODE_BLOCK_DIAG) {
    std::vector<int32_t> prefix(shape->num_seqs + 1, 0);
    for (int b = 0; b < shape->num_seqs; ++b) prefix[b + 1] = prefix[b] + (int32_t)cdiv(lengths[b], kBlock);
    const int64_t ntiles = (int64_t)prefix.back() * H;
    if (ntiles == 0) return JFA_OK;
    int32_t* visits = nullptr;
    if ((rc = visit_region(JFA_KERNEL_FWD, ntiles, &visits))) return rc;
    if ((rc = put(prefix.data(), prefix.size() * sizeof(int32_t), ws + L.prefix))) return rc;
    BdParams p{};
    p.visits = visits;
    p.q = (const uint16_t*)q;
    p.k = (const uint16_t*)k;
    p.v = (const uint16_t*)v;
    p.o = (uint16_t*)o;
    p.lse = lse;
    p.offsets = offsets_dev;
    p.blk_prefix = (const int32_t*)(ws + L.prefix);
    p.num_seqs = shape->num_seqs;
    p.num_heads = H;
    p.num_kv_heads = kv_heads(shape);
    p.total_tokens = shape->total_tokens;
    p.num_tiles = ntiles;
    p.num_programs = (int)std::min<int64_t>(max_programs(op, kBdWgPerCu), cdiv(ntiles, kBdWaves));
    p.scale = scale;
    p.scale_log2 = scale * kLog2eHost;
    p.rope = rope;
    return launch_status(launch(JFA_KERNEL_FWD, [&] { return launch_bd_fwd(p, D, stream); }),
                         "block-diagonal forward launch");
  }

  Schedule sc;
  const int P = max_programs(op, kFwdWgPerCu);
  std::vector<int32_t> table;  // key chunks and cut sequences
  int nc = 0, ncut = 0;
  int kmode = mode;           // kernel mode (kSelfChunks when self-attention keys are cut)
  int64_t merge_rows = 0;     // self-attention: query rows of the cut sequences
  SelfSplit split;
  if (mode == JFA_MODE_SELF && L.self_part_cap > 0 && self_split_plan(lengths, H, P, op.sched == 1, sc, split)) {
    if (split.nc > L.chunk_cap || split.part_rows * H > L.self_part_cap)
      return fail(JFA_ERR_WORKSPACE, "internal: key chunk capacity");
    kmode = kSelfChunks;
    nc = split.nc;
    ncut = split.ncut;
    merge_rows = split.cut_rows;
    table.swap(split.table);
  } else if (mode == JFA_MODE_BROADCAST_Q) {
    KeyChunks kc;
    bq_key_chunks(lengths, H, shape->num_q, kFwdRows, P, true, kc);
    nc = (int)kc.b.size();
    // partial-result slots for the chunks of cut sequences, consecutive per sequence
    std::vector<int32_t> slot(nc, -1), cuts;
    int nslot = 0;
    for (int c = 0; c < nc;) {
      int e = c + 1;
      while (e < nc && kc.b[e] == kc.b[c]) ++e;
      if (e - c > 1) {
        cuts.insert(cuts.end(), {kc.b[c], nslot, e - c});
        for (int i = c; i < e; ++i) slot[i] = nslot++;
      }
      c = e;
    }
    ncut = (int)cuts.size() / 3;
    if (nc > L.chunk_cap || nslot > L.fwd_slot_cap) return fail(JFA_ERR_WORKSPACE, "internal: chunk capacity");
    table = kc.b;
    table.insert(table.end(), kc.k0.begin(), kc.k0.end());
    table.insert(table.end(), kc.len.begin(), kc.len.end());
    table.insert(table.end(), slot.begin(), slot.end());
    table.insert(table.end(), cuts.begin(), cuts.end());
    schedule_fwd(kc.len, H, mode, shape->num_q, kFwdRows, P, op.sched == 1, sc);
  } else {
    schedule_fwd(lengths, H, mode, shape->num_q, kFwdRows, P, op.sched == 1, sc);
  }
  if (sc.tiles.empty()) return JFA_OK;
  if ((int64_t)sc.tiles.size() > L.tile_cap) return fail(JFA_ERR_WORKSPACE, "internal: tile capacity");
  int32_t* visits = nullptr;
  if ((rc = visit_region(JFA_KERNEL_FWD, (int64_t)sc.tiles.size(), &visits))) return rc;
  std::vector<char> buf;
  serialise(sc, L, buf, nullptr, nullptr, table.empty() ? nullptr : &table);
  if ((rc = put(buf.data(), buf.size(), ws))) return rc;
  FwdParams p{};
  p.visits = visits;
  if (!table.empty()) {
    p.chunks = (const int32_t*)(ws + L.chunks);
    p.num_chunks = nc;
    p.part_o = (float*)(ws + L.part_o);
    p.part_lse = (float*)(ws + L.part_lse);
  }
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.o = (uint16_t*)o;
  p.lse = lse;
  p.offsets = offsets_dev;
  p.tiles = (const Tile*)(ws + L.tiles);
  p.seg_ptr = (const int32_t*)(ws + L.seg);
  p.counters = (int32_t*)(ws + L.counters);
  p.num_seqs = shape->num_seqs;
  p.num_heads = H;
  p.num_kv_heads = kv_heads(shape);
  p.num_q = shape->num_q;
  p.num_programs = sc.programs;
  p.total_tokens = shape->total_tokens;
  p.dynamic = op.sched;
  p.scale_log2 = scale * kLog2eHost;
  if ((rc = launch_status(launch(JFA_KERNEL_FWD, [&] { return launch_fwd(p, kmode, D, stream); }),
                          "forward launch")))
    return rc;
  if (ncut == 0) return JFA_OK;
  if (kmode == kSelfChunks)
    return launch_status(launch_self_combine(p, ncut, merge_rows, D, stream), "forward chunk merge");
  return launch_status(launch_bq_combine(p, ncut, D, stream), "forward chunk merge");
}

int jfa_fwd(const jfa_shape* shape, int mode, float scale, const void* q, const void* k, const void* v,
            const int32_t* offsets_dev, const int32_t* offsets_host, void* o, float* lse, void* workspace,
            size_t workspace_bytes, const jfa_opts* opts, void* stream) {
  return fwd_entry(shape, mode, scale, q, k, v, nullptr, 0, offsets_dev, offsets_host, o, lse, workspace,
                   workspace_bytes, opts, stream);
}

int jfa_fwd_noalloc(const jfa_shape* shape, int mode, float scale, const void* q, const void* k, const void* v,
                    const int32_t* offsets_dev, const int32_t* offsets_host, void* o, float* lse,
                    const jfa_opts* opts, void* stream) {
  return fwd_entry(shape, mode, scale, q, k, v, nullptr, 0, offsets_dev, offsets_host, o, lse, nullptr, 0, opts,
                   stream, true);
}

int jfa_fwd_rotary(const jfa_shape* shape, int mode, float scale, const void* q, const void* k, const void* v,
                   const float* rope_cos_sin, int32_t rope_positions, const int32_t* offsets_dev,
                   const int32_t* offsets_host, void* o, float* lse, void* workspace, size_t workspace_bytes,
                   const jfa_opts* opts, void* stream) {
  if (!rope_cos_sin) {
    g_detail.clear();
    return fail(JFA_ERR_NULL_POINTER, "rope_cos_sin is NULL");
  }
  return fwd_entry(shape, mode, scale, q, k, v, rope_cos_sin, rope_positions, offsets_dev, offsets_host, o, lse,
                   workspace, workspace_bytes, opts, stream);
}

// jfa_bwd, and jfa_bwd_rotary with rope non-null (block-diagonal mode only).
static int bwd_entry(const jfa_shape* shape, int mode, float scale, const void* q, const void* k, const void* v,
                     const void* o, const void* dout, const float* lse, const float* rope, int32_t rope_positions,
                     const int32_t* offsets_dev, const int32_t* offsets_host, void* dq, void* dk, void* dv,
                     void* workspace, size_t workspace_bytes, const jfa_opts* opts, void* stream_) {
  g_detail.clear();
  g_bwd_path = JFA_BWD_PATH_OTHER;
  visits_begin();
  hipStream_t stream = (hipStream_t)stream_;
  int rc = check_shape(shape, mode);
  if (rc) return rc;
  if (rope && mode != JFA_MODE_BLOCK_DIAG)
    return fail(JFA_ERR_BAD_MODE, "the fused rotary embedding is built for the block-diagonal mode only");
  Opts op;
  if ((rc = check_opts(opts, op))) return rc;
  if (!q || !k || !v || !o || !dout || !lse || !offsets_dev || !dq || !dk || !dv || !workspace)
    return fail(JFA_ERR_NULL_POINTER, "tensor, offsets_dev and workspace pointers must be non-NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dout, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(lse, 4))
    return fail(JFA_ERR_MISALIGNED, "bf16 tensors must be 16-byte aligned and lse 4-byte aligned");
  if (!aligned(workspace, kAlign)) return fail(JFA_ERR_MISALIGNED, "workspace must be 256-byte aligned");
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(JFA_ERR_BAD_SHAPE, "scale must be positive and finite");
  if (kv_heads(shape) != shape->num_heads)
    return fail(JFA_ERR_BAD_SHAPE, "the backward needs one query head per key/value head (num_kv_heads %d != num_heads %d)",
                shape->num_kv_heads, shape->num_heads);
  Layout L;
  layout_for(shape, mode, JFA_PASS_BWD, op, L);
  if (workspace_bytes < L.total)
    return fail(JFA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, L.total);
  std::vector<int32_t> lengths;
  if ((rc = intake_offsets(shape, offsets_dev, offsets_host, stream, lengths))) return rc;
  if (rope && (rc = check_rope(rope, rope_positions, lengths))) return rc;
  char* ws = (char*)workspace;
  const int H = shape->num_heads, D = shape->head_dim;
  const int64_t T = shape->total_tokens;

  if (mode == JFA_MODE_BLOCK_DIAG) {
    std::vector<int32_t> prefix(shape->num_seqs + 1, 0);
    for (int b = 0; b < shape->num_seqs; ++b) prefix[b + 1] = prefix[b] + (int32_t)cdiv(lengths[b], kBlock);
    const int64_t ntiles = (int64_t)prefix.back() * H;
    if (ntiles == 0) return JFA_OK;
    int32_t* visits = nullptr;
    if ((rc = visit_region(JFA_KERNEL_BWD, ntiles, &visits))) return rc;
    if ((rc = upload(prefix.data(), prefix.size() * sizeof(int32_t), ws + L.prefix, stream))) return rc;
    BdParams p{};
    p.visits = visits;
    p.q = (const uint16_t*)q;
    p.k = (const uint16_t*)k;
    p.v = (const uint16_t*)v;
    p.o_in = (const uint16_t*)o;
    p.dout = (const uint16_t*)dout;
    p.lse_in = lse;
    p.o = (uint16_t*)dq;
    p.dk = (uint16_t*)dk;
    p.dv = (uint16_t*)dv;
    p.offsets = offsets_dev;
    p.blk_prefix = (const int32_t*)(ws + L.prefix);
    p.num_seqs = shape->num_seqs;
    p.num_heads = H;
    p.num_kv_heads = H;
    p.total_tokens = T;
    p.num_tiles = ntiles;
    p.num_programs = (int)std::min<int64_t>(max_programs(op, kBdWgPerCu), cdiv(ntiles, kBdWaves));
    p.scale = scale;
    p.scale_log2 = scale * kLog2eHost;
    p.rope = rope;
    return launch_status(timed_launch(JFA_PASS_BWD, stream, [&] { return launch_bd_bwd(p, D, stream); }),
                         "block-diagonal backward launch");
  }

  const bool bq_split = mode == JFA_MODE_BROADCAST_Q && op.dq_path == 2;
  Schedule sc;
  schedule_bwd(lengths, H, mode, kBwdKeys, max_programs(op, bwd_wg_per_cu(mode, op.dq_path, D)), op.sched == 1, sc);
  if ((int64_t)sc.tiles.size() > L.tile_cap) return fail(JFA_ERR_WORKSPACE, "internal: tile capacity");
  BwdParams p{};
  if ((rc = visit_region(JFA_KERNEL_BWD, (int64_t)sc.tiles.size(), &p.visits))) return rc;
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.o = (const uint16_t*)o;
  p.dout = (const uint16_t*)dout;
  p.lse = lse;
  p.offsets = offsets_dev;
  p.tiles = (const Tile*)(ws + L.tiles);
  p.seg_ptr = (const int32_t*)(ws + L.seg);
  p.counters = (int32_t*)(ws + L.counters);
  p.dk = (uint16_t*)dk;
  p.dv = (uint16_t*)dv;
  p.num_seqs = shape->num_seqs;
  p.num_heads = H;
  p.num_q = shape->num_q;
  p.num_programs = sc.programs;
  p.total_tokens = T;
  p.dynamic = op.sched;
  p.scale = scale;
  p.scale_log2 = scale * kLog2eHost;

  if (mode == JFA_MODE_SELF) {
    if (sc.tiles.empty()) return JFA_OK;
    // Stored-dS path when the caller's budget holds dS of every sequence and head.
    std::vector<int64_t> ds_base(shape->num_seqs + 1, 0);
    for (int b = 0; b < shape->num_seqs; ++b) ds_base[b + 1] = ds_base[b] + ds_blocks(lengths[b]) * H;
    if (op.ds_budget > 0 && ds_base.back() * kDsBlockBytes <= op.ds_budget) {
      Schedule sq;
      schedule_fwd(lengths, H, JFA_MODE_SELF, 0, kDsRows, max_programs(op, kDsWgPerCu), op.sched == 1, sq);
      if ((int64_t)sq.tiles.size() > L.tile2_cap || sq.programs > L.programs2_cap)
        return fail(JFA_ERR_WORKSPACE, "internal: tile capacity");
      if ((rc = visit_region(JFA_KERNEL_BWD_DQ, (int64_t)sq.tiles.size(), &p.dq_visits))) return rc;
      std::vector<char> buf;
      serialise(sc, L, buf, &sq, &ds_base);
      if ((rc = upload(buf.data(), buf.size(), ws, stream))) return rc;
      p.dq = (uint16_t*)dq;
      p.row_aug = (uint16_t*)(ws + L.stats);
      p.ds = ws + L.ds;
      p.ds_base = (const int64_t*)(ws + L.ds_base);
      p.dq_tiles = (const Tile*)(ws + L.tiles2);
      p.dq_seg_ptr = (const int32_t*)(ws + L.seg2);
      p.dq_programs = sq.programs;
      g_bwd_path = JFA_BWD_PATH_STORED_DS;
      if ((rc = launch_status(
               timed_launch(JFA_KERNEL_BWD_PREP, stream, [&] { return launch_bwd_self_prep(p, D, stream); }),
               "backward row-term launch")))
        return rc;
      if ((rc = launch_status(timed_launch(JFA_PASS_BWD, stream, [&] { return launch_bwd_self_dkdv(p, D, stream); }),
                              "backward dK/dV launch")))
        return rc;
      return launch_status(
          timed_launch(JFA_KERNEL_BWD_DQ, stream, [&] { return launch_bwd_self_dq_ds(p, D, stream); }),
          "backward dQ launch");
    }
    Schedule sq;
    schedule_fwd(lengths, H, JFA_MODE_SELF, 0, kDqRows, max_programs(op, kDqWgPerCu), op.sched == 1, sq);
    if ((int64_t)sq.tiles.size() > L.tile2_cap) return fail(JFA_ERR_WORKSPACE, "internal: tile capacity");
    if ((rc = visit_region(JFA_KERNEL_BWD_DQ, (int64_t)sq.tiles.size(), &p.dq_visits))) return rc;
    std::vector<char> buf;
    serialise(sc, L, buf, &sq);
    if ((rc = upload(buf.data(), buf.size(), ws, stream))) return rc;
    p.dq = (uint16_t*)dq;
    p.row_aug = (uint16_t*)(ws + L.stats);
    p.dq_tiles = (const Tile*)(ws + L.tiles2);
    p.dq_seg_ptr = (const int32_t*)(ws + L.seg2);
    p.dq_programs = sq.programs;
    if ((int64_t)sq.programs + sc.programs > device_cus()) {
      // Each kernel fills the chip: one after the other, the dQ kernel writing the row terms.
      g_bwd_path = JFA_BWD_PATH_RECOMPUTE;
      if ((rc = launch_status(
               timed_launch(JFA_KERNEL_BWD_DQ, stream, [&] { return launch_bwd_self_dq(p, D, stream); }),
               "backward dQ launch")))
        return rc;
      return launch_status(timed_launch(JFA_PASS_BWD, stream, [&] { return launch_bwd_self_dkdv(p, D, stream); }),
                           "backward dK/dV launch");
    }
    // Few tiles (the two grids together fit the CUs, so each kernel's time is its longest
    // tile's): the row-term kernel first, then the dQ kernel on the side stream beside the
    // dK/dV kernel on the caller's; neither reads what the other writes, and the caller's
    // stream waits for both.
    p.rows_ready = 1;
    g_bwd_path = JFA_BWD_PATH_RECOMPUTE_SIDE;
    if ((rc = launch_status(
             timed_launch(JFA_KERNEL_BWD_PREP, stream, [&] { return launch_bwd_self_prep(p, D, stream); }),
             "backward row-term launch")))
      return rc;
    SideStream* ss = nullptr;
    std::unique_lock<std::mutex> lock;
    if ((rc = side_stream(&ss, lock))) return rc;
    hipError_t e = hipEventRecord(ss->fork, stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(ss->s, ss->fork, 0);
    if (e != hipSuccess) return hip_fail(e, "forking the side stream");
    if ((rc = launch_status(timed_launch(JFA_KERNEL_BWD_DQ, ss->s, [&] { return launch_bwd_self_dq(p, D, ss->s); }),
                            "backward dQ launch")))
      return rc;
    e = hipEventRecord(ss->join, ss->s);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord (join)");
    rc = launch_status(timed_launch(JFA_PASS_BWD, stream, [&] { return launch_bwd_self_dkdv(p, D, stream); }),
                       "backward dK/dV launch");
    e = hipStreamWaitEvent(stream, ss->join, 0);
    if (rc) return rc;
    if (e != hipSuccess) return hip_fail(e, "joining the side stream");
    return JFA_OK;
  }

  if (bq_split) {
    // Broadcast-Q through the dQ and dK/dV kernels: the dQ kernel (tiles of the shared
    // queries against one sequence's keys) writes each sequence's fp32 dQ contribution
    // and the row terms, the dK/dV kernel (head-pinned key tiles) reads the row terms,
    // and a reduce kernel sums the contributions over the sequences.
    const int64_t Mq = shape->num_q;
    const int p2 = max_programs(op, kDqWgPerCu);
    KeyChunks kc;
    bq_key_chunks(lengths, H, Mq, kDqRows, p2, false, kc);
    const int nc = (int)kc.b.size();
    if (nc > L.chunk_cap) return fail(JFA_ERR_WORKSPACE, "internal: chunk capacity");
    std::vector<int32_t> chunks(kc.b);  // [sequence | first key | keys]
    chunks.insert(chunks.end(), kc.k0.begin(), kc.k0.end());
    chunks.insert(chunks.end(), kc.len.begin(), kc.len.end());
    Schedule sq;  // tiles (chunk, h, query block), longest chunks first, zigzag
    schedule_fwd(kc.len, H, JFA_MODE_BROADCAST_Q, (int)Mq, kDqRows, p2, op.sched == 1, sq);
    if ((int64_t)sq.tiles.size() > L.tile2_cap || sq.programs > L.programs2_cap)
      return fail(JFA_ERR_WORKSPACE, "internal: tile capacity");
    if ((rc = visit_region(JFA_KERNEL_BWD_DQ, (int64_t)sq.tiles.size(), &p.dq_visits))) return rc;
    std::vector<char> buf;
    serialise(sc, L, buf, &sq, nullptr, &chunks);
    if ((rc = upload(buf.data(), buf.size(), ws, stream))) return rc;
    p.bq = 1;
    p.bq_chunks = (const int32_t*)(ws + L.chunks);
    p.num_chunks = nc;
    p.dq_acc = (float*)(ws + L.acc);
    p.row_aug = (uint16_t*)(ws + L.stats);
    p.dq_tiles = (const Tile*)(ws + L.tiles2);
    p.dq_seg_ptr = (const int32_t*)(ws + L.seg2);
    p.dq_programs = sq.programs;
    p.programs_per_head = std::max(1, sc.programs / H);
    if ((rc = launch_status(timed_launch(JFA_KERNEL_BWD_DQ, stream, [&] { return launch_bwd_self_dq(p, D, stream); }),
                            "backward dQ launch")))
      return rc;
    if (!sc.tiles.empty() &&
        (rc = launch_status(timed_launch(JFA_PASS_BWD, stream, [&] { return launch_bwd_self_dkdv(p, D, stream); }),
                            "backward dK/dV launch")))
      return rc;
    return launch_status(launch_dq_seq_reduce(p.dq_acc, (uint16_t*)dq, nc, Mq * H * D, scale, stream), "dq reduce");
  }

  // Broadcast-Q: one fused kernel; dQ summed over all sequences through fp32 atomics
  // (path 0) or per-program partial slabs and a reduce kernel (path 1).
  const bool partials = op.dq_path == 1;
  const int64_t Mq = shape->num_q;
  float* acc = (float*)(ws + L.acc);
  const int ph = std::max(1, sc.programs / H);
  const int64_t acc_elems = partials ? (int64_t)ph * H * Mq * D : Mq * H * D;
  if (!sc.tiles.empty()) {
    std::vector<char> buf;
    serialise(sc, L, buf);
    if ((rc = upload(buf.data(), buf.size(), ws, stream))) return rc;
  }
  if ((rc = launch_status(launch_fill_zero(acc, acc_elems, stream), "dq accumulator fill"))) return rc;
  if (!sc.tiles.empty()) {
    p.dq_acc = acc;
    p.dq_partials = partials ? 1 : 0;
    p.programs_per_head = ph;
    if ((rc = launch_status(timed_launch(JFA_PASS_BWD, stream, [&] { return launch_bwd(p, mode, D, stream); }),
                            "backward launch")))
      return rc;
  }
  if (partials)
    return launch_status(launch_dq_reduce(acc, (uint16_t*)dq, (int)Mq, H, D, ph, scale, stream), "dq reduce");
  return launch_status(launch_cast_scale(acc, (uint16_t*)dq, acc_elems, scale, stream), "dq cast");
}

int jfa_bwd(const jfa_shape* shape, int mode, float scale, const void* q, const void* k, const void* v,
            const void* o, const void* dout, const float* lse, const int32_t* offsets_dev,
            const int32_t* offsets_host, void* dq, void* dk, void* dv, void* workspace,
            size_t workspace_bytes, const jfa_opts* opts, void* stream) {
  return bwd_entry(shape, mode, scale, q, k, v, o, dout, lse, nullptr, 0, offsets_dev, offsets_host, dq, dk, dv,
                   workspace, workspace_bytes, opts, stream);
}

int jfa_bwd_rotary(const jfa_shape* shape, int mode, float scale, const void* q, const void* k, const void* v,
                   const void* o, const void* dout, const float* lse, const float* rope_cos_sin,
                   int32_t rope_positions, const int32_t* offsets_dev, const int32_t* offsets_host, void* dq,
                   void* dk, void* dv, void* workspace, size_t workspace_bytes, const jfa_opts* opts,
                   void* stream) {
  if (!rope_cos_sin) {
    g_detail.clear();
    return fail(JFA_ERR_NULL_POINTER, "rope_cos_sin is NULL");
  }
  return bwd_entry(shape, mode, scale, q, k, v, o, dout, lse, rope_cos_sin, rope_positions, offsets_dev,
                   offsets_host, dq, dk, dv, workspace, workspace_bytes, opts, stream);
}

int jfa_bwd_mxfp8(const jfa_shape* shape, float scale, const uint8_t* q8, const uint8_t* q_scales,
                  const uint8_t* k8, const uint8_t* k_scales, const uint8_t* v8t, const uint8_t* v_scales,
                  int64_t v_tokens, const void* o, const void* dout, const float* lse, const int32_t* offsets_dev,
                  const int32_t* offsets_host, void* dq, void* dk, void* dv, void* workspace,
                  size_t workspace_bytes, const jfa_opts* opts, void* stream_) {
  g_detail.clear();
  g_bwd_path = JFA_BWD_PATH_OTHER;
  hipStream_t stream = (hipStream_t)stream_;
  int rc = check_mx_shape(shape);
  if (rc) return rc;
  Opts op;
  if ((rc = check_opts(opts, op))) return rc;
  if (!q8 || !q_scales || !k8 || !k_scales || !v8t || !v_scales || !o || !dout || !lse || !offsets_dev || !dq || !dk ||
      !dv || !workspace)
    return fail(JFA_ERR_NULL_POINTER, "codes, scales, o, dout, lse, offsets_dev, dq, dk, dv and workspace must be "
                                      "non-NULL");
  if (!aligned(q8, 16) || !aligned(k8, 16) || !aligned(v8t, 16) || !aligned(workspace, kAlign))
    return fail(JFA_ERR_MISALIGNED, "codes 16-byte aligned, workspace 256-byte aligned");
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(JFA_ERR_BAD_SHAPE, "scale must be positive and finite");
  MxBwdLayout M;
  mx_bwd_layout(shape, op, M);
  if (workspace_bytes < M.total)
    return fail(JFA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, M.total);
  std::vector<int32_t> lengths;
  if ((rc = intake_offsets(shape, offsets_dev, offsets_host, stream, lengths))) return rc;
  const std::vector<int64_t> vb = mx_vbase(lengths);
  if (v_tokens != vb.back())
    return fail(JFA_ERR_BAD_SHAPE, "v_tokens %lld differs from jfa_mxfp8_v_tokens() = %lld", (long long)v_tokens,
                (long long)vb.back());
  char* ws = (char*)workspace;
  const int H = shape->num_heads, D = shape->head_dim;
  MxDequantParams p{};
  p.num_heads = H;
  p.head_dim = D;
  p.rows = shape->total_tokens * H;
  p.scales = q_scales;
  p.codes = q8;
  p.out = (uint16_t*)(ws + M.q);
  if ((rc = launch_status(timed_launch(JFA_KERNEL_MX_QUANT, stream, [&] { return launch_mx_dequant_qk(p, stream); }),
                          "MXFP8 decode launch")))
    return rc;
  p.scales = k_scales;
  p.codes = k8;
  p.out = (uint16_t*)(ws + M.k);
  if ((rc = launch_status(timed_launch(JFA_KERNEL_MX_QUANT, stream, [&] { return launch_mx_dequant_qk(p, stream); }),
                          "MXFP8 decode launch")))
    return rc;
  if (vb.back() > 0) {
    std::vector<char> buf(M.groups - M.vbase + (size_t)(vb.back() / kMxVPad) * sizeof(int32_t), 0);
    memcpy(buf.data(), vb.data(), vb.size() * sizeof(int64_t));
    int32_t* gs = reinterpret_cast<int32_t*>(buf.data() + (M.groups - M.vbase));
    for (size_t b = 0; b < lengths.size(); ++b)
      for (int64_t g = vb[b] / kMxVPad; g < vb[b + 1] / kMxVPad; ++g) gs[g] = (int32_t)b;
    if ((rc = upload(buf.data(), buf.size(), ws + M.vbase, stream))) return rc;
    p.codes = v8t;
    p.scales = v_scales;
    p.out = (uint16_t*)(ws + M.v);
    p.offsets = offsets_dev;
    p.vbase = (const int64_t*)(ws + M.vbase);
    p.group_seq = (const int32_t*)(ws + M.groups);
    p.tp = vb.back();
    if ((rc = launch_status(timed_launch(JFA_KERNEL_MX_QUANT, stream, [&] { return launch_mx_dequant_v(p, stream); }),
                            "MXFP8 V decode launch")))
      return rc;
  }
  return bwd_entry(shape, JFA_MODE_SELF, scale, ws + M.q, ws + M.k, ws + M.v, o, dout, lse, nullptr, 0, offsets_dev,
                   offsets_host, dq, dk, dv, ws + M.bwd, workspace_bytes - M.bwd, opts, stream);
}

}  // extern "C"
