// Host tile scheduler; see jfa_sched.h for the rules and their sources.
#include "jfa_sched.h"

#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <numeric>

namespace jfa {
namespace {

constexpr int kSelfMode = 0;
constexpr int kBroadcastMode = 1;

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Tiles sorted by (-L_b, b, h, blk): sequences ordered by decreasing length (stable in
// b), each sequence's tiles in (h, blk) order.
void sorted_tiles(const std::vector<int32_t>& lengths, int num_heads, int rows,
                  const std::vector<int32_t>& rows_of, std::vector<HostTile>& order) {
  const int nb = (int)lengths.size();
  std::vector<int32_t> seq(nb);
  std::iota(seq.begin(), seq.end(), 0);
  std::stable_sort(seq.begin(), seq.end(),
                   [&](int32_t a, int32_t b) { return lengths[a] > lengths[b]; });
  int64_t n = 0;
  for (int b = 0; b < nb; ++b) n += num_heads * cdiv(rows_of[b], rows);
  order.clear();
  order.reserve(n);
  for (int32_t b : seq) {
    const int32_t nblk = (int32_t)cdiv(rows_of[b], rows);
    for (int h = 0; h < num_heads; ++h)
      for (int32_t i = 0; i < nblk; ++i) order.push_back({b, h, i});
  }
}

// Zigzag dealing: sorted position n -> program pos (even pass) or P-1-pos (odd pass).
// Static: one segment per program.  Dynamic: one segment per counter group, the
// group's programs' tiles in sorted order.
void deal_zigzag(const std::vector<HostTile>& order, int max_programs, bool dynamic, Schedule& out) {
  const int64_t n = (int64_t)order.size();
  const int p = (int)std::min<int64_t>(max_programs, n);
  const int g = dynamic ? dynamic_groups(p) : p;
  out.programs = p;
  out.groups = dynamic ? g : 0;
  out.seg_ptr.assign(g + 1, 0);
  out.tiles.resize(n);
  if (p == 0) return;
  const int gsize = p / g;
  auto seg_of = [p, gsize](int64_t i) {
    const int64_t r = i / p, pos = i % p;
    return (int)((r & 1) ? p - 1 - pos : pos) / gsize;
  };
  for (int64_t i = 0; i < n; ++i) out.seg_ptr[seg_of(i) + 1]++;
  for (int i = 0; i < g; ++i) out.seg_ptr[i + 1] += out.seg_ptr[i];
  std::vector<int32_t> fill(out.seg_ptr.begin(), out.seg_ptr.end() - 1);
  for (int64_t i = 0; i < n; ++i) out.tiles[fill[seg_of(i)]++] = order[i];
}

// JFA_LOG=1 in the environment: one line on stderr per schedule built, with the tile
// and program counts and how evenly the tile cost falls on the segments (programs of a
// static schedule, counter groups of a dynamic one).  A tile costs cost_of[b] (its
// sequence's or chunk's key length), or 1 where cost_of is empty (equal-cost tiles).
bool log_enabled() {
  static const bool on = [] {
    const char* e = getenv("JFA_LOG");
    return e && *e && *e != '0';
  }();
  return on;
}

void log_schedule(const char* what, const std::vector<int32_t>& cost_of, const Schedule& s) {
  if (!log_enabled()) return;
  const int segs = (int)s.seg_ptr.size() - 1;
  double total = 0.0, worst = 0.0;
  for (int i = 0; i < segs; ++i) {
    double c = 0.0;
    for (int32_t t = s.seg_ptr[i]; t < s.seg_ptr[i + 1]; ++t) c += cost_of.empty() ? 1.0 : (double)cost_of[s.tiles[t].b];
    total += c;
    worst = std::max(worst, c);
  }
  const double mean = segs > 0 ? total / segs : 0.0;
  fprintf(stderr,
          "jfa schedule %s: tiles %lld, programs %d, %s %d, tile rows %d, cost %.0f, per segment max %.0f mean %.1f "
          "(max/mean %.3f)\n",
          what, (long long)s.tiles.size(), s.programs, s.groups > 0 ? "counter groups" : "static segments", segs,
          s.tile_rows, total, worst, mean, mean > 0.0 ? worst / mean : 0.0);
}

}  // namespace

void schedule_fwd(const std::vector<int32_t>& lengths, int num_heads, int mode, int num_q,
                  int rows, int max_programs, bool dynamic, Schedule& out) {
  std::vector<int32_t> rows_of(lengths.size());
  for (size_t b = 0; b < lengths.size(); ++b)
    rows_of[b] = (mode == kBroadcastMode) ? num_q : lengths[b];
  std::vector<HostTile> order;
  sorted_tiles(lengths, num_heads, rows, rows_of, order);
  out.tile_rows = rows;
  deal_zigzag(order, max_programs, dynamic, out);
  log_schedule(mode == kBroadcastMode ? "broadcast-Q sorted zigzag" : "self sorted zigzag", lengths, out);
}

void schedule_fwd_chunks(const std::vector<int32_t>& cost, const std::vector<int32_t>& rows_of, int num_heads,
                         int rows, int max_programs, bool dynamic, Schedule& out) {
  std::vector<HostTile> order;
  sorted_tiles(cost, num_heads, rows, rows_of, order);
  out.tile_rows = rows;
  deal_zigzag(order, max_programs, dynamic, out);
  log_schedule("self key chunks sorted zigzag", cost, out);
}

void schedule_bwd(const std::vector<int32_t>& lengths, int num_heads, int mode, int rows,
                  int max_programs, bool dynamic, Schedule& out) {
  out.tile_rows = rows;
  if (mode == kSelfMode) {
    std::vector<HostTile> order;
    sorted_tiles(lengths, num_heads, rows, lengths, order);
    deal_zigzag(order, max_programs, dynamic, out);
    log_schedule("self backward sorted zigzag", lengths, out);
    return;
  }
  // Broadcast-Q: head-pinned round robin.
  const int nb = (int)lengths.size();
  int64_t n_head = 0;
  for (int b = 0; b < nb; ++b) n_head += cdiv(lengths[b], rows);
  out.tiles.clear();
  if (n_head == 0) {
    out.programs = 0;
    out.groups = dynamic ? 1 : 0;
    out.seg_ptr = {0};
    log_schedule("broadcast-Q backward head-pinned", {}, out);
    return;
  }
  const int ph = (int)std::max<int64_t>(1, std::min<int64_t>(max_programs / num_heads, n_head));
  out.programs = ph * num_heads;
  out.tiles.reserve(n_head * num_heads);
  if (dynamic) {
    out.groups = num_heads;
    out.seg_ptr.assign(1, 0);
    for (int h = 0; h < num_heads; ++h) {
      for (int b = 0; b < nb; ++b)
        for (int32_t j = 0; j < (int32_t)cdiv(lengths[b], rows); ++j) out.tiles.push_back({b, h, j});
      out.seg_ptr.push_back((int32_t)out.tiles.size());
    }
    log_schedule("broadcast-Q backward head-pinned", {}, out);
    return;
  }
  out.groups = 0;
  out.seg_ptr.assign(1, 0);
  for (int h = 0; h < num_heads; ++h) {
    // program h*ph + r receives tiles r, r + ph, r + 2 ph, ... of head h
    std::vector<HostTile> head;
    head.reserve(n_head);
    for (int b = 0; b < nb; ++b)
      for (int32_t j = 0; j < (int32_t)cdiv(lengths[b], rows); ++j) head.push_back({b, h, j});
    for (int r = 0; r < ph; ++r) {
      for (int64_t i = r; i < n_head; i += ph) out.tiles.push_back(head[i]);
      out.seg_ptr.push_back((int32_t)out.tiles.size());
    }
  }
  log_schedule("broadcast-Q backward head-pinned", {}, out);
}

void schedule_blockdiag(const std::vector<int32_t>& lengths, int num_heads, int block,
                        int max_programs, int min_tiles, Schedule& out) {
  out.tile_rows = block;
  out.groups = 0;
  out.tiles.clear();
  for (int b = 0; b < (int)lengths.size(); ++b)
    for (int32_t j = 0; j < (int32_t)cdiv(lengths[b], block); ++j)
      for (int h = 0; h < num_heads; ++h) out.tiles.push_back({b, h, j});
  const int64_t n = (int64_t)out.tiles.size();
  const int p = (int)std::min<int64_t>(max_programs, cdiv(n, std::max(1, min_tiles)));
  out.programs = p;
  out.seg_ptr.assign(p + 1, 0);
  if (p > 0) {
    const int64_t q = n / p, r = n % p;
    for (int i = 0; i <= p; ++i) out.seg_ptr[i] = (int32_t)(i * q + std::min<int64_t>(i, r));
  }
  log_schedule("block-diagonal", {}, out);
}

}  // namespace jfa
