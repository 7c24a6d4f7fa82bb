// Host tile scheduler (pure C++; no HIP calls).
//
// Rules (aixai.ru page, "Tile balancing and Cluster Launch Control"; yuxiaoba page,
// "load balancing needs a static and a dynamic layer"; bittide page, section 5):
//  * forward tiles cost in proportion to their sequence's key length: sort by that
//    cost, largest first (ties by (b, h, blk)), deal in zigzag (even passes from the
//    first program to the last, odd passes back);
//  * self-attention backward tiles cost in proportion to L_b as well and take the same
//    rule; broadcast-Q backward tiles all cost the same (each loops over the shared
//    queries) and are dealt round robin within head-pinned program groups;
//  * only valid (non-empty) tiles are listed, except broadcast-Q forward tiles of an
//    empty sequence, which still write O = 0 and lse = -inf;
//  * dynamic mode keeps the same order and lets programs take tiles from an atomic
//    counter (one per group).  Forward and self-attention backward tiles form one
//    group per XCD when the program count is a multiple of kXcds: group g is the
//    programs g*P/kXcds .. (g+1)*P/kXcds - 1 (one XCD, see xcd_program_id) and holds,
//    in sorted order, the tiles the zigzag deal gives those programs, so neighbouring
//    tiles of one sequence still meet in one L2; otherwise one group of all tiles;
//  * block-diagonal tiles (one 64-token block of one head, head fastest) get balanced
//    contiguous ranges from divmod.
#pragma once

#include <stdint.h>

#include <vector>

namespace jfa {

constexpr int kXcds = 8;

// Counter groups of a dynamic forward or self-attention backward schedule of P programs.
constexpr int dynamic_groups(int programs) { return programs >= kXcds && programs % kXcds == 0 ? kXcds : 1; }

struct HostTile {
  int32_t b, h, blk;
};

struct Schedule {
  std::vector<HostTile> tiles;   // static: program-major; dynamic: global order
  std::vector<int32_t> seg_ptr;  // static: [P+1]; dynamic: [G+1]
  int32_t programs = 0;          // workgroups to launch
  int32_t tile_rows = 0;         // rows per tile (query rows fwd, key rows bwd, block)
  int32_t groups = 0;            // dynamic: counter groups; static: 0
};

// lengths: L_b for b < B (validated by the caller).
void schedule_fwd(const std::vector<int32_t>& lengths, int num_heads, int mode, int num_q,
                  int rows, int max_programs, bool dynamic, Schedule& out);
// Self-attention key chunks: chunk c (a tile "sequence" of cost[c] keys) has
// ceil(rows_of[c] / rows) query tiles per head (its sequence's rows); same sort and deal.
void schedule_fwd_chunks(const std::vector<int32_t>& cost, const std::vector<int32_t>& rows_of, int num_heads,
                         int rows, int max_programs, bool dynamic, Schedule& out);
void schedule_bwd(const std::vector<int32_t>& lengths, int num_heads, int mode, int rows,
                  int max_programs, bool dynamic, Schedule& out);
// Programs: min(max_programs, ceil(tiles / min_tiles)) (the block-diagonal kernels'
// workgroups hold min_tiles = kBdWaves waves, one tile each at a time).
void schedule_blockdiag(const std::vector<int32_t>& lengths, int num_heads, int block,
                        int max_programs, int min_tiles, Schedule& out);

}  // namespace jfa
