// Host-side scheduler: turns a problem description into per-launch plans.
//
// The scan is serial over chunks inside a unit, so what the scheduler
// controls is which units exist and in which order the hardware dispatches
// them:
//   * a unit is (row, head, block of BV value columns); a row is a sequence,
//     or a chunk-aligned segment of one in the segment-parallel passes;
//   * rows are ordered longest first, so the longest serial chains start
//     first and short rows fill in behind them;
//   * the plan travels by value in the kernel arguments (at most kMaxRows rows
//     per launch; more rows take more launches), so a call needs no device
//     workspace, no host-to-device copy and no synchronisation;
//   * the tile (BV, waves, stages) comes from a fixed table keyed by the
//     problem's shape class, never from timing at run time, so the first call
//     cannot decide the tile of later ones (the failure mode kev pull request
//     #259 describes in its opening section).
#pragma once

#include <stdint.h>

#include <string>
#include <vector>

#include "common.hpp"

namespace gdr {

struct Seq {
  int64_t bos;
  int64_t len;
  int64_t chunk_off;  // first chunk (row of h) of this sequence
};

struct Problem {
  int B = 0, H = 0, DK = 0, DV = 0, N = 0;
  int64_t T = 0;
  int dtype = 0;
  int state_vk = 0;
  std::vector<Seq> seqs;
  int64_t n_chunks = 0;
  std::vector<int32_t> pool_idx;  // empty, or the state-pool row of each sequence
  int pool_size = 0;
};

struct Tile {
  int bv = 0, waves = 0, stages = 0;
};

struct Launch {
  std::vector<Row> rows;
  int grid = 0;
  int n_chunks = 0;    // chunk-parallel launches
  int chunk_base = 0;  // chunk-parallel launches
};

// Parses and validates; on failure returns false and sets err.
bool parse_problem(int B, int64_t T, int H, int DK, int DV, int N, const int32_t* cu_host, int dtype,
                   int state_layout, const int32_t* pool_idx_host, int pool_size, Problem& out, std::string& err);

// Tile for the serial scans: explicit request (validated) or the table.
// `rows` is the number of serial chains per head (sequences, or sequences x
// segments); mode 1 (summaries) also runs DK transition columns.
bool choose_tile(const Problem& p, const int32_t* req /* bv, waves, stages or null */, int mode, int64_t rows,
                 Tile& out, std::string& err);

// Kernel mode of the summary pass: 2 (each block holds half state and half
// transition columns, so all blocks of a (segment, head) run at one pace) for
// bfloat16 storage with DK == DV, else 1 (whole blocks of state columns, then
// of transition columns).
int summary_kernel_mode(const Problem& p);
// Column blocks per (row, head) of a scan launch in host mode `mode`.
int scan_blocks(const Problem& p, const Tile& t, int mode);

// Segment boundaries of one sequence: [t0, t1) token ranges relative to its start.
void segment_bounds(int64_t len, int P, std::vector<int64_t>& t0, std::vector<int64_t>& t1);

// Sub-segments per segment in the summary pass: 2 when the (segment, head)
// chains of a direct pass would leave the CUs with one wave per SIMD
// (bfloat16, DK = DV = 128, fewer than 512 column blocks of 128), so each
// segment's summary is formed from its two halves, else 1.  Depends on the
// problem shape and P only (not on the tile).
int summary_split(const Problem& p, int P);

// Segments per sequence the planner picks for the state scan when the caller
// names none (gdr_state_scan_auto): 0 (the serial scan) unless the serial
// units (sequence, head, 64 value columns) would leave more than half the 256
// CUs idle and the longest sequence has at least 8 chunks; then 32 segments
// for at most 4 non-empty (sequence, head) chains with 1024 or more chunks,
// else 16, halved until every segment of the longest sequence keeps at least
// 4 chunks (from a segment-count sweep of the summaries + compose + final
// pass on MI355X, DK = DV = 128: 64K tokens x 1, 2, 4 heads best at 32;
// x 8 heads, 16K x 2 and x 8, 8K x 4 and 4K x 16 best at 16).  Pools
// (state_indices) always get 0: the segmented passes do not take them.
int auto_segments(const Problem& p);

// Plans.  mode 0 = plain scan, 2 = segmented final pass, 1 = summaries.
// With split = 2 (summaries only) every segment becomes two rows, its first
// ceil(chunks / 2) chunks and the rest, written to summary slots 2s and 2s+1.
std::vector<Launch> plan_scan(const Problem& p, const Tile& t, int mode, int P, bool has_h0, bool has_hT,
                              int split = 1);
std::vector<Launch> plan_chunks(const Problem& p, int blocks_per_chunk);

}  // namespace gdr
