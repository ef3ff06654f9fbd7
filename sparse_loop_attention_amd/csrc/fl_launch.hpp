// Host-side launch entry points of each kernel family (validated arguments in).
#pragma once
#include <hip/hip_runtime.h>

#include "flashloop.h"
#include "fl_common.hpp"

namespace fl {

KvView make_view(const fl_kv_desc& d, const fl_kv_layout& lay);

hipError_t launch_select(const fl_select_args& a, hipStream_t st);
hipError_t launch_exit_check(const fl_exit_args& a, hipStream_t st);
hipError_t launch_commit(const fl_commit_args& a, const KvView& kv, hipStream_t st);

// Workspace layout of an attend call, shared by sizing and launching.
struct AttendPlan {
  bool mfma;            // tiled bf16 MFMA path (else the per-row path)
  int64_t rows;         // active rows per sequence
  int64_t keys;         // key slots per (sequence, head): n_keys (LAZY) or N (FULL)
  int splits;           // unused (0)
  int col_chunks;       // MFMA path: row ranges of the column-mass pass
  int col_rows;         // rows per range (a multiple of 64)
  // full loops over every row: ranges of col_var_rows rows per key block,
  // col_items (block, range) items per (sequence, head) (0 = fixed ranges)
  int col_var_rows, col_items;
  // MFMA path, full loops: the key tiles of a 256-row tile are cut into parts
  // of at most fsplit_u tiles, each a workgroup of its own (0 = no split);
  // f_items workgroups per (sequence, head), f_tiles row tiles
  int fsplit_u, f_items, f_tiles;
  // MFMA path, full loops in one round of workgroups: workgroups per (sequence,
  // head) that each take an early and a late 128-row half (0 = not used)
  int fpair;
  // MFMA path, lazy loops: forward workgroup shape (0: 256 rows and 64-key
  // tiles, 1: 128 and 32, 2: 64 and 32); with lsplit the two passes of a row
  // tile run as two workgroups (f_tiles row tiles per head; partials in
  // off_fpart, counters in off_fcount, the mass of the previous-loop pass in
  // off_lmass)
  int lazy_cfg;
  bool lsplit;
  // byte offsets in the workspace (off_pcol: lazy loops, the previous-loop
  // probabilities' per-key sums of each forward row tile)
  uint64_t off_part, off_logit, off_stat, off_gather, off_fpart, off_fcount, off_ccount, off_lmass, off_pcol, off_total;
  bool col_fused;       // several row ranges: the last range to finish adds them (no reduction launch)
};
// Forward key split of a full loop (0 = none) for n_sh (sequence, head) rows of
// n_rows rows; the same answer at sizing and at launch.
int plan_fwd_split(int64_t n_sh, int64_t n_rows);
// Workgroups per (sequence, head) of the forward pass under key split u.
int fwd_split_items(int64_t n_rows, int u);
// Workgroups per (sequence, head) of a full loop's forward pass with paired
// 128-row halves, or 0 where the grid would exceed one round of workgroups.
int plan_fwd_pair(int64_t n_sh, int64_t n_rows);
// Forward workgroup shape of a lazy loop (AttendPlan::lazy_cfg) and its rows.
int plan_lazy_cfg(int64_t n_sh, int64_t n_rows);
constexpr int lazy_cfg_rows(int cfg) { return cfg == 0 ? 256 : cfg == 1 ? 128 : 64; }
AttendPlan plan_attend(const fl_attend_args& a);
hipError_t launch_attend(const fl_attend_args& a, const KvView& kv, const AttendPlan& p, hipStream_t st);
// Device address of the library's static scratch on the stream's device
// (FLASHLOOP_STATIC_SCRATCH_BYTES; scratch.hip).
hipError_t static_scratch(hipStream_t st, void** out);

}  // namespace fl
