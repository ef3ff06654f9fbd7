// KV store writes: the base and the int4 delta layers.
//
// Page "FlashLoop: Fast and Memory-Efficient Looped Transformers via Lazy
// Updates", section "FlashLoop combines three kinds of savings", paragraph 3:
// the cache is a compressed base plus a chain of compressed corrections; an
// active token writes a 4-bit difference from its previous state, an inactive
// token writes nothing.
#include "fl_common.hpp"
#include "fl_commit.hpp"
#include "fl_launch.hpp"
#include "fl_timing.hpp"

namespace fl {

// slot(l, s, j) = slot_base + r if active_idx[s][r] == j, else -1 (reset) / untouched;
// `slots` points at column l-2 of the slot table, rows `pitch` apart.  A null
// `act` means every token is active (n_act == N, r == j).
__global__ __launch_bounds__(256) void k_slot_map(int32_t* __restrict__ slots, int32_t pitch, int32_t N,
                                                  const int32_t* __restrict__ act, int32_t n_act,
                                                  int32_t slot_base, int32_t reset,
                                                  const int32_t* __restrict__ exit_flags) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int s = blockIdx.y;
  if (j >= N || (exit_flags && exit_flags[s])) return;
  int32_t* dst = slots + (static_cast<int64_t>(s) * N + j) * pitch;
  if (!act) {
    *dst = slot_base + static_cast<int32_t>(j);
    return;
  }
  const int32_t* a = act + static_cast<int64_t>(s) * n_act;
  int lo = 0, hi = n_act;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < j) lo = mid + 1; else hi = mid;
  }
  if (lo < n_act && a[lo] == j) *dst = slot_base + lo;
  else if (reset) *dst = -1;
}

// One 16-lane group per (sequence, active row, head, K|V) row (a null `act`:
// every token, row r = token r).
template <int DT>
__global__ __launch_bounds__(256) void k_commit(KvView kv, uint8_t* __restrict__ arena_w, int32_t l,
                                                const int32_t* __restrict__ act, int32_t n_act,
                                                int32_t slot_base, const void* __restrict__ k_new,
                                                const void* __restrict__ v_new, int32_t src_compact) {
  const int64_t item = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x >> 4);
  const int p = threadIdx.x & 15;
  const int H = kv.H;
  const int64_t total = static_cast<int64_t>(kv.n_seq) * n_act * H * 2;
  if (item >= total) return;                                    // uniform per 16-lane group
  const int which = static_cast<int>(item & 1);
  const int h = static_cast<int>((item >> 1) % H);
  const int64_t sr = (item >> 1) / H;
  const int r = static_cast<int>(sr % n_act);
  const int s = static_cast<int>(sr / n_act);
  if (kv.exited(s)) return;                                     // uniform per 16-lane group
  const int j = act ? act[static_cast<int64_t>(s) * n_act + r] : r;
  const int64_t src_rows = src_compact ? n_act : kv.N;
  const int64_t src_row = src_compact ? r : j;
  const int64_t src_elem = ((static_cast<int64_t>(s) * src_rows + src_row) * H + h) * kv.d;
  commit_row<DT>(kv, arena_w, l, s, j, h, which, slot_base + r, which ? v_new : k_new, src_elem, p);
}

hipError_t launch_commit(const fl_commit_args& a, const KvView& kv, hipStream_t st) {
  uint8_t* arena = static_cast<uint8_t*>(a.kv->arena);
  if (a.version >= 2 && (a.n_active > 0 || a.reset_map)) {
    dim3 g((kv.N + 255) / 256, kv.n_seq);
    TimedLaunch t(st, "slot_map");
    hipLaunchKernelGGL(k_slot_map, g, dim3(256), 0, st,
                       reinterpret_cast<int32_t*>(arena + kv.slot_table) + (a.version - 2), kv.slot_pitch, kv.N,
                       a.active_idx, a.n_active, a.slot_base, a.reset_map, a.exit_flags);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.n_active == 0) return hipSuccess;
  const int64_t items = static_cast<int64_t>(kv.n_seq) * a.n_active * kv.H * 2;
  dim3 grid(static_cast<unsigned>((items + 15) / 16)), block(256);
  const int compact = a.src_layout == FL_ROWS_COMPACT;
  TimedLaunch t(st, a.version == 1 ? "commit_base" : "commit_delta");
  if (kv.dtype == FL_BF16)
    hipLaunchKernelGGL(k_commit<FL_BF16>, grid, block, 0, st, kv, arena, a.version, a.active_idx,
                       a.n_active, a.slot_base, a.k_new, a.v_new, compact);
  else
    hipLaunchKernelGGL(k_commit<FL_F32>, grid, block, 0, st, kv, arena, a.version, a.active_idx,
                       a.n_active, a.slot_base, a.k_new, a.v_new, compact);
  return hipGetLastError();
}

}  // namespace fl
