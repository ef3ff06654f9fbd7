// KV store writes: the base and the int4 delta layers.
//
// Page "FlashLoop: Fast and Memory-Efficient Looped Transformers via Lazy
// Updates", section "FlashLoop combines three kinds of savings", paragraph 3:
// the cache is a compressed base plus a chain of compressed corrections; an
// active token writes a 4-bit difference from its previous state, an inactive
// token writes nothing.
#include "fl_common.hpp"
#include "fl_launch.hpp"
#include "fl_timing.hpp"

namespace fl {

// slot(l, s, j) = slot_base + r if active_idx[s][r] == j, else -1 (reset) / untouched;
// `slots` points at column l-2 of the slot table, rows `pitch` apart.
__global__ __launch_bounds__(256) void k_slot_map(int32_t* __restrict__ slots, int32_t pitch, int32_t N,
                                                  const int32_t* __restrict__ act, int32_t n_act,
                                                  int32_t slot_base, int32_t reset) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int s = blockIdx.y;
  if (j >= N) return;
  const int32_t* a = act + static_cast<int64_t>(s) * n_act;
  int lo = 0, hi = n_act;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < j) lo = mid + 1; else hi = mid;
  }
  int32_t* dst = slots + (static_cast<int64_t>(s) * N + j) * pitch;
  if (lo < n_act && a[lo] == j) *dst = slot_base + lo;
  else if (reset) *dst = -1;
}

// One 16-lane group per (sequence, active row, head, K|V) row; lane p owns the
// 8 elements [8p, 8p+8) of the head row (lanes with 8p >= d idle).  A group of
// 32 elements is 4 consecutive lanes.
template <int DT>
__global__ __launch_bounds__(256) void k_commit(KvView kv, uint8_t* __restrict__ arena_w, int32_t l,
                                                const int32_t* __restrict__ act, int32_t n_act,
                                                int32_t slot_base, const void* __restrict__ k_new,
                                                const void* __restrict__ v_new, int32_t src_compact) {
  const int64_t item = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x >> 4);
  const int p = threadIdx.x & 15;
  const int H = kv.H, d = kv.d;
  const int64_t total = static_cast<int64_t>(kv.n_seq) * n_act * H * 2;
  if (item >= total) return;                                    // uniform per 16-lane group
  const int which = static_cast<int>(item & 1);
  const int h = static_cast<int>((item >> 1) % H);
  const int64_t sr = (item >> 1) / H;
  const int r = static_cast<int>(sr % n_act);
  const int s = static_cast<int>(sr / n_act);
  const int j = act[static_cast<int64_t>(s) * n_act + r];
  const int64_t src_rows = src_compact ? n_act : kv.N;
  const int64_t src_row = src_compact ? r : j;
  const void* src = which ? v_new : k_new;
  const int64_t row = static_cast<int64_t>(s) * H + h;
  const bool live = 8 * p < d;

  float x[8];
  if (live) load8<DT>(src, ((static_cast<int64_t>(s) * src_rows + src_row) * H + h) * d + 8 * p, x);
  if (l == 1) {
    if (live) store8<DT>(arena_w + kv.base[which], (row * kv.N + j) * d + 8 * p, x);
    return;
  }
  float prev[8], delta[8];
  float amax = 0.0f;
  if (live) {
    recon8<DT>(kv, which, s, h, j, l - 1, p, prev, nullptr);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      delta[e] = x[e] - prev[e];
      amax = fmaxf(amax, fabsf(delta[e]));
    }
  }
  amax = group_max<4>(amax);                                    // the 4 lanes of a group of 32
  const float q = fminf(amax / 7.0f, 65504.0f);                 // correctly rounded division
  const uint16_t sbits = f32_to_half_bits(q);
  const float sc = half_bits_to_f32(sbits);
  if (!live) return;
  uint32_t packed = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    int c = 0;
    if (sc != 0.0f) c = static_cast<int>(fminf(fmaxf(__builtin_rintf(delta[e] / sc), -7.0f), 7.0f));
    packed |= (static_cast<uint32_t>(c) & 0xFu) << (4 * e);
  }
  const int64_t rec = kv.record(l, s, slot_base + r, h, which);
  *reinterpret_cast<uint32_t*>(arena_w + kv.codes[l] + rec * (d / 2) + 4 * p) = packed;
  if ((p & 3) == 0)
    *reinterpret_cast<uint16_t*>(arena_w + kv.scales[l] + (rec * (d / 32) + (p >> 2)) * 2) = sbits;
}

hipError_t launch_commit(const fl_commit_args& a, const KvView& kv, hipStream_t st) {
  if (a.n_active == 0) return hipSuccess;
  uint8_t* arena = static_cast<uint8_t*>(a.kv->arena);
  if (a.version >= 2) {
    dim3 g((kv.N + 255) / 256, kv.n_seq);
    TimedLaunch t(st, "slot_map");
    hipLaunchKernelGGL(k_slot_map, g, dim3(256), 0, st,
                       reinterpret_cast<int32_t*>(arena + kv.slot_table) + (a.version - 2), kv.slot_pitch, kv.N,
                       a.active_idx, a.n_active, a.slot_base, a.reset_map);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
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
