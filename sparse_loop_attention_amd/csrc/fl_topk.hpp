// Block-level top-k by radix select: the k largest of n scores, ties to the
// lower index, positions written in ascending order.
//
// Page "FlashLoop: Fast and Memory-Efficient Looped Transformers via Lazy
// Updates", section "FlashLoop combines three kinds of savings": paragraph 1
// keeps the tokens whose hidden state changed most, paragraph 2 the keys with
// the most previous-loop attention mass; both are this selection.
//
// One workgroup of NT threads selects from one segment; thread t owns
// elements [t*EPT, (t+1)*EPT), so the final compaction is in index order.
// Keys are order-preserving bit patterns (larger score -> larger unsigned
// key, -0.0 == +0.0), selected 8 bits at a time from the top with
// wave-aggregated LDS histograms; the selection ends as soon as the crossing
// bin is taken whole.  Keys stay in registers as 32-bit words: the whole key
// of a float, the high word of a double's; a double's low word is reloaded
// through `load` only for keys whose high word ties the selected prefix.
#pragma once
#include "fl_common.hpp"

namespace fl {

__device__ __forceinline__ uint64_t order_key(double x) {
  if (x == 0.0) x = 0.0;                              // -0.0 == +0.0
  const uint64_t u = __double_as_longlong(x);
  return (u & 0x8000000000000000ull) ? ~u : (u | 0x8000000000000000ull);
}
__device__ __forceinline__ uint32_t order_key(float x) {
  if (x == 0.0f) x = 0.0f;
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Histogram replicas: lane l counts into copy l mod kTopkReplicas of a bin
// (copies of one bin adjacent, so they sit in different LDS banks).  In the
// first passes most keys share a few bins (one exponent range), and per-lane
// atomics on one counter serialise; with the copies at most 64 /
// kTopkReplicas lanes of a wave meet on one address.
constexpr int kTopkReplicas = 8;

template <int NT>
struct TopkLds {
  int hist[256 * kTopkReplicas];
  int scan_tmp[NT / 64 + 1];
  int sel_bin, sel_above, sel_count;
};

// Exclusive scan of one int per thread across the NT-thread workgroup;
// `total` receives the sum.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* lds_waves, int& total) {
  constexpr int kWaves = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) lds_waves[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const int w = lane < kWaves ? lds_waves[lane] : 0;
    int wi = w;
#pragma unroll
    for (int o = 1; o < kWaves; o <<= 1) {
      const int t = __shfl_up(wi, o, 64);
      if (lane >= o) wi += t;
    }
    if (lane < kWaves) lds_waves[lane] = wi - w;      // exclusive wave offsets
    if (lane == kWaves - 1) lds_waves[kWaves] = wi;
  }
  __syncthreads();
  const int res = lds_waves[wave] + incl - v;
  total = lds_waves[kWaves];
  __syncthreads();
  return res;
}

// Every thread of the workgroup calls it.  load(i) returns score i (0 <= i <
// n); out(pos, i) stores the pos-th selected position (pos < k).  n <= NT*EPT.
template <typename ScoreT, int EPT, int NT, class Load, class Out>
__device__ __forceinline__ void topk_block(int64_t n, int32_t k, Load load, Out out, TopkLds<NT>& s) {
  constexpr bool WIDE = sizeof(ScoreT) == 8;
  constexpr int kBits = WIDE ? 64 : 32;
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t first = static_cast<int64_t>(tid) * EPT;

  if (k == 0) return;
  if (k >= n) {                                       // everything, already ascending
    for (int64_t i = tid; i < n; i += NT) out(static_cast<int>(i), static_cast<int32_t>(i));
    return;
  }
  // all loads first, at clamped (in-range) positions, so that they are in
  // flight together; a guarded load per element makes each wait for the last
  ScoreT raw[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) raw[e] = load(min(first + e, n - 1));
  uint32_t hi[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e)
    hi[e] = first + e < n ? static_cast<uint32_t>(order_key(raw[e]) >> (WIDE ? 32 : 0)) : 0u;
  auto lo_of = [&](int e) -> uint32_t { return static_cast<uint32_t>(order_key(load(first + e))); };

  if (tid == 0) { s.sel_bin = 0; s.sel_above = 0; s.sel_count = 0; }
  uint32_t pre_hi = 0, msk_hi = 0, pre_lo = 0, msk_lo = 0;   // the selected prefix and its bits
  int k_rem = k;                                      // how many still to take at/below prefix
  for (int shift = kBits - 8; shift >= 0; shift -= 8) {
    const bool low = WIDE && shift < 32;              // a pass over the low word
    const int sh = low || !WIDE ? shift : shift - 32;
    for (int i = tid; i < 256 * kTopkReplicas; i += NT) s.hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      bool act = (first + e < n) && ((hi[e] & msk_hi) == pre_hi);
      uint32_t word = hi[e];
      if (low && act) {
        word = lo_of(e);
        act = (word & msk_lo) == pre_lo;
      }
      const int bin = static_cast<int>((word >> sh) & 0xFF);
      // fast path: every active lane of the wave falls into one bin
      const uint64_t m = __ballot(act);
      if (m == 0) continue;
      const int leader = __ffsll(static_cast<unsigned long long>(m)) - 1;
      const int lbin = __shfl(bin, leader, 64);
      const uint64_t same = __ballot(act && bin == lbin);
      if (same == m) {
        if (lane == leader) atomicAdd(&s.hist[lbin * kTopkReplicas], __popcll(m));
      } else if (act) {
        atomicAdd(&s.hist[bin * kTopkReplicas + (lane & (kTopkReplicas - 1))], 1);
      }
    }
    __syncthreads();
    if (tid < 64) {                                   // one wave finds the crossing bin, top down
      // lane L owns bins 255-4L .. 252-4L (descending)
      int c[4], tot = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int4* hb = reinterpret_cast<const int4*>(s.hist + (255 - 4 * lane - i) * kTopkReplicas);
        c[i] = 0;
#pragma unroll
        for (int r = 0; r < kTopkReplicas / 4; ++r) c[i] += (hb[r].x + hb[r].y) + (hb[r].z + hb[r].w);
        tot += c[i];
      }
      int incl = tot;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
      }
      int above = incl - tot;                         // count in bins strictly above my 4
      int found = -1, found_above = 0, found_count = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (found < 0 && above < k_rem && above + c[i] >= k_rem) {
          found = 255 - 4 * lane - i; found_above = above; found_count = c[i];
        }
        above += c[i];
      }
      if (found >= 0) { s.sel_bin = found; s.sel_above = found_above; s.sel_count = found_count; }
    }
    __syncthreads();
    const uint32_t b = static_cast<uint32_t>(s.sel_bin);
    k_rem -= s.sel_above;
    if (low) { pre_lo |= b << sh; msk_lo |= 0xFFu << sh; }
    else { pre_hi |= b << sh; msk_hi |= 0xFFu << sh; }
    const bool whole_bin = s.sel_count == k_rem;      // every key of the crossing bin is taken
    __syncthreads();
    if (whole_bin) break;
  }
  // The prefix is the k-th largest key on the bits fixed so far (all of them
  // unless the crossing bin was taken whole); take every key above it there
  // and the first k_rem keys equal to it in index order.  cmp: +1 above, 0
  // equal, -1 below.
  auto cmp = [&](int e) -> int {
    const uint32_t h = hi[e] & msk_hi;
    if (h != pre_hi) return h > pre_hi ? 1 : -1;
    if (!WIDE || msk_lo == 0) return 0;
    const uint32_t l = lo_of(e) & msk_lo;
    return l > pre_lo ? 1 : (l == pre_lo ? 0 : -1);
  };
  int n_eq = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) n_eq += (first + e < n && cmp(e) == 0) ? 1 : 0;
  int tot;
  const int eq_before = block_excl_scan<NT>(n_eq, s.scan_tmp, tot);
  int n_sel = 0;
  {
    int eq_rank = eq_before;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      if (first + e >= n) continue;
      const int c = cmp(e);
      if (c > 0) ++n_sel;
      else if (c == 0) { if (eq_rank < k_rem) ++n_sel; ++eq_rank; }
    }
  }
  int pos = block_excl_scan<NT>(n_sel, s.scan_tmp, tot);
  {
    int eq_rank = eq_before;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      if (first + e >= n) continue;
      const int c = cmp(e);
      bool take = false;
      if (c > 0) take = true;
      else if (c == 0) { take = eq_rank < k_rem; ++eq_rank; }
      if (take) {
        if (pos < k) out(pos, static_cast<int32_t>(first + e));
        ++pos;
      }
    }
  }
}

}  // namespace fl
