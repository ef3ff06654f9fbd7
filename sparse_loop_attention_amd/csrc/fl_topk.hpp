// Block-level top-k by radix select: the k largest of n scores, ties to the
// lower index, positions written in ascending order.
//
// Page "FlashLoop: Fast and Memory-Efficient Looped Transformers via Lazy
// Updates", section "FlashLoop combines three kinds of savings": paragraph 1
// keeps the tokens whose hidden state changed most, paragraph 2 the keys with
// the most previous-loop attention mass; both are this selection.
//
// One workgroup of NT threads selects from one segment; element i belongs
// to thread i mod NT (slot i / NT), so that every load of the workgroup is
// one contiguous run of the segment.  Keys are order-preserving bit patterns
// (larger score -> larger unsigned key, -0.0 == +0.0), selected 8 bits at a
// time from the top with wave-aggregated LDS histograms; the selection ends
// as soon as the crossing bin is taken whole.  Keys stay in registers as
// 32-bit words: the whole key of a float, the high word of a double's; a
// double's low word is reloaded through `load` only for keys whose high word
// ties the selected prefix.  Output positions are ranks in index order, from
// per-(slot, wave) ballot counts scanned once.
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
constexpr int kTopkMaxSlots = 64;                     // elements per thread

template <int NT>
struct TopkLds {
  int hist[256 * kTopkReplicas];
  int rank[kTopkMaxSlots * (NT / 64)];                // per (slot, wave) counts, then their exclusive prefix
  int rank_total;
  int sel_bin, sel_above, sel_count;
};

// Ranks in index order of the flagged elements: element (slot e, thread t)
// is index e * NT + t, so the order is slot, then wave, then lane.  flags:
// bit e of a thread's mask flags its slot-e element.  fn(e, rank) is called
// for every flagged element with the number of flagged elements before it;
// the return value is their total.  Every thread of the workgroup calls it.
template <int EPT, int NT, class Fn>
__device__ __forceinline__ int block_rank(uint64_t flags, TopkLds<NT>& s, Fn fn) {
  constexpr int kWaves = NT / 64, kTot = EPT * kWaves, kPer = (kTot + 63) / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const uint64_t b = __ballot((flags >> e) & 1);
    if (lane == 0) s.rank[e * kWaves + wave] = __popcll(b);
  }
  __syncthreads();
  if (wave == 0) {                                    // exclusive scan of the kTot counts in order
    int v[kPer], sum = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int idx = lane * kPer + j;
      v[j] = idx < kTot ? s.rank[idx] : 0;
      sum += v[j];
    }
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o, 64);
      if (lane >= o) incl += t;
    }
    int run = incl - sum;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int idx = lane * kPer + j;
      if (idx < kTot) s.rank[idx] = run;
      run += v[j];
    }
    if (lane == 63) s.rank_total = incl;
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const uint64_t b = __ballot((flags >> e) & 1);
    const int before = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(b >> 32),
                                                 __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(b), 0));
    if ((flags >> e) & 1) fn(e, s.rank[e * kWaves + wave] + before);
  }
  const int total = s.rank_total;
  __syncthreads();                                    // s.rank is free again
  return total;
}

// Every thread of the workgroup calls it.  load(i) returns score i (0 <= i <
// n); out(pos, i) stores the pos-th selected position (pos < k).  n <= NT*EPT.
template <typename ScoreT, int EPT, int NT, class Load, class Out>
__device__ __forceinline__ void topk_block(int64_t n, int32_t k, Load load, Out out, TopkLds<NT>& s) {
  static_assert(EPT <= kTopkMaxSlots, "at most 64 elements per thread");
  constexpr bool WIDE = sizeof(ScoreT) == 8;
  constexpr int kBits = WIDE ? 64 : 32;
  const int tid = threadIdx.x, lane = tid & 63;
  const int n32 = static_cast<int>(n);                // n <= NT * EPT
  auto index = [&](int e) -> int { return e * NT + tid; };

  if (k == 0) return;
  if (k >= n) {                                       // everything, already ascending
    for (int64_t i = tid; i < n; i += NT) out(static_cast<int>(i), static_cast<int32_t>(i));
    return;
  }
  // all loads first, at clamped (in-range) positions, so that they are in
  // flight together; a guarded load per element makes each wait for the last
  ScoreT raw[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) raw[e] = load(min(index(e), n32 - 1));
  uint32_t hi[EPT];
  uint64_t valid = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    hi[e] = index(e) < n32 ? static_cast<uint32_t>(order_key(raw[e]) >> (WIDE ? 32 : 0)) : 0u;
    valid |= static_cast<uint64_t>(index(e) < n32) << e;
  }
  auto lo_of = [&](int e) -> uint32_t { return static_cast<uint32_t>(order_key(load(index(e)))); };

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
      bool act = ((valid >> e) & 1) && ((hi[e] & msk_hi) == pre_hi);
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
      const int lbin = __builtin_amdgcn_readlane(bin, leader);   // leader is wave-uniform
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
  // and the first k_rem keys equal to it in index order.
  uint64_t above = 0, equal = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    if (!((valid >> e) & 1)) continue;
    const uint32_t h = hi[e] & msk_hi;
    int c = 0;
    if (h != pre_hi) c = h > pre_hi ? 1 : -1;
    else if (WIDE && msk_lo != 0) {
      const uint32_t l = lo_of(e) & msk_lo;
      c = l > pre_lo ? 1 : (l == pre_lo ? 0 : -1);
    }
    above |= static_cast<uint64_t>(c > 0) << e;
    equal |= static_cast<uint64_t>(c == 0) << e;
  }
  uint64_t take = above;
  block_rank<EPT, NT>(equal, s, [&](int e, int rank) { take |= static_cast<uint64_t>(rank < k_rem) << e; });
  block_rank<EPT, NT>(take, s, [&](int e, int rank) {
    if (rank < k) out(rank, static_cast<int32_t>(index(e)));
  });
}

}  // namespace fl
