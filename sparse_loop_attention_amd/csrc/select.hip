// Token ranking and key selection kernels.
//
// Page "FlashLoop: Fast and Memory-Efficient Looped Transformers via Lazy
// Updates", section "FlashLoop combines three kinds of savings": paragraph 1
// ranks tokens by how much their hidden state changed (only the top fraction
// is recomputed); paragraph 2 picks keys from the previous loop's attention
// statistics.  Both reduce to "k largest, ties to the lower index, ascending".
#include "fl_common.hpp"
#include "fl_launch.hpp"
#include "fl_timing.hpp"

namespace fl {

// ---------------------------------------------------------------------------
// delta norm: one wave per row, float64 accumulation of (h_cur - h_prev)^2.
// Each lane streams 8 elements (16 B of bf16) per step, 4 steps in flight.
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ double row_change(const void* __restrict__ h_cur, const void* __restrict__ h_prev,
                                             int64_t base, int64_t hidden, int lane) {
  double acc = 0.0;
  constexpr int kUnroll = 4;
  int64_t e = static_cast<int64_t>(lane) * 8;
  for (; e + (kUnroll - 1) * 512 < hidden; e += kUnroll * 512) {
    float a[kUnroll][8], b[kUnroll][8];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      load8<DT>(h_cur, base + e + u * 512, a[u]);
      load8<DT>(h_prev, base + e + u * 512, b[u]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const double t = static_cast<double>(a[u][i]) - static_cast<double>(b[u][i]);
        acc = fma(t, t, acc);
      }
  }
  for (; e < hidden; e += 512) {
    float a[8], b[8];
    load8<DT>(h_cur, base + e, a);
    load8<DT>(h_prev, base + e, b);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const double t = static_cast<double>(a[i]) - static_cast<double>(b[i]);
      acc = fma(t, t, acc);
    }
  }
  return wave_sum_f64(acc);                       // every lane holds the row's sum
}

template <int DT>
__global__ __launch_bounds__(256) void k_delta_norm(const void* __restrict__ h_cur,
                                                    const void* __restrict__ h_prev, int64_t n_rows,
                                                    int64_t hidden, const int32_t* __restrict__ cand,
                                                    int32_t n_cand, double* __restrict__ scores) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= n_rows) return;
  if (cand != nullptr) {
    int lo = 0, hi = n_cand;                      // first index with cand[idx] >= row
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (cand[mid] < row) lo = mid + 1; else hi = mid;
    }
    if (lo >= n_cand || cand[lo] != row) {        // carried row: unchanged, scores exactly 0
      if (lane == 0) scores[row] = 0.0;
      return;
    }
  }
  const double acc = row_change<DT>(h_cur, h_prev, row * hidden, hidden, lane);
  if (lane == 0) scores[row] = acc;
}

// ---------------------------------------------------------------------------
// early exit: one workgroup per sequence takes the largest change of its rows
// (given scores, or the same float64 row sums as the token score) and sets
// the sequence's flag when it is below the threshold.  A set flag stays set.
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(256) void k_exit_check(const double* __restrict__ scores, const void* __restrict__ h_cur,
                                                    const void* __restrict__ h_prev, int32_t n_rows, int32_t hidden,
                                                    double threshold, int32_t* __restrict__ flags,
                                                    double* __restrict__ max_change) {
  __shared__ double red[4];
  const int s = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  double m = 0.0;                                 // changes are >= 0; fmax drops NaN
  if (scores) {
    for (int r = threadIdx.x; r < n_rows; r += 256) m = fmax(m, scores[static_cast<int64_t>(s) * n_rows + r]);
    for (int o = 32; o > 0; o >>= 1) m = fmax(m, __shfl_xor(m, o, 64));
  } else {
    for (int r = wave; r < n_rows; r += 4)
      m = fmax(m, row_change<DT>(h_cur, h_prev, (static_cast<int64_t>(s) * n_rows + r) * hidden, hidden, lane));
  }
  if (lane == 0) red[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = fmax(fmax(red[0], red[1]), fmax(red[2], red[3]));
    if (max_change) max_change[s] = m;
    if (m < threshold) flags[s] = 1;
  }
}

hipError_t launch_exit_check(const fl_exit_args& a, hipStream_t st) {
  TimedLaunch t(st, "exit_check");
  if (a.h_dtype == FL_BF16 && !a.scores)
    hipLaunchKernelGGL(k_exit_check<FL_BF16>, dim3(a.n_seq), dim3(256), 0, st, a.scores, a.h_cur, a.h_prev,
                       a.n_rows, a.hidden, a.threshold, a.exit_flags, a.max_change);
  else
    hipLaunchKernelGGL(k_exit_check<FL_F32>, dim3(a.n_seq), dim3(256), 0, st, a.scores, a.h_cur, a.h_prev,
                       a.n_rows, a.hidden, a.threshold, a.exit_flags, a.max_change);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// top-k by radix select over order-preserving key bits.
// One 1024-thread workgroup per segment; thread t owns elements
// [t*EPT, (t+1)*EPT) so that the final compaction is in index order.
// ---------------------------------------------------------------------------
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

constexpr int kTopkThreads = 1024;
// Histogram replicas: lane l counts into copy l mod kTopkReplicas of a bin
// (copies of one bin adjacent, so they sit in different LDS banks).  In the
// first passes most keys share a few bins (one exponent range), and
// per-lane atomics on one counter serialise; with the copies at most
// 64 / kTopkReplicas lanes of a wave meet on one address.
constexpr int kTopkReplicas = 8;
constexpr int kTopkWaves = kTopkThreads / 64;

// Exclusive scan of one int per thread across the workgroup; returns the total.
__device__ __forceinline__ int block_excl_scan(int v, int* lds_waves, int& total) {
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
    int w = lane < kTopkWaves ? lds_waves[lane] : 0;
    int wi = w;
#pragma unroll
    for (int o = 1; o < kTopkWaves; o <<= 1) {
      const int t = __shfl_up(wi, o, 64);
      if (lane >= o) wi += t;
    }
    if (lane < kTopkWaves) lds_waves[lane] = wi - w;   // exclusive wave offsets
    if (lane == kTopkWaves - 1) lds_waves[kTopkWaves] = wi;
  }
  __syncthreads();
  const int res = lds_waves[wave] + incl - v;
  total = lds_waves[kTopkWaves];
  __syncthreads();
  return res;
}

// Keys stay in registers as 32-bit words: the whole order key of a float, the
// high word of a double's.  A double's low word is reloaded from the scores
// (a read served by the L2) only where a pass or the final comparison needs
// it, i.e. for keys whose high word ties the selected prefix; every other key
// is decided by its high word.
template <typename ScoreT, int EPT>
__global__ __launch_bounds__(kTopkThreads) void k_topk(const ScoreT* __restrict__ scores,
                                                       int64_t seg_len, int32_t k,
                                                       int32_t* __restrict__ out_idx) {
  constexpr bool WIDE = sizeof(ScoreT) == 8;
  constexpr int kBits = WIDE ? 64 : 32;
  __shared__ __align__(16) int hist[256 * kTopkReplicas];
  __shared__ int scan_tmp[kTopkWaves + 1];
  __shared__ int sel_bin, sel_above, sel_count;

  const int64_t seg = blockIdx.x;
  const ScoreT* src = scores + seg * seg_len;
  int32_t* dst = out_idx + seg * static_cast<int64_t>(k);
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t first = static_cast<int64_t>(tid) * EPT;

  if (k == 0) return;
  if (k >= seg_len) {                                 // everything, already ascending
    for (int64_t i = tid; i < seg_len; i += kTopkThreads) dst[i] = static_cast<int32_t>(i);
    return;
  }
  // all loads first, at clamped (in-range) positions, so that they are in
  // flight together; a guarded load per element makes each wait for the last
  ScoreT raw[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) raw[e] = src[min(first + e, seg_len - 1)];
  uint32_t hi[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e)
    hi[e] = first + e < seg_len ? static_cast<uint32_t>(order_key(raw[e]) >> (WIDE ? 32 : 0)) : 0u;
  auto lo_of = [&](int e) -> uint32_t { return static_cast<uint32_t>(order_key(src[first + e])); };

  if (tid == 0) { sel_bin = 0; sel_above = 0; sel_count = 0; }
  uint32_t pre_hi = 0, msk_hi = 0, pre_lo = 0, msk_lo = 0;   // the selected prefix and its bits
  int k_rem = k;                                      // how many still to take at/below prefix
  for (int shift = kBits - 8; shift >= 0; shift -= 8) {
    const bool low = WIDE && shift < 32;              // a pass over the low word
    const int sh = low || !WIDE ? shift : shift - 32;
    for (int i = tid; i < 256 * kTopkReplicas; i += kTopkThreads) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      bool act = (first + e < seg_len) && ((hi[e] & msk_hi) == pre_hi);
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
        if (lane == leader) atomicAdd(&hist[lbin * kTopkReplicas], __popcll(m));
      } else if (act) {
        atomicAdd(&hist[bin * kTopkReplicas + (lane & (kTopkReplicas - 1))], 1);
      }
    }
    __syncthreads();
    if (tid < 64) {                                   // one wave finds the crossing bin, top down
      // lane L owns bins 255-4L .. 252-4L (descending)
      int c[4], s = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int4* hb = reinterpret_cast<const int4*>(hist + (255 - 4 * lane - i) * kTopkReplicas);
        c[i] = 0;
#pragma unroll
        for (int r = 0; r < kTopkReplicas / 4; ++r) c[i] += (hb[r].x + hb[r].y) + (hb[r].z + hb[r].w);
        s += c[i];
      }
      int incl = s;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
      }
      int above = incl - s;                           // count in bins strictly above my 4
      int found = -1, found_above = 0, found_count = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (found < 0 && above < k_rem && above + c[i] >= k_rem) {
          found = 255 - 4 * lane - i; found_above = above; found_count = c[i];
        }
        above += c[i];
      }
      if (found >= 0) { sel_bin = found; sel_above = found_above; sel_count = found_count; }
    }
    __syncthreads();
    const uint32_t b = static_cast<uint32_t>(sel_bin);
    k_rem -= sel_above;
    if (low) { pre_lo |= b << sh; msk_lo |= 0xFFu << sh; }
    else { pre_hi |= b << sh; msk_hi |= 0xFFu << sh; }
    const bool whole_bin = sel_count == k_rem;        // every key of the crossing bin is taken
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
  for (int e = 0; e < EPT; ++e) n_eq += (first + e < seg_len && cmp(e) == 0) ? 1 : 0;
  int tot;
  int eq_before = block_excl_scan(n_eq, scan_tmp, tot);
  int n_sel = 0;
  {
    int eq_rank = eq_before;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      if (first + e >= seg_len) continue;
      const int c = cmp(e);
      if (c > 0) ++n_sel;
      else if (c == 0) { if (eq_rank < k_rem) ++n_sel; ++eq_rank; }
    }
  }
  int pos = block_excl_scan(n_sel, scan_tmp, tot);
  {
    int eq_rank = eq_before;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      if (first + e >= seg_len) continue;
      const int c = cmp(e);
      bool take = false;
      if (c > 0) take = true;
      else if (c == 0) { take = eq_rank < k_rem; ++eq_rank; }
      if (take) {
        if (pos < k) dst[pos] = static_cast<int32_t>(first + e);
        ++pos;
      }
    }
  }
}

template <typename ScoreT>
static hipError_t launch_topk(const ScoreT* scores, int64_t n_seg, int64_t seg_len, int32_t k,
                              int32_t* out, hipStream_t st) {
  const int64_t per = (seg_len + kTopkThreads - 1) / kTopkThreads;
  dim3 grid(static_cast<unsigned>(n_seg)), block(kTopkThreads);
#define FL_TOPK_CASE(E)                                                                    \
  if (per <= E) {                                                                          \
    TimedLaunch t(st, "topk");                                                             \
    hipLaunchKernelGGL((k_topk<ScoreT, E>), grid, block, 0, st, scores, seg_len, k, out);  \
    return hipGetLastError();                                                              \
  }
  FL_TOPK_CASE(1) FL_TOPK_CASE(2) FL_TOPK_CASE(4) FL_TOPK_CASE(8) FL_TOPK_CASE(16)
  FL_TOPK_CASE(32) FL_TOPK_CASE(64)
#undef FL_TOPK_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_select(const fl_select_args& a, hipStream_t st) {
  if (a.mode == FL_SEL_TOKENS) {
    {
      dim3 grid(static_cast<unsigned>((a.n_rows + 3) / 4)), block(256);
      TimedLaunch t(st, "delta_norm");
      if (a.h_dtype == FL_BF16)
        hipLaunchKernelGGL(k_delta_norm<FL_BF16>, grid, block, 0, st, a.h_cur, a.h_prev, a.n_rows,
                           a.hidden, a.cand_idx, a.n_cand, a.scores);
      else
        hipLaunchKernelGGL(k_delta_norm<FL_F32>, grid, block, 0, st, a.h_cur, a.h_prev, a.n_rows,
                           a.hidden, a.cand_idx, a.n_cand, a.scores);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_topk<double>(a.scores, 1, a.n_rows, a.k, a.out_idx, st);
  }
  return launch_topk<float>(a.key_scores, a.n_seg, a.seg_len, a.k, a.out_idx, st);
}

}  // namespace fl
