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
#include "fl_topk.hpp"

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
// top-k by radix select (fl_topk.hpp): one 1024-thread workgroup per segment.
// ---------------------------------------------------------------------------
constexpr int kTopkThreads = 1024;
// Key workgroups of at most 8 elements per thread keep to 64 VGPRs, so that
// two fit on a CU: the decode batch's 512 key segments then run in one round.
template <typename ScoreT, int EPT>
constexpr int kTopkWavesPerEu = sizeof(ScoreT) == 4 && EPT <= 8 ? 8 : 1;

template <typename ScoreT, int EPT>
__global__ __launch_bounds__(kTopkThreads) __attribute__((amdgpu_waves_per_eu(kTopkWavesPerEu<ScoreT, EPT>))) void k_topk(const ScoreT* __restrict__ scores,
                                                       int64_t seg_len, int32_t k,
                                                       int32_t* __restrict__ out_idx) {
  __shared__ TopkLds<kTopkThreads> lds;
  const ScoreT* src = scores + static_cast<int64_t>(blockIdx.x) * seg_len;
  int32_t* dst = out_idx + static_cast<int64_t>(blockIdx.x) * k;
  topk_block<ScoreT, EPT, kTopkThreads>(seg_len, k, [&](int64_t i) { return src[i]; },
                                        [&](int pos, int32_t idx) { dst[pos] = idx; }, lds);
}

// Token top-k of a later lazy loop, whose candidate rows (the previous
// loop's active set, ascending) are the only rows that may have changed:
// every other row scores exactly 0.  If at least k candidates score above 0,
// the k largest rows are the k largest candidates (all the others score 0,
// below them; ties between candidates still go to the lower row), so the
// selection runs over the candidates alone.  Otherwise, or if a candidate
// scores below 0 or NaN (orders the general selection defines), it leaves
// out_idx[0] = -1 and k_topk_rest selects over every row.  k >= 1.
template <int EPT>
__global__ __launch_bounds__(kTopkThreads) void k_topk_cand(const double* __restrict__ scores,
                                                            const int32_t* __restrict__ cand, int32_t n_cand,
                                                            int32_t k, int32_t* __restrict__ out_idx) {
  __shared__ TopkLds<kTopkThreads> lds;
  __shared__ int s_pos, s_bad;
  if (threadIdx.x == 0) { s_pos = 0; s_bad = 0; }
  __syncthreads();
  int pos = 0, bad = 0;
  for (int i = threadIdx.x; i < n_cand; i += kTopkThreads) {
    const double v = scores[cand[i]];
    pos += v > 0.0 ? 1 : 0;
    bad |= v >= 0.0 ? 0 : 1;
  }
  for (int o = 32; o > 0; o >>= 1) {
    pos += __shfl_xor(pos, o, 64);
    bad |= __shfl_xor(bad, o, 64);
  }
  if ((threadIdx.x & 63) == 0) {
    atomicAdd(&s_pos, pos);
    atomicOr(&s_bad, bad);
  }
  __syncthreads();
  if (s_bad || s_pos < k) {
    if (threadIdx.x == 0) out_idx[0] = -1;
    return;
  }
  topk_block<double, EPT, kTopkThreads>(n_cand, k, [&](int64_t i) { return scores[cand[i]]; },
                                        [&](int p, int32_t i) { out_idx[p] = cand[i]; }, lds);
}

// The general token top-k, where k_topk_cand left out_idx[0] = -1.
template <int EPT>
__global__ __launch_bounds__(kTopkThreads) void k_topk_rest(const double* __restrict__ scores, int64_t n, int32_t k,
                                                            int32_t* __restrict__ out_idx) {
  __shared__ TopkLds<kTopkThreads> lds;
  __shared__ int s_needed;
  if (threadIdx.x == 0) s_needed = out_idx[0] < 0;
  __syncthreads();
  if (!s_needed) return;
  topk_block<double, EPT, kTopkThreads>(n, k, [&](int64_t i) { return scores[i]; },
                                        [&](int p, int32_t i) { out_idx[p] = i; }, lds);
}

static hipError_t launch_topk_cand(const double* scores, const int32_t* cand, int32_t n_cand, int64_t n, int32_t k,
                                   int32_t* out, hipStream_t st) {
  const int64_t per_c = (n_cand + kTopkThreads - 1) / kTopkThreads, per = (n + kTopkThreads - 1) / kTopkThreads;
  dim3 grid(1), block(kTopkThreads);
  bool done = false;
#define FL_CAND_CASE(E)                                                                          \
  if (!done && per_c <= E) {                                                                     \
    TimedLaunch t(st, "topk_tokens");                                                            \
    hipLaunchKernelGGL(k_topk_cand<E>, grid, block, 0, st, scores, cand, n_cand, k, out);       \
    done = true;                                                                                 \
  }
  FL_CAND_CASE(1) FL_CAND_CASE(2) FL_CAND_CASE(4) FL_CAND_CASE(8) FL_CAND_CASE(16) FL_CAND_CASE(32) FL_CAND_CASE(64)
#undef FL_CAND_CASE
  if (!done) return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
#define FL_REST_CASE(E)                                                                          \
  if (per <= E) {                                                                                \
    TimedLaunch t(st, "topk_tokens_rest");                                                              \
    hipLaunchKernelGGL(k_topk_rest<E>, grid, block, 0, st, scores, n, k, out);                  \
    return hipGetLastError();                                                                    \
  }
  FL_REST_CASE(1) FL_REST_CASE(2) FL_REST_CASE(4) FL_REST_CASE(8) FL_REST_CASE(16) FL_REST_CASE(32) FL_REST_CASE(64)
#undef FL_REST_CASE
  return hipErrorInvalidValue;
}

template <typename ScoreT>
static hipError_t launch_topk(const ScoreT* scores, int64_t n_seg, int64_t seg_len, int32_t k,
                              int32_t* out, hipStream_t st, const char* label) {
  const int64_t per = (seg_len + kTopkThreads - 1) / kTopkThreads;
  dim3 grid(static_cast<unsigned>(n_seg)), block(kTopkThreads);
#define FL_TOPK_CASE(E)                                                                    \
  if (per <= E) {                                                                          \
    TimedLaunch t(st, label);                                                              \
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
    if (a.cand_idx && a.k > 0)
      return launch_topk_cand(a.scores, a.cand_idx, a.n_cand, a.n_rows, a.k, a.out_idx, st);
    return launch_topk<double>(a.scores, 1, a.n_rows, a.k, a.out_idx, st, "topk_tokens");
  }
  return launch_topk<float>(a.key_scores, a.n_seg, a.seg_len, a.k, a.out_idx, st, "topk_keys");
}

}  // namespace fl
