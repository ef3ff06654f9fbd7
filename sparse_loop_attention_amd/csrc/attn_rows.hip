// Per-row attention path: fp32 inputs, and few rows against many keys (decode).
//
// Page "FlashLoop: Fast and Memory-Efficient Looped Transformers via Lazy
// Updates", section "FlashLoop combines three kinds of savings", paragraph 2:
// attention uses only the keys chosen from the previous loop's statistics and
// the chosen group keeps the previous loop's probability mass.  Keys are read
// straight from the base+delta chain (paragraph 3), dequantised in registers.
//
// Three launches per call:
//   partial  - one wave per (key split, active row, sequence*head); each
//              16-lane group walks one key at a time (lane p owns 8 of the d
//              elements), keeps an online softmax of the current logits and
//              the fixed-normaliser sums of the previous loop, and stores the
//              raw logits for the column-mass pass;
//   combine  - merges the splits of a row and writes o and lse in place;
//   colmass  - one lane per key slot sums the row probabilities in fixed
//              row order (deterministic, no atomics).
#include "fl_common.hpp"
#include "fl_commit.hpp"
#include "fl_launch.hpp"
#include "fl_timing.hpp"

namespace fl {

constexpr int kKeysPerSplit = 64;     // one wave per split

struct RowArgs {
  const void* q_cur;
  const void* q_prev;
  int32_t q_compact, o_compact;
  const int32_t* act;
  int32_t n_act;
  const int32_t* keys;      // LAZY: [n_seq*H][n_keys]
  int32_t n_keys;
  float* o;
  float* lse;
  float* colmass;
  int32_t version;
  float scale;              // 1/sqrt(d)
  int32_t splits;
  int64_t key_slots;        // logit row length (n_keys or N)
  float* part;              // [sh][rows][splits][4 + 2d]
  float* logit;             // [2][sh][rows][key_slots]
  float* stat;              // [sh][rows][4] = lse_prev, lse_new, valid, -
};

__device__ __forceinline__ int upper_bound_i32(const int32_t* a, int n, int v) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] <= v) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// With FUSE (lazy only) the call also commits this loop's records: versions
// v-1 come from the chain, an active key's version v from k_new/v_new, and
// one extra wave per (row, head) (split index == a.splits) writes that row's
// K and V records (and, for head 0, the row's share of the slot-table column).
template <int DT, bool LAZY, bool FUSE>
__global__ __launch_bounds__(64) void k_rows_partial(KvView kv, RowArgs a, CommitArgs cm) {
  constexpr int kU = LAZY ? 2 : 4;                        // keys per 16-lane group and step
  const int split = blockIdx.x, r = blockIdx.y, sh = blockIdx.z;
  const int H = kv.H, d = kv.d;
  const int s = sh / H, h = sh % H;
  const int lane = threadIdx.x, g = lane >> 4, p = lane & 15;
  const bool live = 8 * p < d;
  const int i = a.act ? a.act[static_cast<int64_t>(s) * a.n_act + r] : r;
  const int32_t* sel = LAZY ? a.keys + static_cast<int64_t>(sh) * a.n_keys : nullptr;
  const int cnt = LAZY ? upper_bound_i32(sel, a.n_keys, i) : i + 1;     // visible key slots
  const int t_begin = split * kKeysPerSplit;
  const int t_end = min(cnt, t_begin + kKeysPerSplit);

  const int64_t rows_q = a.q_compact ? a.n_act : kv.N;
  const int64_t qrow = a.q_compact ? r : i;
  const int64_t qoff = ((static_cast<int64_t>(s) * rows_q + qrow) * H + h) * d + 8 * p;
  float qc[8] = {}, qp[8] = {};
  if (live) {
    load8<DT>(a.q_cur, qoff, qc);
    if (LAZY) load8<DT>(a.q_prev, qoff, qp);
  }
  const int64_t rows_total = a.n_act;
  const int64_t srow = static_cast<int64_t>(sh) * rows_total + r;
  float lse_prev = 0.0f;
  if (LAZY) {
    const int64_t rows_o = a.o_compact ? a.n_act : kv.N;
    const int64_t orow = a.o_compact ? r : i;
    lse_prev = a.lse[(static_cast<int64_t>(s) * rows_o + orow) * H + h];
  }
  float M = -INFINITY, Z = 0.0f, m = 0.0f;
  float acc[8] = {}, accp[8] = {};
  float* lg_cur = a.logit + srow * a.key_slots;
  float* lg_prev = a.logit + (static_cast<int64_t>(kv.n_seq) * H * rows_total + srow) * a.key_slots;

  const int32_t* act_s = a.act ? a.act + static_cast<int64_t>(s) * a.n_act : nullptr;
  if (FUSE && split == a.splits) {
    // this row's records of layer `version` (groups 0, 1: K, V)
    if (g < 2) {
      const int64_t src_rows = cm.src_compact ? a.n_act : kv.N;
      const int64_t src_elem = ((static_cast<int64_t>(s) * src_rows + (cm.src_compact ? r : i)) * H + h) * d;
      commit_row<DT>(kv, cm.arena, a.version, s, i, h, g, cm.slot_base + r, g ? cm.v_new : cm.k_new, src_elem, p);
    }
    if (h == 0) {
      // slot-table entries of the tokens after the previous active row, up to this row
      // (the last row also covers the tail of the sequence)
      const int lo = r > 0 ? act_s[r - 1] + 1 : 0;
      const int hi = r + 1 < a.n_act ? i : kv.N - 1;
      int32_t* col = reinterpret_cast<int32_t*>(cm.arena + kv.slot_table) + (a.version - 2);
      for (int jj = lo + lane; jj <= hi; jj += 64) {
        int32_t* dst = col + (static_cast<int64_t>(s) * kv.N + jj) * kv.slot_pitch;
        if (jj == i) *dst = cm.slot_base + r;
        else if (cm.reset) *dst = -1;
      }
    }
    return;
  }
  // stage the split's key positions and their first four layer slots in LDS:
  // one round of loads for the whole split, so each step below only issues
  // the (independent) base and record loads of its keys
  __shared__ int s_j[kKeysPerSplit];
  __shared__ int s_ra[kKeysPerSplit];                     // fused commit: position in the active list, or -1
  __shared__ i32x4 s_sl[kKeysPerSplit];
  {
    const int t = t_begin + lane;
    int jj = 0, ra = -1;
    i32x4 sl = i32x4{-1, -1, -1, -1};
    if (t < t_end) {
      jj = LAZY ? sel[t] : t;
      if (a.version >= 2) sl = *reinterpret_cast<const i32x4*>(kv.slot_row(s, jj));
      if (FUSE) ra = find_active(act_s, a.n_act, jj);
    }
    s_j[lane] = jj;
    s_ra[lane] = ra;
    s_sl[lane] = sl;
  }
  __syncthreads();

  // group g takes keys t0 .. t0+U-1 of every block of 4U keys
  for (int t0 = t_begin + g * kU; t0 < t_end; t0 += 4 * kU) {
    int j[kU];
    bool ok[kU];
    i32x4 pre[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int t = t0 + u;
      ok[u] = live && t < t_end;
      const int lt = min(t - t_begin, kKeysPerSplit - 1);
      j[u] = s_j[lt];
      pre[u] = s_sl[lt];
    }
    float kc[kU][8], vc[kU][8], kp[kU][8], vp[kU][8];
    if (FUSE) {
      // A reset commit clears layer v for every token it does not write: walk to v-1.
      // Otherwise layer v may hold earlier commits' records: walk to v (an active
      // key's own layer-v entry, possibly being written now, is then overridden).
      if (cm.reset) {
        recon_kv<DT, kU, false>(kv, s, h, j, ok, a.version - 1, p, kp, vp, kc, vc, pre);
#pragma unroll
        for (int u = 0; u < kU; ++u)
#pragma unroll
          for (int e = 0; e < 8; ++e) { kc[u][e] = kp[u][e]; vc[u][e] = vp[u][e]; }
      } else {
        recon_kv<DT, kU, true>(kv, s, h, j, ok, a.version, p, kc, vc, kp, vp, pre);
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int ra = (t0 + u < t_end) ? s_ra[t0 + u - t_begin] : -1;
        if (ra >= 0) {                                    // uniform over the 16-lane group
          float kn[8] = {}, vn[8] = {};
          if (live) {
            const int64_t src_rows = cm.src_compact ? a.n_act : kv.N;
            const int64_t src = ((static_cast<int64_t>(s) * src_rows + (cm.src_compact ? ra : j[u])) * H + h) * d + 8 * p;
            load8<DT>(cm.k_new, src, kn);
            load8<DT>(cm.v_new, src, vn);
          }
          advance8(kn, kp[u], live, kc[u]);
          advance8(vn, vp[u], live, vc[u]);
        }
      }
    } else {
      recon_kv<DT, kU, LAZY>(kv, s, h, j, ok, a.version, p, kc, vc, kp, vp, pre);
    }
    float sc[kU], sp[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      to_working8<DT>(kc[u]);
      to_working8<DT>(vc[u]);
      float dc = 0.0f, dp = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) dc = fmaf(qc[e], kc[u][e], dc);
      sc[u] = group_sum<16>(dc) * a.scale;
      if (LAZY) {
        to_working8<DT>(kp[u]);
        to_working8<DT>(vp[u]);
#pragma unroll
        for (int e = 0; e < 8; ++e) dp = fmaf(qp[e], kp[u][e], dp);
        sp[u] = group_sum<16>(dp) * a.scale;
      }
    }
    // ok[] differs only in lanes with 8p >= d; the logits come from the group sum
    float tmax = -INFINITY;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const bool in = t0 + u < t_end;
      if (in) {
        tmax = fmaxf(tmax, sc[u]);
        if (p == 0) {
          lg_cur[t0 + u] = sc[u];
          if (LAZY) lg_prev[t0 + u] = sp[u];
        }
      }
    }
    if (tmax == -INFINITY) continue;
    const float Mn = fmaxf(M, tmax);
    const float corr = __expf(M - Mn);
    Z *= corr;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= corr;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (t0 + u < t_end) {
        const float w = __expf(sc[u] - Mn);
        Z += w;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, vc[u][e], acc[e]);
        if (LAZY) {
          const float pp = __expf(sp[u] - lse_prev);
          m += pp;
#pragma unroll
          for (int e = 0; e < 8; ++e) accp[e] = fmaf(pp, vp[u][e], accp[e]);
        }
      }
    }
    M = Mn;
  }
  // merge the four 16-lane groups (they hold the same dims, different keys)
#pragma unroll
  for (int o = 16; o <= 32; o <<= 1) {
    const float Mo = __shfl_xor(M, o, 64);
    const float Zo = __shfl_xor(Z, o, 64);
    const float Mn = fmaxf(M, Mo);
    const float c1 = (M == -INFINITY) ? 0.0f : __expf(M - Mn);
    const float c2 = (Mo == -INFINITY) ? 0.0f : __expf(Mo - Mn);
    Z = Z * c1 + Zo * c2;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = acc[e] * c1 + __shfl_xor(acc[e], o, 64) * c2;
    M = Mn;
    if (LAZY) {
      m += __shfl_xor(m, o, 64);
#pragma unroll
      for (int e = 0; e < 8; ++e) accp[e] += __shfl_xor(accp[e], o, 64);
    }
  }
  float* out = a.part + (srow * a.splits + split) * (4 + 2 * d);
  if (lane == 0) { out[0] = M; out[1] = Z; out[2] = m; out[3] = 0.0f; }
  if (g == 0 && live) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      out[4 + 8 * p + e] = acc[e];
      out[4 + d + 8 * p + e] = accp[e];
    }
  }
}

template <bool LAZY>
__global__ __launch_bounds__(64) void k_rows_combine(int32_t n_seq, int32_t H, int32_t d, int32_t N,
                                                     RowArgs a) {
  const int r = blockIdx.x, sh = blockIdx.y, lane = threadIdx.x;
  const int s = sh / H, h = sh % H;
  const int i = a.act ? a.act[static_cast<int64_t>(s) * a.n_act + r] : r;
  const int64_t srow = static_cast<int64_t>(sh) * a.n_act + r;
  const int cnt = LAZY ? upper_bound_i32(a.keys + static_cast<int64_t>(sh) * a.n_keys, a.n_keys, i) : i + 1;
  const int used = (cnt + kKeysPerSplit - 1) / kKeysPerSplit;
  const float* part = a.part + srow * a.splits * (4 + 2 * d);
  float M = -INFINITY;
  for (int c = 0; c < used; ++c) M = fmaxf(M, part[c * (4 + 2 * d)]);
  float Z = 0.0f, m = 0.0f, o0 = 0.0f, o1 = 0.0f, a0 = 0.0f, a1 = 0.0f;
  const int e0 = lane, e1 = lane + 64;
  for (int c = 0; c < used; ++c) {
    const float* pc = part + c * (4 + 2 * d);
    const float w = (pc[0] == -INFINITY) ? 0.0f : __expf(pc[0] - M);
    Z = fmaf(pc[1], w, Z);
    m += pc[2];
    if (e0 < d) { o0 = fmaf(pc[4 + e0], w, o0); a0 += pc[4 + d + e0]; }
    if (e1 < d) { o1 = fmaf(pc[4 + e1], w, o1); a1 += pc[4 + d + e1]; }
  }
  const int64_t rows_o = a.o_compact ? a.n_act : N;
  const int64_t orow = a.o_compact ? r : i;
  float* o = a.o + ((static_cast<int64_t>(s) * rows_o + orow) * H + h) * d;
  float* lse = a.lse + (static_cast<int64_t>(s) * rows_o + orow) * H + h;
  float* st = a.stat + srow * 4;
  if (!LAZY) {
    const float inv = 1.0f / Z;
    if (e0 < d) o[e0] = o0 * inv;
    if (e1 < d) o[e1] = o1 * inv;
    if (lane == 0) {
      const float l = M + __logf(Z);
      *lse = l;
      st[0] = l; st[1] = l; st[2] = 1.0f; st[3] = 0.0f;
    }
    return;
  }
  const float lse_prev = *lse;
  const bool valid = (cnt > 0) && (m > 0.0f);
  if (valid) {
    const float f = m / Z;
    if (e0 < d) o[e0] = fmaf(f, o0, o[e0] - a0);
    if (e1 < d) o[e1] = fmaf(f, o1, o[e1] - a1);
  }
  __syncthreads();   // every lane has read lse_prev before lane 0 rewrites it
  if (lane == 0) {
    const float lnew = valid ? M + __logf(Z) - __logf(m) : lse_prev;
    if (valid) *lse = lnew;
    st[0] = lse_prev; st[1] = lnew; st[2] = valid ? 1.0f : 0.0f; st[3] = 0.0f;
  }
}

template <bool LAZY>
__global__ __launch_bounds__(64) void k_rows_colmass(int32_t n_seq, int32_t H, int32_t N, RowArgs a) {
  const int sh = blockIdx.y;
  const int t = blockIdx.x * 64 + threadIdx.x;
  const int s = sh / H;
  const int64_t slots = LAZY ? a.n_keys : N;
  if (t >= slots) return;
  const int j = LAZY ? a.keys[static_cast<int64_t>(sh) * a.n_keys + t] : t;
  const int32_t* act = a.act ? a.act + static_cast<int64_t>(s) * a.n_act : nullptr;
  const float* lg_cur = a.logit + static_cast<int64_t>(sh) * a.n_act * a.key_slots;
  const float* lg_prev = a.logit + (static_cast<int64_t>(n_seq) * H + sh) * a.n_act * a.key_slots;
  const float* st = a.stat + static_cast<int64_t>(sh) * a.n_act * 4;
  // rows are ascending: start at the first active row i >= j
  int lo = 0, hi = a.n_act;
  if (act == nullptr) {
    lo = min(j, a.n_act);                       // identity rows: row r is token r
  } else {
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (act[mid] < j) lo = mid + 1; else hi = mid;
    }
  }
  float acc = 0.0f;
  for (int r = lo; r < a.n_act; ++r) {
    const float* sr = st + r * 4;
    if (sr[2] == 0.0f) continue;
    const int64_t at = static_cast<int64_t>(r) * a.key_slots + t;
    float v = __expf(lg_cur[at] - sr[1]);
    if (LAZY) v -= __expf(lg_prev[at] - sr[0]);
    acc += v;
  }
  float* c = a.colmass + static_cast<int64_t>(sh) * N + j;
  if (LAZY) *c += acc; else *c = acc;
}

hipError_t launch_rows(const fl_attend_args& x, const KvView& kv, const AttendPlan& p, hipStream_t st) {
  RowArgs a;
  a.q_cur = x.q_cur; a.q_prev = x.q_prev;
  a.q_compact = x.q_layout == FL_ROWS_COMPACT; a.o_compact = x.o_layout == FL_ROWS_COMPACT;
  a.act = x.active_idx; a.n_act = x.n_active;
  a.keys = x.key_idx; a.n_keys = x.n_keys;
  a.o = x.o; a.lse = x.lse; a.colmass = x.colmass;
  a.version = x.version;
  a.scale = 1.0f / sqrtf(static_cast<float>(kv.d));
  a.splits = p.splits;
  a.key_slots = p.keys;
  uint8_t* ws = static_cast<uint8_t*>(x.workspace);
  a.part = reinterpret_cast<float*>(ws + p.off_part);
  a.logit = reinterpret_cast<float*>(ws + p.off_logit);
  a.stat = reinterpret_cast<float*>(ws + p.off_stat);
  const bool lazy = x.mode == FL_ATTEND_LAZY;
  const int sh = kv.n_seq * kv.H;
  const bool fuse = lazy && x.fuse_commit;
  dim3 g1(p.splits + (fuse ? 1 : 0), x.n_active, sh);
  CommitArgs cm{};
  if (fuse) {
    cm.arena = static_cast<uint8_t*>(x.kv->arena);
    cm.k_new = x.k_new; cm.v_new = x.v_new;
    cm.src_compact = x.kv_layout == FL_ROWS_COMPACT;
    cm.slot_base = x.commit_slot_base; cm.reset = x.commit_reset;
  }
  {
    TimedLaunch t(st, fuse ? "rows_partial_commit_lazy" : lazy ? "rows_partial_lazy" : "rows_partial_full");
#define FL_ROWS(DTV, LZ, FU) hipLaunchKernelGGL((k_rows_partial<DTV, LZ, FU>), g1, dim3(64), 0, st, kv, a, cm)
    if (kv.dtype == FL_BF16) {
      if (fuse) FL_ROWS(FL_BF16, true, true);
      else if (lazy) FL_ROWS(FL_BF16, true, false);
      else FL_ROWS(FL_BF16, false, false);
    } else {
      if (fuse) FL_ROWS(FL_F32, true, true);
      else if (lazy) FL_ROWS(FL_F32, true, false);
      else FL_ROWS(FL_F32, false, false);
    }
#undef FL_ROWS
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2(x.n_active, sh);
  {
  TimedLaunch t(st, "rows_combine");
  if (lazy) hipLaunchKernelGGL(k_rows_combine<true>, g2, dim3(64), 0, st, kv.n_seq, kv.H, kv.d, kv.N, a);
  else hipLaunchKernelGGL(k_rows_combine<false>, g2, dim3(64), 0, st, kv.n_seq, kv.H, kv.d, kv.N, a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  dim3 g3(static_cast<unsigned>((p.keys + 63) / 64), sh);
  TimedLaunch t(st, "rows_colmass");
  if (lazy) hipLaunchKernelGGL(k_rows_colmass<true>, g3, dim3(64), 0, st, kv.n_seq, kv.H, kv.N, a);
  else hipLaunchKernelGGL(k_rows_colmass<false>, g3, dim3(64), 0, st, kv.n_seq, kv.H, kv.N, a);
  return hipGetLastError();
}

}  // namespace fl
