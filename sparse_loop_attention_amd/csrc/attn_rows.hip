// Per-row attention path: fp32 inputs, and few rows against many keys (decode).
//
// Page "FlashLoop: Fast and Memory-Efficient Looped Transformers via Lazy
// Updates", section "FlashLoop combines three kinds of savings", paragraph 2:
// attention uses only the keys chosen from the previous loop's statistics and
// the chosen group keeps the previous loop's probability mass.  Keys are read
// straight from the base+delta chain (paragraph 3), dequantised in registers.
//
// One workgroup of 8 waves per (active row, sequence*head): the row's visible
// keys are dealt to the waves in chunks of 64; in each wave a 16-lane group
// walks U keys at a time (lane p owns 8 of the d elements), keeping an
// online softmax of the current logits and the fixed-normaliser sums of the
// previous loop.  The waves merge through LDS and write o and lse in place.
// With a single active row per sequence (decode) the row's logits stay in
// LDS and the same workgroup updates the column mass; otherwise the logits go
// to the workspace and a column-mass kernel sums the rows in fixed order
// (deterministic, no atomics).
#include "fl_common.hpp"
#include "fl_commit.hpp"
#include "fl_launch.hpp"
#include "fl_rows.hpp"
#include "fl_timing.hpp"

namespace fl {

constexpr int kRowWaves = 8;          // waves per workgroup
constexpr size_t kRowColMaxLds = 40960; // largest logit array (bytes) kept in LDS

// With FUSE (lazy only) the call also commits this loop's records: versions
// v-1 come from the chain, an active key's version v from k_new/v_new, and
// wave 0 first writes the row's K and V records of head h (and, for head 0,
// the row's share of the slot-table column).  With COL the workgroup owns
// the only active row of its sequence and updates the column mass itself.
// BASE (full loops over version 1): keys are the base rows, with no chain to
// walk; the smaller register footprint doubles the waves per CU, and with
// them the loads in flight.
template <int DT, bool LAZY, bool FUSE, bool COL, bool BASE = false>
__global__ __launch_bounds__(64 * kRowWaves) void k_rows_wg(KvView kv, RowArgs a, CommitArgs cm) {
  static_assert(!(BASE && LAZY), "BASE serves full loops");
  constexpr int kU = LAZY ? 2 : 4;                        // keys per 16-lane group and step
  const int r = blockIdx.x, sh = blockIdx.y;
  const int H = kv.H, d = kv.d;
  const int s = sh / H, h = sh % H;
  if (kv.exited(s)) return;                               // uniform per workgroup
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, p = lane & 15;
  const bool live = 8 * p < d;
  const int32_t* act_s = a.act ? a.act + static_cast<int64_t>(s) * a.n_act : nullptr;
  const int i = act_s ? act_s[r] : r;
  const int32_t* sel = LAZY ? a.keys + static_cast<int64_t>(sh) * a.n_keys : nullptr;
  const int cnt = LAZY ? wave_count_le(sel, a.n_keys, i) : i + 1;      // visible key slots

  extern __shared__ float s_lg[];                         // COL: logits [LAZY ? 2 : 1][key_slots]
  __shared__ int s_j[kRowWaves][64];
  __shared__ int s_ra[kRowWaves][64];                     // fused commit: position in the active list, or -1
  __shared__ i32x4 s_sl[kRowWaves][64];
  __shared__ float s_mzm[kRowWaves][3];
  __shared__ float s_acc[kRowWaves][2][128];

  if (FUSE && wave == 0) {
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
  }

  const int64_t rows_q = a.q_compact ? a.n_act : kv.N;
  const int64_t qrow = a.q_compact ? r : i;
  const int64_t qoff = ((static_cast<int64_t>(s) * rows_q + qrow) * H + h) * d + 8 * p;
  float qc[8] = {}, qp[8] = {};
  if (live) {
    load8<DT>(a.q_cur, qoff, qc);
    if (LAZY) load8<DT>(a.q_prev, qoff, qp);
  }
  const int64_t srow = static_cast<int64_t>(sh) * a.n_act + r;
  const int64_t rows_o = a.o_compact ? a.n_act : kv.N;
  const int64_t orow = a.o_compact ? r : i;
  float* o_row = a.o + ((static_cast<int64_t>(s) * rows_o + orow) * H + h) * d;
  float* lse_ptr = a.lse + (static_cast<int64_t>(s) * rows_o + orow) * H + h;
  const float lse_prev = LAZY ? *lse_ptr : 0.0f;
  float M = -INFINITY, Z = 0.0f, m = 0.0f;
  float acc[8] = {}, accp[8] = {};
  float* lg_cur = COL ? s_lg : a.logit + srow * a.key_slots;
  float* lg_prev = COL ? s_lg + a.key_slots
                       : a.logit + (static_cast<int64_t>(kv.n_seq) * H * a.n_act + srow) * a.key_slots;

  for (int t_begin = wave * 64; t_begin < cnt; t_begin += kRowWaves * 64) {
    const int t_end = min(cnt, t_begin + 64);
    // stage the chunk's key positions and their first four layer slots in
    // LDS: one round of loads for 64 keys, so that each step below only
    // issues the (independent) base and record loads of its keys
    {
      const int t = t_begin + lane;
      int jj = 0, ra = -1;
      i32x4 sl = i32x4{-1, -1, -1, -1};
      if (t < t_end) {
        jj = LAZY ? sel[t] : t;
        if (!BASE && a.version >= 2) sl = *reinterpret_cast<const i32x4*>(kv.slot_row(s, jj));
        if (FUSE) ra = find_active(act_s, a.n_act, jj);
      }
      s_j[wave][lane] = jj;
      s_ra[wave][lane] = ra;
      s_sl[wave][lane] = sl;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // group g takes keys t0 .. t0+U-1 of every block of 4U keys
    for (int t0 = t_begin + g * kU; t0 < t_end; t0 += 4 * kU) {
      int j[kU];
      bool ok[kU];
      i32x4 pre[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int t = t0 + u;
        ok[u] = live && t < t_end;
        const int lt = min(t - t_begin, 63);
        j[u] = s_j[wave][lt];
        pre[u] = s_sl[wave][lt];
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
          const int ra = (t0 + u < t_end) ? s_ra[wave][t0 + u - t_begin] : -1;
          if (ra >= 0) {                                  // uniform over the 16-lane group
            float kn[8] = {}, vn[8] = {};
            if (live) {
              const int64_t src_rows = cm.src_compact ? a.n_act : kv.N;
              const int64_t src =
                  ((static_cast<int64_t>(s) * src_rows + (cm.src_compact ? ra : j[u])) * H + h) * d + 8 * p;
              load8<DT>(cm.k_new, src, kn);
              load8<DT>(cm.v_new, src, vn);
            }
            advance8(kv, kn, kp[u], live, kc[u]);
            advance8(kv, vn, vp[u], live, vc[u]);
          }
        }
      } else if (BASE) {
        const int64_t row = (static_cast<int64_t>(s) * H + h) * kv.N;
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          if (ok[u]) {
            load8<DT>(kv.arena + kv.base[0], (row + j[u]) * d + 8 * p, kc[u]);
            load8<DT>(kv.arena + kv.base[1], (row + j[u]) * d + 8 * p, vc[u]);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) kc[u][e] = vc[u][e] = 0.0f;
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
        if (t0 + u < t_end) {
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
  }
  // merge the four 16-lane groups of the wave (same dims, different keys)
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
  // then the waves, through LDS, in fixed order
  if (lane == 0) { s_mzm[wave][0] = M; s_mzm[wave][1] = Z; s_mzm[wave][2] = m; }
  if (g == 0 && live) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      s_acc[wave][0][8 * p + e] = acc[e];
      s_acc[wave][1][8 * p + e] = accp[e];
    }
  }
  __syncthreads();
  float Mt = -INFINITY;
#pragma unroll
  for (int w = 0; w < kRowWaves; ++w) Mt = fmaxf(Mt, s_mzm[w][0]);
  float Zt = 0.0f, mt = 0.0f;
#pragma unroll
  for (int w = 0; w < kRowWaves; ++w) {
    const float cw = (s_mzm[w][0] == -INFINITY) ? 0.0f : __expf(s_mzm[w][0] - Mt);
    Zt = fmaf(s_mzm[w][1], cw, Zt);
    mt += s_mzm[w][2];
  }
  const bool valid = LAZY ? (cnt > 0 && mt > 0.0f) : true;
  if (tid < d) {
    float ov = 0.0f, av = 0.0f;
#pragma unroll
    for (int w = 0; w < kRowWaves; ++w) {
      const float cw = (s_mzm[w][0] == -INFINITY) ? 0.0f : __expf(s_mzm[w][0] - Mt);
      ov = fmaf(s_acc[w][0][tid], cw, ov);
      av += s_acc[w][1][tid];
    }
    if (!LAZY) o_row[tid] = ov / Zt;
    else if (valid) o_row[tid] = fmaf(mt / Zt, ov, a.mixture ? (1.0f - mt) * o_row[tid] : o_row[tid] - av);
  }
  const float lnew = LAZY ? (valid ? Mt + __logf(Zt) - __logf(mt) : lse_prev) : Mt + __logf(Zt);
  if (tid == 0) {
    if (!LAZY || valid) *lse_ptr = lnew;
    float* st = a.stat + srow * 4;
    st[0] = LAZY ? lse_prev : lnew; st[1] = lnew; st[2] = valid ? 1.0f : 0.0f; st[3] = 0.0f;
  }
  if (!COL) return;
  // column mass of the only row: c_j = p_ij (full) or c_j += p_ij - p'_ij (lazy)
  float* c = a.colmass + static_cast<int64_t>(sh) * kv.N;
  if (!LAZY) {
    for (int t = tid; t < kv.N; t += 64 * kRowWaves) c[t] = t < cnt ? __expf(lg_cur[t] - lnew) : 0.0f;
  } else if (valid) {
    const float f = mt / Zt;
    for (int t = tid; t < cnt; t += 64 * kRowWaves)
      c[sel[t]] += f * __expf(lg_cur[t] - Mt) - __expf(lg_prev[t] - lse_prev);
  }
}

// 64 key slots per workgroup, the rows split over its 4 waves (wave w takes
// rows lo+w, lo+w+4, ...); the 4 partial sums are added in wave order.
template <bool LAZY>
__global__ __launch_bounds__(256) void k_rows_colmass(int32_t n_seq, int32_t H, int32_t N, RowArgs a) {
  __shared__ float s_part[4][64];
  const int sh = blockIdx.y;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 64 + lane;
  const int s = sh / H;
  if (a.exit_flags && a.exit_flags[s]) return;           // uniform per workgroup
  const int64_t slots = LAZY ? a.n_keys : N;
  const bool live = t < slots;
  const int j = !live ? 0 : LAZY ? a.keys[static_cast<int64_t>(sh) * a.n_keys + t] : t;
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
  if (live) {
    for (int r = lo + w; r < a.n_act; r += 4) {
      const float4 sr = *reinterpret_cast<const float4*>(st + r * 4);
      if (sr.z == 0.0f) continue;
      const int64_t at = static_cast<int64_t>(r) * a.key_slots + t;
      float v = __expf(lg_cur[at] - sr.y);
      if (LAZY) v -= __expf(lg_prev[at] - sr.x);
      acc += v;
    }
  }
  s_part[w][lane] = acc;
  __syncthreads();
  if (w != 0 || !live) return;
  acc = ((s_part[0][lane] + s_part[1][lane]) + s_part[2][lane]) + s_part[3][lane];
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
  a.key_slots = p.keys;
  a.mixture = x.formula == FL_FORMULA_MIXTURE;
  uint8_t* ws = static_cast<uint8_t*>(x.workspace);
  a.logit = reinterpret_cast<float*>(ws + p.off_logit);
  a.stat = reinterpret_cast<float*>(ws + p.off_stat);
  a.exit_flags = kv.exit_flags;
  const bool lazy = x.mode == FL_ATTEND_LAZY;
  const int sh = kv.n_seq * kv.H;
  const bool fuse = lazy && x.fuse_commit;
  // one active row per sequence: the workgroup keeps the logits in LDS and
  // updates the column mass itself
  const size_t lg_bytes = static_cast<size_t>(lazy ? 2 : 1) * p.keys * 4;
  const bool col = x.n_active == 1 && lg_bytes <= kRowColMaxLds;
  const size_t lds = col ? lg_bytes : 0;
  dim3 g1(x.n_active, sh);
  CommitArgs cm{};
  if (fuse) {
    cm.arena = static_cast<uint8_t*>(x.kv->arena);
    cm.k_new = x.k_new; cm.v_new = x.v_new;
    cm.src_compact = x.kv_layout == FL_ROWS_COMPACT;
    cm.slot_base = x.commit_slot_base; cm.reset = x.commit_reset;
  }
  {
    hipError_t e = hipSuccess;
    if (lazy ? launch_decode_lazy(a, kv, cm, fuse, st, &e) : launch_decode_full(a, kv, st, &e)) return e;
  }
  {
    TimedLaunch t(st, fuse ? "rows_attend_commit_lazy" : lazy ? "rows_attend_lazy" : "rows_attend_full");
#define FL_ROWS(DTV, LZ, FU, CO, BA) \
  hipLaunchKernelGGL((k_rows_wg<DTV, LZ, FU, CO, BA>), g1, dim3(64 * kRowWaves), lds, st, kv, a, cm)
#define FL_ROWS_COL(DTV, LZ, FU, BA) \
  do { if (col) FL_ROWS(DTV, LZ, FU, true, BA); else FL_ROWS(DTV, LZ, FU, false, BA); } while (0)
    const bool base = !lazy && x.version == 1;
    if (kv.dtype == FL_BF16) {
      if (fuse) FL_ROWS_COL(FL_BF16, true, true, false);
      else if (lazy) FL_ROWS_COL(FL_BF16, true, false, false);
      else if (base) FL_ROWS_COL(FL_BF16, false, false, true);
      else FL_ROWS_COL(FL_BF16, false, false, false);
    } else {
      if (fuse) FL_ROWS_COL(FL_F32, true, true, false);
      else if (lazy) FL_ROWS_COL(FL_F32, true, false, false);
      else if (base) FL_ROWS_COL(FL_F32, false, false, true);
      else FL_ROWS_COL(FL_F32, false, false, false);
    }
#undef FL_ROWS_COL
#undef FL_ROWS
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || col) return e;
  dim3 g3(static_cast<unsigned>((p.keys + 63) / 64), sh);
  TimedLaunch t(st, "rows_colmass");
  if (lazy) hipLaunchKernelGGL(k_rows_colmass<true>, g3, dim3(256), 0, st, kv.n_seq, kv.H, kv.N, a);
  else hipLaunchKernelGGL(k_rows_colmass<false>, g3, dim3(256), 0, st, kv.n_seq, kv.H, kv.N, a);
  return hipGetLastError();
}

}  // namespace fl
