// Tiled bf16 MFMA attention on gathered key tiles (prefill: many active rows).
//
// Page "FlashLoop: Fast and Memory-Efficient Looped Transformers via Lazy
// Updates", section "FlashLoop combines three kinds of savings": paragraph 2
// (attention on the keys chosen from the previous loop's statistics, keeping
// the chosen group's previous probability mass) and paragraph 4 (the selected
// data is gathered into dense buffers so that sparsity turns into speed).
//
// Launches per call:
//   gather   - walks the base+delta chain of every key slot (all N keys in a
//              full loop, the selected keys in a lazy loop) once, and writes
//              dense tiles: K^ rows [sh][slot][d] in bf16 and V^ transposed
//              [sh][d][slot] as fp16 holding the bf16-rounded values (keys
//              permuted inside each 16-key chunk so that an MFMA operand is
//              one 16-byte LDS read), plus the key positions; a lazy loop
//              gathers versions v-1 and v, and with a fused commit extra
//              blocks write this loop's records;
//   fwd      - one workgroup per 256 (or, for small lazy calls, 128 or 64)
//              query rows of one head; a full loop whose grid would leave CUs
//              idle cuts the heavy row tiles' keys into parts, merged by the
//              part that finishes last.  S^T = K Q^T on v_mfma_f32_32x32x16_bf16 keeps every
//              query in one lane pair, so the row softmax needs a single
//              cross-half exchange; P^T feeds the PV product straight from
//              the accumulators.  A lazy loop makes two passes: the previous
//              loop's probabilities with the fixed normaliser lse_prev (mass
//              m and contribution a, o <- o_prev - a), then the current
//              softmax over the selected keys (o <- o + m * otilde);
//   colmass  - key-major: one workgroup per 256 key slots (and a row range),
//              streaming the query tiles, S = Q K^T with keys in lanes so that
//              the column sums are lane-local; fixed order, no atomics (row
//              ranges are added by a small reduction kernel).
#include <climits>
#include <cstdlib>
#include <type_traits>

#include "fl_common.hpp"
#include "fl_commit.hpp"
#include "fl_launch.hpp"
#include "fl_timing.hpp"

namespace fl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));   // 16-byte chunk (promotes to registers)

struct MfmaArgs {
  // rows
  const int32_t* act;       // [n_seq][n_rows] token positions, or null = identity
  int32_t n_rows;
  const void* q_cur;        // bf16
  const void* q_prev;
  int32_t q_compact, o_compact;
  float* o;
  float* lse;
  float* colmass;
  // keys
  const int32_t* key_idx;   // LAZY: [sh][n_keys]; FULL: null (all N keys)
  int32_t n_keys;           // key slots per head
  int32_t n_keys_pad;       // multiple of 256
  int32_t version;
  float scale;
  // workspace
  uint16_t* kc;             // [sh][n_keys_pad][D]
  uint16_t* kp;
  uint16_t* vtc;            // [sh][D][n_keys_pad] (permuted keys)
  uint16_t* vtp;
  int32_t* kidx;            // [sh][n_keys_pad], INT_MAX for padding
  float* stat;              // [sh][n_rows][4] = lse_prev, lse_new, valid, token
  int32_t n_sh;             // n_seq * H
  // column mass: rows split into col_chunks ranges of col_rows rows; or, with
  // col_var_rows > 0 (full loops, rows = tokens = key slots), key block b's
  // rows [256 b, n_rows) split into ranges of col_var_rows rows, col_items
  // (block, range) items per head in all, at most col_chunks per block
  int32_t col_chunks, col_rows, col_var_rows, col_items;
  float* col_part;          // [col_chunks][sh][n_keys_pad] partial sums (col_chunks > 1)
  // forward key split (full loops): the key tiles of row tile t are cut into
  // ceil(tiles / fsplit_u) parts, one workgroup each (fsplit_u = 0: none)
  int32_t fsplit_u, f_items, f_tiles;   // workgroups and row tiles per head
  float4* fpart;            // [sh][f_items][D/8 + 1][512] partial acc, (max, sum)
  int32_t* fcount;          // [2][sh][f_tiles] parts finished, then the XCDs they ran on (zeroed by the gather)
  // lazy loops with the passes split (non-null): the previous-loop pass's
  // mass m per row [sh][n_rows]; fpart/fcount/f_tiles then hold the
  // current-loop pass's partials and the arrivals per row tile
  float* lmass;
  // lazy loops: per-key sums of the previous-loop probabilities over each
  // forward row tile's rows, [sh][row tiles][n_keys_pad] (row tiles of
  // pcol_rows rows; written by the forward for the key tiles it visits)
  float* pcol;
  int32_t pcol_rows;
  int32_t fpair;            // full loops: workgroups per head taking an early and a late 128-row half (0 = off)
  int32_t* ccount;          // [2][sh][n_keys_pad / 256] column-mass ranges finished, then the XCDs they ran on
                            // (bit x: XCD x), zeroed by the gather; or null
  // run-time check of the split reductions above: every part of a head must
  // run on one XCD (its L2 is where the parts' partial sums meet); a part on
  // another XCD sets FL_DEV_XCD_SPLIT in *dev_status (optional)
  int32_t* dev_status;
  int32_t xcd_test;         // nonzero: report part p's XCD as (XCD ^ (p & 1)), to test the check
  // early exit: sequences with a nonzero flag are skipped by every kernel
  const int32_t* exit_flags;  // [n_seq] or null
  int32_t heads;
  __device__ __forceinline__ bool exited(int s) const { return exit_flags && exit_flags[s]; }
};

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// PV runs in fp16: the probabilities need more than bf16's 8 significant bits
// to keep the output within tolerance; V^ (bf16 values) converts exactly.
__device__ __forceinline__ f32x16 mfma32h(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
// bf16-rounded V^ as fp16 bits; |v| is saturated at 65504 (the fp16 range).
__device__ __forceinline__ uint16_t v_operand_bits(float v) {
  const float b = fminf(fmaxf(round_bf16(v), -65504.0f), 65504.0f);
  return f32_to_half_bits(b);
}

// Workgroup -> (head row sh, tile) map.  Workgroups are handed to the 8 XCDs
// round-robin by linear id, and each XCD has its own L2; with at least 8
// (sequence, head) rows, every XCD gets whole heads (sh = xcd + 8k), so the
// gathered K/V tiles a head's query tiles share stay in one L2.  Tiles of a
// head run heavy (late, causal) first.  Returns false for padding workgroups.
__device__ __forceinline__ bool map_block(int n_sh, int n_tiles, int& sh, int& tile) {
  const int b = blockIdx.x;
  if (n_sh >= 8) {
    const int xcd = b & 7, local = b >> 3;
    sh = xcd + 8 * (local / n_tiles);
    tile = n_tiles - 1 - local % n_tiles;
    return sh < n_sh;
  }
  sh = b / n_tiles;
  tile = n_tiles - 1 - b % n_tiles;
  return sh < n_sh;
}
// Lazy loops with the two passes as two workgroups (n_sh >= 8): each XCD
// takes the previous-loop passes (role 1) of all its heads' row tiles, heavy
// first, then their current-loop passes in the same order, so that a row
// tile's current-loop pass starts well after its previous-loop pass (which
// it then finds done: no partial state to store).  Grid: mapped_grid(n_sh,
// 2 * n_tiles).
__device__ __forceinline__ bool map_split(int n_sh, int n_tiles, int& sh, int& tile, int& role) {
  const int b = blockIdx.x;
  const int xcd = b & 7, local = b >> 3;
  const int per_role = (n_sh + 7) / 8 * n_tiles;            // items of one role on this XCD
  role = local < per_role ? 1 : 0;
  const int rem = local % per_role;
  sh = xcd + 8 * (rem / n_tiles);
  tile = n_tiles - 1 - rem % n_tiles;
  return sh < n_sh;
}
__host__ __device__ inline int mapped_grid(int n_sh, int n_tiles) {
  return n_sh >= 8 ? 8 * ((n_sh + 7) / 8) * n_tiles : n_sh * n_tiles;
}

// A float4 read at device scope (past this CU's L1): data another workgroup
// of the XCD stored and acknowledged before counting its arrival.
__device__ __forceinline__ float4 ld4_agent(const float4* q) {
  const float* f = reinterpret_cast<const float*>(q);
  return make_float4(__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                     __hip_atomic_load(f + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                     __hip_atomic_load(f + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                     __hip_atomic_load(f + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ float4 ld4_agent_f(const float* p) { return ld4_agent(reinterpret_cast<const float4*>(p)); }

// The XCD (accelerator complex die) this wave runs on.
__device__ __forceinline__ uint32_t xcc_id() {
  uint32_t x;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID, 0, 4)" : "=s"(x));
  return x;
}

// Part `part` of a split reduction records its XCD in *mask before it counts
// its arrival; the last part (after its own record) compares the mask with
// its own XCD.  Called by one thread per workgroup.
__device__ __forceinline__ uint32_t xcd_bit(const MfmaArgs& a, int part) {
  return 1u << (a.xcd_test ? (xcc_id() ^ static_cast<uint32_t>(part & 1)) : xcc_id());
}
__device__ __forceinline__ void xcd_check(const MfmaArgs& a, int32_t* mask, uint32_t mine) {
  const uint32_t all = static_cast<uint32_t>(__hip_atomic_load(mask, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  if (all != mine && a.dev_status)
    __hip_atomic_fetch_or(a.dev_status, FL_DEV_XCD_SPLIT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int row_token(const MfmaArgs& a, int s, int r) {
  return a.act ? a.act[static_cast<int64_t>(s) * a.n_rows + r] : r;
}

// position of key offset k16 (0..15) inside its 16-key chunk of V^T:
// keys 4..7 and 8..11 swap places, so that k-slot i of lane half h
// (key 8*(i/4) + 4h + i%4) sits at 8h + i.
__device__ __forceinline__ int vt_pos(int k16) {
  const int q = k16 >> 2;
  return ((q == 1) ? 2 : (q == 2) ? 1 : q) * 4 + (k16 & 3);
}

// --------------------------------------------------------------------------- gather
// Grid (1-D): n_sh * n_tiles gather blocks (64 key slots each), then, when the
// commit is fused, the commit blocks (16 head rows each) and the slot-table
// blocks (256 tokens each).  The gather never reads what the fused commit
// writes (layer `version`): an active key's version is derived from k_new/v_new.
// U key slots of a 16-lane group walk their chains together (U = 4: four
// times the loads in flight, for grids too small to fill the chip; U = 1
// keeps the registers, and so the occupancy, of large grids).
constexpr int kCommitRows = 2;                             // active rows per 16-lane group in a lazy commit

template <int DT, int D, bool LAZY, bool FUSE, int U>
__global__ __launch_bounds__(256) void k_gather(KvView kv, MfmaArgs a, CommitArgs cm) {
  __shared__ uint16_t sv[2][64][D + 2];
  const int n_tiles = a.n_keys_pad / 64;
  int b = blockIdx.x;
  const int g = threadIdx.x >> 4, p = threadIdx.x & 15;
  if (a.fcount && b == 0)                                 // the forward pass's arrival counters and XCD masks
    for (int i = threadIdx.x; i < 2 * a.n_sh * a.f_tiles; i += 256) a.fcount[i] = 0;
  if (a.ccount && b == 0)                                 // the column-mass ranges' counters and XCD masks
    for (int i = threadIdx.x; i < 2 * a.n_sh * (a.n_keys_pad / 256); i += 256) a.ccount[i] = 0;
  if (FUSE && b >= a.n_sh * n_tiles) {
    b -= a.n_sh * n_tiles;
    // lazy loops: blocks of their own write the active rows' records (the
    // selected keys are other tokens); a full loop's key groups write them.
    // A 16-lane group takes kCommitRows consecutive active rows of one head,
    // K and V: their chains are walked together (one slot-row read per row
    // for both) with every load in flight at once.
    constexpr int CR = kCommitRows;
    const int row_groups = (a.n_rows + CR - 1) / CR;
    const int64_t items = LAZY ? static_cast<int64_t>(kv.n_seq) * kv.H * row_groups : 0;
    const int n_cb = static_cast<int>((items + 15) / 16);
    if (b < n_cb) {                                       // records of the active rows
      const int64_t item = static_cast<int64_t>(b) * 16 + g;
      if (item >= items) return;
      const int h = static_cast<int>(item % kv.H);
      const int64_t rest = item / kv.H;
      const int r0 = static_cast<int>(rest % row_groups) * CR, s = static_cast<int>(rest / row_groups);
      if (kv.exited(s)) return;                           // uniform per 16-lane group
      const bool live = 8 * p < D;
      int jj[CR];
      bool in[CR], ok[CR];
#pragma unroll
      for (int u = 0; u < CR; ++u) {
        const int r = r0 + u;
        in[u] = r < a.n_rows;                             // uniform per group
        jj[u] = !in[u] ? 0 : a.act ? a.act[static_cast<int64_t>(s) * a.n_rows + r] : r;
        ok[u] = in[u] && live;
      }
      float xk[CR][8], xv[CR][8], unused[CR][8];
      recon_kv<DT, CR, false>(kv, s, h, jj, ok, a.version - 1, p, xk, xv, unused, unused);
      const int64_t src_rows = cm.src_compact ? a.n_rows : kv.N;
      float nk[CR][8], nv[CR][8];
#pragma unroll
      for (int u = 0; u < CR; ++u) {
        if (ok[u]) {
          const int64_t src =
              ((static_cast<int64_t>(s) * src_rows + (cm.src_compact ? r0 + u : jj[u])) * kv.H + h) * D + 8 * p;
          load8<DT>(cm.k_new, src, nk[u]);
          load8<DT>(cm.v_new, src, nv[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < CR; ++u) {
        if (!in[u]) continue;
        float out[8];
        commit_advance8(kv, cm.arena, a.version, s, cm.slot_base + r0 + u, h, 0, nk[u], xk[u], live, p, out);
        commit_advance8(kv, cm.arena, a.version, s, cm.slot_base + r0 + u, h, 1, nv[u], xv[u], live, p, out);
      }
      return;
    }
    b -= n_cb;                                            // slot table column of layer `version`
    const int per_seq = (kv.N + 255) / 256;
    const int s = b / per_seq;
    const int j = (b % per_seq) * 256 + threadIdx.x;
    if (a.version < 2 || s >= kv.n_seq || j >= kv.N || kv.exited(s)) return;
    const int ra = a.act ? find_active(a.act + static_cast<int64_t>(s) * a.n_rows, a.n_rows, j) : j;
    int32_t* dst = reinterpret_cast<int32_t*>(cm.arena + kv.slot_table) +
                   (static_cast<int64_t>(s) * kv.N + j) * kv.slot_pitch + (a.version - 2);
    if (ra >= 0) *dst = cm.slot_base + ra;
    else if (cm.reset) *dst = -1;
    return;
  }
  const int sh = b / n_tiles, tile = b % n_tiles;
  const int s = sh / kv.H, h = sh % kv.H;
  if (kv.exited(s)) return;                               // uniform per workgroup
  const bool live = 8 * p < D;
  // fused commit: the active rows (null: every token, row = token)
  const int32_t* act_s = FUSE && a.act ? a.act + static_cast<int64_t>(s) * a.n_rows : nullptr;
  // the 16-lane group's 4 key slots, U at a time (recon_kv keeps every slot
  // and record load of the U keys in flight at once)
#pragma unroll 1
  for (int k0 = 0; k0 < 4; k0 += U) {
    int jj[U];
    bool ok[U];
#pragma unroll
    for (int kk = 0; kk < U; ++kk) {
      const int t = tile * 64 + g * 4 + k0 + kk;
      int j = -1;
      if (t < a.n_keys) j = a.key_idx ? a.key_idx[static_cast<int64_t>(sh) * a.n_keys + t] : t;
      jj[kk] = j;
      ok[kk] = live && j >= 0;
    }
    float x[U][8], y[U][8], xp[U][8], yp[U][8];
    if (FUSE) {
      // versions v-1 from the chain, version v from this loop's new rows.  A
      // reset commit clears layer v for the tokens it does not write; otherwise
      // layer v may hold earlier commits' records (an active key's own entry is
      // overridden below).  In a full loop every active row is one of the
      // keys, whose group writes its record (version 1: the base row) while
      // deriving the key's new version; version 1 of the other tokens is the
      // stored base.
      int ra[U];
#pragma unroll
      for (int kk = 0; kk < U; ++kk)
        ra[kk] = !ok[kk] ? -1 : act_s ? find_active(act_s, a.n_rows, jj[kk]) : jj[kk];
      const bool base_commit = !LAZY && a.version == 1;
      if (base_commit) {
        bool rd[U];
#pragma unroll
        for (int kk = 0; kk < U; ++kk) rd[kk] = ok[kk] && ra[kk] < 0;
        recon_kv<DT, U, false>(kv, s, h, jj, rd, 1, p, x, y, xp, yp);
      } else if (cm.reset) {
        recon_kv<DT, U, false>(kv, s, h, jj, ok, a.version - 1, p, x, y, xp, yp);
#pragma unroll
        for (int kk = 0; kk < U; ++kk)
#pragma unroll
          for (int e = 0; e < 8; ++e) { xp[kk][e] = x[kk][e]; yp[kk][e] = y[kk][e]; }
      } else {
        recon_kv<DT, U, true>(kv, s, h, jj, ok, a.version, p, x, y, xp, yp);
      }
#pragma unroll
      for (int kk = 0; kk < U; ++kk) {
        if (ra[kk] >= 0) {
          const int64_t src_rows = cm.src_compact ? a.n_rows : kv.N;
          const int64_t src =
              ((static_cast<int64_t>(s) * src_rows + (cm.src_compact ? ra[kk] : jj[kk])) * kv.H + h) * D + 8 * p;
          float kn[8], vn[8];
          load8<DT>(cm.k_new, src, kn);
          load8<DT>(cm.v_new, src, vn);
          if (base_commit) {
#pragma unroll
            for (int e = 0; e < 8; ++e) { x[kk][e] = kn[e]; y[kk][e] = vn[e]; }
            if (live) {
              const int64_t be = ((static_cast<int64_t>(s) * kv.H + h) * kv.N + jj[kk]) * D + 8 * p;
              store8<DT>(cm.arena + kv.base[0], be, kn);
              store8<DT>(cm.arena + kv.base[1], be, vn);
            }
          } else if (!LAZY) {
            commit_advance8(kv, cm.arena, a.version, s, cm.slot_base + ra[kk], h, 0, kn, xp[kk], live, p, x[kk]);
            commit_advance8(kv, cm.arena, a.version, s, cm.slot_base + ra[kk], h, 1, vn, yp[kk], live, p, y[kk]);
          } else {
            advance8(kv, kn, xp[kk], true, x[kk]);
            advance8(kv, vn, yp[kk], true, y[kk]);
          }
        }
      }
    } else if (LAZY) {
      recon_kv<DT, U, true>(kv, s, h, jj, ok, a.version, p, x, y, xp, yp);
    } else {
      recon_kv<DT, U, false>(kv, s, h, jj, ok, a.version, p, x, y, xp, yp);
    }
#pragma unroll
    for (int kk = 0; kk < U; ++kk) {
      const int local = g * 4 + k0 + kk;
      const int t = tile * 64 + local;
      if (live) {
        const int64_t krow = (static_cast<int64_t>(sh) * a.n_keys_pad + t) * D + 8 * p;
        store8<FL_BF16>(a.kc, krow, x[kk]);
        if (LAZY) store8<FL_BF16>(a.kp, krow, xp[kk]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          sv[0][local][8 * p + e] = v_operand_bits(y[kk][e]);
          if (LAZY) sv[1][local][8 * p + e] = v_operand_bits(yp[kk][e]);
        }
      }
      if (p == 0) a.kidx[static_cast<int64_t>(sh) * a.n_keys_pad + t] = jj[kk] >= 0 ? jj[kk] : INT_MAX;
    }
  }
  __syncthreads();
  // V^T: thread handles (dim, 8 consecutive stored positions)
  for (int item = threadIdx.x; item < D * 8; item += 256) {
    const int dim = item >> 3, pos0 = (item & 7) * 8;
#pragma unroll
    for (int which = 0; which < (LAZY ? 2 : 1); ++which) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        // stored position pos -> key offset inside the tile
        int pa = pos0 + e, pb = pos0 + e + 1;
        int ka = (pa & ~15) + vt_pos(pa & 15), kb = (pb & ~15) + vt_pos(pb & 15);   // vt_pos is an involution
        w[e / 2] = static_cast<uint32_t>(sv[which][ka][dim]) | (static_cast<uint32_t>(sv[which][kb][dim]) << 16);
      }
      uint16_t* dst = (which ? a.vtp : a.vtc) + (static_cast<int64_t>(sh) * D + dim) * a.n_keys_pad + tile * 64 + pos0;
      *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// --------------------------------------------------------------------------- fwd
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// max that propagates NaN (IEEE maximum): v_maximum3_f32 on gfx950, with no
// canonicalising copy of each MFMA result first (which fmaxf needs)
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// x combined with the value of lane l ^ 32 (the other key half of the same
// query), without a trip through LDS
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Per-key sums over a wave's 32 query rows of one key tile's probabilities,
// held as the forward holds them (S^T blocks: lane c and c + 32 have query c
// of the two key halves, 16 keys each per 32-key block), in float32.  A
// reduce-scatter over the 32 lanes of each half: at every level a lane keeps
// half of its values and adds its partner's copy of that half (partners: the
// other 16-lane row, then the row, half-row and quad mirrors and swaps), so
// each value moves once.  The lane ends with the sum of one value index of
// the S list (block * 16 + element): its lane index c with two blocks, c / 2
// with one (lanes c and c ^ 1 then hold the same sum).
template <int NKB>
__device__ __forceinline__ float col_reduce(const f32x16 (&S)[NKB], int lane) {
  constexpr int M = 16 * NKB;
  float v[M / 2];
#pragma unroll
  for (int m = 0; m < M / 2; ++m) {
    const int i = m, j = m + M / 2;
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(S[i >> 4][i & 15]),
                                                    __float_as_uint(S[j >> 4][j & 15]), false, false);
    v[m] = __uint_as_float(r[0]) + __uint_as_float(r[1]);   // rows 0, 2: value m; rows 1, 3: value m + M/2
  }
  auto level = [&](int n, bool hi, auto xchg) {
#pragma unroll
    for (int m = 0; m < n; ++m) {
      const float keep = hi ? v[m + n] : v[m], send = hi ? v[m] : v[m + n];
      v[m] = keep + xchg(send);
    }
  };
  level(M / 4, (lane >> 3) & 1, [](float x) { return dpp_mov<kDppRowMirror>(x); });
  level(M / 8, (lane >> 2) & 1, [](float x) { return dpp_mov<kDppRowHalfMirror>(x); });
  level(M / 16, (lane >> 1) & 1, [](float x) { return dpp_mov<kDppQuadSwap2>(x); });
  if constexpr (M == 32) level(1, lane & 1, [](float x) { return dpp_mov<kDppQuadSwap1>(x); });
  else v[0] += dpp_mov<kDppQuadSwap1>(v[0]);
  return v[0];
}

// One wave owns 32 query rows (one per lane pair: lane c and c+32 hold the
// two key halves of query c).  A workgroup of NW waves streams the key tiles
// of one role through LDS; per tile the wave computes S^T = K Q^T (bf16
// MFMA), the probabilities, and O^T += V^T P^T (fp16 MFMA).  The three steps
// are software-pipelined: while the softmax of tile t runs on the VALU, the
// matrix cores work on the QK product of tile t+1 and the PV product of tile
// t-1, which are independent of it.
//
// SOFTMAX role: online softmax over the visible keys (base-2 logits); the
// reference maximum is only moved when a new logit exceeds it by more than
// 2^8 (P stays far inside the fp16 range), so the O rescale is rare.
// FIXED role: probabilities against a fixed normaliser b_fix (the previous
// loop's lse), summed into the mass.
template <int D, int NW, int KT_>
struct FwdTiles {
  static constexpr int KT = KT_;                          // keys per tile: 32 or 64
  static constexpr int NT = 64 * NW;
  static constexpr int KS = D + 8, VS = KT + 8;          // padded LDS row strides (staged through registers)
  static constexpr int KCH = KT * D / 8, VCH = D * KT / 8;
  static constexpr int KPER = (KCH + NT - 1) / NT, VPER = (VCH + NT - 1) / NT;
  // Tiles are staged through registers: the loads of iteration t are stored
  // to LDS at its end, so they overlap its MFMA work; padded rows keep the
  // MFMA operand reads free of bank conflicts.
  static constexpr int RK = D / 8, RV = KT / 8;          // data chunks per K row, per V^T row
  static constexpr int KBUF = KT * KS, VBUF = D * VS;    // buffer elements
  __device__ static __forceinline__ int k_off(int row, int lc) { return row * KS + (lc << 3); }
  __device__ static __forceinline__ int v_off(int row, int lc) { return row * VS + (lc << 3); }
};


// NOPV: the pass needs only the probability mass (no V tiles, no PV product).
// WLIM: the wave computes only its first my_n of the workgroup's n_tiles key
// tiles (the rest lie past its rows' causal limit) and afterwards only helps
// stage the tiles the other waves still use.
// COLS (fixed-normaliser pass): the per-key sums of the probabilities over
// the workgroup's rows are written to col_dst[key slot] for every key tile
// the workgroup visits (the waves' sums meet in scol, [2][NW][KT] floats,
// and are added in wave order).
template <int D, int NW, int KT_, bool FIXED, bool NOPV = false, bool WLIM = false, bool COLS = false>
__device__ __forceinline__ void fwd_pass(const MfmaArgs& a, int n_tiles, const uint16_t* kbase, const uint16_t* vbase,
                                         const int32_t* kx, uint16_t (*sk)[FwdTiles<D, NW, KT_>::KBUF],
                                         uint16_t (*sv)[FwdTiles<D, NW, KT_>::VBUF], int (*skx)[KT_],
                                         const bf16x8 (&qf)[D / 16], int tok, int tok_first, int tok_last, bool blk_full,
                                         float c1, float b_fix, f32x16 (&acc)[D / 32], float& ref, float& lsum,
                                         int my_n = 0, float* col_dst = nullptr, float* scol = nullptr) {
  static_assert(!COLS || (FIXED && !WLIM), "column sums: fixed-normaliser passes over every tile");
  using T = FwdTiles<D, NW, KT_>;
  constexpr int KT = T::KT, NT = T::NT, KS = T::KS, VS = T::VS;
  (void)NT;
  constexpr int DC = D / 16, DB = D / 32;
  constexpr int NKB = KT / 32, NCC = KT / 16;             // 32-key logit blocks, 16-key PV chunks
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, c = lane & 31;
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  ref = -INFINITY;
  lsum = 0.0f;

  int pkx = INT_MAX;
  constexpr int KPER = (KT * D / 8 + NT - 1) / NT, VPER = (D * KT / 8 + NT - 1) / NT;
  u32x4 pk[KPER], pv[VPER];
  int kbuf_pending = 0, vbuf_pending = 0;             // LDS buffers the staged tiles go to
  auto load_k = [&](int buf, int tile) {
#pragma unroll
    for (int i = 0; i < KPER; ++i) {
      const int q = min(tid + NT * i, KT * D / 8 - 1);
      pk[i] = *reinterpret_cast<const u32x4*>(kbase + static_cast<int64_t>(tile * KT + q / (D / 8)) * D + (q % (D / 8)) * 8);
    }
    kbuf_pending = buf;
    pkx = kx[tile * KT + (tid & (KT - 1))];
  };
  auto load_v = [&](int buf, int tile) {
#pragma unroll
    for (int i = 0; i < VPER; ++i) {
      const int q = min(tid + NT * i, D * KT / 8 - 1);
      pv[i] = *reinterpret_cast<const u32x4*>(vbase + static_cast<int64_t>(q / (KT / 8)) * a.n_keys_pad + tile * KT + (q % (KT / 8)) * 8);
    }
    vbuf_pending = buf;
  };
  auto flush_k = [&]() {
#pragma unroll
    for (int i = 0; i < KPER; ++i) {
      const int q = min(tid + NT * i, KT * D / 8 - 1);
      *reinterpret_cast<u32x4*>(&sk[kbuf_pending][(q / (D / 8)) * KS + (q % (D / 8)) * 8]) = pk[i];
    }
  };
  auto flush_v = [&]() {
#pragma unroll
    for (int i = 0; i < VPER; ++i) {
      const int q = min(tid + NT * i, D * KT / 8 - 1);
      *reinterpret_cast<u32x4*>(&sv[vbuf_pending][(q / (KT / 8)) * VS + (q % (KT / 8)) * 8]) = pv[i];
    }
  };
  auto store_kx = [&](int tile) { skx[tile & 3][tid & (KT - 1)] = pkx; };   // identical values from every wave
  auto qk = [&](int buf, f32x16 (&S)[NKB]) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      S[kb] = f32x16{};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&sk[buf][T::k_off(kb * 32 + c, 2 * dc + hh)]);
        S[kb] = mfma32(ka, qf[dc], S[kb]);
      }
    }
  };
  auto pv_acc = [&](int buf, const f16x8 (&P)[NCC]) {
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const f16x8 va = *reinterpret_cast<const f16x8*>(&sv[buf][T::v_off(db * 32 + c, 2 * cc + hh)]);
        acc[db] = mfma32h(va, P[cc], acc[db]);
      }
  };
  // keys of tile `tile` after this lane's row get logit -inf (wave-uniform test)
  auto mask = [&](int tile, f32x16 (&S)[NKB]) {
    const int* kk = skx[tile & 3];
    if (!blk_full || kk[KT - 1] > tok_first) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const i32x4 kv = *reinterpret_cast<const i32x4*>(&kk[kb * 32 + 8 * q4 + 4 * hh]);
#pragma unroll
          for (int k4 = 0; k4 < 4; ++k4)
            if (kv[k4] > tok) S[kb][4 * q4 + k4] = -INFINITY;
        }
    }
  };
  auto rescale = [&](float alpha) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
  };

  if (n_tiles == 0) return;
  // prologue: K tiles 0 and 1 in LDS, logits of tile 0
  load_k(0, 0);
  flush_k();
  store_kx(0);
  if (n_tiles > 1) {
    load_k(1, 1);
    flush_k();
    store_kx(1);
  }
  __syncthreads();
  f32x16 S0[NKB], S1[NKB];
  f16x8 P[NCC];
  if (!WLIM || my_n > 0) qk(0, S0);
  __syncthreads();

  // iteration t: QK(t+1) into Sn, PV(t-1) with P, softmax(t) of Sc into P;
  // K(t+2) and V(t) are loaded for the next iterations.  Tiles past the end
  // are computed on whatever the buffers hold and never used.
  bool resc_prev = false;
  float alpha_prev = 1.0f;
  // The softmax of a tile as a list of small pieces, in dependency order:
  // partial maxima, the reduction and the reference update (SOFTMAX role
  // only), then the exponentials two values at a time (written back into S).
  // The step below issues one piece batch after every MFMA, in source order,
  // so that the scheduler keeps matrix and vector work interleaved.
  constexpr int kMaxPieces = FIXED ? 0 : 4 * NKB;
  constexpr int kExpBase = FIXED ? 0 : 4 * NKB + 5;
  constexpr int kPieces = kExpBase + 8 * NKB;             // 16 values per 32-key block, two per piece
  float mx[4 * NKB];
  float tmax = 0.0f, nref = 0.0f, sub = FIXED ? b_fix : 0.0f, alpha_cur = 1.0f;
  bool resc_cur = false;
  auto piece = [&](f32x16 (&S)[NKB], int q) {
    if (!FIXED && q < kMaxPieces) {
      const int j = q;
      mx[j] = vmax(vmax(S[j >> 2][(j & 3) * 4], S[j >> 2][(j & 3) * 4 + 1]),
                   vmax(S[j >> 2][(j & 3) * 4 + 2], S[j >> 2][(j & 3) * 4 + 3]));
    } else if (!FIXED && q == kMaxPieces) {
      if (NKB == 2) {
#pragma unroll
        for (int j = 0; j < 4; ++j) mx[j] = vmax(mx[j], mx[j + 4]);
      }
      tmax = vmax(vmax(mx[0], mx[1]), vmax(mx[2], mx[3]));
    } else if (!FIXED && q == kMaxPieces + 1) {
      tmax = max_xor32(tmax) * c1;
    } else if (!FIXED && q == kMaxPieces + 2) {
      resc_cur = __ballot(tmax > ref + 8.0f) != 0;         // some row's maximum moved far: exact rescale
      nref = resc_cur ? fmaxf(ref, tmax) : ref;
    } else if (!FIXED && q == kMaxPieces + 3) {
      alpha_cur = (ref == -INFINITY) ? 0.0f : ex2(ref - nref);
      lsum *= alpha_cur;
    } else if (!FIXED && q == kMaxPieces + 4) {
      ref = nref;
      sub = (ref == -INFINITY) ? 0.0f : ref;
    } else {
      const int e = 2 * (q - kExpBase);                   // values e, e+1 (of 16 * NKB)
#pragma unroll
      for (int k = 0; k < 2; ++k) S[(e + k) >> 4][(e + k) & 15] = ex2(fmaf(S[(e + k) >> 4][(e + k) & 15], c1, -sub));
    }
  };
  // P chunk cc (keys 16cc .. 16cc+15) from the exponentials, and its row
  // sum: over the fp16 values the PV product uses (softmax: the output's
  // weights are then normalised exactly), or in float32 for the fixed-
  // normaliser mass, whose terms can all lie below fp16's range and which
  // decides the row's validity and lse
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  typedef float f2v __attribute__((ext_vector_type(2)));
  auto convert = [&](f32x16 (&S)[NKB], int cc) {
    u32x4 pw;                                             // one packed conversion per value pair
#pragma unroll
    for (int i = 0; i < 4; ++i)
      pw[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2v{S[cc >> 1][(cc & 1) * 8 + 2 * i],
                                                                       S[cc >> 1][(cc & 1) * 8 + 2 * i + 1]}, h2));
    P[cc] = __builtin_bit_cast(f16x8, pw);
    float ps = 0.0f;
    if (FIXED) {
#pragma unroll
      for (int i = 0; i < 8; ++i) ps += S[cc >> 1][(cc & 1) * 8 + i];
    } else {
      const h2 one = {1.0f16, 1.0f16};
#pragma unroll
      for (int i = 0; i < 4; ++i) ps = __builtin_amdgcn_fdot2(h2{P[cc][2 * i], P[cc][2 * i + 1]}, one, ps, false);
    }
    lsum += ps;
  };
  // iteration t: QK(t+1) into Sn, PV(t-1) with P, softmax(t) of Sc into P;
  // K(t+2) and V(t) are loaded for the next iterations.  Tiles past the end
  // are computed on whatever the buffers hold and never used.
  // the column sums of tile tt (in scol since the barrier that ended its
  // step): one wave adds the NW waves' values and stores them
  auto col_store = [&](int tt) {
    if (wave == tt % NW && lane < KT) {
      const float* sc = scol + (tt & 1) * NW * KT + lane;
      float sum = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) sum += sc[w * KT];
      col_dst[tt * KT + lane] = sum;
    }
  };
  auto step = [&](int t, f32x16 (&Sc)[NKB], f32x16 (&Sn)[NKB], bool first) {
    load_k(t & 1, min(t + 2, n_tiles - 1));
    if (!NOPV) load_v(t & 1, t);
    if (COLS && !first) col_store(t - 1);
    if (resc_prev) rescale(alpha_prev);
    mask(t, Sc);
    resc_cur = false;
    alpha_cur = 1.0f;
    const bool pv = !NOPV && !first;
    constexpr int NQK = NKB * DC, NPV = NOPV ? 0 : NCC * DB;
    const uint16_t* K = sk[(t + 1) & 1];
    const uint16_t* V = sv[(t + 1) & 1];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) Sn[kb] = f32x16{};
    int done = 0;
    // MFMA operands (K fragments, then V^T fragments) in a 3-entry register
    // ring, read two products ahead of their use
    const int n_mfma = pv ? NQK + NPV : NQK;
    auto fetch = [&](int m) -> u32x4 {
      if (m < NQK) {
        const int kb = m / DC, dc = m % DC;
        return *reinterpret_cast<const u32x4*>(&K[T::k_off(kb * 32 + c, 2 * dc + hh)]);
      }
      const int j = m - NQK, cc = j / DB, db = j % DB;
      return *reinterpret_cast<const u32x4*>(&V[T::v_off(db * 32 + c, 2 * cc + hh)]);
    };
    u32x4 ring[3];
    ring[0] = fetch(0);
    if (n_mfma > 1) ring[1] = fetch(1);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int m = 0; m < NQK + NPV; ++m) {
      if (m >= n_mfma) break;
      if (m + 2 < n_mfma) ring[(m + 2) % 3] = fetch(m + 2);
      if (m < NQK) {
        const int kb = m / DC, dc = m % DC;
        Sn[kb] = mfma32(__builtin_bit_cast(bf16x8, ring[m % 3]), qf[dc], Sn[kb]);
      } else {
        const int j = m - NQK, cc = j / DB, db = j % DB;
        acc[db] = mfma32h(__builtin_bit_cast(f16x8, ring[m % 3]), P[cc], acc[db]);
      }
      const int slots = pv ? NQK + NPV : NQK;
      const int target = min(kPieces, (m + 1) * kPieces / slots);
      for (; done < target; ++done) piece(Sc, done);
      if (pv && m >= NQK && (m - NQK) % DB == DB - 1) {  // the last PV product that reads P[cc]
        const int cc = (m - NQK) / DB;
        for (; done < kExpBase + 4 * (cc + 1); ++done) piece(Sc, done);
        convert(Sc, cc);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, 6, 0);
    }
    for (; done < kPieces; ++done) piece(Sc, done);
    if (!pv) {
#pragma unroll
      for (int cc = 0; cc < NCC; ++cc) convert(Sc, cc);
    }
    // P of this tile is complete here (keeps its conversion from sinking
    // into the next iteration, away from the MFMAs it should overlap)
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc) asm volatile("" ::"v"(P[cc]));
    if (COLS) {                                           // this tile's per-key sums (S is free now)
      const float cs = col_reduce<NKB>(Sc, lane);
      const int idx = NKB == 2 ? c : c >> 1, kb = idx >> 4, e = idx & 15;
      if (NKB == 2 || (c & 1) == 0) scol[((t & 1) * NW + wave) * KT + kb * 32 + 8 * (e >> 2) + 4 * hh + (e & 3)] = cs;
    }
    flush_k();
    if (!NOPV) flush_v();
    store_kx(t + 2);
    __syncthreads();
    resc_prev = resc_cur;
    alpha_prev = alpha_cur;
  };
  // a wave past its own tiles: the PV product of its last tile (whose V
  // buffer is overwritten only at the end of the next step), then staging
  auto idle = [&](int t) {
    if (!NOPV && t == my_n && my_n > 0) {
      if (resc_prev) rescale(alpha_prev);
      pv_acc((t - 1) & 1, P);
    }
    load_k(t & 1, min(t + 2, n_tiles - 1));
    if (!NOPV) load_v(t & 1, t);
    flush_k();
    if (!NOPV) flush_v();
    store_kx(t + 2);
    __syncthreads();
  };
  auto run = [&](int t, f32x16 (&Sc)[NKB], f32x16 (&Sn)[NKB], bool first) {
    if (!WLIM || t < my_n) step(t, Sc, Sn, first);
    else idle(t);
  };
  run(0, S0, S1, true);
  int t = 1;
  for (; t + 1 < n_tiles; t += 2) {
    run(t, S1, S0, false);
    run(t + 1, S0, S1, false);
  }
  if (t < n_tiles) run(t, S1, S0, false);
  if (COLS) col_store(n_tiles - 1);                        // the last tile's sums
  if (NOPV || (WLIM && my_n < n_tiles)) return;
  if (resc_prev) rescale(alpha_prev);                      // PV of the last tile
  pv_acc((n_tiles - 1) & 1, P);
}

// MIX (lazy only): the mixture formula o = m*otilde + (1-m)*o_prev; the
// previous-loop pass then needs only the mass.
// PAIR (full loops, 256-row shape): the rows are cut into 128-row halves and a
// workgroup takes half j on waves 0-3 and half (last - j) on waves 4-7, so
// every workgroup sees about the same number of causal (row, key) pairs.  A
// wave stops computing at its own rows' last key tile; waves w and w + 4
// share a SIMD, so once the early half is done the late half runs alone
// there.  Used when the grid is a single round of workgroups, whose time is
// otherwise that of the last row tile.
template <int D, int NW, int KT_, bool LAZY, bool MIX = false, bool PAIR = false>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW), amdgpu_waves_per_eu(2))) void k_mfma_fwd(int32_t H, int32_t N, MfmaArgs a) {
  using T = FwdTiles<D, NW, KT_>;
  constexpr int KT = T::KT;
  constexpr int DC = D / 16, DB = D / 32;
  constexpr int ROWS = 32 * NW;
  __shared__ __attribute__((aligned(16))) uint16_t sk[2][T::KBUF];
  __shared__ __attribute__((aligned(16))) uint16_t sv[2][T::VBUF];
  __shared__ __attribute__((aligned(16))) int skx[4][KT];
  __shared__ int s_last, s_arrived;
  __shared__ int s_wcount[NW];
  __shared__ float scol[LAZY ? 2 * NW * KT : 1];          // lazy: the previous-loop pass's column sums
  constexpr int NT = 64 * NW;
  // the key split serves full loops in the 256-row, 64-key-tile shape
  constexpr bool kSplit = !LAZY && ROWS == 256 && KT == 64 && !PAIR;
  static_assert(!PAIR || (!LAZY && ROWS == 256 && KT == 64), "paired halves: full loops, 256-row shape");

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hh = lane >> 5, c = lane & 31;
  int sh, qtile, item = 0, part = 0, parts = 1, lrole = 0;
  int r0, wg_last;                                         // first row of this wave, last row of the workgroup
  if (PAIR) {
    int j;
    if (!map_block(a.n_sh, a.fpair, sh, j)) return;
    const int halves = (a.n_rows + 127) / 128, late = halves - 1 - j;
    r0 = wave < 4 ? j * 128 + wave * 32 : late == j ? a.n_rows : late * 128 + (wave - 4) * 32;
    wg_last = min(a.n_rows, (late + 1) * 128) - 1;
  } else if (kSplit && a.fsplit_u > 0) {
    // workgroups in launch order: row tiles heaviest first, the parts of a
    // tile one after another
    int rev;
    if (!map_block(a.n_sh, a.f_items, sh, rev)) return;
    item = a.f_items - 1 - rev;
    int i = item;
    for (qtile = a.f_tiles - 1;; --qtile) {
      const int kt = (min(a.n_rows, ROWS * (qtile + 1)) + KT - 1) / KT;
      parts = (kt + a.fsplit_u - 1) / a.fsplit_u;
      if (i < parts || qtile == 0) break;
      i -= parts;
    }
    part = i;
  } else if (LAZY && a.lmass) {
    if (!map_split(a.n_sh, a.f_tiles, sh, qtile, lrole)) return;
  } else if (!map_block(a.n_sh, (a.n_rows + ROWS - 1) / ROWS, sh, qtile)) {
    return;
  }
  if (!PAIR) {
    r0 = qtile * ROWS + wave * 32;
    wg_last = min(a.n_rows, (qtile + 1) * ROWS) - 1;
  }
  const int s = sh / H, h = sh % H;
  if (a.exited(s)) return;
  const int r = r0 + c;
  const bool vrow = r < a.n_rows;
  const int tok = vrow ? row_token(a, s, r) : -1;         // -1: every key is masked
  const bool blk_full = r0 + 31 < a.n_rows;
  const int tok_first = row_token(a, s, min(r0, a.n_rows - 1));
  const int tok_last = row_token(a, s, min(r0 + 31, a.n_rows - 1));
  const float c1 = a.scale * kLog2e;                      // logits in log2 units

  const int32_t* kx = a.kidx + static_cast<int64_t>(sh) * a.n_keys_pad;
  // key slots visible to a row: those with a token at or before its own
  auto visible = [&](int row) {
    const int last_tok = row_token(a, s, row);
    int lo = 0, hi = a.n_keys;
    while (lo < hi) { const int mid = (lo + hi) >> 1; if (kx[mid] <= last_tok) lo = mid + 1; else hi = mid; }
    return lo;
  };
  int my_n = 0, n_vis;                                     // PAIR: this wave's own key tiles
  if (PAIR) {
    if (lane == 0) s_wcount[wave] = r0 < a.n_rows ? visible(min(r0 + 31, a.n_rows - 1)) : 0;
    __syncthreads();
    n_vis = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) n_vis = max(n_vis, s_wcount[w]);
    my_n = (s_wcount[wave] + KT - 1) / KT;
  } else {
    if (tid == 0) s_last = visible(wg_last);               // key slots visible to the workgroup's last row
    __syncthreads();
    n_vis = s_last;
  }
  const int n_tiles = (n_vis + KT - 1) / KT;

  const int64_t rows_q = a.q_compact ? a.n_rows : N;
  const int64_t qr = a.q_compact ? r : tok;
  auto load_q = [&](const void* src, bf16x8 (&qf)[DC]) {
    const uint16_t* p = static_cast<const uint16_t*>(src) + ((static_cast<int64_t>(s) * rows_q + qr) * H + h) * D + 8 * hh;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) qf[dc] = vrow ? *reinterpret_cast<const bf16x8*>(p + dc * 16) : bf16x8{};
  };
  const int64_t rows_o = a.o_compact ? a.n_rows : N;
  const int64_t orow = a.o_compact ? r : tok;
  float* lse_ptr = a.lse + (static_cast<int64_t>(s) * rows_o + orow) * H + h;
  float* o_ptr = a.o + ((static_cast<int64_t>(s) * rows_o + orow) * H + h) * D;
  float* st_ptr = a.stat + (static_cast<int64_t>(sh) * a.n_rows + r) * 4;
  const int64_t kofs = static_cast<int64_t>(sh) * a.n_keys_pad * D;

  bf16x8 qf[DC];
  f32x16 acc[DB];
  float ref, lsum;
  if (!LAZY) {
    load_q(a.q_cur, qf);
    // a part covers key tiles [t_lo, t_hi) of the row tile
    const int t_lo = part * n_tiles / parts, t_hi = (part + 1) * n_tiles / parts;
    fwd_pass<D, NW, KT_, false, false, PAIR>(a, t_hi - t_lo, a.kc + kofs + static_cast<int64_t>(t_lo) * KT * D,
                                              a.vtc + kofs + t_lo * KT, kx + t_lo * KT, sk, sv, skx, qf, tok,
                                              tok_first, tok_last, blk_full, c1, 0.0f, acc, ref, lsum, my_n);
    if (kSplit && parts > 1) {
      // every part stores its partial state (acc against its own reference
      // max, the max, the lane's sum); the part that finishes last merges all
      // of them in part order (the result does not depend on which one it is).
      // All parts of a head run on one XCD (map_block), whose L2 every CU
      // shares and every CU's vector L1 writes through to: a part's stores
      // are in that L2 once acknowledged (s_waitcnt before the count), and
      // the merging part reads them past its own L1 (device-scope loads).  No
      // L2 writeback or invalidate is needed, which would evict the K/V
      // tiles the other row tiles of the head are streaming.
      constexpr int SLOT = (D / 8 + 1) * NT;
      float4* mine = a.fpart + (static_cast<int64_t>(sh) * a.f_items + item) * SLOT;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          mine[(db * 4 + q4) * NT + tid] =
              make_float4(acc[db][4 * q4], acc[db][4 * q4 + 1], acc[db][4 * q4 + 2], acc[db][4 * q4 + 3]);
      mine[(D / 8) * NT + tid] = make_float4(ref, lsum, 0.0f, 0.0f);
      __builtin_amdgcn_s_waitcnt(0);                       // this lane's stores acknowledged
      __syncthreads();
      int32_t* cnt = a.fcount + static_cast<int64_t>(sh) * a.f_tiles + qtile;
      int32_t* xmask = cnt + static_cast<int64_t>(a.n_sh) * a.f_tiles;
      const uint32_t xbit = xcd_bit(a, part);
      if (tid == 0) {
        __hip_atomic_fetch_or(xmask, static_cast<int32_t>(xbit), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0);
        s_arrived = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();
      if (s_arrived != parts - 1) return;
      if (tid == 0) xcd_check(a, xmask, xbit);
      auto ld4 = [](const float4* q) {
        const float* f = reinterpret_cast<const float*>(q);
        return make_float4(__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                           __hip_atomic_load(f + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                           __hip_atomic_load(f + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                           __hip_atomic_load(f + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      };
      const float4* first = a.fpart + (static_cast<int64_t>(sh) * a.f_items + item - part) * SLOT;
      for (int j = 0; j < parts; ++j) {
        const float4* pj = first + static_cast<int64_t>(j) * SLOT;
        const float4 st = ld4(pj + (D / 8) * NT + tid);
        const float m = j == 0 ? st.x : fmaxf(ref, st.x);
        const float w_run = (j == 0 || ref == -INFINITY) ? 0.0f : ex2(ref - m);
        const float w_new = st.x == -INFINITY ? 0.0f : ex2(st.x - m);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const float4 v = ld4(pj + (db * 4 + q4) * NT + tid);
            acc[db][4 * q4 + 0] = fmaf(w_new, v.x, w_run * acc[db][4 * q4 + 0]);
            acc[db][4 * q4 + 1] = fmaf(w_new, v.y, w_run * acc[db][4 * q4 + 1]);
            acc[db][4 * q4 + 2] = fmaf(w_new, v.z, w_run * acc[db][4 * q4 + 2]);
            acc[db][4 * q4 + 3] = fmaf(w_new, v.w, w_run * acc[db][4 * q4 + 3]);
          }
        lsum = fmaf(w_new, st.y, w_run * lsum);
        ref = m;
      }
    }
    const float l_tot = lsum + __shfl_xor(lsum, 32, 64);
    if (vrow && l_tot > 0.0f) {
      const float inv = 1.0f / l_tot;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int dim = db * 32 + 8 * q4 + 4 * hh;
          *reinterpret_cast<float4*>(o_ptr + dim) =
              make_float4(acc[db][4 * q4] * inv, acc[db][4 * q4 + 1] * inv, acc[db][4 * q4 + 2] * inv,
                          acc[db][4 * q4 + 3] * inv);
        }
      if (hh == 0) {
        const float b = ref + __log2f(l_tot);              // lse in log2 units
        *lse_ptr = b * kLn2;
        *reinterpret_cast<float4*>(st_ptr) = make_float4(b, b, 1.0f, __int_as_float(tok));
      }
    }
    return;
  }
  // lazy: pass 1 over the previous loop's keys with the fixed normaliser
  // lse_prev gives the mass m and contribution a; o_prev - a is written back
  // at once, and pass 2 (current loop, online softmax) adds m * otilde.
  const float b_prev = vrow ? a.lse[(static_cast<int64_t>(s) * rows_o + orow) * H + h] * kLog2e : 0.0f;
  // the previous-loop probabilities' per-key sums over this row tile's rows
  float* col_dst = a.pcol + (static_cast<int64_t>(sh) * ((a.n_rows + ROWS - 1) / ROWS) + qtile) * a.n_keys_pad;
  // o <- o_prev - a (or (1 - m) o_prev), from o as read by ld
  auto prev_update = [&](bool valid, float m, auto ld) {
    if (!valid) return;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int dim = db * 32 + 8 * q4 + 4 * hh;
        float4 op = ld(o_ptr + dim);
        if (MIX) {
          const float keep = 1.0f - m;
          op.x *= keep; op.y *= keep; op.z *= keep; op.w *= keep;
        } else {
          op.x -= acc[db][4 * q4 + 0];
          op.y -= acc[db][4 * q4 + 1];
          op.z -= acc[db][4 * q4 + 2];
          op.w -= acc[db][4 * q4 + 3];
        }
        *reinterpret_cast<float4*>(o_ptr + dim) = op;
      }
  };
  // o <- o + (m / z) acc, the new lse and the row statistics
  auto cur_finish = [&](bool valid, float m, float z, auto ld) {
    if (valid) {
      const float f = z > 0.0f ? m / z : 0.0f;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int dim = db * 32 + 8 * q4 + 4 * hh;
          float4 op = ld(o_ptr + dim);
          op.x = fmaf(f, acc[db][4 * q4 + 0], op.x);
          op.y = fmaf(f, acc[db][4 * q4 + 1], op.y);
          op.z = fmaf(f, acc[db][4 * q4 + 2], op.z);
          op.w = fmaf(f, acc[db][4 * q4 + 3], op.w);
          *reinterpret_cast<float4*>(o_ptr + dim) = op;
        }
    }
    if (vrow && hh == 0) {
      // new lse in log2 units: M + log2 Z - log2 m
      const float b = valid ? ref + __log2f(z) - __log2f(m) : b_prev;
      if (valid) *lse_ptr = b * kLn2;
      *reinterpret_cast<float4*>(st_ptr) =
          make_float4(valid ? b_prev : INFINITY, valid ? b : INFINITY, valid ? 1.0f : 0.0f, __int_as_float(tok));
    }
  };
  auto ld_plain = [](const float* p) { return *reinterpret_cast<const float4*>(p); };
  if (a.lmass) {
    // The two passes as two workgroups of one XCD (map_block: whole heads
    // per XCD).  The previous-loop pass writes o_prev - a and m at once; the
    // workgroup that ends last applies the current-loop pass, from its own
    // registers or from the partial (acc, max, sum) the current-loop pass
    // stored.  Stores are acknowledged before the arrival count, and the
    // other workgroup's data is read past this CU's L1 (device-scope loads).
    constexpr int SLOT = (D / 8 + 1) * NT;
    int32_t* cnt = a.fcount + static_cast<int64_t>(sh) * a.f_tiles + qtile;
    int32_t* xmask = cnt + static_cast<int64_t>(a.n_sh) * a.f_tiles;
    float4* part = a.fpart + (static_cast<int64_t>(sh) * a.f_tiles + qtile) * SLOT;
    float* mrow = a.lmass + static_cast<int64_t>(sh) * a.n_rows + r;
    const uint32_t xbit = xcd_bit(a, lrole);
    auto arrive = [&]() {
      __builtin_amdgcn_s_waitcnt(0);                       // this lane's stores acknowledged
      __syncthreads();
      if (tid == 0) {
        __hip_atomic_fetch_or(xmask, static_cast<int32_t>(xbit), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0);
        s_arrived = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();
      return s_arrived;
    };
    float m;
    bool valid;
    if (lrole == 1) {
      load_q(a.q_prev, qf);
      fwd_pass<D, NW, KT_, true, MIX, false, true>(a, n_tiles, a.kp + kofs, a.vtp + kofs, kx, sk, sv, skx, qf, tok,
                                                   tok_first, tok_last, blk_full, c1, b_prev, acc, ref, lsum, 0,
                                                   col_dst, scol);
      m = lsum + __shfl_xor(lsum, 32, 64);
      valid = vrow && m > 0.0f;
      prev_update(valid, m, ld_plain);
      if (vrow && hh == 0) *mrow = m;
      if (arrive() == 0) return;                           // the current-loop pass ends the tile
      if (tid == 0) xcd_check(a, xmask, xbit);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 v = ld4_agent(part + (db * 4 + q4) * NT + tid);
          acc[db][4 * q4 + 0] = v.x; acc[db][4 * q4 + 1] = v.y;
          acc[db][4 * q4 + 2] = v.z; acc[db][4 * q4 + 3] = v.w;
        }
      const float4 st = ld4_agent(part + (D / 8) * NT + tid);
      ref = st.x;
      lsum = st.y;
    } else {
      load_q(a.q_cur, qf);
      fwd_pass<D, NW, KT_, false>(a, n_tiles, a.kc + kofs, a.vtc + kofs, kx, sk, sv, skx, qf, tok, tok_first,
                                  tok_last, blk_full, c1, 0.0f, acc, ref, lsum);
      if (tid == 0) s_arrived = __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      if (s_arrived == 0) {                                // the previous-loop pass still runs: leave a partial
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            part[(db * 4 + q4) * NT + tid] =
                make_float4(acc[db][4 * q4], acc[db][4 * q4 + 1], acc[db][4 * q4 + 2], acc[db][4 * q4 + 3]);
        part[(D / 8) * NT + tid] = make_float4(ref, lsum, 0.0f, 0.0f);
        if (arrive() == 0) return;                         // the previous-loop pass ends the tile
      }
      if (tid == 0) xcd_check(a, xmask, xbit);
      m = vrow ? __hip_atomic_load(mrow, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0.0f;
      valid = vrow && m > 0.0f;
    }
    cur_finish(valid, m, lsum + __shfl_xor(lsum, 32, 64), ld4_agent_f);
    return;
  }
  load_q(a.q_prev, qf);
  fwd_pass<D, NW, KT_, true, MIX, false, true>(a, n_tiles, a.kp + kofs, a.vtp + kofs, kx, sk, sv, skx, qf, tok,
                                               tok_first, tok_last, blk_full, c1, b_prev, acc, ref, lsum, 0, col_dst,
                                               scol);
  const float m = lsum + __shfl_xor(lsum, 32, 64);
  const bool valid = vrow && m > 0.0f;
  prev_update(valid, m, ld_plain);
  __syncthreads();                                         // pass 2 reuses the tile buffers
  load_q(a.q_cur, qf);
  fwd_pass<D, NW, KT_, false>(a, n_tiles, a.kc + kofs, a.vtc + kofs, kx, sk, sv, skx, qf, tok, tok_first, tok_last,
                         blk_full, c1, 0.0f, acc, ref, lsum);
  cur_finish(valid, m, lsum + __shfl_xor(lsum, 32, 64), ld_plain);
}

// --------------------------------------------------------------------------- colmass
// Key-major: a wave owns 32 key slots (K^ rows in registers, keys in lanes so
// that column sums are lane-local) and streams tiles of 64 query rows through
// LDS; S = Q K^T on the MFMA, p = 2^(s*c1 - b) with the row's final base-2
// normaliser b, summed per key in a fixed order.  The kernel is bound by its
// vector work (one exponential per pair), and four waves per SIMD overlap one
// wave's exponentials with another's MFMAs, so a wave computes a tile's
// logits and then its exponentials (a per-wave pipeline held a second logit
// tile and cost more registers and copies than it hid).  A lazy loop adds
// the current probabilities and subtracts the previous loop's, which the
// forward's fixed-normaliser pass already summed per key and row tile (it
// holds them in registers, so the logits and exponentials of version v-1 are
// not computed twice).  The rows can be split over several workgroups, whose
// per-key partial sums a second kernel adds in a fixed order.
//
// stat rows hold (b_prev, b_cur, valid, token); rows that did not update
// carry b = +inf so that their probabilities vanish.
template <int D>
struct ColTiles {
  static constexpr int QT = 64;
  static constexpr int NT = 512;
  static constexpr int QS = D + 8;
  static constexpr int QCH = QT * D / 8;
  static constexpr int QPER = (QCH + NT - 1) / NT;
};

template <int D>
__device__ __forceinline__ void col_pass(const MfmaArgs& a, int s, int sh, int H, int N, int r_begin, int r_end,
                                         const void* qsrc, const uint16_t* krow, int kj, int kmax,
                                         uint16_t (*sq)[ColTiles<D>::QT * ColTiles<D>::QS], float (*sb)[64],
                                         int (*stok)[64], float c1, float& acc) {
  using T = ColTiles<D>;
  constexpr int QT = T::QT, NT = T::NT, QS = T::QS;
  constexpr int DC = D / 16;
  const int tid = threadIdx.x, lane = tid & 63;
  const int hh = lane >> 5, c = lane & 31;
  const int n_tiles = (r_end - r_begin + QT - 1) / QT;
  if (n_tiles <= 0) return;
  bf16x8 kf[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) kf[dc] = *reinterpret_cast<const bf16x8*>(krow + dc * 16);
  const int64_t rows_q = a.q_compact ? a.n_rows : N;

  u32x4 pq[T::QPER];
  float pb = INFINITY;
  int ptok = -1;
  // branch-free: rows past the range are read clamped and then neutralised
  // this lane's chunk of a query row, and the distance between rows
  const uint16_t* qlane = static_cast<const uint16_t*>(qsrc) + (static_cast<int64_t>(s) * rows_q * H + (sh % H)) * D +
                          (tid % (D / 8)) * 8;
  const int64_t qstride = static_cast<int64_t>(H) * D;
  // Loads of a tile are issued early and used only when the tile is stored,
  // at the end of the iteration (rows past the range, read clamped, are
  // neutralised there), so a wave does not wait for them before its own work.
  // The query rows' positions (row index, or token with by-token queries) of
  // a tile are read one iteration before its query loads, so that those do
  // not wait on a dependent load.
  int qrow[T::QPER];
  auto rload = [&](int tile) {
    const int q0 = r_begin + tile * QT;
#pragma unroll
    for (int i = 0; i < T::QPER; ++i) {
      const int ch = min(tid + NT * i, T::QCH - 1);         // a partial last round repeats the last chunk
      const int rc = min(q0 + ch / (D / 8), r_end - 1);
      qrow[i] = a.q_compact ? rc : row_token(a, s, rc);
    }
  };
  auto gload = [&](int tile) {                              // the tile whose rows rload read last
    const int q0 = r_begin + tile * QT;
#pragma unroll
    for (int i = 0; i < T::QPER; ++i) {
      const int ch = min(tid + NT * i, T::QCH - 1);
      pq[i] = *reinterpret_cast<const u32x4*>(qlane + static_cast<int64_t>(qrow[i]) * qstride +
                                              (ch % (D / 8) - tid % (D / 8)) * 8);
    }
    const int rr = min(q0 + (tid & 63), r_end - 1);         // every wave reads the tile's row statistics
    const float4 st = *reinterpret_cast<const float4*>(a.stat + (static_cast<int64_t>(sh) * a.n_rows + rr) * 4);
    pb = st.y;
    ptok = __float_as_int(st.w);
  };
  // tile: the tile the last gload read, or a later one (past the end: never used)
  auto sstore = [&](int buf, int tile) {
    const int q0 = r_begin + tile * QT;
#pragma unroll
    for (int i = 0; i < T::QPER; ++i) {
      const int ch = min(tid + NT * i, T::QCH - 1);
      const bool ok = q0 + ch / (D / 8) < r_end;
      *reinterpret_cast<u32x4*>(&sq[buf][(ch / (D / 8)) * QS + (ch % (D / 8)) * 8]) = ok ? pq[i] : u32x4{0, 0, 0, 0};
    }
    const bool ok = q0 + (tid & 63) < r_end;
    sb[tile & 3][tid & 63] = ok ? pb : INFINITY;           // identical values from every wave
    stok[tile & 3][tid & 63] = ok ? ptok : -1;
  };
  auto qk = [&](int buf, f32x16 (&S)[2]) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      S[qb] = f32x16{};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const bf16x8 qa = *reinterpret_cast<const bf16x8*>(&sq[buf][(qb * 32 + c) * QS + dc * 16 + 8 * hh]);
        S[qb] = mfma32(qa, kf[dc], S[qb]);
      }
    }
  };
  // pairs (row, key) with the key after the row get logit -inf (wave-uniform test)
  auto mask = [&](int tile, f32x16 (&S)[2]) {
    const int slot = tile & 3;
    if (stok[slot][0] < kmax) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const i32x4 t4 = *reinterpret_cast<const i32x4*>(&stok[slot][qb * 32 + 8 * q4 + 4 * hh]);
#pragma unroll
          for (int k4 = 0; k4 < 4; ++k4)
            if (kj > t4[k4]) S[qb][4 * q4 + k4] = -INFINITY;
        }
    }
  };
  auto expsum = [&](int tile, const f32x16 (&S)[2]) {
    const int slot = tile & 3;
    float part = 0.0f;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 b4 = *reinterpret_cast<const float4*>(&sb[slot][qb * 32 + 8 * q4 + 4 * hh]);
        part += ex2(fmaf(S[qb][4 * q4 + 0], c1, -b4.x));
        part += ex2(fmaf(S[qb][4 * q4 + 1], c1, -b4.y));
        part += ex2(fmaf(S[qb][4 * q4 + 2], c1, -b4.z));
        part += ex2(fmaf(S[qb][4 * q4 + 3], c1, -b4.w));
      }
    acc += part;
  };

  rload(0);
  gload(0);
  sstore(0, 0);
  if (n_tiles > 1) { rload(1); gload(1); sstore(1, 1); }
  rload(min(2, n_tiles - 1));
  __syncthreads();
  // iteration t: logits and exponentials of tile t (the other waves of the
  // SIMD keep the matrix cores busy meanwhile); query tile t+2 is loaded and,
  // once every wave has read tile t's buffer, stored in its place, and the
  // row positions of tile t+3 are read.  Tile t+1 was stored one iteration
  // earlier, before that iteration's barrier.
  f32x16 S[2];
  for (int t = 0; t < n_tiles; ++t) {
    gload(min(t + 2, n_tiles - 1));
    rload(min(t + 3, n_tiles - 1));
    qk(t & 1, S);
    mask(t, S);
    expsum(t, S);
    asm volatile("" ::"v"(acc));
    __syncthreads();
    sstore(t & 1, t + 2);
  }
  __syncthreads();                                           // the buffers are reused by the next pass
}

// The workgroup's column sums (lane pair halves already added).  One row
// range: written at once.  Several: each range stores its partial sums; with
// a.ccount the range that finishes last adds them in range order and writes
// the column mass (all ranges of a head run on one XCD, whose L2 every CU
// shares: the stores are acknowledged before the count, and the sums are read
// past this CU's L1), otherwise k_colmass_reduce does.  Every thread of the
// workgroup calls it.
template <bool LAZY>
__device__ __forceinline__ void col_finish(const MfmaArgs& a, int N, int chunk, int sh, int kblk, int t, int kj,
                                           float acc, int* s_arrived, int n_parts) {
  const int tid = threadIdx.x, hh = (tid & 63) >> 5;
  if (a.col_chunks == 1) {
    if (hh == 0 && t < a.n_keys) {
      float* dst = a.colmass + static_cast<int64_t>(sh) * N + kj;
      if (LAZY) *dst += acc; else *dst = acc;
    }
    return;
  }
  if (hh == 0) a.col_part[(static_cast<int64_t>(chunk) * a.n_sh + sh) * a.n_keys_pad + t] = acc;
  if (!a.ccount) return;
  __builtin_amdgcn_s_waitcnt(0);                          // this lane's store acknowledged
  __syncthreads();
  int32_t* cnt = a.ccount + static_cast<int64_t>(sh) * (a.n_keys_pad / 256) + kblk;
  int32_t* xmask = cnt + static_cast<int64_t>(a.n_sh) * (a.n_keys_pad / 256);
  const uint32_t xbit = xcd_bit(a, chunk);
  if (tid == 0) {
    __hip_atomic_fetch_or(xmask, static_cast<int32_t>(xbit), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);
    *s_arrived = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (*s_arrived != n_parts - 1) return;
  if (tid == 0) xcd_check(a, xmask, xbit);
  if (tid >= 256) return;
  const int tk = kblk * 256 + tid;
  if (tk >= a.n_keys) return;
  float sum = 0.0f;
  for (int ch = 0; ch < n_parts; ++ch)
    sum += __hip_atomic_load(a.col_part + (static_cast<int64_t>(ch) * a.n_sh + sh) * a.n_keys_pad + tk,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  float* dst = a.colmass + static_cast<int64_t>(sh) * N + a.kidx[static_cast<int64_t>(sh) * a.n_keys_pad + tk];
  if (LAZY) *dst += sum; else *dst = sum;
}

template <int D, bool LAZY>
__global__ __attribute__((amdgpu_flat_work_group_size(1, 512), amdgpu_waves_per_eu(4))) void k_mfma_colmass(int32_t H, int32_t N, MfmaArgs a) {
  using T = ColTiles<D>;
  constexpr int QT = T::QT;
  constexpr int KB = 256;                                    // key slots per workgroup (8 waves x 32)
  __shared__ __attribute__((aligned(16))) uint16_t sq[2][QT * T::QS];
  __shared__ __attribute__((aligned(16))) float sb[4][64];
  __shared__ __attribute__((aligned(16))) int stok[4][64];
  __shared__ int s_start;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hh = lane >> 5, c = lane & 31;
  const int n_kblk = a.n_keys_pad / KB;
  int sh, item;
  if (!map_block(a.n_sh, n_kblk * a.col_chunks, sh, item)) return;
  const int chunk = item % a.col_chunks;
  const int kblk = n_kblk - 1 - item / a.col_chunks;        // early keys see the most rows: start them first
  const int s = sh / H;
  if (a.exited(s)) return;
  const int t0 = kblk * KB + wave * 32;
  const int t = t0 + c;
  const int32_t* kx = a.kidx + static_cast<int64_t>(sh) * a.n_keys_pad;
  const int kj = kx[t];                                      // INT_MAX for padding
  const int kmax = kx[min(t0 + 31, a.n_keys - 1)];           // largest real key of this wave
  const float c1 = a.scale * kLog2e;
  if (tid == 0) {                                            // first row that sees the block's first key
    const int kfirst = kx[kblk * KB];
    int lo = 0, hi = a.n_rows;
    while (lo < hi) { const int mid = (lo + hi) >> 1; if (row_token(a, s, mid) < kfirst) lo = mid + 1; else hi = mid; }
    s_start = lo;
  }
  __syncthreads();
  const int c_lo = chunk * a.col_rows;
  const int r_end = min(a.n_rows, c_lo + a.col_rows);
  const int r_begin = max(c_lo, (s_start / QT) * QT);
  const int64_t kofs = (static_cast<int64_t>(sh) * a.n_keys_pad + t) * D + 8 * hh;
  float acc = 0.0f;
  col_pass<D>(a, s, sh, H, N, r_begin, r_end, a.q_cur, a.kc + kofs, kj, kmax, sq, sb, stok, c1, acc);
  if (LAZY && hh == 0) {
    // the previous loop's probabilities, summed by the forward per row tile,
    // are subtracted: each range takes the tiles that start in it, in order
    // (a tile whose last row precedes the key saw none of it, and its entry
    // was not written)
    const int pr = a.pcol_rows, rt = (a.n_rows + pr - 1) / pr;
    const int t_lo = (c_lo + pr - 1) / pr, t_hi = min(rt, (min(a.n_rows, c_lo + a.col_rows) + pr - 1) / pr);
    const float* pc = a.pcol + static_cast<int64_t>(sh) * rt * a.n_keys_pad + t;
    float prev = 0.0f;
#pragma unroll 4
    for (int r = t_lo; r < t_hi; ++r) {
      const float v = pc[static_cast<int64_t>(r) * a.n_keys_pad];
      prev += kj <= row_token(a, s, min((r + 1) * pr, a.n_rows) - 1) ? v : 0.0f;
    }
    acc -= prev;
  }
  acc += __shfl_xor(acc, 32, 64);
  if (hh != 0) return;
  if (a.col_chunks > 1) {                                    // added by k_colmass_reduce
    a.col_part[(static_cast<int64_t>(chunk) * a.n_sh + sh) * a.n_keys_pad + t] = acc;
  } else if (t < a.n_keys) {
    float* dst = a.colmass + static_cast<int64_t>(sh) * N + kj;
    if (LAZY) *dst += acc; else *dst = acc;
  }
}

// Full loops: the same key-major layout in a plain double-buffered loop (no
// second pass, small register footprint: four waves per SIMD hide the
// exponentials behind the other waves' MFMAs).
template <int D>
__global__ __launch_bounds__(512, 1) void k_colmass_full_rows(int32_t H, int32_t N, MfmaArgs a) {
  constexpr int QT = 64;
  constexpr int DC = D / 16;
  constexpr int QS = D + 8;
  constexpr int NT = 512;                                  // 8 waves x 32 keys
  constexpr int KB = 256;                                  // key slots per workgroup
  constexpr int QCH = QT * D / 8;                          // 16-B chunks of one Q tile
  constexpr int PER = (QCH + NT - 1) / NT;
  __shared__ __attribute__((aligned(16))) uint16_t sq[2][QT * QS];
  __shared__ __attribute__((aligned(16))) float sb[2][QT];
  __shared__ __attribute__((aligned(16))) int stok[2][QT];
  __shared__ int s_start, s_arrived;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hh = lane >> 5, c = lane & 31;
  const int n_kblk = a.n_keys_pad / KB;
  int sh, item, chunk, kblk, c_lo, n_parts;
  if (a.col_var_rows > 0) {
    // items heavy first: key blocks in order, each block's ranges in order
    if (!map_block(a.n_sh, a.col_items, sh, item)) return;
    int rem = a.col_items - 1 - item;
    for (kblk = 0;; ++kblk) {
      n_parts = (a.n_rows - kblk * KB + a.col_var_rows - 1) / a.col_var_rows;
      if (rem < n_parts || kblk == n_kblk - 1) break;
      rem -= n_parts;
    }
    chunk = rem;
    c_lo = kblk * KB + chunk * a.col_var_rows;
  } else {
    if (!map_block(a.n_sh, n_kblk * a.col_chunks, sh, item)) return;
    chunk = item % a.col_chunks;
    kblk = n_kblk - 1 - item / a.col_chunks;              // early keys see the most rows: start them first
    c_lo = chunk * a.col_rows;
    n_parts = a.col_chunks;
  }
  const int c_rows = a.col_var_rows > 0 ? a.col_var_rows : a.col_rows;
  const int s = sh / H, h = sh % H;
  if (a.exited(s)) return;
  const int t0 = kblk * KB + wave * 32;
  const int t = t0 + c;
  const int32_t* kx = a.kidx + static_cast<int64_t>(sh) * a.n_keys_pad;
  const int kj = kx[t];                                    // INT_MAX for padding
  const int kmax = kx[min(t0 + 31, a.n_keys - 1)];         // largest real key of this wave
  const float c1 = a.scale * kLog2e;

  bf16x8 kf[DC];
  {
    const uint16_t* kb = a.kc + (static_cast<int64_t>(sh) * a.n_keys_pad + t) * D + 8 * hh;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) kf[dc] = *reinterpret_cast<const bf16x8*>(kb + dc * 16);
  }
  if (tid == 0) {                                          // first row that sees the block's first key
    const int kfirst = kx[kblk * KB];
    int lo = 0, hi = a.n_rows;
    while (lo < hi) { const int mid = (lo + hi) >> 1; if (row_token(a, s, mid) < kfirst) lo = mid + 1; else hi = mid; }
    s_start = lo;
  }
  __syncthreads();
  const int r_end = min(a.n_rows, c_lo + c_rows);
  const int r_begin = max(c_lo, (s_start / QT) * QT);
  const int n_tiles = r_end > r_begin ? (r_end - r_begin + QT - 1) / QT : 0;
  const int64_t rows_q = a.q_compact ? a.n_rows : N;
  const uint16_t* q = static_cast<const uint16_t*>(a.q_cur);

  u32x4 pre[PER];
  float pre_b = INFINITY;
  int pre_tok = -1;
  auto gload = [&](int q0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int ch = tid + NT * i;
      const int rr = q0 + ch / (D / 8);
      pre[i] = u32x4{0, 0, 0, 0};
      if (ch < QCH && rr < r_end) {
        const int64_t qr = a.q_compact ? rr : row_token(a, s, rr);
        pre[i] = *reinterpret_cast<const u32x4*>(q + ((static_cast<int64_t>(s) * rows_q + qr) * H + h) * D +
                                                 (ch % (D / 8)) * 8);
      }
    }
    if (tid < QT) {
      const int rr = q0 + tid;
      pre_b = INFINITY;
      pre_tok = -1;
      if (rr < r_end) {
        const float4 st = *reinterpret_cast<const float4*>(a.stat + (static_cast<int64_t>(sh) * a.n_rows + rr) * 4);
        pre_b = st.y;
        pre_tok = __float_as_int(st.w);
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int ch = tid + NT * i;
      if (ch < QCH) *reinterpret_cast<u32x4*>(&sq[buf][(ch / (D / 8)) * QS + (ch % (D / 8)) * 8]) = pre[i];
    }
    if (tid < QT) { sb[buf][tid] = pre_b; stok[buf][tid] = pre_tok; }
  };
  if (n_tiles > 0) {
    gload(r_begin);
    sstore(0);
  }
  __syncthreads();
  float acc = 0.0f;
  for (int it = 0; it < n_tiles; ++it) {
    const int buf = it & 1;
    const int q0 = r_begin + it * QT;
    if (it + 1 < n_tiles) gload(q0 + QT);
    // the tile's products and exponentials; MASKED: the key after the row
    // contributes nothing (rows past the range carry b = +inf, so their
    // exponentials are 0 either way)
    auto tile = [&](auto masked) {
      constexpr bool MASKED = decltype(masked)::value;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        f32x16 sc = f32x16{};
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
          const bf16x8 qa = *reinterpret_cast<const bf16x8*>(&sq[buf][(qb * 32 + c) * QS + dc * 16 + 8 * hh]);
          sc = mfma32(qa, kf[dc], sc);
        }
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int row0 = qb * 32 + 8 * q4 + 4 * hh;
          const float4 bc = *reinterpret_cast<const float4*>(&sb[buf][row0]);
          const float bcv[4] = {bc.x, bc.y, bc.z, bc.w};
          int tkv[4] = {};
          if (MASKED) {
            const int4 tk = *reinterpret_cast<const int4*>(&stok[buf][row0]);
            tkv[0] = tk.x; tkv[1] = tk.y; tkv[2] = tk.z; tkv[3] = tk.w;
          }
#pragma unroll
          for (int k4 = 0; k4 < 4; ++k4) {
            const float v = ex2(fmaf(sc[4 * q4 + k4], c1, -bcv[k4]));
            acc += (MASKED && kj > tkv[k4]) ? 0.0f : v;
          }
        }
      }
    };
    // wave-uniform: some row of the tile precedes the wave's last key
    if (__builtin_amdgcn_readfirstlane(stok[buf][0] < kmax ? 1 : 0)) tile(std::true_type{});
    else tile(std::false_type{});
    if (it + 1 < n_tiles) sstore(buf ^ 1);
    __syncthreads();
  }
  acc += __shfl_xor(acc, 32, 64);
  col_finish<false>(a, N, chunk, sh, kblk, t, kj, acc, &s_arrived, n_parts);
}

// Sums the per-chunk partial column masses in chunk order.
template <bool LAZY>
__global__ __launch_bounds__(256) void k_colmass_reduce(int32_t N, MfmaArgs a) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<int64_t>(a.n_sh) * a.n_keys_pad) return;
  const int sh = static_cast<int>(i / a.n_keys_pad), t = static_cast<int>(i % a.n_keys_pad);
  if (t >= a.n_keys || a.exited(sh / a.heads)) return;
  float acc = 0.0f;
  for (int ch = 0; ch < a.col_chunks; ++ch) acc += a.col_part[(static_cast<int64_t>(ch) * a.n_sh) * a.n_keys_pad + i];
  float* dst = a.colmass + static_cast<int64_t>(sh) * N + a.kidx[i];
  if (LAZY) *dst += acc; else *dst = acc;
}

// --------------------------------------------------------------------------- launch
// FLASHLOOP_TEST_XCD_SPLIT=1 makes the split reductions' XCD check see
// different XCDs for odd and even parts, so that a test can see the check
// report (the results themselves are unaffected).
static int32_t xcd_test_flag() {
  const char* e = getenv("FLASHLOOP_TEST_XCD_SPLIT");
  return e && e[0] == '1';
}

template <int D>
static hipError_t launch_d(const fl_attend_args& x, const KvView& kv, const AttendPlan& p, hipStream_t st) {
  const bool lazy = x.mode == FL_ATTEND_LAZY;
  MfmaArgs a{};
  a.act = x.active_idx;
  a.n_rows = x.n_active;
  a.q_cur = x.q_cur; a.q_prev = x.q_prev;
  a.q_compact = x.q_layout == FL_ROWS_COMPACT; a.o_compact = x.o_layout == FL_ROWS_COMPACT;
  a.o = x.o; a.lse = x.lse; a.colmass = x.colmass;
  a.key_idx = lazy ? x.key_idx : nullptr;
  a.n_keys = static_cast<int32_t>(p.keys);
  a.n_keys_pad = static_cast<int32_t>((p.keys + 255) / 256 * 256);
  a.version = x.version;
  a.scale = 1.0f / sqrtf(static_cast<float>(D));
  uint8_t* ws = static_cast<uint8_t*>(x.workspace);
  const uint64_t sh = static_cast<uint64_t>(kv.n_seq) * kv.H;
  const uint64_t kbytes = sh * a.n_keys_pad * D * 2;
  a.kc = reinterpret_cast<uint16_t*>(ws + p.off_gather);
  a.vtc = reinterpret_cast<uint16_t*>(ws + p.off_gather + kbytes);
  a.kp = reinterpret_cast<uint16_t*>(ws + p.off_gather + 2 * kbytes);
  a.vtp = reinterpret_cast<uint16_t*>(ws + p.off_gather + 3 * kbytes);
  a.kidx = reinterpret_cast<int32_t*>(ws + p.off_gather + (lazy ? 4 : 2) * kbytes);
  a.stat = reinterpret_cast<float*>(ws + p.off_stat);

  a.n_sh = static_cast<int32_t>(sh);
  a.heads = kv.H;
  // set before the gather launch, which zeroes the counters
  a.ccount = p.col_fused ? reinterpret_cast<int32_t*>(ws + p.off_ccount) : nullptr;
  a.exit_flags = kv.exit_flags;
  a.dev_status = x.dev_status;
  a.xcd_test = xcd_test_flag();
  if (!lazy && p.fsplit_u > 0) {
    a.fsplit_u = p.fsplit_u;
    a.f_items = p.f_items;
    a.f_tiles = p.f_tiles;
    a.fpart = reinterpret_cast<float4*>(ws + p.off_fpart);
    a.fcount = reinterpret_cast<int32_t*>(ws + p.off_fcount);
  }
  if (!lazy) a.fpair = p.fpair;
  if (lazy && p.lsplit) {
    a.f_tiles = p.f_tiles;
    a.fpart = reinterpret_cast<float4*>(ws + p.off_fpart);
    a.fcount = reinterpret_cast<int32_t*>(ws + p.off_fcount);
    a.lmass = reinterpret_cast<float*>(ws + p.off_lmass);
  }
  if (lazy) {
    a.pcol = reinterpret_cast<float*>(ws + p.off_pcol);
    a.pcol_rows = lazy_cfg_rows(p.lazy_cfg);
  }
  const bool fuse = x.fuse_commit;
  CommitArgs cm{};
  int64_t gblocks = static_cast<int64_t>(sh) * (a.n_keys_pad / 64);
  if (fuse) {
    cm.arena = static_cast<uint8_t*>(x.kv->arena);
    cm.k_new = x.k_new; cm.v_new = x.v_new;
    cm.src_compact = x.kv_layout == FL_ROWS_COMPACT;
    cm.slot_base = x.commit_slot_base; cm.reset = x.commit_reset;
    const int64_t items = static_cast<int64_t>(kv.n_seq) * kv.H * ((a.n_rows + kCommitRows - 1) / kCommitRows);
    if (lazy) gblocks += (items + 15) / 16;                                  // the active rows' records
    if (x.version >= 2) gblocks += static_cast<int64_t>(kv.n_seq) * ((kv.N + 255) / 256);   // slot column
  }
  dim3 gg(static_cast<unsigned>(gblocks));
  {
    TimedLaunch t(st, fuse ? (lazy ? "gather_commit_lazy" : "gather_commit_full") : lazy ? "gather_lazy" : "gather_full");
    // four keys per chain walk when the gather blocks alone leave CUs idle
    const bool wide = static_cast<int64_t>(sh) * (a.n_keys_pad / 64) < 512;
#define FL_GATHER(DTV, LZ, FU)                                                                  \
  do {                                                                                         \
    if (wide) hipLaunchKernelGGL((k_gather<DTV, D, LZ, FU, 4>), gg, dim3(256), 0, st, kv, a, cm); \
    else hipLaunchKernelGGL((k_gather<DTV, D, LZ, FU, 1>), gg, dim3(256), 0, st, kv, a, cm);      \
  } while (0)
    if (kv.dtype == FL_BF16) {
      if (lazy && fuse) FL_GATHER(FL_BF16, true, true);
      else if (lazy) FL_GATHER(FL_BF16, true, false);
      else if (fuse) FL_GATHER(FL_BF16, false, true);
      else FL_GATHER(FL_BF16, false, false);
    } else {
      if (lazy && fuse) FL_GATHER(FL_F32, true, true);
      else if (lazy) FL_GATHER(FL_F32, true, false);
      else if (fuse) FL_GATHER(FL_F32, false, true);
      else FL_GATHER(FL_F32, false, false);
    }
#undef FL_GATHER
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // 256-row workgroups with 64-key tiles for full loops; a lazy loop's shape
  // is planned (plan_lazy_cfg)
  const int cfg = lazy ? p.lazy_cfg : 0;
  const int rows_per = lazy_cfg_rows(cfg);
  if ((a.fsplit_u > 0 || a.fpair > 0) && cfg != 0) return hipErrorInvalidConfiguration;   // 256-row tiles only
  const int row_tiles = (a.n_rows + rows_per - 1) / rows_per;
  if (a.lmass && a.f_tiles != row_tiles) return hipErrorInvalidConfiguration;
  dim3 gf(mapped_grid(a.n_sh, a.fsplit_u > 0 ? a.f_items : a.fpair > 0 ? a.fpair : a.lmass ? 2 * row_tiles : row_tiles));
  {
    TimedLaunch t(st, lazy ? "mfma_fwd_lazy" : "mfma_fwd_full");
    const bool mix = lazy && x.formula == FL_FORMULA_MIXTURE;
#define FL_FWD(NWV, KTV, THREADS)                                                                           \
  do {                                                                                                       \
    if (mix) hipLaunchKernelGGL((k_mfma_fwd<D, NWV, KTV, true, true>), gf, dim3(THREADS), 0, st, kv.H, kv.N, a); \
    else if (lazy) hipLaunchKernelGGL((k_mfma_fwd<D, NWV, KTV, true>), gf, dim3(THREADS), 0, st, kv.H, kv.N, a); \
    else hipLaunchKernelGGL((k_mfma_fwd<D, NWV, KTV, false>), gf, dim3(THREADS), 0, st, kv.H, kv.N, a);          \
  } while (0)
    if (a.fpair > 0) hipLaunchKernelGGL((k_mfma_fwd<D, 8, 64, false, false, true>), gf, dim3(512), 0, st, kv.H, kv.N, a);
    else if (cfg == 0) FL_FWD(8, 64, 512);
    else if (cfg == 1 && D <= 96) FL_FWD(4, 64, 256);   // 64-key tiles fit the registers below head_dim 128
    else if (cfg == 1) FL_FWD(4, 32, 256);
    else FL_FWD(2, 32, 128);
#undef FL_FWD
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  a.col_chunks = p.col_chunks;
  a.col_var_rows = p.col_var_rows;
  a.col_items = p.col_items;
  a.col_rows = p.col_rows;
  a.col_part = reinterpret_cast<float*>(ws + p.off_part);
  dim3 gc(mapped_grid(a.n_sh, a.col_var_rows > 0 ? a.col_items : a.n_keys_pad / 256 * a.col_chunks));
  {
    TimedLaunch t(st, lazy ? "mfma_colmass_lazy" : "mfma_colmass_full");
    if (lazy) hipLaunchKernelGGL((k_mfma_colmass<D, true>), gc, dim3(512), 0, st, kv.H, kv.N, a);
    else hipLaunchKernelGGL((k_colmass_full_rows<D>), gc, dim3(512), 0, st, kv.H, kv.N, a);
  }
  if (a.col_chunks > 1 && !a.ccount) {
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t n = static_cast<int64_t>(a.n_sh) * a.n_keys_pad;
    dim3 gr(static_cast<unsigned>((n + 255) / 256));
    TimedLaunch t(st, "colmass_reduce");
    if (lazy) hipLaunchKernelGGL((k_colmass_reduce<true>), gr, dim3(256), 0, st, kv.N, a);
    else hipLaunchKernelGGL((k_colmass_reduce<false>), gr, dim3(256), 0, st, kv.N, a);
  }
  return hipGetLastError();
}

hipError_t launch_mfma(const fl_attend_args& x, const KvView& kv, const AttendPlan& p, hipStream_t st) {
  switch (kv.d) {
    case 64: return launch_d<64>(x, kv, p, st);
    case 96: return launch_d<96>(x, kv, p, st);
    default: return launch_d<128>(x, kv, p, st);
  }
}

}  // namespace fl
