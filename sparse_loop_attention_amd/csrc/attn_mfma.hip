// Tiled bf16 MFMA attention on gathered key tiles (prefill: many active rows).
//
// Page "FlashLoop: Fast and Memory-Efficient Looped Transformers via Lazy
// Updates", section "FlashLoop combines three kinds of savings": paragraph 2
// (attention on the keys chosen from the previous loop's statistics, keeping
// the chosen group's previous probability mass) and paragraph 4 (the selected
// data is gathered into dense buffers so that sparsity turns into speed).
//
// Three launches per call:
//   gather   - walks the base+delta chain of every key slot (all N keys in a
//              full loop, the selected keys in a lazy loop) once, and writes
//              dense tiles: K^ rows [sh][slot][d] in bf16 and V^ transposed
//              [sh][d][slot] as fp16 holding the bf16-rounded values (keys
//              permuted inside each 16-key chunk so that an MFMA operand is
//              one 16-byte LDS read), plus the key positions; a lazy loop
//              gathers versions v-1 and v;
//   fwd      - one workgroup per 128 (full) or 64 (lazy) query rows of one
//              head.  S^T = K Q^T on v_mfma_f32_32x32x16_bf16 keeps every query
//              in one lane, so the row softmax needs a single cross-half
//              exchange; P^T feeds the PV product straight from the
//              accumulators.  In a lazy loop waves pair up: one computes the
//              current softmax over the selected keys, its partner the
//              previous loop's probabilities with the fixed normaliser lse_prev
//              (mass m and contribution a); they combine through LDS into
//              o = m*otilde + o_prev - a;
//   colmass  - key-major: one workgroup per 128 key slots, streaming the
//              query tiles, S = Q K^T with keys in lanes so that the column
//              sums are lane-local; fixed order, no atomics.
#include <climits>

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
__host__ __device__ inline int mapped_grid(int n_sh, int n_tiles) {
  return n_sh >= 8 ? 8 * ((n_sh + 7) / 8) * n_tiles : n_sh * n_tiles;
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
template <int DT, int D, bool LAZY, bool FUSE>
__global__ __launch_bounds__(256) void k_gather(KvView kv, MfmaArgs a, CommitArgs cm) {
  __shared__ uint16_t sv[2][64][D + 2];
  const int n_tiles = a.n_keys_pad / 64;
  int b = blockIdx.x;
  const int g = threadIdx.x >> 4, p = threadIdx.x & 15;
  if (FUSE && b >= a.n_sh * n_tiles) {
    b -= a.n_sh * n_tiles;
    const int64_t items = static_cast<int64_t>(kv.n_seq) * a.n_rows * kv.H * 2;
    const int n_cb = static_cast<int>((items + 15) / 16);
    if (b < n_cb) {                                       // records of the active rows
      const int64_t item = static_cast<int64_t>(b) * 16 + g;
      if (item >= items) return;
      const int which = static_cast<int>(item & 1);
      const int h = static_cast<int>((item >> 1) % kv.H);
      const int64_t sr = (item >> 1) / kv.H;
      const int r = static_cast<int>(sr % a.n_rows), s = static_cast<int>(sr / a.n_rows);
      const int j = a.act[static_cast<int64_t>(s) * a.n_rows + r];
      const int64_t src_rows = cm.src_compact ? a.n_rows : kv.N;
      const int64_t src_elem = ((static_cast<int64_t>(s) * src_rows + (cm.src_compact ? r : j)) * kv.H + h) * D;
      commit_row<DT>(kv, cm.arena, a.version, s, j, h, which, cm.slot_base + r, which ? cm.v_new : cm.k_new,
                     src_elem, p);
      return;
    }
    b -= n_cb;                                            // slot table column of layer `version`
    const int per_seq = (kv.N + 255) / 256;
    const int s = b / per_seq;
    const int j = (b % per_seq) * 256 + threadIdx.x;
    if (s >= kv.n_seq || j >= kv.N) return;
    const int ra = find_active(a.act + static_cast<int64_t>(s) * a.n_rows, a.n_rows, j);
    int32_t* dst = reinterpret_cast<int32_t*>(cm.arena + kv.slot_table) +
                   (static_cast<int64_t>(s) * kv.N + j) * kv.slot_pitch + (a.version - 2);
    if (ra >= 0) *dst = cm.slot_base + ra;
    else if (cm.reset) *dst = -1;
    return;
  }
  const int sh = b / n_tiles, tile = b % n_tiles;
  const int s = sh / kv.H, h = sh % kv.H;
  const bool live = 8 * p < D;
  const int32_t* act_s = FUSE ? a.act + static_cast<int64_t>(s) * a.n_rows : nullptr;
#pragma unroll 1
  for (int kk = 0; kk < 4; ++kk) {
    const int local = g * 4 + kk;
    const int t = tile * 64 + local;
    int j = -1;
    if (t < a.n_keys) j = a.key_idx ? a.key_idx[static_cast<int64_t>(sh) * a.n_keys + t] : t;
    float x[8] = {}, xp[8] = {};
    const int64_t krow = (static_cast<int64_t>(sh) * a.n_keys_pad + t) * D + 8 * p;
    if (live) {
      float y[8] = {}, yp[8] = {};
      if (FUSE) {
        // versions v-1 from the chain, version v from this loop's new rows
        if (j >= 0) {
          // a reset commit clears layer v for the tokens it does not write; otherwise
          // layer v may hold earlier commits' records (an active key's own entry is
          // overridden below)
          const int vw = cm.reset ? a.version - 1 : a.version;
          recon8<DT>(kv, 0, s, h, j, vw, p, x, cm.reset ? nullptr : xp);
          recon8<DT>(kv, 1, s, h, j, vw, p, y, cm.reset ? nullptr : yp);
          if (cm.reset) {
#pragma unroll
            for (int e = 0; e < 8; ++e) { xp[e] = x[e]; yp[e] = y[e]; }
          }
        }
        const int ra = j >= 0 ? find_active(act_s, a.n_rows, j) : -1;
        if (ra >= 0) {
          const int64_t src_rows = cm.src_compact ? a.n_rows : kv.N;
          const int64_t src = ((static_cast<int64_t>(s) * src_rows + (cm.src_compact ? ra : j)) * kv.H + h) * D + 8 * p;
          float kn[8], vn[8];
          load8<DT>(cm.k_new, src, kn);
          load8<DT>(cm.v_new, src, vn);
          advance8(kn, xp, true, x);
          advance8(vn, yp, true, y);
        }
      } else {
        if (j >= 0) recon8<DT>(kv, 0, s, h, j, a.version, p, x, LAZY ? xp : nullptr);
        if (j >= 0) recon8<DT>(kv, 1, s, h, j, a.version, p, y, LAZY ? yp : nullptr);
      }
      store8<FL_BF16>(a.kc, krow, x);
      if (LAZY) store8<FL_BF16>(a.kp, krow, xp);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sv[0][local][8 * p + e] = v_operand_bits(y[e]);
        if (LAZY) sv[1][local][8 * p + e] = v_operand_bits(yp[e]);
      }
    }
    if (p == 0) a.kidx[static_cast<int64_t>(sh) * a.n_keys_pad + t] = j >= 0 ? j : INT_MAX;
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

// Tile geometry: K (KT x D, bf16) and V^T (D x KT, fp16) of one role, 16-byte
// chunks striped over the 256 threads; global loads go to registers first so
// that they overlap the MFMA work on the other LDS buffer.
template <int D, int KT, int NT>
struct TileIO {
  static constexpr int KCH = KT * D / 8;   // 16-byte chunks of a K tile (KT x D bf16)
  static constexpr int VCH = D * KT / 8;   // 16-byte chunks of a V^T tile (D x KT fp16)
  static constexpr int PER = (KCH + VCH) / NT;
  static constexpr int KS = D + 8;         // padded LDS row strides
  static constexpr int VS = KT + 8;
};

template <int D, bool LAZY>
__global__ __launch_bounds__(512, 1) void k_mfma_fwd(int32_t H, int32_t N, MfmaArgs a) {
  constexpr int KT = 64;
  constexpr int DC = D / 16;
  constexpr int DB = D / 32;
  constexpr int NR = LAZY ? 2 : 1;
  constexpr int NT = 512;                                 // 8 waves: 8 row blocks, or 4 x (current, previous)
  constexpr int ROWS = LAZY ? 128 : 256;
  using IO = TileIO<D, KT, NT>;
  constexpr int KS = IO::KS, VS = IO::VS;
  __shared__ __attribute__((aligned(16))) uint16_t sk[2][NR][KT * KS];
  __shared__ __attribute__((aligned(16))) uint16_t sv[2][NR][D * VS];
  __shared__ int skidx[2][KT];
  __shared__ float sm[4][32];
  __shared__ int s_last;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hh = lane >> 5, c = lane & 31;
  int sh, qtile;
  if (!map_block(a.n_sh, (a.n_rows + ROWS - 1) / ROWS, sh, qtile)) return;
  const int s = sh / H, h = sh % H;
  const int blk = LAZY ? (wave >> 1) : wave;
  const int role = LAZY ? (wave & 1) : 0;                 // 0 = current, 1 = previous loop
  const int r0 = qtile * ROWS + blk * 32;                 // first row of this wave's block
  const int r = r0 + c;
  const bool vrow = r < a.n_rows;
  const int tok = vrow ? row_token(a, s, r) : -1;
  const bool blk_full = r0 + 31 < a.n_rows;               // all 32 rows of the block exist
  const int tok_first = row_token(a, s, min(r0, a.n_rows - 1));
  const int tok_last = row_token(a, s, min(r0 + 31, a.n_rows - 1));
  const float c1 = a.scale * kLog2e;                      // logits in log2 units

  bf16x8 qf[DC];
  {
    const uint16_t* q = static_cast<const uint16_t*>(role ? a.q_prev : a.q_cur);
    const int64_t rows_q = a.q_compact ? a.n_rows : N;
    const int64_t qr = a.q_compact ? r : tok;
    const uint16_t* src = q + ((static_cast<int64_t>(s) * rows_q + qr) * H + h) * D + 8 * hh;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) qf[dc] = vrow ? *reinterpret_cast<const bf16x8*>(src + dc * 16) : bf16x8{};
  }
  const int64_t rows_o = a.o_compact ? a.n_rows : N;
  const int64_t orow = a.o_compact ? r : tok;
  float lse_prev = 0.0f;
  if (LAZY && vrow) lse_prev = a.lse[(static_cast<int64_t>(s) * rows_o + orow) * H + h];
  const float b_prev = lse_prev * kLog2e;

  const int32_t* kx = a.kidx + static_cast<int64_t>(sh) * a.n_keys_pad;
  if (tid == 0) {                                        // key slots visible to the workgroup's last row
    const int last_tok = row_token(a, s, min(a.n_rows, (qtile + 1) * ROWS) - 1);
    int lo = 0, hi = a.n_keys;
    while (lo < hi) { const int mid = (lo + hi) >> 1; if (kx[mid] <= last_tok) lo = mid + 1; else hi = mid; }
    s_last = lo;
  }
  const uint16_t* kbase[NR];
  const uint16_t* vbase[NR];
  kbase[0] = a.kc + static_cast<int64_t>(sh) * a.n_keys_pad * D;
  vbase[0] = a.vtc + static_cast<int64_t>(sh) * D * a.n_keys_pad;
  if (LAZY) {
    kbase[NR - 1] = a.kp + static_cast<int64_t>(sh) * a.n_keys_pad * D;
    vbase[NR - 1] = a.vtp + static_cast<int64_t>(sh) * D * a.n_keys_pad;
  }
  __syncthreads();
  const int n_tiles = (s_last + KT - 1) / KT;

  f32x16 acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;                  // current loop, log2 units, lane half
  float mass = 0.0f;                                      // previous loop, lane half

  u32x4 pre[NR][IO::PER];
  int pre_k = INT_MAX;
#define FL_FWD_GLOAD(TILE)                                                              \
  {                                                                                     \
    _Pragma("unroll") for (int w = 0; w < NR; ++w)                                      \
      _Pragma("unroll") for (int i = 0; i < IO::PER; ++i) {                             \
        const int q = tid + NT * i;                                                     \
        if (q < IO::KCH) {                                                              \
          const int row = q / (D / 8), col = (q % (D / 8)) * 8;                         \
          pre[w][i] = *reinterpret_cast<const u32x4*>(kbase[w] + static_cast<int64_t>((TILE) * KT + row) * D + col); \
        } else {                                                                        \
          const int qv = q - IO::KCH;                                                   \
          const int row = qv / (KT / 8), col = (qv % (KT / 8)) * 8;                     \
          pre[w][i] = *reinterpret_cast<const u32x4*>(vbase[w] + static_cast<int64_t>(row) * a.n_keys_pad + (TILE) * KT + col); \
        }                                                                               \
      }                                                                                 \
    if (tid < KT) pre_k = kx[(TILE) * KT + tid];                                        \
  }
#define FL_FWD_SSTORE(BUF)                                                              \
  {                                                                                     \
    _Pragma("unroll") for (int w = 0; w < NR; ++w)                                      \
      _Pragma("unroll") for (int i = 0; i < IO::PER; ++i) {                             \
        const int q = tid + NT * i;                                                     \
        if (q < IO::KCH) {                                                              \
          const int row = q / (D / 8), col = (q % (D / 8)) * 8;                         \
          *reinterpret_cast<u32x4*>(&sk[BUF][w][row * KS + col]) = pre[w][i];           \
        } else {                                                                        \
          const int qv = q - IO::KCH;                                                   \
          const int row = qv / (KT / 8), col = (qv % (KT / 8)) * 8;                     \
          *reinterpret_cast<u32x4*>(&sv[BUF][w][row * VS + col]) = pre[w][i];           \
        }                                                                               \
      }                                                                                 \
    if (tid < KT) skidx[BUF][tid] = pre_k;                                              \
  }
  if (n_tiles > 0) {
    FL_FWD_GLOAD(0)
    FL_FWD_SSTORE(0)
  }
  __syncthreads();

  for (int tile = 0; tile < n_tiles; ++tile) {
    const int buf = tile & 1;
    if (tile + 1 < n_tiles) FL_FWD_GLOAD(tile + 1)
    const int* kk = skidx[buf];
    if (kk[0] <= tok_last) {                              // some key of the tile is visible to the block
      const uint16_t* K = sk[buf][role];
      const uint16_t* V = sv[buf][role];
      f32x16 st[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        st[kb] = f32x16{};
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&K[(kb * 32 + c) * KS + dc * 16 + 8 * hh]);
          st[kb] = mfma32(ka, qf[dc], st[kb]);
        }
      }
      const bool need_mask = !blk_full || kk[KT - 1] > tok_first;
      float pv[32];                                       // raw logits q.k
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float x = st[kb][i];
          if (need_mask && kk[kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3)] > tok) x = -INFINITY;
          pv[kb * 16 + i] = x;
        }
      if (role == 0) {
        float tmax = pv[0];
#pragma unroll
        for (int i = 1; i < 32; ++i) tmax = fmaxf(tmax, pv[i]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        const float m_new = fmaxf(m_run, tmax * c1);      // running max in log2 units (c1 > 0)
        const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;   // fully masked so far: p = 0
        float psum = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) { pv[i] = ex2(fmaf(pv[i], c1, -m_use)); psum += pv[i]; }
        if (__ballot(m_new != m_run)) {                   // the running max moved for some row
          const float alpha = ex2(m_run - m_use);
          l_run *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
        }
        m_run = m_new;
        l_run += psum;
      } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) { pv[i] = ex2(fmaf(pv[i], c1, -b_prev)); mass += pv[i]; }
      }
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        f16x8 pb;
#pragma unroll
        for (int i = 0; i < 8; ++i) pb[i] = static_cast<_Float16>(pv[cc * 8 + i]);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const f16x8 va = *reinterpret_cast<const f16x8*>(&V[(db * 32 + c) * VS + cc * 16 + 8 * hh]);
          acc[db] = mfma32h(va, pb, acc[db]);
        }
      }
    }
    if (tile + 1 < n_tiles) FL_FWD_SSTORE(buf ^ 1)
    __syncthreads();
  }
#undef FL_FWD_GLOAD
#undef FL_FWD_SSTORE

  // ---- epilogue
  float* lse_ptr = a.lse + (static_cast<int64_t>(s) * rows_o + orow) * H + h;
  float* o_ptr = a.o + ((static_cast<int64_t>(s) * rows_o + orow) * H + h) * D;
  float* st_ptr = a.stat + (static_cast<int64_t>(sh) * a.n_rows + r) * 4;
  if (!LAZY) {
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
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
        const float b = m_run + __log2f(l_tot);           // lse in log2 units
        *lse_ptr = b * kLn2;
        *reinterpret_cast<float4*>(st_ptr) = make_float4(b, b, 1.0f, __int_as_float(tok));
      }
    }
    return;
  }
  // lazy: the previous-loop wave hands its mass and contribution to its partner
  float* sa = reinterpret_cast<float*>(&sk[0][0][0]);     // [blk][DB][16][64] floats
  if (role == 1) {
    const float m_tot = mass + __shfl_xor(mass, 32, 64);
    if (hh == 0) sm[blk][c] = m_tot;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) sa[((blk * DB + db) * 16 + i) * 64 + lane] = acc[db][i];
  }
  __syncthreads();
  if (role == 0 && vrow) {
    const float z = l_run + __shfl_xor(l_run, 32, 64);
    const float m = sm[blk][c];
    const bool valid = z > 0.0f && m > 0.0f;
    if (valid) {
      const float f = m / z;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int dim = db * 32 + 8 * q4 + 4 * hh;
          float4 op = *reinterpret_cast<const float4*>(o_ptr + dim);
          const float* av = &sa[((blk * DB + db) * 16 + 4 * q4) * 64 + lane];
          op.x = fmaf(f, acc[db][4 * q4 + 0], op.x - av[0]);
          op.y = fmaf(f, acc[db][4 * q4 + 1], op.y - av[64]);
          op.z = fmaf(f, acc[db][4 * q4 + 2], op.z - av[128]);
          op.w = fmaf(f, acc[db][4 * q4 + 3], op.w - av[192]);
          *reinterpret_cast<float4*>(o_ptr + dim) = op;
        }
    }
    if (hh == 0) {
      // new lse in log2 units: M + log2 Z - log2 m
      const float b = valid ? m_run + __log2f(z) - __log2f(m) : b_prev;
      if (valid) *lse_ptr = b * kLn2;
      *reinterpret_cast<float4*>(st_ptr) =
          make_float4(valid ? b_prev : INFINITY, valid ? b : INFINITY, valid ? 1.0f : 0.0f, __int_as_float(tok));
    }
  }
}

// --------------------------------------------------------------------------- colmass
// stat rows hold (b_prev, b_cur, valid, token) with b = lse * log2(e); rows
// that did not update carry b = +inf so that their probabilities vanish.
template <int D, bool LAZY>
__global__ __launch_bounds__(512, 1) void k_mfma_colmass(int32_t H, int32_t N, MfmaArgs a) {
  constexpr int QT = 64;
  constexpr int DC = D / 16;
  constexpr int QS = D + 8;
  constexpr int NR = LAZY ? 2 : 1;
  constexpr int NT = 512;                                  // 8 waves x 32 keys
  constexpr int KB = 256;                                  // key slots per workgroup
  constexpr int QCH = QT * D / 8;                          // 16-B chunks of one Q tile
  constexpr int PER = (QCH + NT - 1) / NT;
  __shared__ __attribute__((aligned(16))) uint16_t sq[2][NR][QT * QS];
  __shared__ __attribute__((aligned(16))) float sb[2][2][QT];   // [buf][prev|cur][row]
  __shared__ int stok[2][QT];
  __shared__ int s_start;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hh = lane >> 5, c = lane & 31;
  int sh, kblk;
  if (!map_block(a.n_sh, a.n_keys_pad / KB, sh, kblk)) return;
  kblk = a.n_keys_pad / KB - 1 - kblk;                    // early keys see the most rows: start them first
  const int s = sh / H, h = sh % H;
  const int t0 = kblk * KB + wave * 32;
  const int t = t0 + c;
  const int32_t* kx = a.kidx + static_cast<int64_t>(sh) * a.n_keys_pad;
  const int kj = kx[t];                                    // INT_MAX for padding
  const int kmax = kx[min(t0 + 31, a.n_keys - 1)];         // largest real key of this wave
  const float c1 = a.scale * kLog2e;

  bf16x8 kf[NR][DC];
#pragma unroll
  for (int w = 0; w < NR; ++w) {
    const uint16_t* kb = (w ? a.kp : a.kc) + (static_cast<int64_t>(sh) * a.n_keys_pad + t) * D + 8 * hh;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) kf[w][dc] = *reinterpret_cast<const bf16x8*>(kb + dc * 16);
  }
  if (tid == 0) {                                          // first row that sees the block's first key
    const int kfirst = kx[kblk * KB];
    int lo = 0, hi = a.n_rows;
    while (lo < hi) { const int mid = (lo + hi) >> 1; if (row_token(a, s, mid) < kfirst) lo = mid + 1; else hi = mid; }
    s_start = lo;
  }
  __syncthreads();
  const int r_begin = (s_start / QT) * QT;
  const int n_tiles = (a.n_rows - r_begin + QT - 1) / QT;
  const int64_t rows_q = a.q_compact ? a.n_rows : N;

  u32x4 pre[NR][PER];
  float pre_b0 = INFINITY, pre_b1 = INFINITY;
  int pre_tok = -1;
  auto gload = [&](int q0) {
#pragma unroll
    for (int w = 0; w < NR; ++w) {
      const uint16_t* q = static_cast<const uint16_t*>(w ? a.q_prev : a.q_cur);
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int ch = tid + NT * i;
        const int row = ch / (D / 8), col = (ch % (D / 8)) * 8;
        const int rr = q0 + row;
        pre[w][i] = u32x4{0, 0, 0, 0};
        if (ch < QCH && rr < a.n_rows) {
          const int64_t qr = a.q_compact ? rr : row_token(a, s, rr);
          pre[w][i] = *reinterpret_cast<const u32x4*>(q + ((static_cast<int64_t>(s) * rows_q + qr) * H + h) * D + col);
        }
      }
    }
    if (tid < QT) {
      const int rr = q0 + tid;
      pre_b0 = pre_b1 = INFINITY;
      pre_tok = -1;
      if (rr < a.n_rows) {
        const float4 st = *reinterpret_cast<const float4*>(a.stat + (static_cast<int64_t>(sh) * a.n_rows + rr) * 4);
        pre_b0 = st.x; pre_b1 = st.y; pre_tok = __float_as_int(st.w);
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int w = 0; w < NR; ++w)
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int ch = tid + NT * i;
        const int row = ch / (D / 8), col = (ch % (D / 8)) * 8;
        if (ch < QCH) *reinterpret_cast<u32x4*>(&sq[buf][w][row * QS + col]) = pre[w][i];
      }
    if (tid < QT) { sb[buf][0][tid] = pre_b0; sb[buf][1][tid] = pre_b1; stok[buf][tid] = pre_tok; }
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
    // rows of this tile that every key of the wave precedes need no mask
    const bool need_mask = stok[buf][0] < kmax || q0 + QT > a.n_rows;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x16 sc = f32x16{}, sp = f32x16{};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const bf16x8 qa = *reinterpret_cast<const bf16x8*>(&sq[buf][0][(qb * 32 + c) * QS + dc * 16 + 8 * hh]);
        sc = mfma32(qa, kf[0][dc], sc);
        if (LAZY) {
          const bf16x8 qpa = *reinterpret_cast<const bf16x8*>(&sq[buf][NR - 1][(qb * 32 + c) * QS + dc * 16 + 8 * hh]);
          sp = mfma32(qpa, kf[NR - 1][dc], sp);
        }
      }
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int row0 = qb * 32 + 8 * q4 + 4 * hh;
        const float4 bc = *reinterpret_cast<const float4*>(&sb[buf][1][row0]);
        float4 bp = make_float4(0.f, 0.f, 0.f, 0.f);
        if (LAZY) bp = *reinterpret_cast<const float4*>(&sb[buf][0][row0]);
        const float bcv[4] = {bc.x, bc.y, bc.z, bc.w};
        const float bpv[4] = {bp.x, bp.y, bp.z, bp.w};
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
          const int i = 4 * q4 + k4;
          float v = ex2(sc[i] * c1 - bcv[k4]);
          if (LAZY) v -= ex2(sp[i] * c1 - bpv[k4]);
          if (need_mask && kj > stok[buf][row0 + k4]) v = 0.0f;
          acc += v;
        }
      }
    }
    if (it + 1 < n_tiles) sstore(buf ^ 1);
    __syncthreads();
  }
  acc += __shfl_xor(acc, 32, 64);
  if (hh == 0 && t < a.n_keys) {
    float* dst = a.colmass + static_cast<int64_t>(sh) * N + kj;
    if (LAZY) *dst += acc; else *dst = acc;
  }
}

// --------------------------------------------------------------------------- launch
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
  const bool fuse = lazy && x.fuse_commit;
  CommitArgs cm{};
  int64_t gblocks = static_cast<int64_t>(sh) * (a.n_keys_pad / 64);
  if (fuse) {
    cm.arena = static_cast<uint8_t*>(x.kv->arena);
    cm.k_new = x.k_new; cm.v_new = x.v_new;
    cm.src_compact = x.kv_layout == FL_ROWS_COMPACT;
    cm.slot_base = x.commit_slot_base; cm.reset = x.commit_reset;
    const int64_t items = static_cast<int64_t>(kv.n_seq) * a.n_rows * kv.H * 2;
    gblocks += (items + 15) / 16 + static_cast<int64_t>(kv.n_seq) * ((kv.N + 255) / 256);
  }
  dim3 gg(static_cast<unsigned>(gblocks));
  {
    TimedLaunch t(st, fuse ? "gather_commit_lazy" : lazy ? "gather_lazy" : "gather_full");
#define FL_GATHER(DTV, LZ, FU) hipLaunchKernelGGL((k_gather<DTV, D, LZ, FU>), gg, dim3(256), 0, st, kv, a, cm)
    if (kv.dtype == FL_BF16) {
      if (fuse) FL_GATHER(FL_BF16, true, true);
      else if (lazy) FL_GATHER(FL_BF16, true, false);
      else FL_GATHER(FL_BF16, false, false);
    } else {
      if (fuse) FL_GATHER(FL_F32, true, true);
      else if (lazy) FL_GATHER(FL_F32, true, false);
      else FL_GATHER(FL_F32, false, false);
    }
#undef FL_GATHER
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows_per = lazy ? 128 : 256;
  dim3 gf(mapped_grid(a.n_sh, (a.n_rows + rows_per - 1) / rows_per));
  {
    TimedLaunch t(st, lazy ? "mfma_fwd_lazy" : "mfma_fwd_full");
    if (lazy) hipLaunchKernelGGL((k_mfma_fwd<D, true>), gf, dim3(512), 0, st, kv.H, kv.N, a);
    else hipLaunchKernelGGL((k_mfma_fwd<D, false>), gf, dim3(512), 0, st, kv.H, kv.N, a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  dim3 gc(mapped_grid(a.n_sh, a.n_keys_pad / 256));
  {
    TimedLaunch t(st, lazy ? "mfma_colmass_lazy" : "mfma_colmass_full");
    if (lazy) hipLaunchKernelGGL((k_mfma_colmass<D, true>), gc, dim3(512), 0, st, kv.H, kv.N, a);
    else hipLaunchKernelGGL((k_mfma_colmass<D, false>), gc, dim3(512), 0, st, kv.H, kv.N, a);
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
