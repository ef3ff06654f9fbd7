// Lazy attention of one new token per sequence (decode) straight from the
// base + low-bit delta chain, with the commit of the token's records fused in.
//
// Page "FlashLoop: Fast and Memory-Efficient Looped Transformers via Lazy
// Updates", section "FlashLoop combines three kinds of savings": paragraph 2
// (only the keys chosen from the previous loop's statistics are attended,
// and the chosen group keeps the previous loop's probability mass),
// paragraph 3 (keys are a base plus low-bit per-token differences) and
// paragraph 4 (update and compression fused with the compute).  Decode reads
// the compressed cache once per loop, so the kernel is built around keeping
// HBM busy:
//
//  * one workgroup of 8 waves per (sequence, head); two fit on a CU (at most
//    128 VGPRs), so every workgroup of a 32 x 16 decode batch is resident at
//    once; all heads of a sequence run on one XCD, whose L2 then serves the
//    slot rows of keys that several heads select;
//  * the selected keys' positions and slot rows are staged in LDS first, then
//    key t goes to 16-lane group t mod 32 (lane p owns elements [8p, 8p+8));
//    each group issues the loads of its next key before it works on the
//    current one, so one key per group is always in flight;
//  * loads are buffer loads against per-sequence ranges: a layer without a
//    record for the key gets an offset past the range and reads zeros (code 0,
//    scale 0), so the chain walk has no branches;
//  * dequantisation is exact and cheap: a pair of 4-bit (or 2-bit) codes
//    (elements k and k+4) becomes two binary16 values 1024 + u (u = code + 8,
//    or + 2) by OR-ing in a fixed exponent, 1032 (1026) is subtracted in
//    binary16 (exact), and fma_mix adds code * scale (exact) to the float32
//    chain with one rounding, the same sum the store defines;
//  * logits are dot2 products of bf16 pairs: the reconstruction rounded to
//    bf16 (the working dtype) against the bf16 query.
// The full decode loop over the base (version 1) has a streaming kernel of
// its own below (k_decode_full).
#include "fl_common.hpp"
#include "fl_commit.hpp"
#include "fl_rows.hpp"
#include "fl_timing.hpp"
#include "fl_topk.hpp"

namespace fl {

namespace {

constexpr int kDecWaves = 8;
constexpr int kDecD = 128;                 // head_dim of this kernel
constexpr int kDecMaxKeys = 1536;          // staged keys per (sequence, head): 28 bytes of LDS each
constexpr int kDecMaxLayers = 4;           // delta layers walked (versions 2..5)
constexpr int kDecLoopsMaxN = 8192;        // multi-loop kernel: the column-mass row (32 KB) in LDS
constexpr size_t kDecMaxFullLds = 40960;   // full loop: logits of every key (N <= 10240) in LDS
constexpr uint32_t kOut = 0x80000000u;     // an offset past every range: the load returns zeros
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format (gfx9 family)

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t range_of(const uint8_t* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p), static_cast<short>(0), static_cast<int>(bytes),
                                           static_cast<int>(kRsrcWord3));
}

// Raw loads of one key for this lane: base rows (8 bf16 each) and, per delta
// layer, the K and V codes (8 codes of 4 or 2 bits) and scales (binary16 bits).
template <int NL>
struct KeyLoads {
  u32x4_t kb, vb;
  uint32_t kc[NL], vc[NL];
  uint32_t ks[NL], vs[NL];
};

__device__ __forceinline__ void unpack_bf16x8(const u32x4_t w, float x[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// x[e] += code_e * scale for the 8 BITS-wide two's-complement codes of
// `codes` (element e in bits [BITS*e, BITS*e + BITS)); exact products, one
// float32 rounding each.  4-bit: fields k and k+4 sit 16 bits apart already;
// 2-bit: the two code bytes are spread to bytes 0 and 2 first.
template <int BITS>
__device__ __forceinline__ void add_layer(uint32_t codes, uint32_t sbits, float x[8]) {
  constexpr uint32_t kMask = BITS == 4 ? 0x000F000Fu : 0x00030003u;
  constexpr float kBias = 1024.0f + (1 << (BITS - 1));               // 1024 + the offset of u
  const uint32_t w = BITS == 4 ? codes : (codes & 0xFFu) | ((codes & 0xFF00u) << 8);
  const uint32_t u = w ^ (BITS == 4 ? 0x88888888u : 0x00AA00AAu);    // u = code + 2^(BITS-1)
  const float s = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(sbits)));
  const f16x2_t bias = {static_cast<_Float16>(kBias), static_cast<_Float16>(kBias)};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t pr = ((u >> (BITS * k)) & kMask) | 0x64006400u;     // (1024 + u_k, 1024 + u_{k+4})
    const f16x2_t c = __builtin_bit_cast(f16x2_t, pr) - bias;           // (code_k, code_{k+4})
    x[k] = fmaf(s, static_cast<float>(c[0]), x[k]);
    x[k + 4] = fmaf(s, static_cast<float>(c[1]), x[k + 4]);
  }
}

// The 8 values rounded to bf16 (nearest even), as 4 packed pairs.
__device__ __forceinline__ void round_pack8(const float x[8], uint32_t pk[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) pk[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
}

__device__ __forceinline__ float dot_bf16x8(const uint32_t a[4], const u32x4_t b) {
  float d = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t bw = b[i];                 // a scalar copy: bit_cast of a vector element reads element 0
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a[i]), __builtin_bit_cast(bf16x2_t, bw), d, false);
  }
  return d;
}

// acc[e] = acc[e] * c + w * (bf16 pair values of pk)
__device__ __forceinline__ void axpy_bf16x8(float acc[8], float c, float w, const uint32_t pk[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[2 * i] = fmaf(w, __uint_as_float(pk[i] << 16), acc[2 * i] * c);
    acc[2 * i + 1] = fmaf(w, __uint_as_float(pk[i] & 0xFFFF0000u), acc[2 * i + 1] * c);
  }
}

}  // namespace

// One lazy loop, version v = NL + 1, of one (sequence s, head h) row: the
// selected keys' positions and slot rows are staged in LDS (s_j, s_sl; the
// first cnt are visible).  Updates the row's output o_row (global) and its
// column-mass row c_row (global, or LDS in the multi-loop kernel) and returns
// whether the row updated and its new lse.  The sequence's new token i takes
// version v from k_new/v_new and the commit arithmetic (FUSE), or versions
// v-1 and v from trk_prev/trk_cur ([K, V][kDecD] float32 in LDS; TRACK: the
// multi-loop kernel keeps the token's chain on chip, its records being
// written by this same workgroup).  Every thread of the workgroup calls it.
struct StepOut {
  bool valid;
  float lse;
};

// z is 0; the multi-loop kernel passes an opaque 0 made at the start of each
// version's code, so that the layer table is read there (reads at fixed
// kernel-argument offsets would be shared by every version's code and kept
// live throughout, in scalar registers that then spill).
template <int NL, bool FUSE, int BITS, bool TRACK>
__device__ __forceinline__ StepOut lazy_step(const KvView& kv, const CommitArgs& cm, int s, int h, int i,
                                             const void* q_cur, const void* q_prev, int q_compact, float scale,
                                             int mixture, float* o_row, float lse_prev, const int32_t* s_j,
                                             const i32x4* s_sl, int cnt, float* lg_cur, float* lg_prev,
                                             float (*s_mzm)[3], float (*s_acc)[2][kDecD], float* c_row,
                                             const float* trk_prev, const float* trk_cur, int z = 0) {
  const int H = kv.H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, p = lane & 15;
  // per-sequence ranges of the base rows and of each layer's records
  const uint8_t* A = kv.arena;
  const int64_t row_bytes = static_cast<int64_t>(kv.N) * kDecD * 2;
  const int64_t rowb = (static_cast<int64_t>(s) * H + h) * row_bytes;
  const __amdgpu_buffer_rsrc_t rK = range_of(A + kv.base[z] + rowb, static_cast<uint32_t>(row_bytes));
  const __amdgpu_buffer_rsrc_t rV = range_of(A + kv.base[z + 1] + rowb, static_cast<uint32_t>(row_bytes));
  const int ng = kDecD >> (3 + kv.gshift);                // scales per record: 4 (group 32) or 2 (group 64)
  constexpr uint32_t kCodeBytes = kDecD * BITS / 8;       // codes of one head row
  const uint32_t rec_code_bytes = H * 2 * kCodeBytes;    // K and V codes of every head of one slot
  const uint32_t rec_scale_bytes = H * 4 * ng;            // K and V scales of every head of one slot
  __amdgpu_buffer_rsrc_t rC[NL], rS[NL];
  uint32_t cap[NL];
#pragma unroll
  for (int l = 0; l < NL; ++l) {
    cap[l] = static_cast<uint32_t>(kv.cap[l + 2 + z]);
    rC[l] = range_of(A + kv.codes[l + 2 + z] + static_cast<int64_t>(s) * cap[l] * rec_code_bytes,
                     cap[l] * rec_code_bytes);
    rS[l] = range_of(A + kv.scales[l + 2 + z] + static_cast<int64_t>(s) * cap[l] * rec_scale_bytes,
                     cap[l] * rec_scale_bytes);
  }
  const uint32_t lane_b = 16 * p;
  const uint32_t lane_c = h * 2 * kCodeBytes + BITS * p;  // K codes; V codes kCodeBytes on
  const uint32_t lane_s = h * 4 * ng + 2 * (p >> kv.gshift);  // K scale; V scale 2*ng bytes on
  // a reset commit clears layer v for every token it does not write: the walk stops at v-1
  const bool walk_v = !(FUSE && cm.reset);

  const int64_t qoff = ((static_cast<int64_t>(s) * (q_compact ? 1 : kv.N) + (q_compact ? 0 : i)) * H + h) * kDecD;
  const u32x4_t qc = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(q_cur) + qoff + 8 * p);
  const u32x4_t qp = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(q_prev) + qoff + 8 * p);

  auto issue = [&](int k, KeyLoads<NL>& r) {
    const int t = wave * 4 + g + 32 * k;
    const int tt = t < cnt ? t : 0;
    const int j = s_j[tt];
    // TRACK: the new token's versions come from LDS, its loads read zeros
    const bool ok = t < cnt && !(TRACK && j == i);
    const i32x4 sl = s_sl[tt];
    const uint32_t ob = ok ? static_cast<uint32_t>(j) * (kDecD * 2) + lane_b : kOut;
    r.kb = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rK, ob, 0, 0));
    r.vb = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rV, ob, 0, 0));
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      const uint32_t slot = static_cast<uint32_t>(sl[l]);                // -1 (absent) is past every cap
      const bool use = ok && slot < cap[l] && (l + 1 < NL || walk_v);
      const uint32_t oc = use ? slot * rec_code_bytes + lane_c : kOut;
      const uint32_t os = use ? slot * rec_scale_bytes + lane_s : kOut;
      if (BITS == 4) {
        r.kc[l] = __builtin_amdgcn_raw_buffer_load_b32(rC[l], oc, 0, 0);
        r.vc[l] = __builtin_amdgcn_raw_buffer_load_b32(rC[l], oc + kCodeBytes, 0, 0);
      } else {
        r.kc[l] = static_cast<uint16_t>(__builtin_amdgcn_raw_buffer_load_b16(rC[l], oc, 0, 0));
        r.vc[l] = static_cast<uint16_t>(__builtin_amdgcn_raw_buffer_load_b16(rC[l], oc + kCodeBytes, 0, 0));
      }
      r.ks[l] = static_cast<uint16_t>(__builtin_amdgcn_raw_buffer_load_b16(rS[l], os, 0, 0));
      r.vs[l] = static_cast<uint16_t>(__builtin_amdgcn_raw_buffer_load_b16(rS[l], os + 2 * ng, 0, 0));
    }
  };

  float M = -INFINITY, Z = 0.0f, m = 0.0f;
  float acc[8] = {}, accp[8] = {};
  auto consume = [&](int k, const KeyLoads<NL>& r) {
    const int t = wave * 4 + g + 32 * k;
    if (t >= cnt) return;                                 // uniform per 16-lane group
    const bool active = (FUSE || TRACK) && s_j[t] == i;   // the new token: version v from its new row
    float x[8];
    uint32_t pk[4];
    if (TRACK && active) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = trk_prev[8 * p + e];
    } else {
      unpack_bf16x8(r.kb, x);
#pragma unroll
      for (int l = 0; l + 1 < NL; ++l) add_layer<BITS>(r.kc[l], r.ks[l], x);
    }
    round_pack8(x, pk);
    const float sp = group_sum<16>(dot_bf16x8(pk, qp)) * scale;
    int64_t src = 0;
    if (TRACK && active) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = trk_cur[8 * p + e];
    } else if (active) {
      const int64_t src_rows = cm.src_compact ? 1 : kv.N;
      src = ((static_cast<int64_t>(s) * src_rows + (cm.src_compact ? 0 : i)) * H + h) * kDecD + 8 * p;
      float xn[8], xo[8];
      load8<FL_BF16>(cm.k_new, src, xn);
      advance8(kv, xn, x, true, xo);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = xo[e];
    } else {
      add_layer<BITS>(r.kc[NL - 1], r.ks[NL - 1], x);
    }
    round_pack8(x, pk);
    const float sc = group_sum<16>(dot_bf16x8(pk, qc)) * scale;
    if (p == 0) { lg_cur[t] = sc; lg_prev[t] = sp; }
    const float Mn = fmaxf(M, sc);
    const float corr = __expf(M - Mn);
    const float w = __expf(sc - Mn);
    const float pp = __expf(sp - lse_prev);
    Z = fmaf(Z, corr, w);
    m += pp;
    M = Mn;
    if (TRACK && active) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = trk_prev[kDecD + 8 * p + e];
    } else {
      unpack_bf16x8(r.vb, x);
#pragma unroll
      for (int l = 0; l + 1 < NL; ++l) add_layer<BITS>(r.vc[l], r.vs[l], x);
    }
    round_pack8(x, pk);
    axpy_bf16x8(accp, 1.0f, pp, pk);
    if (TRACK && active) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = trk_cur[kDecD + 8 * p + e];
    } else if (active) {
      float xn[8], xo[8];
      load8<FL_BF16>(cm.v_new, src, xn);
      advance8(kv, xn, x, true, xo);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = xo[e];
    } else {
      add_layer<BITS>(r.vc[NL - 1], r.vs[NL - 1], x);
    }
    round_pack8(x, pk);
    axpy_bf16x8(acc, corr, w, pk);
  };

  // two key buffers: the loads of step k+1 are in flight while step k
  // computes (a step past the group's keys loads zeros and is skipped)
  const int nsteps = cnt > wave * 4 ? (cnt - wave * 4 + 31) / 32 : 0;   // steps of the wave's first group
  KeyLoads<NL> ra, rb;
  issue(0, ra);
  for (int k = 0; k < nsteps; k += 2) {
    issue(k + 1, rb);
    consume(k, ra);
    if (k + 1 >= nsteps) break;
    issue(k + 2, ra);
    consume(k + 1, rb);
  }

  // merge the four 16-lane groups of the wave (same elements, different keys)
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
    m += __shfl_xor(m, o, 64);
#pragma unroll
    for (int e = 0; e < 8; ++e) accp[e] += __shfl_xor(accp[e], o, 64);
  }
  // then the waves, through LDS, in fixed order
  if (lane == 0) { s_mzm[wave][0] = M; s_mzm[wave][1] = Z; s_mzm[wave][2] = m; }
  if (g == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      s_acc[wave][0][8 * p + e] = acc[e];
      s_acc[wave][1][8 * p + e] = accp[e];
    }
  }
  __syncthreads();
  float Mt = -INFINITY;
#pragma unroll
  for (int w = 0; w < kDecWaves; ++w) Mt = fmaxf(Mt, s_mzm[w][0]);
  float Zt = 0.0f, mt = 0.0f;
#pragma unroll
  for (int w = 0; w < kDecWaves; ++w) {
    const float cw = (s_mzm[w][0] == -INFINITY) ? 0.0f : __expf(s_mzm[w][0] - Mt);
    Zt = fmaf(s_mzm[w][1], cw, Zt);
    mt += s_mzm[w][2];
  }
  const bool valid = cnt > 0 && mt > 0.0f;
  if (tid < kDecD) {
    float ov = 0.0f, av = 0.0f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float cw = (s_mzm[w][0] == -INFINITY) ? 0.0f : __expf(s_mzm[w][0] - Mt);
      ov = fmaf(s_acc[w][0][tid], cw, ov);
      av += s_acc[w][1][tid];
    }
    if (valid) o_row[tid] = fmaf(mt / Zt, ov, mixture ? (1.0f - mt) * o_row[tid] : o_row[tid] - av);
  }
  const float lnew = valid ? Mt + __logf(Zt) - __logf(mt) : lse_prev;
  // column mass of the row: c_j += p_ij - p'_ij over the visible selected keys
  if (valid) {
    const float f = mt / Zt;
    for (int t = tid; t < cnt; t += 64 * kDecWaves)
      c_row[s_j[t]] += f * __expf(lg_cur[t] - Mt) - __expf(lg_prev[t] - lse_prev);
  }
  return {valid, lnew};
}

// (sequence, head) of a decode workgroup: all heads of a sequence on one XCD
// (workgroup b runs on XCD b % 8), whose L2 then serves the slot rows of keys
// that several heads select.  False for padding workgroups.
__device__ __forceinline__ bool dec_map(const KvView& kv, int& s, int& h) {
  const int H = kv.H;
  if (kv.n_seq >= 8) {
    const int local = blockIdx.x >> 3;
    s = (blockIdx.x & 7) + 8 * (local / H);
    h = local % H;
    return s < kv.n_seq;
  }
  s = blockIdx.x / H;
  h = blockIdx.x % H;
  return true;
}

// NL = version - 1 delta layers (versions 2..v); the previous version is the
// chain through layer NL - 1.
template <int NL, bool FUSE, int BITS>
__global__ __launch_bounds__(64 * kDecWaves) __attribute__((amdgpu_waves_per_eu(4)))
void k_decode_lazy(KvView kv, RowArgs a, CommitArgs cm) {
  const int H = kv.H;
  int s, h;
  if (!dec_map(kv, s, h)) return;
  const int sh = s * H + h;
  if (kv.exited(s)) return;                               // uniform per workgroup
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, p = lane & 15;
  const int nk = a.n_keys;
  const int i = a.act[s];                                 // the sequence's only active row
  const int32_t* sel = a.keys + static_cast<int64_t>(sh) * nk;

  extern __shared__ __align__(16) uint8_t s_dyn[];
  i32x4* s_sl = reinterpret_cast<i32x4*>(s_dyn);         // [nk] slot rows (layers 2..5)
  int32_t* s_j = reinterpret_cast<int32_t*>(s_sl + nk);  // [nk] key positions
  float* lg_cur = reinterpret_cast<float*>(s_j + nk);    // [nk] logits, this loop
  float* lg_prev = lg_cur + nk;                           // [nk] logits, previous loop
  __shared__ float s_mzm[kDecWaves][3];
  __shared__ float s_acc[kDecWaves][2][kDecD];

  if (FUSE && wave == kDecWaves - 1) {
    // this row's records of layer `version` (groups 0, 1: K, V) and, for
    // head 0, its slot-table entry; the other waves stage the keys meanwhile
    if (g < 2) {
      const int64_t src_rows = cm.src_compact ? 1 : kv.N;
      const int64_t src_elem = ((static_cast<int64_t>(s) * src_rows + (cm.src_compact ? 0 : i)) * H + h) * kDecD;
      commit_row<FL_BF16>(kv, cm.arena, a.version, s, i, h, g, cm.slot_base, g ? cm.v_new : cm.k_new, src_elem, p);
    }
    if (h == 0) {
      int32_t* col = reinterpret_cast<int32_t*>(cm.arena + kv.slot_table) + (a.version - 2);
      if (cm.reset) {
        for (int jj = lane; jj < kv.N; jj += 64)
          col[(static_cast<int64_t>(s) * kv.N + jj) * kv.slot_pitch] = jj == i ? cm.slot_base : -1;
      } else if (lane == 0) {
        col[(static_cast<int64_t>(s) * kv.N + i) * kv.slot_pitch] = cm.slot_base;
      }
    }
  } else {
    for (int t = tid; t < nk; t += 64 * (FUSE ? kDecWaves - 1 : kDecWaves)) {
      const int j = sel[t];
      s_j[t] = j;
      s_sl[t] = *reinterpret_cast<const i32x4*>(kv.slot_row(s, j));
    }
  }
  __syncthreads();
  const int cnt = wave_count_le(s_j, nk, i);              // visible keys: a prefix of the ascending list
  const int64_t orow = (static_cast<int64_t>(s) * (a.o_compact ? 1 : kv.N) + (a.o_compact ? 0 : i)) * H + h;
  float* lse_ptr = a.lse + orow;
  const float lse_prev = *lse_ptr;
  const StepOut r = lazy_step<NL, FUSE, BITS, false>(kv, cm, s, h, i, a.q_cur, a.q_prev, a.q_compact, a.scale,
                                                     a.mixture, a.o + orow * kDecD, lse_prev, s_j, s_sl, cnt,
                                                     lg_cur, lg_prev, s_mzm, s_acc,
                                                     a.colmass + static_cast<int64_t>(sh) * kv.N, nullptr, nullptr);
  if (tid == 0) {
    if (r.valid) *lse_ptr = r.lse;
    float* st = a.stat + static_cast<int64_t>(sh) * 4;
    st[0] = lse_prev; st[1] = r.lse; st[2] = r.valid ? 1.0f : 0.0f; st[3] = 0.0f;
  }
}

// LDS of the multi-loop kernel besides its dynamic part (the column-mass row
// and the staged keys).
struct LoopsShared {
  float mzm[kDecWaves][3];
  float acc[kDecWaves][2][kDecD];
  float trk[2][2][kDecD];               // the new token's versions: [version parity][K, V][d]
  float lse;
  TopkLds<64 * kDecWaves> topk;
};

// Loop L of the multi-loop kernel (L is a template argument so that the
// per-loop pointers are read at fixed kernel-argument offsets).
template <int L, int BITS, int EPT>
__device__ __forceinline__ void loops_iter(const KvView& kv, const DecLoopsArgs& a, int s, int h, int i,
                                           int64_t orow, float* s_c, i32x4* s_sl, int32_t* s_j, float* lg_cur,
                                           float* lg_prev, LoopsShared& sm) {
  const int H = kv.H, N = kv.N, nk = a.n_keys, sh = s * H + h;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, p = lane & 15;
  int z;                                                  // an opaque 0 (see lazy_step)
  asm volatile("s_mov_b32 %0, 0" : "=s"(z));
  __syncthreads();                                        // the previous loop's column mass is in place
  topk_block<float, EPT, 64 * kDecWaves>(N, nk, [&](int64_t t) { return s_c[t]; },
                                         [&](int pos, int32_t idx) { s_j[pos] = idx; }, sm.topk);
  __syncthreads();
  const float* trk_prev = &sm.trk[(L - 1) & 1][0][0];
  float* trk_cur = &sm.trk[L & 1][0][0];
  if (wave == kDecWaves - 1) {
    // the token's layer-L records (groups 0, 1: K, V) from its version L-1,
    // and version L for this loop; head 0 also sets its slot-table entry
    if (g < 2) {
      const int64_t src_rows = a.kv_compact ? 1 : N;
      const int64_t src = ((static_cast<int64_t>(s) * src_rows + (a.kv_compact ? 0 : i)) * H + h) * kDecD + 8 * p;
      float xn[8], xp[8], xo[8];
      load8<FL_BF16>(g ? a.v_new[L + z] : a.k_new[L + z], src, xn);
#pragma unroll
      for (int e = 0; e < 8; ++e) xp[e] = trk_prev[g * kDecD + 8 * p + e];
      commit_advance8(kv, a.arena, L, s, a.slot_base[L + z], h, g, xn, xp, true, p, xo);
#pragma unroll
      for (int e = 0; e < 8; ++e) trk_cur[g * kDecD + 8 * p + e] = xo[e];
    }
    if (h == 0 && lane == 0)
      reinterpret_cast<int32_t*>(a.arena + kv.slot_table)[(static_cast<int64_t>(s) * N + i) * kv.slot_pitch + (L - 2)] =
          a.slot_base[L + z];
  } else {
    for (int t = tid; t < nk; t += 64 * (kDecWaves - 1))
      s_sl[t] = *reinterpret_cast<const i32x4*>(kv.slot_row(s, s_j[t]));
  }
  if (a.keys_out) {
    int32_t* ko = a.keys_out + (static_cast<int64_t>(L - a.first) * kv.n_seq * H + sh) * nk;
    for (int t = tid; t < nk; t += 64 * kDecWaves) ko[t] = s_j[t];
  }
  __syncthreads();
  const int cnt = wave_count_le(s_j, nk, i);
  const float lse_prev = sm.lse;
  CommitArgs cm{};
  const StepOut r = lazy_step<L - 1, false, BITS, true>(kv, cm, s, h, i, a.q[L + z], a.q[L - 1 + z], a.q_compact,
                                                        a.scale, a.mixture, a.o + orow * kDecD, lse_prev, s_j, s_sl,
                                                        cnt, lg_cur, lg_prev, sm.mzm, sm.acc, s_c, trk_prev, trk_cur, z);
  __syncthreads();                                        // every thread has read the previous lse
  if (tid == 0) sm.lse = r.lse;
}

// Lazy loops first..last of one new token per sequence in one launch (one
// workgroup per (sequence, head), as k_decode_lazy).  Per loop: the keys are
// the top n_keys of the row's column mass (kept in LDS from loop to loop),
// the token's layer-l record is written (and its version l derived) by the
// last wave while the others stage the keys' slot rows, then the step above
// runs with the token's versions l-1 and l taken from LDS.  The column-mass
// row and lse leave the chip once, after the last loop.  Keys are the same
// sets, and every output the same bits, as loops of select_keys +
// k_decode_lazy.
template <int BITS, int EPT>
__global__ __launch_bounds__(64 * kDecWaves) __attribute__((amdgpu_waves_per_eu(4)))
void k_decode_loops(KvView kv, DecLoopsArgs a) {
  const int H = kv.H;
  int s, h;
  if (!dec_map(kv, s, h)) return;
  const int sh = s * H + h;
  if (kv.exited(s)) return;                               // uniform per workgroup
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, p = lane & 15;
  const int nk = a.n_keys, N = kv.N;
  const int i = a.act[s];

  extern __shared__ __align__(16) uint8_t s_dyn[];
  float* s_c = reinterpret_cast<float*>(s_dyn);                  // [N] column-mass row
  i32x4* s_sl = reinterpret_cast<i32x4*>(s_c + ((N + 3) & ~3));  // [nk] slot rows
  int32_t* s_j = reinterpret_cast<int32_t*>(s_sl + nk);          // [nk] key positions
  float* lg_cur = reinterpret_cast<float*>(s_j + nk);
  float* lg_prev = lg_cur + nk;
  __shared__ LoopsShared sm;

  float* c_glob = a.colmass + static_cast<int64_t>(sh) * N;
  for (int t = tid; t < N; t += 64 * kDecWaves) s_c[t] = c_glob[t];
  const int64_t orow = (static_cast<int64_t>(s) * (a.o_compact ? 1 : N) + (a.o_compact ? 0 : i)) * H + h;
  if (tid == 0) sm.lse = a.lse[orow];
  // the token's version first-1 (its records so far were written by earlier calls)
  if (wave == 0 && g < 2) {
    float x[8] = {};
    recon8<FL_BF16>(kv, g, s, h, i, a.first - 1, p, x, nullptr);
#pragma unroll
    for (int e = 0; e < 8; ++e) sm.trk[(a.first - 1) & 1][g][8 * p + e] = x[e];
  }
  // straight-line code per version (a loop over the versions made the
  // compiler keep every loop-invariant argument live across all of them)
  if (a.first <= 2 && 2 <= a.last) loops_iter<2, BITS, EPT>(kv, a, s, h, i, orow, s_c, s_sl, s_j, lg_cur, lg_prev, sm);
  if (a.first <= 3 && 3 <= a.last) loops_iter<3, BITS, EPT>(kv, a, s, h, i, orow, s_c, s_sl, s_j, lg_cur, lg_prev, sm);
  if (a.first <= 4 && 4 <= a.last) loops_iter<4, BITS, EPT>(kv, a, s, h, i, orow, s_c, s_sl, s_j, lg_cur, lg_prev, sm);
  if (a.first <= 5 && 5 <= a.last) loops_iter<5, BITS, EPT>(kv, a, s, h, i, orow, s_c, s_sl, s_j, lg_cur, lg_prev, sm);
  __syncthreads();
  for (int t = tid; t < N; t += 64 * kDecWaves) c_glob[t] = s_c[t];
  if (tid == 0) a.lse[orow] = sm.lse;
}

// Full (dense) loop over the base of one new token per sequence: keys 0..i
// of the bf16 base, no delta chain.  Key t goes to 16-lane group t mod 32 in
// steps of 32*U keys (each step of the workgroup reads 32*U consecutive key
// rows); the next step's U keys per group are in flight while the current
// ones compute.  The base rows are bf16 already, so the logits are dot2
// products of the loaded words and only V is widened.
template <int U>
__global__ __launch_bounds__(64 * kDecWaves) __attribute__((amdgpu_waves_per_eu(4)))
void k_decode_full(KvView kv, RowArgs a) {
  const int sh = blockIdx.x;
  const int H = kv.H;
  const int s = sh / H, h = sh % H;
  if (kv.exited(s)) return;                               // uniform per workgroup
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, p = lane & 15;
  const int i = a.act[s];                                 // the sequence's only row
  const int cnt = i + 1;                                  // keys 0..i

  extern __shared__ float s_lgf[];                        // [N] logits
  __shared__ float s_mz[kDecWaves][2];
  __shared__ float s_ac[kDecWaves][kDecD];

  const uint8_t* A = kv.arena;
  const int64_t row_bytes = static_cast<int64_t>(kv.N) * kDecD * 2;
  const int64_t rowb = (static_cast<int64_t>(s) * H + h) * row_bytes;
  const __amdgpu_buffer_rsrc_t rK = range_of(A + kv.base[0] + rowb, static_cast<uint32_t>(row_bytes));
  const __amdgpu_buffer_rsrc_t rV = range_of(A + kv.base[1] + rowb, static_cast<uint32_t>(row_bytes));
  const uint32_t lane_b = 16 * p;
  const int64_t qoff = ((static_cast<int64_t>(s) * (a.q_compact ? 1 : kv.N) + (a.q_compact ? 0 : i)) * H + h) * kDecD;
  const u32x4_t qc = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(a.q_cur) + qoff + 8 * p);
  const int64_t orow = (static_cast<int64_t>(s) * (a.o_compact ? 1 : kv.N) + (a.o_compact ? 0 : i)) * H + h;

  struct Rows { u32x4_t kb[U], vb[U]; };
  auto issue = [&](int k, Rows& r) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = wave * 4 + g + 32 * (U * k + u);
      const uint32_t ob = t < cnt ? static_cast<uint32_t>(t) * (kDecD * 2) + lane_b : kOut;
      r.kb[u] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rK, ob, 0, 0));
      r.vb[u] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rV, ob, 0, 0));
    }
  };
  float M = -INFINITY, Z = 0.0f;
  float acc[8] = {};
  auto consume = [&](int k, const Rows& r) {
    float sc[U];
    float tmax = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = wave * 4 + g + 32 * (U * k + u);
      const uint32_t kw[4] = {r.kb[u][0], r.kb[u][1], r.kb[u][2], r.kb[u][3]};
      sc[u] = group_sum<16>(dot_bf16x8(kw, qc)) * a.scale;
      if (t < cnt) {
        if (p == 0) s_lgf[t] = sc[u];
        tmax = fmaxf(tmax, sc[u]);
      } else {
        sc[u] = -INFINITY;                                 // past the row: weight 0
      }
    }
    if (tmax == -INFINITY) return;                        // uniform per 16-lane group
    const float Mn = fmaxf(M, tmax);
    const float corr = __expf(M - Mn);
    Z *= corr;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= corr;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float w = __expf(sc[u] - Mn);
      Z += w;
      const uint32_t vw[4] = {r.vb[u][0], r.vb[u][1], r.vb[u][2], r.vb[u][3]};
      axpy_bf16x8(acc, 1.0f, w, vw);
    }
    M = Mn;
  };

  const int nsteps = cnt > wave * 4 ? (cnt - wave * 4 + 32 * U - 1) / (32 * U) : 0;
  Rows ra, rb;
  issue(0, ra);
  for (int k = 0; k < nsteps; k += 2) {
    issue(k + 1, rb);
    consume(k, ra);
    if (k + 1 >= nsteps) break;
    issue(k + 2, ra);
    consume(k + 1, rb);
  }

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
  }
  if (lane == 0) { s_mz[wave][0] = M; s_mz[wave][1] = Z; }
  if (g == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) s_ac[wave][8 * p + e] = acc[e];
  }
  __syncthreads();
  float Mt = -INFINITY;
#pragma unroll
  for (int w = 0; w < kDecWaves; ++w) Mt = fmaxf(Mt, s_mz[w][0]);
  float Zt = 0.0f;
#pragma unroll
  for (int w = 0; w < kDecWaves; ++w) {
    const float cw = (s_mz[w][0] == -INFINITY) ? 0.0f : __expf(s_mz[w][0] - Mt);
    Zt = fmaf(s_mz[w][1], cw, Zt);
  }
  if (tid < kDecD) {
    float ov = 0.0f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float cw = (s_mz[w][0] == -INFINITY) ? 0.0f : __expf(s_mz[w][0] - Mt);
      ov = fmaf(s_ac[w][tid], cw, ov);
    }
    a.o[orow * kDecD + tid] = ov / Zt;
  }
  const float lnew = Mt + __logf(Zt);
  if (tid == 0) {
    a.lse[orow] = lnew;
    float* st = a.stat + static_cast<int64_t>(sh) * 4;
    st[0] = lnew; st[1] = lnew; st[2] = 1.0f; st[3] = 0.0f;
  }
  // column mass of the only row: c_j = p_ij, 0 past the row
  float* c = a.colmass + static_cast<int64_t>(sh) * kv.N;
  for (int t = tid; t < kv.N; t += 64 * kDecWaves) c[t] = t < cnt ? __expf(s_lgf[t] - lnew) : 0.0f;
}

bool launch_decode_full(const RowArgs& a, const KvView& kv, hipStream_t st, hipError_t* err) {
  if (kv.dtype != FL_BF16 || kv.d != kDecD || a.n_act != 1 || a.act == nullptr || a.version != 1 ||
      static_cast<size_t>(kv.N) * 4 > kDecMaxFullLds || static_cast<uint64_t>(kv.N) * kDecD * 2 > 0x7FFFFFFFull)
    return false;
  const int sh = kv.n_seq * kv.H;
  TimedLaunch t(st, "rows_attend_full");
  hipLaunchKernelGGL((k_decode_full<4>), dim3(sh), dim3(64 * kDecWaves), static_cast<size_t>(kv.N) * 4, st, kv, a);
  *err = hipGetLastError();
  return true;
}

bool launch_decode_lazy(const RowArgs& a, const KvView& kv, const CommitArgs& cm, bool fuse, hipStream_t st,
                        hipError_t* err) {
  const int nl = a.version - 1;
  if (kv.dtype != FL_BF16 || kv.d != kDecD || (kv.bits != 4 && kv.bits != 2) || a.n_act != 1 || nl < 1 ||
      nl > kDecMaxLayers ||
      a.n_keys > kDecMaxKeys)
    return false;
  // every range must fit a buffer descriptor, with offsets below 2^31
  const uint64_t lim = 0x7FFFFFFFull;
  if (static_cast<uint64_t>(kv.N) * kDecD * 2 > lim) return false;
  for (int l = 2; l <= a.version; ++l) {
    const uint64_t cap = static_cast<uint64_t>(kv.cap[l]);
    if (cap * kv.H * kDecD > lim) return false;
  }
  const int sh = kv.n_seq >= 8 ? (kv.n_seq + 7) / 8 * 8 * kv.H : kv.n_seq * kv.H;   // grid (see the kernel's mapping)
  const size_t lds = static_cast<size_t>(a.n_keys) * (16 + 4 + 4 + 4);
  TimedLaunch t(st, fuse ? "rows_attend_commit_lazy" : "rows_attend_lazy");
#define FL_DEC_B(NLV, B)                                                                                   \
  do {                                                                                                       \
    if (fuse) hipLaunchKernelGGL((k_decode_lazy<NLV, true, B>), dim3(sh), dim3(64 * kDecWaves), lds, st, kv, a, cm); \
    else hipLaunchKernelGGL((k_decode_lazy<NLV, false, B>), dim3(sh), dim3(64 * kDecWaves), lds, st, kv, a, cm);     \
  } while (0)
#define FL_DEC(NLV)                                         \
  do {                                                      \
    if (kv.bits == 4) FL_DEC_B(NLV, 4); else FL_DEC_B(NLV, 2); \
  } while (0)
  switch (nl) {
    case 1: FL_DEC(1); break;
    case 2: FL_DEC(2); break;
    case 3: FL_DEC(3); break;
    default: FL_DEC(4); break;
  }
#undef FL_DEC
#undef FL_DEC_B
  *err = hipGetLastError();
  return true;
}

bool launch_decode_loops(const DecLoopsArgs& a, const KvView& kv, hipStream_t st, hipError_t* err) {
  if (kv.dtype != FL_BF16 || kv.d != kDecD || (kv.bits != 4 && kv.bits != 2) || a.first < 2 ||
      a.last - 1 > kDecMaxLayers || a.last < a.first || a.n_keys > kDecMaxKeys || kv.N > kDecLoopsMaxN)
    return false;
  const uint64_t lim = 0x7FFFFFFFull;
  if (static_cast<uint64_t>(kv.N) * kDecD * 2 > lim) return false;
  for (int l = 2; l <= a.last; ++l)
    if (static_cast<uint64_t>(kv.cap[l]) * kv.H * kDecD > lim) return false;
  const int sh = kv.n_seq >= 8 ? (kv.n_seq + 7) / 8 * 8 * kv.H : kv.n_seq * kv.H;
  const size_t lds = static_cast<size_t>((kv.N + 3) & ~3) * 4 + static_cast<size_t>(a.n_keys) * (16 + 4 + 4 + 4);
  TimedLaunch t(st, "decode_loops");
  // the column-mass row takes the dynamic LDS past the default limit
#define FL_LOOPS(B, E)                                                                                      \
  do {                                                                                                       \
    const hipError_t ea = hipFuncSetAttribute(reinterpret_cast<const void*>(k_decode_loops<B, E>),           \
                                              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds)); \
    if (ea != hipSuccess) { *err = ea; return true; }                                                        \
    hipLaunchKernelGGL((k_decode_loops<B, E>), dim3(sh), dim3(64 * kDecWaves), lds, st, kv, a);             \
  } while (0)
  static_assert(kDecLoopsMaxN <= 64 * kDecWaves * 16, "16 column-mass entries per thread");
  if (kv.bits == 4) FL_LOOPS(4, 16); else FL_LOOPS(2, 16);
#undef FL_LOOPS
  *err = hipGetLastError();
  return true;
}

}  // namespace fl
