// Device-side helpers shared by the FlashLoop HIP kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "flashloop.h"

namespace fl {

constexpr int kWave = 64;
typedef int i32x4 __attribute__((ext_vector_type(4)));   // 16-byte int vector (stays in registers)

// ---- scalar conversions ----------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// Two float32 -> two bfloat16, round to nearest even (one v_cvt_pk_bf16_f32);
// a in the low half.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}
// float32 -> bfloat16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return static_cast<uint16_t>(pack_bf16x2(f, 0.0f) & 0xFFFFu);
}
// Value of f rounded to the nearest bfloat16 (ties to even), as float32.
__device__ __forceinline__ float round_bf16(float f) { return __uint_as_float(pack_bf16x2(f, 0.0f) << 16); }
__device__ __forceinline__ float half_bits_to_f32(uint16_t h) {
  _Float16 v = __builtin_bit_cast(_Float16, h);
  return static_cast<float>(v);
}
// float32 -> binary16 bits with round-to-nearest-even (hardware cvt, default mode).
__device__ __forceinline__ uint16_t f32_to_half_bits(float f) {
  _Float16 v = static_cast<_Float16>(f);
  return __builtin_bit_cast(uint16_t, v);
}

// ---- 8-element vector loads (16 B of bf16 or 32 B of fp32) -----------------
// Native clang vector types (not HIP's struct vectors) so that the values
// stay in registers.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t elem, float out[8]) {
  if constexpr (DT == FL_BF16) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(base) + elem);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(v[i] << 16);
      out[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
    }
  } else {
    const f32x4_t* p = reinterpret_cast<const f32x4_t*>(static_cast<const float*>(base) + elem);
    const f32x4_t a = p[0], b = p[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[i] = a[i];
      out[4 + i] = b[i];
    }
  }
}

template <int DT>
__device__ __forceinline__ void store8(void* base, int64_t elem, const float in[8]) {
  if constexpr (DT == FL_BF16) {
    u32x4_t w;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = pack_bf16x2(in[2 * i], in[2 * i + 1]);
    *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(base) + elem) = w;
  } else {
    f32x4_t* p = reinterpret_cast<f32x4_t*>(static_cast<float*>(base) + elem);
    p[0] = f32x4_t{in[0], in[1], in[2], in[3]};
    p[1] = f32x4_t{in[4], in[5], in[6], in[7]};
  }
}

// ---- device view of the KV arena ------------------------------------------
// Records are token-major: record (s, slot, h, which) with which = 0 for K and
// 1 for V has index ((s * cap + slot) * H + h) * 2 + which; its codes are
// d*bits/8 bytes (lane p of a 16-lane group owns the `bits` bytes of elements
// [8p, 8p+8)) and its scales d/group binary16 values (one per 2^gshift lanes).
struct KvView {
  const uint8_t* arena;
  int32_t n_seq, H, d, N, T, dtype;
  int32_t cap[FL_MAX_VERSIONS + 1];
  uint64_t base[2];                              // K, V
  uint64_t slot_table;                           // [n_seq][N][slot_pitch] int32
  int32_t slot_pitch;
  uint64_t codes[FL_MAX_VERSIONS + 1];
  uint64_t scales[FL_MAX_VERSIONS + 1];
  int32_t bits;                                  // bits per delta code: 4 or 2
  int32_t gshift;                                // log2(lanes per scale group): 2 (group 32) or 3 (64)
  const int32_t* exit_flags;                     // [n_seq] or null: nonzero = the sequence has exited

  __device__ __forceinline__ bool exited(int s) const { return exit_flags && exit_flags[s]; }

  // the slots of token j of sequence s in layers 2, 3, ... (entry l-2)
  __device__ __forceinline__ const int32_t* slot_row(int s, int j) const {
    return reinterpret_cast<const int32_t*>(arena + slot_table) +
           (static_cast<int64_t>(s) * N + j) * slot_pitch;
  }
  __device__ __forceinline__ int64_t record(int l, int s, int slot, int h, int which) const {
    return ((static_cast<int64_t>(s) * cap[l] + slot) * H + h) * 2 + which;
  }
  // codes of lane p (8 elements) of record `rec` in layer l, right-aligned
  __device__ __forceinline__ uint32_t load_codes(int l, int64_t rec, int p) const {
    const uint8_t* b = arena + codes[l] + rec * (d * bits / 8) + p * bits;
    return bits == 4 ? *reinterpret_cast<const uint32_t*>(b) : *reinterpret_cast<const uint16_t*>(b);
  }
  __device__ __forceinline__ int64_t scale_index(int64_t rec, int p) const {
    return rec * (d >> (3 + gshift)) + (p >> gshift);
  }
  __device__ __forceinline__ uint16_t load_scale(int l, int64_t rec, int p) const {
    return reinterpret_cast<const uint16_t*>(arena + scales[l])[scale_index(rec, p)];
  }
};

// Adds the deltas of 8 `bits`-wide two's-complement codes (element e in bits
// [bits*e, bits*e + bits) of `codes`), scale `s`, to x[0..7].
__device__ __forceinline__ void add_codes8(uint32_t codes, int bits, float s, float x[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = bits == 4 ? static_cast<int32_t>(codes << (28 - 4 * e)) >> 28      // sign-extend field e
                            : static_cast<int32_t>(codes << (30 - 2 * e)) >> 30;
    x[e] = x[e] + static_cast<float>(c) * s;
  }
}

// Adds the layer-l record of token slot `slot` (sequence s, head h, K or V) to
// the 8 elements [8p, 8p+8) of x.
__device__ __forceinline__ void add_delta8(const KvView& kv, int which, int l, int s, int h, int slot, int p,
                                           float x[8]) {
  const int64_t rec = kv.record(l, s, slot, h, which);
  add_codes8(kv.load_codes(l, rec, p), kv.bits, half_bits_to_f32(kv.load_scale(l, rec, p)), x);
}

// Attention consumes the reconstruction in the store's working dtype: a
// bf16 store's float32 reconstruction is rounded to bf16 (the int4 chain
// itself stays float32).
template <int DT>
__device__ __forceinline__ void to_working8(float x[8]) {
  if constexpr (DT == FL_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = pack_bf16x2(x[2 * i], x[2 * i + 1]);
      x[2 * i] = __uint_as_float(w << 16);
      x[2 * i + 1] = __uint_as_float(w & 0xFFFF0000u);
    }
  }
}

// Reconstructs elements [8p, 8p+8) of token j (sequence s, head h) at
// version v; if `prev` is non-null also returns version v-1 there (v >= 2).
template <int DT>
__device__ __forceinline__ void recon8(const KvView& kv, int which, int s, int h, int j, int v, int p, float x[8],
                                       float* prev) {
  const void* base = kv.arena + kv.base[which];
  load8<DT>(base, ((static_cast<int64_t>(s) * kv.H + h) * kv.N + j) * kv.d + 8 * p, x);
  const int32_t* sr = v >= 2 ? kv.slot_row(s, j) : nullptr;
  for (int l0 = 2; l0 <= v; l0 += 4) {
    const i32x4 sl = *reinterpret_cast<const i32x4*>(sr + (l0 - 2));
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int l = l0 + b;
      if (l > v) break;
      if (prev != nullptr && l == v) {
#pragma unroll
        for (int e = 0; e < 8; ++e) prev[e] = x[e];
      }
      if (sl[b] >= 0 && sl[b] < kv.cap[l]) add_delta8(kv, which, l, s, h, sl[b], p, x);  // out-of-range = absent
    }
  }
}

// K and V of U keys at once (elements [8p, 8p+8) of this lane).  Layers are
// walked in batches of LB: the slot lookups of a whole batch are issued
// together, then every record load of the batch, so a 16-lane group keeps
// U x LB chain reads in flight instead of one dependent pair per layer.  Keys
// with ok[u] == false give zeros.  With PREV, kp/vp receive version v-1.
// `pre[u]`, when given, holds key u's slots of layers 2..5 (read earlier, e.g.
// staged in LDS), so that only the base and record loads remain in the walk.
template <int DT, int U, bool PREV>
__device__ __forceinline__ void recon_kv(const KvView& kv, int s, int h, const int (&j)[U], const bool (&ok)[U],
                                         int v, int p, float (&k)[U][8], float (&vv)[U][8], float (&kp)[U][8],
                                         float (&vp)[U][8], const i32x4* pre = nullptr) {
  constexpr int LB = 4;                                   // one 16-byte slot read per key and batch
  const int d = kv.d;
  const int64_t row = (static_cast<int64_t>(s) * kv.H + h) * kv.N;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (ok[u]) {
      load8<DT>(kv.arena + kv.base[0], (row + j[u]) * d + 8 * p, k[u]);
      load8<DT>(kv.arena + kv.base[1], (row + j[u]) * d + 8 * p, vv[u]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) k[u][e] = vv[u][e] = 0.0f;
    }
  }
  for (int l0 = 2; l0 <= v; l0 += LB) {
    int slot[LB][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      i32x4 sl = i32x4{-1, -1, -1, -1};
      if (ok[u]) sl = (pre != nullptr && l0 == 2) ? pre[u] : *reinterpret_cast<const i32x4*>(kv.slot_row(s, j[u]) + (l0 - 2));
#pragma unroll
      for (int b = 0; b < LB; ++b) {
        const int l = l0 + b;
        slot[b][u] = (l <= v && sl[b] < kv.cap[l]) ? sl[b] : -1;             // out-of-range = absent
      }
    }
    uint32_t ck[LB][U], cv[LB][U];
    uint16_t sk[LB][U], sv[LB][U];
#pragma unroll
    for (int b = 0; b < LB; ++b)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (slot[b][u] >= 0) {
          const int l = l0 + b;
          const int64_t rec = kv.record(l, s, slot[b][u], h, 0);
          ck[b][u] = kv.load_codes(l, rec, p);
          cv[b][u] = kv.load_codes(l, rec + 1, p);
          sk[b][u] = kv.load_scale(l, rec, p);
          sv[b][u] = kv.load_scale(l, rec + 1, p);
        }
      }
#pragma unroll
    for (int b = 0; b < LB; ++b) {
      if (PREV && l0 + b == v) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int e = 0; e < 8; ++e) { kp[u][e] = k[u][e]; vp[u][e] = vv[u][e]; }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (slot[b][u] >= 0) {
          add_codes8(ck[b][u], kv.bits, half_bits_to_f32(sk[b][u]), k[u]);
          add_codes8(cv[b][u], kv.bits, half_bits_to_f32(sv[b][u]), vv[u]);
        }
      }
    }
  }
}

// ---- wave reductions -------------------------------------------------------
// 16-lane (one DPP row) sum: quad swaps, then half-row and row mirrors; every
// lane of the row ends with the row total.  Pure VALU, no LDS round trip.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppQuadSwap1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(WIDTH == 16 || WIDTH == 4, "DPP reductions cover 4 or 16 lanes");
  v += dpp_mov<kDppQuadSwap1>(v);
  v += dpp_mov<kDppQuadSwap2>(v);
  if constexpr (WIDTH == 16) {
    v += dpp_mov<kDppRowHalfMirror>(v);
    v += dpp_mov<kDppRowMirror>(v);
  }
  return v;
}
template <int WIDTH>
__device__ __forceinline__ float group_max(float v) {
  static_assert(WIDTH == 16 || WIDTH == 8 || WIDTH == 4, "DPP reductions cover 4, 8 or 16 lanes");
  v = fmaxf(v, dpp_mov<kDppQuadSwap1>(v));
  v = fmaxf(v, dpp_mov<kDppQuadSwap2>(v));
  if constexpr (WIDTH >= 8) v = fmaxf(v, dpp_mov<kDppRowHalfMirror>(v));
  if constexpr (WIDTH == 16) v = fmaxf(v, dpp_mov<kDppRowMirror>(v));
  return v;
}
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

}  // namespace fl
