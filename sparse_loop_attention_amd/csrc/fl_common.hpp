// Device-side helpers shared by the FlashLoop HIP kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "flashloop.h"

namespace fl {

constexpr int kWave = 64;

// ---- scalar conversions ----------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// float32 -> bfloat16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
// Value of f rounded to the nearest bfloat16 (ties to even), as float32.
__device__ __forceinline__ float round_bf16(float f) {
  return __uint_as_float(static_cast<uint32_t>(f32_to_bf16(f)) << 16);
}
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
template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t elem, float out[8]) {
  if constexpr (DT == FL_BF16) {
    const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem);
    const float4 a = p[0], b = p[1];
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  }
}

template <int DT>
__device__ __forceinline__ void store8(void* base, int64_t elem, const float in[8]) {
  if constexpr (DT == FL_BF16) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = static_cast<uint32_t>(f32_to_bf16(in[2 * i])) |
             (static_cast<uint32_t>(f32_to_bf16(in[2 * i + 1])) << 16);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + elem) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + elem);
    p[0] = make_float4(in[0], in[1], in[2], in[3]);
    p[1] = make_float4(in[4], in[5], in[6], in[7]);
  }
}

// ---- device view of the KV arena ------------------------------------------
struct KvView {
  const uint8_t* arena;
  int32_t n_seq, H, d, N, T, dtype;
  int32_t cap[FL_MAX_VERSIONS + 1];
  uint64_t base[2];                              // K, V
  uint64_t slot_map[FL_MAX_VERSIONS + 1];
  uint64_t codes[2][FL_MAX_VERSIONS + 1];
  uint64_t scales[2][FL_MAX_VERSIONS + 1];

  __device__ __forceinline__ const int32_t* slots(int l) const {
    return reinterpret_cast<const int32_t*>(arena + slot_map[l]);
  }
};

// Adds the layer-l record of token slot `slot` (head row `row` = s*H+h) to the
// 8 elements [8p, 8p+8) of x.
__device__ __forceinline__ void add_delta8(const KvView& kv, int which, int l, int64_t row, int slot,
                                           int p, float x[8]) {
  const int d = kv.d;
  const int64_t rec = row * kv.cap[l] + slot;
  const uint32_t codes =
      *reinterpret_cast<const uint32_t*>(kv.arena + kv.codes[which][l] + rec * (d / 2) + 4 * p);
  const uint16_t sbits =
      *reinterpret_cast<const uint16_t*>(kv.arena + kv.scales[which][l] + (rec * (d / 32) + (p >> 2)) * 2);
  const float s = half_bits_to_f32(sbits);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = static_cast<int>(static_cast<int32_t>(codes << (28 - 4 * e)) >> 28);  // sign-extend nibble e
    x[e] = x[e] + static_cast<float>(c) * s;
  }
}

// Attention consumes the reconstruction in the store's working dtype: a
// bf16 store's float32 reconstruction is rounded to bf16 (the int4 chain
// itself stays float32).
template <int DT>
__device__ __forceinline__ void to_working8(float x[8]) {
  if constexpr (DT == FL_BF16) {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = round_bf16(x[e]);
  }
}

// Reconstructs elements [8p, 8p+8) of token j (head row `row`, sequence s) at
// version v; if `prev` is non-null also returns version v-1 there (v >= 2).
template <int DT>
__device__ __forceinline__ void recon8(const KvView& kv, int which, int s, int64_t row, int j, int v,
                                       int p, float x[8], float* prev) {
  const void* base = kv.arena + kv.base[which];
  load8<DT>(base, (row * kv.N + j) * kv.d + 8 * p, x);
  for (int l = 2; l <= v; ++l) {
    if (prev != nullptr && l == v) {
#pragma unroll
      for (int e = 0; e < 8; ++e) prev[e] = x[e];
    }
    const int slot = kv.slots(l)[static_cast<int64_t>(s) * kv.N + j];
    if (slot >= 0 && slot < kv.cap[l]) add_delta8(kv, which, l, row, slot, p, x);  // out-of-range = absent
  }
}

// ---- wave reductions -------------------------------------------------------
template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = WIDTH / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
template <int WIDTH>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = WIDTH / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

}  // namespace fl
