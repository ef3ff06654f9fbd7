// Device pieces of the low-bit delta commit, shared by the commit kernel and
// by the kernels that fuse the commit into an attention call.
//
// Page "FlashLoop: Fast and Memory-Efficient Looped Transformers via Lazy
// Updates", section "FlashLoop combines three kinds of savings", paragraph 3
// (a 4-bit difference from the previous state, written for active tokens
// only) and paragraph 4 (the KV update and compression are fused with the
// compute).  Group format: 32 (or 64) consecutive elements of a head row
// share one binary16 scale s = f16_rne(min(absmax/q, 65504)); code =
// clamp(rint(d/s), -q, q), 0 when s == 0, with q = 2^(bits-1) - 1 (7 for
// 4-bit codes, 1 for 2-bit).  A 16-lane group covers a head row, lane p
// owning elements [8p, 8p+8), so a scale group is one DPP quad (or half-row).
#pragma once
#include "fl_common.hpp"

namespace fl {

// Quantises this lane's 8 deltas into `bits`-wide fields of `packed`.  All
// lanes of the scale group must call it (dead lanes pass live = false and
// contribute absmax 0).
__device__ __forceinline__ void quantize8(const KvView& kv, const float delta[8], bool live, uint32_t& packed,
                                          uint16_t& sbits, float& sc) {
  float amax = 0.0f;
  if (live) {
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(delta[e]));
  }
  amax = kv.gshift == 3 ? group_max<8>(amax) : group_max<4>(amax);
  const float qmax = static_cast<float>((1 << (kv.bits - 1)) - 1);
  const float q = fminf(amax / qmax, 65504.0f);              // correctly rounded division
  sbits = f32_to_half_bits(q);
  sc = half_bits_to_f32(sbits);
  const uint32_t mask = (1u << kv.bits) - 1u;
  packed = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    int c = 0;
    if (sc != 0.0f) c = static_cast<int>(fminf(fmaxf(__builtin_rintf(delta[e] / sc), -qmax), qmax));
    packed |= (static_cast<uint32_t>(c) & mask) << (kv.bits * e);
  }
}

// Version l of a row whose version l-1 is x_prev: the new row's quantised
// delta is added (exactly what a reader of the written record would add).
__device__ __forceinline__ void advance8(const KvView& kv, const float x_new[8], const float x_prev[8], bool live,
                                         float x_out[8]) {
  float delta[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) delta[e] = x_new[e] - x_prev[e];
  uint32_t packed;
  uint16_t sbits;
  float sc;
  quantize8(kv, delta, live, packed, sbits, sc);
#pragma unroll
  for (int e = 0; e < 8; ++e) x_out[e] = x_prev[e];
  add_codes8(packed, kv.bits, sc, x_out);
}

// Commits a head row whose version l-1 is x_prev and whose new value is x_new
// into layer l >= 2 at record slot `slot` (what commit_row writes), and
// returns version l in x_out (what a reader of the record reconstructs).
// Called by a whole 16-lane group; lane p owns elements [8p, 8p+8).
__device__ __forceinline__ void commit_advance8(const KvView& kv, uint8_t* arena_w, int l, int s, int slot, int h,
                                                int which, const float x_new[8], const float x_prev[8], bool live,
                                                int p, float x_out[8]) {
  float delta[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) delta[e] = x_new[e] - x_prev[e];
  uint32_t packed;
  uint16_t sbits;
  float sc;
  quantize8(kv, delta, live, packed, sbits, sc);
#pragma unroll
  for (int e = 0; e < 8; ++e) x_out[e] = x_prev[e];
  add_codes8(packed, kv.bits, sc, x_out);
  if (!live) return;
  const int64_t rec = kv.record(l, s, slot, h, which);
  uint8_t* cb = arena_w + kv.codes[l] + rec * (kv.d * kv.bits / 8) + p * kv.bits;
  if (kv.bits == 4) *reinterpret_cast<uint32_t*>(cb) = packed;
  else *reinterpret_cast<uint16_t*>(cb) = static_cast<uint16_t>(packed);
  if ((p & ((1 << kv.gshift) - 1)) == 0)
    reinterpret_cast<uint16_t*>(arena_w + kv.scales[l])[kv.scale_index(rec, p)] = sbits;
}

// Position of token j in the ascending active list act[0..n), or -1.
__device__ __forceinline__ int find_active(const int32_t* act, int n, int j) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (act[mid] < j) lo = mid + 1; else hi = mid;
  }
  return (lo < n && act[lo] == j) ? lo : -1;
}

// Commits one head row (sequence s, active position r = token j, head h, K or
// V) into layer l >= 2 at record slot `slot`, or into the base for l == 1.
// Called by a whole 16-lane group; lane p owns elements [8p, 8p+8).
template <int DT>
__device__ __forceinline__ void commit_row(const KvView& kv, uint8_t* arena_w, int l, int s, int j, int h, int which,
                                           int slot, const void* src, int64_t src_elem, int p) {
  const int d = kv.d;
  const bool live = 8 * p < d;
  float x[8] = {};
  if (live) load8<DT>(src, src_elem + 8 * p, x);
  if (l == 1) {
    if (live) store8<DT>(arena_w + kv.base[which], ((static_cast<int64_t>(s) * kv.H + h) * kv.N + j) * d + 8 * p, x);
    return;
  }
  float prev[8] = {}, delta[8];
  if (live) recon8<DT>(kv, which, s, h, j, l - 1, p, prev, nullptr);
#pragma unroll
  for (int e = 0; e < 8; ++e) delta[e] = x[e] - prev[e];
  uint32_t packed;
  uint16_t sbits;
  float sc;
  quantize8(kv, delta, live, packed, sbits, sc);
  if (!live) return;
  const int64_t rec = kv.record(l, s, slot, h, which);
  uint8_t* cb = arena_w + kv.codes[l] + rec * (d * kv.bits / 8) + p * kv.bits;
  if (kv.bits == 4) *reinterpret_cast<uint32_t*>(cb) = packed;
  else *reinterpret_cast<uint16_t*>(cb) = static_cast<uint16_t>(packed);
  if ((p & ((1 << kv.gshift) - 1)) == 0)
    reinterpret_cast<uint16_t*>(arena_w + kv.scales[l])[kv.scale_index(rec, p)] = sbits;
}

// Everything a fused commit needs besides the store view.
struct CommitArgs {
  uint8_t* arena;            // writable arena
  const void* k_new;
  const void* v_new;
  int32_t src_compact;       // rows of k_new/v_new by active position (1) or by token (0)
  int32_t slot_base;
  int32_t reset;             // slot entries of inactive tokens become -1
};

}  // namespace fl
