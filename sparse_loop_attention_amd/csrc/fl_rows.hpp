// Arguments of the per-row attention kernels (few active rows against many
// keys) and the launch of their decode-shaped specialisation.
#pragma once
#include "fl_commit.hpp"

namespace fl {

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
  int64_t key_slots;        // logit row length (n_keys or N)
  int32_t mixture;          // LAZY: o = m*otilde + (1-m)*o_prev instead of m*otilde + o_prev - a
  float* logit;             // [2][sh][rows][key_slots]
  float* stat;              // [sh][rows][4] = lse_prev, lse_new, valid, -
  const int32_t* exit_flags;  // [n_seq] or null: nonzero = skip the sequence (early exit)
};

// Number of entries of the ascending array a[0..n) that are <= v, by a
// 64-way search across the wave: each round the lanes probe 64 evenly spaced
// entries and the ballot of "<= v" (a prefix of the lanes) narrows the range
// 64-fold, so 820 entries take two rounds of loads instead of ten dependent
// ones.  Every lane of the wave must call it; every lane gets the result.
__device__ __forceinline__ int wave_count_le(const int32_t* a, int n, int v) {
  const int lane = threadIdx.x & 63;
  int lo = 0, hi = n;                                     // the count lies in [lo, hi]
  while (lo < hi) {
    const int step = (hi - lo + 63) / 64;
    const int pos = lo + lane * step;
    const uint64_t le = __ballot(pos < hi && a[pos] <= v);
    const int c = __popcll(le);                           // entries lo, lo+step, ... lo+(c-1)*step are <= v
    if (c == 0) return lo;
    const int top = min(hi, lo + c * step);               // entries from here on are > v
    lo = lo + (c - 1) * step + 1;
    hi = top;
  }
  return lo;
}

// Lazy attention of one active row per sequence (decode) on a bf16 store
// with 4- or 2-bit deltas and head_dim 128, at versions 2..5.  Returns false (and
// launches nothing) when the call is outside that shape; otherwise launches
// and sets *err.
bool launch_decode_lazy(const RowArgs& a, const KvView& kv, const CommitArgs& cm, bool fuse, hipStream_t st,
                        hipError_t* err);
// The full loop over the base (version 1) of one row per sequence, same
// shape limits (head_dim 128, bf16, N <= 10240); false when outside them.
bool launch_decode_full(const RowArgs& a, const KvView& kv, hipStream_t st, hipError_t* err);

// Lazy decode loops first..last in one launch (flashloop_decode_loops).
struct DecLoopsArgs {
  uint8_t* arena;                          // writable arena (the token's records, its slot entries)
  const int32_t* act;                      // [n_seq] the new token's position
  int32_t first, last;                     // loops (versions) first..last
  const void* q[FL_MAX_VERSIONS + 1];      // q[l], l = first-1..last
  const void* k_new[FL_MAX_VERSIONS + 1];  // the token's new rows, l = first..last
  const void* v_new[FL_MAX_VERSIONS + 1];
  int32_t slot_base[FL_MAX_VERSIONS + 1];  // the token's record slot in layer l
  int32_t q_compact, o_compact, kv_compact;
  int32_t n_keys;
  float* o;
  float* lse;
  float* colmass;
  int32_t* keys_out;                       // [last-first+1][n_seq*H][n_keys] or null
  float scale;
  int32_t mixture;
};
// Shape limits: bf16 store, head_dim 128, 4- or 2-bit codes, versions up to
// 5, n_keys <= 1536, N <= 8192.  Returns false (nothing launched) outside them.
bool launch_decode_loops(const DecLoopsArgs& a, const KvView& kv, hipStream_t st, hipError_t* err);

}  // namespace fl
