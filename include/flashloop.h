/*
 * flashloop.h -- C ABI of the FlashLoop lazy-update loop step for MI355X (gfx950).
 *
 * Source of the method: the page "FlashLoop: Fast and Memory-Efficient Looped
 * Transformers via Lazy Updates" (rit.work blog), section "FlashLoop combines
 * three kinds of savings".  Paragraph 1: early loops run in full; later loops
 * rank tokens by the change of their hidden state and recompute only the
 * active ones, the others reuse their state and KV entries.  Paragraph 2: keys
 * are chosen from the previous loop's attention statistics and the chosen group
 * keeps the previous loop's probability mass.  Paragraph 3: the KV cache is a
 * compressed base plus a chain of 4-bit corrections written only for active
 * tokens.  Paragraph 4: the selected data is gathered into dense buffers and
 * the KV update and compression are fused with the compute.
 *
 * Conventions shared by every entry point
 *  - Every tensor pointer is a HIP device pointer owned by the caller.  The
 *    library never allocates, frees or copies to the host, never synchronises,
 *    and launches only on the stream it is given (`stream` is a hipStream_t;
 *    NULL is the default stream).  All calls are asynchronous.
 *  - Layouts are row-major and contiguous.  bf16 tensors hold raw bfloat16
 *    bits (uint16); fp32 tensors hold IEEE binary32.
 *  - Index lists are int32, ascending and unique, each value in [0, N).  The
 *    caller guarantees this (the library cannot check device contents without
 *    synchronising); violating it gives unspecified results but never writes
 *    outside the buffers the descriptor and the arguments describe.
 *  - Arguments are validated on the host before any launch.  On failure the
 *    call returns a non-zero fl_status, launches nothing, and
 *    flashloop_last_error() describes the problem.  A failed launch returns
 *    FL_ERR_HIP.  No C++ exception crosses this boundary.
 *  - The library holds no state besides a thread-local error message, the
 *    optional kernel-timing registry below and the per-GPU scratch array of
 *    flashloop_attend_noalloc; calls from several threads are safe.  Calls
 *    that write the same buffers on different streams race, as any two
 *    kernels would.
 */
#ifndef FLASHLOOP_H
#define FLASHLOOP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FLASHLOOP_ABI_VERSION 5
#define FL_MAX_VERSIONS 32          /* versions 1..FL_MAX_VERSIONS */

typedef enum {
  FL_OK = 0,
  FL_ERR_ARG = 1,          /* a null pointer, a size out of range, an inconsistent argument */
  FL_ERR_UNSUPPORTED = 2,  /* valid but not implemented (e.g. head_dim outside {64, 96, 128}) */
  FL_ERR_WORKSPACE = 3,    /* workspace missing or smaller than the *_workspace_bytes query */
  FL_ERR_HIP = 4           /* a HIP launch failed; the message holds hipGetErrorString */
} fl_status;

typedef enum { FL_F32 = 0, FL_BF16 = 1 } fl_dtype;
typedef enum { FL_SEL_TOKENS = 0, FL_SEL_KEYS = 1 } fl_select_mode;
typedef enum { FL_ATTEND_FULL = 0, FL_ATTEND_LAZY = 1 } fl_attend_mode;
typedef enum {
  FL_FORMULA_COLUMN = 0,        /* o <- m*otilde + (o - a): the selected columns are updated */
  FL_FORMULA_MIXTURE = 1        /* o <- m*otilde + (1 - m)*o */
} fl_formula;
typedef enum { FL_ROWS_BY_TOKEN = 0, FL_ROWS_COMPACT = 1 } fl_row_layout;

/* ------------------------------------------------------------------------ */
/* KV store: a base (version 1) plus low-bit delta layers 2..n_versions.     */
/* (section "FlashLoop combines three kinds of savings", paragraph 3)        */
/* ------------------------------------------------------------------------ */
typedef struct {
  int32_t n_seq;        /* independent sequences (decode batch); 1 for prefill */
  int32_t n_heads;      /* H */
  int32_t head_dim;     /* d in {64, 96, 128} */
  int32_t n_tokens;     /* N positions per sequence */
  int32_t n_versions;   /* T >= 1; delta layers 2..T */
  int32_t base_dtype;   /* fl_dtype of the base, and of every K/V/Q/h input */
  int32_t group;        /* quantisation group: 32 or 64 consecutive elements of a head row;
                           must divide head_dim (FL_ERR_UNSUPPORTED otherwise) */
  int32_t delta_bits;   /* bits per delta code: 4 or 2 (0 means 4) */
  int32_t layer_cap[FL_MAX_VERSIONS + 1]; /* [l], l in 2..T: record slots per sequence in layer l */
  void* arena;          /* device memory of flashloop_kv_arena_bytes() bytes, caller-owned */
  uint64_t arena_bytes;
} fl_kv_desc;

/* Byte offsets inside the arena (every array 256-byte aligned):
 *   base_k, base_v  [n_seq][H][N][d]               base_dtype
 *   slot_table      [n_seq][N][slot_pitch]         int32: entry l-2 = record slot of token j in
 *                                                  layer l, or -1 (slot_pitch = n_versions - 1
 *                                                  rounded up to 4; no table when n_versions = 1)
 *   codes[l]        [n_seq][cap_l][H][2][d*b/8]    uint8: K then V codes of one head row, b =
 *                                                  delta_bits: two 4-bit codes per byte (low nibble
 *                                                  = even element) or four 2-bit codes per byte
 *                                                  (lowest bits = first element)
 *   scales[l]       [n_seq][cap_l][H][2][d/group]  binary16 bits: one scale per group
 * A token's slots of every layer sit together (one 16-byte read resolves up
 * to four layers), and records are token-major: the K and V codes of one
 * (token, head) fill one d-byte run (a 128-byte line at d = 128) and the
 * scales of all heads of a token are adjacent, so a sparse set of keys reads
 * whole lines.  The reconstruction of token j at version v is
 *   float(base[j]) + sum_{l=2..v, slot(l, j) >= 0} code * float(scale), added in float32 in increasing l. */
typedef struct {
  uint64_t base_k, base_v;
  uint64_t slot_table;
  uint64_t slot_pitch;
  uint64_t codes[FL_MAX_VERSIONS + 1];
  uint64_t scales[FL_MAX_VERSIONS + 1];
  uint64_t total_bytes;
} fl_kv_layout;

/* Fills *out with the arena layout of *desc (arena pointer not needed).
 * Returns FL_ERR_ARG / FL_ERR_UNSUPPORTED for an invalid descriptor. */
fl_status flashloop_kv_layout(const fl_kv_desc* desc, fl_kv_layout* out);

/* Bytes the caller must allocate for desc->arena; 0 if the descriptor is invalid. */
uint64_t flashloop_kv_arena_bytes(const fl_kv_desc* desc);

/* ------------------------------------------------------------------------ */
/* flashloop_kv_commit -- write one loop's K/V rows into the store.          */
/* (section "FlashLoop combines three kinds of savings", paragraph 3)        */
/* version 1: copies the rows into the base.  version l >= 2: for each active */
/* token j, head h and X in {K, V}: delta = X_new - X^(l-1) in float32, per   */
/* group: s = f16_rne(min(absmax/q, 65504)), code = clamp(rint(delta/s), -q,  */
/* q) (0 when s == 0), q = 2^(delta_bits-1) - 1 (7 for 4-bit codes, 1 for     */
/* 2-bit); records go to slots slot_base + r (r = position in                 */
/* active_idx) and slot(l, j) is set to that slot.  With reset_map != 0     */
/* every other token's slot(l, .) of the sequence is set to -1; with 0 they   */
/* are left as they are (to add rows to a layer written by an earlier call).  */
/* Inactive tokens get no entry.                                              */
/* ------------------------------------------------------------------------ */
typedef struct {
  const fl_kv_desc* kv;
  int32_t version;              /* 1..n_versions */
  const int32_t* active_idx;    /* [n_seq][n_active] ascending token positions */
  int32_t n_active;             /* 0..N; slot_base + n_active <= layer_cap[version] */
  int32_t slot_base;
  int32_t reset_map;
  const void* k_new;            /* [n_seq][R][H][d] base_dtype, R = N (rows by token) or n_active */
  const void* v_new;
  int32_t src_layout;           /* fl_row_layout of k_new / v_new */
  const int32_t* exit_flags;    /* optional [n_seq] device: sequences with a nonzero flag are
                                   skipped (their store is left as it is); see flashloop_exit_check */
} fl_commit_args;

fl_status flashloop_kv_commit(const fl_commit_args* args, void* stream);

/* ------------------------------------------------------------------------ */
/* flashloop_select -- token ranking and key selection.                      */
/* (section "FlashLoop combines three kinds of savings", paragraphs 1 and 2) */
/* TOKENS: scores[i] = sum_k (h_cur[i,k] - h_prev[i,k])^2 accumulated in     */
/*   float64; rows outside cand_idx (when given) are written as 0 without    */
/*   being read (they were carried unchanged).  Then out_idx = the k rows    */
/*   with the largest score, ties to the lower index, ascending.             */
/* KEYS: for each of n_seg segments of key_scores (float32, e.g. column mass */
/*   [n_seq*H][N]), out_idx[seg] = its top-k positions by the same rule.     */
/* -0.0 and +0.0 compare equal; NaN scores give unspecified (in-range) sets. */
/* ------------------------------------------------------------------------ */
typedef struct {
  int32_t mode;                 /* fl_select_mode */
  /* TOKENS */
  const void* h_cur;            /* [n_rows][hidden] h_dtype */
  const void* h_prev;
  int32_t h_dtype;
  int64_t n_rows;               /* 1..65536 */
  int64_t hidden;
  const int32_t* cand_idx;      /* optional, ascending; NULL = all rows */
  int32_t n_cand;
  double* scores;               /* [n_rows] output (float64), required in TOKENS mode */
  /* KEYS */
  const float* key_scores;      /* [n_seg][seg_len] */
  int32_t n_seg;
  int64_t seg_len;              /* 1..65536 */
  /* both */
  int32_t k;                    /* 0..n_rows (TOKENS) or 0..seg_len (KEYS) */
  int32_t* out_idx;             /* [n_seg][k] (TOKENS: [k]) */
} fl_select_args;

fl_status flashloop_select(const fl_select_args* args, void* stream);

/* ------------------------------------------------------------------------ */
/* flashloop_attend -- causal attention over the reconstructed K^, V^.       */
/* (section "FlashLoop combines three kinds of savings", paragraphs 2 and 4) */
/* FULL, version v: for every active row i and head h, over keys j <= i:     */
/*   o_i = sum_j p_ij v^_j, lse_i = log sum_j exp(s_ij), s_ij = q_i.k^_j/sqrt(d),*/
/*   p_ij = exp(s_ij - lse_i); colmass[h][j] = sum over active i >= j of p_ij  */
/*   (every entry of colmass is overwritten).                                */
/* LAZY, version v (reads v-1 and v): S_i = selected keys <= i;               */
/*   p'_ij = exp(q_prev_i.k^(v-1)_j/sqrt(d) - lse_i), m_i = sum p'_ij,         */
/*   a_i = sum p'_ij v^(v-1)_j; otilde_i = softmax over S_i of the current    */
/*   logits applied to v^(v)_j; o_i <- m_i*otilde_i + (o_i - a_i);            */
/*   lse_i <- M + log Z - log m_i; colmass[h][j] += sum_i (p_ij - p'_ij) for   */
/*   selected j, with p_ij = exp(s_ij - lse_i(new)).  Rows with empty S_i or */
/*   m_i == 0 keep o and lse and add nothing to colmass.                     */
/* formula FL_FORMULA_MIXTURE (LAZY only) replaces the output update by the  */
/* other reading of the group keeping its mass, o_i <- m_i*otilde_i +        */
/* (1 - m_i)*o_i (a_i is not needed); lse and colmass are updated as above.  */
/* o, lse and colmass are updated in place; rows that are not active are not */
/* read or written.  Any key tensor entry not described above is untouched.  */
/* Fused commit (fuse_commit != 0; paragraph 4: the KV update and           */
/* compression are fused with the compute): the call also does what          */
/* flashloop_kv_commit(version, active_idx, k_new, v_new, commit_slot_base,  */
/* commit_reset) would do, inside its first kernel; keys that are active in  */
/* this loop derive version `version` from k_new/v_new with the commit's own */
/* float32 arithmetic (version 1: the rows as given) instead of reading the  */
/* records being written, so the store and every output equal                */
/* commit-then-attend bit for bit.  FULL mode with a NULL active_idx commits */
/* every token; where a FULL call takes the per-row path (float32 stores,   */
/* fewer than 64 rows) the commit runs as its own kernel first.              */
/* ------------------------------------------------------------------------ */
typedef struct {
  int32_t mode;                 /* fl_attend_mode */
  const fl_kv_desc* kv;
  int32_t version;              /* FULL: 1..T; LAZY: 2..T */
  const void* q_cur;            /* [n_seq][R][H][d] base_dtype */
  const void* q_prev;           /* LAZY only; same layout */
  int32_t q_layout;             /* fl_row_layout: R = N, or R = n_active */
  const int32_t* active_idx;    /* [n_seq][n_active] ascending; FULL may pass NULL = all rows */
  int32_t n_active;
  const int32_t* key_idx;       /* LAZY: [n_seq][H][n_keys] ascending */
  int32_t n_keys;               /* LAZY: 1..N */
  float* o;                     /* [n_seq][R][H][d] float32, R per o_layout */
  float* lse;                   /* [n_seq][R][H] float32 */
  int32_t o_layout;             /* fl_row_layout */
  float* colmass;               /* [n_seq][H][N] float32 */
  void* workspace;              /* device, >= flashloop_attend_workspace_bytes(args) */
  uint64_t workspace_bytes;
  /* fused commit */
  int32_t fuse_commit;
  const void* k_new;            /* [n_seq][R][H][d] base_dtype, R per kv_layout */
  const void* v_new;
  int32_t kv_layout;            /* fl_row_layout of k_new / v_new */
  int32_t commit_slot_base;     /* slot_base + n_active <= layer_cap[version] */
  int32_t commit_reset;         /* reset_map of the commit */
  int32_t formula;              /* fl_formula (LAZY); FULL requires FL_FORMULA_COLUMN */
  const int32_t* exit_flags;    /* optional [n_seq] device: sequences with a nonzero flag are
                                   skipped (o, lse, colmass and store left as they are) */
  int32_t* dev_status;          /* optional [1] device, caller-zeroed: the kernels OR in FL_DEV_* bits
                                   when a run-time check fails (the call's outputs are then unreliable) */
} fl_attend_args;

/* Bits of fl_attend_args.dev_status.  FL_DEV_XCD_SPLIT: a full loop whose
 * forward pass or column mass is split into parts over several workgroups
 * relies on every part of a head running on one XCD, whose L2 is where the
 * parts' partial results meet (they are not written back past it); a part
 * that ran on another XCD sets this bit. */
#define FL_DEV_XCD_SPLIT 1

uint64_t  flashloop_attend_workspace_bytes(const fl_attend_args* args);
fl_status flashloop_attend(const fl_attend_args* args, void* stream);

/* ------------------------------------------------------------------------ */
/* flashloop_decode_loops -- lazy decode loops first..last in one launch.    */
/* (section "FlashLoop combines three kinds of savings", paragraphs 2-4:     */
/* keys chosen from the previous loop's statistics, a base plus low-bit      */
/* corrections, the update and compression fused with the compute)          */
/* One new token per sequence (active_idx[s]).  The call does what, for      */
/* l = first..last in order, flashloop_select(KEYS, colmass -> the top       */
/* n_keys per (sequence, head)) followed by flashloop_attend(LAZY, version  */
/* l, q_cur = q[l], q_prev = q[l-1], fused commit of k_new[l], v_new[l] at   */
/* slot commit_slot_base[l], commit_reset 0) would do, with the same key     */
/* sets and the same output bits, in one kernel: each (sequence, head)       */
/* keeps its column-mass row, key list and the token's K/V versions on chip  */
/* from loop to loop.  Per-loop queries and new rows are inputs (the shared  */
/* block that produces them is outside this library).                        */
/* In: o, lse, colmass after loop first-1 (and the store through it); out:   */
/* after loop last.  key_idx_out (optional) receives each loop's keys.       */
/* Limits (FL_ERR_UNSUPPORTED): bf16 store, head_dim 128, 4- or 2-bit codes, */
/* last <= 5, n_keys <= 1536, n_tokens <= 8192.  exit_flags are read once,   */
/* at entry (a flagged sequence is skipped for every loop).  No workspace.   */
/* ------------------------------------------------------------------------ */
typedef struct {
  const fl_kv_desc* kv;
  int32_t first_version;        /* >= 2 */
  int32_t last_version;         /* first_version..n_versions, <= 5 */
  const void* q[FL_MAX_VERSIONS + 1];       /* q[l] for l = first-1..last: device [n_seq][R][H][d] bf16 */
  int32_t q_layout;             /* fl_row_layout: R = N (row = token) or R = 1 */
  const int32_t* active_idx;    /* [n_seq] device: the new token's position */
  int32_t n_keys;               /* 1..N keys per (sequence, head) and loop */
  float* o;                     /* [n_seq][R][H][d] */
  float* lse;                   /* [n_seq][R][H] */
  int32_t o_layout;             /* fl_row_layout */
  float* colmass;               /* [n_seq][H][N] */
  const void* k_new[FL_MAX_VERSIONS + 1];   /* k_new[l], v_new[l] for l = first..last: [n_seq][R][H][d] bf16 */
  const void* v_new[FL_MAX_VERSIONS + 1];
  int32_t kv_layout;            /* fl_row_layout of k_new / v_new */
  int32_t commit_slot_base[FL_MAX_VERSIONS + 1];  /* [l]: the token's record slot in layer l (< layer_cap[l]) */
  int32_t* key_idx_out;         /* optional [last-first+1][n_seq][H][n_keys] device */
  int32_t formula;              /* fl_formula */
  const int32_t* exit_flags;    /* optional [n_seq] device */
} fl_decode_loops_args;

fl_status flashloop_decode_loops(const fl_decode_loops_args* args, void* stream);

/* ------------------------------------------------------------------------ */
/* flashloop_attend_noalloc -- flashloop_attend for callers that cannot     */
/* allocate device memory (code under HIP graph capture, serving loops or    */
/* harnesses that forbid hipMalloc).  Same arguments, same kernels, same     */
/* results bit for bit; args->workspace and workspace_bytes are ignored and  */
/* the call's scratch comes from an array the library holds on each GPU      */
/* (FLASHLOOP_STATIC_SCRATCH_BYTES, resident from the library's load on that */
/* GPU until the process ends).  The call allocates nothing.  A call whose   */
/* scratch need (flashloop_attend_workspace_bytes) exceeds that size returns */
/* FL_ERR_WORKSPACE before any launch.  The stream must belong to the        */
/* current device (FL_ERR_ARG otherwise).  Every call on one GPU shares the  */
/* array: calls that overlap on one GPU (several streams or threads) race;   */
/* calls ordered on one stream do not.                                       */
/* ------------------------------------------------------------------------ */
#define FLASHLOOP_STATIC_SCRATCH_BYTES (128ull << 20)
fl_status flashloop_attend_noalloc(const fl_attend_args* args, void* stream);

/* ------------------------------------------------------------------------ */
/* flashloop_exit_check -- early exit per sequence.                           */
/* (page "深度解析循环Transformer架构：隐式推理如何重塑大模型算力效率", on    */
/* looped Transformers, section 四 "开发者实践", item 1 "计算图的动态控制":   */
/* looping stops once the state's change between two loops falls below a     */
/* threshold)  Before a lazy loop, a sequence's change is its largest token   */
/* change: max over its n_rows rows of sum_k (h_cur[r,k] - h_prev[r,k])^2 in  */
/* float64 (the token score of flashloop_select), or the max of precomputed   */
/* scores.  When that maximum is < threshold, exit_flags[s] is set to 1; a    */
/* set flag is never cleared, so later loops passing exit_flags to            */
/* flashloop_attend / flashloop_kv_commit leave the sequence's outputs and    */
/* store as they are, with no host round trip.  max_change[s] (optional)      */
/* receives the maximum.  NaN changes are ignored.  One small launch, no      */
/* workspace; flags and outputs are device memory owned by the caller.        */
/* ------------------------------------------------------------------------ */
typedef struct {
  const double* scores;         /* [n_seq][n_rows] changes (e.g. flashloop_select's scores), or NULL */
  const void* h_cur;            /* used when scores == NULL: [n_seq][n_rows][hidden] h_dtype */
  const void* h_prev;
  int32_t h_dtype;
  int32_t n_seq;                /* 1..65535 */
  int32_t n_rows;               /* rows per sequence, 1..2^24 */
  int32_t hidden;               /* multiple of 8 (hidden-state mode) */
  double threshold;             /* exit when the largest change is < threshold */
  int32_t* exit_flags;          /* [n_seq] in/out, required */
  double* max_change;           /* [n_seq] out, optional */
} fl_exit_args;

fl_status flashloop_exit_check(const fl_exit_args* args, void* stream);

/* ------------------------------------------------------------------------ */
/* Kernel timing (diagnostics, not part of the method).  While enabled, each  */
/* kernel the library launches is bracketed by two hipEvents recorded on the */
/* launch stream.  flashloop_timing_read waits for those events, adds each   */
/* kernel's elapsed time to a per-kernel-name total and returns the totals:  */
/* names_out receives max_entries NUL-padded names of 64 bytes each,         */
/* ms_out the summed milliseconds and launches_out the launch counts.  It    */
/* returns the number of kernel names (which may exceed max_entries).        */
/* flashloop_timing_enable(0) stops recording; (1) starts it and clears the  */
/* totals.  This is the one piece of process-wide state in the library; it   */
/* is guarded by a mutex.                                                    */
/* ------------------------------------------------------------------------ */
fl_status flashloop_timing_enable(int32_t on);
int32_t   flashloop_timing_read(char* names_out, double* ms_out, int64_t* launches_out, int32_t max_entries);

/* ------------------------------------------------------------------------ */
const char* flashloop_last_error(void);  /* thread-local; "" after a successful call */
int32_t     flashloop_abi_version(void); /* FLASHLOOP_ABI_VERSION */

#ifdef __cplusplus
}
#endif
#endif /* FLASHLOOP_H */
