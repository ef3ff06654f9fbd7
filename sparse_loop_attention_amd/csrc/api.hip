// C ABI of the FlashLoop loop step: argument validation, arena layout,
// workspace planning and dispatch.  Host code only; every step of the path
// runs in the kernels of select.hip, kv.hip, attn_rows.hip and attn_mfma.hip.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "flashloop.h"
#include "fl_launch.hpp"
#include "fl_rows.hpp"

namespace {

thread_local char g_err[512] = "";

fl_status fail(fl_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}
fl_status ok() {
  g_err[0] = '\0';
  return FL_OK;
}
fl_status hip_fail(hipError_t e, const char* what) {
  return fail(FL_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

fl_status check_desc(const fl_kv_desc* d, bool need_arena) {
  if (!d) return fail(FL_ERR_ARG, "kv descriptor is NULL");
  if (d->n_seq < 1 || d->n_heads < 1 || d->n_tokens < 1)
    return fail(FL_ERR_ARG, "kv: n_seq, n_heads and n_tokens must be >= 1");
  if (d->n_tokens > (1 << 24)) return fail(FL_ERR_UNSUPPORTED, "kv: n_tokens > 2^24");
  if (d->head_dim != 64 && d->head_dim != 96 && d->head_dim != 128)
    return fail(FL_ERR_UNSUPPORTED, "kv: head_dim %d not in {64, 96, 128}", d->head_dim);
  if (d->n_versions < 1 || d->n_versions > FL_MAX_VERSIONS)
    return fail(FL_ERR_ARG, "kv: n_versions %d outside 1..%d", d->n_versions, FL_MAX_VERSIONS);
  if (d->base_dtype != FL_F32 && d->base_dtype != FL_BF16) return fail(FL_ERR_ARG, "kv: unknown base_dtype");
  if (d->group != 32 && d->group != 64) return fail(FL_ERR_UNSUPPORTED, "kv: group %d not in {32, 64}", d->group);
  if (d->head_dim % d->group)
    return fail(FL_ERR_UNSUPPORTED, "kv: group %d does not divide head_dim %d", d->group, d->head_dim);
  if (d->delta_bits != 0 && d->delta_bits != 2 && d->delta_bits != 4)
    return fail(FL_ERR_UNSUPPORTED, "kv: delta_bits %d not in {2, 4}", d->delta_bits);
  for (int l = 2; l <= d->n_versions; ++l)
    if (d->layer_cap[l] < 0 || d->layer_cap[l] > d->n_tokens)
      return fail(FL_ERR_ARG, "kv: layer_cap[%d] = %d outside 0..n_tokens", l, d->layer_cap[l]);
  if (need_arena && (!d->arena || !aligned(d->arena, 256)))
    return fail(FL_ERR_ARG, "kv: arena is NULL or not 256-byte aligned");
  return FL_OK;
}

void layout_of(const fl_kv_desc* d, fl_kv_layout* o) {
  std::memset(o, 0, sizeof(*o));
  const uint64_t S = d->n_seq, H = d->n_heads, N = d->n_tokens, D = d->head_dim;
  const uint64_t es = d->base_dtype == FL_BF16 ? 2 : 4;
  uint64_t off = 0;
  o->base_k = off; off = align256(off + S * H * N * D * es);
  o->base_v = off; off = align256(off + S * H * N * D * es);
  o->slot_pitch = d->n_versions > 1 ? (static_cast<uint64_t>(d->n_versions - 1) + 3) / 4 * 4 : 0;
  o->slot_table = off; off = align256(off + S * N * o->slot_pitch * 4);
  const uint64_t bits = d->delta_bits ? d->delta_bits : 4;
  for (int l = 2; l <= d->n_versions; ++l) {
    const uint64_t cap = d->layer_cap[l];
    o->codes[l] = off; off = align256(off + S * cap * H * 2 * (D * bits / 8));
    o->scales[l] = off; off = align256(off + S * cap * H * 2 * (D / d->group) * 2);
  }
  o->total_bytes = off;
}

fl_status check_arena(const fl_kv_desc* d, fl_kv_layout* lay) {
  fl_status st = check_desc(d, true);
  if (st != FL_OK) return st;
  layout_of(d, lay);
  if (d->arena_bytes < lay->total_bytes)
    return fail(FL_ERR_ARG, "kv: arena_bytes %llu < required %llu", (unsigned long long)d->arena_bytes,
                (unsigned long long)lay->total_bytes);
  return FL_OK;
}

}  // namespace

namespace fl {

KvView make_view(const fl_kv_desc& d, const fl_kv_layout& lay) {
  KvView v;
  std::memset(&v, 0, sizeof(v));
  v.arena = static_cast<const uint8_t*>(d.arena);
  v.n_seq = d.n_seq; v.H = d.n_heads; v.d = d.head_dim; v.N = d.n_tokens; v.T = d.n_versions;
  v.dtype = d.base_dtype;
  v.base[0] = lay.base_k; v.base[1] = lay.base_v;
  v.slot_table = lay.slot_table;
  v.slot_pitch = static_cast<int32_t>(lay.slot_pitch);
  v.bits = d.delta_bits ? d.delta_bits : 4;
  v.gshift = d.group == 64 ? 3 : 2;
  for (int l = 2; l <= d.n_versions; ++l) {
    v.cap[l] = d.layer_cap[l];
    v.codes[l] = lay.codes[l];
    v.scales[l] = lay.scales[l];
  }
  return v;
}

}  // namespace fl

extern "C" {

int32_t flashloop_abi_version(void) { return FLASHLOOP_ABI_VERSION; }
const char* flashloop_last_error(void) { return g_err; }

fl_status flashloop_kv_layout(const fl_kv_desc* desc, fl_kv_layout* out) {
  if (!out) return fail(FL_ERR_ARG, "layout output is NULL");
  fl_status st = check_desc(desc, false);
  if (st != FL_OK) return st;
  layout_of(desc, out);
  return ok();
}

uint64_t flashloop_kv_arena_bytes(const fl_kv_desc* desc) {
  if (check_desc(desc, false) != FL_OK) return 0;
  fl_kv_layout lay;
  layout_of(desc, &lay);
  ok();
  return lay.total_bytes;
}

fl_status flashloop_kv_commit(const fl_commit_args* a, void* stream) {
  if (!a) return fail(FL_ERR_ARG, "commit args are NULL");
  fl_kv_layout lay;
  fl_status st = check_arena(a->kv, &lay);
  if (st != FL_OK) return st;
  const fl_kv_desc& d = *a->kv;
  if (a->version < 1 || a->version > d.n_versions)
    return fail(FL_ERR_ARG, "commit: version %d outside 1..%d", a->version, d.n_versions);
  if (a->n_active < 0 || a->n_active > d.n_tokens) return fail(FL_ERR_ARG, "commit: n_active out of range");
  if (a->n_active == 0) {
    // no active token: no record; a reset still clears the layer's slots
    if (a->version == 1 || !a->reset_map) return ok();
    fl::KvView kv = fl::make_view(d, lay);
    hipError_t e = fl::launch_commit(*a, kv, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "commit launch");
    return ok();
  }
  if (!a->active_idx || !a->k_new || !a->v_new) return fail(FL_ERR_ARG, "commit: NULL index or K/V pointer");
  if (!aligned(a->k_new, 16) || !aligned(a->v_new, 16) || !aligned(a->active_idx, 4))
    return fail(FL_ERR_ARG, "commit: K/V must be 16-byte aligned");
  if (a->src_layout != FL_ROWS_BY_TOKEN && a->src_layout != FL_ROWS_COMPACT)
    return fail(FL_ERR_ARG, "commit: unknown src_layout");
  if (a->version >= 2) {
    if (a->slot_base < 0 || static_cast<int64_t>(a->slot_base) + a->n_active > d.layer_cap[a->version])
      return fail(FL_ERR_ARG, "commit: slots %d..%d exceed layer_cap[%d] = %d", a->slot_base,
                  a->slot_base + a->n_active, a->version, d.layer_cap[a->version]);
  }
  if (a->exit_flags && !aligned(a->exit_flags, 4)) return fail(FL_ERR_ARG, "commit: exit_flags must be 4-byte aligned");
  fl::KvView kv = fl::make_view(d, lay);
  kv.exit_flags = a->exit_flags;
  hipError_t e = fl::launch_commit(*a, kv, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "commit launch");
  return ok();
}

fl_status flashloop_select(const fl_select_args* a, void* stream) {
  if (!a) return fail(FL_ERR_ARG, "select args are NULL");
  if (a->mode == FL_SEL_TOKENS) {
    if (!a->h_cur || !a->h_prev || !a->scores) return fail(FL_ERR_ARG, "select: NULL h or scores");
    if (a->h_dtype != FL_F32 && a->h_dtype != FL_BF16) return fail(FL_ERR_ARG, "select: unknown h_dtype");
    if (a->n_rows < 1 || a->n_rows > 65536) return fail(FL_ERR_UNSUPPORTED, "select: n_rows outside 1..65536");
    if (a->hidden < 8 || a->hidden % 8) return fail(FL_ERR_UNSUPPORTED, "select: hidden must be a multiple of 8");
    if (!aligned(a->h_cur, 16) || !aligned(a->h_prev, 16) || !aligned(a->scores, 8))
      return fail(FL_ERR_ARG, "select: h must be 16-byte aligned");
    if (a->k < 0 || a->k > a->n_rows) return fail(FL_ERR_ARG, "select: k outside 0..n_rows");
    if (a->cand_idx && (a->n_cand < 0 || a->n_cand > a->n_rows))
      return fail(FL_ERR_ARG, "select: n_cand outside 0..n_rows");
  } else if (a->mode == FL_SEL_KEYS) {
    if (!a->key_scores) return fail(FL_ERR_ARG, "select: NULL key_scores");
    if (a->n_seg < 1) return fail(FL_ERR_ARG, "select: n_seg must be >= 1");
    if (a->seg_len < 1 || a->seg_len > 65536) return fail(FL_ERR_UNSUPPORTED, "select: seg_len outside 1..65536");
    if (a->k < 0 || a->k > a->seg_len) return fail(FL_ERR_ARG, "select: k outside 0..seg_len");
  } else {
    return fail(FL_ERR_ARG, "select: unknown mode %d", a->mode);
  }
  if (a->k > 0 && !a->out_idx) return fail(FL_ERR_ARG, "select: NULL out_idx");
  hipError_t e = fl::launch_select(*a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "select launch");
  return ok();
}

static fl_status check_attend(const fl_attend_args* a, fl_kv_layout* lay) {
  if (!a) return fail(FL_ERR_ARG, "attend args are NULL");
  fl_status st = check_arena(a->kv, lay);
  if (st != FL_OK) return st;
  const fl_kv_desc& d = *a->kv;
  const bool lazy = a->mode == FL_ATTEND_LAZY;
  if (a->mode != FL_ATTEND_FULL && !lazy) return fail(FL_ERR_ARG, "attend: unknown mode %d", a->mode);
  if (a->version < (lazy ? 2 : 1) || a->version > d.n_versions)
    return fail(FL_ERR_ARG, "attend: version %d invalid for this mode", a->version);
  if (a->n_active < (lazy ? 0 : 1) || a->n_active > d.n_tokens)
    return fail(FL_ERR_ARG, "attend: n_active %d out of range", a->n_active);
  if (!lazy && !a->active_idx && a->n_active != d.n_tokens)
    return fail(FL_ERR_ARG, "attend: NULL active_idx requires n_active == n_tokens");
  if (lazy && a->n_active > 0 && !a->active_idx) return fail(FL_ERR_ARG, "attend: LAZY needs active_idx");
  if (!a->q_cur || (lazy && !a->q_prev)) return fail(FL_ERR_ARG, "attend: NULL query");
  if (!aligned(a->q_cur, 16) || (lazy && !aligned(a->q_prev, 16)))
    return fail(FL_ERR_ARG, "attend: queries must be 16-byte aligned");
  if (lazy && (!a->key_idx || a->n_keys < 1 || a->n_keys > d.n_tokens))
    return fail(FL_ERR_ARG, "attend: LAZY needs key_idx with 1 <= n_keys <= n_tokens");
  if (!a->o || !a->lse || !a->colmass) return fail(FL_ERR_ARG, "attend: NULL o, lse or colmass");
  if (!aligned(a->o, 16)) return fail(FL_ERR_ARG, "attend: o must be 16-byte aligned");
  if (a->q_layout != FL_ROWS_BY_TOKEN && a->q_layout != FL_ROWS_COMPACT) return fail(FL_ERR_ARG, "attend: q_layout");
  if (a->o_layout != FL_ROWS_BY_TOKEN && a->o_layout != FL_ROWS_COMPACT) return fail(FL_ERR_ARG, "attend: o_layout");
  if (a->formula != FL_FORMULA_COLUMN && !(lazy && a->formula == FL_FORMULA_MIXTURE))
    return fail(FL_ERR_ARG, "attend: formula %d (FULL needs FL_FORMULA_COLUMN)", a->formula);
  if (a->exit_flags && !aligned(a->exit_flags, 4)) return fail(FL_ERR_ARG, "attend: exit_flags must be 4-byte aligned");
  if (a->fuse_commit) {
    if (!a->k_new || !a->v_new || !aligned(a->k_new, 16) || !aligned(a->v_new, 16))
      return fail(FL_ERR_ARG, "attend: fused commit needs 16-byte aligned k_new and v_new");
    if (a->kv_layout != FL_ROWS_BY_TOKEN && a->kv_layout != FL_ROWS_COMPACT) return fail(FL_ERR_ARG, "attend: kv_layout");
    if (a->version >= 2 && (a->commit_slot_base < 0 ||
                            static_cast<int64_t>(a->commit_slot_base) + a->n_active > d.layer_cap[a->version]))
      return fail(FL_ERR_ARG, "attend: commit slots %d..%d exceed layer_cap[%d] = %d", a->commit_slot_base,
                  a->commit_slot_base + a->n_active, a->version, d.layer_cap[a->version]);
  }
  return FL_OK;
}

uint64_t flashloop_attend_workspace_bytes(const fl_attend_args* a) {
  fl_kv_layout lay;
  if (!a || !a->kv || check_desc(a->kv, false) != FL_OK) return 0;
  (void)lay;
  return fl::plan_attend(*a).off_total;
}

static fl_status attend_impl(const fl_attend_args* a, void* stream, bool static_scratch) {
  fl_kv_layout lay;
  fl_status st = check_attend(a, &lay);
  if (st != FL_OK) return st;
  if (a->n_active == 0) {                          // LAZY with no active rows: nothing changes
    if (a->fuse_commit && a->commit_reset) {        // ... except that the layer's slots are cleared
      fl_commit_args c{};
      c.kv = a->kv; c.version = a->version; c.n_active = 0; c.reset_map = 1;
      c.exit_flags = a->exit_flags;
      fl::KvView kv = fl::make_view(*a->kv, lay);
      kv.exit_flags = a->exit_flags;
      hipError_t e = fl::launch_commit(c, kv, static_cast<hipStream_t>(stream));
      if (e != hipSuccess) return hip_fail(e, "attend launch");
    }
    return ok();
  }
  const fl::AttendPlan p = fl::plan_attend(*a);
  fl_attend_args x = *a;
  if (static_scratch) {
    if (p.off_total > FLASHLOOP_STATIC_SCRATCH_BYTES)
      return fail(FL_ERR_WORKSPACE, "attend_noalloc: the call needs %llu bytes of scratch, more than the %llu the "
                  "library holds per GPU (use flashloop_attend with a workspace)",
                  (unsigned long long)p.off_total, (unsigned long long)FLASHLOOP_STATIC_SCRATCH_BYTES);
    void* ptr = nullptr;
    hipError_t e = fl::static_scratch(static_cast<hipStream_t>(stream), &ptr);
    if (e == hipErrorInvalidValue) return fail(FL_ERR_ARG, "attend_noalloc: the stream belongs to another device");
    if (e != hipSuccess) return hip_fail(e, "attend_noalloc: scratch address");
    x.workspace = ptr;
    x.workspace_bytes = FLASHLOOP_STATIC_SCRATCH_BYTES;
  } else if (p.off_total > 0 && (!a->workspace || a->workspace_bytes < p.off_total || !aligned(a->workspace, 256))) {
    return fail(FL_ERR_WORKSPACE, "attend: workspace needs %llu bytes (256-byte aligned), got %llu",
                (unsigned long long)p.off_total, (unsigned long long)a->workspace_bytes);
  }
  fl::KvView kv = fl::make_view(*a->kv, lay);
  kv.exit_flags = a->exit_flags;
  if (x.fuse_commit && x.mode == FL_ATTEND_FULL && !p.mfma) {
    // the per-row path fuses only LAZY commits: commit first, on the same stream
    fl_commit_args c{};
    c.kv = x.kv; c.version = x.version;
    c.active_idx = x.active_idx;                  // null: every token (the commit kernels take it so)
    c.n_active = x.n_active;
    c.slot_base = x.commit_slot_base; c.reset_map = x.commit_reset;
    c.k_new = x.k_new; c.v_new = x.v_new;
    c.src_layout = x.kv_layout;
    c.exit_flags = x.exit_flags;
    hipError_t e = fl::launch_commit(c, kv, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "attend launch");
  }
  hipError_t e = fl::launch_attend(x, kv, p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "attend launch");
  return ok();
}

fl_status flashloop_attend(const fl_attend_args* a, void* stream) { return attend_impl(a, stream, false); }

fl_status flashloop_attend_noalloc(const fl_attend_args* a, void* stream) { return attend_impl(a, stream, true); }

fl_status flashloop_decode_loops(const fl_decode_loops_args* a, void* stream) {
  if (!a) return fail(FL_ERR_ARG, "decode_loops args are NULL");
  fl_kv_layout lay;
  fl_status st = check_arena(a->kv, &lay);
  if (st != FL_OK) return st;
  const fl_kv_desc& d = *a->kv;
  if (a->first_version < 2 || a->last_version < a->first_version || a->last_version > d.n_versions)
    return fail(FL_ERR_ARG, "decode_loops: versions %d..%d invalid (2 <= first <= last <= %d)", a->first_version,
                a->last_version, d.n_versions);
  if (a->n_keys < 1 || a->n_keys > d.n_tokens) return fail(FL_ERR_ARG, "decode_loops: n_keys outside 1..n_tokens");
  if (!a->active_idx || !aligned(a->active_idx, 4)) return fail(FL_ERR_ARG, "decode_loops: NULL active_idx");
  if (!a->o || !a->lse || !a->colmass || !aligned(a->o, 16))
    return fail(FL_ERR_ARG, "decode_loops: NULL or misaligned o, lse or colmass");
  if (a->q_layout != FL_ROWS_BY_TOKEN && a->q_layout != FL_ROWS_COMPACT) return fail(FL_ERR_ARG, "decode_loops: q_layout");
  if (a->o_layout != FL_ROWS_BY_TOKEN && a->o_layout != FL_ROWS_COMPACT) return fail(FL_ERR_ARG, "decode_loops: o_layout");
  if (a->kv_layout != FL_ROWS_BY_TOKEN && a->kv_layout != FL_ROWS_COMPACT) return fail(FL_ERR_ARG, "decode_loops: kv_layout");
  if (a->formula != FL_FORMULA_COLUMN && a->formula != FL_FORMULA_MIXTURE) return fail(FL_ERR_ARG, "decode_loops: formula");
  if (a->exit_flags && !aligned(a->exit_flags, 4)) return fail(FL_ERR_ARG, "decode_loops: exit_flags must be 4-byte aligned");
  if (a->key_idx_out && !aligned(a->key_idx_out, 4)) return fail(FL_ERR_ARG, "decode_loops: key_idx_out misaligned");
  for (int l = a->first_version - 1; l <= a->last_version; ++l)
    if (!a->q[l] || !aligned(a->q[l], 16)) return fail(FL_ERR_ARG, "decode_loops: q[%d] NULL or misaligned", l);
  for (int l = a->first_version; l <= a->last_version; ++l) {
    if (!a->k_new[l] || !a->v_new[l] || !aligned(a->k_new[l], 16) || !aligned(a->v_new[l], 16))
      return fail(FL_ERR_ARG, "decode_loops: k_new[%d] / v_new[%d] NULL or misaligned", l, l);
    if (a->commit_slot_base[l] < 0 || a->commit_slot_base[l] >= d.layer_cap[l])
      return fail(FL_ERR_ARG, "decode_loops: commit_slot_base[%d] = %d outside layer_cap[%d] = %d", l,
                  a->commit_slot_base[l], l, d.layer_cap[l]);
  }
  fl::KvView kv = fl::make_view(d, lay);
  kv.exit_flags = a->exit_flags;
  fl::DecLoopsArgs x{};
  x.arena = static_cast<uint8_t*>(d.arena);
  x.act = a->active_idx;
  x.first = a->first_version;
  x.last = a->last_version;
  for (int l = 0; l <= FL_MAX_VERSIONS; ++l) {
    x.q[l] = a->q[l];
    x.k_new[l] = a->k_new[l];
    x.v_new[l] = a->v_new[l];
    x.slot_base[l] = a->commit_slot_base[l];
  }
  x.q_compact = a->q_layout == FL_ROWS_COMPACT;
  x.o_compact = a->o_layout == FL_ROWS_COMPACT;
  x.kv_compact = a->kv_layout == FL_ROWS_COMPACT;
  x.n_keys = a->n_keys;
  x.o = a->o; x.lse = a->lse; x.colmass = a->colmass;
  x.keys_out = a->key_idx_out;
  x.scale = 1.0f / sqrtf(static_cast<float>(d.head_dim));
  x.mixture = a->formula == FL_FORMULA_MIXTURE;
  hipError_t e = hipSuccess;
  if (!fl::launch_decode_loops(x, kv, static_cast<hipStream_t>(stream), &e))
    return fail(FL_ERR_UNSUPPORTED, "decode_loops: needs a bf16 store, head_dim 128, 4- or 2-bit codes, versions "
                "up to 5, n_keys <= 1536 and n_tokens <= 8192");
  if (e != hipSuccess) return hip_fail(e, "decode_loops launch");
  return ok();
}

fl_status flashloop_exit_check(const fl_exit_args* a, void* stream) {
  if (!a) return fail(FL_ERR_ARG, "exit args are NULL");
  if (!a->exit_flags || !aligned(a->exit_flags, 4)) return fail(FL_ERR_ARG, "exit: exit_flags NULL or misaligned");
  if (a->n_seq < 1 || a->n_seq > 65535) return fail(FL_ERR_ARG, "exit: n_seq outside 1..65535");
  if (a->n_rows < 1 || a->n_rows > (1 << 24)) return fail(FL_ERR_ARG, "exit: n_rows outside 1..2^24");
  if (a->max_change && !aligned(a->max_change, 8)) return fail(FL_ERR_ARG, "exit: max_change must be 8-byte aligned");
  if (a->scores) {
    if (!aligned(a->scores, 8)) return fail(FL_ERR_ARG, "exit: scores must be 8-byte aligned");
  } else {
    if (!a->h_cur || !a->h_prev) return fail(FL_ERR_ARG, "exit: NULL scores and NULL h");
    if (a->h_dtype != FL_F32 && a->h_dtype != FL_BF16) return fail(FL_ERR_ARG, "exit: unknown h_dtype");
    if (a->hidden < 8 || a->hidden % 8) return fail(FL_ERR_UNSUPPORTED, "exit: hidden must be a multiple of 8");
    if (!aligned(a->h_cur, 16) || !aligned(a->h_prev, 16)) return fail(FL_ERR_ARG, "exit: h must be 16-byte aligned");
  }
  hipError_t e = fl::launch_exit_check(*a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "exit launch");
  return ok();
}

}  // extern "C"
