"""ctypes binding of libflashloop.so (include/flashloop.h): argument marshalling only.

Every function takes torch tensors for device memory and launches on torch's
current stream; all arithmetic happens in the HIP library.  There is no CPU
fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

import torch  # noqa: F401  (loads the HIP runtime that the library binds to)

# FLASHLOOP_LIBRARY selects another build of the same library (e.g. a kernel variant)
LIB_PATH = os.environ.get("FLASHLOOP_LIBRARY",
                          os.path.join(os.path.dirname(os.path.abspath(__file__)), "libflashloop.so"))
MAX_VERSIONS = 32

FL_OK, FL_ERR_ARG, FL_ERR_UNSUPPORTED, FL_ERR_WORKSPACE, FL_ERR_HIP = range(5)
FL_F32, FL_BF16 = 0, 1
FL_FORMULA_COLUMN, FL_FORMULA_MIXTURE = 0, 1
FORMULAS = {"column": FL_FORMULA_COLUMN, "mixture": FL_FORMULA_MIXTURE}
FL_SEL_TOKENS, FL_SEL_KEYS = 0, 1
FL_ATTEND_FULL, FL_ATTEND_LAZY = 0, 1
FL_ROWS_BY_TOKEN, FL_ROWS_COMPACT = 0, 1
FL_DEV_XCD_SPLIT = 1

EXPORTS = ("flashloop_kv_layout", "flashloop_kv_arena_bytes", "flashloop_kv_commit", "flashloop_select",
           "flashloop_attend_workspace_bytes", "flashloop_attend", "flashloop_last_error",
           "flashloop_abi_version", "flashloop_timing_enable", "flashloop_timing_read", "flashloop_exit_check",
           "flashloop_attend_noalloc", "flashloop_decode_loops")
STATIC_SCRATCH_BYTES = 128 << 20        # FLASHLOOP_STATIC_SCRATCH_BYTES


class fl_kv_desc(C.Structure):
    _fields_ = [("n_seq", C.c_int32), ("n_heads", C.c_int32), ("head_dim", C.c_int32),
                ("n_tokens", C.c_int32), ("n_versions", C.c_int32), ("base_dtype", C.c_int32),
                ("group", C.c_int32), ("delta_bits", C.c_int32), ("layer_cap", C.c_int32 * (MAX_VERSIONS + 1)),
                ("arena", C.c_void_p), ("arena_bytes", C.c_uint64)]


class fl_kv_layout(C.Structure):
    _fields_ = [("base_k", C.c_uint64), ("base_v", C.c_uint64),
                ("slot_table", C.c_uint64), ("slot_pitch", C.c_uint64),
                ("codes", C.c_uint64 * (MAX_VERSIONS + 1)), ("scales", C.c_uint64 * (MAX_VERSIONS + 1)),
                ("total_bytes", C.c_uint64)]


class fl_commit_args(C.Structure):
    _fields_ = [("kv", C.POINTER(fl_kv_desc)), ("version", C.c_int32), ("active_idx", C.c_void_p),
                ("n_active", C.c_int32), ("slot_base", C.c_int32), ("reset_map", C.c_int32),
                ("k_new", C.c_void_p), ("v_new", C.c_void_p), ("src_layout", C.c_int32),
                ("exit_flags", C.c_void_p)]


class fl_select_args(C.Structure):
    _fields_ = [("mode", C.c_int32), ("h_cur", C.c_void_p), ("h_prev", C.c_void_p), ("h_dtype", C.c_int32),
                ("n_rows", C.c_int64), ("hidden", C.c_int64), ("cand_idx", C.c_void_p), ("n_cand", C.c_int32),
                ("scores", C.c_void_p), ("key_scores", C.c_void_p), ("n_seg", C.c_int32),
                ("seg_len", C.c_int64), ("k", C.c_int32), ("out_idx", C.c_void_p)]


class fl_attend_args(C.Structure):
    _fields_ = [("mode", C.c_int32), ("kv", C.POINTER(fl_kv_desc)), ("version", C.c_int32),
                ("q_cur", C.c_void_p), ("q_prev", C.c_void_p), ("q_layout", C.c_int32),
                ("active_idx", C.c_void_p), ("n_active", C.c_int32), ("key_idx", C.c_void_p),
                ("n_keys", C.c_int32), ("o", C.c_void_p), ("lse", C.c_void_p), ("o_layout", C.c_int32),
                ("colmass", C.c_void_p), ("workspace", C.c_void_p), ("workspace_bytes", C.c_uint64),
                ("fuse_commit", C.c_int32), ("k_new", C.c_void_p), ("v_new", C.c_void_p), ("kv_layout", C.c_int32),
                ("commit_slot_base", C.c_int32), ("commit_reset", C.c_int32), ("formula", C.c_int32),
                ("exit_flags", C.c_void_p), ("dev_status", C.c_void_p)]


class fl_exit_args(C.Structure):
    _fields_ = [("scores", C.c_void_p), ("h_cur", C.c_void_p), ("h_prev", C.c_void_p), ("h_dtype", C.c_int32),
                ("n_seq", C.c_int32), ("n_rows", C.c_int32), ("hidden", C.c_int32), ("threshold", C.c_double),
                ("exit_flags", C.c_void_p), ("max_change", C.c_void_p)]


V = MAX_VERSIONS + 1


class fl_decode_loops_args(C.Structure):
    _fields_ = [("kv", C.POINTER(fl_kv_desc)), ("first_version", C.c_int32), ("last_version", C.c_int32),
                ("q", C.c_void_p * V), ("q_layout", C.c_int32), ("active_idx", C.c_void_p), ("n_keys", C.c_int32),
                ("o", C.c_void_p), ("lse", C.c_void_p), ("o_layout", C.c_int32), ("colmass", C.c_void_p),
                ("k_new", C.c_void_p * V), ("v_new", C.c_void_p * V), ("kv_layout", C.c_int32),
                ("commit_slot_base", C.c_int32 * V), ("key_idx_out", C.c_void_p), ("formula", C.c_int32),
                ("exit_flags", C.c_void_p)]


class FlashLoopError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"flashloop status {status}: {msg}")
        self.status = status


_lib = None


def lib():
    """The loaded library; raises if it was not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run `python -m sparse_loop_attention_amd.build`")
        L = C.CDLL(LIB_PATH)
        L.flashloop_kv_layout.argtypes = [C.POINTER(fl_kv_desc), C.POINTER(fl_kv_layout)]
        L.flashloop_kv_arena_bytes.argtypes = [C.POINTER(fl_kv_desc)]
        L.flashloop_kv_arena_bytes.restype = C.c_uint64
        L.flashloop_kv_commit.argtypes = [C.POINTER(fl_commit_args), C.c_void_p]
        L.flashloop_select.argtypes = [C.POINTER(fl_select_args), C.c_void_p]
        L.flashloop_attend_workspace_bytes.argtypes = [C.POINTER(fl_attend_args)]
        L.flashloop_attend_workspace_bytes.restype = C.c_uint64
        L.flashloop_attend.argtypes = [C.POINTER(fl_attend_args), C.c_void_p]
        L.flashloop_attend_noalloc.argtypes = [C.POINTER(fl_attend_args), C.c_void_p]
        L.flashloop_decode_loops.argtypes = [C.POINTER(fl_decode_loops_args), C.c_void_p]
        L.flashloop_last_error.restype = C.c_char_p
        L.flashloop_abi_version.restype = C.c_int32
        L.flashloop_timing_enable.argtypes = [C.c_int32]
        L.flashloop_timing_read.argtypes = [C.c_char_p, C.POINTER(C.c_double), C.POINTER(C.c_int64), C.c_int32]
        L.flashloop_timing_read.restype = C.c_int32
        L.flashloop_exit_check.argtypes = [C.POINTER(fl_exit_args), C.c_void_p]
        for f in ("flashloop_kv_layout", "flashloop_kv_commit", "flashloop_select", "flashloop_attend",
                  "flashloop_exit_check", "flashloop_attend_noalloc", "flashloop_decode_loops"):
            getattr(L, f).restype = C.c_int
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != FL_OK:
        raise FlashLoopError(status, lib().flashloop_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return t.data_ptr()


def _stream(stream=None) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def dtype_code(t: torch.dtype) -> int:
    return {torch.float32: FL_F32, torch.bfloat16: FL_BF16}[t]


# --------------------------------------------------------------------------- KV
class KVStore:
    """A KV arena (torch uint8 tensor) and its descriptor."""

    def __init__(self, n_seq: int, n_heads: int, head_dim: int, n_tokens: int, n_versions: int,
                 dtype: torch.dtype, layer_caps: Sequence[int], device="cuda", arena: Optional[torch.Tensor] = None,
                 group: int = 32, delta_bits: int = 4):
        d = fl_kv_desc()
        d.n_seq, d.n_heads, d.head_dim, d.n_tokens = n_seq, n_heads, head_dim, n_tokens
        d.n_versions, d.base_dtype, d.group, d.delta_bits = n_versions, dtype_code(dtype), group, delta_bits
        for i, cap in enumerate(layer_caps):
            d.layer_cap[i + 2] = cap
        self.desc = d
        self.dtype = dtype
        nbytes = kv_arena_bytes(d)
        if nbytes == 0:
            raise FlashLoopError(FL_ERR_ARG, lib().flashloop_last_error().decode())
        self.arena = torch.empty(nbytes, dtype=torch.uint8, device=device) if arena is None else arena
        d.arena = self.arena.data_ptr()
        d.arena_bytes = self.arena.numel()
        self.layout = kv_layout(d)

    def view(self, name: str, layer: int = 0) -> torch.Tensor:
        """A typed view of one arena array (for tests and checkpoints)."""
        d, lay = self.desc, self.layout
        S, H, N, D = d.n_seq, d.n_heads, d.n_tokens, d.head_dim
        if name in ("base_k", "base_v"):
            off = getattr(lay, name)
            es = 2 if self.dtype == torch.bfloat16 else 4
            n = S * H * N * D
            t = self.arena[off:off + n * es].view(self.dtype)
            return t.view(S, H, N, D)
        cap = d.layer_cap[layer]
        if name == "slot_map":                    # [S, N]: slot of each token in `layer`
            off, sp = lay.slot_table, lay.slot_pitch
            return self.arena[off:off + S * N * sp * 4].view(torch.int32).view(S, N, sp)[:, :, layer - 2]
        b, g = (d.delta_bits or 4), d.group
        if name == "codes":                       # [S, cap, H, 2 (K, V), d*bits/8]
            off = lay.codes[layer]
            n = S * cap * H * 2 * (D * b // 8)
            return self.arena[off:off + n].view(S, cap, H, 2, D * b // 8)
        if name == "scales":                      # [S, cap, H, 2 (K, V), d/group] binary16 bits
            off = lay.scales[layer]
            n = S * cap * H * 2 * (D // g)
            return self.arena[off:off + 2 * n].view(torch.int16).view(S, cap, H, 2, D // g)
        raise KeyError(name)


def kv_layout(desc: fl_kv_desc) -> fl_kv_layout:
    out = fl_kv_layout()
    _check(lib().flashloop_kv_layout(C.byref(desc), C.byref(out)))
    return out


def kv_arena_bytes(desc: fl_kv_desc) -> int:
    return int(lib().flashloop_kv_arena_bytes(C.byref(desc)))


def kv_commit(kv: KVStore, version: int, active_idx: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
              slot_base: int = 0, reset_map: bool = True, compact: bool = False,
              exit_flags: Optional[torch.Tensor] = None, stream=None) -> None:
    a = fl_commit_args()
    a.kv = C.pointer(kv.desc)
    a.version = version
    a.active_idx = _ptr(active_idx)
    a.n_active = active_idx.shape[-1]
    a.slot_base, a.reset_map = slot_base, int(reset_map)
    a.k_new, a.v_new = _ptr(k_new), _ptr(v_new)
    a.src_layout = FL_ROWS_COMPACT if compact else FL_ROWS_BY_TOKEN
    a.exit_flags = _ptr(exit_flags)
    _check(lib().flashloop_kv_commit(C.byref(a), _stream(stream)))


# --------------------------------------------------------------------------- select
def select_tokens(h_cur: torch.Tensor, h_prev: torch.Tensor, k: int, scores: torch.Tensor,
                  out_idx: torch.Tensor, cand_idx: Optional[torch.Tensor] = None, stream=None) -> None:
    a = fl_select_args()
    a.mode = FL_SEL_TOKENS
    a.h_cur, a.h_prev, a.h_dtype = _ptr(h_cur), _ptr(h_prev), dtype_code(h_cur.dtype)
    a.n_rows, a.hidden = h_cur.shape[0], h_cur.shape[1]
    a.cand_idx = _ptr(cand_idx)
    a.n_cand = 0 if cand_idx is None else cand_idx.numel()
    a.scores = _ptr(scores)
    a.k, a.out_idx = k, _ptr(out_idx)
    _check(lib().flashloop_select(C.byref(a), _stream(stream)))


def select_keys(key_scores: torch.Tensor, k: int, out_idx: torch.Tensor, stream=None) -> None:
    a = fl_select_args()
    a.mode = FL_SEL_KEYS
    a.key_scores = _ptr(key_scores)
    a.seg_len = key_scores.shape[-1]
    a.n_seg = key_scores.numel() // key_scores.shape[-1]
    a.k, a.out_idx = k, _ptr(out_idx)
    _check(lib().flashloop_select(C.byref(a), _stream(stream)))


# --------------------------------------------------------------------------- attend
def attend_args(kv: KVStore, mode: int, version: int, q_cur, q_prev, active_idx, n_active: int,
                key_idx, o, lse, colmass, workspace=None, q_compact=False, o_compact=False,
                commit=None, formula: str = "column", exit_flags=None, dev_status=None) -> fl_attend_args:
    """`commit` = dict(k_new=, v_new=, compact=False, slot_base=0, reset=True) fuses the
    KV commit of this loop into the call; `formula` is "column" or
    "mixture" (LAZY only); `exit_flags` (int32 [n_seq]) skips exited sequences; `dev_status`
    (int32 [1], zeroed by the caller) receives FL_DEV_* bits of failed run-time checks."""
    a = fl_attend_args()
    a.mode, a.kv, a.version = mode, C.pointer(kv.desc), version
    a.q_cur, a.q_prev = _ptr(q_cur), _ptr(q_prev)
    a.q_layout = FL_ROWS_COMPACT if q_compact else FL_ROWS_BY_TOKEN
    a.active_idx, a.n_active = _ptr(active_idx), n_active
    a.key_idx = _ptr(key_idx)
    a.n_keys = 0 if key_idx is None else key_idx.shape[-1]
    a.o, a.lse, a.colmass = _ptr(o), _ptr(lse), _ptr(colmass)
    a.o_layout = FL_ROWS_COMPACT if o_compact else FL_ROWS_BY_TOKEN
    if workspace is not None:
        a.workspace, a.workspace_bytes = _ptr(workspace), workspace.numel()
    if commit is not None:
        a.fuse_commit = 1
        a.k_new, a.v_new = _ptr(commit["k_new"]), _ptr(commit["v_new"])
        a.kv_layout = FL_ROWS_COMPACT if commit.get("compact", False) else FL_ROWS_BY_TOKEN
        a.commit_slot_base = commit.get("slot_base", 0)
        a.commit_reset = int(commit.get("reset", True))
    a.formula = FORMULAS[formula]
    a.exit_flags = _ptr(exit_flags)
    a.dev_status = _ptr(dev_status)
    return a


def attend_workspace_bytes(a: fl_attend_args) -> int:
    return int(lib().flashloop_attend_workspace_bytes(C.byref(a)))


def attend(a: fl_attend_args, stream=None) -> None:
    _check(lib().flashloop_attend(C.byref(a), _stream(stream)))


def attend_noalloc(a: fl_attend_args, stream=None) -> None:
    """flashloop_attend on the library's own per-GPU scratch (a.workspace is ignored)."""
    _check(lib().flashloop_attend_noalloc(C.byref(a), _stream(stream)))


def decode_loops(kv: KVStore, first: int, last: int, q: dict, active_idx: torch.Tensor, n_keys: int,
                 o: torch.Tensor, lse: torch.Tensor, colmass: torch.Tensor, k_new: dict, v_new: dict,
                 slot_base: dict, keys_out: Optional[torch.Tensor] = None, q_compact: bool = True,
                 o_compact: bool = True, kv_compact: bool = False, formula: str = "column",
                 exit_flags: Optional[torch.Tensor] = None, stream=None) -> None:
    """flashloop_decode_loops: lazy decode loops first..last in one launch.
    q[l] for l = first-1..last, k_new[l], v_new[l], slot_base[l] for
    l = first..last (dicts of tensors / ints, indexed by loop)."""
    a = fl_decode_loops_args()
    a.kv = C.pointer(kv.desc)
    a.first_version, a.last_version = first, last
    for l in range(first - 1, last + 1):
        a.q[l] = _ptr(q[l])
    for l in range(first, last + 1):
        a.k_new[l], a.v_new[l] = _ptr(k_new[l]), _ptr(v_new[l])
        a.commit_slot_base[l] = slot_base[l]
    a.q_layout = FL_ROWS_COMPACT if q_compact else FL_ROWS_BY_TOKEN
    a.o_layout = FL_ROWS_COMPACT if o_compact else FL_ROWS_BY_TOKEN
    a.kv_layout = FL_ROWS_COMPACT if kv_compact else FL_ROWS_BY_TOKEN
    a.active_idx, a.n_keys = _ptr(active_idx), n_keys
    a.o, a.lse, a.colmass = _ptr(o), _ptr(lse), _ptr(colmass)
    a.key_idx_out = _ptr(keys_out)
    a.formula = FORMULAS[formula]
    a.exit_flags = _ptr(exit_flags)
    _check(lib().flashloop_decode_loops(C.byref(a), _stream(stream)))


def exit_check(exit_flags: torch.Tensor, threshold: float, scores: Optional[torch.Tensor] = None,
               h_cur: Optional[torch.Tensor] = None, h_prev: Optional[torch.Tensor] = None,
               max_change: Optional[torch.Tensor] = None, stream=None) -> None:
    """Sets exit_flags[s] (int32 [n_seq], never cleared) where the sequence's
    largest change is below `threshold`: from `scores` (float64 [n_seq, n_rows])
    or from h_cur/h_prev ([n_seq, n_rows, hidden])."""
    a = fl_exit_args()
    a.n_seq = exit_flags.numel()
    if scores is not None:
        a.scores = _ptr(scores)
        a.n_rows = scores.numel() // a.n_seq
    else:
        a.h_cur, a.h_prev, a.h_dtype = _ptr(h_cur), _ptr(h_prev), dtype_code(h_cur.dtype)
        a.hidden = h_cur.shape[-1]
        a.n_rows = h_cur.numel() // (a.n_seq * a.hidden)
    a.threshold = float(threshold)
    a.exit_flags, a.max_change = _ptr(exit_flags), _ptr(max_change)
    _check(lib().flashloop_exit_check(C.byref(a), _stream(stream)))


def timing_enable(on: bool) -> None:
    _check(lib().flashloop_timing_enable(int(on)))


def timing_read() -> dict:
    """{kernel name: (total ms, launches)} since timing_enable(True)."""
    n = lib().flashloop_timing_read(None, None, None, 0)
    names = C.create_string_buffer(64 * max(n, 1))
    ms = (C.c_double * max(n, 1))()
    cnt = (C.c_int64 * max(n, 1))()
    n = lib().flashloop_timing_read(names, ms, cnt, n)
    return {names.raw[64 * i:64 * (i + 1)].rstrip(b"\0").decode(): (ms[i], cnt[i]) for i in range(n)}


def abi_version() -> int:
    return int(lib().flashloop_abi_version())
