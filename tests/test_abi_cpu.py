"""The C ABI on the host: the library loads, exports what the header declares,
computes the arena layout, and rejects invalid arguments before any launch
(no GPU needed: validation runs before any HIP call)."""
import ctypes as C
import os
import re

import pytest

from sparse_loop_attention_amd import abi, configs

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "flashloop.h")


@pytest.fixture(scope="module")
def L():
    return abi.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(flashloop_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) == 13
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(abi.EXPORTS)
    assert abi.abi_version() == 5


def _desc(wl, group=32, bits=4):
    d = abi.fl_kv_desc()
    d.n_seq, d.n_heads, d.head_dim, d.n_tokens = wl.n_seq, wl.n_heads, wl.head_dim, wl.n_tokens
    d.n_versions, d.base_dtype, d.group = wl.n_loops, abi.FL_BF16 if wl.dtype == "bf16" else abi.FL_F32, group
    d.delta_bits = bits
    for i, c in enumerate(wl.layer_caps()):
        d.layer_cap[i + 2] = c
    return d


# every workload with every store format whose group divides its head_dim
# (the others are rejected: test_invalid_descriptors)
LAYOUT_CASES = [pytest.param(name, (g, b), id=f"{name}-{b}b{g}")
                for name, wl in configs.WORKLOADS.items()
                for g, b in [(32, 4), (64, 4), (32, 2), (64, 2)] if wl.head_dim % g == 0]


@pytest.mark.parametrize("name,fmt", LAYOUT_CASES)
def test_arena_layout_bytes(L, name, fmt):
    wl = configs.WORKLOADS[name]
    group, bits = fmt
    d = _desc(wl, group, bits)
    lay = abi.kv_layout(d)
    S, H, N, D = wl.n_seq, wl.n_heads, wl.n_tokens, wl.head_dim
    es = 2 if wl.dtype == "bf16" else 4
    assert lay.base_v - lay.base_k >= S * H * N * D * es
    need = 2 * S * H * N * D * es
    for l, cap in zip(range(2, wl.n_loops + 1), wl.layer_caps()):
        need += S * N * 4 + 2 * S * H * cap * (D * bits // 8 + 2 * (D // group))
        for arr in (lay.codes, lay.scales):
            assert arr[l] % 256 == 0
    assert lay.slot_table % 256 == 0 and lay.slot_pitch == ((wl.n_loops - 1 + 3) // 4) * 4
    need += S * N * 4 * (lay.slot_pitch - (wl.n_loops - 1))
    assert need <= lay.total_bytes <= need + 256 * (3 + 2 * wl.n_loops)
    assert abi.kv_arena_bytes(d) == lay.total_bytes


def test_compression_ratio_single_layer(L):
    """base + int4 deltas vs one bf16 cache per loop: 2.87x on the 4-loop,
    20%-active workload (page: 'up to 6x' KV-cache reduction)."""
    wl = configs.SINGLE_LAYER
    lay = abi.kv_layout(_desc(wl))
    naive = wl.n_loops * 2 * wl.n_heads * wl.n_tokens * wl.head_dim * 2
    slot_maps = lay.slot_pitch * wl.n_tokens * 4
    assert naive / (lay.total_bytes - slot_maps) == pytest.approx(2.87, abs=0.01)


def test_invalid_descriptors(L):
    d = _desc(configs.TINY)
    d.head_dim = 80
    assert abi.kv_arena_bytes(d) == 0
    assert b"head_dim" in L.flashloop_last_error()
    d = _desc(configs.TINY)
    d.group = 16
    assert L.flashloop_kv_layout(C.byref(d), C.byref(abi.fl_kv_layout())) == abi.FL_ERR_UNSUPPORTED
    d = _desc(configs.scaled(configs.DEEP, 320), group=64)                # head_dim 96
    assert L.flashloop_kv_layout(C.byref(d), C.byref(abi.fl_kv_layout())) == abi.FL_ERR_UNSUPPORTED
    assert b"divide" in L.flashloop_last_error()
    d = _desc(configs.TINY)
    d.delta_bits = 3
    assert L.flashloop_kv_layout(C.byref(d), C.byref(abi.fl_kv_layout())) == abi.FL_ERR_UNSUPPORTED
    assert b"delta_bits" in L.flashloop_last_error()
    d = _desc(configs.TINY)
    d.layer_cap[2] = 10 ** 6
    assert L.flashloop_kv_layout(C.byref(d), C.byref(abi.fl_kv_layout())) == abi.FL_ERR_ARG


def test_commit_validation(L):
    a = abi.fl_commit_args()
    assert L.flashloop_kv_commit(C.byref(a), None) == abi.FL_ERR_ARG
    d = _desc(configs.TINY)
    a.kv = C.pointer(d)
    assert L.flashloop_kv_commit(C.byref(a), None) == abi.FL_ERR_ARG      # no arena
    assert b"arena" in L.flashloop_last_error()
    d.arena, d.arena_bytes = 256, 16                                        # fake, too small
    assert L.flashloop_kv_commit(C.byref(a), None) == abi.FL_ERR_ARG
    d.arena_bytes = abi.kv_arena_bytes(d)
    a.version = 3                                                           # > n_versions
    assert L.flashloop_kv_commit(C.byref(a), None) == abi.FL_ERR_ARG
    a.version, a.n_active = 2, 5
    assert L.flashloop_kv_commit(C.byref(a), None) == abi.FL_ERR_ARG      # NULL pointers
    a.active_idx, a.k_new, a.v_new = 256, 256, 256
    a.slot_base = 62                                                        # 62 + 5 > cap 64
    assert L.flashloop_kv_commit(C.byref(a), None) == abi.FL_ERR_ARG
    assert b"layer_cap" in L.flashloop_last_error()
    a.slot_base, a.n_active = 0, 0
    assert L.flashloop_kv_commit(C.byref(a), None) == abi.FL_OK          # nothing to do


def test_select_validation(L):
    a = abi.fl_select_args()
    a.mode = 7
    assert L.flashloop_select(C.byref(a), None) == abi.FL_ERR_ARG
    a.mode = abi.FL_SEL_TOKENS
    assert L.flashloop_select(C.byref(a), None) == abi.FL_ERR_ARG
    a.h_cur = a.h_prev = a.scores = 256
    a.h_dtype, a.n_rows, a.hidden = abi.FL_BF16, 100, 12
    assert L.flashloop_select(C.byref(a), None) == abi.FL_ERR_UNSUPPORTED  # hidden % 8
    a.hidden, a.k = 64, 101
    assert L.flashloop_select(C.byref(a), None) == abi.FL_ERR_ARG
    a.n_rows = 70000
    assert L.flashloop_select(C.byref(a), None) == abi.FL_ERR_UNSUPPORTED
    b = abi.fl_select_args()
    b.mode, b.key_scores, b.n_seg, b.seg_len, b.k = abi.FL_SEL_KEYS, 256, 4, 100, 10
    assert L.flashloop_select(C.byref(b), None) == abi.FL_ERR_ARG          # NULL out_idx
    assert b"out_idx" in L.flashloop_last_error()


def test_attend_validation(L):
    d = _desc(configs.TINY)
    d.arena, d.arena_bytes = 256, abi.kv_arena_bytes(d)
    a = abi.fl_attend_args()
    a.kv = C.pointer(d)
    a.mode = 5
    assert L.flashloop_attend(C.byref(a), None) == abi.FL_ERR_ARG
    a.mode, a.version = abi.FL_ATTEND_LAZY, 1                              # LAZY needs version >= 2
    assert L.flashloop_attend(C.byref(a), None) == abi.FL_ERR_ARG
    a.version, a.n_active = 2, 0
    a.q_cur = a.q_prev = a.o = a.lse = a.colmass = 256
    a.key_idx, a.n_keys = 256, 26
    assert L.flashloop_attend(C.byref(a), None) == abi.FL_OK              # A empty: no-op
    a.n_active, a.active_idx = 64, 256
    need = L.flashloop_attend_workspace_bytes(C.byref(a))
    assert need > 0
    a.workspace, a.workspace_bytes = 256, need - 1
    assert L.flashloop_attend(C.byref(a), None) == abi.FL_ERR_WORKSPACE
    a.mode, a.version, a.active_idx, a.n_active = abi.FL_ATTEND_FULL, 1, None, 10
    assert L.flashloop_attend(C.byref(a), None) == abi.FL_ERR_ARG          # NULL rows need n_active == N


def test_attend_formula_validation(L):
    d = _desc(configs.TINY)
    d.arena, d.arena_bytes = 256, abi.kv_arena_bytes(d)
    a = abi.fl_attend_args()
    a.kv = C.pointer(d)
    a.mode, a.version, a.n_active = abi.FL_ATTEND_LAZY, 2, 0
    a.q_cur = a.q_prev = a.o = a.lse = a.colmass = 256
    a.key_idx, a.n_keys = 256, 26
    a.formula = abi.FL_FORMULA_MIXTURE
    assert L.flashloop_attend(C.byref(a), None) == abi.FL_OK              # LAZY accepts the mixture
    a.formula = 7
    assert L.flashloop_attend(C.byref(a), None) == abi.FL_ERR_ARG
    assert b"formula" in L.flashloop_last_error()
    a.mode, a.version, a.active_idx, a.n_active = abi.FL_ATTEND_FULL, 1, None, 256
    a.formula = abi.FL_FORMULA_MIXTURE
    assert L.flashloop_attend(C.byref(a), None) == abi.FL_ERR_ARG          # FULL: column only


def test_exit_check_validation(L):
    a = abi.fl_exit_args()
    assert L.flashloop_exit_check(C.byref(a), None) == abi.FL_ERR_ARG              # NULL flags
    assert b"exit_flags" in L.flashloop_last_error()
    a.exit_flags, a.n_seq, a.n_rows = 256, 0, 10
    assert L.flashloop_exit_check(C.byref(a), None) == abi.FL_ERR_ARG              # n_seq 0
    a.n_seq = 2
    assert L.flashloop_exit_check(C.byref(a), None) == abi.FL_ERR_ARG              # no scores, no h
    a.h_cur = a.h_prev = 256
    a.h_dtype, a.hidden = abi.FL_BF16, 12
    assert L.flashloop_exit_check(C.byref(a), None) == abi.FL_ERR_UNSUPPORTED      # hidden % 8
    a.exit_flags = 258
    assert L.flashloop_exit_check(C.byref(a), None) == abi.FL_ERR_ARG              # misaligned flags
    a.exit_flags, a.hidden, a.n_rows = 256, 64, 0
    assert L.flashloop_exit_check(C.byref(a), None) == abi.FL_ERR_ARG              # n_rows 0


def test_exit_flags_alignment(L):
    d = _desc(configs.TINY)
    d.arena, d.arena_bytes = 256, abi.kv_arena_bytes(d)
    c = abi.fl_commit_args()
    c.kv = C.pointer(d)
    c.version, c.n_active = 1, 5
    c.active_idx, c.k_new, c.v_new = 256, 256, 256
    c.exit_flags = 258
    assert L.flashloop_kv_commit(C.byref(c), None) == abi.FL_ERR_ARG
    assert b"exit_flags" in L.flashloop_last_error()
    a = abi.fl_attend_args()
    a.kv = C.pointer(d)
    a.mode, a.version, a.n_active = abi.FL_ATTEND_LAZY, 2, 0
    a.q_cur = a.q_prev = a.o = a.lse = a.colmass = 256
    a.key_idx, a.n_keys = 256, 26
    a.exit_flags = 258
    assert L.flashloop_attend(C.byref(a), None) == abi.FL_ERR_ARG


def test_attend_noalloc_rejects_beyond_its_scratch(L):
    """flashloop_attend_noalloc checks the call's scratch need against the
    library's per-GPU array before any HIP call: the 32K full loop (gathered
    tiles of every key) does not fit and is rejected; invalid arguments are
    rejected as by flashloop_attend."""
    wl = configs.LONG_PREFILL
    d = _desc(wl)
    d.arena, d.arena_bytes = 256, abi.kv_arena_bytes(d)
    a = abi.fl_attend_args()
    a.kv = C.pointer(d)
    a.mode, a.version, a.n_active = abi.FL_ATTEND_FULL, 1, wl.n_tokens
    a.q_cur = a.o = a.lse = a.colmass = 256
    assert L.flashloop_attend_workspace_bytes(C.byref(a)) > abi.STATIC_SCRATCH_BYTES
    assert L.flashloop_attend_noalloc(C.byref(a), None) == abi.FL_ERR_WORKSPACE
    assert b"scratch" in L.flashloop_last_error()
    a.mode = 9
    assert L.flashloop_attend_noalloc(C.byref(a), None) == abi.FL_ERR_ARG


def test_decode_loops_validation(L):
    """flashloop_decode_loops rejects invalid arguments before any launch."""
    wl = configs.DECODE
    d = _desc(wl)
    d.arena, d.arena_bytes = 256, abi.kv_arena_bytes(d)
    a = abi.fl_decode_loops_args()
    assert L.flashloop_decode_loops(C.byref(a), None) == abi.FL_ERR_ARG              # no descriptor
    a.kv = C.pointer(d)
    a.first_version, a.last_version, a.n_keys = 1, 4, 820
    assert L.flashloop_decode_loops(C.byref(a), None) == abi.FL_ERR_ARG              # first < 2
    a.first_version = 2
    a.active_idx, a.o, a.lse, a.colmass = 256, 256, 256, 256
    assert L.flashloop_decode_loops(C.byref(a), None) == abi.FL_ERR_ARG              # q[1..4] missing
    assert b"q[1]" in L.flashloop_last_error()
    for l in range(1, 5):
        a.q[l] = 256
    for l in range(2, 5):
        a.k_new[l] = a.v_new[l] = 256
        a.commit_slot_base[l] = wl.layer_caps()[l - 2]                               # one past the capacity
    assert L.flashloop_decode_loops(C.byref(a), None) == abi.FL_ERR_ARG
    assert b"commit_slot_base" in L.flashloop_last_error()
    a.last_version = 5
    assert L.flashloop_decode_loops(C.byref(a), None) == abi.FL_ERR_ARG              # beyond n_versions
