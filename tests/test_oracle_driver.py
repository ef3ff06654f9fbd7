"""The oracle's loop driver on small workloads (CPU only).

Page "FlashLoop: Fast and Memory-Efficient Looped Transformers via Lazy
Updates": early loops run in full, later loops recompute only the active
tokens, inactive tokens reuse their state and KV entries, and active sets
shrink and nest (section "Later loops change only part of the state",
paragraph 3; section "FlashLoop combines three kinds of savings",
paragraphs 1 and 3).
"""
import numpy as np
import pytest

from sparse_loop_attention_amd import configs
from sparse_loop_attention_amd.synth import SyntheticLoops
from oracle import run_prefill, full_attention, token_scores


def test_workload_counts():
    c = configs
    assert (c.TINY.active, c.TINY.n_keys) == ((64,), 26)
    assert (c.SINGLE_LAYER.active, c.SINGLE_LAYER.n_keys, c.SINGLE_LAYER.n_heavy) == ((820, 820), 410, 82)
    assert c.LONG_PREFILL.active == (9831, 4916, 2622) and c.LONG_PREFILL.n_keys == 3277
    assert c.DECODE.n_keys == 820 and c.DECODE.layer_caps() == [8192, 1640, 1640]
    assert c.DEEP.active[0] == 4916 and c.DEEP.active[-1] == 820 and len(c.DEEP.active) == 12
    assert all(a >= b for a, b in zip(c.DEEP.active, c.DEEP.active[1:]))
    assert c.DEEP.n_keys == 1639


def test_synth_is_seeded_and_dtype_exact():
    wl = configs.scaled(configs.SINGLE_LAYER, 128, n_heads=2)
    a = dict(SyntheticLoops(wl))
    b = dict(SyntheticLoops(wl))
    for l in a:
        for name in a[l]:
            assert np.array_equal(a[l][name], b[l][name])
    x = SyntheticLoops(wl)
    x.loop(0)
    q = x.loop(1)["q"]
    bits = q.view(np.uint32) & 0xFFFF
    assert np.all(bits == 0)                      # bf16-representable values


def _run(wl, keep=True):
    return run_prefill(wl, iter(SyntheticLoops(wl)), keep=keep)


def test_tiny_full_then_lazy():
    wl = configs.TINY
    st, hist = _run(wl)
    assert len(hist) == 2
    rec = hist[1].records[2]
    assert rec["rows"].shape == (64,) and np.all(np.diff(rec["rows"]) > 0)
    assert rec["keys"].shape == (1, 26)
    # loop-1 state equals dense attention on the base
    s1 = hist[0]
    o, lse, c = full_attention(s1.q, s1.store.reconstruct("k", 1), s1.store.reconstruct("v", 1),
                               np.arange(wl.n_tokens))
    np.testing.assert_allclose(s1.o, o)
    # inactive rows carry o and lse from loop 1
    inactive = np.setdiff1d(np.arange(wl.n_tokens), rec["rows"])
    np.testing.assert_array_equal(st.o[inactive], s1.o[inactive])
    np.testing.assert_array_equal(st.lse[inactive], s1.lse[inactive])
    # the planted heavy keys are selected (logit boost +4)
    heavy = SyntheticLoops(wl).heavy[0]
    assert set(heavy.tolist()) <= set(rec["keys"][0].tolist())
    # only active tokens wrote a delta at loop 2
    assert np.array_equal(st.store.layers[2]["k"][0].idx, rec["rows"])
    assert np.sum(st.colmass) == pytest.approx(wl.n_tokens, rel=1e-12)


def test_single_layer_scaled_nesting_and_carry():
    wl = configs.scaled(configs.SINGLE_LAYER, 256, n_heads=2)
    st, hist = _run(wl)
    a3 = hist[2].records[3]["rows"]
    a4 = hist[3].records[4]["rows"]
    u4 = hist[3].records[4]["scores"]
    assert np.all(u4[np.setdiff1d(np.arange(wl.n_tokens), a3)] == 0.0)      # I10
    assert set(a4.tolist()) <= set(a3.tolist())                            # I9
    # full loop 2 wrote a dense delta layer, lazy loops one record per active token
    assert st.store.layers[2]["k"][0].idx.shape[0] == wl.n_tokens
    assert st.store.layers[3]["k"][0].idx.shape[0] == wl.n_active(3)
    # carried hidden state: rows outside A4 equal their loop-3 value
    np.testing.assert_array_equal(st.h[np.setdiff1d(np.arange(wl.n_tokens), a4)],
                                  hist[2].h[np.setdiff1d(np.arange(wl.n_tokens), a4)])
    np.testing.assert_allclose(st.colmass.sum(1), wl.n_tokens, rtol=1e-10)
    # token scores at loop 4 are the change made by loop 3
    np.testing.assert_array_equal(u4, token_scores(hist[2].h, hist[1].h))


def test_chain_driver_matches_full_driver():
    """The attention-free chain driver reproduces the full driver's token sets and store."""
    from oracle import run_prefill_chain
    wl = configs.scaled(configs.SINGLE_LAYER, 256, n_heads=2)
    st, hist = _run(wl)
    store, active, _ = run_prefill_chain(wl, iter(SyntheticLoops(wl)))
    for l in range(wl.n_full + 1, wl.n_loops + 1):
        assert np.array_equal(active[l], hist[l - 1].records[l]["rows"])
    for l in range(1, wl.n_loops + 1):
        for w in ("k", "v"):
            assert np.array_equal(store.reconstruct(w, l), st.store.reconstruct(w, l))


def test_decode_with_every_key_equals_full_attention_each_loop():
    """I1 applied loop after loop: when every key is selected, each lazy decode
    loop keeps mass 1 and reproduces full attention of the new token over its
    own version of the store."""
    import dataclasses
    from oracle import build_decode_context, run_decode_loops, to_working_dtype
    wl = dataclasses.replace(configs.scaled(configs.DECODE, 96, n_seq=2, n_heads=2), n_keys=96)
    syn = SyntheticLoops(wl)
    ctx = {l: syn.context_active_sets(l)[1] for l in range(2, wl.n_loops + 1)}
    data = {l: {k: v.copy() for k, v in x.items()} for l, x in SyntheticLoops(wl)}
    store = build_decode_context(wl, 1, ctx, data)
    out = run_decode_loops(wl, store, 1, data)
    last = np.array([wl.n_tokens - 1])
    for l in range(1, wl.n_loops + 1):
        kh = to_working_dtype(store.reconstruct("k", l), wl.dtype)
        vh = to_working_dtype(store.reconstruct("v", l), wl.dtype)
        o, lse, c = full_attention(data[l]["q"][1], kh, vh, last)
        np.testing.assert_allclose(out[l - 1]["o"], o, rtol=1e-9, atol=1e-9)
        np.testing.assert_allclose(out[l - 1]["lse"], lse, rtol=1e-9, atol=1e-9)
        np.testing.assert_allclose(out[l - 1]["colmass"], c, rtol=1e-9, atol=1e-12)
        if l >= 2:
            np.testing.assert_allclose(out[l - 1]["mass"], 1.0, rtol=1e-9)
    # the token's own record sits in every layer, the context's only where it was active
    for l in range(2, wl.n_loops + 1):
        idx = np.concatenate([r.idx for r in store.layers[l]["k"]])
        assert np.array_equal(np.sort(idx), np.union1d(ctx[l], last))


def test_decode_resume_equals_uninterrupted_run():
    """run_decode_loops continued from the state after loop l (start = l + 1)
    gives the uninterrupted run's loops bit for bit."""
    import copy
    from oracle import build_decode_context, run_decode_loops
    wl = configs.scaled(configs.DECODE, 128, n_seq=2, n_heads=2)
    syn = SyntheticLoops(wl)
    ctx = {l: syn.context_active_sets(l)[0] for l in range(2, wl.n_loops + 1)}
    data = {l: {k: v.copy() for k, v in x.items()} for l, x in SyntheticLoops(wl)}
    store = build_decode_context(wl, 0, ctx, data)
    whole = run_decode_loops(wl, copy.deepcopy(store), 0, data)
    for cut in range(1, wl.n_loops):
        st = copy.deepcopy(store)
        head = run_decode_loops(wl, st, 0, data, upto=cut)
        tail = run_decode_loops(wl, st, 0, data, start=cut + 1, state=head[-1])
        for a, b in zip(whole, head + tail):
            for k in ("o", "lse", "colmass"):
                assert np.array_equal(a[k], b[k]), (cut, k)
