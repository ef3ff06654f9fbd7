"""Driver-level invariants of the oracle's prefill loop (CPU only).

The lazy loop's wiring -- which hidden states feed the token score, which
query and which store version feed the previous-loop probabilities p', their
mass m and contribution a, and which feed the current softmax -- is pinned
here through whole runs of ``run_prefill``, not through ``lazy_attention``
alone (page "FlashLoop: Fast and Memory-Efficient Looped Transformers via Lazy
Updates", section "FlashLoop combines three kinds of savings", paragraphs 1-2:
later loops recompute the active tokens and attend to keys chosen from the
previous loop's statistics, the chosen group keeping its previous mass).

I1  every key selected: each lazy loop reproduces full attention of its
    active rows over the store's version l (m = 1 exactly in real arithmetic),
    and the column mass becomes that of the matrix whose row i is the
    probability row of i's last active loop;
I2  every row active and every key selected: each lazy loop is the dense loop
    (o, lse, column mass) and writes a dense delta layer;
I3  a trajectory whose Q, K, V stop changing: a lazy loop leaves o, lse and
    the column mass as they were (the K/V inputs are built on the int4
    lattice, so the store reproduces them exactly and the versions before the
    stop differ from each other).
"""
import dataclasses

import numpy as np
import pytest

import oracle
from oracle import full_attention, run_prefill, to_working_dtype
from sparse_loop_attention_amd import configs
from sparse_loop_attention_amd.synth import SyntheticLoops


def _data(wl):
    return [(l, {k: v.copy() for k, v in x.items()}) for l, x in SyntheticLoops(wl)]


def _version(store, l, dtype):
    return (to_working_dtype(store.reconstruct("k", l), dtype), to_working_dtype(store.reconstruct("v", l), dtype))


@pytest.mark.parametrize("wl", [
    dataclasses.replace(configs.scaled(configs.SINGLE_LAYER, 192, n_heads=2), n_keys=192),
    dataclasses.replace(configs.scaled(configs.DEEP, 160, n_heads=2), n_loops=7, active=(48, 40, 33), n_keys=160),
], ids=["single_layer_192", "deep_160"])
def test_every_key_selected_gives_full_attention_each_loop(wl):
    """I1 at the driver level, loop after loop (active sets nest, so each
    active row's previous state is exact full attention of its loop l-1)."""
    data = _data(wl)
    st, hist = run_prefill(wl, iter(data), keep=True)
    x = dict(data)
    last_active = {}                                     # row -> its last active loop
    n = wl.n_tokens
    for l in range(1, wl.n_loops + 1):
        s = hist[l - 1]
        rows = np.arange(n) if l <= wl.n_full else s.records[l]["rows"]
        for i in rows:
            last_active[int(i)] = l
        if l <= wl.n_full:
            continue
        kh, vh = _version(st.store, l, wl.dtype)
        o, lse, _ = full_attention(x[l]["q"][0][rows], kh, vh, rows)
        np.testing.assert_allclose(s.records[l]["mass"], 1.0, rtol=1e-10)
        np.testing.assert_allclose(s.o[rows], o, rtol=1e-9, atol=1e-10)
        np.testing.assert_allclose(s.lse[rows], lse, rtol=1e-10, atol=1e-10)
        # the column mass is that of the rows' probabilities at their last active loop
        c = np.zeros_like(s.colmass)
        for lam in sorted(set(last_active.values())):
            rr = np.array(sorted(i for i, v in last_active.items() if v == lam))
            kl, vl = _version(st.store, lam, wl.dtype)
            _, _, cl = full_attention(x[lam]["q"][0][rr], kl, vl, rr)
            c += cl
        np.testing.assert_allclose(s.colmass, c, rtol=1e-9, atol=1e-11)


def test_every_row_and_key_is_the_dense_loop():
    """I2 at the driver level: with n_active = N and n_keys = N the lazy loops
    give the dense loop's o, lse and column mass, and each writes a record for
    every token (a dense delta layer)."""
    base = configs.scaled(configs.SINGLE_LAYER, 160, n_heads=2)
    wl = dataclasses.replace(base, active=(160, 160), n_keys=160)
    data = _data(wl)
    st, hist = run_prefill(wl, iter(data), keep=True)
    x = dict(data)
    rows = np.arange(wl.n_tokens)
    for l in range(wl.n_full + 1, wl.n_loops + 1):
        s = hist[l - 1]
        assert np.array_equal(s.records[l]["rows"], rows)
        kh, vh = _version(st.store, l, wl.dtype)
        o, lse, c = full_attention(x[l]["q"][0], kh, vh, rows)
        np.testing.assert_allclose(s.o, o, rtol=1e-9, atol=1e-10)
        np.testing.assert_allclose(s.lse, lse, rtol=1e-10, atol=1e-10)
        np.testing.assert_allclose(s.colmass, c, rtol=1e-9, atol=1e-11)
        for w in ("k", "v"):
            assert np.array_equal(st.store.layers[l][w][0].idx, rows)


def _lattice_loops(wl, stop_after):
    """Inputs of a bf16 workload whose K/V deltas are int4 lattice points:
    loop-1 values are multiples of 1/8 in [-2, 2]; every later loop adds
    c/8 with integer c in [-7, 7] and |c| = 7 at the first element of each
    32-element group (so each group's scale is exactly 1/8 and every code is
    c), until loop ``stop_after``; later loops repeat that loop's h, Q, K, V
    exactly.  All values are bf16-representable."""
    rng = np.random.default_rng(77)
    n, H, d = wl.n_tokens, wl.n_heads, wl.head_dim
    eighths = lambda *shape: rng.integers(-16, 17, shape).astype(np.float32) / 8
    step = lambda: np.where((np.arange(d) % 32 == 0), 7 * rng.choice([-1, 1], (n, H, d)),
                            rng.integers(-7, 8, (n, H, d))).astype(np.float32) / 8
    out = [(0, {"h": eighths(1, n, H * d)})]
    cur = {"h": eighths(1, n, H * d), "q": eighths(1, n, H, d), "k": eighths(1, n, H, d), "v": eighths(1, n, H, d)}
    for l in range(1, wl.n_loops + 1):
        if 1 < l <= stop_after:
            cur = {"h": cur["h"] + eighths(1, n, H * d), "q": cur["q"] + eighths(1, n, H, d),
                   "k": cur["k"] + step()[None], "v": cur["v"] + step()[None]}
        out.append((l, {k: v.copy() for k, v in cur.items()}))
    return out


def test_trajectory_that_stops_changing_is_a_fixed_point():
    """I3 at the driver level: loops 1-3 change Q, K, V (loop 3 lazy), loop 4
    repeats loop 3's inputs; loop 4 leaves o, lse and the column mass of loop 3
    unchanged, although version 3 of the store differs from version 2."""
    base = configs.scaled(configs.SINGLE_LAYER, 160, n_heads=2)
    wl = dataclasses.replace(base, active=(64, 48), n_keys=40)
    data = _lattice_loops(wl, stop_after=3)
    x = dict(data)
    st, hist = run_prefill(wl, iter(data), keep=True)
    # the lattice inputs are stored exactly: version l reproduces loop l's K, V
    for l in range(1, 4):
        rows = np.arange(wl.n_tokens) if l <= wl.n_full else hist[l - 1].records[l]["rows"]
        k = st.store.reconstruct("k", l)
        np.testing.assert_array_equal(k[rows], x[l]["k"][0][rows])
    assert not np.array_equal(st.store.reconstruct("k", 3), st.store.reconstruct("k", 2))
    s3, s4 = hist[2], hist[3]
    assert s4.records[4]["updated"].any()
    np.testing.assert_allclose(s4.o, s3.o, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(s4.lse, s3.lse, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(s4.colmass, s3.colmass, rtol=1e-10, atol=1e-11)


def test_checkpoint_round_trip_resumes_identically(tmp_path):
    """save_state / load_state keep every buffer the next loop reads: a run
    resumed from the checkpoint after each loop ends bit-identical to the
    uninterrupted run."""
    wl = configs.scaled(configs.SINGLE_LAYER, 128, n_heads=2)
    data = _data(wl)
    full, hist = run_prefill(wl, iter(data), keep=True)
    for l in range(1, wl.n_loops):
        path = str(tmp_path / f"after{l}.npz")
        oracle.save_state(hist[l - 1], path)
        res = run_prefill(wl, iter(data), resume=oracle.load_state(path))
        for f in ("o", "lse", "colmass", "h", "q"):
            assert np.array_equal(getattr(full, f), getattr(res, f)), (l, f)
        for l2 in range(2, wl.n_loops + 1):
            for w in ("k", "v"):
                assert np.array_equal(full.store.reconstruct(w, l2), res.store.reconstruct(w, l2))
