"""The oracle's variants (CPU only): the mixture formula (V1) and frozen key
sets (V2).

V1 is the other reading of "the selected group keeps its previous mass"
(page "FlashLoop: Fast and Memory-Efficient Looped Transformers via Lazy
Updates", section "FlashLoop combines three kinds of savings", paragraph 2):
o = m * otilde + (1 - m) * o_prev.  V2 keeps the first lazy loop's key group
(section "Later loops change only part of the state", paragraph 4: the group
that carries the change is small and stable).  Pinned here by closed forms and
special cases that follow from the mathematics.
"""
import math

import numpy as np

from oracle import full_attention, lazy_attention, run_prefill
from sparse_loop_attention_amd import configs
from sparse_loop_attention_amd.synth import SyntheticLoops


def rand(rng, *shape):
    return rng.standard_normal(shape).astype(np.float32)


def _two_versions(rng, n, H, d, change=0.3):
    q0, k0, v0 = rand(rng, n, H, d), rand(rng, n, H, d), rand(rng, n, H, d)
    return (q0, k0, v0), (q0 + change * rand(rng, n, H, d), k0 + change * rand(rng, n, H, d),
                          v0 + change * rand(rng, n, H, d))


def test_mixture_with_every_key_is_full_attention():
    """With S = every key after a full loop, m = 1 and both readings give
    full attention at the new version."""
    rng = np.random.default_rng(12)
    n, H, d = 48, 2, 32
    (q0, k0, v0), (q1, k1, v1) = _two_versions(rng, n, H, d)
    o0, lse0, c0 = full_attention(q0, k0, v0, np.arange(n))
    rows = np.array([0, 5, 17, 47])
    keys = np.tile(np.arange(n), (H, 1))
    o, lse, c, m, upd = lazy_attention(q1[rows], q0[rows], k0, v0, k1, v1, o0[rows], lse0[rows], c0,
                                       rows, keys, formula="mixture")
    o1, lse1, _ = full_attention(q1, k1, v1, np.arange(n))
    np.testing.assert_allclose(m, 1.0, rtol=1e-12)
    np.testing.assert_allclose(o, o1[rows], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, lse1[rows], rtol=1e-12, atol=1e-12)


def test_mixture_single_key_closed_form():
    """S_i = {j}: o = p'_ij v^_j(l) + (1 - p'_ij) o_prev."""
    rng = np.random.default_rng(13)
    n, H, d = 20, 1, 32
    (q0, k0, v0), (q1, k1, v1) = _two_versions(rng, n, H, d)
    o0, lse0, c0 = full_attention(q0, k0, v0, np.arange(n))
    j, i = 4, 13
    rows, keys = np.array([i]), np.array([[j]])
    o, _, c, m, _ = lazy_attention(q1[rows], q0[rows], k0, v0, k1, v1, o0[rows], lse0[rows], c0,
                                   rows, keys, formula="mixture")
    pp = math.exp(float(q0[i, 0].astype(np.float64) @ k0[j, 0].astype(np.float64)) / math.sqrt(d)
                  - lse0[i, 0])
    want = pp * v1[j, 0].astype(np.float64) + (1.0 - pp) * o0[i, 0]
    np.testing.assert_allclose(o[0, 0], want, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(m[0, 0], pp, rtol=1e-12)
    np.testing.assert_allclose(c, c0, rtol=1e-12, atol=1e-14)   # statistics as under R4


def test_mixture_is_not_a_fixed_point():
    """With nothing changed, R4 keeps o; the mixture moves it by
    a - m * o_prev (the selected keys' old contribution counted twice)."""
    rng = np.random.default_rng(14)
    n, H, d = 60, 2, 32
    q, k, v = rand(rng, n, H, d), rand(rng, n, H, d), rand(rng, n, H, d)
    o0, lse0, c0 = full_attention(q, k, v, np.arange(n))
    rows = np.sort(rng.choice(n, 20, replace=False))
    keys = np.stack([np.sort(rng.choice(n, 12, replace=False)) for _ in range(H)])
    ob, lb, cb, mb, _ = lazy_attention(q[rows], q[rows], k, v, k, v, o0[rows], lse0[rows], c0, rows, keys)
    om, lm, cm, mm, upd = lazy_attention(q[rows], q[rows], k, v, k, v, o0[rows], lse0[rows], c0, rows, keys,
                                         formula="mixture")
    np.testing.assert_allclose(ob, o0[rows], rtol=1e-10, atol=1e-12)
    # a_i = sum over S_i of p_ij v_j with the unchanged probabilities, evaluated directly
    s = np.einsum("rhd,nhd->rhn", q[rows].astype(np.float64), k.astype(np.float64)) / math.sqrt(d)
    p = np.exp(s - lse0[rows][:, :, None])
    a = np.zeros_like(o0[rows])
    m = np.zeros(lb.shape)
    for r, i in enumerate(rows):
        for h in range(H):
            sel = keys[h][keys[h] <= i]
            a[r, h] = p[r, h, sel] @ v[sel, h].astype(np.float64)
            m[r, h] = p[r, h, sel].sum()
    want = np.where(upd[:, :, None], o0[rows] + a - m[:, :, None] * o0[rows], o0[rows])
    np.testing.assert_allclose(om, want, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lm, lb, rtol=0, atol=0)          # same statistics as R4
    np.testing.assert_allclose(cm, cb, rtol=0, atol=0)
    np.testing.assert_allclose(mm, m, rtol=1e-10)


def test_frozen_keys_reuse_the_first_lazy_group():
    wl = configs.scaled(configs.SINGLE_LAYER, 256, n_heads=2)
    _, hd = run_prefill(wl, iter(SyntheticLoops(wl)), keep=True)
    _, hf = run_prefill(wl, iter(SyntheticLoops(wl)), keep=True, freeze_keys=True)
    first = wl.n_full + 1
    k_first = hf[first - 1].records[first]["keys"]
    np.testing.assert_array_equal(k_first, hd[first - 1].records[first]["keys"])
    for l in range(first + 1, wl.n_loops + 1):
        np.testing.assert_array_equal(hf[l - 1].records[l]["keys"], k_first)
    # the first lazy loop is identical either way; later ones differ only through the keys
    np.testing.assert_array_equal(hf[first - 1].o, hd[first - 1].o)
    for l in range(first + 1, wl.n_loops + 1):
        if np.array_equal(hd[l - 1].records[l]["keys"], k_first):
            np.testing.assert_array_equal(hf[l - 1].o, hd[l - 1].o)
