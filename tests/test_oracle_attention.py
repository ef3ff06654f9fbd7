"""Pins for the oracle's full and mass-corrected attention (CPU only).

Full attention is pinned to torch's scaled_dot_product_attention (float64, CPU)
and logsumexp.  The mass-corrected lazy formula has no printed example on the
pages (parity unpinned by the pages); it is pinned by invariants that a
dropped term, a wrong sign, a transposed operand or the wrong version would
break: exact full attention when every key is selected, the dense loop when
every token is active, a fixed point when nothing changed, mass preservation
(page "FlashLoop: Fast and Memory-Efficient Looped Transformers via Lazy
Updates", section "FlashLoop combines three kinds of savings", paragraph 2),
and single-key closed forms.
"""
import math

import numpy as np
import pytest
import torch

from oracle import full_attention, lazy_attention


def rand(rng, *shape):
    return rng.standard_normal(shape).astype(np.float32)


def sdpa(q, k, v):
    """torch SDPA in float64 on the CPU; q [R,H,d] for rows 0..R-1 (causal)."""
    Q = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)[None]
    K = torch.from_numpy(k.astype(np.float64)).permute(1, 0, 2)[None]
    V = torch.from_numpy(v.astype(np.float64)).permute(1, 0, 2)[None]
    o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True)
    return o[0].permute(1, 0, 2).numpy()


def test_full_attention_matches_sdpa_and_logsumexp():
    rng = np.random.default_rng(0)
    n, H, d = 70, 3, 64
    q, k, v = rand(rng, n, H, d), rand(rng, n, H, d), rand(rng, n, H, d)
    o, lse, c = full_attention(q, k, v, np.arange(n), chunk=16)
    np.testing.assert_allclose(o, sdpa(q, k, v), rtol=1e-12, atol=1e-12)
    s = torch.einsum("ihd,jhd->hij", torch.from_numpy(q.astype(np.float64)),
                     torch.from_numpy(k.astype(np.float64))) / math.sqrt(d)
    s = s.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, -1).T.numpy(), rtol=1e-12, atol=1e-12)
    # column mass: P recovered from SDPA with one-hot values (v_j = e_j)
    eye = np.broadcast_to(np.eye(n)[:, None, :], (n, H, n)).copy()
    P = sdpa(q, k, eye)                                     # [i, h, j] = p_ij
    np.testing.assert_allclose(c, P.sum(0), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(c.sum(1), n, rtol=1e-12)      # every row sums to one
    assert np.all(c[:, -1] > 0) and np.allclose(c[:, -1], P[-1, :, -1])


def test_full_attention_row_subset():
    rng = np.random.default_rng(1)
    n, H, d = 40, 2, 32
    q, k, v = rand(rng, n, H, d), rand(rng, n, H, d), rand(rng, n, H, d)
    rows = np.array([0, 7, 8, 39])
    o, lse, c = full_attention(q[rows], k, v, rows)
    o_all, lse_all, _ = full_attention(q, k, v, np.arange(n))
    np.testing.assert_allclose(o, o_all[rows], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lse_all[rows], rtol=1e-12)
    np.testing.assert_allclose(c.sum(1), len(rows), rtol=1e-12)
    assert np.all(c[:, 9:39] > 0) and np.all(c[:, 40:] == 0)


def _two_versions(rng, n, H, d, change=0.3):
    q0, k0, v0 = rand(rng, n, H, d), rand(rng, n, H, d), rand(rng, n, H, d)
    q1 = q0 + change * rand(rng, n, H, d)
    k1 = k0 + change * rand(rng, n, H, d)
    v1 = v0 + change * rand(rng, n, H, d)
    return (q0, k0, v0), (q1, k1, v1)


def test_all_keys_selected_gives_full_attention():
    """I1: with S = every key and a full previous loop, m_i = 1, a_i = o_prev_i
    and the lazy rows equal full attention at the new version."""
    rng = np.random.default_rng(2)
    n, H, d = 64, 2, 64
    (q0, k0, v0), (q1, k1, v1) = _two_versions(rng, n, H, d)
    o0, lse0, c0 = full_attention(q0, k0, v0, np.arange(n))
    rows = np.array([3, 10, 11, 40, 63])
    keys = np.tile(np.arange(n), (H, 1))
    o, lse, c, m, upd = lazy_attention(q1[rows], q0[rows], k0, v0, k1, v1, o0[rows], lse0[rows],
                                       c0, rows, keys)
    o1, lse1, c1 = full_attention(q1, k1, v1, np.arange(n))
    assert upd.all()
    np.testing.assert_allclose(m, 1.0, rtol=1e-12)
    np.testing.assert_allclose(o, o1[rows], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, lse1[rows], rtol=1e-12, atol=1e-12)
    # column mass becomes that of the mixed matrix: new rows for A, old rows elsewhere
    _, _, c_new_rows = full_attention(q1[rows], k1, v1, rows)
    others = np.setdiff1d(np.arange(n), rows)
    _, _, c_old_rows = full_attention(q0[others], k0, v0, others)
    np.testing.assert_allclose(c, c_new_rows + c_old_rows, rtol=1e-10, atol=1e-12)


def test_all_active_all_keys_is_dense_loop():
    """I2: A = all rows and S = all keys reproduce the dense loop exactly."""
    rng = np.random.default_rng(3)
    n, H, d = 48, 3, 32
    (q0, k0, v0), (q1, k1, v1) = _two_versions(rng, n, H, d)
    o0, lse0, c0 = full_attention(q0, k0, v0, np.arange(n))
    rows = np.arange(n)
    keys = np.tile(np.arange(n), (H, 1))
    o, lse, c, _, _ = lazy_attention(q1, q0, k0, v0, k1, v1, o0, lse0, c0, rows, keys)
    o1, lse1, c1 = full_attention(q1, k1, v1, rows)
    np.testing.assert_allclose(o, o1, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, lse1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(c, c1, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("frac", [0.1, 0.5])
def test_fixed_point_when_nothing_changed(frac):
    """I3: Q, K, V unchanged -> o, lse and c unchanged for any key subset.
    (The other reading, m*otilde + (1-m)*o_prev, fails this.)"""
    rng = np.random.default_rng(4)
    n, H, d = 80, 2, 64
    q, k, v = rand(rng, n, H, d), rand(rng, n, H, d), rand(rng, n, H, d)
    o0, lse0, c0 = full_attention(q, k, v, np.arange(n))
    rows = np.sort(rng.choice(n, 30, replace=False))
    nk = max(1, int(frac * n))
    keys = np.stack([np.sort(rng.choice(n, nk, replace=False)) for _ in range(H)])
    o, lse, c, m, upd = lazy_attention(q[rows], q[rows], k, v, k, v, o0[rows], lse0[rows], c0,
                                       rows, keys)
    np.testing.assert_allclose(o, o0[rows], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, lse0[rows], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(c, c0, rtol=1e-10, atol=1e-12)
    assert np.all(m[upd] > 0) and np.all(m <= 1 + 1e-12) and upd.any()


def test_single_key_closed_form():
    """I4: S_i = {j}: the renormalised softmax over one key is 1, so
    o = p'_ij * v^_j(l) + o_prev - p'_ij * v^_j(l-1)."""
    rng = np.random.default_rng(5)
    n, H, d = 20, 1, 32
    (q0, k0, v0), (q1, k1, v1) = _two_versions(rng, n, H, d)
    o0, lse0, c0 = full_attention(q0, k0, v0, np.arange(n))
    j, i = 6, 15
    rows = np.array([i])
    keys = np.array([[j]])
    o, lse, c, m, _ = lazy_attention(q1[rows], q0[rows], k0, v0, k1, v1, o0[rows], lse0[rows], c0,
                                     rows, keys)
    pp = math.exp(float(q0[i, 0].astype(np.float64) @ k0[j, 0].astype(np.float64)) / math.sqrt(d)
                  - lse0[i, 0])
    want = pp * v1[j, 0].astype(np.float64) + o0[i, 0] - pp * v0[j, 0].astype(np.float64)
    np.testing.assert_allclose(o[0, 0], want, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(m[0, 0], pp, rtol=1e-12)
    # the single selected column keeps its mass: p_ij = m_i = p'_ij, so c is unchanged
    np.testing.assert_allclose(c, c0, rtol=1e-12, atol=1e-14)
    # lse changes so that exp(s_ij - lse_new) = p'_ij
    s1 = float(q1[i, 0].astype(np.float64) @ k1[j, 0].astype(np.float64)) / math.sqrt(d)
    np.testing.assert_allclose(math.exp(s1 - lse[0, 0]), pp, rtol=1e-12)


def test_empty_selection_and_no_active_rows():
    """I5 and reading R6: rows with no visible selected key, and an empty
    active set, change nothing."""
    rng = np.random.default_rng(6)
    n, H, d = 30, 2, 32
    (q0, k0, v0), (q1, k1, v1) = _two_versions(rng, n, H, d)
    o0, lse0, c0 = full_attention(q0, k0, v0, np.arange(n))
    rows = np.array([2, 25])
    keys = np.array([[5, 9], [3, 29]])       # row 2 sees no selected key in either head
    o, lse, c, m, upd = lazy_attention(q1[rows], q0[rows], k0, v0, k1, v1, o0[rows], lse0[rows],
                                       c0, rows, keys)
    assert not upd[0].any() and upd[1, 0] and upd[1, 1]
    np.testing.assert_array_equal(o[0], o0[2])
    np.testing.assert_array_equal(lse[0], lse0[2])
    empty = np.zeros(0, np.int64)
    o, lse, c, m, upd = lazy_attention(q1[empty], q0[empty], k0, v0, k1, v1, o0[empty],
                                       lse0[empty], c0, empty, keys)
    np.testing.assert_array_equal(c, c0)


def test_mass_preservation_and_column_sum():
    """I6, I7: each updated row keeps sum_{S_i} p_ij = m_i, and sum_j c_j stays N."""
    rng = np.random.default_rng(7)
    n, H, d = 96, 2, 64
    (q0, k0, v0), (q1, k1, v1) = _two_versions(rng, n, H, d, change=0.8)
    o0, lse0, c0 = full_attention(q0, k0, v0, np.arange(n))
    rows = np.sort(rng.choice(n, 40, replace=False))
    keys = np.stack([np.sort(rng.choice(n, 12, replace=False)) for _ in range(H)])
    o, lse, c, m, upd = lazy_attention(q1[rows], q0[rows], k0, v0, k1, v1, o0[rows], lse0[rows],
                                       c0, rows, keys)
    for h in range(H):
        for r, i in enumerate(rows):
            sel = keys[h][keys[h] <= i]
            if not upd[r, h]:
                continue
            s = (q1[i, h].astype(np.float64) @ k1[sel, h].astype(np.float64).T) / math.sqrt(d)
            np.testing.assert_allclose(np.exp(s - lse[r, h]).sum(), m[r, h], rtol=1e-12)
    np.testing.assert_allclose(c.sum(1), n, rtol=1e-12)
    np.testing.assert_allclose(np.delete(c, keys[0], axis=1)[0], np.delete(c0, keys[0], axis=1)[0])


def test_lazy_against_loop_brute_force():
    """Element-by-element pure-Python evaluation on a tiny case (float64)."""
    rng = np.random.default_rng(8)
    n, H, d = 10, 1, 8
    (q0, k0, v0), (q1, k1, v1) = _two_versions(rng, n, H, d)
    o0, lse0, c0 = full_attention(q0, k0, v0, np.arange(n))
    rows = np.array([1, 4, 9])
    keys = np.array([[0, 4, 5, 8]])
    o, lse, c, m, _ = lazy_attention(q1[rows], q0[rows], k0, v0, k1, v1, o0[rows], lse0[rows], c0,
                                     rows, keys)
    dot = lambda a, b: sum(float(x) * float(y) for x, y in zip(a, b))
    cc = [float(x) for x in c0[0]]
    for r, i in enumerate(rows):
        S = [j for j in keys[0] if j <= i]
        pp = {j: math.exp(dot(q0[i, 0], k0[j, 0]) / math.sqrt(d) - lse0[i, 0]) for j in S}
        mm = sum(pp.values())
        sc = {j: dot(q1[i, 0], k1[j, 0]) / math.sqrt(d) for j in S}
        M = max(sc.values())
        Z = sum(math.exp(sc[j] - M) for j in S)
        for t in range(d):
            ot = sum(math.exp(sc[j] - M) * float(v1[j, 0, t]) for j in S) / Z
            at = sum(pp[j] * float(v0[j, 0, t]) for j in S)
            assert abs(o[r, 0, t] - (mm * ot + float(o0[i, 0, t]) - at)) < 1e-12
        assert abs(lse[r, 0] - (M + math.log(Z) - math.log(mm))) < 1e-12
        for j in S:
            cc[j] += mm * math.exp(sc[j] - M) / Z - pp[j]
    np.testing.assert_allclose(c[0], cc, rtol=1e-12, atol=1e-14)
