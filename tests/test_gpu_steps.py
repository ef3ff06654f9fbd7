"""GPU parity of each ABI call against the CPU oracle on identical inputs.

Bars: index sets and int4 codes bit-exact; attention outputs and column mass within
2e-2 x RMS (max abs error), lse within 2e-2 absolute; float64 token scores
within 1e-13 relative.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from sparse_loop_attention_amd import abi

pytestmark = pytest.mark.gpu
DEV = "cuda"


def bf16_round(x):
    from sparse_loop_attention_amd.synth import round_bf16
    return round_bf16(np.asarray(x, np.float32))


def to_dev(x, dtype):
    from sparse_loop_attention_amd.driver import to_device
    return to_device(np.ascontiguousarray(x, np.float32), dtype, DEV)


def rel_err_ok(got, want, tol=2e-2):
    want = np.asarray(want, np.float64)
    got = np.asarray(got, np.float64)
    rms = math.sqrt(float(np.mean(want ** 2)))
    err = float(np.abs(got - want).max()) if want.size else 0.0
    return err <= tol * rms, err, rms


GUARD = 4096                     # elements before and after a guarded buffer (16 KiB of float32)
SENTINEL = -12345.5


def guarded(shape, fill, dtype=torch.float32):
    """A device buffer of `shape` (a view) inside a larger allocation whose
    GUARD elements on either side hold SENTINEL: writes past the buffer show
    up in check_guards.  fill: the buffer's contents (NaN for outputs a call
    must write completely, so that an unwritten element shows up)."""
    n = int(np.prod(shape))
    full = torch.full((n + 2 * GUARD,), SENTINEL, dtype=dtype, device=DEV)
    view = full[GUARD:GUARD + n].view(*shape)
    if isinstance(fill, torch.Tensor):
        view.copy_(fill)
    else:
        view.fill_(fill)
    return full, view


def check_guards(full):
    g = full.cpu()
    assert torch.all(g[:GUARD] == SENTINEL) and torch.all(g[-GUARD:] == SENTINEL), "write outside the buffer"


def lse_abs_err(got, want):
    """lse is compared in absolute terms (nats): an error of e rescales the
    next loop's previous-loop probabilities by exp(e)."""
    return float(np.abs(np.asarray(got, np.float64) - np.asarray(want, np.float64)).max())


# --------------------------------------------------------------------------- select
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("n,hidden,k", [(1, 8, 1), (300, 64, 75), (4096, 2048, 820), (5000, 5280, 1500),
                                         (65536, 64, 6554)])
def test_select_tokens(dtype, n, hidden, k):
    rng = np.random.default_rng(n + hidden)
    h_prev = rng.standard_normal((n, hidden)).astype(np.float32)
    sig = np.exp(rng.standard_normal(n)).astype(np.float32) * 0.1
    h_cur = h_prev + sig[:, None] * rng.standard_normal((n, hidden)).astype(np.float32)
    h_cur[::7] = h_prev[::7]                                       # carried rows: score exactly 0
    if dtype == torch.bfloat16:
        h_prev, h_cur = bf16_round(h_prev), bf16_round(h_cur)
    hc, hp = to_dev(h_cur, dtype), to_dev(h_prev, dtype)
    scores = torch.empty(n, dtype=torch.float64, device=DEV)
    out = torch.empty(k, dtype=torch.int32, device=DEV)
    abi.select_tokens(hc, hp, k, scores, out)
    torch.cuda.synchronize()
    u = scores.cpu().numpy()
    u_ref = oracle.token_scores(h_cur, h_prev)
    np.testing.assert_allclose(u, u_ref, rtol=1e-13, atol=0)
    assert np.all(u[::7] == 0.0)
    got = out.cpu().numpy()
    assert np.array_equal(got, oracle.topk_ascending(u, k))        # same scores -> identical set
    assert np.array_equal(got, oracle.topk_ascending(u_ref, k))


@pytest.mark.parametrize("n,hidden,n_cand,n_still,ks", [
    (2000, 256, 300, 0, (1, 150, 300, 400)),       # 400 > candidates: zeros by index
    (2000, 256, 300, 100, (150, 200, 250, 300)),   # 100 candidates unchanged: k > 200 takes zeros by index
    (32768, 64, 9830, 0, (4915, 9830)),            # the 32K workload's later loops
    (65536, 16, 40000, 7, (20000, 39999))])
def test_select_tokens_candidates(n, hidden, n_cand, n_still, ks):
    """Later lazy loops: only the candidate rows may change, every other row
    scores exactly 0; the selection runs over the candidates while at least k
    of them score above 0, else over every row."""
    rng = np.random.default_rng(n + n_cand + n_still)
    h_prev = rng.standard_normal((n, hidden)).astype(np.float32)
    cand = np.sort(rng.choice(n, n_cand, replace=False)).astype(np.int32)
    h_cur = h_prev.copy()
    moved = cand[rng.permutation(n_cand)[n_still:]]
    h_cur[moved] += rng.standard_normal((len(moved), hidden)).astype(np.float32)
    scores = torch.full((n,), -1.0, dtype=torch.float64, device=DEV)
    u_ref = oracle.token_scores(h_cur, h_prev)
    for k in ks:
        out = torch.full((k,), -7, dtype=torch.int32, device=DEV)
        abi.select_tokens(to_dev(h_cur, torch.float32), to_dev(h_prev, torch.float32), k, scores, out,
                          torch.from_numpy(cand).to(DEV))
        torch.cuda.synchronize()
        np.testing.assert_allclose(scores.cpu().numpy(), u_ref, rtol=1e-13)
        assert np.array_equal(out.cpu().numpy(), oracle.topk_ascending(u_ref, k)), k


@pytest.mark.parametrize("n,k,cand_every", [(32768, 9831, 0), (32768, 4915, 3), (3000, 1500, 0), (3000, 700, 2),
                                             (1000, 999, 0)])
def test_select_tokens_low_word_ties(n, k, cand_every):
    """Token scores whose float64 high words all tie (1 + m 2^-22 + small
    terms, m < 4, share their top 20 mantissa bits): the selection must
    decide on the low words, and rows with equal scores go to the lower
    index.  h_prev = 0 and h_cur = (1 + m 2^-23, j 2^-24, 0, ...), so every
    score x^2 + y^2 is exact in float64 (49 significant bits) on both sides."""
    rng = np.random.default_rng(n + k + cand_every)
    hidden = 8
    h_prev = np.zeros((n, hidden), np.float32)
    h_cur = np.zeros((n, hidden), np.float32)
    m = rng.integers(0, 4, n)
    j = rng.integers(0, 40, n)                                     # repeats: exact ties
    h_cur[:, 0] = (1.0 + m * 2.0 ** -23).astype(np.float32)
    h_cur[:, 1] = (j * 2.0 ** -24).astype(np.float32)
    u_ref = oracle.token_scores(h_cur, h_prev)
    assert len(np.unique((u_ref.view(np.uint64) >> 32))) == 1      # one high word
    cand = None
    if cand_every:
        cand = np.arange(0, n, cand_every, dtype=np.int32)          # the other rows are carried: score 0
        keep = np.zeros(n, bool)
        keep[cand] = True
        h_cur[~keep] = h_prev[~keep]
        u_ref = oracle.token_scores(h_cur, h_prev)
    scores = torch.empty(n, dtype=torch.float64, device=DEV)
    out = torch.full((k,), -7, dtype=torch.int32, device=DEV)
    abi.select_tokens(to_dev(h_cur, torch.float32), to_dev(h_prev, torch.float32), k, scores, out,
                      None if cand is None else torch.from_numpy(cand).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(scores.cpu().numpy(), u_ref)              # one rounding each: identical
    assert np.array_equal(out.cpu().numpy(), oracle.topk_ascending(u_ref, k))


@pytest.mark.parametrize("n_seg,seg_len,k", [(1, 1, 1), (1, 256, 26), (16, 4096, 410), (3, 32768, 3277),
                                             (512, 8192, 820), (55, 16384, 1639), (2, 1000, 1000), (2, 700, 0),
                                             (1, 65536, 6554), (4, 65536, 1)])
def test_select_keys(n_seg, seg_len, k):
    rng = np.random.default_rng(seg_len + k)
    c = rng.random((n_seg, seg_len)).astype(np.float32) * 5
    c[:, ::5] = np.round(c[:, ::5])                                # exact ties
    c[:, ::11] = 0.0
    if seg_len > 3:
        c[:, 3] = -0.0
        c[:, 1] = -1.5                                             # negative mass after lazy updates
    out = torch.empty(n_seg, k, dtype=torch.int32, device=DEV)
    abi.select_keys(torch.from_numpy(c).to(DEV), k, out)
    torch.cuda.synchronize()
    want = oracle.select_keys(c, k) if k else np.zeros((n_seg, 0), np.int32)
    assert np.array_equal(out.cpu().numpy(), want)


@pytest.mark.parametrize("k", [1, 37, 500, 2047])
def test_select_keys_spread_exponents(k):
    """Values spread over many binades: the crossing bin is usually taken whole
    after one or two radix passes, which ends the selection early."""
    rng = np.random.default_rng(k)
    c = (rng.random((3, 2048)) + 1.0) * np.exp2(rng.integers(-60, 60, (3, 2048)))
    c[1] = -c[1]                                                   # all negative
    c = c.astype(np.float32)
    out = torch.empty(3, k, dtype=torch.int32, device=DEV)
    abi.select_keys(torch.from_numpy(c).to(DEV), k, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), oracle.select_keys(c, k))


def test_select_keys_all_equal():
    c = np.full((4, 3000), 0.25, np.float32)
    out = torch.empty(4, 100, dtype=torch.int32, device=DEV)
    abi.select_keys(torch.from_numpy(c).to(DEV), 100, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), np.tile(np.arange(100), (4, 1)))


# --------------------------------------------------------------------------- commit
def _oracle_chain(rng, n, H, d, sets, dtype_np_round):
    st = oracle.KVStore(n, H, d)
    inputs = {}
    k = dtype_np_round(rng.standard_normal((n, H, d)).astype(np.float32))
    v = dtype_np_round(rng.standard_normal((n, H, d)).astype(np.float32))
    inputs[1] = (k.copy(), v.copy())
    st.commit(1, np.arange(n), k, v)
    for l, act in sets.items():
        scale = 10.0 ** rng.uniform(-3, 0.5, (n, 1, 1))
        k = dtype_np_round(k + (scale * rng.standard_normal((n, H, d))).astype(np.float32))
        v = dtype_np_round(v + (scale * rng.standard_normal((n, H, d))).astype(np.float32))
        inputs[l] = (k.copy(), v.copy())
        st.commit(l, act, k[act], v[act])
    return st, inputs


@pytest.mark.parametrize("dtype,d", [(torch.float32, 64), (torch.bfloat16, 96), (torch.bfloat16, 128)])
def test_commit_codes_bit_exact(dtype, d):
    rng = np.random.default_rng(d)
    n, H = 300, 3
    sets = {2: np.arange(n), 3: np.sort(rng.choice(n, 90, replace=False)),
            4: np.sort(rng.choice(n, 40, replace=False))}
    rnd = bf16_round if dtype == torch.bfloat16 else (lambda x: x.astype(np.float32))
    st, inputs = _oracle_chain(rng, n, H, d, sets, rnd)
    kv = abi.KVStore(1, H, d, n, 4, dtype, [n, 90, 40], DEV)
    kv.arena.fill_(0xAB)
    for l in range(1, 5):
        act = np.arange(n) if l == 1 else sets[l]
        kk, vv = inputs[l]
        abi.kv_commit(kv, l, torch.from_numpy(act.astype(np.int32)).to(DEV), to_dev(kk[None], dtype),
                      to_dev(vv[None], dtype))
    torch.cuda.synchronize()
    base_k = kv.view("base_k").float().cpu().numpy()[0]              # [H, N, d]
    np.testing.assert_array_equal(base_k, inputs[1][0].transpose(1, 0, 2))
    for l in range(2, 5):
        slots = kv.view("slot_map", l).cpu().numpy()[0]
        want_slots = np.full(n, -1)
        want_slots[sets[l]] = np.arange(len(sets[l]))
        assert np.array_equal(slots, want_slots)
        for wi, w in enumerate(("k", "v")):
            rec = st.layers[l][w][0]
            codes = kv.view("codes", l).cpu().numpy()[0][:, :, wi]    # [cap, H, d/2]
            scales = kv.view("scales", l).cpu().numpy()[0][:, :, wi]  # [cap, H, d/32]
            assert np.array_equal(codes, oracle.pack_int4(rec.codes)), (l, w)
            assert np.array_equal(scales.view(np.uint16), rec.scales.view(np.uint16)), (l, w)


def test_commit_appends_to_layer_without_reset():
    rng = np.random.default_rng(11)
    n, H, d = 64, 1, 64
    kv = abi.KVStore(1, H, d, n, 2, torch.float32, [20], DEV)
    k1 = rng.standard_normal((1, n, H, d)).astype(np.float32)
    abi.kv_commit(kv, 1, torch.arange(n, dtype=torch.int32, device=DEV)[None], to_dev(k1, torch.float32),
                  to_dev(k1, torch.float32))
    k2 = k1 + 0.1 * rng.standard_normal(k1.shape).astype(np.float32)
    a = torch.tensor([[3, 9, 40]], dtype=torch.int32, device=DEV)
    b = torch.tensor([[63]], dtype=torch.int32, device=DEV)
    abi.kv_commit(kv, 2, a, to_dev(k2, torch.float32), to_dev(k2, torch.float32), slot_base=0, reset_map=True)
    abi.kv_commit(kv, 2, b, to_dev(k2, torch.float32), to_dev(k2, torch.float32), slot_base=3, reset_map=False)
    torch.cuda.synchronize()
    slots = kv.view("slot_map", 2).cpu().numpy()[0]
    want = np.full(n, -1)
    want[[3, 9, 40, 63]] = [0, 1, 2, 3]
    assert np.array_equal(slots, want)


# --------------------------------------------------------------------------- attend
def _setup_attend(rng, n, H, d, dtype, sets, nS=None):
    rnd = bf16_round if dtype == torch.bfloat16 else (lambda x: x.astype(np.float32))
    st, inputs = _oracle_chain(rng, n, H, d, sets, rnd)
    kv = abi.KVStore(1, H, d, n, 1 + len(sets), dtype, [len(sets[l]) for l in sorted(sets)], DEV)
    for l in range(1, 2 + len(sets)):
        act = np.arange(n) if l == 1 else sets[l]
        kk, vv = inputs[l]
        abi.kv_commit(kv, l, torch.from_numpy(act.astype(np.int32)).to(DEV), to_dev(kk[None], dtype),
                      to_dev(vv[None], dtype))
    return st, kv, rnd


@pytest.mark.parametrize("dtype,d,n", [(torch.float32, 64, 256), (torch.bfloat16, 128, 300),
                                       (torch.bfloat16, 96, 200), (torch.float32, 128, 129),
                                       (torch.bfloat16, 64, 1000), (torch.bfloat16, 128, 1333),
                                       (torch.bfloat16, 96, 777), (torch.bfloat16, 128, 63)])
def test_attend_full(dtype, d, n):
    rng = np.random.default_rng(n)
    H = 2
    sets = {2: np.arange(n)}
    st, kv, rnd = _setup_attend(rng, n, H, d, dtype, sets)
    q = rnd(rng.standard_normal((n, H, d)).astype(np.float32) * 1.5)
    for version in (1, 2):
        # outputs NaN-filled (a FULL call writes every o, lse and column-mass
        # entry) inside guard regions; the workspace too has guards
        og, o = guarded((1, n, H, d), float("nan"))
        lg, lse = guarded((1, n, H), float("nan"))
        cg, c = guarded((1, H, n), float("nan"))
        a = abi.attend_args(kv, abi.FL_ATTEND_FULL, version, to_dev(q[None], dtype), None, None, n, None, o, lse, c)
        wsg = torch.full((abi.attend_workspace_bytes(a) + 2 * 256,), 0x5A, dtype=torch.uint8, device=DEV)
        ws = wsg[256:-256]
        a = abi.attend_args(kv, abi.FL_ATTEND_FULL, version, to_dev(q[None], dtype), None, None, n, None, o, lse, c, ws)
        abi.attend(a)
        torch.cuda.synchronize()
        for g in (og, lg, cg):
            check_guards(g)
        assert torch.all(wsg[:256] == 0x5A) and torch.all(wsg[-256:] == 0x5A), "write outside the workspace"
        assert not (torch.isnan(o).any() or torch.isnan(lse).any() or torch.isnan(c).any()), "unwritten output"
        wd = "bf16" if dtype == torch.bfloat16 else "fp32"
        o_r, lse_r, c_r = oracle.full_attention(q, oracle.to_working_dtype(st.reconstruct("k", version), wd),
                                                oracle.to_working_dtype(st.reconstruct("v", version), wd),
                                                np.arange(n))
        for got, want in ((o[0], o_r), (c[0], c_r)):
            ok, err, rms = rel_err_ok(got.cpu().numpy(), want)
            assert ok, (version, err, rms)
        assert lse_abs_err(lse[0].cpu().numpy(), lse_r) <= 2e-2, version


@pytest.mark.parametrize("d,n,H", [(128, 2048, 8), (64, 1024, 16), (96, 1800, 8), (128, 2500, 12)])
def test_attend_full_key_split(d, n, H):
    """Full loops on grids of about one round (at least 8 heads, few row
    tiles) cut the heavy row tiles' keys into parts merged by the last part
    to finish: outputs within tolerance of the oracle, and identical from run
    to run whichever part finishes last."""
    rng = np.random.default_rng(1000 + n)
    dtype = torch.bfloat16
    st, kv, rnd = _setup_attend(rng, n, H, d, dtype, {})
    q = rnd(rng.standard_normal((n, H, d)).astype(np.float32) * 1.5)
    outs = []
    for rep in range(3):
        o = torch.zeros(1, n, H, d, device=DEV)
        lse = torch.zeros(1, n, H, device=DEV)
        c = torch.full((1, H, n), 7.0, device=DEV)
        a = abi.attend_args(kv, abi.FL_ATTEND_FULL, 1, to_dev(q[None], dtype), None, None, n, None, o, lse, c)
        ws = torch.full((abi.attend_workspace_bytes(a),), 0xA5, dtype=torch.uint8, device=DEV)
        a = abi.attend_args(kv, abi.FL_ATTEND_FULL, 1, to_dev(q[None], dtype), None, None, n, None, o, lse, c, ws)
        abi.attend(a)
        torch.cuda.synchronize()
        outs.append((o.cpu().numpy(), lse.cpu().numpy(), c.cpu().numpy()))
    o_r, lse_r, c_r = oracle.full_attention(q, oracle.to_working_dtype(st.reconstruct("k", 1), "bf16"),
                                            oracle.to_working_dtype(st.reconstruct("v", 1), "bf16"), np.arange(n))
    for got, want in zip((outs[0][0], outs[0][2]), (o_r[None], c_r[None])):
        ok, err, rms = rel_err_ok(got, want)
        assert ok, (err, rms)
    assert lse_abs_err(outs[0][1], lse_r[None]) <= 2e-2
    for rep in (1, 2):
        for x, y in zip(outs[0], outs[rep]):
            assert np.array_equal(x, y)


@pytest.mark.parametrize("dtype,n,H,d,version,subset,reset", [
    (torch.bfloat16, 700, 3, 128, 1, False, True),     # the base of every token (NULL active_idx)
    (torch.bfloat16, 700, 3, 128, 2, False, True),
    (torch.bfloat16, 700, 3, 64, 3, True, False),      # some rows, into a layer that already holds records
    (torch.bfloat16, 640, 2, 96, 3, True, True),
    (torch.float32, 300, 2, 64, 2, False, True),       # per-row path: the commit runs as its own kernel
])
def test_attend_full_fused_commit(dtype, n, H, d, version, subset, reset):
    """A FULL call with the commit fused writes the same store and gives the
    same o, lse and column mass, bit for bit, as commit-then-attend."""
    rng = np.random.default_rng(3000 + n + version)
    rnd = bf16_round if dtype == torch.bfloat16 else (lambda x: x.astype(np.float32))
    xs = {l: [rnd(rng.standard_normal((1, n, H, d)) * (1.0 + 0.1 * l)) for _ in range(2)] for l in (1, 2, 3)}
    q = rnd(rng.standard_normal((1, n, H, d)) * 1.5)
    rows = np.sort(rng.choice(n, size=n // 3, replace=False)) if subset else np.arange(n)
    early = None if reset else np.sort(rng.choice(np.setdiff1d(np.arange(n), rows), size=40, replace=False))
    dev_rows = torch.from_numpy(rows.astype(np.int32)).to(DEV)[None]
    outs = []
    for fuse in (False, True):
        kv = abi.KVStore(1, H, d, n, 3, dtype, [n, n], DEV)
        kv.arena.zero_()
        every = torch.arange(n, dtype=torch.int32, device=DEV)[None]
        for l in range(1, version):
            abi.kv_commit(kv, l, every, to_dev(xs[l][0], dtype), to_dev(xs[l][1], dtype))
        slot_base = 0
        if not reset:                                      # records of other tokens already in the layer
            abi.kv_commit(kv, version, torch.from_numpy(early.astype(np.int32)).to(DEV)[None],
                          to_dev(xs[version][0] * 0.5, dtype), to_dev(xs[version][1] * 0.5, dtype))
            slot_base = len(early)
        k_new, v_new = to_dev(xs[version][0], dtype), to_dev(xs[version][1], dtype)
        o = torch.zeros(1, n, H, d, device=DEV)
        lse = torch.zeros(1, n, H, device=DEV)
        c = torch.full((1, H, n), 7.0, device=DEV)
        act = dev_rows if subset else None
        commit = dict(k_new=k_new, v_new=v_new, slot_base=slot_base, reset=reset) if fuse else None
        if not fuse:
            abi.kv_commit(kv, version, dev_rows, k_new, v_new, slot_base=slot_base, reset_map=reset)
        a = abi.attend_args(kv, abi.FL_ATTEND_FULL, version, to_dev(q, dtype), None, act, len(rows), None, o, lse,
                            c, commit=commit)
        ws = torch.empty(max(abi.attend_workspace_bytes(a), 256), dtype=torch.uint8, device=DEV)
        a = abi.attend_args(kv, abi.FL_ATTEND_FULL, version, to_dev(q, dtype), None, act, len(rows), None, o, lse,
                            c, ws, commit=commit)
        abi.attend(a)
        torch.cuda.synchronize()
        outs.append((kv.arena.cpu(), o.cpu(), lse.cpu(), c.cpu()))
    for x, y, name in zip(outs[0], outs[1], ("arena", "o", "lse", "colmass")):
        assert torch.equal(x, y), name


def test_attend_full_fused_exit_flags():
    """A FULL call (paired row halves, per-block column-mass ranges, fused
    commit) over two sequences of which one has exited: the exited sequence's
    o, lse, column mass and store are left as they were, and the other's equal
    those of a call without flags, bit for bit."""
    rng = np.random.default_rng(4242)
    n, H, d, S = 2048, 16, 128, 2                         # 32 head rows x 8 row tiles: one round
    dtype = torch.bfloat16
    x1 = [bf16_round(rng.standard_normal((S, n, H, d))) for _ in range(2)]
    x2 = [bf16_round(rng.standard_normal((S, n, H, d)) * 1.1) for _ in range(2)]
    q = bf16_round(rng.standard_normal((S, n, H, d)) * 1.5)
    outs = []
    for flags in (None, [0, 1]):
        kv = abi.KVStore(S, H, d, n, 2, dtype, [n], DEV)
        kv.arena.zero_()
        every = torch.arange(n, dtype=torch.int32, device=DEV)[None].repeat(S, 1).contiguous()
        abi.kv_commit(kv, 1, every, to_dev(x1[0], dtype), to_dev(x1[1], dtype))
        o = torch.zeros(S, n, H, d, device=DEV)
        lse = torch.zeros(S, n, H, device=DEV)
        c = torch.full((S, H, n), 7.0, device=DEV)
        ef = None if flags is None else torch.tensor(flags, dtype=torch.int32, device=DEV)
        commit = dict(k_new=to_dev(x2[0], dtype), v_new=to_dev(x2[1], dtype))
        a = abi.attend_args(kv, abi.FL_ATTEND_FULL, 2, to_dev(q, dtype), None, None, n, None, o, lse, c,
                            commit=commit, exit_flags=ef)
        ws = torch.empty(abi.attend_workspace_bytes(a), dtype=torch.uint8, device=DEV)
        a = abi.attend_args(kv, abi.FL_ATTEND_FULL, 2, to_dev(q, dtype), None, None, n, None, o, lse, c, ws,
                            commit=commit, exit_flags=ef)
        abi.attend(a)
        torch.cuda.synchronize()
        outs.append((o.cpu(), lse.cpu(), c.cpu(), kv.view("slot_map", 2).cpu(), kv.view("codes", 2).cpu(),
                     kv.view("scales", 2).cpu()))
    ref, got = outs
    for x, y, name in zip(ref[:3], got[:3], ("o", "lse", "colmass")):
        assert torch.equal(x[0], y[0]), name
    assert torch.all(got[0][1] == 0) and torch.all(got[1][1] == 0) and torch.all(got[2][1] == 7.0)
    for x, y, name in zip(ref[3:], got[3:], ("slots", "codes", "scales")):
        assert torch.equal(x[0], y[0]), name
        assert torch.all(y[1] == 0), name                 # never written for the exited sequence


@pytest.mark.parametrize("d,n,H", [(64, 2048, 32), (128, 1900, 32), (128, 4000, 16)])
def test_attend_full_paired_halves(d, n, H):
    """Full loops whose grid is one round of workgroups: each workgroup takes
    an early and a late 128-row half (the second case has an odd number of
    halves, so one workgroup per head has only the early one; the third ends
    in a ragged half), and each wave stops at its own rows' last key tile."""
    rng = np.random.default_rng(2000 + n)
    dtype = torch.bfloat16
    st, kv, rnd = _setup_attend(rng, n, H, d, dtype, {})
    q = rnd(rng.standard_normal((n, H, d)).astype(np.float32) * 1.5)
    o = torch.zeros(1, n, H, d, device=DEV)
    lse = torch.zeros(1, n, H, device=DEV)
    c = torch.full((1, H, n), 7.0, device=DEV)
    a = abi.attend_args(kv, abi.FL_ATTEND_FULL, 1, to_dev(q[None], dtype), None, None, n, None, o, lse, c)
    ws = torch.full((abi.attend_workspace_bytes(a),), 0xA5, dtype=torch.uint8, device=DEV)
    a = abi.attend_args(kv, abi.FL_ATTEND_FULL, 1, to_dev(q[None], dtype), None, None, n, None, o, lse, c, ws)
    abi.attend(a)
    torch.cuda.synchronize()
    o_r, lse_r, c_r = oracle.full_attention(q, oracle.to_working_dtype(st.reconstruct("k", 1), "bf16"),
                                            oracle.to_working_dtype(st.reconstruct("v", 1), "bf16"), np.arange(n))
    for got, want in ((o[0], o_r), (c[0], c_r)):
        ok, err, rms = rel_err_ok(got.cpu().numpy(), want)
        assert ok, (err, rms)
    assert lse_abs_err(lse[0].cpu().numpy(), lse_r) <= 2e-2


@pytest.mark.parametrize("dtype,d,n,na,ns", [(torch.float32, 64, 256, 64, 26), (torch.bfloat16, 128, 512, 103, 52),
                                             (torch.bfloat16, 96, 300, 300, 300), (torch.bfloat16, 128, 700, 1, 70),
                                             (torch.bfloat16, 128, 2000, 600, 200), (torch.bfloat16, 64, 1500, 1500, 150),
                                             (torch.bfloat16, 96, 900, 65, 900), (torch.bfloat16, 128, 3000, 64, 1)])
def test_attend_lazy(dtype, d, n, na, ns):
    rng = np.random.default_rng(n + na)
    H = 3
    act = np.sort(rng.choice(n, na, replace=False)).astype(np.int32)
    sets = {2: act}
    st, kv, rnd = _setup_attend(rng, n, H, d, dtype, sets)
    q0 = rnd(rng.standard_normal((n, H, d)).astype(np.float32))
    q1 = rnd(q0 + 0.3 * rng.standard_normal((n, H, d)).astype(np.float32))
    wd = "bf16" if dtype == torch.bfloat16 else "fp32"
    rec = lambda w, l: oracle.to_working_dtype(st.reconstruct(w, l), wd)
    o0, lse0, c0 = oracle.full_attention(q0, rec("k", 1), rec("v", 1), np.arange(n))
    keys = oracle.select_keys(c0, ns)
    og, o = guarded((1, n, H, d), torch.from_numpy(o0.astype(np.float32)[None]))
    lg, lse = guarded((1, n, H), torch.from_numpy(lse0.astype(np.float32)[None]))
    cg, c = guarded((1, H, n), torch.from_numpy(c0.astype(np.float32)[None]))
    qc = to_dev(q1[act][None], dtype)
    qp = to_dev(q0[act][None], dtype)
    a = abi.attend_args(kv, abi.FL_ATTEND_LAZY, 2, qc, qp, torch.from_numpy(act).to(DEV)[None], na,
                        torch.from_numpy(keys).to(DEV)[None], o, lse, c, None, q_compact=True)
    ws = torch.empty(abi.attend_workspace_bytes(a), dtype=torch.uint8, device=DEV)
    a = abi.attend_args(kv, abi.FL_ATTEND_LAZY, 2, qc, qp, torch.from_numpy(act).to(DEV)[None], na,
                        torch.from_numpy(keys).to(DEV)[None], o, lse, c, ws, q_compact=True)
    abi.attend(a)
    torch.cuda.synchronize()
    for g in (og, lg, cg):
        check_guards(g)
    o_r, lse_r, c_r, m, upd = oracle.lazy_attention(
        q1[act], q0[act], rec("k", 1), rec("v", 1), rec("k", 2), rec("v", 2), o0[act], lse0[act], c0, act, keys)
    got_o = o[0].cpu().numpy()
    ok, err, rms = rel_err_ok(got_o[act], o_r)
    assert ok, ("o", err, rms)
    inactive = np.setdiff1d(np.arange(n), act)
    assert np.array_equal(got_o[inactive], o0.astype(np.float32)[inactive])      # untouched
    err = float(np.abs(lse[0].cpu().numpy()[act].astype(np.float64) - lse_r).max())
    assert err <= 2e-2, ("lse max abs error", err)
    ok, err, rms = rel_err_ok(c[0].cpu().numpy(), c_r)
    assert ok, ("colmass", err, rms)
