"""GPU parity of decode-shaped lazy attention (one active row per sequence,
read straight from the base + delta chain) against the CPU oracle.

Covers every delta depth of the decode kernel (versions 2..5), both scale
groups and both code widths (4 and 2 bits), rows in the middle of the sequence (keys after the row are not
visible), a row that sees no selected key, the fused commit with and without
reset, key counts on both sides of the kernel's LDS staging limit (1536
keys), and the full loop over the base on both sides of its LDS limit.  Bars: codes and slot tables bit-exact; o, lse, column mass within
2e-2 x RMS; the fused commit bit-identical to commit-then-attend.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from sparse_loop_attention_amd import abi
from sparse_loop_attention_amd.synth import round_bf16

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF = torch.bfloat16


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(DEV).to(BF)


def _close(got, want, what):
    want = np.asarray(want, np.float64)
    rms = math.sqrt(float(np.mean(want ** 2)))
    err = float(np.abs(np.asarray(got, np.float64) - want).max())
    assert err <= 2e-2 * rms, f"{what}: max err {err:.3e} > 2e-2 * RMS {rms:.3e}"


def _build(rng, S, n, H, d, versions, group, sizes, caps=None, bits=4):
    """S sequences, each an oracle store and the same records in one GPU
    store; layer l holds `sizes[l]` random tokens per sequence (slots
    0..sizes[l]-1 of caps[l])."""
    caps = caps or sizes
    sts, kin, vin = [], {l: [] for l in range(1, versions + 1)}, {l: [] for l in range(1, versions + 1)}
    acts = {l: [] for l in range(2, versions + 1)}
    for _ in range(S):
        st = oracle.KVStore(n, H, d, group=group, bits=bits)
        k = round_bf16(rng.standard_normal((n, H, d)).astype(np.float32))
        v = round_bf16(rng.standard_normal((n, H, d)).astype(np.float32))
        st.commit(1, np.arange(n), k, v)
        kin[1].append(k.copy()); vin[1].append(v.copy())
        for l in range(2, versions + 1):
            act = np.sort(rng.choice(n, sizes[l], replace=False)).astype(np.int32)
            scale = 10.0 ** rng.uniform(-3, 0.5, (n, 1, 1))
            k = round_bf16(k + (scale * rng.standard_normal((n, H, d))).astype(np.float32))
            v = round_bf16(v + (scale * rng.standard_normal((n, H, d))).astype(np.float32))
            st.commit(l, act, k[act], v[act])
            kin[l].append(k.copy()); vin[l].append(v.copy()); acts[l].append(act)
        sts.append(st)
    kv = abi.KVStore(S, H, d, n, versions, BF, [caps[l] for l in range(2, versions + 1)], DEV, group=group,
                     delta_bits=bits)
    abi.kv_commit(kv, 1, torch.arange(n, dtype=torch.int32, device=DEV).repeat(S, 1),
                  _dev(np.stack(kin[1])), _dev(np.stack(vin[1])))
    for l in range(2, versions + 1):
        abi.kv_commit(kv, l, torch.from_numpy(np.stack(acts[l])).to(DEV), _dev(np.stack(kin[l])),
                      _dev(np.stack(vin[l])))
    return sts, kv


def _rec(st, w, l):
    return oracle.to_working_dtype(st.reconstruct(w, l), "bf16")


def _row_state(rng, sts, rows, version, keys, H, d):
    """Queries of the rows and their previous-loop state (full attention at
    version - 1), per sequence."""
    n = sts[0].n
    out = []
    for s, st in enumerate(sts):
        i = rows[s]
        q0 = round_bf16(rng.standard_normal((1, H, d)).astype(np.float32))
        q1 = round_bf16(q0 + 0.3 * rng.standard_normal((1, H, d)).astype(np.float32))
        o0, lse0, c0 = oracle.full_attention(q0, _rec(st, "k", version - 1), _rec(st, "v", version - 1),
                                             np.array([i]))
        c0 = c0 + rng.uniform(0, 0.5, (H, n))                 # mass of earlier rows of the sequence
        out.append((q0, q1, o0, lse0, c0))
    return out


def _gpu_inputs(state, rows, keys):
    q0 = np.stack([x[0] for x in state])                      # [S, 1, H, d]
    q1 = np.stack([x[1] for x in state])
    o = torch.from_numpy(np.stack([x[2] for x in state]).astype(np.float32)).to(DEV)
    lse = torch.from_numpy(np.stack([x[3] for x in state]).astype(np.float32)).to(DEV)
    c = torch.from_numpy(np.stack([x[4] for x in state]).astype(np.float32)).to(DEV)
    act = torch.tensor(np.asarray(rows, np.int32)[:, None], device=DEV)
    kt = torch.from_numpy(np.ascontiguousarray(keys, np.int32)).to(DEV)
    return _dev(q1), _dev(q0), act, kt, o, lse, c


def _attend(kv, version, q1, q0, act, kt, o, lse, c, commit=None):
    a = abi.attend_args(kv, abi.FL_ATTEND_LAZY, version, q1, q0, act, 1, kt, o, lse, c, None,
                        q_compact=True, o_compact=True, commit=commit)
    ws = torch.empty(max(256, abi.attend_workspace_bytes(a)), dtype=torch.uint8, device=DEV)
    a = abi.attend_args(kv, abi.FL_ATTEND_LAZY, version, q1, q0, act, 1, kt, o, lse, c, ws,
                        q_compact=True, o_compact=True, commit=commit)
    abi.attend(a)
    torch.cuda.synchronize()


def _keys(rng, S, H, n, nk, rows, force=None):
    out = np.zeros((S, H, nk), np.int32)
    for s in range(S):
        for h in range(H):
            pick = rng.choice(n, nk, replace=False)
            if force is not None and h == 0:
                pick[0] = force[s]                            # the row itself among the keys
                pick = np.unique(pick)
                while len(pick) < nk:
                    pick = np.unique(np.append(pick, rng.integers(0, n)))
            out[s, h] = np.sort(pick)
    return out


def _check_against_oracle(sts, state, rows, keys, version, o, lse, c):
    for s, st in enumerate(sts):
        q0, q1, o0, lse0, c0 = state[s]
        o_r, lse_r, c_r, _, _ = oracle.lazy_attention(
            q1, q0, _rec(st, "k", version - 1), _rec(st, "v", version - 1), _rec(st, "k", version),
            _rec(st, "v", version), o0, lse0, c0, np.array([rows[s]]), keys[s])
        _close(o[s].cpu().numpy(), o_r, f"seq {s} o")
        err = float(np.abs(lse[s].cpu().numpy().astype(np.float64) - lse_r).max())
        assert err <= 2e-2, f"seq {s} lse: max abs err {err:.3e}"
        _close(c[s].cpu().numpy(), c_r, f"seq {s} colmass")


@pytest.mark.parametrize("version,group,bits", [(2, 32, 4), (3, 32, 4), (4, 32, 4), (5, 32, 4), (3, 64, 4),
                                                (5, 64, 4), (2, 32, 2), (4, 32, 2), (5, 64, 2)])
def test_decode_depths_and_groups(version, group, bits):
    rng = np.random.default_rng(100 * version + group + bits)
    S, n, H, d, nk = 3, 640, 2, 128, 64
    sizes = {l: [n, 300, 150, 40][l - 2] for l in range(2, version + 1)}
    sts, kv = _build(rng, S, n, H, d, version, group, sizes, bits=bits)
    rows = [n - 1, 333, 17]                                   # the last token, the middle, near the start
    keys = _keys(rng, S, H, n, nk, rows, force=rows)
    state = _row_state(rng, sts, rows, version, keys, H, d)
    q1, q0, act, kt, o, lse, c = _gpu_inputs(state, rows, keys)
    _attend(kv, version, q1, q0, act, kt, o, lse, c)
    _check_against_oracle(sts, state, rows, keys, version, o, lse, c)


def test_decode_row_with_no_visible_key():
    rng = np.random.default_rng(5)
    S, n, H, d, nk = 2, 400, 2, 128, 40
    sts, kv = _build(rng, S, n, H, d, 3, 32, {2: 200, 3: 100})
    rows = [3, n - 1]                                         # sequence 0: every selected key is after row 3
    keys = np.stack([np.stack([np.sort(rng.choice(np.arange(10, n), nk, replace=False)) for _ in range(H)]),
                     _keys(rng, 1, H, n, nk, rows[1:])[0]]).astype(np.int32)
    state = _row_state(rng, sts, rows, 3, keys, H, d)
    q1, q0, act, kt, o, lse, c = _gpu_inputs(state, rows, keys)
    o_in, lse_in, c_in = o.clone(), lse.clone(), c.clone()
    _attend(kv, 3, q1, q0, act, kt, o, lse, c)
    assert torch.equal(o[0], o_in[0]) and torch.equal(lse[0], lse_in[0]) and torch.equal(c[0], c_in[0])
    _check_against_oracle(sts[1:], state[1:], rows[1:], keys[1:], 3, o[1:], lse[1:], c[1:])


@pytest.mark.parametrize("nk", [1536, 1537])
def test_decode_key_count_at_staging_limit(nk):
    rng = np.random.default_rng(nk)
    S, n, H, d = 2, 3000, 2, 128
    sts, kv = _build(rng, S, n, H, d, 3, 32, {2: 900, 3: 300})
    rows = [n - 1, 2100]
    keys = _keys(rng, S, H, n, nk, rows)
    state = _row_state(rng, sts, rows, 3, keys, H, d)
    q1, q0, act, kt, o, lse, c = _gpu_inputs(state, rows, keys)
    _attend(kv, 3, q1, q0, act, kt, o, lse, c)
    _check_against_oracle(sts, state, rows, keys, 3, o, lse, c)


def _arena_parts(kv, versions):
    out = {"base_k": kv.view("base_k").cpu(), "base_v": kv.view("base_v").cpu()}
    for l in range(2, versions + 1):
        out[f"slots{l}"] = kv.view("slot_map", l).cpu()
        out[f"codes{l}"] = kv.view("codes", l).cpu()
        out[f"scales{l}"] = kv.view("scales", l).cpu()
    return out


@pytest.mark.parametrize("reset", [False, True])
def test_decode_fused_commit_equals_commit_then_attend(reset):
    """The new token's records (slot 0 of layer v: reset; the slot after the
    context's: append) written inside the attention call give the same store
    and outputs, bit for bit, as a commit followed by attend; the token is
    among its own keys in head 0."""
    S, n, H, d, version, nk = 2, 500, 3, 128, 3, 50
    res = []
    for fuse in (False, True):
        rng = np.random.default_rng(77)
        ctx = {2: 200, 3: 120}
        sts, kv = _build(rng, S, n, H, d, version, 32, ctx, caps={2: 200, 3: 121})
        rows = [n - 1, 250]
        keys = _keys(rng, S, H, n, nk, rows, force=rows)
        state = _row_state(rng, sts, rows, version, keys, H, d)
        q1, q0, act, kt, o, lse, c = _gpu_inputs(state, rows, keys)
        k_new = _dev(round_bf16(rng.standard_normal((S, 1, H, d)).astype(np.float32)))
        v_new = _dev(round_bf16(rng.standard_normal((S, 1, H, d)).astype(np.float32)))
        slot = 0 if reset else ctx[version]                 # after the context's records
        if fuse:
            _attend(kv, version, q1, q0, act, kt, o, lse, c,
                    commit=dict(k_new=k_new, v_new=v_new, compact=True, slot_base=slot, reset=reset))
        else:
            abi.kv_commit(kv, version, act, k_new, v_new, slot_base=slot, reset_map=reset, compact=True)
            _attend(kv, version, q1, q0, act, kt, o, lse, c)
        res.append((o.cpu(), lse.cpu(), c.cpu(), _arena_parts(kv, version)))
    (oa, la, ca, aa), (ob, lb, cb, ab) = res
    for k in aa:
        assert torch.equal(aa[k], ab[k]), k
    assert torch.equal(oa, ob) and torch.equal(la, lb) and torch.equal(ca, cb)


@pytest.mark.parametrize("n", [700, 10240, 10241])
def test_decode_full_loop(n):
    """Full loop over the base (version 1) for one row per sequence: the last
    token, a middle row and the first token; N on both sides of the limit of
    logits kept in LDS (10240)."""
    rng = np.random.default_rng(n)
    S, H, d = 3, 2, 128
    sts, kv = _build(rng, S, n, H, d, 1, 32, {})
    rows = [n - 1, n // 3, 0]
    q = np.stack([round_bf16(rng.standard_normal((1, H, d)).astype(np.float32) * 1.5) for _ in range(S)])
    o = torch.zeros(S, 1, H, d, device=DEV)
    lse = torch.zeros(S, 1, H, device=DEV)
    c = torch.full((S, H, n), 7.0, device=DEV)
    act = torch.tensor(np.asarray(rows, np.int32)[:, None], device=DEV)
    a = abi.attend_args(kv, abi.FL_ATTEND_FULL, 1, _dev(q), None, act, 1, None, o, lse, c, None,
                        q_compact=True, o_compact=True)
    ws = torch.empty(max(256, abi.attend_workspace_bytes(a)), dtype=torch.uint8, device=DEV)
    a = abi.attend_args(kv, abi.FL_ATTEND_FULL, 1, _dev(q), None, act, 1, None, o, lse, c, ws,
                        q_compact=True, o_compact=True)
    abi.attend(a)
    torch.cuda.synchronize()
    for s, st in enumerate(sts):
        o_r, lse_r, c_r = oracle.full_attention(q[s], _rec(st, "k", 1), _rec(st, "v", 1), np.array([rows[s]]))
        _close(o[s].cpu().numpy(), o_r, f"seq {s} o")
        err = float(np.abs(lse[s].cpu().numpy().astype(np.float64) - lse_r).max())
        assert err <= 2e-2, f"seq {s} lse: max abs err {err:.3e}"
        _close(c[s].cpu().numpy(), c_r, f"seq {s} colmass")
        assert torch.all(c[s][:, rows[s] + 1:] == 0)           # nothing past the row


@pytest.mark.parametrize("S", [8, 10])
def test_decode_many_sequences(S):
    """From 8 sequences on, the heads of a sequence share an XCD; a count
    that is not a multiple of 8 leaves workgroups with no sequence."""
    rng = np.random.default_rng(S)
    n, H, d, nk, version = 500, 3, 128, 50, 4
    sts, kv = _build(rng, S, n, H, d, version, 32, {2: n, 3: 100, 4: 60})
    rows = [int(x) for x in rng.integers(0, n, S)]
    rows[0] = n - 1
    keys = _keys(rng, S, H, n, nk, rows, force=rows)
    state = _row_state(rng, sts, rows, version, keys, H, d)
    q1, q0, act, kt, o, lse, c = _gpu_inputs(state, rows, keys)
    _attend(kv, version, q1, q0, act, kt, o, lse, c)
    _check_against_oracle(sts, state, rows, keys, version, o, lse, c)
