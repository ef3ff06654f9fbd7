"""Pins for the oracle's int4 delta codec and base+delta chain (CPU only).

Page "FlashLoop: Fast and Memory-Efficient Looped Transformers via Lazy
Updates", section "FlashLoop combines three kinds of savings", paragraph 3:
the KV cache is a base plus low-bit corrections, written only for active
tokens, 4 bits in the main setting.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import (KVStore, dequantize_groups, f16_rne, pack_int4, quantize_groups,
                    unpack_int4)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "int4_group_examples.json")


def _all_finite_halves():
    """Every finite binary16 value as an exact Fraction, decoded from its bits."""
    out = []
    for bits in range(0x7C00):                     # positive finite halves
        e, m = bits >> 10, bits & 0x3FF
        if e == 0:
            v = Fraction(m, 1 << 24)
        else:
            v = Fraction(1024 + m, 1 << 10) * (Fraction(2) ** (e - 15))
        out.append((v, bits))
    return out


def test_f16_rne_against_exhaustive_table():
    halves = _all_finite_halves()
    vals = [v for v, _ in halves]
    import bisect
    rng = np.random.default_rng(0)
    xs = np.concatenate([
        (rng.random(3000) * 2.0 ** rng.integers(-26, 16, 3000)).astype(np.float32),
        np.array([v for v, _ in halves[::97]], dtype=np.float64).astype(np.float32),
        # exact midpoints between neighbouring halves (ties -> even mantissa)
        np.array([float((halves[i][0] + halves[i + 1][0]) / 2) for i in range(0, 0x7BFF, 131)],
                 np.float32),
    ])
    got = f16_rne(xs).view(np.uint16)
    for x, g in zip(xs, got):
        fx = Fraction(float(x))
        if fx > vals[-1] + (vals[-1] - vals[-2]) / 2:
            continue                               # overflow range, not used by the codec
        j = bisect.bisect_left(vals, fx)
        cands = [c for c in (j - 1, j) if 0 <= c < len(vals)]
        best = min(cands, key=lambda c: (abs(vals[c] - fx), halves[c][1] & 1))
        assert int(g) == halves[best][1], (float(x), hex(int(g)), hex(halves[best][1]))


def _golden_cases():
    with open(GOLDEN) as f:
        data = json.load(f)
    return data["group"], data["cases"]


@pytest.mark.parametrize("case", _golden_cases()[1], ids=lambda c: c["name"])
def test_golden_int4_examples(case):
    group = _golden_cases()[0]
    delta = np.zeros(group, np.float32)
    for i, s in enumerate(case["delta"]):
        delta[i] = np.float32(s)
    codes, scales = quantize_groups(delta[None], group)
    assert int(scales.view(np.uint16)[0, 0]) == int(case["scale_bits"], 16)
    want = np.zeros(group, np.int8)
    want[:len(case["codes"])] = case["codes"]
    assert codes[0].tolist() == want.tolist()
    packed = np.zeros(group // 2, np.uint8)
    hexes = case["packed"].split()
    packed[:len(hexes)] = [int(h, 16) for h in hexes]
    assert pack_int4(codes[0]).tolist() == packed.tolist()
    assert unpack_int4(packed).tolist() == want.tolist()


def test_lattice_round_trip_is_exact():
    rng = np.random.default_rng(5)
    for _ in range(200):
        s = np.float16(rng.random() * 2.0 ** rng.integers(-14, 8))
        if s == 0:
            continue
        codes = rng.integers(-7, 8, 32)
        codes[rng.integers(0, 32)] = rng.choice([-7, 7])        # absmax = 7 s
        delta = (codes.astype(np.float32) * np.float32(s)).astype(np.float32)
        c, sc = quantize_groups(delta[None])
        assert sc[0, 0] == s
        assert c[0].tolist() == codes.tolist()
        assert np.array_equal(dequantize_groups(c, sc)[0], delta)


def test_odd_symmetry_and_error_bound():
    rng = np.random.default_rng(6)
    delta = (rng.standard_normal((500, 4, 96)) * 10.0 ** rng.uniform(-4, 2, (500, 4, 1))).astype(np.float32)
    c, s = quantize_groups(delta)
    cn, sn = quantize_groups(-delta)
    assert np.array_equal(cn, -c) and np.array_equal(sn, s)
    assert c.min() >= -7 and c.max() <= 7
    deq = dequantize_groups(c, s)
    g = delta.reshape(500, 4, 3, 32)
    a = np.abs(g).max(-1)
    sf = s.astype(np.float64)
    bound = sf / 2 + np.maximum(0.0, a - 7 * sf) + 1e-6 * a
    err = np.abs(g - deq.reshape(500, 4, 3, 32)).max(-1)
    assert np.all(err <= bound)
    # the scale is the nearest half to absmax/7
    assert np.all(np.abs(sf - a / 7.0) <= np.maximum(2.0 ** -25, np.abs(a / 7.0) * 2.0 ** -11) + 1e-12)


def test_pack_nibble_order():
    codes = np.array([1, -1, 7, -7, 0, -8 + 1, 3, 4], np.int8)
    p = pack_int4(codes)
    assert p.tolist() == [0xF1, 0x97, 0x90, 0x43]
    assert unpack_int4(p).tolist() == codes.tolist()


def test_chain_lattice_deltas_reconstruct_exactly():
    """Deltas chosen on the int4 lattice make every version exact (reading of
    'a base plus a sequence of corrections'); inactive tokens carry."""
    rng = np.random.default_rng(7)
    n, H, d = 12, 2, 64
    st = KVStore(n, H, d)
    k1 = rng.standard_normal((n, H, d)).astype(np.float32)
    v1 = rng.standard_normal((n, H, d)).astype(np.float32)
    st.commit(1, np.arange(n), k1, v1)
    truth = {"k": k1.copy(), "v": v1.copy()}
    history = {1: {"k": k1.copy(), "v": v1.copy()}}
    for l, act in ((2, np.arange(n)), (3, np.array([1, 4, 5, 9])), (4, np.array([4, 9]))):
        new = {}
        for w in ("k", "v"):
            s = np.float16(2.0 ** rng.integers(-6, 0))
            codes = rng.integers(-7, 8, (act.size, H, d))
            codes[..., 0] = 7
            codes[..., 32] = -7
            new[w] = truth[w][act] + codes.astype(np.float32) * np.float32(s)
        st.commit(l, act, new["k"], new["v"])
        for w in ("k", "v"):
            truth[w][act] = new[w]
        history[l] = {w: truth[w].copy() for w in ("k", "v")}
    for l in range(1, 5):
        for w in ("k", "v"):
            assert np.array_equal(st.reconstruct(w, l), history[l][w]), (l, w)
    # token 0 is inactive after loop 2: versions 2..4 agree
    assert np.array_equal(st.reconstruct("k", 4)[0], st.reconstruct("k", 2)[0])
    assert np.array_equal(st.reconstruct("k", 3, np.array([4, 0])), history[3]["k"][[4, 0]])


def test_chain_delta_is_against_previous_reconstruction():
    rng = np.random.default_rng(8)
    n, H, d = 6, 1, 32
    st = KVStore(n, H, d)
    k1 = rng.standard_normal((n, H, d)).astype(np.float32)
    st.commit(1, np.arange(n), k1, k1)
    k2 = k1 + rng.standard_normal((n, H, d)).astype(np.float32)
    st.commit(2, np.arange(n), k2, k2)
    rec2 = st.reconstruct("k", 2)
    k3 = k2 + 0.01 * rng.standard_normal((n, H, d)).astype(np.float32)
    recs = st.commit(3, np.arange(n), k3, k3)
    # closed loop: the layer-3 codes quantise k3 - khat2, not k3 - k2
    c, s = quantize_groups(k3 - rec2)
    assert np.array_equal(recs["k"].codes, c) and np.array_equal(recs["k"].scales, s)
    err3 = np.abs(st.reconstruct("k", 3) - k3).max()
    assert err3 <= np.abs(k3 - rec2).max() / 7 / 2 * 1.01 + 1e-7


def test_working_dtype_rounding_matches_torch_bfloat16():
    """Reading R9: attention operands are the reconstruction rounded to bf16;
    pinned to torch's float32 -> bfloat16 conversion (nearest-even)."""
    import torch
    from oracle import to_working_dtype
    rng = np.random.default_rng(9)
    x = (rng.standard_normal(200000) * 10.0 ** rng.uniform(-30, 30, 200000)).astype(np.float32)
    # exact bf16 half-way cases: low 16 bits == 0x8000, both parities of the kept bit
    mid = (rng.integers(0, 2 ** 31, 2000, dtype=np.uint32) & np.uint32(0x7F7F0000)) | np.uint32(0x8000)
    x = np.concatenate([x, mid.view(np.float32), np.array([0.0, -0.0, 1.0, -3.5], np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = to_working_dtype(x, "bf16")
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    assert to_working_dtype(x, "fp32") is not None and np.array_equal(to_working_dtype(x, "fp32"), x)


# ---------------------------------------------------------------- lower-bit deltas and larger groups
@pytest.mark.parametrize("bits,group", [(2, 32), (2, 64), (4, 64)])
def test_lattice_round_trip_other_formats(bits, group):
    """delta = s * integers in [-q, q] with absmax = q*s (s a float16 value)
    round-trips exactly, for q = 2^(bits-1) - 1."""
    from oracle import quantize_groups, dequantize_groups
    rng = np.random.default_rng(31)
    q = (1 << (bits - 1)) - 1
    n, d = 40, 128
    s = np.float16(rng.uniform(0.01, 4.0, (n, d // group))).astype(np.float32)
    ints = rng.integers(-q, q + 1, (n, d // group, group))
    ints[..., 0] = q                                    # absmax = q*s in every group
    delta = (ints * s[..., None]).astype(np.float32).reshape(n, d)
    codes, scales = quantize_groups(delta, group, bits)
    assert np.array_equal(scales.astype(np.float32), s)
    assert np.array_equal(codes.reshape(n, d // group, group), ints)
    assert np.array_equal(dequantize_groups(codes, scales, group), delta)


@pytest.mark.parametrize("bits,group", [(2, 32), (2, 64), (4, 64)])
def test_error_bound_and_symmetry_other_formats(bits, group):
    """|delta - deq| <= s/2 + |absmax - q*s| per element, codes odd-symmetric,
    a zero group gives s = 0 and zero codes."""
    from oracle import quantize_groups, dequantize_groups
    rng = np.random.default_rng(32)
    q = (1 << (bits - 1)) - 1
    delta = (rng.standard_normal((64, 128)) * np.exp(rng.standard_normal((64, 1)))).astype(np.float32)
    delta[3, :group] = 0.0
    codes, scales = quantize_groups(delta, group, bits)
    assert codes.min() >= -q and codes.max() <= q
    deq = dequantize_groups(codes, scales, group)
    g = delta.reshape(64, -1, group)
    s = scales.astype(np.float32)
    bound = s / 2 + np.abs(np.abs(g).max(-1) - q * s)
    err = np.abs(g - deq.reshape(64, -1, group)).max(-1)
    assert np.all(err <= bound * (1 + 1e-6) + 1e-30)
    neg, _ = quantize_groups(-delta, group, bits)
    assert np.array_equal(neg, -codes)
    assert scales[3, 0] == 0 and not codes[3, :group].any()


def test_two_bit_packing():
    """2-bit fields: lowest bits = first element; -1 is binary 11."""
    from oracle import pack_codes, unpack_codes
    codes = np.array([[1, -1, 0, 1, -1, -1, 0, 0]], np.int8)
    packed = pack_codes(codes, 2)
    # byte 0: e0=01, e1=11, e2=00, e3=01 -> 0b01_00_11_01; byte 1: 11, 11, 00, 00 -> 0b00_00_11_11
    assert packed.tolist() == [[0b01001101, 0b00001111]]
    assert np.array_equal(unpack_codes(packed, 2), codes)
    rng = np.random.default_rng(33)
    c = rng.integers(-1, 2, (5, 128)).astype(np.int8)
    assert np.array_equal(unpack_codes(pack_codes(c, 2), 2), c)
    c4 = rng.integers(-7, 8, (5, 128)).astype(np.int8)
    assert np.array_equal(unpack_codes(pack_codes(c4, 4), 4), c4)


def test_store_with_two_bit_layers_reconstructs_lattice_chain():
    """A chain of lattice deltas reconstructs exactly at every version with
    2-bit codes and 64-element groups too."""
    from oracle import KVStore
    rng = np.random.default_rng(34)
    n, H, d = 16, 2, 128
    st = KVStore(n, H, d, group=64, bits=2)
    base = rng.standard_normal((n, H, d)).astype(np.float32)
    st.commit(1, np.arange(n), base, base)
    x = base.copy()
    for l in (2, 3):
        idx = np.sort(rng.choice(n, 6, replace=False))
        s = np.float16(rng.uniform(0.05, 0.5, (6, H, d // 64))).astype(np.float32)
        ints = rng.integers(-1, 2, (6, H, d // 64, 64))
        ints[..., 0] = 1
        step = (ints * s[..., None]).reshape(6, H, d).astype(np.float32)
        new = (x[idx] + step).astype(np.float32)
        # representable exactly: the delta against the reconstruction is the lattice step
        st.commit(l, idx, new, new)
        x[idx] = new
        assert np.array_equal(st.reconstruct("k", l), x)


LOWBIT_GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "lowbit_group_examples.json")


def _lowbit_cases():
    with open(LOWBIT_GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _lowbit_cases(), ids=lambda c: c["name"])
def test_golden_lowbit_examples(case):
    """Hand-derived 2-bit and 64-element-group cases: scales, codes, packed bytes."""
    from oracle import pack_codes, unpack_codes
    bits, group, n = case["bits"], case["group"], case["length"]
    delta = np.zeros(n, np.float32)
    for i, s in case["delta"].items():
        delta[int(i)] = np.float32(s)
    codes, scales = quantize_groups(delta[None], group, bits)
    assert [int(b) for b in scales.view(np.uint16)[0]] == [int(b, 16) for b in case["scale_bits"]]
    want = np.zeros(n, np.int8)
    for i, c in case["codes"].items():
        want[int(i)] = c
    assert codes[0].tolist() == want.tolist()
    packed = np.zeros(n * bits // 8, np.uint8)
    for i, h in case["packed"].items():
        packed[int(i)] = int(h, 16)
    assert pack_codes(codes[0], bits).tolist() == packed.tolist()
    assert unpack_codes(packed, bits).tolist() == want.tolist()
