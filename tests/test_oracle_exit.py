"""Pins for the oracle's early exit (reading E1, CPU only).

Page "深度解析循环Transformer架构：隐式推理如何重塑大模型算力效率" (looped
Transformers), section 四 "开发者实践", item 1 "计算图的动态控制": the loop
stops once the change of the state between two loops falls below a
threshold.  Reading E1: before each lazy loop, the sequence's change is its
largest token score (the change of the previous loop); a change below tau
ends the sequence's loops, keeping the last loop's outputs.

The pins tie the exit decision to quantities computed independently of it:
the scores the no-exit run records at each loop (strict comparison, the
maximum rather than a sum or mean, the loop whose change is read), exact
rational squared norms of the decode token's hidden state, and a trajectory
whose state stops changing.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from sparse_loop_attention_amd import configs
from sparse_loop_attention_amd.synth import SyntheticLoops


def _data(wl):
    return [(l, {k: v.copy() for k, v in x.items()}) for l, x in SyntheticLoops(wl)]


PREFILL = configs.scaled(configs.SINGLE_LAYER, 256, n_heads=2)
LONG = configs.scaled(configs.LONG_PREFILL, 256, n_heads=2)       # one full loop, three lazy loops


def _same_state(a, b):
    for x, y in ((a.o, b.o), (a.lse, b.lse), (a.colmass, b.colmass)):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("wl", [PREFILL, LONG], ids=["single_layer_256", "long_prefill_256"])
def test_prefill_exit_bounds(wl):
    data = _data(wl)
    base, hist = oracle.run_prefill(wl, iter(data), keep=True)
    st0 = oracle.run_prefill(wl, iter(data), exit_threshold=0.0)          # a change is never < 0
    assert st0.exited_at is None and st0.loop == wl.n_loops
    _same_state(st0, base)
    st_inf = oracle.run_prefill(wl, iter(data), exit_threshold=math.inf)  # exits before the first lazy loop
    assert st_inf.exited_at == wl.n_full + 1 and st_inf.loop == wl.n_full
    _same_state(st_inf, hist[wl.n_full - 1])


@pytest.mark.parametrize("wl", [PREFILL, LONG], ids=["single_layer_256", "long_prefill_256"])
def test_prefill_exit_threshold_against_recorded_scores(wl):
    """tau equal to loop l's largest recorded score: no exit at l (strict);
    the next double up: exit exactly at l, with the state of loop l-1."""
    data = _data(wl)
    base, hist = oracle.run_prefill(wl, iter(data), keep=True)
    lazy = list(range(wl.n_full + 1, wl.n_loops + 1))
    peak = {l: float(np.max(hist[l - 1].records[l]["scores"])) for l in lazy}
    for l in lazy:
        # the first lazy loop whose largest change is below tau is where the run stops
        for tau, expect_here in ((peak[l], False), (float(np.nextafter(peak[l], np.inf)), True)):
            expect = next((j for j in lazy if peak[j] < tau), None)
            st = oracle.run_prefill(wl, iter(data), exit_threshold=tau)
            assert st.exited_at == expect, (l, tau)
            if expect_here:
                assert expect is not None and expect <= l
            if expect is not None:
                _same_state(st, hist[expect - 2])
    # the largest score, not a sum or a mean: a tau between the largest score
    # and the sum of the scores exits, one below the largest does not
    l = lazy[-1]
    scores = hist[l - 1].records[l]["scores"]
    if np.count_nonzero(scores) > 1 and all(peak[j] > peak[l] for j in lazy[:-1]):
        tau = 0.5 * (peak[l] + float(np.sum(scores)))
        assert tau > peak[l]
        st = oracle.run_prefill(wl, iter(data), exit_threshold=tau)
        assert st.exited_at is not None and st.exited_at <= l


DECODE = configs.scaled(configs.DECODE, 300, n_seq=3, n_heads=2)


def _decode_setup(wl):
    syn = SyntheticLoops(wl)
    ctx = {l: syn.context_active_sets(l) for l in range(2, wl.n_loops + 1)}
    data = {l: {k: v.copy() for k, v in x.items()} for l, x in SyntheticLoops(wl)}
    return ctx, data


def _exact_change(a, b):
    """Exact squared L2 distance of two float32 rows (rational arithmetic)."""
    return sum((Fraction(float(x)) - Fraction(float(y))) ** 2 for x, y in zip(a.ravel(), b.ravel()))


def test_decode_exit_against_exact_change():
    wl = DECODE
    ctx, data = _decode_setup(wl)
    for s in range(wl.n_seq):
        sets = {l: ctx[l][s] for l in ctx}
        base, _ = oracle.run_decode_seq(wl, None, s, sets, data)
        assert len(base) == wl.n_loops
        change = {l: _exact_change(data[l - 1]["h"][s], data[l - 2]["h"][s]) for l in range(2, wl.n_loops + 1)}
        for l in range(2, wl.n_loops + 1):
            for tau, exits_by_l in ((float(change[l]) * (1 - 1e-9), False), (float(change[l]) * (1 + 1e-9), True)):
                first = next((j for j in range(2, wl.n_loops + 1) if change[j] < Fraction(tau)), None)
                out, _ = oracle.run_decode_seq(wl, None, s, sets, data, exit_threshold=tau)
                ran = wl.n_loops if first is None else first - 1
                assert len(out) == ran, (s, l, tau)
                if exits_by_l:
                    assert first is not None and first <= l
                for a, b in zip(out, base):
                    for key in ("o", "lse", "colmass"):
                        assert np.array_equal(a[key], b[key])


def test_decode_exit_when_the_state_stops_changing():
    """The new token's hidden state at loop 2 equals loop 1's: its change read
    before loop 3 is exactly 0, so any tau > 0 ends the sequence after loop 2
    (and tau = 0 never does)."""
    wl = DECODE
    ctx, data = _decode_setup(wl)
    s = 1
    data[2]["h"][s] = data[1]["h"][s]
    sets = {l: ctx[l][s] for l in ctx}
    out, _ = oracle.run_decode_seq(wl, None, s, sets, data, exit_threshold=1e-300)
    assert len(out) == 2
    out0, _ = oracle.run_decode_seq(wl, None, s, sets, data, exit_threshold=0.0)
    assert len(out0) == wl.n_loops
