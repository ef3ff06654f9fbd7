"""flashloop_decode_loops (lazy decode loops 2..T in one launch) on the GPU.

It must give what the per-loop calls give -- flashloop_select(KEYS) then
flashloop_attend(LAZY) with the commit fused, loop after loop -- bit for bit
(the same key sets, records, o, lse and column mass), and it is compared with
the oracle's decode driver (keys bit-exact, o and column mass within 2e-2 x
RMS, lse within 2e-2 absolute); page "FlashLoop: Fast and Memory-Efficient
Looped Transformers via Lazy Updates", section "FlashLoop combines three kinds
of savings", paragraphs 2-4.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
from sparse_loop_attention_amd import configs, driver
from sparse_loop_attention_amd.synth import SyntheticLoops

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _runs(wl, formula="column"):
    syn = SyntheticLoops(wl)
    ctx_sets = {l: syn.context_active_sets(l) for l in range(2, wl.n_loops + 1)}
    inputs = driver.upload_loops(wl, syn, DEV)
    out = []
    for single in (False, True):
        run = driver.DecodeRun(wl, inputs, ctx_sets, DEV, formula=formula, single_launch=single)
        run.kv.arena.zero_()
        run.build_context()
        recs = run.run(record=True)
        torch.cuda.synchronize()
        out.append((run, recs))
    return ctx_sets, out


CASES = [
    pytest.param(configs.scaled(configs.DECODE, 640, n_seq=3, n_heads=2), 4, 32, "column", id="640x3-4b32"),
    pytest.param(configs.scaled(configs.DECODE, 1000, n_seq=9, n_heads=3), 4, 32, "column", id="1000x9-4b32"),
    pytest.param(configs.scaled(configs.DECODE, 700, n_seq=2, n_heads=2), 2, 32, "column", id="700x2-2b32"),
    pytest.param(configs.scaled(configs.DECODE, 700, n_seq=2, n_heads=2), 4, 64, "column", id="700x2-4b64"),
    pytest.param(configs.scaled(configs.DECODE, 800, n_seq=3, n_heads=2), 4, 32, "mixture", id="800x3-mixture"),
    pytest.param(dataclasses.replace(configs.scaled(configs.DECODE, 600, n_seq=2, n_heads=2), n_loops=5,
                                     context_active=(None, 120, 120, 40)), 4, 32, "column", id="600x2-5loops"),
]


@pytest.mark.parametrize("wl,bits,group,formula", CASES)
def test_single_launch_equals_per_loop_calls(wl, bits, group, formula):
    wl = dataclasses.replace(wl, delta_bits=bits, group=group)
    _, ((run_m, recs_m), (run_s, recs_s)) = _runs(wl, formula)
    for l in range(2, wl.n_loops + 1):
        assert torch.equal(recs_m[l - 1].keys, recs_s[l - 1].keys), f"loop {l} keys"
    for name in ("o", "lse", "colmass"):
        assert torch.equal(getattr(recs_m[-1], name), getattr(recs_s[-1], name)), name
    assert torch.equal(run_m.kv.arena, run_s.kv.arena)


@pytest.mark.parametrize("wl,bits,group,formula", CASES[:2] + CASES[-1:])
def test_single_launch_matches_oracle(wl, bits, group, formula):
    wl = dataclasses.replace(wl, delta_bits=bits, group=group)
    ctx_sets, (_, (run_s, recs_s)) = _runs(wl, formula)
    data = {l: {k: v.copy() for k, v in x.items()} for l, x in SyntheticLoops(wl)}
    for s in range(wl.n_seq):
        ref, _ = oracle.run_decode_seq(wl, None, s, {l: ctx_sets[l][s] for l in ctx_sets}, data, formula=formula)
        for l in range(2, wl.n_loops + 1):
            assert np.array_equal(recs_s[l - 1].keys.cpu().numpy()[s], ref[l - 1]["keys"]), f"seq {s} loop {l} keys"
        want = ref[-1]
        for name, tol in (("o", None), ("lse", 2e-2), ("colmass", None)):
            got = getattr(recs_s[-1], name).cpu().numpy()[s].astype(np.float64)
            w = np.asarray(want[name], np.float64)
            err = float(np.abs(got - w).max())
            bar = tol if tol is not None else 2e-2 * math.sqrt(float(np.mean(w ** 2)))
            assert err <= bar, f"seq {s} {name}: {err:.3e} > {bar:.3e}"


def test_single_launch_full_size_decode():
    """The decode workload at full size (32 sequences x 8192 tokens, 16 heads,
    3 lazy loops): the single launch equals the per-loop calls bit for bit, and
    sequences 0 and 31 match the oracle."""
    wl = configs.DECODE
    ctx_sets, ((run_m, recs_m), (run_s, recs_s)) = _runs(wl)
    print("[decode_loops] full size: both runs done", flush=True)
    for l in range(2, wl.n_loops + 1):
        assert torch.equal(recs_m[l - 1].keys, recs_s[l - 1].keys), f"loop {l} keys"
    for name in ("o", "lse", "colmass"):
        assert torch.equal(getattr(recs_m[-1], name), getattr(recs_s[-1], name)), name
    assert torch.equal(run_m.kv.arena, run_s.kv.arena)
    data = {}
    for l, x in SyntheticLoops(wl):
        data[l] = {k: v[[0, wl.n_seq - 1]].copy() for k, v in x.items()}
    for si, s in enumerate((0, wl.n_seq - 1)):
        ref, _ = oracle.run_decode_seq(wl, None, si, {l: ctx_sets[l][s] for l in ctx_sets}, data)
        got_o = recs_s[-1].o.cpu().numpy()[s].astype(np.float64)
        w = ref[-1]["o"]
        assert float(np.abs(got_o - w).max()) <= 2e-2 * math.sqrt(float(np.mean(w ** 2))), f"seq {s} o"
        assert float(np.abs(recs_s[-1].lse.cpu().numpy()[s] - ref[-1]["lse"]).max()) <= 2e-2, f"seq {s} lse"
