"""Early exit per sequence on the GPU (flashloop_exit_check and the exit flags
of attend / commit) against the CPU oracle's reading E1.

Exit decisions are integers decided by float64 maxima; every threshold here
sits far (relative 1e-6 or more) from every change the run compares it with,
so both sides take the same decisions.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from sparse_loop_attention_amd import abi, configs, driver
from sparse_loop_attention_amd.synth import SyntheticLoops

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _check_o(got, want, what):
    want = np.asarray(want, np.float64)
    rms = math.sqrt(float(np.mean(want ** 2)))
    err = float(np.abs(np.asarray(got, np.float64) - want).max())
    assert err <= 2e-2 * rms, f"{what}: max err {err:.3e} > 2e-2 * RMS {rms:.3e}"

def _check_abs(got, want, what, tol=2e-2):
    """lse: max abs error (nats); an error of e rescales the next loop's p' by exp(e)."""
    err = float(np.abs(np.asarray(got, np.float64) - np.asarray(want, np.float64)).max())
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol}"



def _between(lo, hi):
    """A threshold strictly between two changes, far from both."""
    assert lo < hi * (1 - 1e-5)
    return math.sqrt(lo * hi) if lo > 0 else hi / 2


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_exit_check_kernel(dtype):
    rng = np.random.default_rng(7)
    S, R, Dh = 5, 37, 520
    h_prev = rng.standard_normal((S, R, Dh)).astype(np.float32)
    scale = np.exp(rng.uniform(-6, 0, (S, R, 1))).astype(np.float32)
    h_cur = (h_prev + scale * rng.standard_normal((S, R, Dh))).astype(np.float32)
    hc = torch.from_numpy(h_cur).to(DEV).to(dtype)
    hp = torch.from_numpy(h_prev).to(DEV).to(dtype)
    a64 = hc.double().cpu().numpy()
    b64 = hp.double().cpu().numpy()
    want = ((a64 - b64) ** 2).sum(-1).max(-1)                       # per sequence, float64
    order = np.sort(want)
    tau = _between(order[1], order[2])                              # two sequences below
    flags = torch.zeros(S, dtype=torch.int32, device=DEV)
    mx = torch.zeros(S, dtype=torch.float64, device=DEV)
    abi.exit_check(flags, tau, h_cur=hc, h_prev=hp, max_change=mx)
    torch.cuda.synchronize()
    np.testing.assert_allclose(mx.cpu().numpy(), want, rtol=1e-12)
    assert flags.cpu().numpy().tolist() == (want < tau).astype(np.int32).tolist()
    # precomputed scores give the same maxima; set flags stay set at tau = 0
    scores = torch.from_numpy(((a64 - b64) ** 2).sum(-1)).to(DEV)
    mx2 = torch.zeros(S, dtype=torch.float64, device=DEV)
    abi.exit_check(flags, 0.0, scores=scores, max_change=mx2)
    torch.cuda.synchronize()
    assert np.array_equal(mx2.cpu().numpy(), scores.cpu().numpy().max(-1))
    assert flags.cpu().numpy().tolist() == (want < tau).astype(np.int32).tolist()


def _prefill_peaks(wl, data):
    _, hist = oracle.run_prefill(wl, iter(data), keep=True)
    lazy = list(range(wl.n_full + 1, wl.n_loops + 1))
    return lazy, {l: float(np.max(hist[l - 1].records[l]["scores"])) for l in lazy}


@pytest.mark.parametrize("wl", [configs.scaled(configs.LONG_PREFILL, 640, n_heads=2),
                                configs.scaled(configs.DEEP, 320, n_heads=3)],
                         ids=["long_prefill_640", "deep_320"])
def test_prefill_early_exit_matches_oracle(wl):
    data = [(l, {k: v.copy() for k, v in x.items()}) for l, x in SyntheticLoops(wl)]
    lazy, peak = _prefill_peaks(wl, data)
    # exit before the second lazy loop whose largest change is below the one before it
    target = next(l for l in lazy[1:] if peak[l] < peak[l - 1] * (1 - 1e-5) and all(
        peak[j] > peak[l - 1] * (1 - 1e-5) for j in lazy if j < l))
    tau = _between(peak[target], peak[target - 1])
    st = oracle.run_prefill(wl, iter(data), exit_threshold=tau)
    assert st.exited_at == target
    inputs = driver.upload_loops(wl, SyntheticLoops(wl), DEV)
    run = driver.PrefillRun(wl, inputs, DEV, exit_threshold=tau)
    for rep in range(2):                                            # flags are reset by every run
        recs = run.run(record=True)
        torch.cuda.synchronize()
        for l in lazy:
            assert int(recs[l - 1].exited.item()) == int(l >= target), (rep, l)
        last = recs[target - 2]
        for l in range(target, wl.n_loops + 1):                     # nothing changes after the exit
            for name in ("o", "lse", "colmass"):
                assert torch.equal(getattr(recs[l - 1], name), getattr(last, name)), (l, name)
        _check_o(run.o.cpu().numpy(), st.o, "o")
        _check_abs(run.lse.cpu().numpy(), st.lse, "lse")
        _check_o(run.colmass.cpu().numpy(), st.colmass, "colmass")


def test_decode_early_exit_matches_oracle():
    wl = configs.scaled(configs.DECODE, 600, n_seq=6, n_heads=2)
    syn = SyntheticLoops(wl)
    ctx = {l: syn.context_active_sets(l) for l in range(2, wl.n_loops + 1)}
    data = {l: {k: v.copy() for k, v in x.items()} for l, x in SyntheticLoops(wl)}
    change = np.array([[float(((data[l - 1]["h"][s].astype(np.float64) - data[l - 2]["h"][s]) ** 2).sum())
                        for l in range(2, wl.n_loops + 1)] for s in range(wl.n_seq)])
    # a threshold between two of the loop-3 changes, away from every change
    vals = np.sort(change.ravel())
    mid = np.sort(change[:, 1])
    tau = _between(mid[len(mid) // 2 - 1], mid[len(mid) // 2])
    assert np.all(np.abs(vals - tau) > 1e-6 * tau)
    inputs = driver.upload_loops(wl, syn, DEV)
    run = driver.DecodeRun(wl, inputs, ctx, DEV, exit_threshold=tau)
    run.build_context()
    recs = run.run(record=True)
    torch.cuda.synchronize()
    ran = []
    for s in range(wl.n_seq):
        ref, _ = oracle.run_decode_seq(wl, None, s, {l: ctx[l][s] for l in ctx}, data, exit_threshold=tau)
        ran.append(len(ref))
        for l in range(1, wl.n_loops + 1):
            assert int(recs[l - 1].exited[s].item()) == int(l > len(ref)), (s, l)
        _check_o(recs[-1].o.cpu().numpy()[s], ref[-1]["o"], f"seq {s} o")
        _check_abs(recs[-1].lse.cpu().numpy()[s], ref[-1]["lse"], f"seq {s} lse")
        _check_o(recs[-1].colmass.cpu().numpy()[s], ref[-1]["colmass"], f"seq {s} colmass")
    assert min(ran) < wl.n_loops and max(ran) > min(ran)            # sequences exit at different loops
