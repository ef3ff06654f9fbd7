"""The run-time check of the split reductions (GPU).

A full loop whose forward pass is cut into key parts, or whose column mass
is cut into row ranges, merges the parts' partial results in the part that
finishes last, and a lazy loop whose two passes run as two workgroups meets
them in the one that ends last; this relies on every part of a head running
on one XCD, whose L2 is where they meet.  Each part records its XCD; a mismatch sets
FL_DEV_XCD_SPLIT in the call's dev_status word.  After every loop of the
prefill workloads at full size the word must be 0; with the host-set test
flag (odd parts report another XCD) the check must fire, with the outputs
unchanged.
"""
import dataclasses
import os

import numpy as np
import pytest
import torch

from sparse_loop_attention_amd import abi, configs, driver
from sparse_loop_attention_amd.driver import to_device
from sparse_loop_attention_amd.synth import SyntheticLoops, round_bf16

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("name", ["single_layer", "long_prefill", "deep"])
def test_no_split_part_runs_on_another_xcd(name):
    wl = configs.WORKLOADS[name]
    inputs = driver.upload_loops(wl, SyntheticLoops(wl), DEV)
    run = driver.PrefillRun(wl, inputs, DEV)
    for step in range(2):
        run.run()
    torch.cuda.synchronize()
    assert int(run.dev_status.item()) == 0


def _full_call(S, H, N, d, seed, status):
    rng = np.random.default_rng(seed)
    bf = lambda *shape: to_device(round_bf16(rng.standard_normal(shape).astype(np.float32)), torch.bfloat16, DEV)
    kv = abi.KVStore(S, H, d, N, 1, torch.bfloat16, [], DEV)
    every = torch.arange(N, dtype=torch.int32, device=DEV)[None].repeat(S, 1).contiguous()
    abi.kv_commit(kv, 1, every, bf(S, N, H, d), bf(S, N, H, d))
    q = bf(S, N, H, d)
    o = torch.zeros(S, N, H, d, device=DEV)
    lse = torch.zeros(S, N, H, device=DEV)
    c = torch.zeros(S, H, N, device=DEV)
    a = abi.attend_args(kv, abi.FL_ATTEND_FULL, 1, q, None, None, N, None, o, lse, c)
    ws = torch.empty(abi.attend_workspace_bytes(a), dtype=torch.uint8, device=DEV)
    abi.attend(abi.attend_args(kv, abi.FL_ATTEND_FULL, 1, q, None, None, N, None, o, lse, c, ws, dev_status=status))
    torch.cuda.synchronize()
    return o, lse, c


@pytest.mark.parametrize("S,H,N,d", [(1, 8, 2048, 128), (1, 16, 4096, 128)],
                         ids=["key-split forward", "column-mass ranges"])
def test_forced_mismatch_is_reported(S, H, N, d):
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    ref = _full_call(S, H, N, d, 7, status)
    assert int(status.item()) == 0
    os.environ["FLASHLOOP_TEST_XCD_SPLIT"] = "1"
    try:
        got = _full_call(S, H, N, d, 7, status)
    finally:
        del os.environ["FLASHLOOP_TEST_XCD_SPLIT"]
    assert int(status.item()) & abi.FL_DEV_XCD_SPLIT
    for x, y in zip(ref, got):
        assert torch.equal(x, y)


def test_forced_mismatch_is_reported_lazy():
    """A lazy loop with its two passes as two workgroups (16 heads, 1229 of
    4096 rows active: well under one round of workgroups)."""
    wl = dataclasses.replace(configs.scaled(configs.LONG_PREFILL, 4096), n_loops=2, n_full=1)
    assert wl.n_heads >= 8
    inputs = driver.upload_loops(wl, SyntheticLoops(wl), DEV)
    run = driver.PrefillRun(wl, inputs, DEV, overlap=False)
    run.run(upto=1)
    snap = run.snapshot()
    run.run(start=2)
    torch.cuda.synchronize()
    assert int(run.dev_status.item()) == 0
    ref = [x.clone() for x in (run.o, run.lse, run.colmass)]
    run.restore(snap)
    os.environ["FLASHLOOP_TEST_XCD_SPLIT"] = "1"
    try:
        run.run(start=2)
        torch.cuda.synchronize()
    finally:
        del os.environ["FLASHLOOP_TEST_XCD_SPLIT"]
    assert int(run.dev_status.item()) & abi.FL_DEV_XCD_SPLIT
    for x, y in zip(ref, (run.o, run.lse, run.colmass)):
        assert torch.equal(x, y)
