"""flashloop_attend_noalloc (the entry point for callers that cannot allocate)
against flashloop_attend with a caller workspace: the same kernels, so every
output and every arena byte must be identical.  Calls run back to back on the
library's per-GPU scratch, a smaller one after a larger one, so the second
call starts on the first call's leftovers; a full-loop call with the forward
key split (partial states and counters in the scratch) is included."""
import numpy as np
import pytest
import torch

from sparse_loop_attention_amd import abi
from sparse_loop_attention_amd.driver import to_device
from sparse_loop_attention_amd.synth import round_bf16

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(S, H, N, d, na, ns, seed):
    rng = np.random.default_rng(seed)
    bf = lambda *shape: to_device(round_bf16(rng.standard_normal(shape).astype(np.float32)), torch.bfloat16, DEV)
    x = {"k1": bf(S, N, H, d), "v1": bf(S, N, H, d), "k2": bf(S, N, H, d), "v2": bf(S, N, H, d),
         "q1": bf(S, N, H, d), "q2": bf(S, N, H, d)}
    x["act"] = torch.from_numpy(np.stack([np.sort(rng.choice(N, na, replace=False)) for _ in range(S)])
                                .astype(np.int32)).to(DEV)
    kv = abi.KVStore(S, H, d, N, 2, torch.bfloat16, [na], DEV)
    kv.arena.zero_()
    every = torch.arange(N, dtype=torch.int32, device=DEV)[None].repeat(S, 1).contiguous()
    abi.kv_commit(kv, 1, every, x["k1"], x["v1"])
    o = torch.zeros(S, N, H, d, device=DEV)
    lse = torch.zeros(S, N, H, device=DEV)
    c = torch.zeros(S, H, N, device=DEV)
    a = abi.attend_args(kv, abi.FL_ATTEND_FULL, 1, x["q1"], None, None, N, None, o, lse, c)
    ws = torch.empty(max(abi.attend_workspace_bytes(a), 256), dtype=torch.uint8, device=DEV)
    abi.attend(abi.attend_args(kv, abi.FL_ATTEND_FULL, 1, x["q1"], None, None, N, None, o, lse, c, ws))
    x["keys"] = torch.empty(S, H, ns, dtype=torch.int32, device=DEV)
    abi.select_keys(c, ns, x["keys"])
    x.update(kv=kv, o=o, lse=lse, c=c, N=N, na=na)
    return x


def _call(x, mode, noalloc):
    """One attend call on copies of the case's state; returns (o, lse, colmass, arena)."""
    kv = x["kv"]
    arena0 = kv.arena.clone()
    o, lse, c = x["o"].clone(), x["lse"].clone(), x["c"].clone()
    if mode == "full":
        args = lambda ws: abi.attend_args(kv, abi.FL_ATTEND_FULL, 1, x["q1"], None, None, x["N"], None, o, lse, c, ws)
    else:
        commit = dict(k_new=x["k2"], v_new=x["v2"])
        args = lambda ws: abi.attend_args(kv, abi.FL_ATTEND_LAZY, 2, x["q2"], x["q1"], x["act"], x["na"], x["keys"],
                                          o, lse, c, ws, commit=commit)
    need = abi.attend_workspace_bytes(args(None))
    assert 0 < need <= abi.STATIC_SCRATCH_BYTES
    if noalloc:
        abi.attend_noalloc(args(None))
    else:
        ws = torch.full((need,), 0x5A, dtype=torch.uint8, device=DEV)
        abi.attend(args(ws))
    torch.cuda.synchronize()
    out = (o.cpu(), lse.cpu(), c.cpu(), kv.arena.cpu())
    kv.arena.copy_(arena0)
    return out


def test_noalloc_equals_workspace_calls():
    big = _case(4, 16, 2560, 128, 2048, 512, 1)         # 256-row lazy workgroups, fused commit
    small = _case(1, 3, 700, 96, 150, 70, 2)            # a smaller call after it
    split = _case(1, 8, 2048, 128, 2048, 205, 3)        # full loop with the forward key split
    for x, mode in ((big, "lazy"), (small, "lazy"), (split, "full"), (small, "full")):
        want = _call(x, mode, noalloc=False)
        got = _call(x, mode, noalloc=True)
        for w, g, name in zip(want, got, ("o", "lse", "colmass", "arena")):
            assert torch.equal(w, g), (mode, x["N"], name)
        assert torch.isfinite(got[0]).all()


def test_noalloc_rejects_a_call_beyond_its_scratch():
    """The 32K full loop needs more scratch than the library holds: rejected
    with FL_ERR_WORKSPACE before any launch, the message names the size."""
    S, H, N, d = 1, 16, 32768, 128
    kv = abi.KVStore(S, H, d, N, 1, torch.bfloat16, [], DEV)
    q = torch.empty(S, N, H, d, dtype=torch.bfloat16, device=DEV)
    o = torch.empty(S, N, H, d, device=DEV)
    lse = torch.empty(S, N, H, device=DEV)
    c = torch.empty(S, H, N, device=DEV)
    a = abi.attend_args(kv, abi.FL_ATTEND_FULL, 1, q, None, None, N, None, o, lse, c)
    assert abi.attend_workspace_bytes(a) > abi.STATIC_SCRATCH_BYTES
    with pytest.raises(abi.FlashLoopError) as e:
        abi.attend_noalloc(a)
    assert e.value.status == abi.FL_ERR_WORKSPACE and "scratch" in str(e.value)
