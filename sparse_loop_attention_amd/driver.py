"""Runs the loops of a workload through the C ABI on one GPU.

The sequence follows the page "FlashLoop: Fast and Memory-Efficient Looped
Transformers via Lazy Updates", section "FlashLoop combines three kinds of
savings": loops 1..F run in full (commit the base or a dense delta layer, full
causal attention); each later loop ranks tokens by the change of the previous
loop, selects keys from the previous loop's column mass, commits int4 deltas
of the active tokens and runs mass-corrected attention.

The per-loop inputs come from a synthetic stand-in for the shared block (the
model weights are not available), which produces every row of h and Q per
loop; a looped model recomputes only the active rows and carries the others.
The active sets are nested (loop l ranks the rows of loop l-1's set), so a
row that is a candidate in loop l was active in every earlier loop: its
effective state is the previous loops' output for that row.  The token scores
therefore read h of loops l-1 and l-2 directly, and attention reads the active
rows' queries of loops l and l-1 by token from those loops' outputs.

The token selection of a loop depends only on the hidden states and on the
previous loop's active set, not on any attention result, so PrefillRun issues
it on a second stream (default priority) that runs ahead of the attention
chain; a loop's attention waits for its own selection only.  Each wait costs
a cross-stream synchronisation, which only pays where the attention chain
keeps the GPU busy meanwhile (4096 tokens or more).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np
import torch

from . import abi
from .configs import Workload
from .synth import SyntheticLoops, to_bf16_bits


def torch_dtype(wl: Workload) -> torch.dtype:
    return torch.bfloat16 if wl.dtype == "bf16" else torch.float32


def to_device(x: np.ndarray, dtype: torch.dtype, device) -> torch.Tensor:
    """float32 values already representable in `dtype` -> device tensor (exact)."""
    if dtype == torch.bfloat16:
        bits = to_bf16_bits(x)
        return torch.from_numpy(bits.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(device)


def upload_loops(wl: Workload, loops: SyntheticLoops, device="cuda") -> Dict[int, Dict[str, torch.Tensor]]:
    dt = torch_dtype(wl)
    out = {}
    for l, x in loops:
        out[l] = {name: to_device(arr, dt, device) for name, arr in x.items()}
    return out


class CallTimer:
    """hipEvent pairs around each ABI call, on the stream the call is issued
    on (diagnostics: the benchmark's per-call medians).  ``calls[name]`` holds
    (start, end) event pairs; ``ms()`` waits for them."""

    def __init__(self):
        self.calls: Dict[str, list] = {}

    def __call__(self, name: str):
        timer = self

        class _Span:
            def __enter__(self):
                self.a = torch.cuda.Event(enable_timing=True)
                self.b = torch.cuda.Event(enable_timing=True)
                self.a.record(torch.cuda.current_stream())
                return self

            def __exit__(self, *exc):
                self.b.record(torch.cuda.current_stream())
                timer.calls.setdefault(name, []).append((self.a, self.b))
                return False

        return _Span()

    def ms(self) -> Dict[str, List[float]]:
        torch.cuda.synchronize()
        return {k: [a.elapsed_time(b) for a, b in v] for k, v in self.calls.items()}


class _NoTimer:
    def __call__(self, name: str):
        return self

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        return False


_NO_TIMER = _NoTimer()


@dataclass
class LoopRecord:
    rows: Optional[torch.Tensor] = None
    keys: Optional[torch.Tensor] = None
    scores: Optional[torch.Tensor] = None
    o: Optional[torch.Tensor] = None
    lse: Optional[torch.Tensor] = None
    colmass: Optional[torch.Tensor] = None
    arena: Optional[torch.Tensor] = None
    exited: Optional[torch.Tensor] = None      # early exit: flags after the loop


class PrefillRun:
    """GPU state of one prefill workload (n_seq = 1) and its loop sequence."""

    def __init__(self, wl: Workload, inputs: Dict[int, Dict[str, torch.Tensor]], device="cuda", fuse: bool = True,
                 formula: str = "column", freeze_keys: bool = False, exit_threshold: Optional[float] = None,
                 overlap: Optional[bool] = None):
        """formula "column" (default) or "mixture"; freeze_keys reuses the first
        lazy loop's key group in every later lazy loop; exit_threshold enables
        the early exit (the sequence stops before the first lazy loop whose
        largest token change is below it); overlap runs the token selection on
        a second stream (None: from 8192 tokens up; at 4096 tokens the lazy
        loops measured 0.28 ms with it and 0.225 ms without, at 16384 and
        32768 tokens 8.10 vs 8.33 ms and 2.36 vs 2.42 ms)."""
        assert wl.n_seq == 1 and not wl.decode
        self.wl, self.inp, self.dev, self.fuse = wl, inputs, device, fuse
        self.formula, self.freeze_keys = formula, freeze_keys
        self.exit_threshold = exit_threshold
        self.exit_flags = torch.zeros(1, dtype=torch.int32, device=device) if exit_threshold is not None else None
        n, H, d = wl.n_tokens, wl.n_heads, wl.head_dim
        dt = torch_dtype(wl)
        self.kv = abi.KVStore(1, H, d, n, wl.n_loops, dt, wl.layer_caps(), device,
                              group=wl.group, delta_bits=wl.delta_bits)
        self.o = torch.empty(n, H, d, dtype=torch.float32, device=device)
        self.lse = torch.empty(n, H, dtype=torch.float32, device=device)
        self.colmass = torch.empty(H, n, dtype=torch.float32, device=device)
        # one score buffer per lazy loop: a loop's selection may run before the
        # previous loop's readers of its scores
        self.scores_l = {l: torch.empty(n, dtype=torch.float64, device=device)
                         for l in range(wl.n_full + 1, wl.n_loops + 1)}
        if overlap is None:
            overlap = n >= 8192
        self.side = torch.cuda.Stream(device=device) if overlap else None
        self.all_rows = torch.arange(n, dtype=torch.int32, device=device)
        self.act = {l: torch.empty(wl.n_active(l), dtype=torch.int32, device=device)
                    for l in range(wl.n_full + 1, wl.n_loops + 1)}
        self.keys_l = {l: torch.empty(H, wl.n_keys, dtype=torch.int32, device=device)
                       for l in range(wl.n_full + 1, wl.n_loops + 1)}
        # FL_DEV_* bits of failed run-time checks in the attention kernels (0: none)
        self.dev_status = torch.zeros(1, dtype=torch.int32, device=device)
        self.workspace = None
        ws = 0
        for l in range(1, wl.n_loops + 1):
            if l in self.inp:                      # loops whose inputs were drawn
                ws = max(ws, abi.attend_workspace_bytes(self._attend_args(l)))
        self.workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=device)
        self.timer = _NO_TIMER

    # -------------------------------------------------------------- checkpoints
    def state_tensors(self) -> Dict[str, torch.Tensor]:
        """Every buffer a later loop reads: the outputs (o, lse, column mass),
        the KV arena and the per-loop index sets and scores."""
        out = {"o": self.o, "lse": self.lse, "colmass": self.colmass, "arena": self.kv.arena}
        for l in self.act:
            out[f"act{l}"], out[f"keys{l}"], out[f"scores{l}"] = self.act[l], self.keys_l[l], self.scores_l[l]
        if self.exit_flags is not None:
            out["exit_flags"] = self.exit_flags
        return out

    def snapshot(self, arena: bool = True) -> Dict[str, torch.Tensor]:
        """Device copies of the state (see restore)."""
        return {k: v.clone() for k, v in self.state_tensors().items() if arena or k != "arena"}

    def restore(self, snap: Dict[str, torch.Tensor]) -> None:
        cur = self.state_tensors()
        for k, v in snap.items():
            cur[k].copy_(v)

    def save_state(self, path: str, loop: int) -> None:
        """Checkpoint after loop `loop` (torch file of host tensors, no pickled objects)."""
        torch.cuda.synchronize()
        torch.save({"loop": torch.tensor(loop), **{k: v.cpu() for k, v in self.state_tensors().items()}}, path)

    def load_state(self, path: str) -> int:
        """Restores a checkpoint written by save_state; returns its loop."""
        snap = torch.load(path, weights_only=True)
        loop = int(snap.pop("loop"))
        self.restore({k: v.to(self.dev) for k, v in snap.items()})
        return loop

    def _attend_args(self, l: int):
        wl = self.wl
        if l <= wl.n_full:
            # every row; with fusion the call also commits every token's K/V
            commit = dict(k_new=self.inp[l]["k"], v_new=self.inp[l]["v"]) if self.fuse else None
            return abi.attend_args(self.kv, abi.FL_ATTEND_FULL, l, self.inp[l]["q"], None, None, wl.n_tokens,
                                   None, self.o, self.lse, self.colmass, self.workspace, commit=commit,
                                   dev_status=self.dev_status)
        na = wl.n_active(l)
        commit = dict(k_new=self.inp[l]["k"], v_new=self.inp[l]["v"]) if self.fuse else None
        # the active rows' queries of loops l and l-1, read by token
        return abi.attend_args(self.kv, abi.FL_ATTEND_LAZY, l, self.inp[l]["q"], self.inp[l - 1]["q"],
                               self.act[l], na, self.keys_l[l], self.o, self.lse, self.colmass, self.workspace,
                               commit=commit, formula=self.formula, exit_flags=self.exit_flags,
                               dev_status=self.dev_status)

    # ------------------------------------------------------------------ loops
    def full_loop(self, l: int) -> None:
        x = self.inp[l]
        t = self.timer
        if not self.fuse:
            with t(f"loop{l}.kv_commit"):
                abi.kv_commit(self.kv, l, self.all_rows, x["k"], x["v"])
        with t(f"loop{l}.attend"):
            abi.attend(self._attend_args(l))

    def lazy_loop(self, l: int, cand: Optional[torch.Tensor]) -> torch.Tensor:
        wl, x = self.wl, self.inp[l]
        act, na, scores = self.act[l], wl.n_active(l), self.scores_l[l]
        t = self.timer
        # the change of the candidate rows during loop l-1 (every row after the full loops);
        # on the second stream it runs beside the previous loop's attention and this
        # loop's key selection, which do not depend on it
        if self.side is not None:
            with torch.cuda.stream(self.side), t(f"loop{l}.select_tokens"):
                abi.select_tokens(self.inp[l - 1]["h"][0], self.inp[l - 2]["h"][0], na, scores, act, cand)
        else:
            with t(f"loop{l}.select_tokens"):
                abi.select_tokens(self.inp[l - 1]["h"][0], self.inp[l - 2]["h"][0], na, scores, act, cand)
        first = wl.n_full + 1
        if self.freeze_keys and l > first:
            self.keys_l[l].copy_(self.keys_l[first])
        else:
            with t(f"loop{l}.select_keys"):
                abi.select_keys(self.colmass, wl.n_keys, self.keys_l[l])
        if self.side is not None:
            torch.cuda.current_stream().wait_stream(self.side)
        if self.exit_flags is not None:          # early exit: no later library call touches the sequence
            abi.exit_check(self.exit_flags, self.exit_threshold, scores=scores)
        if not self.fuse:
            with t(f"loop{l}.kv_commit"):
                abi.kv_commit(self.kv, l, act, x["k"], x["v"], exit_flags=self.exit_flags)
        with t(f"loop{l}.attend"):
            abi.attend(self._attend_args(l))
        return act

    def run(self, upto: Optional[int] = None, record: bool = False, start: int = 1) -> List[LoopRecord]:
        """Loops start..upto (default: all).  start > 1 continues from the
        state the buffers hold (the loops before it must have run, or a
        checkpoint been restored)."""
        wl = self.wl
        T = wl.n_loops if upto is None else upto
        recs: List[LoopRecord] = []
        cand = None if start <= wl.n_full + 1 else self.act[start - 1]
        if self.exit_flags is not None and start == 1:
            self.exit_flags.zero_()
        if self.side is not None:
            # the selection buffers are reused: earlier steps' readers finish first
            self.side.wait_stream(torch.cuda.current_stream())
        for l in range(start, T + 1):
            if l <= wl.n_full:
                self.full_loop(l)
                cand = None
                rec = LoopRecord()
            else:
                act = self.lazy_loop(l, cand)
                cand = act
                rec = LoopRecord(rows=act.clone() if record else None,
                                 keys=self.keys_l[l].clone() if record else None,
                                 scores=self.scores_l[l].clone() if record else None)
            if record:
                rec.o, rec.lse, rec.colmass = self.o.clone(), self.lse.clone(), self.colmass.clone()
                rec.arena = self.kv.arena.clone()
                if self.exit_flags is not None:
                    rec.exited = self.exit_flags.clone()
            recs.append(rec)
        if self.side is not None:
            torch.cuda.current_stream().wait_stream(self.side)
        return recs


class DecodeRun:
    """Decode workload: n_seq sequences, one new query per sequence and loop."""

    def __init__(self, wl: Workload, inputs: Dict[int, Dict[str, torch.Tensor]], ctx_sets: Dict[int, List[np.ndarray]],
                 device="cuda", fuse: bool = True, formula: str = "column", freeze_keys: bool = False,
                 exit_threshold: Optional[float] = None, single_launch: bool = False):
        """single_launch runs the lazy loops 2..T as one flashloop_decode_loops
        call (key selection, commit and attention of every loop in one kernel)
        instead of select_keys + attend per loop; it re-selects keys every loop
        and takes no early exit between loops."""
        assert wl.decode
        if single_launch and (freeze_keys or exit_threshold is not None or not fuse):
            raise ValueError("single_launch: no frozen keys, no early exit, commit fused")
        self.single_launch = single_launch
        self.wl, self.inp, self.dev, self.fuse = wl, inputs, device, fuse
        self.formula, self.freeze_keys = formula, freeze_keys
        self.exit_threshold = exit_threshold
        self.exit_flags = (torch.zeros(wl.n_seq, dtype=torch.int32, device=device)
                           if exit_threshold is not None else None)
        S, n, H, d = wl.n_seq, wl.n_tokens, wl.n_heads, wl.head_dim
        dt = torch_dtype(wl)
        self.kv = abi.KVStore(S, H, d, n, wl.n_loops, dt, wl.layer_caps(), device,
                              group=wl.group, delta_bits=wl.delta_bits)
        self.ctx = {}
        for l in range(1, wl.n_loops + 1):
            if l == 1:
                idx = np.tile(np.arange(n - 1, dtype=np.int32), (S, 1))
            else:
                idx = np.stack(ctx_sets[l]).astype(np.int32)
            self.ctx[l] = torch.from_numpy(idx).to(device)
        self.last = torch.full((S, 1), n - 1, dtype=torch.int32, device=device)
        self.o = torch.empty(S, 1, H, d, dtype=torch.float32, device=device)
        self.lse = torch.empty(S, 1, H, dtype=torch.float32, device=device)
        self.colmass = torch.empty(S, H, n, dtype=torch.float32, device=device)
        self.keys = torch.empty(S, H, wl.n_keys, dtype=torch.int32, device=device)
        # single launch: every lazy loop's keys [loop - 2][S][H][n_keys]
        self.keys_all = (torch.empty(max(wl.n_loops - 1, 1), S, H, wl.n_keys, dtype=torch.int32, device=device)
                         if single_launch else None)
        ws = 0
        for l in range(1, wl.n_loops + 1):
            ws = max(ws, abi.attend_workspace_bytes(self._args(l, None)))
        self.workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=device)
        self.timer = _NO_TIMER

    # -------------------------------------------------------------- checkpoints
    def state_tensors(self) -> Dict[str, torch.Tensor]:
        """Every buffer a later loop reads: the new token's outputs, its
        column-mass rows, the key sets and the KV arena."""
        out = {"o": self.o, "lse": self.lse, "colmass": self.colmass, "keys": self.keys, "arena": self.kv.arena}
        if self.exit_flags is not None:
            out["exit_flags"] = self.exit_flags
        return out

    snapshot = PrefillRun.snapshot
    restore = PrefillRun.restore
    save_state = PrefillRun.save_state
    load_state = PrefillRun.load_state

    def _args(self, l, ws):
        x = self.inp[l]
        if l == 1:
            return abi.attend_args(self.kv, abi.FL_ATTEND_FULL, 1, x["q"], None, self.last, 1, None,
                                   self.o, self.lse, self.colmass, ws, q_compact=True, o_compact=True)
        commit = None
        if self.fuse:
            commit = dict(k_new=x["k"], v_new=x["v"], slot_base=self.ctx[l].shape[1], reset=False)
        return abi.attend_args(self.kv, abi.FL_ATTEND_LAZY, l, x["q"], self.inp[l - 1]["q"], self.last, 1,
                               self.keys, self.o, self.lse, self.colmass, ws, q_compact=True, o_compact=True,
                               commit=commit, formula=self.formula, exit_flags=self.exit_flags)

    def build_context(self) -> None:
        for l in range(1, self.wl.n_loops + 1):
            x = self.inp[l]
            abi.kv_commit(self.kv, l, self.ctx[l], x["k"], x["v"], slot_base=0, reset_map=True)

    def loop(self, l: int) -> None:
        wl, x = self.wl, self.inp[l]
        t = self.timer
        slot_base = 0 if l == 1 else self.ctx[l].shape[1]
        if l >= 2 and self.exit_flags is not None:   # early exit of each sequence, from its new token's change
            abi.exit_check(self.exit_flags, self.exit_threshold, h_cur=self.inp[l - 1]["h"], h_prev=self.inp[l - 2]["h"])
        if l == 1 or not self.fuse:
            with t(f"loop{l}.kv_commit"):
                abi.kv_commit(self.kv, l, self.last, x["k"], x["v"], slot_base=slot_base, reset_map=False,
                              exit_flags=self.exit_flags)
        if l >= 2 and not (self.freeze_keys and l > 2):
            with t(f"loop{l}.select_keys"):
                abi.select_keys(self.colmass, wl.n_keys, self.keys)
        with t(f"loop{l}.attend"):
            abi.attend(self._args(l, self.workspace))

    def lazy_loops_single(self, first: int, last: int) -> None:
        """Lazy loops first..last in one flashloop_decode_loops call."""
        wl, x = self.wl, self.inp
        with self.timer(f"loops{first}-{last}.decode_loops"):
            abi.decode_loops(self.kv, first, last, {l: x[l]["q"] for l in range(first - 1, last + 1)}, self.last,
                             wl.n_keys, self.o, self.lse, self.colmass, {l: x[l]["k"] for l in range(first, last + 1)},
                             {l: x[l]["v"] for l in range(first, last + 1)},
                             {l: self.ctx[l].shape[1] for l in range(first, last + 1)},
                             keys_out=self.keys_all[first - 2:last - 1], formula=self.formula)

    def run(self, record: bool = False, start: int = 1, upto: Optional[int] = None) -> List[LoopRecord]:
        """Loops start..upto (default: all); start > 1 continues from the
        state the buffers hold."""
        recs = []
        if self.exit_flags is not None and start == 1:
            self.exit_flags.zero_()
        if self.single_launch:
            last = self.wl.n_loops if upto is None else upto
            if start == 1:
                self.loop(1)
                if record:
                    recs.append(LoopRecord(o=self.o.clone(), lse=self.lse.clone(), colmass=self.colmass.clone()))
            first = max(2, start)
            if first <= last:
                self.lazy_loops_single(first, last)
                if record:                  # the keys of every loop; the outputs after the last
                    for l in range(first, last + 1):
                        recs.append(LoopRecord(keys=self.keys_all[l - 2].clone()))
                    recs[-1].o, recs[-1].lse, recs[-1].colmass = self.o.clone(), self.lse.clone(), self.colmass.clone()
            return recs
        for l in range(start, (self.wl.n_loops if upto is None else upto) + 1):
            self.loop(l)
            if record:
                recs.append(LoopRecord(keys=self.keys.clone() if l >= 2 else None, o=self.o.clone(),
                                       lse=self.lse.clone(), colmass=self.colmass.clone(),
                                       exited=None if self.exit_flags is None else self.exit_flags.clone()))
        return recs
