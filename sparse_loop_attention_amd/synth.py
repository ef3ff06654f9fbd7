"""Seeded synthetic inputs for the looped-attention workloads.

This module only draws inputs: it holds none of the method's arithmetic
(no scores, no selection, no attention, no quantisation).  It stands in for
the shared block of a looped transformer, whose weights are not available:
every loop l produces new hidden states h and new Q/K/V for every token, and
the method decides which of them it actually consumes (page "FlashLoop: Fast
and Memory-Efficient Looped Transformers via Lazy Updates", section "Later
loops change only part of the state": most tokens change less and less from
loop to loop, a small group keeps changing).

Recipe (all draws from numpy ``PCG64`` streams keyed by
``SeedSequence([seed, seq, loop, tensor])``, so every tensor can be drawn
independently and in parallel):

* per-token change scale sigma_i: ``0.1*exp(z)``, z ~ N(0,1) (lognormal), or
  ``0.05*(1-U)^(-1/1.5)`` (Pareto, alpha = 1.5);
* loop 0: h ~ N(0,1); loop 1: Q, K, V ~ N(0,1), h = h0 + sigma*eps;
* loop l >= 2: ``X_l = X_{l-1} + sigma_i * 0.7^(l-1) * eps`` for X in {h,Q,K,V};
* planted heavy keys: a seeded unit vector u per (sequence, head); every query
  gets ``+8u`` and every heavy key ``+(sqrt(d)/2)u`` (an expected logit boost
  of +4), at seeded positions that stay fixed across loops;
* every value is rounded to the working dtype (bf16 round-to-nearest-even, or
  fp32) after each loop, and returned as float32 arrays holding those values.

Shapes: h [n_seq, N, H*d]; q, k, v [n_seq, N, H, d].  Decode workloads carry
the new token's rows only for h and q (N = 1: its hidden state, which the
early-exit test reads, and its query).
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Iterator, Optional, Tuple

import numpy as np

from .configs import Workload

_T_H, _T_Q, _T_K, _T_V = 0, 1, 2, 3
_SIGMA, _HEAVY, _UVEC, _DENSITY = 100, 101, 102, 103


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); float32 out."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-representable."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *key])))


def _workers() -> int:
    return max(1, min(16, len(__import__("os").sched_getaffinity(0))))


class SyntheticLoops:
    """Iterates the per-loop inputs of one workload.

    ``loop(l)`` must be called with l = 0, 1, 2, ... in order; it returns a
    dict of float32 arrays that stay valid until the next call (copy what you
    keep).
    """

    def __init__(self, wl: Workload, seqs: Optional[Tuple[int, ...]] = None):
        self.wl = wl
        self.seqs = tuple(range(wl.n_seq)) if seqs is None else tuple(seqs)
        n, h, d = wl.n_tokens, wl.n_heads, wl.head_dim
        self.sigma = np.stack([self._sigma(s) for s in self.seqs])            # [S, N]
        self.heavy = [self._heavy(s) for s in self.seqs]                      # S x [n_heavy]
        self.uvec = np.stack([self._uvec(s) for s in self.seqs])              # [S, H, d]
        self._state: Dict[str, np.ndarray] = {}
        self._next = 0
        nq = 1 if wl.decode else n        # decode: the new token's rows only
        self.shapes = {"h": (nq, h * d), "q": (nq, h, d), "k": (n, h, d), "v": (n, h, d)}

    # -- per-sequence constants ------------------------------------------------
    def _sigma(self, s: int) -> np.ndarray:
        g = _rng(self.wl.seed, s, _SIGMA)
        n = self.wl.n_tokens
        if self.wl.sigma_model == "pareto":
            u = g.random(n)
            return (0.05 * (1.0 - u) ** (-1.0 / 1.5)).astype(np.float32)
        return (0.1 * np.exp(g.standard_normal(n))).astype(np.float32)

    def _heavy(self, s: int) -> np.ndarray:
        if self.wl.n_heavy == 0:
            return np.zeros(0, np.int64)
        g = _rng(self.wl.seed, s, _HEAVY)
        return np.sort(g.choice(self.wl.n_tokens, size=self.wl.n_heavy, replace=False))

    def _uvec(self, s: int) -> np.ndarray:
        g = _rng(self.wl.seed, s, _UVEC)
        u = g.standard_normal((self.wl.n_heads, self.wl.head_dim))
        return (u / np.linalg.norm(u, axis=1, keepdims=True)).astype(np.float32)

    def context_active_sets(self, layer: int) -> list:
        """Decode workloads: stored-context positions that hold a delta at ``layer``.

        Layer density None means every context position (0..N-2); otherwise the
        top positions by sigma (ties to the lower index), listed ascending, so
        equal counts give nested (identical) sets.
        """
        cnt = self.wl.context_active[layer - 2]
        n_ctx = self.wl.n_tokens - 1
        out = []
        for i in range(len(self.seqs)):
            if cnt is None:
                out.append(np.arange(n_ctx, dtype=np.int32))
            else:
                sig = self.sigma[i, :n_ctx]
                order = np.lexsort((np.arange(n_ctx), -sig))
                out.append(np.sort(order[:cnt]).astype(np.int32))
        return out

    # -- trajectories ------------------------------------------------------------
    def _round(self, x: np.ndarray) -> np.ndarray:
        return round_bf16(x) if self.wl.dtype == "bf16" else x.astype(np.float32)

    def _draw(self, si: int, loop: int, name: str) -> np.ndarray:
        s = self.seqs[si]
        tid = {"h": _T_H, "q": _T_Q, "k": _T_K, "v": _T_V}[name]
        g = _rng(self.wl.seed, s, loop, tid)
        return g.standard_normal(self.shapes[name], dtype=np.float32)

    def _first(self, si: int, name: str) -> np.ndarray:
        wl = self.wl
        x = self._draw(si, 1, name)
        if name == "q":
            x += np.float32(8.0) * self.uvec[si][None]
        elif name == "k" and wl.n_heavy:
            x[self.heavy[si]] += np.float32(math.sqrt(wl.head_dim) / 2.0) * self.uvec[si][None]
        return self._round(x)

    def _step(self, si: int, loop: int, name: str, prev: np.ndarray) -> np.ndarray:
        eps = self._draw(si, loop, name)
        sig = self.sigma[si]
        if name in ("q", "h") and self.wl.decode:
            sig = sig[-1:]
        scale = (sig * np.float32(0.7 ** (loop - 1))).astype(np.float32)
        shape = (-1,) + (1,) * (eps.ndim - 1)
        return self._round(prev + scale.reshape(shape) * eps)

    def names(self, loop: int):
        if loop == 0:
            return ("h",)
        return ("h", "q", "k", "v")

    def loop(self, l: int) -> Dict[str, np.ndarray]:
        if l != self._next:
            raise ValueError(f"loops must be drawn in order: expected {self._next}, got {l}")
        self._next += 1
        jobs = []
        for name in self.names(l):
            if name not in self._state:
                self._state[name] = np.empty((len(self.seqs),) + self.shapes[name], np.float32)
            for si in range(len(self.seqs)):
                jobs.append((name, si))

        def run(job):
            name, si = job
            st = self._state[name]
            if l == 0:
                st[si] = self._draw(si, 0, "h")
                st[si] = self._round(st[si])
            elif l == 1 and name != "h":
                st[si] = self._first(si, name)
            else:
                st[si] = self._step(si, l, name, st[si])

        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(run, jobs))
        return {name: self._state[name] for name in self.names(l)}

    def __iter__(self) -> Iterator[Tuple[int, Dict[str, np.ndarray]]]:
        for l in range(0, self.wl.n_loops + 1):
            yield l, self.loop(l)
