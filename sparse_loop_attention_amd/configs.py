"""The five synthetic workloads and their loop schedules.

Source: page "FlashLoop: Fast and Memory-Efficient Looped Transformers via Lazy
Updates" (rit.work blog), section "FlashLoop combines three kinds of savings":
early loops run in full, later loops recompute only an active fraction of the
tokens and attend to a selected fraction of the keys; the KV cache is a base
plus 4-bit corrections.  The pages give no counts, so fractions become counts
here, once, as integers: ``k = ceil(f * n)`` with exact rational arithmetic for
the stated percentages.  Both the HIP path and the oracle receive these ints.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from fractions import Fraction
from typing import List, Optional, Tuple


def ceil_frac(f: Fraction, n: int) -> int:
    """ceil(f*n) with exact rationals (no float rounding at x.0 boundaries)."""
    v = f * n
    return int(-((-v.numerator) // v.denominator))


@dataclass(frozen=True)
class Workload:
    name: str
    n_seq: int              # independent sequences (decode batch), 1 for prefill
    n_heads: int
    head_dim: int
    n_tokens: int           # N: positions per sequence
    dtype: str              # "fp32" | "bf16" (working dtype of h, Q, K, V and the KV base)
    n_loops: int            # T
    n_full: int             # F: loops 1..F run densely
    active: Tuple[int, ...]  # nA for lazy loops F+1..T
    n_keys: int             # nS: selected keys per (sequence, head)
    group: int = 32         # quantisation group of the delta codes (32 or 64)
    delta_bits: int = 4     # bits per delta code (4, or 2)
    seed: int = 0
    n_heavy: int = 0        # planted heavy keys per sequence
    sigma_model: str = "lognormal"   # per-token change scale: "lognormal" | "pareto"
    decode: bool = False
    # decode only: active counts of the stored context's delta layers 2..T
    # (None = dense over the context)
    context_active: Tuple[Optional[int], ...] = field(default_factory=tuple)

    @property
    def hidden(self) -> int:
        return self.n_heads * self.head_dim

    def n_active(self, loop: int) -> int:
        """Active rows at 1-based loop ``loop`` (all rows in full loops)."""
        if loop <= self.n_full:
            return self.n_tokens
        return self.active[loop - self.n_full - 1]

    def layer_caps(self) -> List[int]:
        """Record capacity of each delta layer 2..T (index 0 = layer 2)."""
        caps = []
        for l in range(2, self.n_loops + 1):
            if self.decode:
                ctx = self.context_active[l - 2]
                caps.append((self.n_tokens - 1 if ctx is None else ctx) + 1)
            else:
                caps.append(self.n_active(l))
        return caps


def _c5_active(n: int) -> Tuple[int, ...]:
    # Geometric shrink 30% -> 5% over loops 5..16: f_l = 0.30 * (1/6)^((l-5)/11).
    out = []
    for l in range(5, 17):
        f = 0.30 * (1.0 / 6.0) ** ((l - 5) / 11.0)
        out.append(int(math.ceil(f * n - 1e-9)))
    return tuple(out)


TINY = Workload(
    name="tiny", n_seq=1, n_heads=1, head_dim=64, n_tokens=256, dtype="fp32",
    n_loops=2, n_full=1, active=(ceil_frac(Fraction(1, 4), 256),),
    n_keys=ceil_frac(Fraction(1, 10), 256), seed=1, n_heavy=5)

SINGLE_LAYER = Workload(
    name="single_layer", n_seq=1, n_heads=16, head_dim=128, n_tokens=4096, dtype="bf16",
    n_loops=4, n_full=2, active=(ceil_frac(Fraction(1, 5), 4096),) * 2,
    n_keys=ceil_frac(Fraction(1, 10), 4096), seed=2,
    n_heavy=ceil_frac(Fraction(2, 100), 4096))

LONG_PREFILL = Workload(
    name="long_prefill", n_seq=1, n_heads=16, head_dim=128, n_tokens=32768, dtype="bf16",
    n_loops=4, n_full=1,
    active=tuple(ceil_frac(Fraction(p, 100), 32768) for p in (30, 15, 8)),
    n_keys=ceil_frac(Fraction(1, 10), 32768), seed=3,
    n_heavy=ceil_frac(Fraction(2, 100), 32768))

DECODE = Workload(
    name="decode", n_seq=32, n_heads=16, head_dim=128, n_tokens=8192, dtype="bf16",
    n_loops=4, n_full=1, active=(1, 1, 1),
    n_keys=ceil_frac(Fraction(1, 10), 8192), seed=4,
    n_heavy=ceil_frac(Fraction(2, 100), 8192), decode=True,
    context_active=(None, ceil_frac(Fraction(1, 5), 8191), ceil_frac(Fraction(1, 5), 8191)))

DEEP = Workload(
    name="deep", n_seq=1, n_heads=55, head_dim=96, n_tokens=16384, dtype="bf16",
    n_loops=16, n_full=4, active=_c5_active(16384),
    n_keys=ceil_frac(Fraction(1, 10), 16384), seed=5,
    n_heavy=ceil_frac(Fraction(2, 100), 16384), sigma_model="pareto")

WORKLOADS = {w.name: w for w in (TINY, SINGLE_LAYER, LONG_PREFILL, DECODE, DEEP)}


def scaled(w: Workload, n_tokens: int, n_seq: Optional[int] = None, n_heads: Optional[int] = None) -> Workload:
    """Same workload shape rules at a smaller size (for parity tests).

    Fractions are re-derived from the full-size counts so that schedules keep
    their shape; every count stays >= 1.
    """
    import dataclasses
    frac_a = [Fraction(a, w.n_tokens) for a in w.active]
    act = tuple(max(1, ceil_frac(f, n_tokens)) for f in frac_a) if not w.decode else w.active
    ctx = tuple(None if c is None else max(1, ceil_frac(Fraction(c, w.n_tokens - 1), n_tokens - 1))
                for c in w.context_active)
    return dataclasses.replace(
        w, n_tokens=n_tokens, active=act,
        n_keys=max(1, ceil_frac(Fraction(w.n_keys, w.n_tokens), n_tokens)),
        n_heavy=max(1, ceil_frac(Fraction(w.n_heavy, w.n_tokens), n_tokens)) if w.n_heavy else 0,
        context_active=ctx,
        n_seq=w.n_seq if n_seq is None else n_seq,
        n_heads=w.n_heads if n_heads is None else n_heads)
