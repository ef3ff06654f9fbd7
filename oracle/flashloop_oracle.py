"""Plain, slow CPU oracle of the FlashLoop lazy-update loop step.

TEST INFRASTRUCTURE ONLY: imported by tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the HIP path.  It shares no code with
the HIP library (no kernels, headers, tables or helpers); only the seeded input
generator is common to both sides.

Source ("[FL]"): the page "FlashLoop: Fast and Memory-Efficient Looped
Transformers via Lazy Updates" (rit.work blog).  Its sections are cited as
  [FL/late]    "Later loops change only part of the state"
  [FL/savings] "FlashLoop combines three kinds of savings"
with the paragraph number inside the section (par. 1 = first paragraph).

Precision.  The pages fix none.  Attention, softmax statistics and the
token-change score are evaluated in float64.  The int4 codec and the KV
reconstruction chain are evaluated in float32, because their results decide
integers (the 4-bit codes) and the HIP path takes those decisions in float32;
both sides therefore take the same decision in the same precision.

Readings of points the page leaves open:
  R1 tokens are ranked at loop l by the change of the previous loop,
     ||h_eff^(l-1) - h_eff^(l-2)||^2 (a loop cannot know its own change before
     computing it); squared L2 over the whole hidden row, float64.
  R2 ties in any top-k go to the lower index; results are returned ascending.
  R3 keys are selected per (sequence, head) by the previous loop's column mass
     c_j = sum_{i>=j} p_ij; the causal limit is applied per row.
  R4 mass-corrected attention (the "column update" reading):
        o_i = m_i * otilde_i + (o_prev_i - a_i)
     m_i = previous-loop probability mass of the row on the selected keys,
     a_i = those keys' previous contribution to the row's output,
     otilde_i = softmax over the selected keys with the current Q, K, V.
  R5 previous-loop probabilities are exp(s' - lse_prev), where a lazy loop's
     lse is the implied normaliser M + log Z - log m.
  R6 a row whose selected set (after the causal limit) is empty, or whose mass
     m is 0, keeps o, lse and contributes nothing to c.
  R7 int4 codec: symmetric codes -7..7, one float16 scale per group of 32
     consecutive elements of a head row, s = f16_rne(min(absmax/7, 65504)),
     code = rint(delta/s) clamped to [-7, 7] (0 when s == 0), low nibble =
     even element; delta is taken against the previous reconstruction.
     The workload's delta_bits (2 or 4) and group (32 or 64) generalise it:
     codes -q..q with q = 2^(bits-1) - 1, s from absmax/q; 2-bit codes sit
     four to a byte, lowest bits first (variant V3, lower-bit deltas and
     larger groups, [FL/savings] par. 3).
  R8 loop 1 stores the base (working dtype); every later loop, full or lazy,
     appends one delta layer holding records of that loop's active tokens.
  R9 all attention reads the reconstructed K^, V^ of every key, in the
     working dtype of the workload: the float32 reconstruction is rounded to
     bfloat16 (nearest-even) for bf16 workloads, as the version-1 base already
     is; queries are used as given.  The int4 chain itself (R7, R8) stays in
     float32.
Variants (off by default):
  V1 formula="mixture", the other grammatical reading of keeping the group's
     mass:  o_i = m_i * otilde_i + (1 - m_i) * o_prev_i  (no previous-loop
     contribution a_i is needed).  The page gives no statistics for it; lse
     and the column mass are updated exactly as under R4 (the selected
     group's part of the row: lse = M + log Z - log m, c_j += p_ij - p'_ij on
     the selected keys), so only the output formula differs.
  V2 freeze_keys=True: the keys chosen for the first lazy loop are reused by
     every later lazy loop ([FL/late] par. 4 calls the group that carries the
     change small and stable) instead of being re-chosen from each loop's
     column mass.
  E1 exit_threshold=tau: early exit per sequence.  The page on looped
     Transformers ("深度解析循环Transformer架构：隐式推理如何重塑大模型算力效率",
     section 四 "开发者实践", item 1 "计算图的动态控制": dynamic loop depth)
     stops iterating once the change of the state between two loops falls
     below a threshold; it fixes neither the measure nor when it is taken.
     Reading: before each lazy loop l the sequence's change is the largest
     token score of R1, max_i ||h_eff^(l-1)_i - h_eff^(l-2)_i||^2 (float64;
     a decode sequence has the new token's row only); if it is < tau the
     sequence runs no further loops and keeps the outputs and store of loop
     l-1.  (The page's sketch also discards the state of the loop that made
     the small change; here that loop's outputs, already computed and within
     tau of the previous ones, are kept.)  Full loops always run.
The page prints no worked example of the mass-corrected formula (R4); it is
pinned by invariants that follow from the mathematics (full attention when
every key is selected, the dense loop when every row and key is, a fixed point
when nothing changed, mass preservation, single-key closed forms) and by a
loop-level evaluation; see tests/test_oracle_attention.py.  The loop driver's
wiring (which hidden states, queries and store versions each lazy loop reads)
is pinned by the same invariants applied to whole runs of run_prefill
(tests/test_oracle_prefill_driver.py) and of the decode driver
(tests/test_oracle_driver.py).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

__all__ = [
    "to_working_dtype", "token_scores", "topk_ascending", "select_keys", "f16_rne", "quantize_groups",
    "dequantize_groups", "pack_int4", "unpack_int4", "pack_codes", "unpack_codes", "KVStore", "full_attention",
    "lazy_attention", "LoopState", "save_state", "load_state", "lazy_loop",
    "run_prefill", "run_prefill_chain", "build_decode_context",
    "run_decode_loops", "run_decode_seq",
]

F32 = np.float32
F64 = np.float64


def to_working_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the workload's dtype (reading R9); float32 out.

    bf16: keep the upper 16 bits of the float32 pattern after adding half an
    ulp of bf16, with ties to the even bf16 pattern (round-to-nearest-even);
    values are finite here.  fp32: unchanged.
    """
    x = np.ascontiguousarray(x, dtype=F32)
    if dtype == "fp32":
        return x
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    rounded = ((bits + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return (rounded & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(F32)


# --------------------------------------------------------------------------- #
# Step 1: token selection  ([FL/savings] par. 1; [FL/late] par. 3)
# --------------------------------------------------------------------------- #
def token_scores(h_cur: np.ndarray, h_prev: np.ndarray) -> np.ndarray:
    """u_i = sum_k (h_cur[i,k] - h_prev[i,k])^2 in float64 (reading R1).

    [FL/savings] par. 1: tokens are ranked by how much their hidden state
    changed; rows that were carried unchanged score exactly 0.
    """
    diff = h_cur.astype(F64) - h_prev.astype(F64)
    return np.einsum("ik,ik->i", diff, diff)


def topk_ascending(scores: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest scores; ties to the lower index; ascending (R2)."""
    scores = np.asarray(scores)
    n = scores.shape[0]
    if not 0 <= k <= n:
        raise ValueError("k out of range")
    if np.isnan(scores).any():
        raise ValueError("NaN score")
    order = np.lexsort((np.arange(n), -scores.astype(F64)))
    return np.sort(order[:k]).astype(np.int32)


def select_keys(colmass: np.ndarray, k: int) -> np.ndarray:
    """Per-head key selection from the previous loop's column mass (R3).

    [FL/savings] par. 2: keys are chosen from the previous loop's attention
    statistics.  colmass [H, N] -> [H, k] ascending int32.
    """
    return np.stack([topk_ascending(colmass[h], k) for h in range(colmass.shape[0])])


# --------------------------------------------------------------------------- #
# Step 4: the int4 delta codec  ([FL/savings] par. 3)
# --------------------------------------------------------------------------- #
def f16_rne(x: np.ndarray) -> np.ndarray:
    """Round float32 to IEEE binary16, nearest-even (numpy's own conversion)."""
    return np.asarray(x, dtype=F32).astype(np.float16)


def quantize_groups(delta: np.ndarray, group: int = 32, bits: int = 4):
    """float32 delta [..., d] -> (codes int8 [..., d], scales float16 [..., d/group]).

    Reading R7 with q = 2^(bits-1) - 1 (7 for the default 4-bit codes, 1 for
    2-bit codes): s = f16_rne(min(absmax/q, 65504)), code = clamp(rint(delta/s),
    -q, q), 0 when s == 0.  All arithmetic in float32 (correctly rounded
    division, rint half-to-even), so the codes are a pure function of the
    float32 delta.
    """
    delta = np.asarray(delta, dtype=F32)
    qmax = (1 << (bits - 1)) - 1
    d = delta.shape[-1]
    g = delta.reshape(delta.shape[:-1] + (d // group, group))
    absmax = np.max(np.abs(g), axis=-1)
    q = np.minimum(absmax / F32(qmax), F32(65504.0))
    scales = f16_rne(q)
    sf = scales.astype(F32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(sf == 0, F32(0), g / np.where(sf == 0, F32(1), sf))
    codes = np.clip(np.rint(ratio), -qmax, qmax).astype(np.int8)
    return codes.reshape(delta.shape), scales


def dequantize_groups(codes: np.ndarray, scales: np.ndarray, group: int = 32) -> np.ndarray:
    """code * float(scale) in float32 (the product is exact)."""
    d = codes.shape[-1]
    c = codes.astype(F32).reshape(codes.shape[:-1] + (d // group, group))
    return (c * scales.astype(F32)[..., None]).reshape(codes.shape)


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """Two's-complement nibbles, low nibble = even element -> uint8 [..., d/2]."""
    c = (codes.astype(np.int16) & 0xF).astype(np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    lo = (packed & 0xF).astype(np.int16)
    hi = (packed >> 4).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def pack_codes(codes: np.ndarray, bits: int = 4) -> np.ndarray:
    """bits-wide two's-complement fields, element e of each byte's run at bit
    bits*(e mod (8/bits)) (lowest bits = first element) -> uint8 [..., d*bits/8]."""
    if bits == 4:
        return pack_int4(codes)
    per = 8 // bits
    c = (codes.astype(np.int16) & ((1 << bits) - 1)).astype(np.uint8)
    out = np.zeros(codes.shape[:-1] + (codes.shape[-1] // per,), np.uint8)
    for e in range(per):
        out |= (c[..., e::per] << (bits * e)).astype(np.uint8)
    return out


def unpack_codes(packed: np.ndarray, bits: int = 4) -> np.ndarray:
    if bits == 4:
        return unpack_int4(packed)
    per = 8 // bits
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * per,), np.int8)
    for e in range(per):
        f = ((packed >> (bits * e)) & ((1 << bits) - 1)).astype(np.int16)
        out[..., e::per] = np.where(f >= (1 << (bits - 1)), f - (1 << bits), f)
    return out


@dataclass
class _Records:
    idx: np.ndarray        # [n] token positions
    codes: np.ndarray      # [n, H, d] int8
    scales: np.ndarray     # [n, H, d/group] float16


class KVStore:
    """One sequence's KV cache: a base plus a chain of int4 delta layers (R8).

    [FL/savings] par. 3: the cache is a compressed base and a sequence of
    compressed corrections; active tokens write a low-bit difference from
    their previous state, inactive tokens write no entry.
    """

    def __init__(self, n_tokens: int, n_heads: int, head_dim: int, group: int = 32, bits: int = 4):
        self.n, self.h, self.d, self.group, self.bits = n_tokens, n_heads, head_dim, group, bits
        self.base = {"k": np.zeros((n_tokens, n_heads, head_dim), F32),
                     "v": np.zeros((n_tokens, n_heads, head_dim), F32)}
        self.layers: Dict[int, Dict[str, List[_Records]]] = {}

    def reconstruct(self, which: str, version: int, tokens: Optional[np.ndarray] = None) -> np.ndarray:
        """X^(version) = float(base) + sum of the token's deltas in layers 2..version,
        accumulated in float32 in increasing layer order."""
        sel = np.arange(self.n) if tokens is None else np.asarray(tokens)
        x = self.base[which][sel].astype(F32).copy()
        pos = np.full(self.n, -1, np.int64)
        pos[sel] = np.arange(sel.shape[0])
        for l in range(2, version + 1):
            for rec in self.layers.get(l, {}).get(which, []):
                rows = pos[rec.idx]
                hit = rows >= 0
                if hit.any():
                    deq = dequantize_groups(rec.codes[hit], rec.scales[hit], self.group)
                    x[rows[hit]] = x[rows[hit]] + deq
        return x

    def commit(self, version: int, idx: np.ndarray, k_new: np.ndarray, v_new: np.ndarray):
        """Write loop ``version``'s K/V rows of tokens ``idx`` (O-1).

        version 1 stores the base; later versions store int4 deltas against the
        version-1 reconstruction of the same tokens.  Returns the records.
        """
        idx = np.asarray(idx, np.int64)
        out = {}
        for which, new in (("k", k_new), ("v", v_new)):
            new = np.asarray(new, F32)
            if version == 1:
                self.base[which][idx] = new
                continue
            prev = self.reconstruct(which, version - 1, idx)
            delta = new - prev                      # float32 subtraction
            codes, scales = quantize_groups(delta, self.group, self.bits)
            rec = _Records(idx.copy(), codes, scales)
            self.layers.setdefault(version, {"k": [], "v": []})[which].append(rec)
            out[which] = rec
        return out

    def bytes_stored(self, base_elem_bytes: int) -> int:
        b = 2 * self.n * self.h * self.d * base_elem_bytes
        for layer in self.layers.values():
            for recs in layer.values():
                for r in recs:
                    b += r.idx.shape[0] * self.h * (self.d // 2 + 2 * (self.d // self.group))
        return b


# --------------------------------------------------------------------------- #
# Step 0 / Step 3: attention
# --------------------------------------------------------------------------- #
def full_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, rows: np.ndarray,
                   chunk: int = 1024):
    """Causal softmax attention of rows ``rows`` over keys 0..i (O-2), float64.

    q [n_rows, H, d] (the queries of ``rows``), k, v [N, H, d].
    Returns o [n_rows, H, d], lse [n_rows, H], colmass [H, N] with
    colmass[h, j] = sum over the given rows i >= j of p_ij.
    """
    rows = np.asarray(rows, np.int64)
    n_rows, n_heads, d = q.shape
    n = k.shape[0]
    scale = 1.0 / math.sqrt(d)
    o = np.zeros((n_rows, n_heads, d), F64)
    lse = np.zeros((n_rows, n_heads), F64)
    colmass = np.zeros((n_heads, n), F64)
    for h in range(n_heads):
        kh = k[:, h, :].astype(F64)
        vh = v[:, h, :].astype(F64)
        for r0 in range(0, n_rows, chunk):
            r1 = min(n_rows, r0 + chunk)
            rr = rows[r0:r1]
            nk = int(rr.max()) + 1          # keys past the last row are masked for all
            s = (q[r0:r1, h, :].astype(F64) @ kh[:nk].T) * scale
            mask = np.arange(nk)[None, :] <= rr[:, None]
            s = np.where(mask, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            z = e.sum(axis=1, keepdims=True)
            l = m + np.log(z)
            p = np.exp(s - l)
            o[r0:r1, h, :] = p @ vh[:nk]
            lse[r0:r1, h] = l[:, 0]
            colmass[h, :nk] += p.sum(axis=0)
    return o, lse, colmass


def lazy_attention(q_cur, q_prev, k_prev, v_prev, k_cur, v_cur, o_prev, lse_prev, colmass_prev,
                   rows: np.ndarray, keys: np.ndarray, chunk: int = 1024, formula: str = "column"):
    """Mass-corrected attention on the selected keys (O-5, readings R4-R6), float64.

    [FL/savings] par. 2: keys are selected from the previous loop's
    statistics; the selected group keeps the previous loop's probability mass
    instead of being renormalised to 1, so the result approximates full
    attention.  [FL/late] par. 4: the change between adjacent loops is carried
    by a small, stable group of keys ("updating 10% of attention columns").

    q_cur, q_prev, o_prev: [n_rows, H, d] for the active rows ``rows``;
    lse_prev [n_rows, H]; k_*, v_* [N, H, d] reconstructions at versions l-1
    and l; colmass_prev [H, N]; keys [H, nS] ascending.  formula "column"
    is R4, "mixture" the variant V1 (module docstring).
    Returns (o [n_rows,H,d], lse [n_rows,H], colmass [H,N], m [n_rows,H],
    updated [n_rows,H] bool).
    """
    if formula not in ("column", "mixture"):
        raise ValueError(f"unknown formula {formula!r}")
    rows = np.asarray(rows, np.int64)
    n_rows, n_heads, d = q_cur.shape
    scale = 1.0 / math.sqrt(d)
    o = np.array(o_prev, F64, copy=True)
    lse = np.array(lse_prev, F64, copy=True)
    colmass = np.array(colmass_prev, F64, copy=True)
    mass = np.zeros((n_rows, n_heads), F64)
    updated = np.zeros((n_rows, n_heads), bool)
    for h in range(n_heads):
        sel = np.asarray(keys[h], np.int64)
        kp = k_prev[sel, h, :].astype(F64)
        vp = v_prev[sel, h, :].astype(F64)
        kc = k_cur[sel, h, :].astype(F64)
        vc = v_cur[sel, h, :].astype(F64)
        dcol = np.zeros(sel.shape[0], F64)
        for r0 in range(0, n_rows, chunk):
            r1 = min(n_rows, r0 + chunk)
            rr = rows[r0:r1]
            mask = sel[None, :] <= rr[:, None]
            # previous loop's probabilities on the selected keys
            sp = (q_prev[r0:r1, h, :].astype(F64) @ kp.T) * scale
            pp = np.exp(np.where(mask, sp - lse_prev[r0:r1, h].astype(F64)[:, None], -np.inf))
            m = pp.sum(axis=1)
            a = pp @ vp
            # current softmax restricted to the selected keys
            sc = np.where(mask, (q_cur[r0:r1, h, :].astype(F64) @ kc.T) * scale, -np.inf)
            any_key = mask.any(axis=1)
            mx = np.where(any_key, sc.max(axis=1), 0.0)
            e = np.where(mask, np.exp(sc - mx[:, None]), 0.0)
            z = e.sum(axis=1)
            ok = any_key & (m > 0)
            zs = np.where(ok, z, 1.0)
            otil = (e @ vc) / zs[:, None]
            op = o_prev[r0:r1, h, :].astype(F64)
            if formula == "column":
                o_new = m[:, None] * otil + (op - a)
            else:
                o_new = m[:, None] * otil + (1.0 - m)[:, None] * op
            lse_new = mx + np.log(zs) - np.log(np.where(ok, m, 1.0))
            p = (m / zs)[:, None] * e
            o[r0:r1, h, :] = np.where(ok[:, None], o_new, o[r0:r1, h, :])
            lse[r0:r1, h] = np.where(ok, lse_new, lse[r0:r1, h])
            dcol += np.where(ok[:, None], p - pp, 0.0).sum(axis=0)
            mass[r0:r1, h] = m
            updated[r0:r1, h] = ok
        colmass[h, sel] += dcol
    return o, lse, colmass, mass, updated


# --------------------------------------------------------------------------- #
# Loop drivers
# --------------------------------------------------------------------------- #
@dataclass
class LoopState:
    """Per-sequence state after a loop (everything carried for inactive rows).

    This is also the checkpoint a run resumes from (``run_prefill(resume=)``,
    ``save_state`` / ``load_state``): every buffer the next loop reads."""
    loop: int
    h: Optional[np.ndarray]        # [N, D] effective hidden state (prefill only)
    q: np.ndarray                  # [Nq, H, d] effective queries
    o: np.ndarray                  # [Nq, H, d] float64
    lse: np.ndarray                # [Nq, H] float64
    colmass: np.ndarray            # [H, N] float64
    store: KVStore
    records: Dict[int, dict] = field(default_factory=dict)   # loop -> details
    exited_at: Optional[int] = None                          # E1: the loop that was not run
    h_prev: Optional[np.ndarray] = None                      # [N, D] h_eff of the loop before (prefill)
    frozen_keys: Optional[np.ndarray] = None                 # V2: the first lazy loop's key group


def _copy_state(st: LoopState) -> LoopState:
    import copy
    return copy.deepcopy(st)


def save_state(st: LoopState, path: str) -> None:
    """Checkpoint of a LoopState as an .npz archive of plain arrays (no pickles)."""
    arrs = {"loop": np.array(st.loop), "o": st.o, "lse": st.lse, "colmass": st.colmass, "q": st.q,
            "store_shape": np.array([st.store.n, st.store.h, st.store.d, st.store.group, st.store.bits]),
            "base_k": st.store.base["k"], "base_v": st.store.base["v"]}
    for name in ("h", "h_prev", "frozen_keys"):
        if getattr(st, name) is not None:
            arrs[name] = getattr(st, name)
    for l, layer in st.store.layers.items():
        for which, recs in layer.items():
            for r, rec in enumerate(recs):
                for part in ("idx", "codes", "scales"):
                    arrs[f"layer{l}_{which}_{r}_{part}"] = getattr(rec, part)
    np.savez(path, **arrs)


def load_state(path: str) -> LoopState:
    """Inverse of save_state (records and exit information are not kept)."""
    z = np.load(path, allow_pickle=False)
    n, H, d, group, bits = (int(v) for v in z["store_shape"])
    store = KVStore(n, H, d, group, bits)
    store.base["k"][...] = z["base_k"]
    store.base["v"][...] = z["base_v"]
    layers: Dict[int, Dict[str, Dict[int, dict]]] = {}
    for key in z.files:
        if key.startswith("layer"):
            head, which, r, part = key.split("_")
            layers.setdefault(int(head[5:]), {}).setdefault(which, {}).setdefault(int(r), {})[part] = z[key]
    for l in sorted(layers):
        store.layers[l] = {w: [_Records(recs[r]["idx"], recs[r]["codes"], recs[r]["scales"]) for r in sorted(recs)]
                           for w, recs in layers[l].items()}
    get = lambda name: z[name] if name in z.files else None
    return LoopState(int(z["loop"]), get("h"), z["q"], z["o"], z["lse"], z["colmass"], store,
                     h_prev=get("h_prev"), frozen_keys=get("frozen_keys"))


def lazy_loop(wl, st: LoopState, x: dict, l: int, seq: int = 0, formula: str = "column",
              keys: Optional[np.ndarray] = None, operand_dtype: Optional[str] = None):
    """One lazy loop l on the state ``st`` after loop l-1, in place ([FL/savings]
    par. 1-3).  Steps, in the page's order: rank the tokens by the change their
    hidden state made in loop l-1 and keep the top n_active (R1); choose each
    head's keys from loop l-1's column mass (R3) unless ``keys`` is given; the
    shared block recomputes only the active rows (the others carry h, Q, o, lse);
    the active tokens write their K/V differences as layer l (R8); then
    mass-corrected attention of the active rows on the selected keys (R4-R6),
    whose previous-loop part uses the active rows' loop-(l-1) queries and the
    store at version l-1, and whose current part uses their loop-l queries and
    version l.  ``operand_dtype`` overrides the dtype attention's K^, V^ are
    rounded to (R9; "fp32" keeps the float32 reconstruction, to measure what
    the rounding costs).  Returns the loop's record (rows, keys, scores, mass, ...)."""
    od = wl.dtype if operand_dtype is None else operand_dtype
    u = token_scores(st.h, st.h_prev)
    rows = topk_ascending(u, wl.n_active(l))
    if keys is None:
        keys = select_keys(st.colmass, wl.n_keys)
    # the shared block recomputes only the active rows; others carry
    st.h_prev = st.h.copy()
    st.h[rows] = x["h"][seq][rows]
    q_prev_rows = st.q[rows].copy()
    st.q[rows] = x["q"][seq][rows]
    k_prev_hat = to_working_dtype(st.store.reconstruct("k", l - 1), od)
    v_prev_hat = to_working_dtype(st.store.reconstruct("v", l - 1), od)
    recs = st.store.commit(l, rows, x["k"][seq][rows], x["v"][seq][rows])
    k_hat = to_working_dtype(st.store.reconstruct("k", l), od)
    v_hat = to_working_dtype(st.store.reconstruct("v", l), od)
    o_r, lse_r, st.colmass, m, upd = lazy_attention(
        st.q[rows], q_prev_rows, k_prev_hat, v_prev_hat, k_hat, v_hat,
        st.o[rows], st.lse[rows], st.colmass, rows, keys, formula=formula)
    st.o[rows] = o_r
    st.lse[rows] = lse_r
    st.loop = l
    return dict(rows=rows, keys=keys, scores=u, mass=m, updated=upd, records=recs)


def run_prefill(wl, loops, upto: Optional[int] = None, keep: bool = False, seq: int = 0,
                formula: str = "column", freeze_keys: bool = False, exit_threshold: Optional[float] = None,
                resume: Optional[LoopState] = None, operand_dtype: Optional[str] = None):
    """Run loops 1..T of a prefill workload on one sequence.

    ``loops`` yields (l, dict(h, q, k, v)) with l = 0..T, arrays shaped
    [S, N, ...] (sequence ``seq`` is used); values are already in the
    working dtype.  Early loops run in full; later loops select tokens and
    keys, commit deltas of the active tokens and run mass-corrected attention
    ([FL/savings] par. 1-3).  ``formula`` and ``freeze_keys`` select the
    variants V1 and V2, ``exit_threshold`` the early exit E1 (module
    docstring).  ``resume`` continues from a checkpoint (the state after loop
    resume.loop; ``loops`` may still start at 0, earlier loops are skipped).
    ``operand_dtype`` as in lazy_loop, for full loops too.  Returns the final
    LoopState (and, with keep=True, the list of states after every loop that
    ran).
    """
    n, H, d = wl.n_tokens, wl.n_heads, wl.head_dim
    T = wl.n_loops if upto is None else upto
    history = []
    if resume is None:
        st, start = None, 0
        h0 = None
    else:
        st, start = _copy_state(resume), resume.loop + 1
    for l, x in loops:
        if l > T:
            break
        if l < start:
            continue
        if l == 0:
            h0 = x["h"][seq].copy()
            continue
        rec = {}
        if l <= wl.n_full:
            rows = np.arange(n, dtype=np.int32)
            if st is None:
                st = LoopState(0, h0, None, None, None, None, KVStore(n, H, d, wl.group, wl.delta_bits))
            st.h_prev, st.h = st.h, x["h"][seq].copy()
            st.q = x["q"][seq].copy()
            st.store.commit(l, rows, x["k"][seq], x["v"][seq])
            od = wl.dtype if operand_dtype is None else operand_dtype
            kh = to_working_dtype(st.store.reconstruct("k", l), od)
            vh = to_working_dtype(st.store.reconstruct("v", l), od)
            st.o, st.lse, st.colmass = full_attention(st.q, kh, vh, rows)
            st.loop = l
            rec.update(rows=rows)
        else:
            if exit_threshold is not None and float(np.max(token_scores(st.h, st.h_prev))) < exit_threshold:
                st.exited_at = l                   # E1: loops l.. are not run
                break
            rec = lazy_loop(wl, st, x, l, seq, formula, keys=st.frozen_keys, operand_dtype=operand_dtype)
            if freeze_keys:
                st.frozen_keys = rec["keys"]
        st.records = {l: rec}
        if keep:
            history.append(_copy_state(st))
    return (st, history) if keep else st


def run_prefill_chain(wl, loops, upto: Optional[int] = None, seq: int = 0):
    """Token selection and KV commits of loops 1..upto, without attention.

    Neither step depends on attention ([FL/savings] par. 1 and 3: tokens are
    ranked by their own hidden-state change, and active tokens write their
    K/V difference), so the active sets and the whole base+delta store of a
    large workload are computed here from the inputs alone.  Returns
    (store, active: {loop: rows}, inputs_by_loop: {loop: dict(q, k, v)} of the
    queries/keys/values the loops consumed, h_eff after the last loop).
    """
    n, H, d = wl.n_tokens, wl.n_heads, wl.head_dim
    T = wl.n_loops if upto is None else upto
    store = KVStore(n, H, d, wl.group, wl.delta_bits)
    h_eff = h_prev_eff = None
    active = {}
    for l, x in loops:
        if l > T:
            break
        if l == 0:
            h_eff = x["h"][seq].copy()
            continue
        if l <= wl.n_full:
            rows = np.arange(n, dtype=np.int32)
            h_prev_eff, h_eff = h_eff, x["h"][seq].copy()
        else:
            u = token_scores(h_eff, h_prev_eff)
            rows = topk_ascending(u, wl.n_active(l))
            h_prev_eff = h_eff.copy()
            h_eff[rows] = x["h"][seq][rows]
        store.commit(l, rows, x["k"][seq][rows], x["v"][seq][rows])
        active[l] = rows
    return store, active, h_eff


def build_decode_context(wl, seq_index: int, ctx_sets: Dict[int, np.ndarray], loops_data) -> KVStore:
    """The stored context of one decode sequence (positions 0..N-2): the base
    from loop 1 and one delta layer per later loop for the positions in
    ``ctx_sets[l]`` (O-6's fixed context)."""
    n, H, d = wl.n_tokens, wl.n_heads, wl.head_dim
    si = seq_index
    store = KVStore(n, H, d, wl.group, wl.delta_bits)
    ctx = np.arange(n - 1)
    for l in range(1, wl.n_loops + 1):
        x = loops_data[l]
        sel = ctx if l == 1 else np.asarray(ctx_sets[l], np.int64)
        store.commit(l, sel, x["k"][si][sel], x["v"][si][sel])
    return store


def run_decode_loops(wl, store: KVStore, seq_index: int, loops_data, formula: str = "column",
                     freeze_keys: bool = False, exit_threshold: Optional[float] = None,
                     start: int = 1, upto: Optional[int] = None, state: Optional[dict] = None):
    """The T decode loops of the new token at position N-1 over a built
    context: loop 1 attends in full over version 1, loops l >= 2 select keys
    from that row's column mass, commit the token's own delta and run
    mass-corrected attention over version l (variants V1, V2 and the early
    exit E1 as in run_prefill; E1 reads the new token's hidden state,
    ``loops_data[l]["h"]`` for l = 0..T).  ``start``/``upto`` run loops
    start..upto only; a start > 1 continues from ``state``, the dict that the
    loop before returned (its o, lse, colmass, and keys under V2), with
    ``store`` holding that loop's records.  Returns a list of per-loop dicts,
    one per loop that ran."""
    n = wl.n_tokens
    si = seq_index
    last = np.array([n - 1])
    out = []
    o = lse = colmass = None
    q_prev = None
    frozen = None
    if start > 1:
        o, lse, colmass = (np.array(state[k], copy=True) for k in ("o", "lse", "colmass"))
        q_prev = loops_data[start - 1]["q"][si].copy()
        if freeze_keys and start > 2:
            frozen = state["keys"]
    for l in range(start, (wl.n_loops if upto is None else upto) + 1):
        x = loops_data[l]
        q = x["q"][si]                       # [1, H, d]
        if l >= 2 and exit_threshold is not None:
            u = token_scores(loops_data[l - 1]["h"][si], loops_data[l - 2]["h"][si])
            if float(np.max(u)) < exit_threshold:
                break                              # E1: loops l.. are not run
        store.commit(l, last, x["k"][si][last], x["v"][si][last])
        if l == 1:
            kh = to_working_dtype(store.reconstruct("k", 1), wl.dtype)
            vh = to_working_dtype(store.reconstruct("v", 1), wl.dtype)
            o, lse, colmass = full_attention(q, kh, vh, last)
            out.append(dict(o=o.copy(), lse=lse.copy(), colmass=colmass.copy()))
        else:
            keys = frozen if frozen is not None else select_keys(colmass, wl.n_keys)
            if freeze_keys:
                frozen = keys
            kp = to_working_dtype(store.reconstruct("k", l - 1), wl.dtype)
            vp = to_working_dtype(store.reconstruct("v", l - 1), wl.dtype)
            kc = to_working_dtype(store.reconstruct("k", l), wl.dtype)
            vc = to_working_dtype(store.reconstruct("v", l), wl.dtype)
            o, lse, colmass, m, upd = lazy_attention(q, q_prev, kp, vp, kc, vc, o, lse, colmass,
                                                     last, keys, formula=formula)
            out.append(dict(o=o.copy(), lse=lse.copy(), colmass=colmass.copy(), keys=keys, mass=m))
        q_prev = q.copy()
    return out


def run_decode_seq(wl, inputs, seq_index: int, ctx_sets: Dict[int, np.ndarray], loops_data,
                   formula: str = "column", freeze_keys: bool = False, exit_threshold: Optional[float] = None):
    """Decode workload, one sequence (O-6): the stored context, then the T
    loops of the new token.  ``loops_data[l]`` holds dict(h [S,1,H*d],
    q [S,1,H,d], k [S,N,H,d], v [S,N,H,d]) (l = 0: h only).  Returns
    (per-loop dicts, store)."""
    store = build_decode_context(wl, seq_index, ctx_sets, loops_data)
    return run_decode_loops(wl, store, seq_index, loops_data, formula, freeze_keys, exit_threshold), store
