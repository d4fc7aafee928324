"""Acceptance checks of a computed result against the oracle.

TEST INFRASTRUCTURE (see the package header).

Top-K (per query): the computed row must hold exactly K_eff distinct positions in [0, V)
in its first K_eff slots and -1 after them, and every position in which it differs from the
oracle's set must have an fp32 score within 1e-6 relative of the oracle's K-th score (the
"band").  In strict mode (inputs whose scores are exact in fp32 under any summation order,
or planted ties between bit-identical keys) the sets must be identical.

Attention: max |O - O_ref| within a stated bound (2e-2 for bf16 storage, 1e-5 for the fp32
reference mode), and the log-sum-exp within its own bound when it is returned.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np


@dataclass
class TopkCheck:
    ok: bool
    n_outside_band: int = 0
    n_in_band_diff: int = 0
    msgs: List[str] = field(default_factory=list)


def check_topk_row(got: np.ndarray, ref, strict: bool = False) -> TopkCheck:
    got = np.asarray(got, dtype=np.int64)
    K = got.shape[0]
    k_eff = ref.k_eff
    V = ref.S32.shape[0]
    msgs = []
    head, tail = got[:k_eff], got[k_eff:]
    if np.any(tail != -1):
        msgs.append(f"slots past K_eff={k_eff} are not all -1")
    if np.any(head < 0) or np.any(head >= V):
        msgs.append(f"entries outside [0, {V}): {head[(head < 0) | (head >= V)][:8]}")
        return TopkCheck(False, msgs=msgs)
    if np.unique(head).size != k_eff:
        msgs.append("duplicate positions")
    want = set(ref.idx[:k_eff].tolist())
    have = set(head.tolist())
    diff = np.array(sorted(want ^ have), dtype=np.int64)
    n_out = int((~ref.band[diff]).sum()) if diff.size else 0
    if strict and diff.size:
        msgs.append(f"strict: {diff.size} positions differ, e.g. {diff[:8]}")
    if n_out:
        bad = diff[~ref.band[diff]]
        msgs.append(f"{n_out} differing positions outside the 1e-6 band, e.g. {bad[:8]} "
                    f"scores {ref.S32[bad[:8]]} kth {ref.kth}")
    return TopkCheck(ok=not msgs, n_outside_band=n_out, n_in_band_diff=int(diff.size) - n_out,
                     msgs=msgs)


def check_topk(got: np.ndarray, refs, strict: bool = False) -> TopkCheck:
    """got [T, K] indexed by query id; refs: oracle results of the queries to check."""
    total = TopkCheck(ok=True)
    for ref in refs:
        c = check_topk_row(got[ref.t], ref, strict=strict)
        total.n_outside_band += c.n_outside_band
        total.n_in_band_diff += c.n_in_band_diff
        if not c.ok:
            total.ok = False
            total.msgs += [f"query {ref.t}: {m}" for m in c.msgs]
    return total


@dataclass
class AttnCheck:
    ok: bool
    max_abs: float
    worst: tuple
    rel: float
    lse_max_abs: Optional[float] = None
    msgs: List[str] = field(default_factory=list)


def check_attention(O: np.ndarray, O_ref: np.ndarray, tol: float, lse=None, lse_ref=None,
                    lse_tol: Optional[float] = None) -> AttnCheck:
    O = np.asarray(O, dtype=np.float64)
    O_ref = np.asarray(O_ref, dtype=np.float64)
    d = np.abs(O - O_ref)
    d = np.where(np.isnan(d), np.inf, d)
    worst = np.unravel_index(int(np.argmax(d)), d.shape) if d.size else ()
    mx = float(d.max()) if d.size else 0.0
    scale = float(np.abs(O_ref).max()) if O_ref.size else 0.0
    msgs = []
    if not mx <= tol:
        msgs.append(f"max |O - O_ref| = {mx:.3e} > {tol:.1e} at {worst}")
    lmx = None
    if lse is not None and lse_ref is not None:
        a = np.asarray(lse, dtype=np.float64)
        b = np.asarray(lse_ref, dtype=np.float64)
        both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
        dl = np.where(both_inf, 0.0, np.abs(a - b))
        dl = np.where(np.isnan(dl), np.inf, dl)
        lmx = float(dl.max()) if dl.size else 0.0
        if lse_tol is not None and not lmx <= lse_tol:
            msgs.append(f"max |lse - lse_ref| = {lmx:.3e} > {lse_tol:.1e}")
    return AttnCheck(ok=not msgs, max_abs=mx, worst=tuple(int(i) for i in worst),
                     rel=mx / scale if scale else float("inf"), lse_max_abs=lmx, msgs=msgs)
