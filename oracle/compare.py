"""Comparison rule between a device result and the float64 oracle.

TEST INFRASTRUCTURE ONLY (used by ``tests/``, ``__graft_entry__.smoke()``).

The EAGLE-4 page (yuxiaoba.github.io, section "Reading correctness marks
alongside speed") separates exact token agreement from near-tie numerical
choices, and says floating-point order may swap nearly tied logits only under
an explicit tolerance. The explicit tolerance used here, per draft row b:

  tau_b = 1e-3 * max_v |s_b[v]|       (s = oracle scores of that stage)
  gap_b = s_(k) - s_(k+1)             (k-th minus (k+1)-th oracle score)

Rule 1 (gap_b > tau_b): the device returns exactly the oracle's set.
Rule 2 (gap_b <= tau_b, boundary tie band): k distinct ids in [0, V); every
        id scoring above s_(k) + tau_b is present; every returned id scores
        at least s_(k) - tau_b.
Order:  consecutive device ids follow the oracle's order (higher score, then
        lower index) unless their oracle scores are within tau_b.
Logits: |got - exact| <= rtol * max(|exact|, 1e-2 * max_j |exact_j|), with
        rtol = 2e-3 for bf16 and 1e-5 for fp32, exact = the oracle's
        full-rank logit at the *device's* id.
Scores: (diagnostic) |got - s[id]| <= f * max_v |s[v]| + a_id, f = 1e-4
        (bf16) or 1e-6 (fp32), where a_id allows one bf16 step of one
        component of z: the stored z is the fp32 accumulator rounded to
        bf16, and when the exact z_j lies within the accumulator's own
        rounding error of a bf16 midpoint, an accumulation order other than
        the oracle's exact-then-round may land on the neighbouring bf16
        value. a_id = max_j |P[id, j]| * ulp_bf16(z_j) (0 for fp32 heads,
        whose z is not rounded to bf16). Such a step moves scores by far
        less than tau, so the index rules are unaffected.
"""
from __future__ import annotations

import numpy as np

LOGIT_RTOL = {"bf16": 2e-3, "fp32": 1e-5}
SCORE_TOL = {"bf16": 1e-4, "fp32": 1e-6}


def check_candidates(got_idx, s_row: np.ndarray, oracle_idx, tau: float,
                     gap: float, s_k: float) -> list[str]:
    """Index rule for one row; returns a list of violations (empty = pass)."""
    errs: list[str] = []
    k = len(oracle_idx)
    V = s_row.shape[0]
    g = np.asarray(got_idx, dtype=np.int64).ravel()
    if g.shape[0] != k:
        return [f"expected {k} ids, got {g.shape[0]}"]
    if np.any(g < 0) or np.any(g >= V):
        return [f"id out of range [0, {V}): {g[(g < 0) | (g >= V)][:4]}"]
    if len(set(g.tolist())) != k:
        return ["duplicate ids"]
    if gap > tau:
        if set(g.tolist()) != set(np.asarray(oracle_idx).tolist()):
            extra = sorted(set(g.tolist()) - set(np.asarray(oracle_idx).tolist()))
            miss = sorted(set(np.asarray(oracle_idx).tolist()) - set(g.tolist()))
            errs.append(f"set differs outside the tie band (gap {gap:.3g} > tau {tau:.3g}):"
                        f" extra {extra[:4]} missing {miss[:4]}")
    else:
        must = np.nonzero(s_row > s_k + tau)[0]
        missing = sorted(set(must.tolist()) - set(g.tolist()))
        if missing:
            errs.append(f"ids above s_k + tau missing: {missing[:4]}")
        low = g[s_row[g] < s_k - tau]
        if low.size:
            errs.append(f"ids below s_k - tau returned: {low[:4]}")
    sg = s_row[g]
    for j in range(k - 1):
        a, b = sg[j], sg[j + 1]
        in_order = a > b or (a == b and g[j] < g[j + 1])
        if not in_order and abs(a - b) > tau:
            errs.append(f"order broken at {j}: ids {g[j]},{g[j + 1]} scores {a:.6g},{b:.6g}")
            break
    return errs


def check_logits(got: np.ndarray, exact: np.ndarray, dtype: str) -> list[str]:
    """Logit rule for one row (got and exact aligned with the device ids)."""
    got = np.asarray(got, dtype=np.float64).ravel()
    exact = np.asarray(exact, dtype=np.float64).ravel()
    rtol = LOGIT_RTOL[dtype]
    floor = 1e-2 * float(np.max(np.abs(exact))) if exact.size else 0.0
    bound = rtol * np.maximum(np.abs(exact), floor)
    bad = np.nonzero(~(np.abs(got - exact) <= bound))[0]
    if bad.size:
        j = bad[0]
        return [f"{bad.size} logits off (first at {j}: got {got[j]:.8g}, exact {exact[j]:.8g},"
                f" bound {bound[j]:.3g})"]
    return []


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values (8 significant bits) at |x|; 0 at x == 0."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(x > 0, x, 1.0)))
    return np.where(x > 0, 2.0 ** (e - 7), 0.0)


def z_step_allowance(P_rows: np.ndarray, z_row: np.ndarray, dtype: str) -> np.ndarray:
    """a_id of the score rule for the given rows of P (float64) and the
    oracle's stored z of the draft row: max_j |P[id, j]| * ulp_bf16(z_j)."""
    if dtype != "bf16":
        return np.zeros(P_rows.shape[0])
    return np.max(np.abs(P_rows) * ulp_bf16(z_row)[None, :], axis=1)


def check_scores(got: np.ndarray, s_at: np.ndarray, s_row_absmax: float,
                 dtype: str, allowance: np.ndarray | None = None) -> list[str]:
    """Score diagnostic for one row (`allowance` = a_id per entry)."""
    got = np.asarray(got, dtype=np.float64).ravel()
    tol = SCORE_TOL[dtype] * s_row_absmax
    if allowance is not None:
        tol = tol + np.asarray(allowance, dtype=np.float64).ravel()
    bad = np.nonzero(~(np.abs(got - s_at) <= tol))[0]
    if bad.size:
        j = bad[0]
        return [f"{bad.size} scores off (first at {j}: got {got[j]:.8g}, exact {s_at[j]:.8g})"]
    return []


def band_counts(gap: np.ndarray, tau: np.ndarray) -> dict:
    """How many rows fall under rule 1 and rule 2."""
    inside = int(np.sum(gap <= tau))
    return {"rule1_rows": int(gap.shape[0] - inside), "band_rows": inside}
