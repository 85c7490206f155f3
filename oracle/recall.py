"""Retrieval quality of the low-rank head against the full head (test infrastructure).

TEST INFRASTRUCTURE ONLY: used by ``tests/`` and by the recall sweep of
``bench.py``; never by the library. It shares no code with the HIP path.

"EAGLE-4" (yuxiaoba.github.io/tech/en/eagle-4), section "Retrieve vocabulary
candidates cheaply, then score them exactly": the low-rank stage exists only
to pick the tokens that the full-rank head then scores, so what it costs in
draft quality is the full head's best tokens it fails to pick; the same
section weighs a rank-512 head against a rank-128 one on that trade. The
measure written out, for one draft row:

  F_b  = the first b tokens of the full head (O5 of ``lowrank_head``)
  C_k  = the first k low-rank candidates (O1-O3), in candidate order
  recall(b, k) = |F_b  intersect  C_k| / b

and a table reports its mean over rows. C_k is a prefix of a longer
candidate list: the candidate order is a total order, so the first k of the
k_max best are the k best.

Parity status: pinned in ``tests/test_oracle_pins.py`` by hand-worked
intersections, an exactly factorised head (low-rank scores equal to the
full logits, recall 1 for every k >= b), a head whose low-rank scores are
the full logits negated (recall max(0, k - (V - b)) / b in closed form),
k = V, and monotonicity in k.
"""
from __future__ import annotations

import numpy as np

from .lowrank_head import full_head, lowrank_head

__all__ = ["recall_hits", "recall_table", "recall_sweep"]


def recall_hits(cand_idx: np.ndarray, full_idx: np.ndarray, b: int, k: int) -> np.ndarray:
    """Per row: how many of the first b full-head tokens are among the first k candidates."""
    cand_idx = np.asarray(cand_idx)
    full_idx = np.asarray(full_idx)
    if cand_idx.shape[0] != full_idx.shape[0]:
        raise ValueError("candidate and full-head rows differ")
    if not (1 <= b <= full_idx.shape[1] and 1 <= k <= cand_idx.shape[1]):
        raise ValueError(f"b = {b} or k = {k} outside the lists given")
    return np.array([len(set(full_idx[i, :b].tolist()) & set(cand_idx[i, :k].tolist()))
                     for i in range(cand_idx.shape[0])], dtype=np.int64)


def recall_table(cand_idx: np.ndarray, full_idx: np.ndarray, bs, ks) -> list[dict]:
    """recall(b, k) averaged over rows, for every b in bs and k in ks."""
    out = []
    for b in bs:
        for k in ks:
            hits = recall_hits(cand_idx, full_idx, b, k)
            out.append({"b": int(b), "k": int(k), "recall": float(hits.sum()) / (b * len(hits)),
                        "hits": hits})
    return out


def recall_sweep(Q: np.ndarray, P: np.ndarray, W: np.ndarray, H: np.ndarray, dtype: str,
                 bs, ks, rows: np.ndarray | None = None) -> dict:
    """The oracle's own recall table: its low-rank candidates (k = max ks) and
    its full-head order (b = max bs) over the given rows of H."""
    lo = lowrank_head(Q, P, None, H, max(ks), dtype, rows=rows)
    fu = full_head(W, H, max(bs), dtype, rows=rows)
    return {"cand_idx": lo["idx"], "full_idx": fu["idx"], "lowrank": lo, "full": fu,
            "table": recall_table(lo["idx"], fu["idx"], bs, ks)}
