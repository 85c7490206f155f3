"""CPU float64 oracle of the draft distribution over a node's candidates.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: used by ``tests/``
and never by the library, with which it shares no code.

What it computes follows two passages of "EAGLE-4: One Flexible Drafter for
All Batch Sizes and Hardware" and one of "EAGLE-4 Triples Qwen3 Inference
Speed by Adapting to Serving Load":

* section "Retrieve vocabulary candidates cheaply, then score them exactly":
  the low-rank stage only selects candidates; the probabilities come from
  the exact logits of the full-rank head;
* section "Why a draft tree needs a cost model": products of draft
  probabilities along a path approximate the benefit of drafting it;
* "EAGLE-4 Triples Qwen3 ...", section "Runtime-sized speculation": a
  top-k of 1 makes the speculation a chain, larger values a tree of
  continuations.

Written out, for one tree node (one draft row) with candidates (id_j, l_j),
j < k, and the path probability p_parent of the node:

  D1  p_j = exp(l_j - m) / sum_i exp(l_i - m),  m = max_i l_i, over the
      candidates that exist (a NaN logit marks an empty candidate slot and
      gets p = 0);
  D2  the branches: the nb candidates of highest p_j, in order, equal
      probabilities going to the lower token id;
  D3  each branch's path probability p_parent * p_j.

Readings (listed in the design notes): the normaliser runs over the k
candidates only, because the full-vocabulary normaliser would need all V
exact logits, which is the cost the method avoids; no temperature (the pages
name none). Parity: D1-D3 are pinned by closed forms in
``tests/test_oracle_pins.py`` (uniform logits, logits log(1..k), shift
invariance, empty slots, nb = 1 and nb = k).
"""
from __future__ import annotations

import numpy as np


def draft_distribution(logits: np.ndarray) -> np.ndarray:
    """D1 for each row of a (B, k) logit array: float64 probabilities."""
    l64 = np.asarray(logits, dtype=np.float64)
    valid = ~np.isnan(l64)
    m = np.max(np.where(valid, l64, -np.inf), axis=1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.where(valid, np.exp(np.where(valid, l64, 0.0) - m), 0.0)
    s = e.sum(axis=1, keepdims=True)
    return np.divide(e, s, out=np.zeros_like(e), where=s > 0)


def branch_order(p_row: np.ndarray, id_row: np.ndarray) -> np.ndarray:
    """D2 for one row: candidate positions by decreasing p, then lower id."""
    return np.lexsort((np.asarray(id_row, dtype=np.int64), -np.asarray(p_row, dtype=np.float64)))


def branches(logits: np.ndarray, idx: np.ndarray, nb: int, parent: np.ndarray | None = None):
    """D1-D3 for (B, k) logits and ids: (probs, branch ids, branch probs,
    branch path probs); ranks past the existing candidates hold id -1 and 0."""
    p = draft_distribution(logits)
    B, k = p.shape
    par = np.ones(B) if parent is None else np.asarray(parent, dtype=np.float64)
    br_i = np.full((B, nb), -1, dtype=np.int64)
    br_p = np.zeros((B, nb))
    for b in range(B):
        order = branch_order(p[b], idx[b])
        order = [j for j in order if not np.isnan(logits[b, j])][:nb]
        br_i[b, :len(order)] = np.asarray(idx[b])[order]
        br_p[b, :len(order)] = p[b, order]
    return p, br_i, br_p, br_p * par[:, None]
