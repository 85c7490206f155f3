"""CPU float64 oracle of the low-rank draft LM head (test infrastructure).

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or runs
this module: it is used by ``tests/``, by ``__graft_entry__.smoke()`` and by
the ``cpu_baseline`` leg of ``bench.py``. It shares no code with the HIP
library; both take their inputs from the ``gen`` module.

What it computes follows "EAGLE-4" (yuxiaoba.github.io/tech/en/eagle-4),
section "Retrieve vocabulary candidates cheaply, then score them exactly":
every token of the vocabulary is first ranked with a cheap rank-r
factorisation of the head, the k best ranked tokens are kept, and the
original head's weights then give those k tokens, and no others, their exact
logits. The alphasignal news page (section "Runtime-sized speculation", item
"Low-rank candidate head") describes the same head as a factorisation of the
token prediction into two smaller matrices. Written out, for each draft row b:

  O1  z_b  = Q . h_b                      (rank r), stored in the weight dtype
  O2  s_b[v] = P[v, :] . z_b              for every vocabulary row v
  O3  C_b = the first k rows of the vocabulary under the total order
        u < v  <=>  s[u] > s[v]  or  (s[u] == s[v] and u < v)
  O4  logit_b[j] = W[C_b[j], :] . h_b     (exact, full rank)
  O5  (baseline, the full head the method replaces) L_b = W . h_b over all
        rows, and its first k rows under the same order.

Every dot product is taken in float64 over the exact values of the stored
(bf16 or fp32) inputs. Library primitives used as steps: ``numpy.matmul`` for
the dot products and a stable ``numpy.argsort`` for the order of O3.

Readings of points the pages leave open (each is listed with its reason in
the design notes of the repository):

* z is materialised in the weight dtype: the float64 sum is rounded to fp32
  and then, for bf16 weights, to bf16 (both round-to-nearest-even), because
  the second contraction multiplies stored z by stored P.
* no bias, softmax, temperature or scaling in either stage: the low-rank
  stage only selects candidates.
* each row is an independent selection; ties in score go to the lower index.
* the tolerance band of the comparison rule uses tau_b = 1e-3 * max_v |s_b[v]|.

Parity status: O1-O5 are pinned by the tests in ``tests/test_oracle_pins.py``
(exact factorisation r = d, brute force over all subsets on tiny vocabularies,
k = 1 / k = V special cases, scaling and permutation invariants, hand-worked
rounding cases, and torch's bf16 conversion). The pages print no numeric
example for the head, so no pin comes from the pages' own values.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "to_f64", "round_fp32", "round_bf16", "round_weight_dtype",
    "down_projection", "vocab_scores", "topk_order", "selection_stats",
    "exact_logits", "lowrank_head", "full_head", "ROW_CHUNK",
]

ROW_CHUNK = 64          # rows of scores held at once (memory only)
VOCAB_CHUNK = 8192      # vocabulary rows of W widened to float64 at once


# ----------------------------------------------------------------- values

def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of stored bf16 bit patterns or fp32 numbers."""
    if dtype == "bf16":
        assert a.dtype == np.uint16, a.dtype
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "fp32":
        assert a.dtype == np.float32, a.dtype
        return a.astype(np.float64)
    if dtype == "fp64":
        return np.asarray(a, dtype=np.float64)
    raise ValueError(dtype)


def round_fp32(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest fp32 (ties to even), as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32-representable values to the nearest bf16 (ties to even).

    bf16 is the top half of an fp32 word: add 0x7FFF plus the lowest kept
    bit, then clear the low 16 bits.
    """
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    assert np.array_equal(f.astype(np.float64), np.asarray(x, dtype=np.float64)), \
        "round_bf16 expects fp32-representable input"
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) & np.uint64(0xFFFF0000)
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def round_weight_dtype(z: np.ndarray, dtype: str) -> np.ndarray:
    """Store a float64 sum the way the head stores z: fp32, then bf16."""
    if dtype == "fp64":
        return np.asarray(z, dtype=np.float64)
    z32 = round_fp32(z)
    return round_bf16(z32) if dtype == "bf16" else z32


# ------------------------------------------------------------ the method

def down_projection(Q64: np.ndarray, H64: np.ndarray, dtype: str) -> np.ndarray:
    """O1: z_b = Q . h_b for every row, stored in the weight dtype.

    Q64 is r x d, H64 is B x d (float64 values); returns B x r.
    """
    z = H64 @ Q64.T
    return round_weight_dtype(z, dtype)


def vocab_scores(P64: np.ndarray, zt: np.ndarray) -> np.ndarray:
    """O2: s_b[v] = P[v, :] . z_b for every vocabulary row (B x V, float64)."""
    return zt @ P64.T


def topk_order(s_row: np.ndarray, k: int) -> np.ndarray:
    """O3: the first k vocabulary rows under 'higher score, then lower index'.

    A stable sort of the negated scores keeps equal scores in index order.
    """
    return np.argsort(-s_row, kind="stable")[:k].astype(np.int64)


def selection_stats(s_row: np.ndarray, idx_row: np.ndarray) -> dict:
    """k-th and (k+1)-th scores, their gap and the tolerance band tau."""
    k = len(idx_row)
    s_k = float(s_row[idx_row[-1]])
    if k < s_row.shape[0]:
        rest = np.ones(s_row.shape[0], dtype=bool)
        rest[idx_row] = False
        s_k1 = float(np.max(s_row[rest]))
    else:
        s_k1 = -np.inf
    tau = 1e-3 * float(np.max(np.abs(s_row)))
    return {"s_k": s_k, "s_k1": s_k1, "gap": s_k - s_k1, "tau": tau}


def exact_logits(W: np.ndarray, H64: np.ndarray, rows: np.ndarray,
                 vocab: np.ndarray, dtype: str) -> np.ndarray:
    """O4: W[v, :] . h_b in float64 for paired (row, vocab) indices."""
    rows = np.asarray(rows, dtype=np.int64)
    vocab = np.asarray(vocab, dtype=np.int64)
    Wv = to_f64(W[vocab.ravel()], dtype).reshape(vocab.shape + (W.shape[1],))
    Hb = H64[rows.ravel()].reshape(rows.shape + (H64.shape[1],))
    return np.sum(Wv * Hb, axis=-1)


def lowrank_head(Q: np.ndarray, P: np.ndarray, W: np.ndarray | None,
                 H: np.ndarray, k: int, dtype: str,
                 rows: np.ndarray | None = None,
                 keep_scores: bool = False) -> dict:
    """O1-O4 over the given rows of H (all rows by default).

    Returns ``idx`` (n x k, int64), ``score`` (n x k), ``logits`` (n x k, or
    None when W is None), per-row ``gap`` / ``tau`` / ``s_k`` / ``s_k1``,
    ``z`` (n x r) and, with ``keep_scores``, the full ``s`` (n x V).
    """
    rows = np.arange(H.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    Q64 = to_f64(Q, dtype)
    P64 = to_f64(P, dtype)
    H64 = to_f64(H[rows], dtype)
    n = len(rows)
    out = {"rows": rows, "idx": np.empty((n, k), np.int64),
           "score": np.empty((n, k)), "gap": np.empty(n), "tau": np.empty(n),
           "s_k": np.empty(n), "s_k1": np.empty(n)}
    zt = down_projection(Q64, H64, dtype)
    out["z"] = zt
    if keep_scores:
        out["s"] = np.empty((n, P64.shape[0]))
    for lo in range(0, n, ROW_CHUNK):
        hi = min(n, lo + ROW_CHUNK)
        s = vocab_scores(P64, zt[lo:hi])
        for i in range(hi - lo):
            idx = topk_order(s[i], k)
            st = selection_stats(s[i], idx)
            out["idx"][lo + i] = idx
            out["score"][lo + i] = s[i][idx]
            for key in ("gap", "tau", "s_k", "s_k1"):
                out[key][lo + i] = st[key]
        if keep_scores:
            out["s"][lo:hi] = s
    if W is not None:
        rr = np.repeat(np.arange(n)[:, None], k, axis=1)
        out["logits"] = exact_logits(W, H64, rr, out["idx"], dtype)
    else:
        out["logits"] = None
    return out


def full_head(W: np.ndarray, H: np.ndarray, k: int, dtype: str,
              rows: np.ndarray | None = None, keep_logits: bool = False) -> dict:
    """O5: dense logits W . h_b over all V, then the first k under the order.

    W is widened to float64 a block of vocabulary rows at a time (memory
    only; each logit is still one float64 dot product).
    """
    rows = np.arange(H.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    H64 = to_f64(H[rows], dtype)
    V = W.shape[0]
    L = np.empty((len(rows), V))
    for lo in range(0, V, VOCAB_CHUNK):
        hi = min(V, lo + VOCAB_CHUNK)
        L[:, lo:hi] = H64 @ to_f64(W[lo:hi], dtype).T
    n = len(rows)
    out = {"rows": rows, "idx": np.empty((n, k), np.int64), "logits": np.empty((n, k)),
           "gap": np.empty(n), "tau": np.empty(n), "s_k": np.empty(n), "s_k1": np.empty(n)}
    for i in range(n):
        idx = topk_order(L[i], k)
        st = selection_stats(L[i], idx)
        out["idx"][i] = idx
        out["logits"][i] = L[i][idx]
        for key in ("gap", "tau", "s_k", "s_k1"):
            out[key][i] = st[key]
    if keep_logits:
        out["L"] = L
    return out
