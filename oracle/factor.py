"""CPU float64 oracle of building the low-rank head (P, Q) from W.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: used by ``tests/``
and never by the library, with which it shares no code.

The pages say the drafter's token prediction is factored into smaller
matrices ("EAGLE-4 Triples Qwen3 Inference Speed by Adapting to Serving
Load", section "Runtime-sized speculation", item "Low-rank candidate head")
and that the low-rank head retrieves candidates for the original full-rank
head ("EAGLE-4: One Flexible Drafter for All Batch Sizes and Hardware",
section "Retrieve vocabulary candidates cheaply, then score them exactly"),
but not how the factors are obtained. Reading R19: they come from W itself
by a randomized range finder with subspace iteration (the standard
randomized low-rank approximation of Halko, Martinsson and Tropp, 2011,
their algorithm for subspace iteration), written here in their steps:

  F1  Y = W . Omega                      (Omega: d x r Gaussian, an input)
  F2  Y = orth(Y)
  F3  q times:  Z = orth(W^T . Y);  Y = orth(W . Z)
  F4  P = Y (V x r, orthonormal columns),  Q = Y^T . W (r x d)

so that P . Q = Y Y^T W, the projection of W onto the captured column
space; with W of rank r exactly, P . Q = W. orth() is CholeskyQR2: the Gram
matrix G = X^T X, its Cholesky factor G = R^T R, X <- X R^-1, done twice
(the second pass restores orthogonality lost to rounding in the first).
Library primitives used as steps: numpy.matmul, numpy.linalg.cholesky and a
triangular solve. The last step rounds P and Q to the weight dtype (RNE).

Parity: pinned in ``tests/test_oracle_pins.py`` by an exactly rank-r W
(P . Q = W), orthonormal P, and the Eckart-Young optimum from
numpy.linalg.svd on matrices with a known spectrum (the error approaches
the optimum as q grows).
"""
from __future__ import annotations

import numpy as np

from .lowrank_head import round_weight_dtype, to_f64


def orth(X: np.ndarray) -> np.ndarray:
    """CholeskyQR2 of a tall matrix (float64): orthonormal columns spanning X."""
    for _ in range(2):
        G = X.T @ X
        L = np.linalg.cholesky(G)               # G = L L^T, R = L^T
        X = np.linalg.solve(L, X.T).T           # X R^-1 = (L^-1 X^T)^T
    return X


def range_finder(W64: np.ndarray, omega: np.ndarray, q: int) -> np.ndarray:
    """F1-F3: the orthonormal basis Y (V x r)."""
    Y = orth(W64 @ np.asarray(omega, dtype=np.float64))
    for _ in range(q):
        Z = orth(W64.T @ Y)
        Y = orth(W64 @ Z)
    return Y


def factor(W: np.ndarray, omega: np.ndarray, q: int, dtype: str, round_out: bool = True):
    """F1-F4 on stored W (bf16 bit patterns or fp32): (P, Q), float64 values,
    rounded to the weight dtype unless round_out is False."""
    W64 = to_f64(W, dtype)
    Y = range_finder(W64, omega, q)
    P, Q = Y, Y.T @ W64
    if round_out:
        P, Q = round_weight_dtype(P, dtype), round_weight_dtype(Q, dtype)
    return P, Q
