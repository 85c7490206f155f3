"""Seeded synthetic inputs for the low-rank draft LM head.

This module only *draws* inputs. It holds none of the head's arithmetic (no
down-projection, no vocabulary scores, no selection, no rescoring): the GPU
library and the CPU oracle both consume the arrays it returns, and neither
imports the other.

Workload shapes (a 27B-class drafter head, V = 151936, d = 5120) and the
structure of the rows (a single draft row, a 64-node draft tree, 256 requests
x 8 draft positions) follow the EAGLE-4 pages: the low-rank candidate head of
"EAGLE-4" (yuxiaoba.github.io, section "Retrieve vocabulary candidates
cheaply, then score them exactly"), the 64-node tree of the drafters-under-load
wiki page (TL;DR, Ling-3 UBTree), and the load levels of the release table.

Generation recipe (the pages fix none of it; these are the readings used):

* Q (r x d), P (V x r) and E (V x d) are i.i.d. normal with standard deviation
  1/sqrt(d) (so z = Q.h is O(1) for an RMS-normalised h).
* Q and P are rounded to the weight dtype first; then
  W = round(P~ . Q~ + 0.1 E), computed in float64 and rounded once
  (round-to-nearest-even).
* Hidden rows are N(0, 1), divided by their root-mean-square (no epsilon, no
  gain) in float64 and rounded to the weight dtype.
* Tree rows: node 0 is the root; node i >= 1 takes a parent uniformly from
  {0 .. i-1}; the root's raw row is N(0, 1) and a child's raw row is
  0.8 * raw_parent + 0.6 * N(0, 1); every row is then RMS-normalised.
* Random streams: numpy PCG64, SeedSequence(1000 + config id) spawned into
  one child per tensor (Q, P, E, H, tree); E and W are drawn in 8192-row
  chunks, each from its own grandchild, so the result does not depend on how
  many threads fill it.

bf16 arrays are returned as ``uint16`` bit patterns, fp32 arrays as
``float32``.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

__all__ = ["HeadConfig", "CONFIGS", "make", "make_custom", "make_lowrank_set", "make_hidden",
           "bf16_bits_to_f32", "CHUNK_ROWS"]

CHUNK_ROWS = 8192


@dataclass(frozen=True)
class HeadConfig:
    cid: int
    name: str
    B: int
    d: int
    V: int
    r: int
    k: int
    dtype: str          # "bf16" or "fp32"
    rows: str           # "iid" or "tree"


CONFIGS = {
    1: HeadConfig(1, "tiny fp32 head", 1, 256, 4096, 32, 8, "fp32", "iid"),
    2: HeadConfig(2, "batch-1 bf16 drafter head", 1, 5120, 151936, 128, 32, "bf16", "iid"),
    3: HeadConfig(3, "batch-1 higher rank", 1, 5120, 151936, 512, 64, "bf16", "iid"),
    4: HeadConfig(4, "64-node draft tree", 64, 5120, 151936, 128, 32, "bf16", "tree"),
    5: HeadConfig(5, "high-load batch", 2048, 5120, 151936, 256, 64, "bf16", "iid"),
}


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values once, to nearest-even, into the storage dtype."""
    if dtype == "fp32":
        return x.astype(np.float32)
    # bf16 keeps 8 significant bits: clear the low 45 of float64's 52
    # mantissa bits with round-to-nearest-even, after which the value is
    # exactly representable in float32 and its top 16 bits are the bf16.
    u = np.ascontiguousarray(x, dtype=np.float64).view(np.uint64)
    lsb = (u >> np.uint64(45)) & np.uint64(1)
    u = (u + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)
    f = u.view(np.float64).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 values (exact)."""
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _as_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def _normal(seq: np.random.SeedSequence, shape, std: float) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(seq))
    return g.standard_normal(shape) * std


def _rms_normalise(raw: np.ndarray) -> np.ndarray:
    return raw / np.sqrt(np.mean(raw * raw, axis=1, keepdims=True))


def _tree_parents(seq: np.random.SeedSequence, n: int) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(seq))
    parents = np.full(n, -1, dtype=np.int64)
    for i in range(1, n):
        parents[i] = g.integers(0, i)
    return parents


def make_hidden(cfg: HeadConfig, h_seq: np.random.SeedSequence,
                tree_seq: np.random.SeedSequence, B: int | None = None):
    """Hidden rows H (B x d) in the storage dtype, plus tree parents or None."""
    B = cfg.B if B is None else B
    parents = None
    if cfg.rows == "tree":
        parents = _tree_parents(tree_seq, B)
        noise = _normal(h_seq, (B, cfg.d), 1.0)
        raw = np.empty((B, cfg.d))
        raw[0] = noise[0]
        for i in range(1, B):
            raw[i] = 0.8 * raw[parents[i]] + 0.6 * noise[i]
    else:
        raw = _normal(h_seq, (B, cfg.d), 1.0)
    return _round_to_dtype(_rms_normalise(raw), cfg.dtype), parents


def _make_W(Pt: np.ndarray, Qt: np.ndarray, e_seq: np.random.SeedSequence,
            cfg: HeadConfig, e_scale: float = 0.1) -> np.ndarray:
    V, d = cfg.V, cfg.d
    Pf = _as_f64(Pt, cfg.dtype)
    Qf = _as_f64(Qt, cfg.dtype)
    n_chunks = (V + CHUNK_ROWS - 1) // CHUNK_ROWS
    children = e_seq.spawn(n_chunks)
    out = np.empty((V, d), dtype=np.uint16 if cfg.dtype == "bf16" else np.float32)
    std = 1.0 / math.sqrt(d)

    def fill(i: int) -> None:
        lo, hi = i * CHUNK_ROWS, min(V, (i + 1) * CHUNK_ROWS)
        x = Pf[lo:hi] @ Qf
        if e_scale != 0.0:
            x += e_scale * _normal(children[i], (hi - lo, d), std)
        out[lo:hi] = _round_to_dtype(x, cfg.dtype)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(n_chunks)))
    return out


def make(cid: int, *, B: int | None = None, with_W: bool = True,
         e_scale: float = 0.1) -> dict:
    """All inputs of one configuration.

    Returns a dict with ``cfg``, ``Q`` (r x d), ``P`` (V x r), ``W`` (V x d,
    or None when ``with_W`` is False), ``H`` (B x d) and ``parents`` (tree
    configs only). ``B`` overrides the row count (rows are a prefix of the
    full set for i.i.d. rows; for the tree, a smaller tree from the same seed).
    """
    cfg = CONFIGS[cid]
    sq, sp, se, sh, st = np.random.SeedSequence(1000 + cid).spawn(5)
    std = 1.0 / math.sqrt(cfg.d)
    Qt = _round_to_dtype(_normal(sq, (cfg.r, cfg.d), std), cfg.dtype)
    Pt = _round_to_dtype(_normal(sp, (cfg.V, cfg.r), std), cfg.dtype)
    W = _make_W(Pt, Qt, se, cfg, e_scale) if with_W else None
    H, parents = make_hidden(cfg, sh, st, B)
    return {"cfg": cfg, "Q": Qt, "P": Pt, "W": W, "H": H, "parents": parents}


def make_lowrank_set(cid: int, set_id: int, *, B: int | None = None) -> dict:
    """An extra, independent (Q, P, H) set for cache-cold timing rotation.

    Same shapes and distributions as configuration ``cid``; seeded from
    SeedSequence([1000 + cid, set_id]) so every set is distinct.
    """
    cfg = CONFIGS[cid]
    sq, sp, sh, st = np.random.SeedSequence([1000 + cid, set_id]).spawn(4)
    std = 1.0 / math.sqrt(cfg.d)
    Qt = _round_to_dtype(_normal(sq, (cfg.r, cfg.d), std), cfg.dtype)
    Pt = _round_to_dtype(_normal(sp, (cfg.V, cfg.r), std), cfg.dtype)
    H, _ = make_hidden(cfg, sh, st, B)
    return {"cfg": cfg, "Q": Qt, "P": Pt, "H": H}


def make_custom(V: int, d: int, r: int, B: int, dtype: str = "bf16", *, seed: int = 0,
                rows: str = "iid", e_scale: float = 0.1) -> dict:
    """Inputs of the same recipe at arbitrary shapes (ragged and edge cases).

    Seeded from SeedSequence([2000, seed, V, d, r, B]); k is left to the caller.
    """
    cfg = HeadConfig(0, "custom", B, d, V, r, min(64, V), dtype, rows)
    sq, sp, se, sh, st = np.random.SeedSequence([2000, seed, V, d, r, B]).spawn(5)
    std = 1.0 / math.sqrt(d)
    Qt = _round_to_dtype(_normal(sq, (r, d), std), dtype)
    Pt = _round_to_dtype(_normal(sp, (V, r), std), dtype)
    W = _make_W(Pt, Qt, se, cfg, e_scale)
    H, parents = make_hidden(cfg, sh, st, B)
    return {"cfg": cfg, "Q": Qt, "P": Pt, "W": W, "H": H, "parents": parents}
