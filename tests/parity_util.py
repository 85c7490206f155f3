"""Shared helpers of the GPU parity tests: move generated inputs to the
device and compare device results with the float64 oracle, row by row, under
the rule of oracle/compare.py."""
from __future__ import annotations

import numpy as np
import torch

import oracle


def dev(a: np.ndarray, device) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def check_lowrank(inp: dict, k: int, idx, score, logits, rows=None) -> tuple[list, dict]:
    """Device candidates / scores / logits on `rows` against oracle O1-O4."""
    dt = inp["cfg"].dtype
    H = inp["H"]
    rows = np.arange(H.shape[0]) if rows is None else np.asarray(rows)
    ref = oracle.lowrank_head(inp["Q"], inp["P"], None, H, k, dt, rows=rows, keep_scores=True)
    h64 = oracle.to_f64(H[rows], dt)
    errs = []
    for i, b in enumerate(rows):
        s = ref["s"][i]
        e = oracle.check_candidates(idx[b], s, ref["idx"][i], ref["tau"][i], ref["gap"][i], ref["s_k"][i])
        if score is not None:
            ids = np.clip(idx[b].astype(np.int64), 0, inp["P"].shape[0] - 1)
            allow = oracle.z_step_allowance(oracle.to_f64(inp["P"][ids], dt), ref["z"][i], dt)
            e += oracle.check_scores(score[b], s[idx[b]], float(np.max(np.abs(s))), dt, allow)
        if logits is not None:
            exact = oracle.exact_logits(inp["W"], h64, np.full(k, i), idx[b].astype(np.int64), dt)
            e += oracle.check_logits(logits[b], exact, dt)
        errs += [f"row {b}: {m}" for m in e]
    stats = oracle.band_counts(ref["gap"], ref["tau"])
    stats["exact_rows"] = int(sum(np.array_equal(idx[b], ref["idx"][i]) for i, b in enumerate(rows)))
    return errs, stats


def check_full(inp: dict, k: int, idx, logits, rows=None) -> tuple[list, dict]:
    """Device full-head baseline on `rows` against oracle O5."""
    dt = inp["cfg"].dtype
    H = inp["H"]
    rows = np.arange(H.shape[0]) if rows is None else np.asarray(rows)
    ref = oracle.full_head(inp["W"], H, k, dt, rows=rows, keep_logits=True)
    errs = []
    for i, b in enumerate(rows):
        L = ref["L"][i]
        e = oracle.check_candidates(idx[b], L, ref["idx"][i], ref["tau"][i], ref["gap"][i], ref["s_k"][i])
        e += oracle.check_logits(logits[b], L[idx[b]], dt)
        errs += [f"row {b}: {m}" for m in e]
    stats = oracle.band_counts(ref["gap"], ref["tau"])
    return errs, stats


def check_properties(idx: np.ndarray, score: np.ndarray, V: int) -> list:
    """What holds for every row at any size: ids distinct and in range,
    scores in candidate order (higher first, lower id on ties), finite."""
    errs = []
    if np.any(idx < 0) or np.any(idx >= V):
        errs.append("ids out of range")
    srt = np.sort(idx, axis=1)
    if np.any(srt[:, 1:] == srt[:, :-1]):
        errs.append("duplicate ids in a row")
    if score is not None:
        if not np.all(np.isfinite(score)):
            errs.append("non-finite scores")
        a, b = score[:, :-1], score[:, 1:]
        ok = (a > b) | ((a == b) & (idx[:, :-1] < idx[:, 1:]))
        if not np.all(ok):
            errs.append(f"{int(np.sum(~ok))} adjacent pairs out of order")
    return errs
