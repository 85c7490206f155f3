"""GPU parity of the HIP head against the float64 oracle, through the C ABI.

Rule (oracle/compare.py): candidate ids bit-exact as a set wherever the
oracle's k-th/(k+1)-th gap exceeds 1e-3 * max|score|, boundary swaps only
inside that band; logits within 2e-3 (bf16) or 1e-5 (fp32) relative.
"""
import functools
import math
import sys

import numpy as np
import pytest
import torch

import gen
import oracle
import rank_lm_head_amd as lr
from parity_util import check_full, check_lowrank, check_properties, dev

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def np_(t):
    return None if t is None else t.cpu().numpy()


@functools.lru_cache(maxsize=1)
def config(cid: int):
    say(f"[gen] config {cid}")
    inp = gen.make(cid)
    t = {x: dev(inp[x], DEV) for x in ("Q", "P", "W", "H")}
    return inp, t


def head_for(inp, t, B_max=None, k_max=None):
    cfg = inp["cfg"]
    return lr.Head(t["Q"], t["P"], t["W"], B_max=B_max or cfg.B, k_max=k_max or cfg.k)


# ------------------------------------------------------------ tiny fp32 head

def test_tiny_fp32_every_call():
    inp, t = config(1)
    k = inp["cfg"].k
    head = head_for(inp, t)
    say("[run] c1 candidates / logits / draft / full_topk / dense")
    idx, score = head.candidates(t["H"], k)
    lg = head.logits(t["H"], idx)
    didx, dscore, dlg = head.draft(t["H"], k)
    fidx, flog = head.full_topk(t["H"], k)
    dense = head.dense_logits(t["H"])
    torch.cuda.synchronize()
    idx, score, lg = np_(idx), np_(score), np_(lg)
    errs, stats = check_lowrank(inp, k, idx, score, lg)
    assert not errs, errs
    assert np.array_equal(np_(didx), idx) and np.array_equal(np_(dlg), lg)
    assert np.array_equal(np_(dscore), score)
    errs, _ = check_full(inp, k, np_(fidx), np_(flog))
    assert not errs, errs
    L = oracle.full_head(inp["W"], inp["H"], k, "fp32", keep_logits=True)["L"]
    dn = np_(dense)
    # a priori bound of an fp32 dot product of length d: d * 2^-24 * sum |w_i h_i|
    absdot = np.abs(oracle.to_f64(inp["W"], "fp32")) @ np.abs(oracle.to_f64(inp["H"], "fp32")[0])
    assert np.all(np.abs(dn[0] - L[0]) <= inp["cfg"].d * 2.0 ** -24 * absdot)
    say(f"[ok] c1 {stats}")


# ----------------------------------------------- small heads: tiles and tails

@pytest.mark.parametrize("dt", ["bf16", "fp32"])
@pytest.mark.parametrize("V,d,r,B,k", [
    (1000, 136, 40, 19, 7),      # ragged vocabulary tile, k tail in both contractions, ragged rows
    (4099, 264, 24, 33, 64),     # k = 64, three row tiles, V % 16 == 3
    (17, 64, 16, 2, 17),         # k = V
    (10, 32, 8, 1, 1),           # V below one tile
    (2500, 512, 512, 5, 33),     # r at its maximum
])
def test_small_heads(dt, V, d, r, B, k):
    inp = gen.make_custom(V, d, r, B, dt, seed=V + d)
    t = {x: dev(inp[x], DEV) for x in ("Q", "P", "W", "H")}
    head = lr.Head(t["Q"], t["P"], t["W"], B_max=B, k_max=k)
    say(f"[run] small {dt} V={V} d={d} r={r} B={B} k={k}")
    idx, score, lg = head.draft(t["H"], k)
    fidx, flog = head.full_topk(t["H"], k)
    torch.cuda.synchronize()
    errs, stats = check_lowrank(inp, k, np_(idx), np_(score), np_(lg))
    assert not errs, errs[:5]
    errs, _ = check_full(inp, k, np_(fidx), np_(flog))
    assert not errs, errs[:5]
    say(f"[ok] {stats}")


@pytest.mark.parametrize("V,d,r,B,k", [
    (5000, 256, 128, 3, 64),     # streaming path, 3 rows, k = 64
    (30000, 512, 256, 4, 40),    # streaming path, 4 rows, many blocks
    (777, 64, 32, 1, 5),
    (300, 1032, 8, 2, 3),        # k < 4, r = 8, d not a multiple of 512
    (9000, 8200, 64, 1, 16),     # d beyond the long-row kernel: matrix-core full head
    (5000, 256, 128, 5, 64),     # five rows: the register-list pass, 11 idle rows in its column tile
    (30000, 512, 256, 8, 40),    # eight rows, many blocks (register-list pass)
    (777, 64, 32, 6, 5),
    (300, 1032, 8, 7, 3),        # seven rows, r = 8 (LDS-staged pass), d not a multiple of 512
    (9000, 8200, 64, 8, 16),     # eight rows with d beyond the streaming down-projection
    (30000, 5120, 512, 4, 64),   # four rows at the drafter head's d, r at its maximum
    (200000, 64, 32, 8, 16),     # 391 rows per slice: the deepest score buffer
])
def test_streaming_path_shapes(V, d, r, B, k):
    inp = gen.make_custom(V, d, r, B, "bf16", seed=V + r)
    t = {x: dev(inp[x], DEV) for x in ("Q", "P", "W", "H")}
    head = lr.Head(t["Q"], t["P"], t["W"], B_max=B, k_max=k)
    say(f"[run] streaming V={V} d={d} r={r} B={B} k={k}")
    idx, score, lg = head.draft(t["H"], k)
    fidx, flog = head.full_topk(t["H"], k)
    torch.cuda.synchronize()
    errs, stats = check_lowrank(inp, k, np_(idx), np_(score), np_(lg))
    assert not errs, errs[:5]
    errs, _ = check_full(inp, k, np_(fidx), np_(flog))
    assert not errs, errs[:5]
    say(f"[ok] {stats}")


@pytest.mark.parametrize("V,d,r,B,k", [
    (20000, 256, 96, 130, 48),   # wide batch tile: two row tiles, the second ragged; K tail of 32
    (6000, 384, 192, 64, 64),    # narrow batch tile exactly full, k = 64 (r = 192: not the register-list pass)
    (12345, 200, 72, 65, 10),    # one row past the narrow tile; K = 64 + 8
    (257, 64, 16, 9, 9),         # two vocabulary blocks, the second holding one row
    (3000, 200, 72, 300, 16),    # z on the GEMM kernel: r = 64 + 8, d = 3 * 64 + 8, ragged row tile
    (5000, 512, 256, 512, 64),   # z on the GEMM kernel, full tiles
    (40000, 256, 256, 600, 64),  # strip kernel: three batch tiles, strip groups on the XCDs, ragged last strip
    (7000, 5128, 64, 100, 32),   # split down-projection: 11 K parts, the last one 8 columns wide
    (30000, 5120, 512, 8, 64),   # eight rows at r = 512 (register-list pass, z in LDS)
    (100, 64, 16, 300, 8),       # strip kernel: one partial strip (V < 256), two batch tiles
    (20000, 256, 128, 200, 32),  # strip kernel with one batch tile (129-256 rows), strips spread evenly
    (5000, 128, 64, 129, 16),    # strip kernel at its lowest row count, 127 idle rows in the tile
    (3000, 64, 8, 300, 16),      # strip kernel at r = 8: K steps mostly past the row, zero z chunks
    (3000, 1000, 128, 600, 16),  # z on the GEMM kernel split over K (4 parts), the last K stage partial
])
def test_batch_path_shapes(V, d, r, B, k):
    inp = gen.make_custom(V, d, r, B, "bf16", seed=V + B)
    t = {x: dev(inp[x], DEV) for x in ("Q", "P", "W", "H")}
    head = lr.Head(t["Q"], t["P"], t["W"], B_max=B, k_max=k)
    say(f"[run] batch V={V} d={d} r={r} B={B} k={k}")
    idx, score, lg = head.draft(t["H"], k)
    fidx, flog = head.full_topk(t["H"], k)
    torch.cuda.synchronize()
    errs, stats = check_lowrank(inp, k, np_(idx), np_(score), np_(lg))
    assert not errs, errs[:5]
    errs, _ = check_full(inp, k, np_(fidx), np_(flog))
    assert not errs, errs[:5]
    say(f"[ok] {stats}")


@pytest.mark.parametrize("V,d,r,B,k", [
    (20, 64, 32, 12, 20),        # one slice of 20 rows, k = V: its 4-entry list is deep, the merge recomputes it
    (10, 64, 32, 6, 3),          # V below one 16-row tile: every wave's tile is its last, partly past V
    (257, 64, 32, 9, 9),         # two slices of 128 and 129 rows, 16-row column tile with 7 idle rows
    (1000, 136, 32, 12, 5),      # ragged last 16-row tile of every wave
    (300, 1032, 32, 20, 3),      # k < 4: lists of 3
    (12345, 200, 64, 33, 10),    # 64-row column tiles at r = 64, 31 idle rows
    (20000, 512, 256, 32, 40),   # z in LDS: 32-row column tiles at r = 256
    (30000, 512, 512, 16, 64),   # z in LDS: r = 512 on one column tile
    (6000, 384, 128, 64, 64),    # z in LDS: 64 rows at r = 128, k = 64
    (20000, 512, 256, 12, 32),   # z in registers at r = 256 (one column tile)
    (8000, 264, 64, 57, 20),     # two rows of Q per down-projection block, last group of h 1 row
    (9000, 256, 128, 30, 32),    # z in registers at r = 128 (32-row column tiles)
    (200000, 64, 32, 40, 16),    # 391 rows per slice
    (20000, 512, 256, 64, 32),   # z in LDS: 64 rows at r = 256
    (5000, 256, 512, 24, 64),    # z in LDS: 32-row column tiles at r = 512
    (30000, 512, 512, 40, 16),   # z in LDS: 64 rows at r = 512
])
def test_rows_path_shapes(V, d, r, B, k):
    """5 to 64 rows: the matrix-core pass that keeps each slice's best in
    registers, then the merge."""
    inp = gen.make_custom(V, d, r, B, "bf16", seed=V + 3 * B)
    t = {x: dev(inp[x], DEV) for x in ("Q", "P", "W", "H")}
    head = lr.Head(t["Q"], t["P"], t["W"], B_max=B, k_max=k)
    say(f"[run] rows V={V} d={d} r={r} B={B} k={k}")
    idx, score, lg = head.draft(t["H"], k)
    torch.cuda.synchronize()
    errs, stats = check_lowrank(inp, k, np_(idx), np_(score), np_(lg))
    assert not errs, errs[:5]
    say(f"[ok] {stats}")


@pytest.mark.parametrize("B", [16, 64])
def test_rows_path_best_inside_one_slice(B):
    """P's rows in one slice scaled by 8 (exact in bf16), so that most of
    every row's k best sit in that slice: its 4-entry lists are full at the
    merge's bound and the merge recomputes the slice's scores, which must
    equal the listed ones bit for bit for the result to be right."""
    V, d, r, k = 20000, 256, 64, 32
    inp = gen.make_custom(V, d, r, B, "bf16", seed=77 + B)
    inp2 = dict(inp)
    inp2["P"] = inp["P"].copy()
    n = 79                                   # slices of this vocabulary (256 rows per block or fewer)
    lo, hi = V * 3 // n, V * 4 // n
    f = (inp["P"][lo:hi].astype(np.uint32) << np.uint32(16)).view(np.float32) * np.float32(8)
    inp2["P"][lo:hi] = (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    t = {x: dev(inp2[x], DEV) for x in ("Q", "P", "W", "H")}
    head = lr.Head(t["Q"], t["P"], t["W"], B_max=B, k_max=k)
    say(f"[run] rows best inside one slice B={B}")
    idx, score, lg = head.draft(t["H"], k)
    torch.cuda.synchronize()
    ids = np_(idx)
    inside = ((ids >= lo) & (ids < hi)).sum(axis=1)
    assert np.all(inside >= 5), inside
    errs, _ = check_lowrank(inp2, k, ids, np_(score), np_(lg))
    assert not errs, errs[:5]


def test_batch_duplicate_rows_tie_to_the_lower_id():
    """Bitwise-equal vocabulary rows in different vocabulary blocks: the
    batch path returns them in id order (8 draft rows)."""
    V, B = 3000, 8
    inp = gen.make_custom(V, 128, 32, B, "bf16", seed=15)
    t = {x: dev(inp[x], DEV) for x in ("Q", "P", "W", "H")}
    head = lr.Head(t["Q"], t["P"], t["W"], B_max=B, k_max=4)
    tok = int(np_(head.candidates(t["H"], 1)[0])[0, 0])
    assume = tok not in (0, V - 1)
    if not assume:
        pytest.skip("row 0's best token sits at an end of the vocabulary")
    P2 = t["P"].clone()
    for dst in (0, V - 1):
        P2[dst] = t["P"][tok]
    h2 = lr.Head(t["Q"], P2, t["W"], B_max=B, k_max=4)
    idx, score = h2.candidates(t["H"], 3)
    assert np_(idx)[0].tolist() == [0, tok, V - 1]
    assert len(set(np_(score)[0].tolist())) == 1


@pytest.mark.parametrize("B", [1, 8, 16, 64, 300])
def test_all_scores_tied(B):
    """Every score equal: the k lowest ids win, in order (forces the merge's
    exhaustive path, since every entry reaches the sampled threshold)."""
    V, d, r, k = 5000, 128, 64, 32
    inp = gen.make_custom(V, d, r, B, "bf16", seed=9)
    t = {x: dev(inp[x], DEV) for x in ("Q", "P", "W", "H")}
    t["P"].zero_()
    t["W"].zero_()
    head = lr.Head(t["Q"], t["P"], t["W"], B_max=B, k_max=k)
    idx, score, lg = head.draft(t["H"], k)
    fidx, flog = head.full_topk(t["H"], k)
    torch.cuda.synchronize()
    want = np.tile(np.arange(k), (B, 1))
    assert np.array_equal(np_(idx), want) and np.array_equal(np_(fidx), want)
    assert not np.any(np_(score)) and not np.any(np_(lg)) and not np.any(np_(flog))


def test_empty_batch_is_a_noop():
    inp = gen.make_custom(300, 64, 16, 4, "bf16", seed=1)
    t = {x: dev(inp[x], DEV) for x in ("Q", "P", "W", "H")}
    head = lr.Head(t["Q"], t["P"], t["W"], B_max=4, k_max=8)
    idx, score, lg = head.draft(t["H"][:0], 8)
    assert idx.shape == (0, 8) and lg.shape == (0, 8)
    fidx, flog = head.full_topk(t["H"][:0], 8)
    torch.cuda.synchronize()
    assert fidx.numel() == 0


def test_calls_reject_bad_arguments_on_a_real_handle():
    inp = gen.make_custom(300, 64, 16, 4, "bf16", seed=2)
    t = {x: dev(inp[x], DEV) for x in ("Q", "P", "W", "H")}
    head = lr.Head(t["Q"], t["P"], t["W"], B_max=4, k_max=8)
    L = head.lib
    H = t["H"]
    out = torch.empty(64, dtype=torch.int32, device=DEV)
    import ctypes
    p = lambda x: ctypes.c_void_p(x.data_ptr())
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert L.lrhead_candidates(head._h, p(H), 5, 4, p(out), None, s) == lr._lib.ERANGE     # B > B_max
    assert L.lrhead_candidates(head._h, p(H), 1, 9, p(out), None, s) == lr._lib.ERANGE     # k > k_max
    assert L.lrhead_candidates(head._h, p(H), 1, 0, p(out), None, s) == lr._lib.ERANGE     # k < 1
    assert L.lrhead_candidates(head._h, ctypes.c_void_p(H.data_ptr() + 2), 1, 4, p(out), None, s) == lr._lib.EALIGN
    assert L.fullhead_topk(head._h, p(H), 1, 4, None, p(out), s) == lr._lib.EINVAL
    assert L.fullhead_logits(head._h, p(H), 1, p(out), 9, p(out), s) == lr._lib.ERANGE
    torch.cuda.synchronize()


# ---------------------------------------------------- the five configurations

def _sample_rows(B: int) -> np.ndarray:
    if B <= 64:
        return np.arange(B)
    return np.unique(np.concatenate([np.linspace(0, B - 1, 126).astype(int), [1, B - 2]]))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("cid", [2, 3, 4, 5])
def test_config_draft_head(cid):
    inp, t = config(cid)
    cfg = inp["cfg"]
    head = head_for(inp, t)
    say(f"[run] c{cid} draft head B={cfg.B} r={cfg.r} k={cfg.k}")
    idx, score, lg = head.draft(t["H"], cfg.k)
    torch.cuda.synchronize()
    idx, score, lg = np_(idx), np_(score), np_(lg)
    assert not check_properties(idx, score, cfg.V)
    assert np.all(np.isfinite(lg))
    # every row, in chunks that bound the oracle's float64 score block
    errs, exact, n_rows = [], 0, 0
    for lo in range(0, cfg.B, 256):
        rows = np.arange(lo, min(cfg.B, lo + 256))
        e, stats = check_lowrank(inp, cfg.k, idx, score, lg, rows=rows)
        errs += e
        exact += stats["exact_rows"]
        n_rows += len(rows)
    say(f"[ok?] c{cid} rows checked {n_rows}, identical to the oracle {exact}, errors {len(errs)}")
    assert not errs, errs[:5]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("cid", [2, 3, 4, 5])
def test_config_full_head_baseline(cid):
    inp, t = config(cid)
    cfg = inp["cfg"]
    head = head_for(inp, t)
    say(f"[run] c{cid} full head B={cfg.B} k={cfg.k}")
    fidx, flog = head.full_topk(t["H"], cfg.k)
    torch.cuda.synchronize()
    fidx, flog = np_(fidx), np_(flog)
    assert not check_properties(fidx, flog, cfg.V)
    rows = _sample_rows(cfg.B)
    errs, stats = check_full(inp, cfg.k, fidx, flog, rows=rows)
    say(f"[ok?] c{cid} full rows checked {len(rows)} {stats} errors {len(errs)}")
    assert not errs, errs[:5]


# ------------------------------------------------------ invariants on the GPU

@pytest.mark.parametrize("B", [1, 4, 8, 20, 64, 300])
def test_h_times_two_doubles_everything_bitwise(B):
    """h -> 2h is exact in bf16: z, scores and logits double bit for bit and
    the ids stay (one-row pass, LDS-staged and register-list streaming
    passes, the latter with the merge's own and separate rescoring)."""
    inp = gen.make_custom(5000, 256, 64, B, "bf16", seed=4)
    t = {x: dev(inp[x], DEV) for x in ("Q", "P", "W", "H")}
    head = lr.Head(t["Q"], t["P"], t["W"], B_max=B, k_max=32)
    a = [np_(x) for x in head.draft(t["H"], 32)]
    b = [np_(x) for x in head.draft((t["H"].float() * 2).to(torch.bfloat16), 32)]
    assert np.array_equal(a[0], b[0])
    assert np.array_equal(2 * a[1], b[1]) and np.array_equal(2 * a[2], b[2])


@pytest.mark.parametrize("B", [1, 4, 8, 40, 300])
def test_vocabulary_permutation_maps_the_ids(B):
    """Rows of P and W permuted together (P2[v] = P[perm[v]]): every score
    moves with its row, so each row's top-k scores, and the logits of the
    tokens behind them, come out bit for bit the same, at ids that map back
    through perm (one-row pass, LDS-staged, register-list and strip paths).
    Equal scores come out in each call's own id order (ties resolve to the
    lower id), and at the row's k-th score the ids may differ; the scores
    may not."""
    V, k = 3000, 16
    inp = gen.make_custom(V, 256, 64, B, "bf16", seed=41)
    t = {x: dev(inp[x], DEV) for x in ("Q", "P", "W", "H")}
    perm = np.random.default_rng(41).permutation(V)
    pt = torch.from_numpy(perm).to(DEV)
    P2, W2 = t["P"][pt].contiguous(), t["W"][pt].contiguous()
    ha = lr.Head(t["Q"], t["P"], t["W"], B_max=B, k_max=k)
    a = [np_(x) for x in ha.draft(t["H"], k)]
    b = [np_(x) for x in lr.Head(t["Q"], P2, W2, B_max=B, k_max=k).draft(t["H"], k)]
    mapped = perm[b[0]].astype(np.int32)
    # the permuted call's logits are the original head's at the mapped ids
    la = np_(ha.logits(t["H"], torch.from_numpy(mapped).to(DEV)))
    torch.cuda.synchronize()
    assert np.array_equal(a[1], b[1]), "top-k scores differ"
    assert np.array_equal(la, b[2])
    for row in range(B):
        assert len(set(mapped[row].tolist())) == k, row
        # equal scores inside the list hold the same ids, ordered by each
        # call's own numbering; at the k-th score only the scores must agree
        for v in set(a[1][row].tolist()) - {float(a[1][row, -1])}:
            sa, sb = a[1][row] == v, b[1][row] == v
            assert sorted(a[0][row][sa].tolist()) == sorted(mapped[row][sb].tolist()), (row, v)
            la_of = dict(zip(a[0][row][sa].tolist(), a[2][row][sa].tolist()))
            assert all(la_of[i] == x for i, x in zip(mapped[row][sb].tolist(), b[2][row][sb].tolist())), (row, v)


@pytest.mark.parametrize("B", [1, 4, 8, 64, 300])
def test_graph_replays_match_eager_calls(B):
    """The draft call captured in a HIP graph, as the bench times it, gives on
    every replay the bits of the eager call on the same rows: the rows change
    between replays, and eager calls and synchronisations run in between (one
    row, LDS-staged, register-list and strip paths; nothing the calls need is
    carried over in the workspace)."""
    V, d, r, k = 20000, 512, 128, 32
    inp = gen.make_custom(V, d, r, B, "bf16", seed=77)
    t = {x: dev(inp[x], DEV) for x in ("Q", "P", "W", "H")}
    H2 = dev(gen.make_custom(V, d, r, B, "bf16", seed=78)["H"], DEV)
    head = lr.Head(t["Q"], t["P"], t["W"], B_max=B, k_max=k)
    refs = [[np_(x) for x in head.draft(h, k)] for h in (t["H"], H2)]
    hbuf = t["H"].clone()
    out = (torch.empty((B, k), dtype=torch.int32, device=DEV), torch.empty((B, k), dtype=torch.float32, device=DEV),
           torch.empty((B, k), dtype=torch.float32, device=DEV))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        head.draft(hbuf, k, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        head.draft(hbuf, k, out=out)
    torch.cuda.synchronize()
    for trial in range(6):
        which = trial % 2
        hbuf.copy_(t["H"] if which == 0 else H2)
        g.replay()
        torch.cuda.synchronize()
        got = [np_(x) for x in out]
        for a, b in zip(refs[which], got):
            assert np.array_equal(a, b), (trial, B)
        # eager work of the program between replays
        eager = [np_(x) for x in head.draft(H2 if which == 0 else t["H"], k)]
        for a, b in zip(refs[1 - which], eager):
            assert np.array_equal(a, b), (trial, B)


@pytest.mark.parametrize("B", [1, 4, 8, 20, 64])
def test_draft_logits_equal_rescoring_bitwise(B):
    """The draft call's logits (speculative per-slice rescoring and the merge's
    own, on the few-row paths) are the bits fullhead_logits gives for the same
    ids: every kernel uses one row-dot order."""
    inp = gen.make_custom(20000, 5120, 128, B, "bf16", seed=31)
    t = {x: dev(inp[x], DEV) for x in ("Q", "P", "W", "H")}
    head = lr.Head(t["Q"], t["P"], t["W"], B_max=B, k_max=32)
    idx, score, lg = head.draft(t["H"], 32)
    lg2 = head.logits(t["H"], idx)
    torch.cuda.synchronize()
    assert np.array_equal(np_(lg), np_(lg2))
    errs, _ = check_lowrank(inp, 32, np_(idx), np_(score), np_(lg))
    assert not errs, errs[:5]


def test_one_row_pass_ties_inside_a_slice():
    """One-row pass: nine bitwise copies of the best low-rank row at
    consecutive ids. Every slice of that pass holds at least 64 rows, so nine
    consecutive ids span at most two slices and five or more copies share
    one; that slice's 4-entry list is full at the merge's bound, so the merge
    also reads its raw scores. All copies come out first, in id order."""
    V, k = 20000, 16
    inp = gen.make_custom(V, 256, 64, 1, "bf16", seed=21)
    t = {x: dev(inp[x], DEV) for x in ("Q", "P", "W", "H")}
    head = lr.Head(t["Q"], t["P"], t["W"], B_max=1, k_max=k)
    tok = int(np_(head.candidates(t["H"], 1)[0])[0, 0])
    start = 5000 if not 5000 <= tok < 5009 else 9000
    dups = list(range(start, start + 9))
    inp2 = dict(inp)
    inp2["P"] = inp["P"].copy()
    for dst in dups:
        inp2["P"][dst] = inp["P"][tok]
    P2 = dev(inp2["P"], DEV)
    h2 = lr.Head(t["Q"], P2, t["W"], B_max=1, k_max=k)
    idx, score, lg = h2.draft(t["H"], k)
    torch.cuda.synchronize()
    tied = sorted(dups + [tok])
    assert np_(idx)[0, :10].tolist() == tied
    assert len(set(np_(score)[0, :10].tolist())) == 1
    errs, _ = check_lowrank(inp2, k, np_(idx), np_(score), np_(lg))
    assert not errs, errs[:5]


def test_duplicate_rows_tie_to_the_lower_id():
    V = 3000
    inp = gen.make_custom(V, 128, 32, 1, "bf16", seed=5)
    t = {x: dev(inp[x], DEV) for x in ("Q", "P", "W", "H")}
    head = lr.Head(t["Q"], t["P"], t["W"], B_max=1, k_max=4)
    tok = int(np_(head.candidates(t["H"], 1)[0])[0, 0])
    ftok = int(np_(head.full_topk(t["H"], 1)[0])[0, 0])
    assert tok not in (0, V - 1) and ftok not in (0, V - 1)
    P2, W2 = t["P"].clone(), t["W"].clone()
    for dst in (0, V - 1):          # bitwise copies of the best rows, below and above
        P2[dst] = t["P"][tok]
        W2[dst] = t["W"][ftok]
    h2 = lr.Head(t["Q"], P2, W2, B_max=1, k_max=4)
    idx, score = h2.candidates(t["H"], 3)
    assert np_(idx)[0].tolist() == [0, tok, V - 1]
    assert len(set(np_(score)[0].tolist())) == 1
    assert np_(h2.candidates(t["H"], 1)[0])[0, 0] == 0
    fidx, flog = h2.full_topk(t["H"], 3)
    assert np_(fidx)[0].tolist() == [0, ftok, V - 1]
    assert len(set(np_(flog)[0].tolist())) == 1


@pytest.mark.parametrize("B", [1, 4, 8, 16, 40, 300])
def test_ties_inside_one_slice_go_to_the_lower_ids(B):
    """Bitwise copies of the best low-rank row inside one vocabulary slice, at
    ids that share a lane and ids in different lanes: every tied copy must come
    out in id order. With five tied entries the slice's 4-entry list is full at
    the bound, so the merge also reads that slice's raw scores."""
    V, k = 3000, 6
    inp = gen.make_custom(V, 128, 32, B, "bf16", seed=12)
    t = {x: dev(inp[x], DEV) for x in ("Q", "P", "W", "H")}
    head = lr.Head(t["Q"], t["P"], t["W"], B_max=B, k_max=k)
    tok = int(np_(head.candidates(t["H"][:1], 1)[0])[0, 0])
    # V = 3000 gives 12 slices of 250 rows; slice 1 is ids [250, 500): ids
    # 253, 256, 320 and 380 sit in lanes 3, 6, 6, 2 as elements 0, 0, 1, 2
    dups = [x for x in (253, 256, 320, 380, 441) if x != tok][:4]
    inp2 = dict(inp)
    inp2["P"] = inp["P"].copy()
    for dst in dups:
        inp2["P"][dst] = inp["P"][tok]
    P2 = dev(inp2["P"], DEV)
    h2 = lr.Head(t["Q"], P2, t["W"], B_max=B, k_max=k)
    idx, score, lg = h2.draft(t["H"], k)
    torch.cuda.synchronize()
    tied = sorted(dups + [tok])
    got = np_(idx)[0].tolist()
    assert got[:5] == tied, (got, tied)
    assert len(set(np_(score)[0, :5].tolist())) == 1
    errs, _ = check_lowrank(inp2, k, np_(idx), np_(score), np_(lg))
    assert not errs, errs[:5]


@pytest.mark.parametrize("V,d,r,B,dt,ties", [
    (20000, 512, 128, 1, "bf16", False),   # one-row pass
    (20000, 512, 128, 1, "bf16", True),    # one-row pass, boundary ties: the merge reads raw scores
    (20000, 512, 128, 4, "bf16", False),   # four-row streaming path (scores staged in LDS, raw copy)
    (20000, 512, 128, 4, "bf16", True),    # four rows, boundary ties: the merge reads raw scores
    (20000, 512, 128, 8, "bf16", False),   # eight rows: the register-list pass
    (20000, 512, 128, 8, "bf16", True),    # eight rows, boundary ties: the merge recomputes slices
    (4096, 256, 32, 1, "fp32", False),     # fp32 (matrix-core slice lists and merge)
    (20000, 512, 128, 40, "bf16", False),  # register-list pass, down-projection in 8-row groups
    (20000, 512, 128, 40, "bf16", True),   # register-list pass, boundary ties: the merge recomputes slices
    (20000, 512, 256, 40, "bf16", False),  # register-list pass with z in LDS (40 rows at r = 256)
    (20000, 512, 128, 300, "bf16", False), # strip kernel (two batch tiles), split down-projection in the score scratch
])
def test_repeat_calls_and_poisoned_workspace_are_bitwise_stable(V, d, r, B, dt, ties):
    """Repeated calls agree bit for bit, also after the workspace is filled
    with garbage between calls: no call reads what an earlier call left. With
    `ties`, all but 20 rows of P are zero, so that the k-th best score is a
    tie shared by thousands of rows and the merges take their raw-score
    paths."""
    inp = gen.make_custom(V, d, r, B, dt, seed=6)
    t = {x: dev(inp[x], DEV) for x in ("Q", "P", "W", "H")}
    if ties:
        t["P"][20:].zero_()
    head = lr.Head(t["Q"], t["P"], t["W"], B_max=B, k_max=64)
    say(f"[run] poisoned workspace V={V} d={d} r={r} B={B} {dt} ties={ties}")
    ref = [np_(x) for x in head.draft(t["H"], 64)]
    for trial in range(5):
        head.workspace.fill_(0xFF if trial % 2 else 0x7F)     # NaN / large garbage
        got = [np_(x) for x in head.draft(t["H"], 64)]
        for a, b in zip(ref, got):
            assert np.array_equal(a, b, equal_nan=True)
    f1 = [np_(x) for x in head.full_topk(t["H"], 64)]
    f2 = [np_(x) for x in head.full_topk(t["H"], 64)]
    assert all(np.array_equal(a, b) for a, b in zip(f1, f2))
    if ties:
        inp2 = dict(inp)
        inp2["P"] = inp["P"].copy()
        inp2["P"][20:] = 0
        errs, _ = check_lowrank(inp2, 64, *ref)
        assert not errs, errs[:5]


# ------------------------------------------- draft distribution (D1-D3)

def check_branch(logits, idx, nb, parent, probs, br_i, br_p, br_path):
    """Device branch outputs against oracle D1-D3 on the device's own logits:
    probabilities within 1e-5 relative (fp32 exp and sum against float64),
    branch ids equal up to neighbours whose probabilities are within 1e-6."""
    p_ref, bi_ref, bp_ref, bpath_ref = oracle.branches(logits, idx, nb, parent)
    errs = []
    if not np.allclose(probs, p_ref, rtol=1e-5, atol=1e-7):
        errs.append(f"probs off by {np.max(np.abs(probs - p_ref)):.3g}")
    for b in range(logits.shape[0]):
        got, want = br_i[b].tolist(), bi_ref[b].tolist()
        if got != want:
            pm = {int(i): float(p_ref[b][j]) for j, i in enumerate(idx[b]) if not np.isnan(logits[b, j])}
            for r, (g, w) in enumerate(zip(got, want)):
                if g != w and not (g in pm and w in pm and abs(pm[g] - pm[w]) <= 1e-6 * max(pm[w], 1e-30)):
                    errs.append(f"row {b} rank {r}: id {g}, oracle {w}")
        if not np.allclose(br_p[b], bp_ref[b], rtol=1e-5, atol=1e-7):
            errs.append(f"row {b}: branch probabilities")
        if not np.allclose(br_path[b], bpath_ref[b], rtol=1e-5, atol=1e-7):
            errs.append(f"row {b}: path probabilities")
    return errs


def test_branch_after_a_draft_call_matches_the_oracle():
    """Draft distribution on the candidates of a real draft call (batch-1 and a
    64-node tree), nb = 1 (a chain), 4 and k, with parent path probabilities."""
    for cid in (2, 4):
        inp, t = config(cid)
        cfg = inp["cfg"]
        head = head_for(inp, t)
        idx, _, lg = head.draft(t["H"], cfg.k)
        parent = torch.rand(cfg.B, device=DEV, generator=torch.Generator(DEV).manual_seed(cid))
        for nb in (1, 4, cfg.k):
            say(f"[run] branch c{cid} nb={nb}")
            out = lr.branch(lg, idx, nb, parent)
            torch.cuda.synchronize()
            errs = check_branch(np_(lg), np_(idx), nb, np_(parent), *[np_(x) for x in out])
            assert not errs, errs[:5]


def test_branch_edge_cases():
    """Equal logits (ties to the lower id), empty slots (NaN), k = 1, large shifts."""
    rng = np.random.default_rng(5)
    B, k = 6, 64
    l = rng.normal(size=(B, k)).astype(np.float32) * 4
    l[0] = 1.25                                   # all tied
    l[1, 40:] = np.nan                            # fewer candidates than branches below
    l[2] += 80.0                                  # exp overflows without the max subtraction
    l[3, ::3] = l[3, 0]                           # many ties with the row's first logit
    ids = np.stack([rng.permutation(100000)[:k] for _ in range(B)]).astype(np.int32)
    ids[1, 40:] = 0x7FFFFFFF
    for nb in (1, 5, 48, 64):
        out = lr.branch(torch.from_numpy(l).to(DEV), torch.from_numpy(ids).to(DEV), nb)
        torch.cuda.synchronize()
        errs = check_branch(l, ids, nb, None, *[np_(x) for x in out])
        assert not errs, (nb, errs[:5])
    one = lr.branch(torch.tensor([[3.0]], device=DEV), torch.tensor([[17]], dtype=torch.int32, device=DEV), 1)
    assert np_(one[0]).tolist() == [[1.0]] and np_(one[1]).tolist() == [[17]]


# ------------------------------------------------ building P and Q (F1-F4)

def _bf16_np(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def check_factor_close(P_g, Q_g, P_o, Q_o):
    """Device P, Q (bf16) against the oracle's (float64 values of bf16):
    equal up to two bf16 steps of each value plus 1e-4 of the largest (the
    device sums in fp32 where the oracle sums in float64; the final rounding
    to bf16 can then land one step apart)."""
    errs = []
    for name, g, o in (("P", P_g, P_o), ("Q", Q_g, Q_o)):
        tol = 2 * oracle.ulp_bf16(np.abs(o)) + 1e-4 * np.abs(o).max()
        bad = np.abs(g - o) > tol
        if bad.any():
            errs.append(f"{name}: {int(bad.sum())} of {bad.size} elements off, worst {np.abs(g - o).max():.3g}")
    return errs


@pytest.mark.parametrize("V,d,r,q", [
    (3000, 256, 32, 1),     # ragged tiles in V
    (20000, 1024, 64, 2),   # two iterations
    (4096, 200, 8, 0),      # no iteration, d not a multiple of 64
    (9000, 1000, 128, 1),   # r >= 128: 256-row GEMM tiles of the panel halves; ragged tiles in V and d
    (6000, 512, 256, 1),    # two tiles of r
    (3001, 256, 32, 1),     # V not a multiple of 8: the W products on the vector ALU
    (2000, 260, 64, 1),     # d not a multiple of 8: the W products on the vector ALU
])
def test_factor_matches_the_oracle(V, d, r, q):
    from oracle import factor as fa
    rng = np.random.default_rng(V + r)
    Wf = (rng.normal(size=(V, r)) @ rng.normal(size=(r, d)) / math.sqrt(d)
          + 0.1 * rng.normal(size=(V, d)) / math.sqrt(d))
    W = oracle.round_bf16(oracle.round_fp32(Wf))
    Wb = (W.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    omega = rng.normal(size=(d, r)).astype(np.float32)
    say(f"[run] factor V={V} d={d} r={r} q={q}")
    P, Q = lr.factor(dev(Wb, DEV), r, torch.from_numpy(omega).to(DEV), q)
    torch.cuda.synchronize()
    P_o, Q_o = fa.factor(Wb, omega, q, "bf16")
    P_g = oracle.to_f64(_bf16_np(P), "bf16")
    Q_g = oracle.to_f64(_bf16_np(Q), "bf16")
    errs = check_factor_close(P_g, Q_g, P_o, Q_o)
    assert not errs, errs
    e_g = np.linalg.norm(W - P_g @ Q_g)
    e_o = np.linalg.norm(W - P_o @ Q_o)
    assert abs(e_g - e_o) <= 1e-2 * e_o, (e_g, e_o)


def test_factor_at_the_drafter_head_size():
    """V = 151936, d = 5120, r = 128, q = 1 on the batch-1 workload's W: the
    columns of P are orthonormal (to bf16 precision) and P.Q approximates W
    at least as well as the generator's own rank-128 part P0.Q0 does."""
    inp, t = config(2)
    W = t["W"]
    d, r = W.shape[1], 128
    omega = torch.randn(d, r, generator=torch.Generator(DEV).manual_seed(1), device=DEV)
    say("[run] factor at V=151936 d=5120 r=128")
    P, Q = lr.factor(W, r, omega, 1)
    torch.cuda.synchronize()
    Pf, Qf, Wf = P.float(), Q.float(), W.float()
    gram = Pf.T @ Pf
    assert torch.allclose(gram, torch.eye(r, device=DEV), atol=2e-2), float((gram - torch.eye(r, device=DEV)).abs().max())
    rows = torch.arange(0, W.shape[0], 97, device=DEV)
    err = torch.linalg.norm(Wf[rows] - Pf[rows] @ Qf)
    planted = torch.linalg.norm(Wf[rows] - t["P"][rows].float() @ t["Q"].float())
    assert err <= 1.02 * planted, (float(err), float(planted))


# ------------------------------------------------ retrieval recall (f2)

RECALL_B, RECALL_K = (1, 4, 8), (8, 16, 32, 64)


def _recall_against_the_oracle(inp, t, rows):
    """recall(b, k) from the two GPU paths (lrhead_candidates, fullhead_topk)
    and from the oracle's own lists, row by row: equal on every row whose GPU
    lists are the oracle's; elsewhere the lists must differ from the
    oracle's by tie-band swaps only (the parity rule)."""
    from oracle import recall
    head = lr.Head(t["Q"], t["P"], t["W"], B_max=t["H"].shape[0], k_max=64)
    cidx, _ = head.candidates(t["H"], max(RECALL_K))
    fidx, flog = head.full_topk(t["H"], max(RECALL_B))
    torch.cuda.synchronize()
    c, f, fl = np_(cidx).astype(np.int64), np_(fidx).astype(np.int64), np_(flog)
    head.close()
    errs, _ = check_lowrank(inp, max(RECALL_K), c, None, None, rows=rows)
    assert not errs, errs[:4]
    errs, _ = check_full(inp, max(RECALL_B), f, fl, rows=rows)
    assert not errs, errs[:4]
    ref = recall.recall_sweep(inp["Q"], inp["P"], inp["W"], inp["H"], inp["cfg"].dtype, RECALL_B, RECALL_K,
                              rows=rows)
    got = recall.recall_table(c[rows], f[rows], RECALL_B, RECALL_K)
    n_diff = 0
    for eg, eo in zip(got, ref["table"]):
        b, k = eg["b"], eg["k"]
        for i in range(len(rows)):
            same = (set(c[rows[i], :k].tolist()) == set(ref["cand_idx"][i, :k].tolist())
                    and set(f[rows[i], :b].tolist()) == set(ref["full_idx"][i, :b].tolist()))
            if same:
                assert eg["hits"][i] == eo["hits"][i], (b, k, rows[i])
            else:
                n_diff += int(eg["hits"][i] != eo["hits"][i])
    say(f"[recall] " + " ".join(f"b{e['b']}k{e['k']}={e['recall']:.3f}" for e in got)
        + f" (rows differing by tie-band swaps: {n_diff})")
    return got


@pytest.mark.parametrize("r", [16, 32, 64])
def test_recall_from_the_gpu_paths_matches_the_oracle(r):
    inp = gen.make_custom(6000, 512, r, 24, "bf16", seed=r)
    t = {x: dev(inp[x], DEV) for x in ("Q", "P", "W", "H")}
    got = _recall_against_the_oracle(inp, t, np.arange(24))
    for e in got:   # at k = 64 of 6000 tokens the best full-head token is retrieved in most rows
        if e["b"] == 1 and e["k"] == 64:
            assert e["recall"] >= 0.5


@pytest.mark.timeout(600)
@pytest.mark.parametrize("cid", [2, 3])
def test_recall_at_the_drafter_head_size(cid):
    inp, t = config(cid)
    _recall_against_the_oracle(inp, t, np.arange(inp["H"].shape[0]))


# ------------------------------------------------ 4 GiB of full-head weights

@pytest.mark.timeout(900)
def test_full_head_with_4_gib_of_weights():
    # V * d * 2 bytes = 2^32: the batch path's tile copies size their buffer
    # to the block's tile, not to the rest of the matrix, so no size wraps.
    # Rows 0 .. 4 (the first tile) are planted as the rows' clear winners.
    V, d, B, k, r = 262144, 8192, 5, 8, 8
    g = torch.Generator(device=DEV).manual_seed(77)
    sd = 1.0 / math.sqrt(d)
    W = torch.empty(V, d, dtype=torch.bfloat16, device=DEV)
    for c0 in range(0, V, 16384):
        W[c0:c0 + 16384] = (torch.randn(16384, d, generator=g, device=DEV) * sd).to(torch.bfloat16)
    h = torch.randn(B, d, generator=g, device=DEV)
    H = (h / h.pow(2).mean(dim=1, keepdim=True).sqrt()).to(torch.bfloat16)
    W[:B] = (4.0 * H.float() * sd).to(torch.bfloat16)
    Q = (torch.randn(r, d, generator=g, device=DEV) * sd).to(torch.bfloat16)
    P = (torch.randn(V, r, generator=g, device=DEV) * sd).to(torch.bfloat16)
    head = lr.Head(Q, P, W, B_max=B, k_max=k)
    say("[run] full_topk, V=262144 d=8192 B=5")
    fidx, flog = head.full_topk(H, k)
    torch.cuda.synchronize()
    head.close()
    idx, lg = np_(fidx).astype(np.int64), np_(flog)
    assert idx[:, 0].tolist() == list(range(B))
    inp = {"cfg": gen.HeadConfig(0, "4 GiB W", B, d, V, r, k, "bf16", "iid"),
           "W": W.view(torch.int16).cpu().numpy().view(np.uint16),
           "H": H.view(torch.int16).cpu().numpy().view(np.uint16)}
    del W, P
    torch.cuda.empty_cache()
    errs, _ = check_full(inp, k, idx, lg)
    assert not errs, errs[:4]
