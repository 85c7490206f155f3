"""Pins of the CPU oracle to facts outside itself.

The EAGLE-4 pages ("EAGLE-4", section "Retrieve vocabulary candidates cheaply,
then score them exactly") describe the head in words and print no worked
example, so every pin here is a closed form, a special case that reduces to
an independent routine, a brute force on tiny inputs, or an invariant. Each is
chosen so that a plausible slip in the oracle (a transposed operand, a missing
rounding of z, a reversed order, a wrong tie-break, a dropped term) fails at
least one of them.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import gen
import oracle
from oracle import compare


# ------------------------------------------------------------- helpers

def fsum_dot(a, b) -> float:
    # products of bf16/fp32 values are exact in float64; fsum rounds once
    return math.fsum((np.asarray(a, np.float64) * np.asarray(b, np.float64)).tolist())


def brute_topk(scores: list, k: int) -> list:
    """Repeatedly take the maximal score, lowest index on ties (plain loop)."""
    left = list(range(len(scores)))
    out = []
    for _ in range(k):
        best = left[0]
        for v in left[1:]:
            if scores[v] > scores[best]:
                best = v
        out.append(best)
        left.remove(best)
    return out


def precedes(s, u, v) -> bool:
    return s[u] > s[v] or (s[u] == s[v] and u < v)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    # bf16 bits of values that are already bf16-representable (small ints)
    return (np.asarray(x, np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ------------------------------------------------- rounding of z (reading)

def test_round_bf16_hand_cases():
    one = 1.0
    cases = [
        (1.0, 1.0),
        (one + 2.0 ** -8, 1.0),                       # halfway, even is 1.0
        (one + 3 * 2.0 ** -8, one + 2.0 ** -6),       # halfway, even is 1+2^-6
        (one + 2.0 ** -8 + 2.0 ** -20, one + 2.0 ** -7),  # just above halfway
        (-(one + 2.0 ** -8 + 2.0 ** -20), -(one + 2.0 ** -7)),
        (3.0, 3.0),
        (0.0, 0.0),
        (2.0 ** -100 * (1 + 2.0 ** -9), 2.0 ** -100),  # below halfway
    ]
    for x, want in cases:
        assert oracle.round_bf16(np.array([x]))[0] == want, x


def test_round_bf16_matches_torch():
    g = np.random.default_rng(7)
    x = g.standard_normal(200000).astype(np.float32)
    # force exact halfway cases: low 16 bits = 0x8000
    u = x.view(np.uint32).copy()
    u[:5000] = (u[:5000] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    x = u.view(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = oracle.round_bf16(x.astype(np.float64))
    assert np.array_equal(got, want.astype(np.float64))


def test_z_is_fp32_then_bf16():
    """O1 stores z as bf16(fp32(sum)), not as a single rounding of the sum."""
    Q = np.ones((1, 3))
    h_tie = np.array([[1.0, 2.0 ** -8, 2.0 ** -30]])     # fp32 drops 2^-30 -> tie
    h_up = np.array([[1.0, 2.0 ** -8, 2.0 ** -20]])      # fp32 keeps 2^-20 -> up
    assert oracle.down_projection(Q, h_tie, "bf16")[0, 0] == 1.0
    assert oracle.down_projection(Q, h_up, "bf16")[0, 0] == 1.0 + 2.0 ** -7
    assert oracle.down_projection(Q, h_tie, "fp32")[0, 0] == 1.0 + 2.0 ** -8
    # the product really is Q . h (not h . Q^T of the wrong operand)
    Q2 = np.array([[1.0, 2.0, 3.0], [0.0, -1.0, 4.0]])
    h2 = np.array([[1.0, 10.0, 100.0]])
    assert np.array_equal(oracle.down_projection(Q2, h2, "fp32")[0], [321.0, 390.0])


# --------------------------------------------- P1: exact factorisation r = d

@pytest.mark.parametrize("shape", ["c1", "c2_slice"])
def test_identity_factorisation_equals_full_head(shape):
    """Q = I_d, P = W~, E = 0: z~ = h~, scores = full-head logits."""
    if shape == "c1":
        inp = gen.make(1)
        W, H, dt, k = inp["W"], inp["H"], "fp32", 8
        eye = np.eye(W.shape[1], dtype=np.float32)
    else:
        inp = gen.make(2, with_W=False)
        cfg = inp["cfg"]
        # a W of c2's width: rows P~[v] . Q~ (bf16) on the first 2048 vocab rows
        Wf = oracle.to_f64(inp["P"][:2048], "bf16") @ oracle.to_f64(inp["Q"], "bf16")
        W = f32_to_bf16_bits(oracle.round_bf16(oracle.round_fp32(Wf)).astype(np.float32))
        H, dt, k = inp["H"], "bf16", cfg.k
        eye = f32_to_bf16_bits(np.eye(W.shape[1], dtype=np.float32))
    lr = oracle.lowrank_head(eye, W, W, H, k, dt, keep_scores=True)
    fh = oracle.full_head(W, H, k, dt, keep_logits=True)
    h64 = oracle.to_f64(H, dt)
    assert np.array_equal(lr["z"], h64)                 # z~ == h~ bit for bit
    assert np.array_equal(lr["idx"], fh["idx"])
    assert np.allclose(lr["logits"], lr["score"], rtol=1e-13, atol=0)
    # independent check: plain-loop fsum dot products and a selection loop
    w64 = oracle.to_f64(W, dt)
    exact = [fsum_dot(w64[v], h64[0]) for v in range(w64.shape[0])]
    assert brute_topk(exact, k) == lr["idx"][0].tolist()
    assert np.allclose(lr["logits"][0], [exact[v] for v in lr["idx"][0]], rtol=1e-12, atol=1e-15)


def test_orthogonal_factorisation_float64():
    """Random orthogonal Q, P = W Q^T, no rounding: candidates = full top-k."""
    g = np.random.default_rng(3)
    d, V, k = 48, 600, 10
    Qm, _ = np.linalg.qr(g.standard_normal((d, d)))
    W = g.standard_normal((V, d))
    P = W @ Qm.T
    H = g.standard_normal((3, d))
    lr = oracle.lowrank_head(Qm, P, W, H, k, "fp64", keep_scores=True)
    for b in range(3):
        exact = [fsum_dot(W[v], H[b]) for v in range(V)]
        assert lr["idx"][b].tolist() == brute_topk(exact, k)
        assert np.allclose(lr["s"][b], exact, rtol=0, atol=1e-12)
        assert np.allclose(lr["logits"][b], [exact[v] for v in lr["idx"][b]], atol=1e-12)


def test_rank_r_exact_head():
    """W = P Q exactly (rank r < d, orthonormal rows): same top-k as the full head."""
    g = np.random.default_rng(11)
    d, r, V, k = 64, 16, 400, 7
    Qm = np.linalg.qr(g.standard_normal((d, d)))[0][:r]
    P = g.standard_normal((V, r))
    W = P @ Qm
    H = g.standard_normal((2, d))
    lr = oracle.lowrank_head(Qm, P, W, H, k, "fp64")
    for b in range(2):
        exact = [fsum_dot(W[v], H[b]) for v in range(V)]
        assert lr["idx"][b].tolist() == brute_topk(exact, k)


# ----------------------------------------------- P2: brute force, tiny V

def test_bruteforce_subsets_with_ties():
    g = np.random.default_rng(5)
    for trial in range(25):
        V = int(g.integers(2, 13))
        r, d = int(g.integers(1, 4)), int(g.integers(1, 5))
        P = g.integers(-2, 3, (V, r)).astype(np.float32)
        Q = g.integers(-2, 3, (r, d)).astype(np.float32)
        H = g.integers(-2, 3, (1, d)).astype(np.float32)
        z = [fsum_dot(Q[j], H[0]) for j in range(r)]
        s = [fsum_dot(P[v], z) for v in range(V)]
        for k in range(1, V + 1):
            got = oracle.lowrank_head(Q, P, None, H, k, "fp32")["idx"][0].tolist()
            winners = [set(S) for S in itertools.combinations(range(V), k)
                       if all(precedes(s, u, v) for u in S for v in range(V) if v not in S)]
            assert len(winners) == 1
            assert set(got) == winners[0], (trial, k)
            assert all(precedes(s, got[j], got[j + 1]) for j in range(k - 1))


# ------------------------------------------------- P3: special cases

def test_k1_is_first_argmax_and_kV_is_total_order():
    g = np.random.default_rng(9)
    for _ in range(20):
        V, r = 50, 4
        P = g.integers(-3, 4, (V, r)).astype(np.float32)    # many exact ties
        Q = np.eye(r, dtype=np.float32)
        H = g.integers(-3, 4, (1, r)).astype(np.float32)
        lr = oracle.lowrank_head(Q, P, None, H, 1, "fp32", keep_scores=True)
        assert lr["idx"][0, 0] == int(np.argmax(lr["s"][0]))
        full = oracle.lowrank_head(Q, P, None, H, V, "fp32", keep_scores=True)
        order = full["idx"][0].tolist()
        s = full["s"][0]
        assert sorted(order) == list(range(V))
        assert all(precedes(s, order[j], order[j + 1]) for j in range(V - 1))


def test_batch_equals_stack_of_rows():
    inp = gen.make(1)
    H = np.concatenate([inp["H"], gen.make_lowrank_set(1, 1, B=3)["H"]])
    both = oracle.lowrank_head(inp["Q"], inp["P"], inp["W"], H, 8, "fp32")
    for b in range(H.shape[0]):
        one = oracle.lowrank_head(inp["Q"], inp["P"], inp["W"], H[b:b + 1], 8, "fp32")
        assert np.array_equal(one["idx"][0], both["idx"][b])
        assert np.array_equal(one["logits"][0], both["logits"][b])


# ------------------------------------------------- P4: invariants

def _double_bits(H, dt):
    if dt == "fp32":
        return (H * np.float32(2)).astype(np.float32)
    f = gen.bf16_bits_to_f32(H) * np.float32(2)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


@pytest.mark.parametrize("cid", [1, 2])
def test_scaling_h_by_two(cid):
    inp = gen.make(cid, with_W=(cid == 1))
    dt = inp["cfg"].dtype
    P = inp["P"] if cid == 1 else inp["P"][:20000]
    W = inp["W"]            # None for the bf16 case: z, ids and scores only
    a = oracle.lowrank_head(inp["Q"], P, W, inp["H"], inp["cfg"].k, dt)
    b = oracle.lowrank_head(inp["Q"], P, W, _double_bits(inp["H"], dt), inp["cfg"].k, dt)
    assert np.array_equal(b["z"], 2 * a["z"])
    assert np.array_equal(b["idx"], a["idx"])
    assert np.array_equal(b["score"], 2 * a["score"])
    if W is not None:
        assert np.array_equal(b["logits"], 2 * a["logits"])


def test_vocab_permutation_and_duplicate_rows():
    inp = gen.make(1)
    Q, P, W, H = inp["Q"], inp["P"], inp["W"], inp["H"]
    k = 8
    base = oracle.lowrank_head(Q, P, W, H, k, "fp32")
    assert base["gap"][0] > base["tau"][0]
    perm = np.random.default_rng(1).permutation(P.shape[0])
    moved = oracle.lowrank_head(Q, P[perm], W[perm], H, k, "fp32")
    assert set(perm[moved["idx"][0]].tolist()) == set(base["idx"][0].tolist())
    assert np.array_equal(perm[moved["idx"][0]], base["idx"][0])
    assert np.array_equal(moved["logits"][0], base["logits"][0])
    top = int(base["idx"][0, 0])
    # copy the best row to a higher and to a lower index: ties go low
    P_hi = P.copy(); P_hi[-1] = P[top]
    assert oracle.lowrank_head(Q, P_hi, None, H, 1, "fp32")["idx"][0, 0] == min(top, P.shape[0] - 1)
    two = oracle.lowrank_head(Q, P_hi, None, H, 2, "fp32")["idx"][0].tolist()
    assert two == [top, P.shape[0] - 1]
    if top > 0:
        P_lo = P.copy(); P_lo[0] = P[top]
        assert oracle.lowrank_head(Q, P_lo, None, H, 1, "fp32")["idx"][0, 0] == 0


def test_exact_logits_against_fsum():
    inp = gen.make(1)
    W64 = oracle.to_f64(inp["W"], "fp32")
    h64 = oracle.to_f64(inp["H"], "fp32")
    vs = np.array([0, 17, 4095, 2048])
    got = oracle.exact_logits(inp["W"], h64, np.zeros_like(vs), vs, "fp32")
    want = [fsum_dot(W64[v], h64[0]) for v in vs]
    assert np.allclose(got, want, rtol=1e-14, atol=1e-16)


def test_full_head_against_plain_loop():
    inp = gen.make(1)
    fh = oracle.full_head(inp["W"], inp["H"], 8, "fp32")
    W64 = oracle.to_f64(inp["W"], "fp32")
    h64 = oracle.to_f64(inp["H"], "fp32")[0]
    exact = [fsum_dot(W64[v], h64) for v in range(W64.shape[0])]
    assert fh["idx"][0].tolist() == brute_topk(exact, 8)
    assert np.allclose(fh["logits"][0], [exact[v] for v in fh["idx"][0]], rtol=1e-13)


# ------------------------------------------------- P5: generator statistics

def test_generator_statistics():
    c = gen.make(5, with_W=False, B=256)
    cfg = c["cfg"]
    std = 1 / math.sqrt(cfg.d)
    Q64 = oracle.to_f64(c["Q"], "bf16")
    P64 = oracle.to_f64(c["P"], "bf16")
    H64 = oracle.to_f64(c["H"], "bf16")
    assert abs(Q64.std() / std - 1) < 0.01
    assert abs(P64.std() / std - 1) < 0.01
    assert np.allclose(np.sqrt(np.mean(H64 ** 2, axis=1)), 1.0, atol=4e-3)
    z = oracle.down_projection(Q64, H64, "bf16")
    assert abs(z.std() - 1) < 0.03
    s = oracle.vocab_scores(P64[:20000], z[:32])
    assert abs(s.std() / math.sqrt(cfg.r / cfg.d) - 1) < 0.03
    t = gen.make(4, with_W=False)
    H4 = oracle.to_f64(t["H"], "bf16")
    par = t["parents"]
    assert par[0] == -1 and all(0 <= par[i] < i for i in range(1, 64))
    corr = [np.corrcoef(H4[i], H4[par[i]])[0, 1] for i in range(1, 64)]
    assert abs(np.mean(corr) - 0.8) < 0.03
    one = gen.make(1)
    resid = oracle.to_f64(one["W"], "fp32") - oracle.to_f64(one["P"], "fp32") @ oracle.to_f64(one["Q"], "fp32")
    assert abs(resid.std() / (0.1 / math.sqrt(256)) - 1) < 0.02


def test_generator_is_reproducible_and_chunk_independent():
    a = gen.make(1)
    b = gen.make(1)
    for key in ("Q", "P", "W", "H"):
        assert np.array_equal(a[key], b[key])
    # a W row depends only on its chunk's seed, not on the thread schedule
    rows = gen._make_W(a["P"], a["Q"], np.random.SeedSequence(1001).spawn(5)[2], a["cfg"])
    assert np.array_equal(rows, a["W"])


# ------------------------------------------------- the comparison rule itself

def test_comparison_rule_catches_planted_mistakes():
    inp = gen.make(1)
    lr = oracle.lowrank_head(inp["Q"], inp["P"], inp["W"], inp["H"], 8, "fp32", keep_scores=True)
    s, idx = lr["s"][0], lr["idx"][0]
    tau, gap, s_k = lr["tau"][0], lr["gap"][0], lr["s_k"][0]
    ok = compare.check_candidates(idx, s, idx, tau, gap, s_k)
    assert ok == []
    far = idx.copy(); far[3] = int(np.argmin(s))
    assert compare.check_candidates(far, s, idx, tau, gap, s_k)
    dup = idx.copy(); dup[1] = dup[0]
    assert compare.check_candidates(dup, s, idx, tau, gap, s_k)
    rev = idx[::-1].copy()
    if abs(s[idx[0]] - s[idx[-1]]) > tau:
        assert compare.check_candidates(rev, s, idx, tau, gap, s_k)
    # inside the band, swapping the k-th with the (k+1)-th is allowed
    order = np.argsort(-s, kind="stable")
    s_band = s.copy(); s_band[order[8]] = s_k - tau / 2      # (k+1)-th inside the band
    swapped = idx.copy(); swapped[-1] = order[8]
    assert compare.check_candidates(swapped, s_band, idx, tau, tau / 2, s_k) == []
    s_band[order[8]] = s_k - 2 * tau                          # now outside: not allowed
    assert compare.check_candidates(swapped, s_band, idx, tau, 2 * tau, s_k)
    ex = lr["logits"][0]
    assert compare.check_logits(ex * (1 + 1e-6), ex, "fp32") == []
    assert compare.check_logits(ex * (1 + 3e-5), ex, "fp32")
    assert compare.check_logits(ex * (1 + 1e-3), ex, "bf16") == []
    assert compare.check_logits(ex * (1 + 3e-3), ex, "bf16")


def test_score_allowance_covers_one_bf16_step_of_z_and_no_more():
    """The score diagnostic allows one bf16 step in one component of the
    stored z (an fp32 accumulation order other than exact-then-round may
    round the other way), and still catches larger errors."""
    import torch
    # ulp_bf16 against torch's bf16 spacing: nextafter in bf16 via the bit pattern
    x = np.array([1.0, -1.5976550329942256, 0.06, 3.0e-3, 200.0])
    xb = torch.tensor(x, dtype=torch.float64).to(torch.bfloat16)
    nxt = (xb.view(torch.int16) + 1).view(torch.bfloat16).to(torch.float64)
    spacing = (nxt - xb.to(torch.float64)).abs().numpy()
    assert np.array_equal(compare.ulp_bf16(xb.to(torch.float64).numpy()), spacing)
    assert compare.ulp_bf16(np.array([0.0]))[0] == 0.0
    inp = gen.make_custom(3000, 512, 64, 1, "bf16", seed=21)
    lr = oracle.lowrank_head(inp["Q"], inp["P"], None, inp["H"], 16, "bf16", keep_scores=True)
    z, s, idx = lr["z"][0], lr["s"][0], lr["idx"][0]
    P = oracle.to_f64(inp["P"], "bf16")
    allow = compare.z_step_allowance(P[idx], z, "bf16")
    smax = float(np.max(np.abs(s)))
    # the component whose single step moves the candidates' scores most
    j = int(np.argmax(np.max(np.abs(P[idx]) * compare.ulp_bf16(z)[None, :], axis=0)))
    for steps, ok in ((1, True), (-1, True), (4, False)):
        z2 = z.copy()
        z2[j] += steps * compare.ulp_bf16(z[j:j + 1])[0]
        got = P[idx] @ z2
        errs = compare.check_scores(got, s[idx], smax, "bf16", allow)
        assert (errs == []) == ok, (steps, errs)
    # without the allowance the one-step case is not always within the base tolerance
    z2 = z.copy(); z2[j] += compare.ulp_bf16(z[j:j + 1])[0]
    assert np.max(np.abs(P[idx] @ z2 - s[idx])) <= compare.SCORE_TOL["bf16"] * smax + np.max(allow)
    assert compare.z_step_allowance(P[idx], z, "fp32").max() == 0.0


def test_selection_stats_hand_row():
    s = np.array([-5.0, 1.0, 2.0, 1.0])
    idx = oracle.topk_order(s, 2)
    assert idx.tolist() == [2, 1]                  # tie 1.0 at ids 1 and 3: lower first
    st = oracle.selection_stats(s, idx)
    assert st["s_k"] == 1.0 and st["s_k1"] == 1.0 and st["gap"] == 0.0
    assert st["tau"] == 5e-3                       # 1e-3 * max |s|, the |-5| counts
    st1 = oracle.selection_stats(s, oracle.topk_order(s, 1))
    assert st1["gap"] == 1.0
    st4 = oracle.selection_stats(s, oracle.topk_order(s, 4))
    assert st4["s_k1"] == -np.inf


def test_golden_snapshot_of_tiny_config():
    """The oracle still reproduces the snapshot written by tests/golden/make_golden.py."""
    import json, os
    path = os.path.join(os.path.dirname(__file__), "golden", "c1_oracle.json")
    snap = json.load(open(path))
    inp = gen.make(1)
    lr = oracle.lowrank_head(inp["Q"], inp["P"], inp["W"], inp["H"], 8, "fp32")
    fh = oracle.full_head(inp["W"], inp["H"], 8, "fp32")
    assert lr["idx"].tolist() == snap["lowrank_idx"]
    assert np.allclose(lr["logits"], snap["lowrank_logits"], rtol=1e-15, atol=0)
    assert np.allclose(lr["score"], snap["lowrank_score"], rtol=1e-15, atol=0)
    assert fh["idx"].tolist() == snap["full_idx"]
    assert np.allclose(fh["logits"], snap["full_logits"], rtol=1e-15, atol=0)


# ------------------------------------------- draft distribution (D1-D3)

def test_distribution_uniform_logits_give_one_over_k_and_id_order():
    """Equal logits: every probability is 1/k and the branches come in token-id order."""
    k = 7
    ids = np.array([[40, 3, 17, 9, 100, 5, 66]])
    p, bi, bp, bpath = oracle.branches(np.full((1, k), 2.5), ids, 3, parent=np.array([0.5]))
    assert np.allclose(p, 1.0 / k, rtol=0, atol=1e-15)
    assert bi[0].tolist() == [3, 5, 9]
    assert np.allclose(bp, 1.0 / k) and np.allclose(bpath, 0.5 / k)


def test_distribution_of_log_weights_is_the_normalised_weights():
    """Logits log(w_j): p_j = w_j / sum(w) exactly (closed form of the softmax)."""
    w = np.array([1.0, 2.0, 3.0, 4.0, 10.0])
    ids = np.array([[11, 12, 13, 14, 15]])
    p, bi, bp, _ = oracle.branches(np.log(w)[None, :], ids, 2)
    assert np.allclose(p[0], w / w.sum(), rtol=1e-14, atol=0)
    assert bi[0].tolist() == [15, 14]
    assert np.allclose(bp[0], [10 / 20, 4 / 20], rtol=1e-14)


def test_distribution_is_shift_invariant_and_sums_to_one():
    rng = np.random.default_rng(3)
    l = rng.normal(size=(5, 32)) * 3
    ids = np.tile(np.arange(32), (5, 1))
    p1 = oracle.draft_distribution(l)
    p2 = oracle.draft_distribution(l + 1000.0)   # large shift: only the max-subtracted form survives it
    assert np.allclose(p1, p2, rtol=1e-12, atol=1e-300)
    assert np.allclose(p1.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    # nb = k orders every candidate by probability
    _, bi, bp, _ = oracle.branches(l, ids, 32)
    assert all(np.all(np.diff(bp[b]) <= 0) for b in range(5))
    assert all(sorted(bi[b].tolist()) == list(range(32)) for b in range(5))
    # nb = 1 is the argmax (first maximum)
    _, b1, _, _ = oracle.branches(l, ids, 1)
    assert b1[:, 0].tolist() == np.argmax(l, axis=1).tolist()


def test_distribution_empty_slots_get_nothing():
    """NaN logits (empty candidate slots) get probability 0 and are never branches."""
    l = np.array([[0.0, np.nan, np.log(3.0), np.nan]])
    ids = np.array([[7, 0x7FFFFFFF, 9, 0x7FFFFFFF]])
    p, bi, bp, _ = oracle.branches(l, ids, 4)
    assert np.allclose(p[0], [0.25, 0.0, 0.75, 0.0], rtol=1e-15, atol=0)
    assert bi[0].tolist() == [9, 7, -1, -1] and bp[0].tolist() == [0.75, 0.25, 0.0, 0.0]


def test_distribution_against_a_plain_loop():
    """D1 written out element by element with math.exp and math.fsum."""
    rng = np.random.default_rng(4)
    l = rng.normal(size=(3, 9))
    p = oracle.draft_distribution(l)
    for b in range(3):
        m = max(l[b])
        e = [math.exp(x - m) for x in l[b]]
        s = math.fsum(e)
        assert np.allclose(p[b], [x / s for x in e], rtol=1e-15, atol=0)


# ------------------------------------------------ building P and Q (F1-F4)

def _spectrum_matrix(rng, V, d, sigma):
    """U diag(sigma) V^T with random orthonormal U (V x n), V (d x n)."""
    n = len(sigma)
    U, _ = np.linalg.qr(rng.normal(size=(V, n)))
    Vt, _ = np.linalg.qr(rng.normal(size=(d, n)))
    return (U * np.asarray(sigma)) @ Vt.T


def test_factor_recovers_an_exactly_low_rank_w():
    """W of rank r exactly: P.Q = W (before the final rounding), P orthonormal."""
    from oracle import factor as fa
    rng = np.random.default_rng(11)
    V, d, r = 600, 80, 12
    W = rng.normal(size=(V, r)) @ rng.normal(size=(r, d))
    omega = rng.normal(size=(d, r))
    for q in (0, 1):
        P, Q = fa.factor(W, omega, q, "fp64", round_out=False)
        assert np.allclose(P @ Q, W, rtol=0, atol=1e-9 * np.abs(W).max())
        assert np.allclose(P.T @ P, np.eye(r), atol=1e-12)


def test_factor_error_approaches_the_truncated_svd_optimum():
    """A known decaying spectrum: the error of P.Q is at least the Eckart-Young
    optimum sqrt(sum of the discarded sigma^2) (numpy.linalg.svd agrees with
    the construction) and comes within 2% of it after two iterations."""
    from oracle import factor as fa
    rng = np.random.default_rng(12)
    V, d, r = 500, 120, 10
    sigma = 1.0 / (1.0 + np.arange(60)) ** 1.2
    W = _spectrum_matrix(rng, V, d, sigma)
    s_np = np.linalg.svd(W, compute_uv=False)
    assert np.allclose(s_np[:60], sigma, rtol=1e-10)
    opt = math.sqrt(float(np.sum(sigma[r:] ** 2)))
    omega = rng.normal(size=(d, r))
    errs = []
    for q in (0, 1, 2):
        P, Q = fa.factor(W, omega, q, "fp64", round_out=False)
        errs.append(np.linalg.norm(W - P @ Q))
        assert errs[-1] >= opt * (1 - 1e-12)
    assert errs[2] <= errs[0] and errs[2] <= 1.02 * opt, (errs, opt)


def test_factor_orth_is_cholesky_qr2():
    """orth() returns orthonormal columns spanning the input (its R factor is
    triangular), checked against numpy's Householder QR."""
    from oracle import factor as fa
    rng = np.random.default_rng(13)
    X = rng.normal(size=(300, 9)) * np.logspace(0, 3, 9)    # condition number ~1e3
    Y = fa.orth(X)
    assert np.allclose(Y.T @ Y, np.eye(9), atol=1e-13)
    Qh, _ = np.linalg.qr(X)
    assert np.allclose(np.abs(Y.T @ Qh), np.eye(9), atol=1e-10)    # same columns up to sign


# ------------------------------------------------ retrieval recall (f2)

def test_recall_hand_intersections():
    from oracle import recall
    cand = np.array([[3, 1, 2, 7], [0, 5, 6, 9]])
    full = np.array([[1, 5, 4], [6, 0, 2]])
    # row 0: {1, 5} & {3, 1, 2} = {1}; row 1: {6, 0} & {0, 5, 6} = {0, 6}
    assert recall.recall_hits(cand, full, 2, 3).tolist() == [1, 2]
    # row 0: {1, 5, 4} & {3, 1, 2, 7} = {1}; row 1: {6, 0, 2} & {0, 5, 6, 9} = {0, 6}
    assert recall.recall_hits(cand, full, 3, 4).tolist() == [1, 2]
    t = recall.recall_table(cand, full, [1], [1, 4])
    assert [(e["b"], e["k"], e["recall"]) for e in t] == [(1, 1, 0.0), (1, 4, 1.0)]
    with pytest.raises(ValueError):
        recall.recall_hits(cand, full, 4, 2)


def test_recall_of_an_exactly_factorised_head_is_min_k_b_over_b():
    # small integers: W = P.Q, z = Q.h and both stages are exact in fp32, so
    # the low-rank scores are the full logits and the two orders coincide
    from oracle import recall
    rng = np.random.default_rng(5)
    V, d, r, n = 40, 6, 6, 5
    Q = rng.integers(-3, 4, (r, d)).astype(np.float32)
    P = rng.integers(-3, 4, (V, r)).astype(np.float32)
    W = (P.astype(np.float64) @ Q.astype(np.float64)).astype(np.float32)
    H = rng.integers(-3, 4, (n, d)).astype(np.float32)
    sw = recall.recall_sweep(Q, P, W, H, "fp32", bs=[1, 3, 5], ks=[1, 2, 3, 5, 8, 40])
    for e in sw["table"]:
        assert e["recall"] == min(e["k"], e["b"]) / e["b"], e


def test_recall_of_a_negated_head_has_its_closed_form():
    # P = -W with Q = I: the low-rank order is the full order reversed, so
    # F_b and C_k overlap in max(0, k - (V - b)) tokens (no ties: continuous W)
    from oracle import recall
    rng = np.random.default_rng(11)
    V, d, n = 12, 5, 4
    W = rng.standard_normal((V, d)).astype(np.float32)
    P = -W
    Q = np.eye(d, dtype=np.float32)
    H = rng.standard_normal((n, d)).astype(np.float32)
    sw = recall.recall_sweep(Q, P, W, H, "fp32", bs=[1, 3, 5], ks=list(range(1, V + 1)))
    for e in sw["table"]:
        assert e["recall"] == max(0, e["k"] - (V - e["b"])) / e["b"], e


def test_recall_is_one_at_k_equals_v_and_grows_with_k():
    from oracle import recall
    inp = gen.make_custom(300, 64, 8, 6, "bf16", seed=3)
    ks = [1, 2, 4, 8, 16, 32, 64, 128, 300]
    sw = recall.recall_sweep(inp["Q"], inp["P"], inp["W"], inp["H"], "bf16", bs=[1, 4, 8], ks=ks)
    by_b = {}
    for e in sw["table"]:
        by_b.setdefault(e["b"], []).append(e["recall"])
    for b, rs in by_b.items():
        assert rs[-1] == 1.0
        assert all(x <= y for x, y in zip(rs, rs[1:])), (b, rs)
    # the oracle's lists are its own O3 / O5 orders
    assert np.array_equal(sw["cand_idx"], oracle.lowrank_head(inp["Q"], inp["P"], None, inp["H"], 300, "bf16")["idx"])
