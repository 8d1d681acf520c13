"""Pins for the CPU oracle: each test checks it against something other than
itself -- hand-worked cases, closed forms of special cases, invariants that the
definitions force, brute force on tiny inputs, or a library routine."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import crisp_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ------------------------------------------------------------------ noise floor (hand-worked)

def test_noise_floor_golden_cases():
    g = json.load(open(os.path.join(GOLD, "noise_floor_cases.json")))
    for c in g["cases"]:
        p = np.array(c["p"], np.float32)
        mu = float(O.noise_floor_f32(p))
        assert abs(mu - c["mu"]) <= 1e-7, c
        sel = O.vs_select_direction(p, c["alpha"])
        assert sel.tolist() == c["selected"], c
    for c in g["min_blocks_cases"]:
        p = np.array(c["p"], np.float32)
        sel = O.vs_select_direction(p, c["alpha"], c["min_blocks"])
        assert sel.tolist() == c["selected"], c


def test_threshold_monotone_in_alpha():
    rng = np.random.default_rng(3)
    for _ in range(50):
        p = rng.dirichlet(np.full(40, 0.3)).astype(np.float32)
        prev = None
        for a in [0.25, 0.5, 1.0, 1.25, 1.5, 2.0, 4.0]:
            s = set(O.vs_select_direction(p, a).tolist())
            if prev is not None:
                assert s <= prev
            prev = s


def test_residual_rescale_keeps_selection_and_lowers_mu():
    """Moving mass from the non-anchor blocks onto the sink block scales every
    residual score and mu by the same factor: mu drops and the selected set is
    unchanged (the floor follows the sink, CRISP §4)."""
    rng = np.random.default_rng(5)
    for _ in range(30):
        nb = 50
        p = rng.dirichlet(np.full(nb, 0.5))
        p[0] += 0.2
        p /= p.sum()
        resid = 1 - p[0] - p[-1]
        f = 0.5                                   # half of the residual moves to the sink
        q = p.copy()
        q[1:-1] *= f
        q[0] += resid * (1 - f)
        mu_p = O.noise_floor_f32(p.astype(np.float32))
        mu_q = O.noise_floor_f32(q.astype(np.float32))
        assert mu_q < mu_p
        # away from float32 rounding at the threshold the sets agree
        thr = float(O.threshold_f32(p.astype(np.float32), 1.0))
        if np.min(np.abs(p[1:-1] - thr)) > 1e-5 * thr:
            assert O.vs_select_direction(p.astype(np.float32), 1.0).tolist() == \
                O.vs_select_direction(q.astype(np.float32), 1.0).tolist()


def test_vs_lists_golden():
    g = json.load(open(os.path.join(GOLD, "vs_lists_case.json")))
    lists = O.vs_block_lists(np.array(g["sv"]), np.array(g["ss"]), g["nb"])
    assert [l.tolist() for l in lists] == g["lists"]


def test_vs_lists_properties():
    rng = np.random.default_rng(7)
    for _ in range(20):
        nb = int(rng.integers(3, 60))
        sv = np.sort(rng.choice(nb, size=int(rng.integers(0, nb)), replace=False))
        ss = np.sort(rng.choice(nb, size=int(rng.integers(0, nb)), replace=False))
        lists = O.vs_block_lists(sv, ss, nb)
        for qb, l in enumerate(lists):
            assert l[0] == 0 and l[-1] == qb and np.all(np.diff(l) > 0)
            # membership by brute force over every key block
            for kb in range(qb + 1):
                want = kb in (0, qb) or kb in set(sv.tolist()) or (qb - kb) in set(ss.tolist())
                assert (kb in set(l.tolist())) == want


# ------------------------------------------------------------------ proxy attention

def test_proxy_rows_are_softmax_and_scores_sum_to_one():
    n, b, d = 1024, 128, 64
    q, k = _rand((b, d), 1), _rand((n, d), 2)
    A = O.proxy_attention(q, k)
    assert np.allclose(A.sum(1), 1.0, atol=1e-12)
    pos = n - b + np.arange(b)
    assert np.all(A[np.arange(n)[None, :] > pos[:, None]] == 0)
    assert abs(O.vertical_scores(A, b).sum() - 1) < 1e-12
    assert abs(O.slash_scores(A, b).sum() - 1) < 1e-12


def test_proxy_matches_literal_loops():
    n, b, d = 24, 4, 8
    q, k = _rand((b, d), 11), _rand((n, d), 12)
    A0, pv0, ps0, cs0 = O.proxy_literal(q, k, blk=4, w_sink=4, w_local=4)
    A = O.proxy_attention(q, k)
    assert np.allclose(A, A0, atol=1e-13)
    assert np.allclose(O.vertical_scores(A, 4), pv0, atol=1e-13)
    assert np.allclose(O.slash_scores(A, 4), ps0, atol=1e-13)
    assert abs(O.c_struct(A, 4, 4) - cs0) < 1e-13
    # uneven windows (not multiples of the block) through the same literal definition
    _, _, _, cs1 = O.proxy_literal(q, k, blk=4, w_sink=3, w_local=6)
    assert abs(O.c_struct(A, 3, 6) - cs1) < 1e-13


def test_proxy_zero_query_closed_form():
    """Q = 0: every proxy row is uniform over its q_r + 1 causal keys."""
    n, b, d = 1024, 128, 32
    A = O.proxy_attention(np.zeros((b, d)), _rand((n, d), 4))
    nb = n // b
    q = n - b + np.arange(b)
    pv_want = np.array([sum(max(0, min(q[r], (kb + 1) * b - 1) - kb * b + 1) / (q[r] + 1) for r in range(b)) / b
                        for kb in range(nb)])
    assert np.allclose(O.vertical_scores(A, b), pv_want, atol=1e-13)
    # diagonal o is present on row r iff o <= q_r, each with weight 1/(q_r+1)
    a_s = np.array([sum(1.0 / (q[r] + 1) for r in range(b) if o <= q[r]) / b for o in range(n)])
    assert np.allclose(O.slash_scores(A, b), a_s.reshape(nb, b).sum(1), atol=1e-13)
    cs_want = sum((b + r + 1) / (q[r] + 1) for r in range(b)) / b
    assert abs(O.c_struct(A, b, b) - cs_want) < 1e-13


def test_proxy_one_hot_limit():
    """A single overwhelming key takes all the mass: p^v and C_struct become indicators."""
    n, b, d = 1024, 128, 16
    q = np.zeros((b, d)); q[:, 0] = 1.0
    k = np.zeros((n, d))
    j = 300
    k[j, 0] = 1e4
    A = O.proxy_attention(q, k)
    pv = O.vertical_scores(A, b)
    want = np.zeros(n // b); want[j // b] = 1.0
    assert np.allclose(pv, want, atol=1e-12)
    ps = O.slash_scores(A, b)
    # row r puts its mass on offset q_r - j
    a_s = np.zeros(n)
    for r in range(b):
        a_s[n - b + r - j] += 1.0 / b
    assert np.allclose(ps, a_s.reshape(-1, b).sum(1), atol=1e-12)
    assert O.c_struct(A, b, b) < 1e-12


def test_c_struct_equals_anchor_blocks_of_vertical_score():
    """With w_sink = w_local = b the anchor windows are exactly the first and last block (CRISP §4)."""
    n, b, d = 2048, 128, 64
    A = O.proxy_attention(_rand((b, d), 8), _rand((n, d), 9))
    pv = O.vertical_scores(A, b)
    assert abs(O.c_struct(A, b, b) - (pv[0] + pv[-1])) < 1e-13


def test_route_rule_and_monotone_in_tau():
    assert O.route_decision(np.float32(0.3), 0.3)            # ">=": equality routes to VS
    assert not O.route_decision(np.nextafter(np.float32(0.3), np.float32(0)), 0.3)
    cs = np.random.default_rng(2).uniform(0, 1, 100).astype(np.float32)
    prev = None
    for tau in [0.1, 0.2, 0.3, 0.5, 0.8]:
        s = {i for i, c in enumerate(cs) if O.route_decision(c, tau)}
        if prev is not None:
            assert s <= prev
        prev = s


# ------------------------------------------------------------------ pooled estimation

def test_pe_probabilities_block_constant_inputs():
    """Inputs constant within each block pool to those constants, so P is the
    causal row softmax of the small constant matrix (scipy)."""
    from scipy.special import softmax
    nb, blk, d = 5, 4, 8
    qc, kc = _rand((nb, d), 21), _rand((nb, d), 22)
    q = np.repeat(qc, blk, axis=0)
    k = np.repeat(kc, blk, axis=0)
    P = O.pe_probabilities(q, k, blk)
    L = qc @ kc.T / math.sqrt(d)
    for qb in range(nb):
        assert np.allclose(P[qb, :qb + 1], softmax(L[qb, :qb + 1]), atol=1e-14)
        assert np.all(P[qb, qb + 1:] == 0)


def test_pe_cut_brute_force_minimum_cardinality():
    """The gamma-cumsum prefix solves FlexPrefill's dual problem (CRISP §2):
    among all subsets of causal entries whose mass reaches gamma*T it has the
    fewest elements, and no subset of that size carries more mass."""
    rng = np.random.default_rng(13)
    for trial in range(40):
        nb = int(rng.integers(2, 5))                       # at most 10 causal entries
        P = O.pe_probabilities(rng.standard_normal((nb * 2, 4)) * 3, rng.standard_normal((nb * 2, 4)) * 3, 2)
        gamma = float(rng.uniform(0.3, 0.99))
        qi, ki = np.tril_indices(nb)
        vals = P[qi, ki]
        T = vals.sum()
        best = None
        for r in range(1, vals.size + 1):
            masses = [sum(vals[list(c)]) for c in itertools.combinations(range(vals.size), r)]
            ok = [m for m in masses if m >= gamma * T]
            if ok:
                best = (r, max(ok))
                break
        _, info = O.pe_cut(P, gamma)
        assert info["kstar"] == best[0]
        assert abs(info["prefix"] - best[1]) < 1e-12


def test_pe_cut_gamma_limits_and_monotone():
    rng = np.random.default_rng(17)
    nb = 12
    P = O.pe_probabilities(rng.standard_normal((nb * 4, 8)), rng.standard_normal((nb * 4, 8)), 4)
    full, _ = O.pe_cut(P, 1.0)
    assert np.array_equal(full, np.tril(np.ones((nb, nb), bool)))
    prev = None
    for gamma in [0.1, 0.5, 0.8, 0.9, 0.95, 0.99, 1.0]:
        m, _ = O.pe_cut(P, gamma)
        assert np.all(m[np.arange(nb), 0]) and np.all(m[np.arange(nb), np.arange(nb)])
        assert not np.any(np.triu(m, 1))
        if prev is not None:
            assert np.all(m[prev])
        prev = m


def test_pe_cut_ties_go_to_lower_flat_index():
    """Two equal non-anchor entries (3,1) and (3,2) straddle the cut: the one
    with the lower row-major flat index is taken.  Sorted masses by hand:
    1, .5, .5, .4, .4, .4, .3, .2, .15, .15 (T = 4); gamma*T = 3.8 is first
    reached by the ninth entry."""
    P = np.array([[1.0, 0, 0, 0],
                  [0.5, 0.5, 0, 0],
                  [0.4, 0.2, 0.4, 0],
                  [0.3, 0.15, 0.15, 0.4]])
    m, info = O.pe_cut(P, 0.95)
    assert info["kstar"] == 9
    assert m[3, 1] and not m[3, 2]
    assert not O.pe_tie(info)        # 3.85 vs 3.8: far from the target, equal values are no tie
    _, info_t = O.pe_cut(P, 3.85 / 4)
    assert O.pe_tie(info_t)          # the target sits exactly on a prefix sum
    m2, info2 = O.pe_cut(P, 0.9)     # 3.6 reached by the eighth entry (0.2 at (2,1))
    assert info2["kstar"] == 8 and m2[2, 1] and not m2[3, 1] and not m2[3, 2]


def test_pe_cut_stops_at_first_prefix_reaching_target_exactly():
    """Dyadic masses make every prefix sum exact: sorted (value, flat index)
    1 (0,0); .5 (1,0) (1,1) (2,0) (3,3); .25 (2,1) (2,2) (3,1); .125 (3,0) (3,2)
    give prefix sums 1, 1.5, 2, 2.5, 3, 3.25, 3.5, 3.75, 3.875, 4 (T = 4).
    With gamma = 7/8, gamma*T = 3.5 equals the seventh prefix, and the pages
    stop accumulating once the mass reaches gamma [CRISP §2, PE path], so seven
    entries are kept and (3,1), the eighth, is not."""
    P = np.array([[1.0, 0, 0, 0],
                  [0.5, 0.5, 0, 0],
                  [0.5, 0.25, 0.25, 0],
                  [0.125, 0.25, 0.125, 0.5]])
    m, info = O.pe_cut(P, 0.875)
    assert info["kstar"] == 7 and info["prefix"] == 3.5 == info["target"]
    want = np.array([[1, 0, 0, 0],
                     [1, 1, 0, 0],
                     [1, 1, 1, 0],
                     [1, 0, 0, 1]], bool)                   # (3,0) is an anchor, (3,1) stays out
    assert np.array_equal(m, want)
    # a hair above 7/8 needs the eighth entry
    m8, info8 = O.pe_cut(P, float(np.nextafter(0.875, 1.0)))
    assert info8["kstar"] == 8 and m8[3, 1]
    # the same through the decision function, which takes gamma as the float32 parameter
    _, _, _, lists, info2 = O.decide_from_scores(0, np.float32(0), None, None, P.astype(np.float32), 4, 0.3, 1.0,
                                                 0.875)
    assert info2["kstar"] == 7 and [l.tolist() for l in lists] == [[0], [0, 1], [0, 1, 2], [0, 3]]


def test_coverage_cut_stops_at_first_prefix_reaching_target_exactly():
    """Scores .5 .25 .125 .125 (dyadic, exact sums): gamma = .75 is reached
    exactly by the first two blocks, so the budget is {0, 1} plus the anchor 3
    [CRISP §2, accumulated until the mass reaches gamma]."""
    p = np.array([0.5, 0.25, 0.125, 0.125], np.float32)
    keep, info = O.coverage_cut(p, 0.75)
    assert info["kstar"] == 2 and sorted(keep.tolist()) == [0, 1]
    sel, _ = O.vs_select_coverage(p, 0.75)
    assert sel.tolist() == [0, 1, 3]
    keep, info = O.coverage_cut(p, float(np.nextafter(0.75, 1.0)))
    assert info["kstar"] == 3


def test_jsd_router_at_equality():
    """The router sends a head to Vertical-Slash when JSD >= tau [CRISP §2]:
    identical distributions have JSD exactly 0, which meets tau = 0; a JSD equal
    to the float32 tau meets it, the next double below does not."""
    a = np.array([0.25, 0.25, 0.5])
    assert O.jsd(a, a) == 0.0 and O.route_jsd(O.jsd(a, a), 0.0)
    assert O.route_jsd(0.25, 0.25)
    assert not O.route_jsd(float(np.nextafter(0.25, 0.0)), 0.25)
    # tau is the float32 parameter: float32(0.1) is above 0.1, so JSD = 0.1 stays Pooled-Estimation
    assert not O.route_jsd(0.1, 0.1) and O.route_jsd(float(np.float32(0.1)), 0.1)


# ------------------------------------------------------------------ attention

def _sdpa(q, k, v):
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True)[0, 0].numpy()


def test_dense_attention_matches_library_sdpa():
    n, d = 256, 32
    q, k, v = _rand((n, d), 31), _rand((n, d), 32), _rand((n, d), 33)
    assert np.allclose(O.dense_causal_attention(q, k, v), _sdpa(q, k, v), atol=1e-12)


def test_all_blocks_selected_is_dense_attention():
    n, d, blk = 512, 32, 64
    q, k, v = _rand((n, d), 41), _rand((n, d), 42), _rand((n, d), 43)
    o = O.block_sparse_attention(q, k, v, O.dense_lists(n // blk), blk)
    assert np.allclose(o, _sdpa(q, k, v), atol=1e-12)


def test_block_sparse_matches_explicit_mask_matrix():
    n, d, blk = 96, 8, 8
    rng = np.random.default_rng(44)
    q, k, v = _rand((n, d), 45), _rand((n, d), 46), _rand((n, d), 47)
    nb = n // blk
    lists = []
    for qb in range(nb):
        s = {kb for kb in range(qb + 1) if rng.random() < 0.4}
        if qb % 3:                       # some rows without the diagonal block, one empty row
            s |= {qb}
        lists.append(sorted(s))
    lists[2] = []
    o = O.block_sparse_attention(q, k, v, lists, blk)
    M = O.mask_matrix(lists, n, blk)
    assert np.allclose(o, O.masked_attention_literal(q, k, v, M), atol=1e-12)


def test_attention_is_causal():
    n, d, blk = 256, 16, 32
    q, k, v = _rand((n, d), 51), _rand((n, d), 52), _rand((n, d), 53)
    lists = O.dense_lists(n // blk)
    o = O.block_sparse_attention(q, k, v, lists, blk)
    i = 150
    k2, v2 = k.copy(), v.copy()
    k2[i + 1:] += 5.0
    v2[i + 1:] -= 3.0
    o2 = O.block_sparse_attention(q, k2, v2, lists, blk)
    assert np.allclose(o[:i + 1], o2[:i + 1], atol=1e-14)
    assert not np.allclose(o[i + 1:], o2[i + 1:])


# ------------------------------------------------------------------ whole head on generated inputs

def test_select_head_on_tiny_generated_layer():
    """Tiny fp32 case: head 0 (sink + recency + 3 needles) routes to VS and keeps
    its needle blocks; head 1 (diffuse) routes to PE."""
    from workloads import synth
    spec = synth.make_spec(synth.TINY_FP32_4K)
    cfg = spec.cfg
    Q, K, V = synth.generate(spec)
    r0 = O.select_head(Q[0].astype(np.float64), K[0].astype(np.float64), 128, 128, 128, cfg.tau, cfg.alpha, cfg.gamma)
    assert r0["route"] == 1 and r0["c_struct"] >= cfg.tau
    for nb_id in spec.needle_blocks[0]:
        assert nb_id in set(r0["sv"].tolist())
    r1 = O.select_head(Q[1].astype(np.float64), K[1].astype(np.float64), 128, 128, 128, cfg.tau, cfg.alpha, cfg.gamma)
    assert r1["route"] == 0
    # decisions recomputed from float32-rounded scores agree with the float64 run
    rt, sv, ss, lists, _ = O.decide_from_scores(1, np.float32(r0["c_struct"]), r0["pv"], r0["ps"], None,
                                                cfg.nb, cfg.tau, cfg.alpha, cfg.gamma)
    assert rt == 1 and np.array_equal(sv, r0["sv"]) and np.array_equal(ss, r0["ss"])


def test_dense_fallback_cases():
    q, k = _rand((256, 16), 61), _rand((256, 16), 62)
    r = O.select_head(q, k, 128, 128, 128, 0.3, 1.0, 0.95)
    assert r["route"] == -1 and [l.tolist() for l in r["lists"]] == [[0], [0, 1]]
    q, k = _rand((512, 16), 63), _rand((512, 16), 64)
    r = O.select_head(q, k, 128, 128, 128, 0.3, 1.0, 0.95, dense_below_n=1024)
    assert r["route"] == -1


# ------------------------------------------------------------------ variants: median floor, coverage budget, JSD router

def test_median_floor_golden_cases():
    """Hand-worked: non-anchor scores .1 .2 .05 .3 have median (.1 + .2)/2 = .15,
    so alpha = 1 keeps blocks 2 (.2) and 4 (.3) plus the anchors; with an odd
    count .3 .1 .05 the median is .1 and only block 1 exceeds it."""
    p = np.array([0.5, 0.1, 0.2, 0.05, 0.3, 0.2], np.float32)
    assert O.median_floor_f32(p) == np.float32(0.15)
    assert O.vs_select_median(p, 1.0).tolist() == [0, 2, 4, 5]
    p = np.array([0.4, 0.3, 0.1, 0.05, 0.15], np.float32)
    assert O.median_floor_f32(p) == np.float32(0.1)
    assert O.vs_select_median(p, 1.0).tolist() == [0, 1, 4]
    assert O.vs_select_median(p, 0.4).tolist() == [0, 1, 2, 3, 4]     # .1 > .04, .05 > .04
    assert O.vs_select_median(p, 0.6).tolist() == [0, 1, 2, 4]        # .05 is not > .06


def test_median_floor_is_robust_to_one_dominant_block():
    """The pages' motivation for the median: one dominant block lifts the mean
    floor above a weak genuine block.  Here mu = (1 - .3 - .18)/9 = .0578 drops
    block 7 (.03) under the mean rule, while the median of the nine non-anchor
    scores is .01 and keeps it."""
    p = np.array([0.3, 0.4, 0.02, 0.02, 0.01, 0.01, 0.01, 0.03, 0.01, 0.01, 0.18], np.float32)
    assert abs(float(p.astype(np.float64).sum()) - 1.0) < 1e-6
    assert 7 not in O.vs_select_direction(p, 1.0).tolist()
    assert O.median_floor_f32(p) == np.float32(0.01)
    assert O.vs_select_median(p, 1.0).tolist() == [0, 1, 2, 3, 7, 10]


def test_median_floor_matches_library_median():
    rng = np.random.default_rng(71)
    for nb in [3, 4, 5, 64, 65, 1000]:
        p = rng.random(nb).astype(np.float32)
        ref = float(np.median(p[1:-1].astype(np.float64)))
        assert abs(float(O.median_floor_f32(p)) - ref) <= 2 * np.finfo(np.float32).eps * ref


def test_coverage_golden_and_ties():
    """Scores .5 .1 .2 .05 .3 .2 (sum 1.35), gamma .95: target 1.2825; sorted
    .5 .3 .2 .2 .1 reach 1.3 at the fifth entry, so every block but 3 is kept.
    Four equal scores with gamma .5: the two lowest indices are taken."""
    p = np.array([0.5, 0.1, 0.2, 0.05, 0.3, 0.2], np.float32)
    sel, info = O.vs_select_coverage(p, 0.95)
    assert sel.tolist() == [0, 1, 2, 4, 5] and info["kstar"] == 5
    q = np.array([0.25, 0.25, 0.25, 0.25, 0.0, 0.0], np.float32)
    keep, info = O.coverage_cut(q, 0.5)
    assert sorted(keep.tolist()) == [0, 1] and info["kstar"] == 2
    sel, _ = O.vs_select_coverage(q, 0.5)
    assert sel.tolist() == [0, 1, 5]                                   # anchors 0 and N_b - 1 added


def test_coverage_brute_force_minimum_cardinality():
    """The coverage prefix is a smallest subset reaching gamma of the mass, and
    no subset of that size carries more."""
    rng = np.random.default_rng(73)
    for trial in range(60):
        nb = int(rng.integers(3, 11))
        p = rng.dirichlet(np.full(nb, float(rng.uniform(0.2, 3.0))))
        gamma = float(rng.uniform(0.3, 0.99))
        T = p.sum()
        best = None
        for r in range(1, nb + 1):
            ok = [sum(p[list(c)]) for c in itertools.combinations(range(nb), r) if sum(p[list(c)]) >= gamma * T]
            if ok:
                best = (r, max(ok))
                break
        keep, info = O.coverage_cut(p, gamma)
        assert info["kstar"] == best[0] == len(keep)
        assert abs(info["prefix"] - best[1]) < 1e-12


def test_coverage_limits_and_monotone():
    rng = np.random.default_rng(79)
    p = rng.dirichlet(np.full(40, 0.5)).astype(np.float32)
    assert O.vs_select_coverage(p, 1.0)[0].tolist() == list(range(40))
    prev = set()
    for gamma in [0.1, 0.3, 0.6, 0.9, 0.95, 0.99]:
        s = set(O.vs_select_coverage(p, gamma)[0].tolist())
        assert {0, 39} <= s and prev <= s
        prev = s


def test_jsd_matches_library_and_limits():
    from scipy.spatial.distance import jensenshannon
    rng = np.random.default_rng(83)
    for trial in range(20):
        a = rng.dirichlet(np.ones(17))
        b = rng.dirichlet(np.ones(17) * 0.3)
        assert abs(O.jsd(a, b) - jensenshannon(a, b) ** 2) < 1e-12
        assert abs(O.jsd(a, b) - O.jsd(b, a)) < 1e-15
        assert O.jsd(a, a) == 0.0
    a = np.array([0.5, 0.5, 0.0, 0.0])
    b = np.array([0.0, 0.0, 0.25, 0.75])
    assert abs(O.jsd(a, b) - math.log(2.0)) < 1e-15                    # disjoint supports


def test_pooled_estimate_closed_forms():
    """Q = 0 gives the uniform distribution over blocks; adding one vector to
    every key shifts every pooled logit equally and changes nothing; a block
    whose mean key is a large multiple of the pooled query takes all the mass."""
    rng = np.random.default_rng(89)
    blk, nb, d = 4, 6, 8
    k = rng.standard_normal((nb * blk, d))
    q0 = np.zeros((blk, d))
    assert np.allclose(O.pooled_estimate(q0, k, blk), np.full(nb, 1.0 / nb), atol=1e-15)
    q = rng.standard_normal((blk, d))
    a = O.pooled_estimate(q, k, blk)
    assert abs(a.sum() - 1.0) < 1e-12
    assert np.allclose(O.pooled_estimate(q, k + rng.standard_normal(d), blk), a, atol=1e-12)
    k2 = k.copy()
    k2[2 * blk:3 * blk] += 200.0 * q.mean(axis=0) / np.linalg.norm(q.mean(axis=0))
    assert O.pooled_estimate(q, k2, blk)[2] > 1 - 1e-12
    # a logit gap far beyond exp's range still gives the exact one-hot limit (the
    # softmax is evaluated relative to its largest logit)
    k3 = k.copy()
    k3[4 * blk:5 * blk] += 1e5 * q.mean(axis=0) / np.linalg.norm(q.mean(axis=0))
    want = np.zeros(nb); want[4] = 1.0
    assert np.array_equal(O.pooled_estimate(q, k3, blk), want)


def test_pooled_estimate_block_constant_keys_library_softmax():
    """Keys constant within each block pool to those constants, and query rows
    c + e_r with sum_r e_r = 0 pool to c, so a_bar is the softmax (scipy) of
    K_const . c / sqrt(d) over the blocks [CRISP §2: softmax after pooling both
    queries and keys, at the attention scale].  The rows differ from one
    another, so pooling by a sum (b * c) or a dropped 1/sqrt(d) both move a_bar
    far outside the tolerance."""
    from scipy.special import softmax
    rng = np.random.default_rng(97)
    blk, nb, d = 4, 7, 16
    kc = rng.standard_normal((nb, d))
    k = np.repeat(kc, blk, axis=0)
    c = rng.standard_normal(d)
    e = rng.standard_normal((blk, d)) * 2.0
    e -= e.mean(axis=0)
    q = c[None, :] + e
    want = softmax(kc @ c / math.sqrt(d))
    got = O.pooled_estimate(q, k, blk)
    assert np.allclose(got, want, atol=1e-14)
    assert np.abs(softmax(kc @ c) - want).max() > 1e-2           # the scale matters on this input
    assert np.abs(softmax(kc @ (blk * c) / math.sqrt(d)) - want).max() > 1e-2   # and so does the mean


def test_jsd_router_threshold_and_variants_on_tiny_layer():
    """JSD routing is VS iff JSD >= tau, so the VS set shrinks as tau grows;
    the variants produce valid lists (ascending, anchors present, causal)."""
    from workloads import synth
    spec = synth.make_spec(synth.TINY_FP32_4K)
    cfg = spec.cfg
    Q, K, V = synth.generate(spec)
    js = []
    for h in range(2):
        q, k = Q[h].astype(np.float64), K[h].astype(np.float64)
        r = O.select_head(q, k, 128, 128, 128, 0.0, cfg.alpha, cfg.gamma, router="jsd", budget="coverage")
        assert r["route"] == 1 and 0.0 <= r["jsd"] <= math.log(2.0)
        js.append(r["jsd"])
        for budget in ["mean", "median", "coverage"]:
            r = O.select_head(q, k, 128, 128, 128, 0.0, cfg.alpha, cfg.gamma, router="jsd", budget=budget)
            for qb, l in enumerate(r["lists"]):
                assert l[0] == 0 and l[-1] == qb and np.all(np.diff(l) > 0)
    for tau in [0.0, min(js), max(js), max(js) + 1e-9]:
        vs = [O.route_jsd(j, tau) for j in js]
        assert vs == [j >= float(np.float32(tau)) for j in js]


def test_coverage_budget_grows_with_n_noise_floor_stays_flat():
    """The mass-cliff argument (CRISP §4): on a concentrated head whose anchors hold
    less than gamma of the proxy mass, a cumulative-coverage budget must take
    background blocks, whose per-block mass falls as 1/n, so it grows linearly in
    n; the noise floor (threshold at the mean non-anchor block) keeps the planted
    blocks only.  Head: the second concentrated query head of a KV group (its
    recency block is aligned with the group's first head, so its anchors are
    weaker), length-compensated generator, n = 4k .. 32k."""
    from workloads import synth
    cov_sizes = []
    for n in (4096, 8192, 16384, 32768):
        cfg = synth.custom_config("conc-pair", n, 2, 1, "fp32", seed=11, conc_frac=1.0, sink=(6.0, 6.0),
                                  needles=(3, 3))
        spec = synth.make_spec(cfg)
        assert spec.lead[0] == 0 and spec.concentrated[1]
        q = synth.rows(spec, "q", 1, n - 128, n).astype(np.float64)
        k = synth.rows(spec, "k", 0, 0, n).astype(np.float64)
        A = O.proxy_attention(q, k)
        pv = O.vertical_scores(A, 128).astype(np.float32)
        assert O.route_decision(np.float32(O.c_struct(A, 128, 128)), cfg.tau)   # a Vertical-Slash head
        floor = O.vs_select_direction(pv, cfg.alpha)
        planted = sorted({0, cfg.nb - 1, *spec.needle_blocks[0]})
        assert floor.tolist() == planted                                        # flat: the planted blocks
        cov = O.vs_select_coverage(pv, cfg.gamma)
        cov = cov[0] if isinstance(cov, tuple) else cov
        assert set(planted) <= set(np.asarray(cov).tolist())
        cov_sizes.append(len(cov))
    for a, b in zip(cov_sizes, cov_sizes[1:]):
        assert b >= 1.8 * a, cov_sizes                                          # ~doubles with n
    assert cov_sizes[0] > len(planted)
