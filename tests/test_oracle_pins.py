"""Pins of the CPU oracle to facts the page and the mathematics fix.

Page: chzhyang.github.io, "大模型投机解码：Medusa、MTP、EAGLE、DFlash、DDTree 与 DSpark",
cited as [SD §n]. Each test names the fact it checks. None of them re-types the
oracle's own formula: they use a worked example, closed forms, distribution tests,
library routines for special cases and brute force on tiny inputs.
"""
import itertools
import json
import math
import os
import zlib

import numpy as np
import pytest
from scipy import special, stats

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def logits_of(probs):
    with np.errstate(divide="ignore"):
        return np.log(np.asarray(probs, dtype=np.float64)).astype(np.float32)


def sample_from(rng, probs, n):
    """n iid draws from a discrete distribution (test-side sampler)."""
    c = np.cumsum(np.asarray(probs, dtype=np.float64))
    c /= c[-1]
    return np.minimum(np.searchsorted(c, rng.random(n), side="right"), len(c) - 1).astype(np.int32)


def grid_u(rng, shape):
    return (rng.integers(0, 1 << 24, size=shape) / float(1 << 24)).astype(np.float32)


# --------------------------------------------------------------------------
# Distribution shaping: special cases that reduce to a library routine.
# --------------------------------------------------------------------------

def test_transform_matches_scipy_softmax():
    rng = np.random.default_rng(7)
    for T in (1.0, 0.7, 2.5):
        x = (rng.standard_normal(257) * 3).astype(np.float32)
        ok, p = oracle.transform_row(x, T)
        ref = special.softmax(x.astype(np.float64) / np.float64(np.float32(T)))
        assert ok
        np.testing.assert_allclose(p, ref, rtol=1e-12, atol=0)


def test_transform_topk_keeps_exactly_k_lowest_id_on_ties():
    # ids 3, 5, 8 tie at the kth value; k = 4 keeps the best (id 1) and 3, 5, 8 ... then
    # with k = 3 only ids 1, 3, 5 survive (lower ids win the tie).
    x = np.full(10, -1.0, np.float32)
    x[1] = 5.0
    x[[3, 5, 8]] = 2.0
    ok, p = oracle.transform_row(x, 1.0, top_k=3)
    assert ok
    assert set(np.nonzero(p)[0].tolist()) == {1, 3, 5}
    ref = special.softmax(np.array([5.0, 2.0, 2.0]))
    np.testing.assert_allclose(p[[1, 3, 5]], ref, rtol=1e-12)
    # top_k = 1 is one-hot at the lowest-id maximum
    y = np.array([0.0, 3.0, 1.0, 3.0], np.float32)
    ok, p = oracle.transform_row(y, 0.3, top_k=1)
    assert ok and p.tolist() == [0.0, 1.0, 0.0, 0.0]
    # top_k >= V and top_k == 0 are both "off"
    ok0, p0 = oracle.transform_row(y, 0.3, top_k=0)
    ok1, p1 = oracle.transform_row(y, 0.3, top_k=4)
    np.testing.assert_array_equal(p0, p1)
    np.testing.assert_allclose(p0, special.softmax(y.astype(np.float64) / np.float64(np.float32(0.3))), rtol=1e-12)


def test_transform_neg_inf_and_nonfinite_rows():
    x = np.array([-np.inf, 0.0, -np.inf, 0.0], np.float32)
    ok, p = oracle.transform_row(x, 1.0)
    assert ok and p.tolist() == [0.0, 0.5, 0.0, 0.5]
    for bad in ([-np.inf] * 4, [0.0, np.nan, 1.0, 2.0], [0.0, np.inf, 1.0, 2.0]):
        ok, p = oracle.transform_row(np.array(bad, np.float32), 1.0)
        assert not ok and not p.any()
    # top-k never keeps NaN: a NaN outside the kept set leaves the row valid
    ok, p = oracle.transform_row(np.array([0.0, np.nan, 1.0, 2.0], np.float32), 1.0, top_k=2)
    assert ok
    np.testing.assert_allclose(p, [0, 0, *special.softmax([1.0, 2.0])], rtol=1e-12)


def test_argmax_lowest_id_and_nan():
    assert oracle.argmax_row(np.array([1, 4, 4, 2], np.float32)) == 1
    assert oracle.argmax_row(np.array([np.nan, -np.inf, -np.inf], np.float32)) == 1
    assert oracle.argmax_row(np.array([np.nan, np.nan], np.float32)) == -1
    rng = np.random.default_rng(3)
    x = rng.standard_normal(1000).astype(np.float32)
    assert oracle.argmax_row(x) == int(np.argmax(x))


# --------------------------------------------------------------------------
# [SD §1] worked example: A B C D -> A B R.
# --------------------------------------------------------------------------

def test_worked_example_golden():
    g = json.load(open(os.path.join(GOLD, "worked_example.json")))
    V = g["V"]
    tgt = np.stack([logits_of(r) for r in g["target_probs"]])
    dft = np.stack([logits_of(r) for r in g["draft_probs"]])
    y = np.array(g["draft_tokens"], np.int32)
    for u in g["uniform_sets"]:
        out = oracle.verify_chain(tgt, dft, y, np.array(u, np.float32), None, 1, len(y), V, 1.0)
        A, nxt = int(out["A"][0]), int(out["next"][0])
        committed = y[:A].tolist() + [nxt]
        assert A == g["expected"]["accepted_len"]
        assert nxt == g["expected"]["next_token"]
        assert committed == g["expected"]["committed"]
        assert 3 not in committed          # D is never kept
        assert out["status"][0] == 0


def test_truncation_property_random():
    """Nothing after the first rejection is used: changing the rows and the
    tokens after position A changes neither A nor the final token."""
    rng = np.random.default_rng(11)
    B, K, V = 400, 5, 12
    tgt = (rng.standard_normal((B * (K + 1), V)) * 2).astype(np.float32)
    dft = (rng.standard_normal((B * K, V)) * 2).astype(np.float32)
    y = rng.integers(0, V, B * K).astype(np.int32)
    u = grid_u(rng, B * (K + 1))
    out = oracle.verify_chain(tgt, dft, y, u, None, B, K, V, 1.0)
    tgt2, dft2, y2 = tgt.copy(), dft.copy(), y.copy()
    for b in range(B):
        A = int(out["A"][b])
        if A < K:
            # scramble every later draft position (rows A+1.., tokens A+1..) and later target rows
            for i in range(A + 1, K):
                dft2[b * K + i] = rng.standard_normal(V) * 5
                y2[b * K + i] = rng.integers(0, V)
            for i in range(A + 1, K + 1):
                tgt2[b * (K + 1) + i] = rng.standard_normal(V) * 5
    out2 = oracle.verify_chain(tgt2, dft2, y2, u, None, B, K, V, 1.0)
    np.testing.assert_array_equal(out["A"], out2["A"])
    np.testing.assert_array_equal(out["next"], out2["next"])
    assert (out["A"] < K).any() and (out["A"] == K).any()


# --------------------------------------------------------------------------
# [SD §1] distribution-identical sampling: chi-square on tiny vocabularies.
# --------------------------------------------------------------------------

def _chi2_ok(obs, expected_p, n, pmin=1e-3):
    expected_p = np.asarray(expected_p, dtype=np.float64)
    zero = expected_p == 0
    assert obs[zero].sum() == 0, "a zero-probability token was emitted"
    e = expected_p[~zero] * n
    o = obs[~zero]
    if len(o) < 2:
        return True
    stat, pv = stats.chisquare(o, e)
    return pv >= pmin


CHI_CASES = {
    # name: (p rows [K+1], q rows [K])
    "q_equals_p": ([[.1, .2, .3, .4], [.25, .25, .25, .25], [.7, .1, .1, .1], [.4, .3, .2, .1]],
                   [[.1, .2, .3, .4], [.25, .25, .25, .25], [.7, .1, .1, .1]]),
    "q_uniform": ([[.05, .15, .5, .3, 0, 0], [.6, .1, .1, .1, .05, .05], [0, 0, 0, .5, .5, 0], [.3, .3, .1, .1, .1, .1]],
                  [[1 / 6] * 6, [1 / 6] * 6, [1 / 6] * 6]),
    "q_one_hot": ([[.2, .3, .5], [.5, .25, .25], [.1, .1, .8], [.3, .3, .4]],
                  [[0, 1, 0], [1, 0, 0], [0, 0, 1]]),
    "disjoint_support": ([[.5, .5, 0, 0], [0, .2, .8, 0], [.25, .25, .25, .25], [.1, .2, .3, .4]],
                         [[0, 0, .5, .5], [.9, 0, 0, .1], [.25, .25, .25, .25]]),
    "disjoint_later": ([[.4, .3, .2, .1], [0, .2, .8, 0], [.25, .25, .25, .25], [.1, .2, .3, .4]],
                       [[.1, .2, .3, .4], [.9, 0, 0, .1], [.25, .25, .25, .25]]),
    "zeros_both_sides": ([[0, .3, .7, 0, 0, 0, 0, 0], [.1, 0, 0, .4, .5, 0, 0, 0], [0, 0, 0, 0, 0, 0, .5, .5],
                          [.125] * 8],
                         [[.5, .5, 0, 0, 0, 0, 0, 0], [0, 0, .2, .3, .5, 0, 0, 0], [0, 0, 0, 0, 0, .2, .3, .5]]),
}


@pytest.mark.parametrize("name", sorted(CHI_CASES))
def test_chi_square_outputs_follow_target(name):
    P, Q = CHI_CASES[name]
    K = len(Q)
    V = len(P[0])
    n = 400_000
    rng = np.random.default_rng(zlib.crc32(name.encode()))     # the same seed in every process
    tgt_row = np.stack([logits_of(r) for r in P])
    dft_row = np.stack([logits_of(r) for r in Q])
    tgt = np.tile(tgt_row, (n, 1))
    dft = np.tile(dft_row, (n, 1))
    y = np.stack([sample_from(rng, Q[i], n) for i in range(K)], axis=1).reshape(-1)
    u = grid_u(rng, n * (K + 1))
    out = oracle.verify_chain(tgt, dft, y, u, None, n, K, V, 1.0, want_probs=False)
    A, nxt = out["A"], out["next"]
    yk = y.reshape(n, K)
    assert (out["status"] == 0).all()
    # token emitted at position j among trials that reach j, j = 0..K
    tested = 0
    for j in range(K + 1):
        reach = A >= j
        if reach.sum() < 2000:
            continue                    # e.g. disjoint supports never pass position 0
        tok = np.where(A[reach] > j, yk[reach][:, j] if j < K else -1, nxt[reach])
        obs = np.bincount(tok, minlength=V)
        assert _chi2_ok(obs, P[j], int(reach.sum())), f"position {j}"
        tested += 1
    assert tested >= 1
    # Given that position 1 is reached, the token there follows p1 whatever token
    # was committed at position 0: expected[a, b] = #(t0 = a, reached) * p1(b).
    reach = A >= 1
    if reach.sum() < 2000:
        return
    t0 = yk[reach][:, 0]
    t1 = np.where(A[reach] > 1, yk[reach][:, 1], nxt[reach])
    obs = np.bincount(t0 * V + t1, minlength=V * V).reshape(V, V)
    n_a = obs.sum(1)
    for a in range(V):
        if n_a[a] >= 2000:
            assert _chi2_ok(obs[a], P[1], int(n_a[a])), f"t1 given t0={a}"


def test_chi_square_detects_a_planted_mistake():
    """Sanity of the test itself: drawing the correction with the accept test's
    uniform (u_A instead of u_k) must fail the same chi-square check."""
    P, Q = CHI_CASES["q_uniform"]
    K, V, n = len(Q), len(P[0]), 400_000
    rng = np.random.default_rng(5)
    tgt = np.tile(np.stack([logits_of(r) for r in P]), (n, 1))
    dft = np.tile(np.stack([logits_of(r) for r in Q]), (n, 1))
    y = np.stack([sample_from(rng, Q[i], n) for i in range(K)], axis=1).reshape(-1)
    u = grid_u(rng, (n, K + 1))
    out = oracle.verify_chain(tgt, dft, y, u.reshape(-1), None, n, K, V, 1.0, want_probs=False)
    A = out["A"]
    # re-run with u_k replaced by u_A for the rejected trials (the planted mistake)
    u_bad = u.copy()
    rej = A < K
    u_bad[rej, K] = u[rej, A[rej]]
    bad = oracle.verify_chain(tgt, dft, y, u_bad.reshape(-1), None, n, K, V, 1.0, want_probs=False)
    j = 0
    reach = bad["A"] >= j
    tok = np.where(bad["A"][reach] > j, y.reshape(n, K)[reach][:, j], bad["next"][reach])
    assert not _chi2_ok(np.bincount(tok, minlength=V), P[j], int(reach.sum()))


def test_special_case_q_equals_p_accepts_everything():
    rng = np.random.default_rng(2)
    B, K, V = 300, 4, 16
    D = (rng.standard_normal((B, K + 1, V)) * 2).astype(np.float32)
    tgt = D.reshape(-1, V)
    dft = D[:, :K].reshape(-1, V)
    y = rng.integers(0, V, B * K).astype(np.int32)
    u = grid_u(rng, B * (K + 1))
    out = oracle.verify_chain(tgt, dft, y, u, None, B, K, V, 0.8)
    assert (out["A"] == K).all()
    assert (out["R"] == 0).all()


def test_special_case_one_hot_draft():
    """q one-hot at y: acceptance probability p(y); the correction follows
    p(. | t != y)."""
    p = np.array([.1, .35, .2, .05, .3])
    V, n, yv = 5, 300_000, 1
    q = np.zeros(V); q[yv] = 1
    rng = np.random.default_rng(8)
    tgt = np.tile(np.stack([logits_of(p), logits_of(p)]), (n, 1))
    dft = np.tile(logits_of(q)[None], (n, 1))
    y = np.full(n, yv, np.int32)
    u = grid_u(rng, 2 * n)
    out = oracle.verify_chain(tgt, dft, y, u, None, n, 1, V, 1.0, want_probs=False)
    acc = (out["A"] == 1).mean()
    assert abs(acc - p[yv]) < 4 * math.sqrt(p[yv] * (1 - p[yv]) / n)
    rej = out["A"] == 0
    cond = p.copy(); cond[yv] = 0; cond /= cond.sum()
    assert _chi2_ok(np.bincount(out["next"][rej], minlength=V), cond, int(rej.sum()))


def test_special_case_k0_draws_from_row0():
    p = np.array([.5, .125, .125, .25])
    n, V = 200_000, 4
    rng = np.random.default_rng(9)
    tgt = np.tile(logits_of(p)[None], (n, 1))
    cu = np.zeros(n + 1, np.int32)
    out = oracle.verify_chain(tgt, np.zeros((0, V), np.float32), np.zeros(0, np.int32),
                              grid_u(rng, n), cu, n, 0, V, 1.0, want_probs=False)
    assert (out["A"] == 0).all()
    assert _chi2_ok(np.bincount(out["next"], minlength=V), p, n)


def test_margin_flags():
    # p(y) = 0.5, q(y) = 1.0, u = 0.5 exactly: u*q == p -> accepted, flagged as a margin case
    V = 2
    tgt = np.stack([logits_of([.5, .5]), logits_of([.5, .5])])
    dft = logits_of([1.0, 0.0])[None]
    out = oracle.verify_chain(tgt, dft, np.array([0], np.int32), np.array([0.5, 0.3], np.float32),
                              None, 1, 1, V, 1.0)
    assert out["A"][0] == 1 and out["margin"][0] & oracle.MARGIN_ACCEPT
    out = oracle.verify_chain(tgt, dft, np.array([0], np.int32), np.array([0.25, 0.3], np.float32),
                              None, 1, 1, V, 1.0)
    assert out["A"][0] == 1 and out["margin"][0] == 0
    # the extra-token draw at u = 0.5 sits exactly on the CDF step between ids 0 and 1
    out = oracle.verify_chain(tgt, dft, np.array([0], np.int32), np.array([0.25, 0.5], np.float32),
                              None, 1, 1, V, 1.0)
    assert out["next"][0] == 1 and out["margin"][0] & oracle.MARGIN_SAMPLE


def test_bad_token_and_nonfinite_rows():
    V = 4
    tgt = np.zeros((3, V), np.float32)
    dft = np.zeros((2, V), np.float32)
    out = oracle.verify_chain(tgt, dft, np.array([7, 0], np.int32), np.zeros(3, np.float32),
                              None, 1, 2, V, 1.0)
    assert out["A"][0] == 0 and out["status"][0] == oracle.BAD_TOKEN
    # residual at a bad token: r = max(p - q, 0) with p == q uniform -> R = 0 -> drawn from p
    assert 0 <= out["next"][0] < V
    tgt[1] = np.nan
    out = oracle.verify_chain(tgt, dft, np.array([1, 1], np.int32), np.zeros(3, np.float32),
                              None, 1, 2, V, 1.0)
    assert out["A"][0] == 1 and out["status"][0] == oracle.NONFINITE and out["next"][0] == -1
    # a non-finite row after the first rejection is not reported
    tgt2 = np.zeros((3, V), np.float32); tgt2[2] = np.nan
    dft2 = np.zeros((2, V), np.float32); dft2[0, 0] = 10.0   # q0 peaks at 0, p0 uniform
    u = np.array([0.99999994, 0, 0], np.float32)
    out = oracle.verify_chain(tgt2, dft2, np.array([0, 1], np.int32), u, None, 1, 2, V, 1.0)
    assert out["A"][0] == 0 and out["status"][0] == 0


# --------------------------------------------------------------------------
# [SD §1] greedy: T = 0 is the argmax rule; tiny T reaches it too.
# --------------------------------------------------------------------------

def test_greedy_equivalence_T0_and_tiny_T():
    rng = np.random.default_rng(4)
    B, K, V = 200, 4, 64
    # tie-free rows with min gap delta = 1/64 (distinct multiples of delta)
    delta = 1.0 / 64
    perm = np.stack([rng.permutation(V) for _ in range(B * (K + 1))])
    tgt = (perm * delta).astype(np.float32)
    dperm = np.stack([rng.permutation(V) for _ in range(B * K)])
    dft = (dperm * delta).astype(np.float32)
    g = np.argmax(tgt, axis=1).reshape(B, K + 1)
    take = rng.random((B, K)) < 0.6
    y = np.where(take, g[:, :K], rng.integers(0, V, (B, K))).astype(np.int32).reshape(-1)
    u = grid_u(rng, B * (K + 1))
    ref = oracle.verify_greedy(tgt, y, None, B, K, V)
    # the argmax rule by hand
    yk = y.reshape(B, K)
    for b in range(B):
        A = next((i for i in range(K) if yk[b, i] != g[b, i]), K)
        assert ref["A"][b] == A and ref["next"][b] == g[b, A]
    t0 = oracle.verify_chain(tgt, dft, y, u, None, B, K, V, 0.0)
    np.testing.assert_array_equal(t0["A"], ref["A"])
    np.testing.assert_array_equal(t0["next"], ref["next"])
    tiny = np.float32(delta / 800)
    tt = oracle.verify_chain(tgt, dft, y, u, None, B, K, V, float(tiny))
    np.testing.assert_array_equal(tt["A"], ref["A"])
    np.testing.assert_array_equal(tt["next"], ref["next"])


# --------------------------------------------------------------------------
# [SD §5 DSpark] prefix survival and expected advance.
# --------------------------------------------------------------------------

def test_expected_advance_closed_form_matches_monte_carlo():
    """On V = 2 with q = (1, 0) and p_i = (c_i, 1 - c_i) the chain accepts
    position i with probability c_i, so E[A + 1] = 1 + sum_j prod_{i<=j} c_i,
    which is the expected advance of the length chooser at k = K."""
    c = np.array([0.9, 0.8, 0.75, 0.6, 0.95], np.float32)
    K, V, n = len(c), 2, 400_000
    rng = np.random.default_rng(12)
    P = [[float(ci), 1 - float(ci)] for ci in c] + [[0.5, 0.5]]
    tgt = np.tile(np.stack([logits_of(r) for r in P]), (n, 1))
    dft = np.tile(np.stack([logits_of([1.0, 0.0])] * K), (n, 1))
    y = np.zeros(n * K, np.int32)
    out = oracle.verify_chain(tgt, dft, y, grid_u(rng, n * (K + 1)), None, n, K, V, 1.0, want_probs=False)
    closed = 1 + sum(np.prod(c[:j + 1].astype(np.float64)) for j in range(K))
    mc = (out["A"] + 1).astype(np.float64)
    assert abs(mc.mean() - closed) < 4 * mc.std() / math.sqrt(n)
    sel = oracle.select_len(c[None], 1, K, 0.0)
    assert sel["k"][0] == K
    assert abs(sel["adv"][0] - closed) < 1e-6


def test_select_len_properties():
    rng = np.random.default_rng(13)
    B, K = 2000, 8
    six = rng.random((B, K, 6))
    conf = np.sort(six, axis=-1)[..., 4].astype(np.float32)   # Beta(5, 2)
    sel = oracle.select_len(conf, B, K, 0.15)
    # survival is non-increasing, so the best k is the number of positions whose
    # fp32 survival exceeds the cost (the increments s_j - cost change sign once)
    s = np.multiply.accumulate(conf, axis=1, dtype=np.float32)
    np.testing.assert_array_equal(sel["k"], (s > np.float32(0.15)).sum(1))
    for b in range(50):
        k = sel["k"][b]
        np.testing.assert_allclose(sel["adv"][b], 1 + s[b, :k].astype(np.float64).sum(), rtol=1e-12)
    np.testing.assert_array_equal(sel["cu"], np.concatenate([[0], np.cumsum(sel["k"])]))
    # c == 1 and cost < 1 -> K; cost >= 1 -> 0; raising the cost never raises k
    ones = np.ones((3, K), np.float32)
    assert (oracle.select_len(ones, 3, K, 0.99)["k"] == K).all()
    assert (oracle.select_len(ones, 3, K, 1.0)["k"] == 0).all()
    prev = None
    for cost in (0.0, 0.05, 0.15, 0.3, 0.6, 0.9):
        k = oracle.select_len(conf, B, K, cost)["k"]
        if prev is not None:
            assert (k <= prev).all()
        prev = k
    # E[k*] for Beta(5,2) at cost 0.15 is about 4.9
    assert 4.6 < sel["k"].mean() < 5.2


def test_cost_model_example():
    """[SD §2] illustrative numbers: a 3 + 13 + 2 ms round gives 18/4 = 4.5 ms per
    token with 3 accepted drafts and 18/2 = 9 ms with 1 (A excludes the extra token)."""
    per_round = 3 + 13 + 2
    assert per_round / (3 + 1) == 4.5
    assert per_round / (1 + 1) == 9.0


# --------------------------------------------------------------------------
# [SD §5 DDTree] best-first tree under a node budget, and the walk.
# --------------------------------------------------------------------------

def _all_prefix_closed_sets(V, K, size):
    """Every prefix-closed set of `size` prefixes (tuples of token ids) of the
    V-ary trie of depth K."""
    start = frozenset()
    seen = {start}
    frontier = [start]
    for _ in range(size):
        nxt = []
        for s in frontier:
            cands = [(t,) for t in range(V)] + [u + (t,) for u in s if len(u) < K for t in range(V)]
            for c in cands:
                if c in s:
                    continue
                ns = s | {c}
                if ns not in seen:
                    seen.add(ns)
                    nxt.append(ns)
        frontier = nxt
    return frontier


def _Q(marg, u):
    return float(np.prod([float(marg[d][t]) for d, t in enumerate(u)]))


@pytest.mark.parametrize("V,K,N", [(2, 2, 4), (3, 2, 5), (3, 3, 7), (2, 3, 7), (3, 3, 5)])
def test_tree_brute_force_optimal(V, K, N):
    rng = np.random.default_rng(V * 100 + K * 10 + N)
    for trial in range(6):
        Z = rng.standard_normal((K, V)) * 1.5
        marg = special.softmax(Z, axis=1).astype(np.float32)
        out = oracle.build_tree(marg[None], 1, K, V, N)
        n = int(out["n_nodes"][0])
        total = sum(V ** m for m in range(1, K + 1))
        assert n == min(N, total + 1)
        tok, par, dep = out["token"][0], out["parent"][0], out["depth"][0]
        # reconstruct prefixes
        pref = {0: ()}
        for i in range(1, n):
            assert 0 <= par[i] < i
            assert dep[i] == dep[par[i]] + 1
            pref[i] = pref[par[i]] + (int(tok[i]),)
        chosen = frozenset(pref[i] for i in range(1, n))
        best = max(_all_prefix_closed_sets(V, K, n - 1), key=lambda s: sum(_Q(marg, u) for u in s))
        got = sum(_Q(marg, u) for u in chosen)
        want = sum(_Q(marg, u) for u in best)
        assert got >= want * (1 - 1e-6)


def test_tree_invariants_and_full_trie():
    rng = np.random.default_rng(21)
    B, K, V, N = 6, 4, 50, 64
    marg = special.softmax(rng.standard_normal((B, K, V)) * 2.5, axis=2).astype(np.float32)
    out = oracle.build_tree(marg, B, K, V, N)
    for b in range(B):
        n = out["n_nodes"][b]
        assert n == N
        sc, par, dep, anc, tok = (out[k][b] for k in ("score", "parent", "depth", "anc_mask", "token"))
        assert sc[0] == 1.0 and par[0] == -1 and anc[0] == 1
        for i in range(1, n):
            p = par[i]
            assert p < i and dep[i] == dep[p] + 1 <= K
            assert sc[i] <= sc[i - 1]                        # scores never increase in node order
            assert int(anc[i]) == int(anc[p]) | (1 << i)      # mask follows the parent chain
            assert sc[i] == np.float32(sc[p] * marg[b, dep[p], tok[i]])
        # siblings carry distinct tokens
        for p in range(n):
            kids = [tok[i] for i in range(1, n) if par[i] == p]
            assert len(kids) == len(set(kids))
    # trie smaller than the budget: everything is taken
    m2 = special.softmax(rng.standard_normal((1, 2, 3)), axis=2).astype(np.float32)
    o2 = oracle.build_tree(m2, 1, 2, 3, 64)
    assert o2["n_nodes"][0] == 1 + 3 + 9


def test_tree_depth1_is_top_list():
    """With budget N the depth-1 children are a prefix of the sorted marginal
    (q desc, id asc): a tree never skips a better sibling."""
    rng = np.random.default_rng(22)
    K, V, N = 3, 40, 20
    marg = special.softmax(rng.standard_normal((1, K, V)) * 2.5, axis=2).astype(np.float32)
    marg[0, 0, 7] = marg[0, 0, 3]          # a tie: id 3 must come first
    out = oracle.build_tree(marg, 1, K, V, N)
    kids = [int(out["token"][0][i]) for i in range(1, N) if out["parent"][0][i] == 0]
    order = sorted(range(V), key=lambda t: (-float(marg[0, 0, t]), t))
    assert kids == order[:len(kids)]


def _one_hot_rows(tokens, V):
    r = np.full((len(tokens), V), -5.0, np.float32)
    r[np.arange(len(tokens)), tokens] = 5.0
    return r


def test_tree_walk_hand_built():
    # root 0 -> 1 (tok 4), 2 (tok 7); 1 -> 3 (tok 2); 3 -> 4 (tok 9)
    V, N = 12, 6
    token = np.array([[-1, 4, 7, 2, 9, -1]], np.int32)
    parent = np.array([[-1, 0, 0, 1, 3, -1]], np.int32)
    nn = np.array([5], np.int32)
    # full walk to the deepest node, then the extra token from node 4's row
    rows = _one_hot_rows([4, 2, 0, 9, 11, 0], V)[None]
    out = oracle.verify_tree(rows, token, parent, nn, 1, N, V)
    assert out["A"][0] == 3 and out["path"][0][:4].tolist() == [1, 3, 4, -1] and out["next"][0] == 11
    # walk ending early at node 2 (a leaf): next is node 2's argmax
    rows = _one_hot_rows([7, 0, 5, 0, 0, 0], V)[None]
    out = oracle.verify_tree(rows, token, parent, nn, 1, N, V)
    assert out["A"][0] == 1 and out["path"][0][0] == 2 and out["next"][0] == 5
    # immediate miss
    rows = _one_hot_rows([3, 0, 0, 0, 0, 0], V)[None]
    out = oracle.verify_tree(rows, token, parent, nn, 1, N, V)
    assert out["A"][0] == 0 and (out["path"][0] == -1).all() and out["next"][0] == 3
    # a tie in the target row goes to the lower id (4 over 7)
    rows = _one_hot_rows([4, 0, 0, 0, 0, 0], V)
    rows[0, 7] = 5.0
    rows[1, 2] = 5.0
    out = oracle.verify_tree(rows[None], token, parent, nn, 1, N, V)
    assert out["path"][0][0] == 1


def test_tree_walk_expected_length_monte_carlo():
    """If the target's token at depth d is drawn from q_{d+1} independently, the
    walk reaches node u with probability Q(u), so E[accepted] = sum_u Q(u)."""
    rng = np.random.default_rng(23)
    K, V, N, n = 3, 4, 9, 60_000
    marg = special.softmax(rng.standard_normal((1, K, V)) * 1.2, axis=2).astype(np.float32)
    tree = oracle.build_tree(marg, 1, K, V, N)
    nn = int(tree["n_nodes"][0])
    dep = tree["depth"][0]
    rows = np.full((n, N, V), -5.0, np.float32)
    for node in range(nn):
        d = dep[node]
        if d < K:
            draws = sample_from(rng, marg[0, d].astype(np.float64), n)
        else:
            draws = rng.integers(0, V, n)
        rows[np.arange(n), node, draws] = 5.0
    tok = np.tile(tree["token"], (n, 1))
    par = np.tile(tree["parent"], (n, 1))
    out = oracle.verify_tree(rows, tok, par, np.full(n, nn, np.int32), n, N, V)
    expect = sum(float(tree["score"][0][i]) for i in range(1, nn))
    a = out["A"].astype(np.float64)
    assert abs(a.mean() - expect) < 4 * a.std() / math.sqrt(n)


# --------------------------------------------------------------------------
# Sampled tree walk ([SD §5 DDTree]: the walk follows the token the target
# picks; here the target picks by sampling its own row at each node)
# --------------------------------------------------------------------------

# root 0 -> 1 (tok 1), 2 (tok 3); 1 -> 3 (tok 0), 4 (tok 2); 3 -> 5 (tok 1)
WALK_TOKEN = np.array([-1, 1, 3, 0, 2, 1], np.int32)
WALK_PARENT = np.array([-1, 0, 0, 1, 1, 3], np.int32)
WALK_P = np.array([[.1, .4, .2, .3], [.5, .1, .3, .1], [.25, .25, .25, .25],
                   [.2, .6, .1, .1], [.7, .1, .1, .1], [.1, .1, .1, .7]])


def _walk_trials(n, rng, uniforms=None, T=1.0):
    N, V = WALK_P.shape
    rows = np.tile(logits_of(WALK_P)[None], (n, 1, 1))
    u = grid_u(rng, (n, N)) if uniforms is None else uniforms
    out = oracle.verify_tree_sampled(rows, np.tile(WALK_TOKEN, (n, 1)), np.tile(WALK_PARENT, (n, 1)),
                                     np.full(n, N, np.int32), u, n, N, V, T)
    return out, u


def _committed(out, n):
    """Token sequence each trial commits: the path's tokens, then next."""
    seqs = []
    for b in range(n):
        a = out["A"][b]
        seqs.append([int(WALK_TOKEN[c]) for c in out["path"][b][:a]] + [int(out["next"][b])])
    return seqs


def test_sampled_walk_tokens_follow_the_target():
    """Committed tokens are draws from the target given the tokens before them:
    the first follows p_root; given it lands on child c, the second follows p_c."""
    n = 200_000
    rng = np.random.default_rng(41)
    out, _ = _walk_trials(n, rng)
    assert (out["status"] == 0).all()
    A, path = out["A"], out["path"]
    first = np.where(A >= 1, WALK_TOKEN[np.maximum(path[:, 0], 0)], out["next"])
    assert _chi2_ok(np.bincount(first, minlength=4), WALK_P[0], n)
    for c in (1, 2):
        sel = (A >= 1) & (path[:, 0] == c)
        second = np.where(A[sel] >= 2, WALK_TOKEN[np.maximum(path[sel, 1], 0)], out["next"][sel])
        assert _chi2_ok(np.bincount(second, minlength=4), WALK_P[c], int(sel.sum())), f"child {c}"
    # third token given the path 1 -> 3
    sel = (A >= 2) & (path[:, 0] == 1) & (path[:, 1] == 3)
    third = np.where(A[sel] >= 3, WALK_TOKEN[np.maximum(path[sel, 2], 0)], out["next"][sel])
    assert _chi2_ok(np.bincount(third, minlength=4), WALK_P[3], int(sel.sum()))


def test_sampled_walk_planted_mistake_is_detected():
    """Sanity of the test above: reusing the root's uniform at every node (one
    draw instead of independent draws) must fail the conditional check."""
    n = 200_000
    rng = np.random.default_rng(43)
    u = np.repeat(grid_u(rng, (n, 1)), WALK_P.shape[0], axis=1)
    out, _ = _walk_trials(n, rng, uniforms=u)
    A, path = out["A"], out["path"]
    sel = (A >= 1) & (path[:, 0] == 1)
    second = np.where(A[sel] >= 2, WALK_TOKEN[np.maximum(path[sel, 1], 0)], out["next"][sel])
    assert not _chi2_ok(np.bincount(second, minlength=4), WALK_P[1], int(sel.sum()))


def test_sampled_walk_expected_length_closed_form():
    """The walk reaches node u iff the target's draws spell u's path, so
    E[accepted] = sum over draft nodes of the product of p_parent(token) along
    the path."""
    n = 100_000
    rng = np.random.default_rng(47)
    out, _ = _walk_trials(n, rng)
    reach = np.zeros(len(WALK_TOKEN))
    reach[0] = 1.0
    for c in range(1, len(WALK_TOKEN)):
        reach[c] = reach[WALK_PARENT[c]] * WALK_P[WALK_PARENT[c], WALK_TOKEN[c]]
    expect = reach[1:].sum()
    a = out["A"].astype(np.float64)
    assert abs(a.mean() - expect) < 4 * a.std() / math.sqrt(n)
    # the path is a chain of parent -> child links starting at the root
    for b in range(200):
        node = 0
        for c in out["path"][b][:out["A"][b]]:
            assert WALK_PARENT[c] == node
            node = c
        assert (out["path"][b][out["A"][b]:] == -1).all()


def test_sampled_walk_small_temperature_is_the_argmax_walk():
    """For tie-free rows with minimum gap delta and T <= delta/800 every
    non-maximal weight underflows, so the sampled walk is the argmax walk for
    every uniform; T == 0 is the argmax walk by definition."""
    rng = np.random.default_rng(53)
    B, N, V = 64, 6, 9
    rows = np.stack([rng.permutation(V) for _ in range(B * N)]).astype(np.float32).reshape(B, N, V)
    # plant matches so that walks go deep
    for b in range(B):
        for n in range(N):
            kids = [c for c in range(1, N) if WALK_PARENT[c] == n]
            if kids and rng.random() < 0.7:
                t = WALK_TOKEN[rng.choice(kids)]
                rows[b, n, t] = V + 1.0
    tok = np.tile(WALK_TOKEN, (B, 1))
    par = np.tile(WALK_PARENT, (B, 1))
    nn = np.full(B, N, np.int32)
    ref = oracle.verify_tree(rows, tok, par, nn, B, N, V)
    assert (ref["A"] >= 2).any()
    for T in (0.0, 1.0 / 800):
        u = grid_u(rng, (B, N))
        u[:, 0] = 1.0 - 2.0 ** -24            # the extreme uniforms too
        u[:, 1] = 0.0
        out = oracle.verify_tree_sampled(rows, tok, par, nn, u, B, N, V, T)
        assert (out["A"] == ref["A"]).all() and (out["next"] == ref["next"]).all()
        assert (out["path"] == ref["path"]).all()


def test_sampled_walk_top1_is_the_argmax_walk():
    """Top-1 truncation keeps only the lowest-id maximum, so the sampled walk is
    the argmax walk for every temperature and uniform (ties included)."""
    rng = np.random.default_rng(59)
    B, N, V = 48, 6, 7
    rows = rng.integers(0, 4, size=(B, N, V)).astype(np.float32)     # many ties
    tok = np.tile(WALK_TOKEN, (B, 1))
    par = np.tile(WALK_PARENT, (B, 1))
    nn = np.full(B, N, np.int32)
    ref = oracle.verify_tree(rows, tok, par, nn, B, N, V)
    for T in (0.3, 1.0, 5.0):
        out = oracle.verify_tree_sampled(rows, tok, par, nn, grid_u(rng, (B, N)), B, N, V, T, 1)
        assert (out["A"] == ref["A"]).all() and (out["next"] == ref["next"]).all()
        assert (out["path"] == ref["path"]).all()


def test_sampled_walk_topk_follows_the_truncated_target():
    """With top-k = 2 every pick follows the row's two largest probabilities,
    renormalised; the other tokens are never committed."""
    n = 200_000
    rng = np.random.default_rng(61)
    N, V = WALK_P.shape
    rows = np.tile(logits_of(WALK_P)[None], (n, 1, 1))
    u = grid_u(rng, (n, N))
    out = oracle.verify_tree_sampled(rows, np.tile(WALK_TOKEN, (n, 1)), np.tile(WALK_PARENT, (n, 1)),
                                     np.full(n, N, np.int32), u, n, N, V, 1.0, 2)
    A, path = out["A"], out["path"]
    first = np.where(A >= 1, WALK_TOKEN[np.maximum(path[:, 0], 0)], out["next"])
    p0 = WALK_P[0].copy()
    keep = np.argsort(-p0, kind="stable")[:2]
    trunc = np.zeros_like(p0)
    trunc[keep] = p0[keep] / p0[keep].sum()
    assert _chi2_ok(np.bincount(first, minlength=V), trunc, n)
    # given the walk reached node 1, the next pick follows node 1's truncated row
    sel = (A >= 1) & (path[:, 0] == 1)
    second = np.where(A[sel] >= 2, WALK_TOKEN[np.maximum(path[sel, 1], 0)], out["next"][sel])
    p1 = WALK_P[1].copy()
    keep1 = np.argsort(-p1, kind="stable")[:2]
    t1 = np.zeros_like(p1)
    t1[keep1] = p1[keep1] / p1[keep1].sum()
    assert _chi2_ok(np.bincount(second, minlength=V), t1, int(sel.sum()))


def test_sampled_walk_nonfinite_row_and_one_hot_rows():
    N, V = WALK_P.shape
    # one-hot target rows spell the path root -> 1 -> 3 -> 5, then token 2
    picks = [1, 0, 0, 1, 0, 2]
    rows = np.full((1, N, V), -np.inf, np.float32)
    for n, t in enumerate(picks):
        rows[0, n, t] = 0.0
    u = np.full((1, N), 0.999, np.float32)
    out = oracle.verify_tree_sampled(rows, WALK_TOKEN[None], WALK_PARENT[None], np.array([N], np.int32),
                                     u, 1, N, V, 0.8)
    assert out["A"][0] == 3 and out["path"][0][:3].tolist() == [1, 3, 5] and out["next"][0] == 2
    assert out["status"][0] == 0
    # a NaN row on the path stops the walk there with next = -1 and the flag
    rows[0, 3, :] = np.nan
    out = oracle.verify_tree_sampled(rows, WALK_TOKEN[None], WALK_PARENT[None], np.array([N], np.int32),
                                     u, 1, N, V, 0.8)
    assert out["A"][0] == 2 and out["next"][0] == -1 and out["status"][0] == oracle.NONFINITE


# --------------------------------------------------------------------------
# Ragged verify modes and a per-position cost table ([SD §9 DSpark], [SD §5 DSpark])
# --------------------------------------------------------------------------

def test_select_len_table_closed_form_and_constant_table():
    # c == 1 gives s_j == 1, so f(k) = 1 + k - sum of the first k costs:
    # costs (0.5, 2, 0.1, 0.1) give f = 1, 1.5, 0.5, 1.4, 2.3 -> k* = 4, advance 5
    out = oracle.select_len_table(np.ones((1, 4), np.float32), 1, 4,
                                  np.array([0.5, 2.0, 0.1, 0.1], np.float32))
    assert out["k"][0] == 4 and out["adv"][0] == 5.0
    # ... and with the last cost raised to 1.5: f = 1, 1.5, 0.5, 1.4, 0.9 -> k* = 1, advance 2
    out = oracle.select_len_table(np.ones((1, 4), np.float32), 1, 4,
                                  np.array([0.5, 2.0, 0.1, 1.5], np.float32))
    assert out["k"][0] == 1 and out["adv"][0] == 2.0
    # a constant table is the scalar rule (itself pinned to the survival closed form)
    rng = np.random.default_rng(21)
    B, K = 3000, 8
    conf = np.sort(rng.random((B, K, 6)), axis=-1)[..., 4].astype(np.float32)
    for cost in (0.0, 0.15, 0.5):
        a = oracle.select_len_table(conf, B, K, np.full(K, cost, np.float32))
        b = oracle.select_len(conf, B, K, cost)
        np.testing.assert_array_equal(a["k"], b["k"])
        np.testing.assert_array_equal(a["adv"], b["adv"])
        np.testing.assert_array_equal(a["cu"], b["cu"])


def test_select_len_table_monotone_in_cost():
    # raising costs element-wise adds a non-decreasing amount to sum_{j<=k} cost,
    # so the smallest maximiser can only move to a shorter length
    rng = np.random.default_rng(22)
    B, K = 2000, 8
    conf = rng.random((B, K)).astype(np.float32) ** 0.2
    base = (rng.random(K) * 0.3).astype(np.float32)
    prev = oracle.select_len_table(conf, B, K, base)["k"]
    for step in range(5):
        base = (base + (rng.random(K) * 0.1).astype(np.float32)).astype(np.float32)
        k = oracle.select_len_table(conf, B, K, base)["k"]
        assert (k <= prev).all()
        prev = k
    assert (oracle.select_len_table(conf, B, K, np.full(K, -1.0, np.float32))["k"] == K).all()
    assert (oracle.select_len_table(conf, B, K, np.full(K, 1.5, np.float32))["k"] == 0).all()


def _window(rng, B, K, V, T=1.0):
    D = rng.normal(0, 2, (B, K + 1, V))
    tgt = (D + rng.normal(0, 0.5, D.shape)).astype(np.float32)
    dft = D[:, :K].astype(np.float32)
    y = np.zeros((B, K), np.int32)
    for b in range(B):
        for i in range(K):
            z = dft[b, i].astype(np.float64) / T
            p = np.exp(z - z.max())
            y[b, i] = rng.choice(V, p=p / p.sum())
    return tgt, dft, y, grid_u(rng, B * (K + 1))


def test_capped_commits_what_compact_commits():
    rng = np.random.default_rng(23)
    B, K, V = 40, 6, 50
    tgt, dft, y, u = _window(rng, B, K, V)
    cap = rng.integers(0, K + 1, B).astype(np.int32)
    cap[:3] = (-2, K + 5, K)                      # clamped to [0, K]
    out = oracle.verify_chain_capped(tgt, dft, y, u, cap, B, K, V, 1.0)
    full = oracle.verify_chain(tgt, dft, y, u, None, B, K, V, 1.0)
    kc = np.clip(cap, 0, K)
    # compact: only the first kc positions (and kc+1 target rows / uniforms) exist
    t_rows = np.concatenate([tgt[b, :kc[b] + 1] for b in range(B)])
    d_rows = np.concatenate([dft[b, :kc[b]] for b in range(B)])
    y_c = np.concatenate([y[b, :kc[b]] for b in range(B)])
    u_c = np.concatenate([u.reshape(B, K + 1)[b, :kc[b] + 1] for b in range(B)])
    cu = np.concatenate([[0], np.cumsum(kc)]).astype(np.int32)
    comp = oracle.verify_chain(t_rows, d_rows, y_c, u_c, cu, B, K, V, 1.0)
    np.testing.assert_array_equal(out["A"], comp["A"])
    np.testing.assert_array_equal(out["next"], comp["next"])
    np.testing.assert_array_equal(out["A_full"], full["A"])
    np.testing.assert_array_equal(out["probs"], full["probs"])
    # the committed length is the full-window rejection point, capped
    np.testing.assert_array_equal(out["A"], np.minimum(full["A"], kc))
    # cap == K is the static (full-window) verification itself
    allk = oracle.verify_chain_capped(tgt, dft, y, u, np.full(B, K, np.int32), B, K, V, 1.0)
    np.testing.assert_array_equal(allk["A"], full["A"])
    np.testing.assert_array_equal(allk["next"], full["next"])


def test_compact_kv_hand_example():
    # [SD §5 DDTree]: only the accepted path stays in the KV cache. Rows hold
    # their own index; draft node n sits at row base + n - 1.
    kv = (np.arange(12)[:, None] * np.ones((1, 16))).astype(np.uint8)
    path = np.full((2, 6), -1, np.int32)
    path[0, :3] = (2, 4, 5)          # sequence 0: region rows 0..4
    path[1, :2] = (1, 2)             # sequence 1: region rows 6..10, already in place
    out = oracle.compact_kv(kv, [0, 6], path, [3, 2], 2, 6)
    np.testing.assert_array_equal(out[:, 0], [1, 3, 4, 3, 4, 5, 6, 7, 8, 9, 10, 11])
    # a region past the buffer is left alone (sequence 0: rows 8..12 of 12); an
    # entry outside [1, N-1] is skipped (node 9, node 6 == N)
    out = oracle.compact_kv(kv, [8, 0], np.array([[2, 3, -1, -1, -1, -1],
                                                  [9, 6, 3, -1, -1, -1]], np.int32), [2, 3], 2, 6)
    np.testing.assert_array_equal(out[:, 0], [0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11][:2] + [2] +
                                  [3, 4, 5, 6, 7, 8, 9, 10, 11])


# --------------------------------------------------------------------------
# EAGLE-2-style verification tree ([SD §4 EAGLE-2])
# --------------------------------------------------------------------------

def _trie_candidates(m):
    """The full trie over the per-depth lists of marginals m [K, V]: BFS order,
    each node's children by rank, so candidates of one depth are in
    lexicographic rank-tuple order."""
    K, V = m.shape
    lists = [np.lexsort((np.arange(V), -m[d].astype(np.float64))) for d in range(K)]
    par, tok, prob = [-1], [-1], [1.0]
    level = [0]
    for d in range(K):
        nxt = []
        for c in level:
            for r in range(V):
                par.append(c)
                tok.append(int(lists[d][r]))
                prob.append(float(m[d, lists[d][r]]))
                nxt.append(len(par) - 1)
        level = nxt
    return np.array(par, np.int32), np.array(tok, np.int32), np.array(prob, np.float32)


@pytest.mark.parametrize("N", [2, 5, 13, 40, 64])
def test_rerank_of_the_full_trie_is_the_ddtree(N):
    # re-ranking the whole factorised trie by cumulative confidence gives the
    # best-first DDTree of the same marginals (itself pinned by brute force)
    rng = np.random.default_rng(31 + N)
    K, V = 4, 3
    m = special.softmax(rng.normal(0, 1.5, (K, V)), axis=-1).astype(np.float32)
    par, tok, prob = _trie_candidates(m)
    M = len(par)
    rr = oracle.rerank_tree(par[None], tok[None], prob[None], [M], 1, M, N)
    bt = oracle.build_tree(m[None], 1, K, V, N)
    for key in ("token", "parent", "depth", "score", "anc_mask", "n_nodes"):
        np.testing.assert_array_equal(rr[key], bt[key], err_msg=key)


def test_rerank_brute_force_and_bad_candidates():
    rng = np.random.default_rng(32)
    for trial in range(300):
        M = int(rng.integers(2, 9))
        N = int(rng.integers(2, 7))
        par = np.array([-1] + [int(rng.integers(0, i)) for i in range(1, M)], np.int32)
        prob = rng.random(M).astype(np.float32)
        prob[0] = 1.0
        tok = rng.integers(0, 50, M).astype(np.int32)
        rr = oracle.rerank_tree(par[None], tok[None], prob[None], [M], 1, M, N)
        conf = np.ones(M, np.float32)
        for i in range(1, M):
            conf[i] = np.float32(conf[par[i]] * prob[i])
        kept = set(int(c) for c in rr["cand"][0, 1:rr["n_nodes"][0]])
        size = min(N - 1, M - 1)
        best = -1.0
        for S in itertools.combinations(range(1, M), size):
            if all(par[i] == 0 or par[i] in S for i in S):
                best = max(best, float(sum(conf[i] for i in S)))
        assert len(kept) == size
        assert all(par[i] == 0 or par[i] in kept for i in kept)
        assert abs(sum(float(conf[i]) for i in kept) - best) < 1e-6
        # node order: confidence never increases, parents come first
        sc = rr["score"][0, 1:rr["n_nodes"][0]]
        assert (np.diff(sc) <= 0).all()
        pr = rr["parent"][0, 1:rr["n_nodes"][0]]
        assert (pr < np.arange(1, rr["n_nodes"][0])).all()
    # a bad parent, a probability outside [0, 1] or NaN drops the subtree
    par = np.array([-1, 0, 1, 0, 3, 5, 0], np.int32)
    prob = np.array([1, 0.9, 0.8, 1.5, 0.9, 0.5, np.nan], np.float32)
    tok = np.arange(7, dtype=np.int32)
    rr = oracle.rerank_tree(par[None], tok[None], prob[None], [7], 1, 7, 10)
    assert rr["n_nodes"][0] == 3
    np.testing.assert_array_equal(rr["cand"][0, :3], [0, 1, 2])


# --------------------------------------------------------------------------
# Tie order of the best-first tree across depths ([SD §5 DDTree])
# --------------------------------------------------------------------------

def test_tree_cross_depth_ties_golden():
    """Hand-derived numbering where depth-1 and depth-2 prefixes tie in Q
    (tests/golden/tree_cross_depth_ties.json states the derivation)."""
    with open(os.path.join(GOLD, "tree_cross_depth_ties.json"), encoding="utf-8") as f:
        g = json.load(f)
    m = np.array(g["marginals"], np.float32)[None]
    out = oracle.build_tree(m, 1, g["K"], g["V"], g["N"])
    ex = g["expected"]
    assert int(out["n_nodes"][0]) == ex["n_nodes"]
    for key in ("token", "parent", "depth", "score"):
        np.testing.assert_array_equal(out[key][0], np.array(ex[key]).astype(out[key].dtype), err_msg=key)
    np.testing.assert_array_equal(out["anc_mask"][0].astype(np.int64), ex["anc_mask"])


def _tied_marginals(kind, K, V, rng):
    if kind == "uniform":
        return np.full((K, V), 1.0 / V, np.float32)
    if kind == "pairs":                 # every value appears twice in a row
        half = special.softmax(rng.normal(0, 1.0, (K, (V + 1) // 2)), axis=-1) / 2
        return np.repeat(half, 2, axis=1)[:, :V].astype(np.float32)
    if kind == "certain":               # rows with a q = 1 entry: a child ties its parent
        m = special.softmax(rng.normal(0, 1.0, (K, V)), axis=-1).astype(np.float32)
        m[1::2] = 0.0
        m[1::2, 0] = 1.0
        return m
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["uniform", "pairs", "certain"])
@pytest.mark.parametrize("N", [5, 13, 40])
def test_rerank_of_the_full_trie_with_ties_is_the_ddtree(kind, N):
    # with tied marginals the two orders must also agree on every tie across
    # depths: (Q desc, depth asc, rank tuple asc) on the trie is the
    # re-ranking's (confidence desc, depth asc, BFS index asc)
    rng = np.random.default_rng(71 + N)
    K, V = 4, 3
    m = _tied_marginals(kind, K, V, rng)
    par, tok, prob = _trie_candidates(m)
    M = len(par)
    rr = oracle.rerank_tree(par[None], tok[None], prob[None], [M], 1, M, N)
    bt = oracle.build_tree(m[None], 1, K, V, N)
    for key in ("token", "parent", "depth", "score", "anc_mask", "n_nodes"):
        np.testing.assert_array_equal(rr[key], bt[key], err_msg=key)


# --------------------------------------------------------------------------
# Validity checks used where the oracle's decision sits at a rounding margin
# --------------------------------------------------------------------------

def _chain_case(rng, B, K, V, sig=2.0, noise=0.7):
    d = (rng.standard_normal((B * K, V)) * sig).astype(np.float32)
    t = np.zeros((B * (K + 1), V), np.float32)
    for b in range(B):
        t[b * (K + 1):b * (K + 1) + K] = d[b * K:(b + 1) * K] + rng.standard_normal((K, V)) * noise
        t[b * (K + 1) + K] = rng.standard_normal(V) * sig
    y = np.array([sample_from(rng, special.softmax(d[r].astype(np.float64)), 1)[0]
                  for r in range(B * K)], np.int32)
    u = grid_u(rng, B * (K + 1))
    return t, d, y, u


def test_check_chain_accepts_the_oracle_and_rejects_planted_mistakes():
    rng = np.random.default_rng(41)
    B, K, V = 300, 4, 40
    t, d, y, u = _chain_case(rng, B, K, V)
    ref = oracle.verify_chain(t, d, y, u, None, B, K, V, 1.0)
    valid, st = oracle.check_chain(t, d, y, u, None, B, K, V, 1.0, ref["A"], ref["next"])
    assert (valid == 3).all()
    np.testing.assert_array_equal(st, ref["status"])
    clear = ref["margin"] == 0
    # A one position later than a clear rejection, or one earlier than a clear
    # accept, fails the accept bits
    later = ref["A"] < K
    v2, _ = oracle.check_chain(t, d, y, u, None, B, K, V, 1.0, np.minimum(ref["A"] + 1, K), ref["next"])
    assert ((v2 & oracle.CHECK_A) == 0)[later & clear].all()
    earlier = ref["A"] > 0
    v3, _ = oracle.check_chain(t, d, y, u, None, B, K, V, 1.0, np.maximum(ref["A"] - 1, 0), ref["next"])
    assert ((v3 & oracle.CHECK_A) == 0)[earlier & clear].all()
    # a neighbouring token is not the draw at that point
    for shift in (1, -1):
        nx = (ref["next"] + shift) % V
        v4, _ = oracle.check_chain(t, d, y, u, None, B, K, V, 1.0, ref["A"], nx)
        assert ((v4 & oracle.CHECK_NEXT) == 0)[clear].all()
        assert (v4 & oracle.CHECK_A).all()
    # the same with top-k truncation and a packed layout
    cu = np.concatenate([[0], np.cumsum(rng.integers(0, K + 1, 60))]).astype(np.int32)
    rows_t = np.concatenate([np.arange(b * (K + 1), b * (K + 1) + cu[b + 1] - cu[b] + 1) for b in range(60)])
    rows_d = np.concatenate([np.arange(b * K, b * K + cu[b + 1] - cu[b]) for b in range(60)])
    args = (t[rows_t], d[rows_d], y[rows_d], u[rows_t], cu, 60, K, V, 0.8)
    r5 = oracle.verify_chain(*args, top_k=5)
    v5, s5 = oracle.check_chain(*args, r5["A"], r5["next"], top_k=5)
    assert (v5 == 3).all()
    np.testing.assert_array_equal(s5, r5["status"])
    v6, _ = oracle.check_chain(*args, r5["A"], (r5["next"] + 1) % V, top_k=5)
    assert ((v6 & oracle.CHECK_NEXT) == 0)[r5["margin"] == 0].all()


def test_check_chain_takes_either_side_of_a_margin():
    # the margin cases of test_margin_flags: u*q == p exactly (accepting and
    # rejecting are both within the slack) and a draw exactly on a CDF step
    V = 2
    tgt = np.stack([logits_of([.5, .5]), logits_of([.5, .5])])
    dft = logits_of([1.0, 0.0])[None]
    y = np.array([0], np.int32)
    u = np.array([0.5, 0.3], np.float32)
    for A, nx in ((1, 0), (0, 1)):
        v, _ = oracle.check_chain(tgt, dft, y, u, None, 1, 1, V, 1.0, [A], [nx])
        assert v[0] == 3, (A, nx)
    # after a rejection the residual [p - q]+ is one-hot at id 1: id 0 is never drawn
    v, _ = oracle.check_chain(tgt, dft, y, u, None, 1, 1, V, 1.0, [0], [0])
    assert v[0] == oracle.CHECK_A
    u = np.array([0.25, 0.5], np.float32)
    for nx in (0, 1):
        v, _ = oracle.check_chain(tgt, dft, y, u, None, 1, 1, V, 1.0, [1], [nx])
        assert v[0] == 3, nx
    v, _ = oracle.check_chain(tgt, dft, y, u, None, 1, 1, V, 1.0, [0], [1])
    assert v[0] == oracle.CHECK_NEXT       # u*q = 0.25 < p = 0.5: a rejection is not allowed


def test_check_tree_sampled_accepts_the_oracle_and_rejects_planted_mistakes():
    rng = np.random.default_rng(42)
    B, K, V, N = 40, 4, 6, 12
    marg = special.softmax(rng.standard_normal((B, K, V)) * 1.5, axis=2).astype(np.float32)
    tree = oracle.build_tree(marg, B, K, V, N)
    target = (rng.standard_normal((B, N, V)) * 1.5).astype(np.float32)
    u = grid_u(rng, (B, N))
    ref = oracle.verify_tree_sampled(target, tree["token"], tree["parent"], tree["n_nodes"], u, B, N, V, 1.0)
    args = (target, tree["token"], tree["parent"], tree["n_nodes"], u, B, N, V, 1.0)
    assert (oracle.check_tree_sampled(*args, ref["path"], ref["A"], ref["next"]) == 1).all()
    clear = ref["margin"] == 0
    bad = oracle.check_tree_sampled(*args, ref["path"], ref["A"], (ref["next"] + 1) % V)
    assert (bad[clear] == 0).all()
    # a walk cut one step short names a child's token as the extra token
    long = ref["A"] > 0
    cut = ref["path"].copy()
    A2 = np.maximum(ref["A"] - 1, 0)
    nx2 = ref["next"].copy()
    for b in np.nonzero(long)[0]:
        nx2[b] = tree["token"][b, cut[b, A2[b]]]
        cut[b, A2[b]] = -1
    bad = oracle.check_tree_sampled(*args, cut, A2, nx2)
    assert (bad[long] == 0).all()


def test_check_select_len():
    rng = np.random.default_rng(43)
    B, K, cost = 400, 8, 0.15
    conf = rng.beta(5, 2, (B, K)).astype(np.float32)
    ref = oracle.select_len(conf, B, K, cost)
    assert (oracle.check_select_len(conf, B, K, cost, ref["k"]) == 1).all()
    clear = ref["margin"] == 0
    for shift in (1, -1):
        k2 = ref["k"] + shift
        ok = oracle.check_select_len(conf, B, K, cost, k2)
        inside = (k2 >= 0) & (k2 <= K)
        assert (ok[clear & inside] == 0).all() and (ok[~inside] == 0).all()
    # s_1 == cost exactly: k = 0 (the rule) and k = 1 are both within the slack
    c = np.array([[0.5, 0.9]], np.float32)
    assert oracle.check_select_len(c, 1, 2, 0.5, [0])[0] == 1
    assert oracle.check_select_len(c, 1, 2, 0.5, [1])[0] == 1
    assert oracle.check_select_len(c, 1, 2, 0.5, [2])[0] == 0


# --------------------------------------------------------------------------
# EAGLE-2-style expansion ([SD §4 EAGLE-2]: expand by cumulative confidence)
# --------------------------------------------------------------------------

def _expand_full_trie(m, W):
    """Expansion steps that expand every node: each expanded node's children
    are all V tokens with the depth's marginal as their probability."""
    K, V = m.shape
    M = sum(V ** d for d in range(K + 1))
    cand = oracle.empty_candidates(1, M)
    exp_ids = np.full((1, W), -1, np.int32)
    for d in range(K):
        ct = np.tile(np.arange(V, dtype=np.int32), (1, W, 1))
        cp = np.tile(m[d], (1, W, 1)).astype(np.float32)
        cand = oracle.expand_tree(cand, exp_ids, ct, cp, 1, M, W, V)
        exp_ids = cand["expand"]
    return cand, M


@pytest.mark.parametrize("N", [4, 9, 20, 40])
def test_expanding_every_node_then_reranking_is_the_ddtree(N):
    # with a budget that expands every node, the candidates are the whole
    # factorised trie, and re-ranking them gives the best-first DDTree of the
    # same marginals (itself pinned by brute force)
    rng = np.random.default_rng(61 + N)
    K, V = 3, 3
    m = special.softmax(rng.normal(0, 1.5, (K, V)), axis=-1).astype(np.float32)
    cand, M = _expand_full_trie(m, V ** (K - 1))
    assert cand["n_cand"][0] == M
    rr = oracle.rerank_tree(cand["parent"], cand["token"], cand["prob"], cand["n_cand"], 1, M, N)
    bt = oracle.build_tree(m[None], 1, K, V, N)
    for key in ("token", "parent", "depth", "score", "anc_mask", "n_nodes"):
        np.testing.assert_array_equal(rr[key], bt[key], err_msg=key)
    # the re-ranking's own confidences are the ones the expansion stored
    np.testing.assert_array_equal(rr["score"][0, 1:], cand["conf"][0, rr["cand"][0, 1:]])


def test_expansion_keeps_the_best_branches_brute_force():
    rng = np.random.default_rng(62)
    for trial in range(200):
        W, C = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        M = 1 + W * C * 3
        cand = oracle.empty_candidates(1, M)
        ids = np.full((1, W), -1, np.int32)
        for layer in range(3):
            ct = rng.integers(0, 50, (1, W, C)).astype(np.int32)
            cp = (rng.integers(0, 9, (1, W, C)) / 8.0).astype(np.float32)     # coarse: frequent ties
            n0 = int(cand["n_cand"][0]) or 1
            cand = oracle.expand_tree(cand, ids, ct, cp, 1, M, W, C)
            new = list(range(n0, int(cand["n_cand"][0])))
            ids = cand["expand"]
            chosen = [int(i) for i in ids[0] if i >= 0]
            conf = cand["conf"][0]
            usable = [i for i in new if conf[i] >= 0]
            assert len(chosen) == min(W, len(usable))
            # the chosen set has the largest total confidence of any set of its size,
            # listed best first, ties by the lower index
            best = max((sum(float(conf[i]) for i in S) for S in itertools.combinations(usable, len(chosen))),
                       default=0.0)
            assert abs(sum(float(conf[i]) for i in chosen) - best) < 1e-7
            keys = [(-float(conf[i]), i) for i in chosen]
            assert keys == sorted(keys)
            if len(chosen) < len(usable):
                worst = min(float(conf[i]) for i in chosen)
                assert all(float(conf[i]) <= worst for i in usable if i not in chosen)
                assert all(i > max(j for j in chosen if conf[j] == worst)
                           for i in usable if i not in chosen and conf[i] == worst)
    # the candidates re-rank as usable trees (every parent precedes its child)
    rr = oracle.rerank_tree(cand["parent"], cand["token"], cand["prob"], cand["n_cand"], 1, M, 8)
    assert (rr["parent"][0, 1:rr["n_nodes"][0]] < np.arange(1, rr["n_nodes"][0])).all()


def test_expansion_root_invalid_slots_and_capacity():
    B, M, W, C = 1, 7, 2, 2
    cand = oracle.empty_candidates(B, M)
    # first step: the root is created and is the one node expanded (slot 1 ignored)
    out = oracle.expand_tree(cand, [[5, 9]], [[[7, 8], [1, 2]]], [[[0.25, 0.5], [0.9, 0.9]]], B, M, W, C)
    assert out["n_cand"][0] == 3
    np.testing.assert_array_equal(out["parent"][0, :3], [-1, 0, 0])
    np.testing.assert_array_equal(out["token"][0, :3], [-1, 7, 8])
    np.testing.assert_array_equal(out["conf"][0, :3], [1.0, 0.25, 0.5])
    np.testing.assert_array_equal(out["expand"][0], [2, 1])
    # second step: slot 0 names candidate 2 (expanded), slot 1 an index past the
    # candidates (skipped); a NaN probability is stored but never usable
    out = oracle.expand_tree(out, [[2, 11]], [[[3, 4], [5, 6]]], [[[np.nan, 0.5], [0.5, 0.5]]], B, M, W, C)
    assert out["n_cand"][0] == 5
    np.testing.assert_array_equal(out["parent"][0, 3:5], [2, 2])
    assert out["conf"][0, 3] == -1.0 and out["conf"][0, 4] == 0.25
    np.testing.assert_array_equal(out["expand"][0], [4, -1])
    out = oracle.expand_tree(out, [[4, 3]], [[[1, 2], [3, 4]]], [[[1.0, 1.0], [1.0, 1.0]]], B, M, W, C)
    assert out["n_cand"][0] == 7                       # candidate 3 is unusable: only node 4 expands
    np.testing.assert_array_equal(out["parent"][0, 5:7], [4, 4])
    np.testing.assert_array_equal(out["expand"][0], [5, 6])      # equal confidences: lower index first
    # full arrays: nothing more is appended and nothing is left to expand
    out = oracle.expand_tree(out, [[5, 6]], [[[1, 2], [3, 4]]], [[[1.0, 1.0], [1.0, 1.0]]], B, M, W, C)
    assert out["n_cand"][0] == 7
    np.testing.assert_array_equal(out["expand"][0], [-1, -1])
    # children past the end of the arrays are dropped
    small = oracle.expand_tree(oracle.empty_candidates(1, 4), [[0, 0]], [[[1, 2, 3, 4, 5], [0] * 5]],
                               [[[0.1, 0.2, 0.3, 0.4, 0.5], [0.0] * 5]], 1, 4, 2, 5)
    assert small["n_cand"][0] == 4
    np.testing.assert_array_equal(small["token"][0], [-1, 1, 2, 3])
    np.testing.assert_array_equal(small["expand"][0], [3, 2])
