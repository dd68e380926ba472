"""Pins of the oracle's acceptance rule, bonus draw, outcome law and top-N (CPU only).

What each pin fixes:
  * the worked examples printed on the pages (App. F.1, App. F.3), from tests/golden/;
  * losslessness by exact enumeration of every draft tuple on a tiny vocabulary;
  * Monte Carlo through the actual Philox-driven sampler;
  * the outcome law summing to one and matching the realised outcomes (Prop. 1);
  * E[committed] = sum_k A_k (telescoping of Eq. 6);
  * temperature 0 against an independent argmax-prefix matcher;
  * top-N against a hand-built example and order invariants.
"""
import itertools
import json
from pathlib import Path

import numpy as np
import pytest
import torch
from scipy import stats

import oracle
from oracle import PROPOSAL_POINT as POINT, PROPOSAL_SOFTMAX as SOFT

GOLDEN = Path(__file__).parent / "golden"


def _tiny_rows(K, V=8, d=16, T=1.0, seed=0, sigma=0.5):
    """Target and proposal rows from a tiny head through the oracle's own pipeline."""
    g = torch.Generator().manual_seed(seed)
    head = oracle.Head((0.6 * torch.randn(V, d, generator=g)), 1 + 0.01 * torch.randn(d, generator=g),
                       1e-6, "f32")
    h = torch.randn(K + 1, d, generator=g)
    z = oracle.block_logits(head, h)
    G = oracle.block_logits(head, h[:K] + sigma * torch.randn(K, d, generator=g))
    P = np.array([oracle.probs(z[i], T) for i in range(K + 1)])
    Q = np.array([oracle.probs(G[i], T) for i in range(K)])
    return z, G, P, Q


# ---- worked examples printed on the pages ---------------------------------------------
def test_f1_worked_example():
    gold = json.loads((GOLDEN / "f1_worked_example.json").read_text())
    e = gold["expected"]
    d1, d2, b, c = 0, 1, 2, 3
    P = np.zeros((3, 4))
    P[0, d1], P[0, c] = gold["p_row0_d1"], 1 - gold["p_row0_d1"]
    P[1, d2], P[1, b], P[1, c] = gold["p_row1_d2"], gold["p_row1_b"], 1 - gold["p_row1_d2"] - gold["p_row1_b"]
    P[2] = 0.25
    table, marg, flags = oracle.outcome_table(P, None, [d1, d2], POINT)
    assert flags == 0
    assert table[1, b] == pytest.approx(e["P(1,b)"], abs=1e-15)
    assert marg == pytest.approx([e["P(0)"], e["P(1)"], e["P(2)"]], abs=1e-15)
    # the chain printed on the page: accept d1, reject d2, then draw b from the residual
    a1 = oracle.accept_prob(P[0], None, d1, POINT)
    a2 = oracle.accept_prob(P[1], None, d2, POINT)
    r = oracle.residual(P[1], None, d2, POINT)
    assert a1 * (1 - a2) == pytest.approx(e["accept d1 then reject d2"], abs=1e-15)
    assert r[b] / r.sum() == pytest.approx(e["residual draw of b"], abs=1e-15)


def test_f3_softmax_proposal_on_argmax_draft():
    gold = json.loads((GOLDEN / "f3_counterexample.json").read_text())
    p = np.array([gold["p_d"], 1 - gold["p_d"]])
    q = np.array([gold["q_d"], 1 - gold["q_d"]])
    e = gold["expected"]
    for mode, key in ((SOFT, "softmax proposal: probability of committing d"),
                      (POINT, "point-mass proposal: probability of committing d")):
        alpha = oracle.accept_prob(p, q, 0, mode)
        r = oracle.residual(p, q, 0, mode)
        commit_d = alpha + (1 - alpha) * r[0] / r.sum()
        assert commit_d == pytest.approx(e[key], abs=1e-15)


# ---- losslessness by exact enumeration --------------------------------------------------
def _committed_law(P, Q, mode, draft_weight):
    """Exact law of the committed token at every position, enumerating draft tuples.

    Returns reach[j] = Pr(position j is reached) and law[j, v] = Pr(reach j, commit v).
    Rows do not depend on the drafted prefix here, so the target law at j is P[j].
    """
    K, V = Q.shape if Q is not None else (P.shape[0] - 1, P.shape[1])
    reach = np.zeros(K + 1)
    law = np.zeros((K + 1, V))
    for drafts in itertools.product(range(V), repeat=K):
        w = draft_weight(drafts)
        if w == 0.0:
            continue
        prob_here = w
        for j in range(K):
            q = Q[j] if Q is not None else None
            alpha = oracle.accept_prob(P[j], q, drafts[j], mode)
            reach[j] += prob_here
            law[j, drafts[j]] += prob_here * alpha
            r = oracle.residual(P[j], q, drafts[j], mode)
            if r.sum() > 0:
                law[j] += prob_here * (1 - alpha) * r / r.sum()
            prob_here *= alpha
        reach[K] += prob_here
        law[K] += prob_here * P[K]
    return reach, law


@pytest.mark.parametrize("K", [1, 2, 3, 4])
@pytest.mark.parametrize("T", [1.0, 0.7])
def test_lossless_softmax_proposal_drafts_from_q(K, T):
    _, _, P, Q = _tiny_rows(K, T=T, seed=K)
    reach, law = _committed_law(P, Q, SOFT, lambda ds: np.prod([Q[i, d] for i, d in enumerate(ds)]))
    for j in range(K + 1):
        assert np.max(np.abs(law[j] / reach[j] - P[j])) < 1e-12


@pytest.mark.parametrize("K", [1, 3, 4])
def test_lossless_point_mass_for_every_fixed_draft(K):
    _, _, P, _ = _tiny_rows(K, T=1.0, seed=10 + K)
    V = P.shape[1]
    for drafts in itertools.islice(itertools.product(range(V), repeat=K), 0, None, 37):
        reach, law = _committed_law(P, None, POINT, lambda ds: float(ds == drafts))
        for j in range(K + 1):
            if reach[j] > 0:
                assert np.max(np.abs(law[j] / reach[j] - P[j])) < 1e-12


def test_softmax_proposal_on_argmax_drafts_is_not_lossless():
    # the enumeration has the power to see the App. F.3 failure
    _, _, P, Q = _tiny_rows(2, T=1.0, seed=3)
    drafts = tuple(int(np.argmax(Q[i])) for i in range(2))
    reach, law = _committed_law(P, Q, SOFT, lambda ds: float(ds == drafts))
    assert np.max(np.abs(law[0] / reach[0] - P[0])) > 1e-3


# ---- the actual sampler, driven by Philox ---------------------------------------------------
def _run_sampler(z, g, drafts, T, mode, n, seed=11):
    K = len(drafts)
    rows = np.arange(K + 1)
    out = []
    for off in range(n):
        u, v = oracle.philox.block_uniforms_np(seed, off, 0, rows)
        out.append(oracle.verify_request(z, g, drafts, T, mode, u, v))
    return out


@pytest.mark.parametrize("mode", [SOFT, POINT])
def test_monte_carlo_sampler_is_lossless(mode):
    K, n = 2, 30_000
    z, G, P, Q = _tiny_rows(K, T=1.0, seed=21)
    rng = np.random.default_rng(0)
    counts = np.zeros((K + 1, P.shape[1]))
    for off in range(n):
        drafts = [int(rng.choice(P.shape[1], p=Q[i])) for i in range(K)]
        u, v = oracle.philox.block_uniforms_np(5, off, 0, np.arange(K + 1))
        k, committed, _ = oracle.verify_request(z, G if mode == SOFT else None, drafts, 1.0, mode, u, v)
        for j in range(k + 1):
            counts[j, committed[j]] += 1
    for j in range(K + 1):
        expected = P[j] * counts[j].sum()
        keep = expected > 5
        chi = stats.chisquare(counts[j][keep], expected[keep] * counts[j][keep].sum() / expected[keep].sum())
        assert chi.pvalue > 1e-4


@pytest.mark.parametrize("mode", [POINT, SOFT])
def test_outcome_law_matches_realised_outcomes(mode):
    # Prop. 1 (App. F.1): with the decoder equal to the target, Eq. 6 is the law of (k, a)
    K, n = 3, 30_000
    z, G, P, Q = _tiny_rows(K, T=1.0, seed=33)
    drafts = [int(np.argmax(Q[i])) for i in range(K)]
    table, marg, _ = oracle.outcome_table(P, Q if mode == SOFT else None, drafts, mode)
    assert table.sum() == pytest.approx(1.0, abs=1e-12)
    counts = np.zeros_like(table)
    total_committed = 0
    for k, committed, _ in _run_sampler(z, G if mode == SOFT else None, drafts, 1.0, mode, n):
        counts[k, committed[k]] += 1
        total_committed += k + 1
    keep = table * n > 5
    chi = stats.chisquare(counts[keep], table[keep] * counts[keep].sum() / table[keep].sum())
    assert chi.pvalue > 1e-4
    # E[committed] = sum_k A_k with A_k the probability of reaching row k
    A = np.cumprod([1.0] + [oracle.accept_prob(P[i], Q[i] if mode == SOFT else None, drafts[i], mode)
                            for i in range(K)])
    assert np.sum((np.arange(K + 1) + 1) * marg) == pytest.approx(A.sum(), abs=1e-12)
    se = np.sqrt(K * K / n)
    assert abs(total_committed / n - A.sum()) < 5 * se


@pytest.mark.parametrize("mode", [POINT, SOFT])
@pytest.mark.parametrize("T", [1.0, 0.5, 2.0])
def test_outcome_law_sums_to_one(mode, T):
    for seed in range(5):
        _, _, P, Q = _tiny_rows(4, V=16, T=T, seed=seed)
        drafts = [int(x) for x in np.random.default_rng(seed).integers(0, 16, 4)]
        table, marg, _ = oracle.outcome_table(P, Q if mode == SOFT else None, drafts, mode)
        assert table.sum() == pytest.approx(1.0, abs=1e-12)
        assert table.sum(axis=1) == pytest.approx(marg, abs=1e-14)
        if mode == POINT:   # Eq. 6: P(k, d_k) = 0 and P(k, a) = A_k p_k(a)
            for k in range(4):
                assert table[k, drafts[k]] == 0.0


# ---- temperature 0 ------------------------------------------------------------------------
def _argmax_prefix(z, drafts):
    """Independent greedy matcher: accept while the draft equals the row's argmax."""
    k = 0
    while k < len(drafts) and drafts[k] == int(np.argmax(z[k])):
        k += 1
    return k, list(drafts[:k]) + [int(np.argmax(z[k]))]


@pytest.mark.parametrize("mode", [SOFT, POINT])
def test_temperature_zero_is_argmax_prefix_matching(mode):
    rng = np.random.default_rng(4)
    for trial in range(300):
        K, V = int(rng.integers(1, 6)), int(rng.integers(2, 9))
        z = rng.integers(0, 4, size=(K + 1, V)).astype(np.float64)   # many exact ties
        g = rng.standard_normal((K, V))
        drafts = [int(np.argmax(z[i])) if rng.random() < 0.7 else int(rng.integers(0, V)) for i in range(K)]
        u, v = rng.random(K + 1), rng.random(K + 1)
        k, committed, flags = oracle.verify_request(z, g if mode == SOFT else None, drafts, 0, mode, u, v)
        kk, cc = _argmax_prefix(z, drafts)
        assert k == kk and committed[:k + 1] == cc and committed[k + 1:] == [-1] * (K - k)
        # with many ties the gap flag fires whenever a deciding row has a shared maximum
        shared = any(np.sum(z[i] == z[i].max()) > 1 for i in range(k + 1))
        assert bool(flags & oracle.FLAG_LOGIT_GAP) == shared
        # scoring at T = 0 puts all mass on the greedy outcome
        P = np.array([oracle.probs(z[i], 0) for i in range(K + 1)])
        Q = np.array([oracle.probs(g[i], 0) for i in range(K)]) if mode == SOFT else None
        table, _, _ = oracle.outcome_table(P, Q, drafts, mode)
        assert table[kk, cc[-1]] == pytest.approx(1.0) and table.sum() == pytest.approx(1.0)


# ---- bonus draw ------------------------------------------------------------------------------
def test_inverse_cdf_steps():
    r = np.array([0.1, 0.0, 0.3, 0.6])
    assert oracle.inverse_cdf(r, 0.05)[0] == 0
    assert oracle.inverse_cdf(r, 0.2)[0] == 2      # zero-mass token 1 is never drawn
    assert oracle.inverse_cdf(r, 0.999)[0] == 3
    assert oracle.inverse_cdf(r * 7.0, 0.2)[0] == 2  # unnormalised r works the same
    tok, flags = oracle.inverse_cdf(r, 0.1 / 1.0 + 1e-12)
    assert tok == 2 and flags & oracle.FLAG_CDF_TIE
    tok, flags = oracle.inverse_cdf(np.array([0.0, 0.5, 0.0]), 0.3)
    assert tok == 1 and flags == 0


def test_inverse_cdf_window_is_absolute():
    # a small residual mass (Z = 1e-3): the window stays 1e-8 of probability mass
    r = np.array([0.1, 0.0, 0.3, 0.6]) * 1e-3
    tok, flags = oracle.inverse_cdf(r, (1e-4 + 5e-9) / 1e-3)
    assert tok == 2 and flags & oracle.FLAG_CDF_TIE
    tok, flags = oracle.inverse_cdf(r, (1e-4 + 5e-8) / 1e-3)
    assert tok == 2 and not flags & oracle.FLAG_CDF_TIE


def test_committed_count_includes_bonus():
    # tau convention (paper §3, §5.1): a round commits the accepted prefix plus one bonus token
    rng = np.random.default_rng(8)
    z, G, P, Q = _tiny_rows(4, T=1.0, seed=8)
    for off in range(200):
        drafts = [int(rng.choice(8, p=Q[i])) for i in range(4)]
        u, v = oracle.philox.block_uniforms_np(1, off, 0, np.arange(5))
        k, committed, _ = oracle.verify_request(z, G, drafts, 1.0, SOFT, u, v)
        n_committed = sum(c >= 0 for c in committed)
        assert n_committed == k + 1
        assert committed[:k] == drafts[:k]
        if k < 4:   # the bonus at a rejection is never the rejected token when q >= p there
            r = oracle.residual(P[k], Q[k], drafts[k], SOFT)
            assert r[committed[k]] > 0


def test_invalid_inputs_commit_nothing():
    z = np.zeros((3, 4))
    z[1, 2] = np.nan
    k, committed, flags = oracle.verify_request(z, None, [0, 1], 1.0, POINT, [0.5] * 3, [0.5] * 3)
    assert k == -1 and committed == [-1, -1, -1] and flags == oracle.FLAG_INVALID
    k, committed, flags = oracle.verify_request(np.zeros((3, 4)), None, [0, 4], 1.0, POINT,
                                                [0.5] * 3, [0.5] * 3)
    assert k == -1 and flags == oracle.FLAG_INVALID


def test_zero_residual_falls_back_to_target_row():
    # p = q and the draft token has no mass under either (exp underflows to 0):
    # alpha = 0 and the residual max(p - q, 0) is zero everywhere
    z = np.array([[0.0, 0.0, -1000.0], [0.0, 0.0, 0.7]])
    g = np.array([[0.0, 0.0, -1000.0]])
    p0 = oracle.probs(z[0], 1.0)
    k, committed, flags = oracle.verify_request(z, g, [2], 1.0, SOFT, [0.5, 0.5], [0.7, 0.7])
    assert k == 0 and flags & oracle.FLAG_ZERO_RESIDUAL
    assert committed[0] == oracle.inverse_cdf(p0, 0.7)[0]


# ---- top-N -------------------------------------------------------------------------------------
def test_top_n_hand_example():
    table = np.array([[0.0, 0.2, 0.05, 0.0],
                      [0.2, 0.0, 0.1, 0.05],
                      [0.0, 0.0, 0.4, 0.0]])
    lens, toks, pr, flags = oracle.top_n(table, 4)
    assert list(zip(lens, toks)) == [(2, 2), (0, 1), (1, 0), (1, 2)]   # tie 0.2: smaller k first
    assert pr == pytest.approx([0.4, 0.2, 0.2, 0.1])
    assert flags & oracle.FLAG_TOPN_TIE
    lens, toks, pr, flags = oracle.top_n(table, 9)    # fewer outcomes than N: padded
    assert list(lens[6:]) == [-1, -1, -1] and list(toks[6:]) == [-1, -1, -1] and list(pr[6:]) == [0, 0, 0]
    assert sorted(zip(lens[:6], toks[:6])) == sorted(zip(*np.nonzero(table)))
    same = np.array([[0.0, 0.3, 0.3]])
    lens, toks, _, _ = oracle.top_n(same, 2)
    assert list(toks) == [1, 2]                        # equal P and k: smaller token first


@pytest.mark.parametrize("N", [1, 8, 20])
def test_top_n_order_invariants(N):
    _, _, P, Q = _tiny_rows(4, V=64, d=16, T=1.0, seed=N)
    drafts = [int(np.argmax(Q[i])) for i in range(4)]
    table, _, _ = oracle.outcome_table(P, Q, drafts, SOFT)
    lens, toks, pr, _ = oracle.top_n(table, N)
    chosen = set(zip(lens.tolist(), toks.tolist()))
    worst = pr[N - 1]
    # every outcome left out is no more probable than the last one chosen
    for k in range(5):
        for a in range(64):
            if (k, a) not in chosen:
                assert table[k, a] <= worst
    assert np.all(np.diff(pr) <= 0)
    assert np.array_equal(pr, table[lens, toks])
