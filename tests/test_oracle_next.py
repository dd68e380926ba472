"""Pins of the oracle's next-row functions: anchor replacement, cache lookup, the
calibrated length score and SSD's geometric fan-out (JetSpec++ paper §4.1, §4.3,
App. B.1, App. F.2)."""
import itertools
import json
from pathlib import Path

import numpy as np
import torch

import oracle

GOLDEN = Path(__file__).resolve().parent / "golden"


# ---- SSD geometric fan-out (App. F.2) -------------------------------------------------
def test_fanout_worked_example():
    ex = json.loads((GOLDEN / "f4_fanout_example.json").read_text())
    a, rho, gamma, B = ex["alpha"], ex["rho"], ex["gamma"], ex["B"]
    P = oracle.ssd_length_law(a, gamma)
    w = P ** (1.0 / (1.0 + rho))
    all_lengths = oracle.fanout_objective(P, B * w / w.sum(), rho)
    assert abs(all_lengths - ex["expected"]["hit mass of the series over all lengths 0..4"]) < 5e-4
    F, Fi, obj, M = oracle.geometric_fanout(a, rho, gamma, B)
    assert abs(obj - ex["expected"]["hit mass of the series rescaled over lengths {0,1,2,4} (the maximiser)"]) < 5e-4
    assert [k for k in range(gamma + 1) if F[k] >= 1.0] == ex["expected"]["active lengths of the maximiser"]
    assert int(Fi.sum()) == B and np.all(Fi[F == 0] == 0)


def test_fanout_length_law_sums_to_one():
    for a in (0.1, 0.5, 0.93):
        for g in (1, 4, 15):
            assert abs(oracle.ssd_length_law(a, g).sum() - 1.0) < 1e-12


def test_fanout_beats_every_active_set():
    # brute force over every set of active lengths (the proof restricts to top-M sets)
    for a, rho, gamma, B in [(0.6, 1.0, 4, 10), (0.8, 0.5, 5, 12), (0.3, 2.0, 3, 6), (0.9, 1.5, 6, 20)]:
        P = oracle.ssd_length_law(a, gamma)
        _, _, obj, _ = oracle.geometric_fanout(a, rho, gamma, B)
        best = 0.0
        for r in range(1, gamma + 2):
            for S in itertools.combinations(range(gamma + 1), r):
                w = np.array([P[k] ** (1.0 / (1.0 + rho)) for k in S])
                F = np.zeros(gamma + 1)
                F[list(S)] = B * w / w.sum()
                if np.all(F[list(S)] >= 1.0):
                    best = max(best, oracle.fanout_objective(P, F, rho))
        assert abs(obj - best) < 1e-12, (a, rho, gamma, B, obj, best)


def test_fanout_equal_marginal_gains():
    # the stationarity condition of the proof: P(k) rho F_k^(-rho-1) is one constant on
    # the active lengths
    for a, rho, gamma, B in [(0.6, 1.0, 4, 10), (0.85, 0.7, 8, 16)]:
        P = oracle.ssd_length_law(a, gamma)
        F, _, _, _ = oracle.geometric_fanout(a, rho, gamma, B)
        g = [P[k] * rho * F[k] ** (-rho - 1.0) for k in range(gamma + 1) if F[k] > 0]
        assert max(g) - min(g) < 1e-12 * max(g)
        assert abs(F.sum() - B) < 1e-9


def test_fanout_largest_remainders():
    F, Fi, _, _ = oracle.geometric_fanout(0.6, 1.0, 4, 10)
    # floors 3, 2, 2, 0, 1 leave 2 anchors for the largest remainders (k = 1: .631, k = 4: .934)
    assert list(Fi) == [3, 3, 2, 0, 2]


# ---- calibrated length score (App. B.1) -------------------------------------------------
def test_calibrated_lengths_telescope_and_closed_form():
    rng = np.random.default_rng(3)
    p = rng.uniform(0.0, 1.0, size=(5, 16))
    s, f = oracle.calibrated_lengths(p)
    assert np.all(f == 0)
    assert np.all(np.abs(s.sum(axis=1) - 1.0) < 1e-12)
    c = np.full((1, 7), 0.8)
    s, _ = oracle.calibrated_lengths(c)
    # constant estimates give the geometric law of the fan-out model
    assert np.allclose(s[0], oracle.ssd_length_law(0.8, 7), rtol=0, atol=1e-15)
    s, _ = oracle.calibrated_lengths(np.array([[1.0, 1.0, 0.0, 0.5]]))
    assert list(s[0]) == [0.0, 0.0, 1.0, 0.0, 0.0]


def test_calibrated_lengths_invalid():
    s, f = oracle.calibrated_lengths(np.array([[0.5, 1.5], [0.5, np.nan], [0.2, 0.3]]))
    assert list(f) == [oracle.FLAG_INVALID, oracle.FLAG_INVALID, 0]
    assert np.all(s[:2] == 0.0)


# ---- anchor replacement and cache lookup (§4.3, §4.1) -----------------------------------
def _identity_head(V):
    return oracle.Head(torch.eye(V, dtype=torch.float32), torch.ones(V, dtype=torch.float32), 1e-6, "f32")


def _rows(V, tokens, scale=4.0):
    h = np.full((len(tokens), V), 0.1)
    for i, t in enumerate(tokens):
        h[i, t] = scale
    return torch.tensor(h, dtype=torch.float32)


def test_anchor_replace_first_mismatch():
    V = 16
    head = _identity_head(V)
    # decoder argmaxes 3, 5, 7, 9, 11 over rows 0..4; the drafts match rows 0 and 1 only
    hid = _rows(V, [3, 5, 7, 9, 11])[None]
    pos, tok, fl = oracle.anchor_replace(head, hid, np.array([[3, 5, 8, 9]]))
    assert (pos[0], tok[0], fl[0]) == (2, 7, 0)
    pos, tok, _ = oracle.anchor_replace(head, hid, np.array([[3, 5, 7, 9]]))
    assert (pos[0], tok[0]) == (4, 11)   # every draft matches: the row after the block
    pos, tok, _ = oracle.anchor_replace(head, hid, np.array([[0, 5, 7, 9]]))
    assert (pos[0], tok[0]) == (0, 3)
    pos, tok, fl = oracle.anchor_replace(head, hid, np.array([[3, 5, 99, 9]]))
    assert (pos[0], tok[0], fl[0]) == (-1, -1, oracle.FLAG_INVALID)


def test_anchor_replace_tie_lowest_id_flagged():
    V = 16
    head = _identity_head(V)
    h = _rows(V, [6, 6])
    h[0, 2] = h[0, 6]                        # a tie in row 0: token 2 wins
    pos, tok, fl = oracle.anchor_replace(head, h[None], np.array([[6]]))
    assert (pos[0], tok[0]) == (0, 2) and fl[0] & oracle.FLAG_LOGIT_GAP


def test_cache_lookup_hits_and_misses():
    out_len = np.array([[2, 0, 2, -1], [1, 1, 3, 0]])
    out_tok = np.array([[7, 4, 9, -1], [5, 6, 2, 1]])
    committed = np.array([[10, 11, 9, -1, -1], [1, 6, -1, -1, -1]])
    n_acc = np.array([2, 1])
    assert list(oracle.cache_lookup(n_acc, committed, out_len, out_tok)) == [2, 1]
    assert list(oracle.cache_lookup(np.array([0, -1]), np.array([[8, -1, -1, -1, -1]] * 2),
                                    out_len, out_tok)) == [-1, -1]
