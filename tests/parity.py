"""Shared helpers of the GPU parity tests: run the library and the oracle on the same
seeded inputs and compare them to the bar the method fixes.

  * accepted length, committed tokens and top-N (length, token) pairs: bit-exact,
    except for requests either side flags as a near-tie (|u - alpha| < 1e-4, top-2
    logit gap < 1e-3, the sampling target within 1e-8 of a CDF step, or adjacent
    top-(N+1) probabilities within 1e-3); those are counted and checked for validity;
  * logits: |GPU - oracle| <= 2e-2 absolute;
  * probabilities (outcome probabilities, length marginals): 1e-3 relative where the
    oracle's value is >= 1e-30, else the GPU value must be <= 1e-30.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import draft_block_verification_rmsnorm_amd as jsv
import oracle
import synth

LOGIT_ABS = 2e-2
PROB_REL = 1e-3
PROB_FLOOR = 1e-30
DECISION_TIES = oracle.FLAG_ACCEPT_TIE | oracle.FLAG_LOGIT_GAP | oracle.FLAG_CDF_TIE


def say(*a):
    print(*a, flush=True, file=sys.stderr)


class Case:
    """A head on the GPU plus the oracle's view of the same weights."""

    def __init__(self, head_cpu: synth.HeadData, dev, f64_weight=False):
        self.cpu = head_cpu
        self.dev = dev
        ws = head_cpu.weight_scale
        self.gpu = jsv.LMHead(head_cpu.weight.to(dev), head_cpu.norm_weight.to(dev), head_cpu.eps,
                              weight_scale=None if ws is None else ws.to(dev))
        w = head_cpu.weight.float().double().numpy() if f64_weight else head_cpu.weight
        self.oh = oracle.Head(w, head_cpu.norm_weight, head_cpu.eps, head_cpu.dtype, weight_scale=ws)


def run_verify(case: Case, blk: synth.BlockData, T, mode, seed, offset, ws, with_logits=True):
    dev = case.dev
    B, K = blk.draft_tokens.shape
    dl = blk.draft_logits.to(dev) if mode == jsv.PROPOSAL_SOFTMAX else None
    lo = torch.empty(B, K + 1, case.cpu.vocab, dtype=torch.float32, device=dev) if with_logits else None
    out = jsv.verify_block(case.gpu, blk.hidden.to(dev), blk.draft_tokens.to(dev), dl, T, mode, seed,
                           offset, ws, logits_out=lo)
    torch.cuda.synchronize()
    got = {"n_accepted": out.n_accepted.cpu().numpy(), "committed": out.committed.cpu().numpy(),
           "flags": out.flags.cpu().numpy().astype(np.int64)}
    if with_logits:
        got["logits"] = lo.cpu().numpy()
    ref = oracle.verify_block(case.oh, blk.hidden, blk.draft_tokens.numpy(),
                              blk.draft_logits if mode == oracle.PROPOSAL_SOFTMAX else None, T, mode,
                              seed, offset)
    return got, ref


def compare_verify(got, ref, drafts, stats):
    """Exact on (k, committed) unless flagged; returns nothing, updates `stats`."""
    B = drafts.shape[0]
    for b in range(B):
        stats["requests"] += 1
        fg, fr = int(got["flags"][b]), int(ref["flags"][b])
        assert (fg & oracle.FLAG_INVALID) == (fr & oracle.FLAG_INVALID), (b, fg, fr)
        if (fg | fr) & DECISION_TIES:
            stats["near_ties"] += 1
            k = int(got["n_accepted"][b])
            K = drafts.shape[1]
            assert 0 <= k <= K
            c = got["committed"][b]
            assert np.array_equal(c[:k], drafts[b, :k]) and c[k] >= 0 and np.all(c[k + 1:] == -1)
            if int(ref["n_accepted"][b]) != k or not np.array_equal(c, ref["committed"][b]):
                stats["near_tie_mismatch"] += 1
            continue
        assert int(got["n_accepted"][b]) == int(ref["n_accepted"][b]), (b, got["n_accepted"][b], ref["n_accepted"][b])
        assert np.array_equal(got["committed"][b], ref["committed"][b]), (b, got["committed"][b], ref["committed"][b])
        stats["exact"] += 1
        stats["committed_tokens"] += int(got["n_accepted"][b]) + 1


def compare_logits(got_logits, ref_logits, stats):
    d = float(np.max(np.abs(got_logits.astype(np.float64) - ref_logits)))
    stats["max_logit_err"] = max(stats.get("max_logit_err", 0.0), d)
    assert d <= LOGIT_ABS, d


def run_score(case: Case, hidden, drafts, G, T, mode, N, ws):
    dev = case.dev
    dl = G.to(dev) if mode == jsv.PROPOSAL_SOFTMAX else None
    out = jsv.score_outcomes(case.gpu, hidden.to(dev), drafts.to(dev), dl, T, mode, N, ws)
    torch.cuda.synchronize()
    got = {k: getattr(out, k).cpu().numpy() for k in ("out_len", "out_token", "out_prob", "len_marginal", "flags")}
    ref = oracle.score_outcomes(case.oh, hidden, drafts.numpy(), G if mode == oracle.PROPOSAL_SOFTMAX else None,
                                T, mode, N)
    return got, ref


def close_prob(g, r):
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    big = r >= PROB_FLOOR
    ok_big = np.abs(g[big] - r[big]) <= PROB_REL * r[big]
    return bool(np.all(ok_big) and np.all(np.abs(g[~big]) <= PROB_FLOOR))


def compare_score(got, ref, stats):
    B = got["flags"].shape[0]
    for b in range(B):
        stats["requests"] += 1
        fg, fr = int(got["flags"][b]), int(ref["flags"][b])
        assert (fg & oracle.FLAG_INVALID) == (fr & oracle.FLAG_INVALID), (b, fg, fr)
        if fr & oracle.FLAG_INVALID:
            continue
        # length marginals: fp64 products of alphas (relative 1e-3)
        assert close_prob(got["len_marginal"][b], ref["len_marginal"][b]), (got["len_marginal"][b], ref["len_marginal"][b])
        tab = ref["tables"][b]
        valid = got["out_len"][b] >= 0
        # every returned probability matches the oracle's table entry of that outcome
        gl, gt, gp = got["out_len"][b][valid], got["out_token"][b][valid], got["out_prob"][b][valid]
        assert close_prob(gp, tab[gl, gt]), (gp, tab[gl, gt])
        if (fg | fr) & (DECISION_TIES | oracle.FLAG_TOPN_TIE):
            stats["near_ties"] += 1
            continue
        assert np.array_equal(got["out_len"][b], ref["out_len"][b]), (got["out_len"][b], ref["out_len"][b])
        assert np.array_equal(got["out_token"][b], ref["out_token"][b]), (got["out_token"][b], ref["out_token"][b])
        assert close_prob(got["out_prob"][b], ref["out_prob"][b])
        stats["exact"] += 1


def new_stats():
    return {"requests": 0, "exact": 0, "near_ties": 0, "near_tie_mismatch": 0, "committed_tokens": 0}
