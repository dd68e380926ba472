"""GPU parity: the HIP library against the CPU oracle on the same seeded inputs.

Sizes: the tiny f32 case (d=256, V=1024, K=4) over 1000 blocks; the Qwen3-8B LM-head
shape (d=4096, V=151936, K=16, B=1) at T = 0 and 1 in both proposal modes; K=32 B=4;
d=5120; scoring with top-8; and the edge cases (ragged vocabularies, many row passes,
invalid inputs, top_n = 64, run-to-run bit identity).  Everything calls the C ABI through
the ctypes binding.
"""
import numpy as np
import pytest
import torch

import draft_block_verification_rmsnorm_amd as jsv
import oracle
import synth
from parity import (Case, compare_logits, compare_score, compare_verify, new_stats, run_score,
                    run_verify, say)

pytestmark = pytest.mark.gpu
SOFT, POINT = jsv.PROPOSAL_SOFTMAX, jsv.PROPOSAL_POINT


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    jsv.load_library()
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def tiny(dev):
    return Case(synth.head_for(synth.CONFIGS["tiny"]), dev)


@pytest.fixture(scope="module")
def qwen(dev):
    return Case(synth.head_for(synth.CONFIGS["qwen8b_k16"]), dev, f64_weight=True)


# ---- LM head ---------------------------------------------------------------------------
@pytest.mark.parametrize("V,d,dtype,rows", [
    (1024, 256, synth.F32, 5), (1000, 256, synth.BF16, 3), (4099, 512, synth.BF16, 17),
    (2048, 4096, synth.BF16, 40), (777, 5120, synth.BF16, 33), (300, 1024, synth.F32, 1),
    (4099, 512, synth.FP8, 17), (1000, 5120, synth.FP8, 33),
    # bf16 heads staged through LDS with fewer quarters per group than ring slots
    (3001, 1024, synth.BF16, 17), (2050, 2048, synth.BF16, 1), (5003, 3072, synth.BF16, 16),
    (3001, 2048, synth.FP8, 17), (1500, 4096, synth.FP8, 33), (777, 4096, synth.FP8, 1),
])
def test_lmhead_logits(dev, V, d, dtype, rows):
    say(f"lmhead V={V} d={d} {dtype} rows={rows}")
    head = synth.random_head(V, d, dtype, seed=V + d)
    case = Case(head, dev)
    g = torch.Generator().manual_seed(rows)
    h = torch.randn(rows, d, generator=g).to(head.norm_weight.dtype)
    z = jsv.lmhead_logits(case.gpu, h.to(dev))
    torch.cuda.synchronize()
    ref = oracle.lmhead_logits(case.oh, h)
    err = float(np.max(np.abs(z.cpu().numpy().astype(np.float64) - ref)))
    say(f"  max |dz| = {err:.3e}")
    assert err <= 2e-2
    assert err <= 1e-3   # internal alarm: the expected error is ~1e-6


# ---- verification: tiny oracle case --------------------------------------------------------
@pytest.mark.parametrize("T", [0.0, 1.0])
def test_verify_tiny_1000_blocks(tiny, dev, T):
    cfg = synth.CONFIGS["tiny"]
    ws = jsv.new_workspace(tiny.gpu, 1, cfg.K)
    st = new_stats()
    for blk_id in range(1000):
        if blk_id % 250 == 0:
            say(f"tiny verify T={T} block {blk_id}")
        blk = synth.make_block(tiny.cpu, 1, cfg.K, cfg.sigma, T, seed=blk_id)
        got, ref = run_verify(tiny, blk, T, SOFT, 0, blk_id, ws)
        compare_verify(got, ref, blk.draft_tokens.numpy(), st)
        compare_logits(got["logits"], ref["logits"], st)
    say(f"  {st}")
    assert st["exact"] >= 950


@pytest.mark.parametrize("mode", [SOFT, POINT])
def test_verify_tiny_batched_modes(tiny, dev, mode):
    cfg = synth.CONFIGS["tiny"]
    ws = jsv.new_workspace(tiny.gpu, 8, cfg.K)
    st = new_stats()
    for seed in range(20):
        T = [0.0, 0.5, 1.0, 2.0][seed % 4]
        say(f"tiny batched mode={mode} seed={seed} T={T}")
        blk = synth.make_block(tiny.cpu, 8, cfg.K, cfg.sigma, T, seed=10_000 + seed)
        got, ref = run_verify(tiny, blk, T, mode, seed, 3 * seed, ws)
        compare_verify(got, ref, blk.draft_tokens.numpy(), st)
    say(f"  {st}")
    assert st["exact"] >= 150


# ---- verification: Qwen3-8B LM-head shape ----------------------------------------------------
@pytest.mark.parametrize("T,mode", [(0.0, SOFT), (1.0, SOFT), (1.0, POINT)])
def test_verify_qwen8b_k16(qwen, dev, T, mode):
    cfg = synth.CONFIGS["qwen8b_k16"]
    ws = jsv.new_workspace(qwen.gpu, 1, cfg.K)
    st = new_stats()
    for seed in range(3):
        say(f"qwen8b K=16 verify T={T} mode={mode} seed={seed}")
        blk = synth.make_block(qwen.cpu, 1, cfg.K, cfg.sigma, T, seed=seed)
        got, ref = run_verify(qwen, blk, T, mode, seed, 0, ws)
        compare_verify(got, ref, blk.draft_tokens.numpy(), st)
        compare_logits(got["logits"], ref["logits"], st)
    say(f"  {st}")
    assert st["exact"] >= 2


def _cdf_drift(zg, zo, g, T):
    """How far the logit error can move a bonus decision: the largest difference of the
    residual CDFs built from two logit rows (same draft logits g, or the target row alone
    when g is None), plus the move of the total Z (t = v Z moves by at most that), in
    float64 and in units of probability mass."""
    def resid(z):
        p = np.exp((z - z.max()) / T)
        p /= p.sum()
        if g is None:
            return p
        q = np.exp((g - g.max()) / T)
        q /= q.sum()
        return np.maximum(p - q, 0.0)
    cg, co = np.cumsum(resid(np.asarray(zg, np.float64))), np.cumsum(resid(np.asarray(zo, np.float64)))
    return float(np.max(np.abs(cg - co)) + abs(cg[-1] - co[-1]))


def test_cdf_drift_within_window(qwen, dev):
    """The kernel's fp32-accumulated logits move the residual CDF by less than half the CDF
    near-tie window at the Qwen3-8B shape, on every row of several blocks (K = 16 and the
    K = 32 generator), so a bonus draw that the logit error could flip is always flagged."""
    T = 1.0
    worst = 0.0
    for name, seeds in (("qwen8b_k16", 3), ("qwen8b_k32_b4", 2)):
        cfg = synth.CONFIGS[name]
        ws = jsv.new_workspace(qwen.gpu, 1, cfg.K)
        for seed in range(seeds):
            say(f"{name} CDF drift seed={seed}")
            blk = synth.make_block(qwen.cpu, 1, cfg.K, cfg.sigma, T, seed=100 + seed)
            got, ref = run_verify(qwen, blk, T, SOFT, seed, 0, ws)
            zo = ref["logits"][0]
            G = blk.draft_logits[0].numpy().astype(np.float64)
            for i in range(cfg.K + 1):
                dr = _cdf_drift(got["logits"][0, i], zo[i], G[i] if i < cfg.K else None, T)
                worst = max(worst, dr)
    say(f"  largest CDF drift {worst:.3e} (window {oracle.CDF_TIE:.0e})")
    assert worst < 0.5 * oracle.CDF_TIE


def test_verify_qwen8b_fp8(dev):
    """The fp8 (E4M3 weights, bf16 states) head at the Qwen3-8B shape: exact against the
    oracle's quantised target."""
    cfg = synth.CONFIGS["qwen8b_k16_fp8"]
    case = Case(synth.head_for(cfg), dev, f64_weight=True)
    ws = jsv.new_workspace(case.gpu, 1, cfg.K)
    st = new_stats()
    for T in (0.0, 1.0):
        for seed in range(2):
            say(f"qwen8b fp8 verify T={T} seed={seed}")
            blk = synth.make_block(case.cpu, 1, cfg.K, cfg.sigma, T, seed=60 + seed)
            got, ref = run_verify(case, blk, T, SOFT, seed, 3, ws)
            compare_verify(got, ref, blk.draft_tokens.numpy(), st)
            compare_logits(got["logits"], ref["logits"], st)
    say(f"  {st}")
    assert st["exact"] >= 3


def test_verify_qwen8b_k32_b4(qwen, dev):
    cfg = synth.CONFIGS["qwen8b_k32_b4"]
    ws = jsv.new_workspace(qwen.gpu, cfg.batch, cfg.K)
    st = new_stats()
    for T in (0.0, 1.0):
        say(f"qwen8b K=32 B=4 verify T={T}")
        blk = synth.make_block(qwen.cpu, cfg.batch, cfg.K, cfg.sigma, T, seed=40 + int(T))
        got, ref = run_verify(qwen, blk, T, SOFT, 5, 9, ws)
        compare_verify(got, ref, blk.draft_tokens.numpy(), st)
        compare_logits(got["logits"], ref["logits"], st)
    say(f"  {st}")
    assert st["exact"] >= 6


def test_verify_ragged_vocab_staged_head(dev):
    """bf16 head with d = 1024 (one quarter per group, three ring slots), a ragged
    vocabulary and two passes of 17 rows; softmax proposal at T = 1, so the draft logits
    travel by DMA too."""
    head = synth.random_head(3001, 1024, synth.BF16, seed=31)
    case = Case(head, dev)
    ws = jsv.new_workspace(case.gpu, 2, 16)
    st = new_stats()
    for seed in range(4):
        say(f"ragged V=3001 d=1024 B=2 K=16 seed={seed}")
        blk = synth.make_block(head, 2, 16, 0.5, 1.0, seed=seed)
        got, ref = run_verify(case, blk, 1.0, SOFT, seed, 1, ws)
        compare_verify(got, ref, blk.draft_tokens.numpy(), st)
        compare_logits(got["logits"], ref["logits"], st)
    say(f"  {st}")
    assert st["exact"] >= 6


def test_verify_split_d_ragged(dev):
    """More rows than one pass holds, on a ragged vocabulary: the LM head splits d into
    blocks of 1024 columns (two here) and sums their partial products.  B = 3, K = 32
    (99 rows, seven tiles), V = 5003, both temperatures and both proposals."""
    head = synth.random_head(5003, 2048, synth.BF16, seed=41)
    case = Case(head, dev)
    ws = jsv.new_workspace(case.gpu, 3, 32)
    st = new_stats()
    for T, mode in ((0.0, SOFT), (1.0, SOFT), (1.0, POINT)):
        for seed in range(2):
            say(f"split-d V=5003 d=2048 B=3 K=32 T={T} mode={mode} seed={seed}")
            blk = synth.make_block(head, 3, 32, 0.3, T, seed=70 + seed)
            got, ref = run_verify(case, blk, T, mode, seed, 4, ws)
            compare_verify(got, ref, blk.draft_tokens.numpy(), st)
            compare_logits(got["logits"], ref["logits"], st)
    say(f"  {st}")
    assert st["exact"] >= 12


def test_verify_d5120(dev):
    head = synth.head_for(synth.CONFIGS["d5120_k16_b1"])
    case = Case(head, dev, f64_weight=True)
    st = new_stats()
    for name in ("d5120_k16_b1", "d5120_k32_b2"):
        cfg = synth.CONFIGS[name]
        ws = jsv.new_workspace(case.gpu, cfg.batch, cfg.K)
        for T in (0.0, 1.0):
            say(f"{name} verify T={T}")
            blk = synth.make_block(head, cfg.batch, cfg.K, cfg.sigma, T, seed=50 + int(T))
            got, ref = run_verify(case, blk, T, SOFT, 1, 2, ws)
            compare_verify(got, ref, blk.draft_tokens.numpy(), st)
            compare_logits(got["logits"], ref["logits"], st)
    say(f"  {st}")
    assert st["exact"] >= 4


def test_sampler_law_point_mass_any_draft(tiny, dev):
    """Losslessness through the GPU sampler itself: with the point-mass proposal the token
    committed at row 0 is distributed as p_0 for any fixed draft (App. F.3), so over many
    Philox offsets its histogram must pass a chi-square test against the oracle's p_0."""
    from scipy import stats as sps
    cfg = synth.CONFIGS["tiny"]
    B, K, T = 8, cfg.K, 1.0
    blk = synth.make_block(tiny.cpu, 1, K, cfg.sigma, T, seed=777)
    hid = blk.hidden.expand(B, -1, -1).contiguous().to(dev)
    drafts = blk.draft_tokens.expand(B, -1).contiguous().to(dev)
    ws = jsv.new_workspace(tiny.gpu, B, K)
    out = jsv.VerifyOut(B, K, dev)
    calls = 3000
    toks = torch.empty(calls, B, dtype=torch.int32, device=dev)
    say(f"sampler law: {calls} calls x {B} requests")
    for off in range(calls):
        jsv.verify_block(tiny.gpu, hid, drafts, None, T, POINT, 5, off, ws, out=out)
        toks[off] = out.committed[:, 0]
    torch.cuda.synchronize()
    t = toks.cpu().numpy().ravel()
    z0 = oracle.block_logits(tiny.oh, blk.hidden[0, :1])[0]
    p0 = oracle.probs(z0, T)
    n = t.size
    counts = np.bincount(t, minlength=p0.size).astype(np.float64)
    exp = p0 * n
    big = exp >= 5.0
    obs = np.append(counts[big], counts[~big].sum())
    ex = np.append(exp[big], exp[~big].sum())
    chi2 = float(((obs - ex) ** 2 / ex).sum())
    pval = float(sps.chi2.sf(chi2, obs.size - 1))
    say(f"  chi2 {chi2:.1f} on {obs.size - 1} dof, p = {pval:.3g}; draft token mass {p0[int(drafts[0, 0])]:.3f}")
    assert pval > 1e-4


def test_score_marginals_sum_to_one(tiny, dev):
    """P(k) over k = 0..K telescopes to 1 (§4.2 Eq. 6), on the GPU's own float64 products."""
    cfg = synth.CONFIGS["tiny"]
    ws = jsv.new_workspace(tiny.gpu, 8, cfg.K, 8)
    for mode in (SOFT, POINT):
        blk = synth.make_block(tiny.cpu, 8, cfg.K, cfg.sigma, 1.0, seed=4242 + mode)
        out = jsv.score_outcomes(tiny.gpu, blk.hidden.to(dev), blk.draft_tokens.to(dev),
                                 blk.draft_logits.to(dev) if mode == SOFT else None, 1.0, mode, 8, ws)
        torch.cuda.synchronize()
        s = out.len_marginal.cpu().numpy().sum(axis=1)
        say(f"  mode {mode}: |sum P(k) - 1| max {np.abs(s - 1).max():.2e}")
        assert np.all(np.abs(s - 1.0) < 1e-12)


# ---- scoring -----------------------------------------------------------------------------------
@pytest.mark.parametrize("mode", [SOFT, POINT])
@pytest.mark.parametrize("T", [1.0, 0.0])
def test_score_tiny(tiny, dev, mode, T):
    cfg = synth.CONFIGS["tiny"]
    ws = jsv.new_workspace(tiny.gpu, 4, cfg.K, 8)
    st = new_stats()
    for seed in range(10):
        say(f"tiny score mode={mode} T={T} seed={seed}")
        blk = synth.make_block(tiny.cpu, 4, cfg.K, cfg.sigma, T if T > 0 else 1.0, seed=200 + seed)
        hp = synth.predicted_hidden(blk.hidden, seed)
        got, ref = run_score(tiny, hp, blk.draft_tokens, blk.draft_logits, T, mode, 8, ws)
        compare_score(got, ref, st)
    say(f"  {st}")
    assert st["exact"] >= 30


@pytest.mark.parametrize("mode", [SOFT, POINT])
def test_score_qwen8b_k16(qwen, dev, mode):
    cfg = synth.CONFIGS["qwen8b_k16"]
    ws = jsv.new_workspace(qwen.gpu, 1, cfg.K, 8)
    st = new_stats()
    for seed in range(2):
        say(f"qwen8b score mode={mode} seed={seed}")
        blk = synth.make_block(qwen.cpu, 1, cfg.K, cfg.sigma, 1.0, seed=seed)
        hp = synth.predicted_hidden(blk.hidden, seed)
        got, ref = run_score(qwen, hp, blk.draft_tokens, blk.draft_logits, 1.0, mode, 8, ws)
        compare_score(got, ref, st)
    say(f"  {st}")
    assert st["exact"] >= 1


def test_score_k32_b4_d5120_fp8(qwen, dev):
    """Scoring at the other shapes: K = 32 with B = 4 (four row passes), d = 5120, and the
    fp8 head; top-8, T = 1, softmax proposal."""
    st = new_stats()
    cfg = synth.CONFIGS["qwen8b_k32_b4"]
    ws = jsv.new_workspace(qwen.gpu, cfg.batch, cfg.K, 8)
    blk = synth.make_block(qwen.cpu, cfg.batch, cfg.K, cfg.sigma, 1.0, seed=31)
    say("score qwen8b K=32 B=4")
    got, ref = run_score(qwen, synth.predicted_hidden(blk.hidden, 31), blk.draft_tokens,
                         blk.draft_logits, 1.0, SOFT, 8, ws)
    compare_score(got, ref, st)
    for name in ("d5120_k16_b1", "qwen8b_k16_fp8"):
        cfg = synth.CONFIGS[name]
        case = Case(synth.head_for(cfg), dev, f64_weight=True)
        ws = jsv.new_workspace(case.gpu, 1, cfg.K, 8)
        blk = synth.make_block(case.cpu, 1, cfg.K, cfg.sigma, 1.0, seed=33)
        say(f"score {name}")
        got, ref = run_score(case, synth.predicted_hidden(blk.hidden, 33), blk.draft_tokens,
                             blk.draft_logits, 1.0, SOFT, 8, ws)
        compare_score(got, ref, st)
        del case
    say(f"  {st}")
    assert st["exact"] >= 3


def test_split_d_block_in_a_workspace_sized_for_the_largest_block(dev):
    """A workspace sized for B = 8, K = 32 (264 rows: row passes) serves a B = 3, K = 32
    block, which takes the split-d LM head and needs its planes."""
    head = synth.random_head(5003, 2048, synth.BF16, seed=47)
    case = Case(head, dev)
    ws = jsv.new_workspace(case.gpu, 8, 32)
    st = new_stats()
    for T in (0.0, 1.0):
        say(f"split-d B=3 K=32 in an 8 x 32 workspace, T={T}")
        blk = synth.make_block(head, 3, 32, 0.3, T, seed=90)
        got, ref = run_verify(case, blk, T, SOFT, 5, 6, ws)
        compare_verify(got, ref, blk.draft_tokens.numpy(), st)
        compare_logits(got["logits"], ref["logits"], st)
    say(f"  {st}")
    assert st["exact"] >= 4


def test_score_split_d_ragged(dev):
    """Scoring through the split-d LM head on a ragged vocabulary (V = 5003, two blocks of
    d, 99 rows): both proposals, top-8, T = 1; the 4-byte access path of the combine."""
    head = synth.random_head(5003, 2048, synth.BF16, seed=43)
    case = Case(head, dev)
    ws = jsv.new_workspace(case.gpu, 3, 32, 8)
    st = new_stats()
    for mode in (SOFT, POINT):
        for seed in range(2):
            say(f"score split-d V=5003 d=2048 B=3 K=32 mode={mode} seed={seed}")
            blk = synth.make_block(head, 3, 32, 0.3, 1.0, seed=80 + seed)
            hp = synth.predicted_hidden(blk.hidden, seed)
            got, ref = run_score(case, hp, blk.draft_tokens, blk.draft_logits, 1.0, mode, 8, ws)
            compare_score(got, ref, st)
    say(f"  {st}")
    assert st["exact"] >= 6


def test_verify_qwen8b_k16_more_seeds(qwen, dev):
    """Eight more seeds of the benchmark block at T = 1 (softmax proposal): exact except
    at flagged near-ties."""
    cfg = synth.CONFIGS["qwen8b_k16"]
    ws = jsv.new_workspace(qwen.gpu, 1, cfg.K)
    st = new_stats()
    for seed in range(10, 18):
        blk = synth.make_block(qwen.cpu, 1, cfg.K, cfg.sigma, 1.0, seed=seed)
        got, ref = run_verify(qwen, blk, 1.0, SOFT, seed, seed, ws, with_logits=False)
        compare_verify(got, ref, blk.draft_tokens.numpy(), st)
    say(f"  {st}")
    assert st["exact"] >= 6


# ---- edge cases ---------------------------------------------------------------------------------
def test_edge_max_block_ragged_vocab(dev):
    # B = 8, K = 32: 264 rows in nine passes over a vocabulary that is not a multiple of 16
    head = synth.random_head(1009, 512, synth.BF16, seed=5)
    case = Case(head, dev)
    ws = jsv.new_workspace(case.gpu, 8, 32, 64)
    st = new_stats()
    for T in (0.0, 1.0):
        say(f"edge B=8 K=32 V=1009 T={T}")
        blk = synth.make_block(head, 8, 32, 0.3, T, seed=77)
        got, ref = run_verify(case, blk, T, SOFT, 3, 4, ws)
        compare_verify(got, ref, blk.draft_tokens.numpy(), st)
        compare_logits(got["logits"], ref["logits"], st)
        got, ref = run_score(case, blk.hidden, blk.draft_tokens, blk.draft_logits, max(T, 0.7), SOFT, 64, ws)
        compare_score(got, ref, st)
    say(f"  {st}")


def test_edge_small_vocab_and_k1(dev):
    head = synth.random_head(10, 256, synth.F32, seed=9)
    case = Case(head, dev)
    ws = jsv.new_workspace(case.gpu, 3, 1, 16)
    st = new_stats()
    for seed in range(10):
        T = 1.0 if seed % 2 else 0.0
        say(f"edge V=10 K=1 seed={seed}")
        blk = synth.make_block(head, 3, 1, 0.5, T, seed=seed)
        got, ref = run_verify(case, blk, T, SOFT, seed, 0, ws)
        compare_verify(got, ref, blk.draft_tokens.numpy(), st)
        got, ref = run_score(case, blk.hidden, blk.draft_tokens, blk.draft_logits, 1.0, POINT, 16, ws)
        compare_score(got, ref, st)   # fewer outcomes than top_n: padded
    say(f"  {st}")


def test_edge_invalid_requests(tiny, dev):
    cfg = synth.CONFIGS["tiny"]
    ws = jsv.new_workspace(tiny.gpu, 3, cfg.K, 8)
    blk = synth.make_block(tiny.cpu, 3, cfg.K, cfg.sigma, 1.0, seed=1)
    blk.hidden[0, 2, 7] = float("nan")            # request 0: non-finite logits
    blk.draft_tokens[1, 3] = tiny.cpu.vocab        # request 1: draft token out of range
    st = new_stats()
    say("edge invalid requests")
    got, ref = run_verify(tiny, blk, 1.0, SOFT, 0, 0, ws, with_logits=False)
    assert got["n_accepted"][0] == -1 and got["n_accepted"][1] == -1
    assert np.all(got["committed"][:2] == -1)
    assert got["flags"][0] & jsv.FLAG_INVALID and got["flags"][1] & jsv.FLAG_INVALID
    compare_verify(got, ref, blk.draft_tokens.numpy(), st)
    got, ref = run_score(tiny, blk.hidden, blk.draft_tokens, blk.draft_logits, 1.0, SOFT, 8, ws)
    compare_score(got, ref, st)
    assert st["exact"] >= 2


def test_stages_equal_block_and_runs_are_bit_identical(qwen, dev):
    cfg = synth.CONFIGS["qwen8b_k16"]
    ws = jsv.new_workspace(qwen.gpu, 1, cfg.K)
    blk = synth.make_block(qwen.cpu, 1, cfg.K, cfg.sigma, 1.0, seed=123)
    h, d, g = blk.hidden.to(dev), blk.draft_tokens.to(dev), blk.draft_logits.to(dev)
    say("stages vs block, bit identity")
    outs = []
    for rep in range(3):
        lo = torch.empty(1, cfg.K + 1, qwen.cpu.vocab, device=dev)
        o = jsv.verify_block(qwen.gpu, h, d, g, 1.0, SOFT, 9, rep % 2, ws, logits_out=lo)
        outs.append((o, lo))
    o2 = jsv.verify_stats(qwen.gpu, h, d, g, 1.0, SOFT, 9, 0, ws)
    jsv.verify_sample(qwen.gpu, h, d, g, 1.0, SOFT, 9, 0, ws, out=o2)
    torch.cuda.synchronize()
    assert torch.equal(outs[0][1], outs[1][1]) and torch.equal(outs[0][1], outs[2][1])
    assert torch.equal(outs[0][0].committed, outs[2][0].committed)
    assert torch.equal(outs[0][0].committed, o2.committed)
    assert torch.equal(outs[0][0].n_accepted, o2.n_accepted)
    assert torch.equal(outs[0][0].flags, o2.flags)


# ---- next rows: anchor replacement, cache lookup, calibrated lengths ---------------------------
def _compare_anchor(out, pos, tok, fl, st):
    gp, gt, gf = (out.position.cpu().numpy(), out.token.cpu().numpy(), out.flags.cpu().numpy())
    for b in range(pos.shape[0]):
        st["requests"] += 1
        assert (int(gf[b]) & oracle.FLAG_INVALID) == (int(fl[b]) & oracle.FLAG_INVALID)
        if (int(gf[b]) | int(fl[b])) & oracle.FLAG_LOGIT_GAP:
            st["near_ties"] += 1
            continue
        assert (int(gp[b]), int(gt[b])) == (int(pos[b]), int(tok[b])), (b, gp[b], gt[b], pos[b], tok[b])
        st["exact"] += 1


def test_anchor_replace_tiny_and_qwen(tiny, qwen, dev):
    st = new_stats()
    cfg = synth.CONFIGS["tiny"]
    ws = jsv.new_workspace(tiny.gpu, 8, cfg.K)
    for seed in range(40):
        blk = synth.make_block(tiny.cpu, 8, cfg.K, cfg.sigma, 0.0, seed=900 + seed)
        hp = synth.predicted_hidden(blk.hidden, seed=seed)
        out = jsv.anchor_replace(tiny.gpu, hp.to(dev), blk.draft_tokens.to(dev), ws)
        torch.cuda.synchronize()
        _compare_anchor(out, *oracle.anchor_replace(tiny.oh, hp, blk.draft_tokens.numpy()), st)
    for name in ("qwen8b_k16", "qwen8b_k32_b4"):
        cfg = synth.CONFIGS[name]
        ws = jsv.new_workspace(qwen.gpu, cfg.batch, cfg.K)
        blk = synth.make_block(qwen.cpu, cfg.batch, cfg.K, cfg.sigma, 0.0, seed=77)
        hp = synth.predicted_hidden(blk.hidden, seed=77)
        say(f"anchor replacement {name}")
        out = jsv.anchor_replace(qwen.gpu, hp.to(dev), blk.draft_tokens.to(dev), ws)
        torch.cuda.synchronize()
        _compare_anchor(out, *oracle.anchor_replace(qwen.oh, hp, blk.draft_tokens.numpy()), st)
    say(f"  {st}")
    assert st["exact"] >= 0.9 * st["requests"]


def test_anchor_replace_invalid_draft(tiny, dev):
    cfg = synth.CONFIGS["tiny"]
    ws = jsv.new_workspace(tiny.gpu, 2, cfg.K)
    blk = synth.make_block(tiny.cpu, 2, cfg.K, cfg.sigma, 0.0, seed=5)
    d = blk.draft_tokens.clone()
    d[1, 2] = cfg.vocab + 3
    out = jsv.anchor_replace(tiny.gpu, blk.hidden.to(dev), d.to(dev), ws)
    torch.cuda.synchronize()
    pos, tok, fl = oracle.anchor_replace(tiny.oh, blk.hidden, d.numpy())
    assert int(out.position[1]) == -1 and int(out.token[1]) == -1 and int(out.flags[1]) & jsv.FLAG_INVALID
    assert int(out.position[0]) == int(pos[0]) or (int(fl[0]) | int(out.flags[0])) & jsv.FLAG_LOGIT_GAP


def test_cache_lookup_matches_oracle(tiny, dev):
    cfg = synth.CONFIGS["tiny"]
    B, K, N = 8, cfg.K, 16
    ws = jsv.new_workspace(tiny.gpu, B, K, N)
    hits = 0
    for seed in range(10):
        blk = synth.make_block(tiny.cpu, B, K, cfg.sigma, 1.0, seed=1300 + seed)
        hp = synth.predicted_hidden(blk.hidden, seed=seed)
        dl = blk.draft_logits.to(dev)
        sc = jsv.score_outcomes(tiny.gpu, hp.to(dev), blk.draft_tokens.to(dev), dl, 1.0, SOFT, N, ws)
        vo = jsv.verify_block(tiny.gpu, blk.hidden.to(dev), blk.draft_tokens.to(dev), dl, 1.0, SOFT, seed, 0, ws)
        hit = jsv.cache_lookup(vo.n_accepted, vo.committed, sc.out_len, sc.out_token)
        torch.cuda.synchronize()
        ref = oracle.cache_lookup(vo.n_accepted.cpu().numpy(), vo.committed.cpu().numpy(),
                                  sc.out_len.cpu().numpy(), sc.out_token.cpu().numpy())
        assert np.array_equal(hit.cpu().numpy(), ref)
        hits += int((ref >= 0).sum())
    say(f"  cache hits {hits} of {10 * B} rounds (top {N} of predicted states)")


def test_calibrated_lengths_bit_exact(dev):
    rng = np.random.default_rng(11)
    for B, K in ((1, 1), (16, 16), (7, 32)):
        p = rng.uniform(0.0, 1.0, size=(B, K))
        if B > 2:
            p[1, K // 2] = 1.5
            p[2, 0] = np.nan
        out, fl = jsv.calibrated_lengths(torch.tensor(p, dtype=torch.float64, device=dev))
        torch.cuda.synchronize()
        ref, rf = oracle.calibrated_lengths(p)
        assert np.array_equal(out.cpu().numpy(), ref), (B, K)
        assert np.array_equal(fl.cpu().numpy(), rf)
