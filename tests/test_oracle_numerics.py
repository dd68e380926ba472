"""Pins of the oracle's RMSNorm, LM head and softmax against closed forms and
library routines (CPU only)."""
import numpy as np
import pytest
import torch

import oracle


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100_000).astype(np.float32) * s for s in (1e-3, 1, 1e4)])
    specials = np.array([0.0, -0.0, 1.0, 1.00390625, 1.005859375, 3.3895314e38, 1e-40, -2.5], np.float32)
    x = np.concatenate([x, specials])
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    got = oracle.bf16_round(x)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_rmsnorm_constant_row_closed_form():
    # a row c*1 has mean square c^2, so RMSNorm gives gamma * c / sqrt(c^2 + eps)
    d, eps = 64, 1e-6
    gamma = np.linspace(0.5, 1.5, d).astype(np.float32)
    for c in (0.25, 1.0, 3.0, -2.0):
        h = np.full((1, d), c, np.float32)
        got = oracle.rmsnorm(h, gamma, eps, "f32")[0]
        want = gamma.astype(np.float64) * c / np.sqrt(c * c + eps)
        assert np.allclose(got, want, rtol=3e-7, atol=0)
        got16 = oracle.rmsnorm(h, gamma, eps, "bf16")[0]
        assert np.allclose(got16, want, rtol=2 ** -8, atol=0)


def test_rmsnorm_matches_torch_library():
    g = torch.Generator().manual_seed(3)
    h = torch.randn(7, 256, generator=g)
    gamma = 1 + 0.1 * torch.randn(256, generator=g)
    ref = torch.nn.functional.rms_norm(h.double(), (256,), gamma.double(), 1e-6).numpy()
    got = oracle.rmsnorm(h, gamma, 1e-6, "f32")
    assert np.allclose(got, ref, rtol=5e-7, atol=1e-7)
    # the bf16 variant is the f32 value rounded once to bf16
    got16 = oracle.rmsnorm(h.bfloat16(), gamma.bfloat16(), 1e-6, "bf16")
    f32 = oracle.rmsnorm(h.bfloat16(), gamma.bfloat16(), 1e-6, "f32")
    assert np.array_equal(got16, oracle.bf16_round(f32.astype(np.float32)).astype(np.float64))


def test_rmsnorm_gamma_and_eps_matter():
    h = np.full((1, 8), 1e-3, np.float32)
    a = oracle.rmsnorm(h, np.ones(8, np.float32), 1e-6, "f32")
    b = oracle.rmsnorm(h, np.ones(8, np.float32), 1e-2, "f32")
    assert a[0, 0] > 0.7 and b[0, 0] < 0.02          # eps inside the square root
    c = oracle.rmsnorm(h, 2 * np.ones(8, np.float32), 1e-6, "f32")
    assert np.allclose(c, 2 * a)


def test_lm_head_matches_torch_matmul():
    g = torch.Generator().manual_seed(5)
    W = torch.randn(1000, 96, generator=g).bfloat16()
    x = torch.randn(5, 96, generator=g).double()
    got = oracle.lm_head_logits(x.numpy(), W, chunk=64)
    ref = (x @ W.double().T).numpy()
    assert np.allclose(got, ref, rtol=0, atol=1e-12)
    # the contraction runs over d, not V: a transposed operand would not even conform
    assert got.shape == (5, 1000)
    # row v of W produces column v of the logits
    got1 = oracle.lm_head_logits(np.eye(96)[:1], W)
    assert np.allclose(got1[0], W.double()[:, 0].numpy())


def test_softmax_hand_built():
    p = np.array([0.8, 0.15, 0.05])
    assert np.allclose(oracle.probs(np.log(p), 1.0), p, rtol=1e-14)
    # temperature 1/2 squares the probabilities before renormalising
    assert np.allclose(oracle.probs(np.log(p), 0.5), p ** 2 / np.sum(p ** 2), rtol=1e-14)
    # shift invariance
    assert np.allclose(oracle.probs(np.log(p) + 1000.0, 1.0), p, rtol=1e-14)


def test_temperature_zero_is_argmax_lowest_id_on_ties():
    z = np.array([0.1, 2.0, -1.0, 2.0])
    assert np.array_equal(oracle.probs(z, 0), [0, 1, 0, 0])
    assert oracle.top2_gap(z) == 0.0
    assert oracle.top2_gap(np.array([1.0, 3.0, 2.5])) == pytest.approx(0.5)


def test_block_logits_pipeline_shapes():
    head = oracle.Head(torch.randn(50, 32).bfloat16(), torch.ones(32).bfloat16(), 1e-6, "bf16")
    h = torch.randn(2, 3, 32).bfloat16()
    z = oracle.block_logits(head, h)
    assert z.shape == (2, 3, 50)
    x = oracle.rmsnorm(h.reshape(6, 32), head.norm_weight, 1e-6, "bf16")
    assert np.allclose(z.reshape(6, 50), x @ head.weight.double().numpy().T)


def test_e4m3_decode_matches_format_definition():
    """OCP FP8 E4M3 (the fp8 head's codes): sign, 4 exponent bits with bias 7, 3 mantissa
    bits; exponent 0 is subnormal (m * 2^-9); S.1111.111 is NaN and there are no
    infinities.  The oracle decodes codes through torch; this pins that decoding to the
    definition written out here, for all 256 codes."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    got = oracle.reference._as_f64(codes.view(torch.float8_e4m3fn))
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            assert np.isnan(got[c]), c
            continue
        val = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
        assert got[c] == (-val if s else val), (c, got[c], val)


def test_fp8_head_logits_closed_form():
    """z = scale_v * (x . e4m3(code_v)) with x rounded to bf16: the same as the float64
    product of x with the dequantised rows."""
    rng = np.random.default_rng(5)
    V, d = 64, 32
    codes = torch.tensor(rng.normal(0, 30, size=(V, d)), dtype=torch.float32).to(torch.float8_e4m3fn)
    scale = torch.tensor(rng.uniform(1e-4, 1e-3, size=V), dtype=torch.float32)
    gamma = torch.tensor(1 + 0.01 * rng.normal(size=d), dtype=torch.float32).to(torch.bfloat16)
    h = torch.tensor(rng.normal(size=(3, d)), dtype=torch.float32).to(torch.bfloat16)
    head = oracle.Head(codes, gamma, 1e-6, "fp8", weight_scale=scale)
    z = oracle.block_logits(head, h)
    x = oracle.rmsnorm(h, gamma, 1e-6, "bf16")
    wdq = codes.to(torch.float32).double().numpy() * scale.double().numpy()[:, None]
    assert np.allclose(z, x @ wdq.T, rtol=1e-13, atol=1e-15)
    assert np.all(oracle.bf16_round(x.astype(np.float32)) == x)  # x sits on the bf16 grid
