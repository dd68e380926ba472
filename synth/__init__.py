"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module draws inputs only.  It holds none of the verification arithmetic: the
draft logits that stand in for a draft model are produced with torch's own
`rms_norm` and `matmul` from perturbed hidden states, as the workload recipe says.

Workload recipe (shapes of the Qwen3-8B / 14B LM heads on which the method's
verification budgets 16 and 32 are reported):
  W      ~ N(0, w_std^2), stored in the weight dtype, [V, d] row-major
  gamma  = 1 + N(0, 0.01^2), stored in the weight dtype, [d]
  h      ~ N(0, 1) in the weight dtype, [B, K+1, d]
  G_i    = W . rms_norm(h_i + eps_i) in float32, eps_i ~ N(0, sigma^2), i < K
  d_i    = argmax G_i at T = 0, else drawn from softmax(G_i / T)
  h_pred = h + N(0, 0.3^2)   (stand-in for adapter-predicted states, scoring only)
W and gamma come from seed 1000 + config id; everything else from the run seed.
An fp8 config quantises that bf16 W per vocabulary row: scale = max|W_v| / 448 (the
largest E4M3 value), codes = E4M3(W_v / scale) rounded to nearest even; gamma and the
hidden states stay bf16.  The quantised head is the target the verification runs on.
"""
from __future__ import annotations

from dataclasses import dataclass
from functools import lru_cache

import torch

BF16 = "bf16"
F32 = "f32"
FP8 = "fp8"
_TORCH_DTYPE = {BF16: torch.bfloat16, F32: torch.float32}
_ACT_DTYPE = {BF16: torch.bfloat16, F32: torch.float32, FP8: torch.bfloat16}

# sigma of the draft perturbation, bisected at T = 0 so that the mean number of
# committed tokens per block (accepted drafts + 1 bonus) is about 8 at K = 16 and
# about 14 at K = 32 (tests/tune_sigma.py prints these values).
SIGMA_K16_D4096 = 0.0432
SIGMA_K32_D4096 = 0.0248
SIGMA_K16_D5120 = 0.0494
SIGMA_K32_D5120 = 0.0311
SIGMA_TINY = 0.5


@dataclass(frozen=True)
class Config:
    name: str
    vocab: int
    hidden: int
    K: int
    batch: int
    dtype: str
    w_std: float
    sigma: float
    head_seed: int
    eps: float = 1e-6


CONFIGS = {
    "tiny": Config("tiny d=256 V=1024 K=4 B=1 f32", 1024, 256, 4, 1, F32, 0.05, SIGMA_TINY, 1001),
    "qwen8b_k16": Config("Qwen3-8B LM head d=4096 V=151936 K=16 B=1 bf16", 151936, 4096, 16, 1, BF16,
                         0.02, SIGMA_K16_D4096, 1002),
    "qwen8b_k32_b4": Config("Qwen3-8B LM head d=4096 V=151936 K=32 B=4 bf16", 151936, 4096, 32, 4, BF16,
                            0.02, SIGMA_K32_D4096, 1002),
    "d5120_k16_b1": Config("d=5120 V=151936 K=16 B=1 bf16", 151936, 5120, 16, 1, BF16, 0.02,
                           SIGMA_K16_D5120, 1005),
    "d5120_k32_b2": Config("d=5120 V=151936 K=32 B=2 bf16", 151936, 5120, 32, 2, BF16, 0.02,
                           SIGMA_K32_D5120, 1005),
    "qwen8b_k16_fp8": Config("Qwen3-8B LM head d=4096 V=151936 K=16 B=1 fp8 (E4M3 W, bf16 x)", 151936,
                             4096, 16, 1, FP8, 0.02, SIGMA_K16_D4096, 1002),
}


@dataclass
class HeadData:
    weight: torch.Tensor        # [V, d] CPU, weight dtype (float8_e4m3fn codes for fp8)
    norm_weight: torch.Tensor   # [d]    CPU, activation dtype
    eps: float
    dtype: str
    weight_scale: torch.Tensor | None = None   # [V] float32 row scales of an fp8 head

    def dequantized(self, v0=0, v1=None):
        """Rows [v0, v1) of W as float32 values (codes times row scales for fp8)."""
        w = self.weight[v0:v1].float()
        if self.weight_scale is not None:
            w = w * self.weight_scale[v0:v1, None]
        return w

    @property
    def vocab(self):
        return int(self.weight.shape[0])

    @property
    def hidden(self):
        return int(self.weight.shape[1])


@dataclass
class BlockData:
    hidden: torch.Tensor         # [B, K+1, d] weight dtype
    draft_tokens: torch.Tensor   # [B, K] int32
    draft_logits: torch.Tensor   # [B, K, V] float32


def _gen(seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _normal_rows(seed, rows, cols, std, dtype, step=4096):
    """[rows, cols] N(0, std^2) in `dtype`; chunk c of `step` rows uses its own generator
    (seed, c), so the result does not depend on how many threads draw it."""
    from concurrent.futures import ThreadPoolExecutor
    out = torch.empty(rows, cols, dtype=dtype)

    def fill(c):
        v0 = c * step
        n = min(step, rows - v0)
        g = _gen(seed * 1_000_003 + c)
        out[v0:v0 + n] = (torch.randn(n, cols, generator=g) * std).to(dtype)

    nchunks = (rows + step - 1) // step
    with ThreadPoolExecutor(max_workers=max(1, min(16, torch.get_num_threads()))) as ex:
        list(ex.map(fill, range(nchunks)))
    return out


@lru_cache(maxsize=2)
def make_head(vocab, hidden, dtype, w_std, seed, eps=1e-6):
    """LM head weight and RMSNorm weight, drawn once per (shape, seed)."""
    td = _TORCH_DTYPE[dtype]
    w = _normal_rows(seed, vocab, hidden, w_std, td)
    g = _gen(seed)
    gamma = (1.0 + 0.01 * torch.randn(hidden, generator=g)).to(td)
    return HeadData(w, gamma, float(eps), dtype)


def quantize_fp8(head: HeadData) -> HeadData:
    """Per-row E4M3 quantisation of a bf16 head (the fp8 workload recipe above)."""
    w = head.weight.float()
    amax = w.abs().amax(dim=1)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax)).float()
    codes = (w / scale[:, None]).to(torch.float8_e4m3fn)
    return HeadData(codes, head.norm_weight.to(torch.bfloat16), head.eps, FP8, scale)


@lru_cache(maxsize=2)
def _fp8_head(vocab, hidden, w_std, seed, eps):
    return quantize_fp8(make_head(vocab, hidden, BF16, w_std, seed, eps))


def head_for(cfg: Config):
    if cfg.dtype == FP8:
        return _fp8_head(cfg.vocab, cfg.hidden, cfg.w_std, cfg.head_seed, cfg.eps)
    return make_head(cfg.vocab, cfg.hidden, cfg.dtype, cfg.w_std, cfg.head_seed, cfg.eps)


def draft_logits_for(head: HeadData, hidden_rows, chunk=16384):
    """G = W . rms_norm(x) in float32 for rows x [R, d], with torch's own ops."""
    x = torch.nn.functional.rms_norm(hidden_rows.float(), (head.hidden,),
                                     head.norm_weight.float(), head.eps)
    out = torch.empty(x.shape[0], head.vocab, dtype=torch.float32)
    for v0 in range(0, head.vocab, chunk):
        wc = head.dequantized(v0, v0 + chunk)
        out[:, v0:v0 + wc.shape[0]] = x @ wc.T
    return out


def make_block(head: HeadData, batch, K, sigma, T, seed, hidden_std=1.0):
    """One verification block per request: target states, drafts and draft logits."""
    g = _gen(seed)
    td = _ACT_DTYPE[head.dtype]
    d, V = head.hidden, head.vocab
    h = (torch.randn(batch, K + 1, d, generator=g) * hidden_std).to(td)
    noise = torch.randn(batch, K, d, generator=g) * sigma
    G = draft_logits_for(head, (h[:, :K].float() + noise).reshape(batch * K, d)).reshape(batch, K, V)
    if T == 0:
        drafts = torch.argmax(G, dim=-1)
    else:
        pr = torch.softmax(G.double() / T, dim=-1).reshape(batch * K, V)
        drafts = torch.multinomial(pr, 1, generator=g).reshape(batch, K)
    return BlockData(h, drafts.to(torch.int32).contiguous(), G.contiguous())


def predicted_hidden(hidden, seed, std=0.3):
    """Stand-in for adapter-predicted states: h + N(0, std^2), in the same dtype."""
    g = _gen(seed + 7919)
    return (hidden.float() + std * torch.randn(hidden.shape, generator=g)).to(hidden.dtype)


def random_head(vocab, hidden, dtype, seed, w_std=0.05, eps=1e-6):
    """Small uncached head for tests (same recipe as make_head; fp8 quantises it)."""
    if dtype == FP8:
        return quantize_fp8(make_head.__wrapped__(vocab, hidden, BF16, w_std, seed, eps))
    return make_head.__wrapped__(vocab, hidden, dtype, w_std, seed, eps)
