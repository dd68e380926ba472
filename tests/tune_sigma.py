"""Bisect the draft-perturbation sigma so that mean committed tokens per block hit a target.

Run by hand (`python tests/tune_sigma.py`); it prints the values stored in synth/.
At T = 0 a block commits the argmax-matching prefix plus one bonus token, so with
independent rows whose argmax agreement rate is a, E[committed] = sum_{k=0..K} a^k.
The target argmax comes from the oracle's own RMSNorm + LM head (float64); the draft
argmax from synth's draft-logit recipe.
"""
from __future__ import annotations

import sys
from pathlib import Path

import numpy as np
import torch

sys.path.insert(0, str(Path(__file__).resolve().parents[1]))
import oracle  # noqa: E402
import synth  # noqa: E402


def expected_committed(a, K):
    return sum(a ** k for k in range(K + 1))


class Agreement:
    def __init__(self, head, rows=512, seed=12345):
        g = torch.Generator().manual_seed(seed)
        self.head = head
        self.h = torch.randn(rows, head.hidden, generator=g).to(head.weight.dtype)
        self.noise = torch.randn(rows, head.hidden, generator=g)
        oh = oracle.Head(head.weight, head.norm_weight, head.eps, head.dtype)
        self.target = np.argmax(oracle.block_logits(oh, self.h), axis=1)

    def __call__(self, sigma):
        G = synth.draft_logits_for(self.head, self.h.float() + sigma * self.noise)
        return float(np.mean(self.target == torch.argmax(G, dim=1).numpy()))


def tune(agree, K, target, lo=0.0, hi=0.2, iters=9):
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if expected_committed(agree(mid), K) > target:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


if __name__ == "__main__":
    for d, seed in ((4096, 1002), (5120, 1005)):
        head = synth.make_head(151936, d, synth.BF16, 0.02, seed)
        agree = Agreement(head)
        for K, target in ((16, 8.0), (32, 14.0)):
            s = tune(agree, K, target)
            a = agree(s)
            print(f"d={d} K={K} target={target}: sigma={s:.4f} agreement={a:.4f} "
                  f"E[committed]={expected_committed(a, K):.2f}", flush=True)
