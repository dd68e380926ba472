"""MI355X-native draft-block verification: final RMSNorm + LM head, lossless
rejection sampling of a draft block, and foresight outcome scoring.

The work happens in libjsverify.so (HIP kernels for gfx950, C ABI in
include/jsverify.h); `jsverify` is its thin ctypes binding.
"""
from .jsverify import (FLAG_ACCEPT_TIE, FLAG_CDF_TIE, FLAG_INVALID, FLAG_LOGIT_GAP,  # noqa: F401
                       FLAG_TOPN_TIE, FLAG_ZERO_RESIDUAL, PROPOSAL_POINT, PROPOSAL_SOFTMAX, AnchorOut,
                       LMHead, ScoreOut, VerifyOut, anchor_replace, cache_lookup, calibrated_lengths,
                       geometric_fanout, lmhead_logits, load_library, new_workspace, score_outcomes,
                       verify_block, verify_sample, verify_stats, workspace_bytes)
