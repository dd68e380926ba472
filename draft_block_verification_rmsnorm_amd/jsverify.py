"""Thin Python binding of libjsverify (include/jsverify.h) over ctypes.

Argument marshalling only: every step of verification and scoring runs in the HIP
kernels of the library.  Tensors are torch tensors on the GPU; the binding passes
their device pointers and the current HIP stream.  The functions keep the C names
without the `jsv_` prefix.  Shape, dtype and device errors raise ValueError;
non-OK statuses from the library raise RuntimeError.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

import torch

LIB_PATH = Path(__file__).resolve().parent / "libjsverify.so"

JSV_OK, JSV_EINVAL, JSV_EUNSUPPORTED, JSV_EWORKSPACE, JSV_EHIP = 0, -1, -2, -3, -4
JSV_BF16, JSV_F32, JSV_FP8 = 0, 1, 2
PROPOSAL_SOFTMAX, PROPOSAL_POINT = 0, 1

FLAG_ACCEPT_TIE = 1 << 0
FLAG_LOGIT_GAP = 1 << 1
FLAG_CDF_TIE = 1 << 2
FLAG_INVALID = 1 << 3
FLAG_ZERO_RESIDUAL = 1 << 4
FLAG_TOPN_TIE = 1 << 5

EXPORTED = ("jsv_workspace_bytes", "jsv_lmhead_logits", "jsv_verify_block", "jsv_verify_stats",
            "jsv_verify_sample", "jsv_score_outcomes", "jsv_anchor_replace", "jsv_cache_lookup",
            "jsv_calibrated_lengths", "jsv_geometric_fanout", "jsv_status_string", "jsv_version")

_DTYPES = {torch.bfloat16: JSV_BF16, torch.float32: JSV_F32, torch.float8_e4m3fn: JSV_FP8}


class _Head(ctypes.Structure):
    _fields_ = [("weight", ctypes.c_void_p), ("norm_weight", ctypes.c_void_p),
                ("vocab", ctypes.c_int64), ("hidden", ctypes.c_int64),
                ("eps", ctypes.c_float), ("dtype", ctypes.c_int32), ("weight_scale", ctypes.c_void_p)]


_lib = None


def load_library(path: Path | str | None = None) -> ctypes.CDLL:
    """Load libjsverify.so and declare its signatures.  Raises if it is not built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = Path(path) if path is not None else LIB_PATH
    if not p.exists():
        raise RuntimeError(f"{p} is not built: run `python -m draft_block_verification_rmsnorm_amd.build` "
                           "(the HIP library is required; there is no fallback)")
    lib = ctypes.CDLL(str(p))
    vp, i32, i64, u64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                  ctypes.c_uint64, ctypes.c_float, ctypes.c_size_t)
    hp = ctypes.POINTER(_Head)
    lib.jsv_workspace_bytes.argtypes = [hp, i32, i32, i32]
    lib.jsv_workspace_bytes.restype = sz
    lib.jsv_lmhead_logits.argtypes = [hp, vp, i64, vp, vp, sz, vp]
    lib.jsv_lmhead_logits.restype = i32
    verify_args = [hp, vp, vp, vp, i32, i32, f32, i32, u64, u64, vp, vp, vp, vp, vp, sz, vp]
    lib.jsv_verify_block.argtypes = verify_args
    lib.jsv_verify_block.restype = i32
    lib.jsv_verify_stats.argtypes = verify_args
    lib.jsv_verify_stats.restype = i32
    lib.jsv_verify_sample.argtypes = verify_args
    lib.jsv_verify_sample.restype = i32
    lib.jsv_score_outcomes.argtypes = [hp, vp, vp, vp, i32, i32, f32, i32, i32, vp, vp, vp, vp, vp,
                                       vp, sz, vp]
    lib.jsv_score_outcomes.restype = i32
    lib.jsv_anchor_replace.argtypes = [hp, vp, vp, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.jsv_anchor_replace.restype = i32
    lib.jsv_cache_lookup.argtypes = [vp, vp, i32, i32, vp, vp, i32, vp, vp]
    lib.jsv_cache_lookup.restype = i32
    lib.jsv_calibrated_lengths.argtypes = [vp, i32, i32, vp, vp, vp]
    lib.jsv_calibrated_lengths.restype = i32
    f64 = ctypes.c_double
    lib.jsv_geometric_fanout.argtypes = [f64, f64, i32, i32, ctypes.POINTER(f64), ctypes.POINTER(i32),
                                         ctypes.POINTER(f64)]
    lib.jsv_geometric_fanout.restype = i32
    lib.jsv_status_string.argtypes = [i32]
    lib.jsv_status_string.restype = ctypes.c_char_p
    lib.jsv_version.argtypes = []
    lib.jsv_version.restype = i32
    if path is None:
        _lib = lib
    return lib


def _check(status: int):
    if status != JSV_OK:
        msg = load_library().jsv_status_string(status).decode()
        raise RuntimeError(f"libjsverify: {msg} (status {status})")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, name, dtype, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


class LMHead:
    """The target's final RMSNorm weight and LM-head weight, on one GPU.

    An fp8 head (weight in torch.float8_e4m3fn) takes `weight_scale`, one float32 scale
    per vocabulary row, and a bfloat16 norm_weight; its hidden states are bfloat16."""

    def __init__(self, weight: torch.Tensor, norm_weight: torch.Tensor, eps: float = 1e-6,
                 weight_scale: torch.Tensor | None = None):
        if weight.dtype not in _DTYPES:
            raise ValueError("weight must be bfloat16, float32 or float8_e4m3fn")
        _need(weight, "weight", weight.dtype)
        fp8 = weight.dtype == torch.float8_e4m3fn
        self.act_dtype = torch.bfloat16 if fp8 else weight.dtype
        _need(norm_weight, "norm_weight", self.act_dtype, (weight.shape[1],), weight.device)
        if fp8:
            _need(weight_scale, "weight_scale", torch.float32, (weight.shape[0],), weight.device)
        self.weight, self.norm_weight, self.eps = weight, norm_weight, float(eps)
        self.weight_scale = weight_scale if fp8 else None
        self.dtype = weight.dtype
        self.vocab, self.hidden = int(weight.shape[0]), int(weight.shape[1])
        self._c = _Head(weight.data_ptr(), norm_weight.data_ptr(), self.vocab, self.hidden,
                        self.eps, _DTYPES[weight.dtype],
                        weight_scale.data_ptr() if fp8 else None)

    @property
    def device(self):
        return self.weight.device


def workspace_bytes(head: LMHead, batch: int, K: int, top_n: int = 0) -> int:
    n = load_library().jsv_workspace_bytes(ctypes.byref(head._c), batch, K, top_n)
    if n == 0:
        raise ValueError("unsupported head or block shape")
    return int(n)


def new_workspace(head: LMHead, batch: int, K: int, top_n: int = 0) -> torch.Tensor:
    """A device workspace big enough for (batch, K, top_n)."""
    return torch.empty(workspace_bytes(head, batch, K, top_n), dtype=torch.uint8, device=head.device)


def lmhead_logits(head: LMHead, hidden: torch.Tensor, out: torch.Tensor | None = None, stream=None):
    """RMSNorm + LM head of hidden [rows, d] -> fp32 logits [rows, V]."""
    _need(hidden, "hidden", head.act_dtype, device=head.device)
    if hidden.dim() != 2 or hidden.shape[1] != head.hidden:
        raise ValueError("hidden must be [rows, hidden]")
    rows = hidden.shape[0]
    if out is None:
        out = torch.empty(rows, head.vocab, dtype=torch.float32, device=head.device)
    _need(out, "out", torch.float32, (rows, head.vocab), head.device)
    _check(load_library().jsv_lmhead_logits(ctypes.byref(head._c), _ptr(hidden), rows, _ptr(out),
                                            None, 0, _stream(stream)))
    return out


def _block_checks(head, hidden, draft_tokens, draft_logits, mode, temperature):
    if hidden is not None:
        _need(hidden, "hidden", head.act_dtype, device=head.device)
        if hidden.dim() != 3 or hidden.shape[2] != head.hidden:
            raise ValueError("hidden must be [B, K+1, hidden]")
        B, K = hidden.shape[0], hidden.shape[1] - 1
        _need(draft_tokens, "draft_tokens", torch.int32, (B, K), head.device)
    else:
        _need(draft_tokens, "draft_tokens", torch.int32, device=head.device)
        B, K = draft_tokens.shape
    if mode == PROPOSAL_SOFTMAX and temperature > 0:
        if draft_logits is None:
            raise ValueError("the softmax proposal needs draft_logits")
    if draft_logits is not None:
        _need(draft_logits, "draft_logits", torch.float32, (B, K, head.vocab), head.device)
    return B, K


class VerifyOut:
    def __init__(self, B, K, device):
        self.n_accepted = torch.empty(B, dtype=torch.int32, device=device)
        self.committed = torch.empty(B, K + 1, dtype=torch.int32, device=device)
        self.flags = torch.empty(B, dtype=torch.int32, device=device)


def _verify_call(fn, head, hidden, draft_tokens, draft_logits, temperature, mode, seed, offset,
                 workspace, out, logits_out, stream):
    B, K = _block_checks(head, hidden, draft_tokens, draft_logits, mode, temperature)
    _need(workspace, "workspace", torch.uint8, device=head.device)
    if logits_out is not None:
        _need(logits_out, "logits_out", torch.float32, (B, K + 1, head.vocab), head.device)
    if out is None:
        out = VerifyOut(B, K, head.device)
    _check(fn(ctypes.byref(head._c), _ptr(hidden), _ptr(draft_tokens), _ptr(draft_logits), B, K,
              float(temperature), int(mode), int(seed) & (2 ** 64 - 1), int(offset) & (2 ** 64 - 1),
              _ptr(out.n_accepted), _ptr(out.committed), _ptr(out.flags), _ptr(logits_out),
              _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def verify_block(head, hidden, draft_tokens, draft_logits, temperature, mode, seed, offset,
                 workspace, out=None, logits_out=None, stream=None) -> VerifyOut:
    """jsv_verify_block: accept/reject the drafts of every request and draw the bonus."""
    return _verify_call(load_library().jsv_verify_block, head, hidden, draft_tokens, draft_logits,
                        temperature, mode, seed, offset, workspace, out, logits_out, stream)


def verify_stats(head, hidden, draft_tokens, draft_logits, temperature, mode, seed, offset,
                 workspace, out=None, logits_out=None, stream=None) -> VerifyOut:
    """jsv_verify_stats: first half of verify_block (RMSNorm, LM head, statistics)."""
    return _verify_call(load_library().jsv_verify_stats, head, hidden, draft_tokens, draft_logits,
                        temperature, mode, seed, offset, workspace, out, logits_out, stream)


def verify_sample(head, hidden, draft_tokens, draft_logits, temperature, mode, seed, offset,
                  workspace, out=None, logits_out=None, stream=None) -> VerifyOut:
    """jsv_verify_sample: second half of verify_block (acceptance scan, bonus token)."""
    return _verify_call(load_library().jsv_verify_sample, head, hidden, draft_tokens, draft_logits,
                        temperature, mode, seed, offset, workspace, out, logits_out, stream)


class ScoreOut:
    def __init__(self, B, K, top_n, device):
        self.out_len = torch.empty(B, top_n, dtype=torch.int32, device=device)
        self.out_token = torch.empty(B, top_n, dtype=torch.int32, device=device)
        self.out_prob = torch.empty(B, top_n, dtype=torch.float32, device=device)
        self.len_marginal = torch.empty(B, K + 1, dtype=torch.float64, device=device)
        self.flags = torch.empty(B, dtype=torch.int32, device=device)


def score_outcomes(head, hidden_pred, draft_tokens, draft_logits, temperature, mode, top_n,
                   workspace, out=None, stream=None) -> ScoreOut:
    """jsv_score_outcomes: outcome law of the block and its top_n outcomes."""
    B, K = _block_checks(head, hidden_pred, draft_tokens, draft_logits, mode, temperature)
    _need(workspace, "workspace", torch.uint8, device=head.device)
    if out is None:
        out = ScoreOut(B, K, top_n, head.device)
    _check(load_library().jsv_score_outcomes(
        ctypes.byref(head._c), _ptr(hidden_pred), _ptr(draft_tokens), _ptr(draft_logits), B, K,
        float(temperature), int(mode), int(top_n), _ptr(out.out_len), _ptr(out.out_token),
        _ptr(out.out_prob), _ptr(out.len_marginal), _ptr(out.flags), _ptr(workspace),
        workspace.numel(), _stream(stream)))
    return out


class AnchorOut:
    def __init__(self, B, device):
        self.position = torch.empty(B, dtype=torch.int32, device=device)
        self.token = torch.empty(B, dtype=torch.int32, device=device)
        self.flags = torch.empty(B, dtype=torch.int32, device=device)


def anchor_replace(head, hidden_pred, draft_tokens, workspace, out=None, stream=None) -> AnchorOut:
    """jsv_anchor_replace: first position whose decoder argmax differs from the draft, and
    that token (K and the argmax of row K when every draft matches)."""
    B, K = _block_checks(head, hidden_pred, draft_tokens, None, PROPOSAL_POINT, 0.0)
    _need(workspace, "workspace", torch.uint8, device=head.device)
    if out is None:
        out = AnchorOut(B, head.device)
    _check(load_library().jsv_anchor_replace(
        ctypes.byref(head._c), _ptr(hidden_pred), _ptr(draft_tokens), B, K, _ptr(out.position),
        _ptr(out.token), _ptr(out.flags), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def cache_lookup(n_accepted, committed, out_len, out_token, hit_index=None, stream=None):
    """jsv_cache_lookup: index of the realised (k, a) in the cached top-N list, or -1."""
    dev = n_accepted.device
    B = n_accepted.shape[0]
    _need(n_accepted, "n_accepted", torch.int32, (B,), dev)
    if committed.dim() != 2 or committed.shape[0] != B:
        raise ValueError("committed must be [B, K+1]")
    K = committed.shape[1] - 1
    _need(committed, "committed", torch.int32, (B, K + 1), dev)
    if out_len.dim() != 2 or out_len.shape[0] != B:
        raise ValueError("out_len must be [B, top_n]")
    top_n = out_len.shape[1]
    _need(out_len, "out_len", torch.int32, (B, top_n), dev)
    _need(out_token, "out_token", torch.int32, (B, top_n), dev)
    if hit_index is None:
        hit_index = torch.empty(B, dtype=torch.int32, device=dev)
    _need(hit_index, "hit_index", torch.int32, (B,), dev)
    _check(load_library().jsv_cache_lookup(_ptr(n_accepted), _ptr(committed), B, K, _ptr(out_len),
                                           _ptr(out_token), top_n, _ptr(hit_index), _stream(stream)))
    return hit_index


def calibrated_lengths(p_tilde, out=None, flags=None, stream=None):
    """jsv_calibrated_lengths: G(k) - G(k+1) from per-position estimates p_tilde [B, K]."""
    if p_tilde.dim() != 2:
        raise ValueError("p_tilde must be [B, K]")
    B, K = p_tilde.shape
    dev = p_tilde.device
    _need(p_tilde, "p_tilde", torch.float64, (B, K), dev)
    if out is None:
        out = torch.empty(B, K + 1, dtype=torch.float64, device=dev)
    if flags is None:
        flags = torch.empty(B, dtype=torch.int32, device=dev)
    _need(out, "out", torch.float64, (B, K + 1), dev)
    _need(flags, "flags", torch.int32, (B,), dev)
    _check(load_library().jsv_calibrated_lengths(_ptr(p_tilde), B, K, _ptr(out), _ptr(flags),
                                                 _stream(stream)))
    return out, flags


def geometric_fanout(alpha: float, rho: float, gamma: int, B: int):
    """jsv_geometric_fanout (host): (F_real list, F_int list, hit mass)."""
    fr = (ctypes.c_double * (gamma + 1))()
    fi = (ctypes.c_int32 * (gamma + 1))()
    hm = ctypes.c_double()
    if not (1 <= gamma <= 64):
        raise ValueError("gamma must be in 1..64")
    _check(load_library().jsv_geometric_fanout(float(alpha), float(rho), int(gamma), int(B), fr, fi,
                                               ctypes.byref(hm)))
    return list(fr), list(fi), hm.value
