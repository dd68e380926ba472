"""Plain, slow CPU reference of draft-block verification and outcome scoring.

TEST INFRASTRUCTURE.  Only tests/, the smoke check in __graft_entry__.py and the
cpu_baseline leg of bench.py may import or run this module.  The product path
(the HIP library and its Python binding) never calls it, and it shares no code
with that path: not a kernel, header, table, helper or constant generator.

Everything is float64 NumPy unless a step fixes a rounding point (RMSNorm, where
the value handed to the LM head is rounded to the weight dtype).  Every function
states the passage of the method it follows; "JetSpec++ paper" is the paper text
"JetSpec++: Foresight Parallel Drafting with Self Refinements".

Notation: a request holds K draft tokens d_0..d_{K-1} and K+1 target rows.  Row
i < K is the target distribution p_i that verifies d_i; row K is the distribution
after the whole block ("position gamma+1" in the paper's 1-based notation).

Readings of points the pages leave open:
  * RMSNorm formula, epsilon and rounding points are not on the pages; the plain
    definition gamma * h / sqrt(mean(h^2) + eps) is used, computed in fp32 steps
    and rounded once to the weight dtype before the LM head.
  * The proposal q is the draft logits' softmax at the same temperature as p.
  * Temperature 0 means p is the point mass on the argmax, ties to the lowest id, and
    verification is argmax-prefix matching: the proposal q plays no role, so at T = 0
    both proposals give the same result (the point-mass formulas apply).
  * A zero residual mass (only possible for a draft token that q gives no mass)
    falls back to sampling the target row itself, and is flagged.
  * An invalid request (non-finite logits, draft token outside the vocabulary)
    commits nothing: n_accepted = -1, committed all -1, flag bit 3.
"""
from __future__ import annotations

import numpy as np

from .philox import block_uniforms_np

# ---- per-request flag bits (the C header documents the same bits) -------------
FLAG_ACCEPT_TIE = 1 << 0      # |u_i - alpha_i| < ACCEPT_TIE at a row the scan reached (T > 0)
FLAG_LOGIT_GAP = 1 << 1       # top-2 logit gap < LOGIT_GAP_TIE at a deciding row (T = 0)
FLAG_CDF_TIE = 1 << 2         # sampling target within CDF_TIE (probability mass) of a CDF step, or fell through
FLAG_INVALID = 1 << 3         # non-finite logits or a draft token outside [0, V)
FLAG_ZERO_RESIDUAL = 1 << 4   # residual mass Z = 0: sampled the target row instead
FLAG_TOPN_TIE = 1 << 5        # adjacent top-(N+1) outcome probabilities within TOPN_TIE (relative)

ACCEPT_TIE = 1e-4
LOGIT_GAP_TIE = 1e-3
# The CDF window is absolute, in units of probability mass: an error dz in the logits
# moves C(a) by at most sum_w p(w) |dz_w| / T whatever the residual mass Z is, so a window
# relative to Z would shrink exactly where the residual is small and the draw sensitive.
CDF_TIE = 1e-8
TOPN_TIE = 1e-3

PROPOSAL_SOFTMAX = 0   # q = softmax(draft_logits / T); accept min(1, p/q)   (paper §3)
PROPOSAL_POINT = 1     # q = point mass on the draft token; accept p(d)      (paper App. F.3)


# ---- rounding helpers ------------------------------------------------------------
def bf16_round(x):
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.asarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    bits = ((bits + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    out = (bits & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(np.float32)
    return np.where(np.isnan(x), x, out)


def _as_f64(a):
    """Any CPU array-like (NumPy, or a torch tensor of any float dtype, E4M3 codes
    included) as float64 NumPy."""
    if hasattr(a, "detach"):
        import torch
        t = a.detach().to("cpu")
        if t.dtype == torch.float8_e4m3fn:
            t = t.to(torch.float32)   # every E4M3 value is a float32 value
        return t.to(torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


# ---- a1: final RMSNorm ------------------------------------------------------------
def rmsnorm(h, gamma, eps, dtype):
    """Target's final norm before the LM head (JetSpec++ paper §4.2 'Decoder', App. B.1).

    h: [..., d] values of the input dtype; gamma: [d].  Returns float64 values that are
    exactly representable in `dtype` ('bf16' or 'f32'):
        r   = fp32( 1 / sqrt( sum(h^2)/d + eps ) )      (sum in fp64)
        y   = fp32( fp32(h * r) * gamma )
        out = bf16(y) for 'bf16', y for 'f32'
    """
    h32 = _as_f64(h).astype(np.float32)
    g32 = _as_f64(gamma).astype(np.float32)
    d = h32.shape[-1]
    ms = np.sum(h32.astype(np.float64) ** 2, axis=-1) / d
    r = (1.0 / np.sqrt(ms + float(np.float32(eps)))).astype(np.float32)
    y = (h32 * r[..., None]).astype(np.float32)
    y = (y * g32).astype(np.float32)
    if dtype == "bf16":
        y = bf16_round(y)
    elif dtype != "f32":
        raise ValueError(dtype)
    return y.astype(np.float64)


# ---- a2: LM head ------------------------------------------------------------------
def lm_head_logits(xhat, weight, chunk=8192):
    """z = xhat . W^T in float64 (paper §4.2 'Decoder': the target's LM head).

    xhat: [M, d] float64; weight: [V, d] (NumPy or torch CPU tensor).  Products of
    bf16 values are exact in float64, so z differs from the exact sum only by the
    float64 summation order.  W is converted to float64 one vocabulary chunk at a time.
    """
    xhat = np.asarray(xhat, dtype=np.float64)
    V = weight.shape[0]
    z = np.empty((xhat.shape[0], V), dtype=np.float64)
    for v0 in range(0, V, chunk):
        wc = _as_f64(weight[v0:v0 + chunk])
        z[:, v0:v0 + wc.shape[0]] = xhat @ wc.T
    return z


# ---- a3/a4: softmax at temperature T -------------------------------------------------
def probs(z_row, T):
    """Next-token distribution at temperature T (paper §3; App. F.1 Assumption 1(iv)).

    T > 0: softmax(z / T).  T = 0: point mass on the argmax, ties to the lowest id.
    """
    z_row = np.asarray(z_row, dtype=np.float64)
    if T == 0:
        p = np.zeros_like(z_row)
        p[int(np.argmax(z_row))] = 1.0
        return p
    e = np.exp((z_row - z_row.max()) / T)
    return e / e.sum()


def top2_gap(z_row):
    """Largest minus second-largest logit (0 when the top value is shared)."""
    z_row = np.asarray(z_row, dtype=np.float64)
    i = int(np.argmax(z_row))
    rest = np.delete(z_row, i)
    return float(z_row[i] - rest.max()) if rest.size else np.inf


# ---- a5: acceptance probability ------------------------------------------------------
def accept_prob(p, q, d, mode):
    """alpha = min(1, p(d)/q(d)) (paper §3); point-mass proposal: alpha = p(d) (App. F.3).

    Written without a division where p(d) = 0 (alpha = 0) or p(d) >= q(d) (alpha = 1).
    """
    pd = float(p[d])
    if mode == PROPOSAL_POINT:
        return pd
    qd = float(q[d])
    if pd == 0.0:
        return 0.0
    if pd >= qd:
        return 1.0
    return pd / qd


# ---- a6: residual and inverse-CDF bonus draw ------------------------------------------
def residual(p, q, d, mode):
    """Unnormalised residual at a rejection: max(p - q, 0) (paper §3); for the point-mass
    proposal, p with the draft token removed (App. F.3)."""
    if mode == PROPOSAL_POINT:
        r = np.array(p, dtype=np.float64, copy=True)
        r[d] = 0.0
        return r
    return np.maximum(np.asarray(p, np.float64) - np.asarray(q, np.float64), 0.0)


def inverse_cdf(r, v):
    """Draw a token from the unnormalised r with uniform v in [0,1) by inversion.

    C(a) = r_0 + ... + r_a summed left to right in float64; Z = C(V-1); t = v * Z;
    the token is the first a with C(a) > t.  Returns (token, flags): FLAG_CDF_TIE if t
    lies within CDF_TIE of either end of the chosen step, or if rounding left no such a
    (then the last token with r > 0 is taken).
    """
    C = np.cumsum(np.asarray(r, dtype=np.float64))
    Z = float(C[-1])
    t = v * Z
    a = int(np.searchsorted(C, t, side="right"))
    flags = 0
    if a >= C.shape[0]:
        a = int(np.nonzero(np.asarray(r) > 0)[0][-1])
        flags |= FLAG_CDF_TIE
    lo = float(C[a - 1]) if a > 0 else 0.0
    hi = float(C[a])
    if (t - lo) < CDF_TIE or (hi - t) < CDF_TIE:
        flags |= FLAG_CDF_TIE
    return a, flags


# ---- the rule for one request -----------------------------------------------------------
def verify_request(z, g, drafts, T, mode, u, v):
    """Verify one draft block (paper §3 rule; App. F.3 for the point-mass proposal).

    z: [K+1, V] target logits; g: [K, V] draft logits (softmax mode) or None;
    drafts: K token ids; u, v: [K+1] uniforms (row i uses u[i] to accept d_i and
    v[i] when the bonus is drawn at row i).
    Returns (n_accepted k, committed [K+1] with -1 padding, flags).
    Left to right, d_i is accepted iff u_i < alpha_i; k is the first rejection (K if
    none).  The bonus comes from the residual at row k, or from p_K when all K drafts
    are accepted.  At T = 0 the draws collapse to argmax-prefix matching.
    """
    z = np.asarray(z, dtype=np.float64)
    K = len(drafts)
    V = z.shape[1]
    if T == 0:
        # greedy verification compares each draft with the row's argmax; q plays no role
        g, mode = None, PROPOSAL_POINT
    invalid = (not np.all(np.isfinite(z))) or any(not (0 <= int(d) < V) for d in drafts)
    if g is not None:
        invalid = invalid or not np.all(np.isfinite(np.asarray(g, np.float64)))
    if invalid:
        return -1, [-1] * (K + 1), FLAG_INVALID
    flags = 0
    if T == 0:
        am = [int(np.argmax(z[i])) for i in range(K + 1)]
        k = K
        for i in range(K):
            if int(drafts[i]) != am[i]:
                k = i
                break
        bonus = am[k]
        if any(top2_gap(z[i]) < LOGIT_GAP_TIE for i in range(k + 1)):
            flags |= FLAG_LOGIT_GAP
    else:
        P = [probs(z[i], T) for i in range(K + 1)]
        Q = [probs(g[i], T) for i in range(K)] if mode == PROPOSAL_SOFTMAX else [None] * K
        alpha = [accept_prob(P[i], Q[i], int(drafts[i]), mode) for i in range(K)]
        k = K
        for i in range(K):
            if not (u[i] < alpha[i]):
                k = i
                break
        for i in range(min(k, K - 1) + 1 if K > 0 else 0):
            if abs(u[i] - alpha[i]) < ACCEPT_TIE:
                flags |= FLAG_ACCEPT_TIE
        r = residual(P[k], Q[k], int(drafts[k]), mode) if k < K else P[K]
        if not (r.sum() > 0.0):
            flags |= FLAG_ZERO_RESIDUAL
            r = P[k]
        bonus, f = inverse_cdf(r, v[k])
        flags |= f
    committed = [int(x) for x in drafts[:k]] + [int(bonus)] + [-1] * (K - k)
    return k, committed, flags


# ---- a7: outcome law ------------------------------------------------------------------
def outcome_table(P, Q, drafts, mode):
    """Probability of every verification outcome (k, a) under the rule (paper §4.2 Eq. 6).

    P: [K+1, V] target (decoder) distributions; Q: [K, V] proposals or None (point mass).
    A_0 = 1, A_{k+1} = A_k * alpha_k.  For k < K:
        P(k)   = A_k (1 - alpha_k)
        P(k,a) = P(k) * r_k(a) / Z_k      with r_k the residual and Z_k its mass,
    which for the point-mass proposal is A_k * p_k(a), a != d_k -- Eq. 6 itself.
    P(K) = A_K and P(K, a) = A_K * p_K(a).  A zero residual mass falls back to p_k,
    as the sampler does.  Returns (table [K+1, V], marginals [K+1], flags).
    """
    K = len(drafts)
    V = len(P[0])
    table = np.zeros((K + 1, V), dtype=np.float64)
    marg = np.zeros(K + 1, dtype=np.float64)
    flags = 0
    A = 1.0
    for k in range(K):
        q = Q[k] if Q is not None else None
        alpha = accept_prob(P[k], q, int(drafts[k]), mode)
        Pk = A * (1.0 - alpha)
        marg[k] = Pk
        if Pk > 0.0:
            r = residual(P[k], q, int(drafts[k]), mode)
            Z = r.sum()
            if Z > 0.0:
                table[k] = Pk * r / Z
            else:
                flags |= FLAG_ZERO_RESIDUAL
                table[k] = Pk * np.asarray(P[k], np.float64)
        A = A * alpha
    marg[K] = A
    table[K] = A * np.asarray(P[K], np.float64)
    return table, marg, flags


# ---- a8: top-N selection ------------------------------------------------------------------
def top_n(table, N):
    """The N most probable outcomes with P > 0 (paper §4.2 Eq. 7; App. B.1 'Cache size').

    Order: P descending, then k ascending, then token ascending (smaller index first on
    ties, as in App. F.2).  Fewer than N outcomes are padded with (-1, -1, 0).
    Returns (lens, tokens, probs, flags); FLAG_TOPN_TIE when two adjacent entries among
    the first N+1 differ by less than TOPN_TIE relative.
    """
    ks, ts = np.nonzero(table > 0.0)
    vals = table[ks, ts]
    order = np.lexsort((ts, ks, -vals))
    lens = np.full(N, -1, dtype=np.int64)
    toks = np.full(N, -1, dtype=np.int64)
    pr = np.zeros(N, dtype=np.float64)
    n = min(N, order.size)
    lens[:n] = ks[order[:n]]
    toks[:n] = ts[order[:n]]
    pr[:n] = vals[order[:n]]
    flags = 0
    head = vals[order[:N + 1]]
    for i in range(head.size - 1):
        if head[i] - head[i + 1] < TOPN_TIE * head[i]:
            flags |= FLAG_TOPN_TIE
    return lens, toks, pr, flags


# ---- whole calls (the three library entry points) ---------------------------------------------
class Head:
    """LM head: weight [V, d], RMSNorm weight [d], epsilon and dtype ('bf16' | 'f32' |
    'fp8').  An 'fp8' head holds E4M3 codes (a torch float8_e4m3fn tensor) and one scale
    per vocabulary row, W[v] = weight_scale[v] * e4m3(code); its normalised state is
    rounded to bf16 (weight-only quantisation; the verified target is the quantised one,
    paper App. F.3 and §5 on the NVFP4 results)."""

    def __init__(self, weight, norm_weight, eps, dtype, weight_scale=None):
        self.weight = weight
        self.norm_weight = norm_weight
        self.eps = float(np.float32(eps))
        self.dtype = dtype
        self.act_dtype = "bf16" if dtype == "fp8" else dtype
        self.weight_scale = None if weight_scale is None else _as_f64(weight_scale)
        if dtype == "fp8" and self.weight_scale is None:
            raise ValueError("an fp8 head needs row scales")
        self.vocab, self.hidden = int(weight.shape[0]), int(weight.shape[1])


def block_logits(head, hidden):
    """RMSNorm then LM head for rows [..., d] -> float64 logits [..., V]."""
    h = _as_f64(hidden)
    lead = h.shape[:-1]
    xhat = rmsnorm(h.reshape(-1, head.hidden), head.norm_weight, head.eps, head.act_dtype)
    z = lm_head_logits(xhat, head.weight)
    if head.weight_scale is not None:
        z = z * head.weight_scale[None, :]
    return z.reshape(*lead, head.vocab)


def verify_block(head, hidden, draft_tokens, draft_logits, T, mode, seed, offset):
    """The whole verification call: hidden [B, K+1, d] -> per-request (k, committed, flags).

    Uniforms come from Philox4x32-10 with counter (row, request, offset) and key seed.
    Returns dict with n_accepted [B], committed [B, K+1], flags [B] and logits [B, K+1, V].
    """
    drafts = np.asarray(draft_tokens)
    B, K = drafts.shape
    z = block_logits(head, hidden)
    g = _as_f64(draft_logits) if draft_logits is not None else None
    if mode == PROPOSAL_SOFTMAX and g is None and T > 0:
        raise ValueError("softmax proposal needs draft logits")
    n_acc = np.zeros(B, dtype=np.int64)
    committed = np.full((B, K + 1), -1, dtype=np.int64)
    flags = np.zeros(B, dtype=np.int64)
    rows = np.arange(K + 1)
    for b in range(B):
        u, v = block_uniforms_np(seed, offset, b, rows)
        k, c, f = verify_request(z[b], None if g is None else g[b], drafts[b], T, mode, u, v)
        n_acc[b], committed[b], flags[b] = k, c, f
    return {"n_accepted": n_acc, "committed": committed, "flags": flags, "logits": z}


def score_outcomes(head, hidden_pred, draft_tokens, draft_logits, T, mode, N):
    """Foresight scoring: outcome law from predicted states, and its top-N.

    Returns dict with out_len, out_token, out_prob [B, N], len_marginal [B, K+1],
    flags [B] and the full tables [B, K+1, V].
    """
    drafts = np.asarray(draft_tokens)
    B, K = drafts.shape
    z = block_logits(head, hidden_pred)
    g = _as_f64(draft_logits) if draft_logits is not None else None
    if mode == PROPOSAL_SOFTMAX and g is None and T > 0:
        raise ValueError("softmax proposal needs draft logits")
    V = z.shape[-1]
    out = {"out_len": np.full((B, N), -1, np.int64), "out_token": np.full((B, N), -1, np.int64),
           "out_prob": np.zeros((B, N)), "len_marginal": np.zeros((B, K + 1)),
           "flags": np.zeros(B, np.int64), "tables": np.zeros((B, K + 1, V))}
    for b in range(B):
        invalid = (not np.all(np.isfinite(z[b]))) or any(not (0 <= int(d) < V) for d in drafts[b])
        if g is not None and mode == PROPOSAL_SOFTMAX and T > 0:
            invalid = invalid or not np.all(np.isfinite(g[b]))
        if invalid:
            out["flags"][b] = FLAG_INVALID
            continue
        P = [probs(z[b, i], T) for i in range(K + 1)]
        use_q = mode == PROPOSAL_SOFTMAX and T > 0
        Q = [probs(g[b, i], T) for i in range(K)] if use_q else None
        table, marg, f1 = outcome_table(P, Q, drafts[b], mode if use_q else PROPOSAL_POINT)
        if T == 0:
            f1 |= FLAG_LOGIT_GAP if any(top2_gap(z[b, i]) < LOGIT_GAP_TIE
                                        for i in range(int(np.argmax(marg)) + 1)) else 0
        lens, toks, pr, f2 = top_n(table, N)
        out["out_len"][b], out["out_token"][b], out["out_prob"][b] = lens, toks, pr
        out["len_marginal"][b] = marg
        out["flags"][b] = f1 | f2
        out["tables"][b] = table
    return out


def lmhead_logits(head, hidden_rows):
    """RMSNorm + LM head for rows [M, d] -> float64 logits [M, V]."""
    return block_logits(head, hidden_rows)


# ---- next rows: anchor replacement, cache lookup, calibrated lengths, SSD fan-out --------
def anchor_replace(head, hidden_pred, draft_tokens):
    """Anchor replacement (paper §4.3 "Anchor Replacement"): the decoder reads the
    predicted states of the block and finds the first position at which its most likely
    token differs from the draft; that token is written there.

    hidden_pred [B, K+1, d]; draft_tokens [B, K].  Returns position [B] (first i < K with
    argmax z_i != d_i, or K when every draft matches), token [B] (the argmax of that row;
    the argmax of row K when every draft matches) and flags [B] (LOGIT_GAP when a row up
    to the position has a top-2 gap < 1e-3; INVALID for non-finite logits or a draft
    outside the vocabulary, with position = token = -1).  Ties go to the lowest id.
    """
    drafts = np.asarray(draft_tokens)
    B, K = drafts.shape
    z = block_logits(head, hidden_pred)
    V = z.shape[-1]
    pos = np.full(B, -1, np.int64)
    tok = np.full(B, -1, np.int64)
    flags = np.zeros(B, np.int64)
    for b in range(B):
        if (not np.all(np.isfinite(z[b]))) or any(not (0 <= int(x) < V) for x in drafts[b]):
            flags[b] = FLAG_INVALID
            continue
        am = [int(np.argmax(z[b, i])) for i in range(K + 1)]
        k = next((i for i in range(K) if am[i] != int(drafts[b, i])), K)
        pos[b], tok[b] = k, am[k]
        if any(top2_gap(z[b, i]) < LOGIT_GAP_TIE for i in range(k + 1)):
            flags[b] = FLAG_LOGIT_GAP
    return pos, tok, flags


def cache_lookup(n_accepted, committed, out_len, out_token):
    """Cache hit test (paper §4.1): the realised outcome of a round is (k, a) with k the
    accepted count and a the bonus token committed at position k; it hits when it is one
    of the cached (length, token) pairs.  Returns the index of the first matching entry per
    request, or -1 (a miss, or an invalid round with k < 0)."""
    n_accepted = np.asarray(n_accepted)
    committed = np.asarray(committed)
    out_len, out_token = np.asarray(out_len), np.asarray(out_token)
    res = np.full(n_accepted.shape[0], -1, np.int64)
    for b in range(n_accepted.shape[0]):
        k = int(n_accepted[b])
        if k < 0:
            continue
        a = int(committed[b, k])
        for i in range(out_len.shape[1]):
            if int(out_len[b, i]) == k and int(out_token[b, i]) == a:
                res[b] = i
                break
    return res


def calibrated_lengths(p_tilde):
    """Calibrated length score (paper App. B.1, Eq. 12): with per-position estimates p~_i
    for the 1-based positions i = 1..K of a block, G(k) = prod_{i <= k} p~_i (G(0) = 1) and
    P~(k) = G(k) - G(k+1) for k = 0..K, with G(K+1) = 0.

    p_tilde [B, K] in [0, 1] -> (scores [B, K+1] float64, flags [B]); a request with an
    estimate outside [0, 1] (or not a number) is flagged INVALID and scored 0."""
    p = np.asarray(p_tilde, dtype=np.float64)
    B, K = p.shape
    out = np.zeros((B, K + 1))
    flags = np.zeros(B, np.int64)
    for b in range(B):
        if not np.all((p[b] >= 0.0) & (p[b] <= 1.0)):
            flags[b] = FLAG_INVALID
            continue
        G = [1.0]
        for i in range(K):
            G.append(G[-1] * p[b, i])
        G.append(0.0)
        out[b] = [G[k] - G[k + 1] for k in range(K + 1)]
    return out, flags


def ssd_length_law(alpha, gamma):
    """P_alpha(k) of the fan-out model (paper App. F.2): alpha^k (1 - alpha) for k < gamma,
    alpha^gamma for k = gamma."""
    return np.array([alpha ** k * (1.0 - alpha) for k in range(gamma)] + [alpha ** gamma])


def fanout_objective(P, F, rho):
    """Surrogate hit mass sum_k P(k) (1 - F_k^-rho) over active lengths (F_k >= 1)."""
    return float(sum(P[k] * (1.0 - F[k] ** (-rho)) for k in range(len(P)) if F[k] >= 1.0))


def geometric_fanout(alpha, rho, gamma, B):
    """SSD's geometric fan-out as the maximiser of the surrogate problem (paper App. F.2,
    Proposition 2(a) and its proof): the active lengths are the M lengths of largest
    P_alpha(k) for some M (ties to the lower k); on them F_k = B P^(1/(1+rho)) / sum P^(1/(1+rho));
    a candidate counts only when every active F_k >= 1, and the best candidate maximises
    sum_k P(k) (1 - F_k^-rho).  The integer allocation rounds F down and hands the
    remaining anchors to the largest remainders (ties to the lower k), as the paper does
    for its Table 11.

    Returns (F_real [gamma+1], F_int [gamma+1], hit_mass of F_real, active M)."""
    P = ssd_length_law(alpha, gamma)
    order = sorted(range(gamma + 1), key=lambda k: (-P[k], k))
    best = None
    for M in range(1, gamma + 2):
        act = order[:M]
        w = np.array([P[k] ** (1.0 / (1.0 + rho)) for k in act])
        F = np.zeros(gamma + 1)
        F[act] = B * w / w.sum()
        if np.any(F[act] < 1.0):
            continue
        obj = fanout_objective(P, F, rho)
        if best is None or obj > best[0]:
            best = (obj, F, M)
    obj, F, M = best
    Fi = np.floor(F).astype(np.int64)
    rem = B - int(Fi.sum())
    frac = sorted(range(gamma + 1), key=lambda k: (-(F[k] - Fi[k]), k))
    for k in frac[:rem]:
        Fi[k] += 1
    return F, Fi, obj, M
