/*
 * libjsverify -- draft-block verification and foresight outcome scoring on MI355X.
 *
 * The method these calls implement is described in "JetSpec++: Foresight Parallel
 * Drafting with Self Refinements" (the paper text):
 *   - the speculative-sampling acceptance rule and its bonus token (§3 Preliminaries);
 *   - the point-mass proposal for a fixed draft (App. F.3 Lossless Verification);
 *   - the decoder's final norm + LM head (§4.2 "Decoder", App. B.1);
 *   - the outcome law over (accepted length k, bonus token a) (§4.2 Eq. 6) and the
 *     selection of the most probable outcomes (§4.2 Eq. 7, App. B.1 "Cache size").
 *
 * Conventions for every call
 *   - Pointers named as device pointers are contiguous row-major device memory owned
 *     by the caller.  The library never allocates device memory.
 *   - `ws` is a caller-owned device workspace of at least jsv_workspace_bytes() bytes
 *     (16-byte aligned, contents need no initialisation).  Two calls that overlap in
 *     time must not share a workspace.
 *   - Calls enqueue kernels on `hip_stream` (a hipStream_t; NULL = the null stream)
 *     and return without synchronising.  Outputs are valid once the stream reaches
 *     the end of the call.
 *   - Argument errors are detected on the host before anything is enqueued and are
 *     returned synchronously.  Conditions only the device can see are reported per
 *     request in `flags` (JSV_FLAG_*).  A HIP launch error returns JSV_EHIP.
 *   - Rows: a request holds K draft tokens d_0..d_{K-1} and K+1 target rows.  Row
 *     i < K verifies d_i; row K is the distribution after the whole block (the
 *     paper's position gamma+1).  Hidden states are laid out [B][K+1][d].
 *   - Temperature T > 0 samples from softmax(z / T); T = 0 is greedy: the target
 *     distribution is the point mass on the argmax, ties to the lowest token id
 *     (App. F.1 Assumption 1(iv)), so verification is argmax-prefix matching.
 *   - Randomness: Philox4x32-10 (Salmon et al., SC'11) with key (lo32(seed),
 *     hi32(seed)) and counter (row i, request b, lo32(offset), hi32(offset)); output
 *     word x0 gives u_i = x0 * 2^-32 for the acceptance test of row i, words x1, x2
 *     give v_i = (x1 * 2^21 + (x2 >> 11)) * 2^-53 for a bonus drawn at row i.
 *   - Supported shapes: hidden / 256 (bf16) or hidden / 128 (f32) in {1, 2, 4, 8, 12, 16, 20},
 *     hidden / 256 in {2, 4, 8, 12, 16, 20} for fp8 (so d = 4096 and 5120 for bf16 and
 *     fp8); 1 <= vocab <= 2^22; 1 <= K <= 32; 1 <= B <= 8.
 *     Anything else returns JSV_EUNSUPPORTED or JSV_EINVAL.
 */
#ifndef JSVERIFY_H
#define JSVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  JSV_OK = 0,
  JSV_EINVAL = -1,        /* null pointer, negative size, bad enum value, K/B/top_n out of range */
  JSV_EUNSUPPORTED = -2,  /* a shape this build has no kernel for (hidden not a multiple of 256 ...) */
  JSV_EWORKSPACE = -3,    /* ws_bytes smaller than jsv_workspace_bytes() */
  JSV_EHIP = -4           /* the HIP runtime returned an error while enqueueing */
} jsv_status;

/* Element type of an LM head.  JSV_FP8 is a weight-only quantised head: `weight` holds OCP
   FP8 E4M3 codes (one byte per element) and `weight_scale` one fp32 scale per vocabulary
   row, W[v][j] = weight_scale[v] * e4m3(weight[v][j]); the RMSNorm weight and the hidden
   states are bf16 and the normalised state is rounded to bf16, as for JSV_BF16.  Results
   are exact with respect to that quantised head (paper App. F.3: the rule is lossless with
   respect to the target it verifies against). */
typedef enum { JSV_BF16 = 0, JSV_F32 = 1, JSV_FP8 = 2 } jsv_dtype;

typedef enum {
  /* q_i = softmax(draft_logits_i / T); accept d_i with probability min(1, p_i(d_i)/q_i(d_i));
     bonus from the residual max(p - q, 0) (paper §3). */
  JSV_PROPOSAL_SOFTMAX = 0,
  /* q_i = point mass on d_i; accept with probability p_i(d_i); bonus from p_i with d_i
     removed (paper App. F.3).  Lossless for any draft fixed before verification. */
  JSV_PROPOSAL_POINT = 1
} jsv_proposal;

/* Per-request flag bits written to `flags`. */
#define JSV_FLAG_ACCEPT_TIE    (1u << 0) /* T > 0: |u_i - alpha_i| < 1e-4 at a row the scan reached   */
#define JSV_FLAG_LOGIT_GAP     (1u << 1) /* T = 0: top-2 logit gap < 1e-3 at a row that decided k or a */
#define JSV_FLAG_CDF_TIE       (1u << 2) /* bonus target within 1e-8 (probability mass) of a CDF step,
                                            or rounding left it past the last step          */
#define JSV_FLAG_INVALID       (1u << 3) /* non-finite logits or a draft token outside [0, vocab)       */
#define JSV_FLAG_ZERO_RESIDUAL (1u << 4) /* residual mass 0 at the rejected row: sampled p_k instead    */
#define JSV_FLAG_TOPN_TIE      (1u << 5) /* adjacent outcomes among the top N+1 within 1e-3 relative    */

/* The target's final norm and LM head (paper §4.2 "Decoder"; App. B.1). */
typedef struct {
  const void* weight;       /* device, [vocab][hidden] row-major, element type `dtype`        */
  const void* norm_weight;  /* device, [hidden] RMSNorm gain gamma, element type `dtype`      */
  int64_t vocab;            /* V >= 1                                                          */
  int64_t hidden;           /* d                                                               */
  float eps;                /* RMSNorm epsilon: x = gamma * h / sqrt(mean(h^2) + eps)          */
  int32_t dtype;            /* jsv_dtype of weight, norm_weight and hidden states             */
  const float* weight_scale;/* device, [vocab] fp32 row scales for JSV_FP8; ignored otherwise  */
} jsv_lm_head;

/* Bytes of workspace any call with at most `batch` requests, `K` drafts and `top_n`
   outcomes needs, including room for the [batch][K+1][vocab] fp32 logits when the
   caller does not supply them.  Returns 0 when the arguments are invalid. */
size_t jsv_workspace_bytes(const jsv_lm_head* head, int32_t batch, int32_t K, int32_t top_n);

/* Final RMSNorm then LM head for `rows` hidden states (paper §4.2 "Decoder"):
     x = round_dtype( fp32( fp32(h * r) * gamma ) ),
     r = fp32( 1 / sqrt(mean(h^2) + eps) )   (evaluated in float64, rounded once)
     logits[m][v] = sum_j x[m][j] * W[v][j]  (fp32 accumulate)
   hidden: device [rows][hidden] in `dtype`; logits: device [rows][vocab] fp32.       */
jsv_status jsv_lmhead_logits(const jsv_lm_head* head, const void* hidden, int64_t rows,
                             float* logits, void* ws, size_t ws_bytes, void* hip_stream);

/* Verify a block (paper §3; App. F.3 for JSV_PROPOSAL_POINT).
   hidden:       device [B][K+1][hidden], `dtype`: target states of the verified rows
   draft_tokens: device [B][K] int32
   draft_logits: device [B][K][vocab] fp32 for JSV_PROPOSAL_SOFTMAX, NULL for POINT
   Left to right, d_i is accepted iff u_i < alpha_i; k is the first rejection (K if none).
   The bonus token is drawn by inverse CDF from the residual at row k (or p_K when
   k = K) with uniform v_k; at T = 0 it is the argmax of row k.
   Outputs (device): n_accepted [B] (k in 0..K; -1 for an invalid request),
   committed [B][K+1] (d_0..d_{k-1}, bonus, then -1), flags [B] or NULL,
   logits_out [B][K+1][vocab] fp32 or NULL (then the logits live in `ws`).
   A round commits n_accepted + 1 tokens: the accepted prefix plus the bonus (§3). */
jsv_status jsv_verify_block(const jsv_lm_head* head, const void* hidden,
                            const int32_t* draft_tokens, const float* draft_logits,
                            int32_t B, int32_t K, float temperature, int32_t mode,
                            uint64_t seed, uint64_t offset,
                            int32_t* n_accepted, int32_t* committed, uint32_t* flags,
                            float* logits_out, void* ws, size_t ws_bytes, void* hip_stream);

/* The two halves of jsv_verify_block, for callers that want to time or interleave them.
   jsv_verify_stats runs the fused RMSNorm + LM head with its per-row softmax statistics
   (one stream over W; writes the logits and statistics into logits_out / ws only).
   jsv_verify_sample then runs the acceptance scan and draws the bonus token, writing
   n_accepted, committed and flags.  Call them in this order on one stream with the same
   arguments and workspace; jsv_verify_block is exactly the two in sequence. */
jsv_status jsv_verify_stats(const jsv_lm_head* head, const void* hidden,
                            const int32_t* draft_tokens, const float* draft_logits,
                            int32_t B, int32_t K, float temperature, int32_t mode,
                            uint64_t seed, uint64_t offset,
                            int32_t* n_accepted, int32_t* committed, uint32_t* flags,
                            float* logits_out, void* ws, size_t ws_bytes, void* hip_stream);
jsv_status jsv_verify_sample(const jsv_lm_head* head, const void* hidden,
                             const int32_t* draft_tokens, const float* draft_logits,
                             int32_t B, int32_t K, float temperature, int32_t mode,
                             uint64_t seed, uint64_t offset,
                             int32_t* n_accepted, int32_t* committed, uint32_t* flags,
                             const float* logits_out, void* ws, size_t ws_bytes,
                             void* hip_stream);

/* Foresight outcome scoring (paper §4.2 Eq. 6 and Eq. 7; App. B.1).
   hidden_pred: device [B][K+1][hidden], predicted states of the block under verification.
   With A_0 = 1 and A_{k+1} = A_k * alpha_k (alpha from the same rule as verification):
     P(k)   = A_k (1 - alpha_k),   P(k, a) = P(k) * r_k(a) / Z_k   for k < K,
     P(K)   = A_K,                 P(K, a) = A_K * p_K(a),
   where r_k is the residual of row k and Z_k its mass; for JSV_PROPOSAL_POINT this is
   exactly Eq. 6.  The top_n outcomes with P > 0 are returned ordered by P descending,
   then k ascending, then token ascending; missing entries are (-1, -1, 0).
   Outputs (device): out_len, out_token [B][top_n] int32; out_prob [B][top_n] fp32;
   len_marginal [B][K+1] fp64 or NULL; flags [B] or NULL.  1 <= top_n <= 64. */
jsv_status jsv_score_outcomes(const jsv_lm_head* head, const void* hidden_pred,
                              const int32_t* draft_tokens, const float* draft_logits,
                              int32_t B, int32_t K, float temperature, int32_t mode,
                              int32_t top_n, int32_t* out_len, int32_t* out_token,
                              float* out_prob, double* len_marginal, uint32_t* flags,
                              void* ws, size_t ws_bytes, void* hip_stream);

/* Anchor replacement (paper §4.3 "Anchor Replacement"): the decoder reads predicted states
   of the block and finds the first position whose most likely token differs from the
   draft; its token is the replacement.  This is the greedy (T = 0) rule applied to the
   decoder's logits.
   hidden_pred:  device [B][K+1][hidden], `dtype`
   draft_tokens: device [B][K] int32
   Outputs (device): position [B] (first i < K with argmax z_i != d_i, or K when every
   draft matches; -1 for an invalid request), token [B] (the argmax of that row, lowest
   id on ties), flags [B] or NULL (JSV_FLAG_LOGIT_GAP, JSV_FLAG_INVALID).
   Needs jsv_workspace_bytes(head, B, K, 0) of workspace. */
jsv_status jsv_anchor_replace(const jsv_lm_head* head, const void* hidden_pred,
                              const int32_t* draft_tokens, int32_t B, int32_t K,
                              int32_t* position, int32_t* token, uint32_t* flags, void* ws,
                              size_t ws_bytes, void* hip_stream);

/* Cache hit test (paper §4.1): the realised outcome of request b is (k, a) with
   k = n_accepted[b] and a = committed[b][k]; it hits when some entry i of the cached
   list (out_len[b][i], out_token[b][i]) equals it.
   n_accepted [B], committed [B][K+1] (as written by jsv_verify_block), out_len and
   out_token [B][top_n] (as written by jsv_score_outcomes): device int32.
   Output: hit_index [B] (device int32), the first matching entry, or -1 for a miss or
   an invalid round (k < 0).  1 <= top_n <= 64, 1 <= K <= 32, B >= 1. */
jsv_status jsv_cache_lookup(const int32_t* n_accepted, const int32_t* committed, int32_t B,
                            int32_t K, const int32_t* out_len, const int32_t* out_token,
                            int32_t top_n, int32_t* hit_index, void* hip_stream);

/* Calibrated length score (paper App. B.1, Eq. 12): from per-position acceptance estimates
   p_tilde[b][i] in [0, 1] of the 1-based positions i = 1..K, G(k) = prod_{i <= k} p_tilde_i
   (G(0) = 1, G(K+1) = 0) and len_score[b][k] = G(k) - G(k+1), k = 0..K, in float64.
   p_tilde: device [B][K] double; len_score: device [B][K+1] double; flags [B] or NULL.
   A request with an estimate outside [0, 1] or not a number is flagged JSV_FLAG_INVALID
   and scored 0.  1 <= K <= 32, B >= 1. */
jsv_status jsv_calibrated_lengths(const double* p_tilde, int32_t B, int32_t K, double* len_score,
                                  uint32_t* flags, void* hip_stream);

/* SSD's geometric fan-out (paper App. F.2, Proposition 2(a)): anchors per accepted length
   k = 0..gamma under the length law P(k) = alpha^k (1 - alpha) (k < gamma), alpha^gamma
   (k = gamma), and the surrogate hit curve 1 - F^-rho, for a cache of B anchors.  The
   active lengths are the M most likely ones (ties to the lower k) for the M whose series
   F_k = B P(k)^(1/(1+rho)) / sum_active P^(1/(1+rho)) keeps every active F_k >= 1 and
   captures the most hit mass sum_k P(k) (1 - F_k^-rho).  F_int rounds F_real down and
   gives the remaining anchors to the largest remainders (ties to the lower k).
   Host call (no device work): F_real [gamma+1] double, F_int [gamma+1] int32, hit_mass
   (may be NULL).  0 < alpha < 1, rho > 0, 1 <= gamma <= 64, 2 <= B <= 1e6. */
jsv_status jsv_geometric_fanout(double alpha, double rho, int32_t gamma, int32_t B,
                                double* F_real, int32_t* F_int, double* hit_mass);

/* Static text for a status code. */
const char* jsv_status_string(jsv_status status);

/* Library ABI version (major * 10000 + minor * 100 + patch). */
int32_t jsv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* JSVERIFY_H */
