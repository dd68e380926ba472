// Host side of libjsverify: argument validation, workspace carve-up and kernel
// orchestration on the caller's stream.  The C ABI is declared in include/jsverify.h.
#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "jsv_internal.h"
#include "jsverify.h"

using namespace jsv;

namespace {

constexpr float kLog2e = 1.4426950408889634f;

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  static int cache[64] = {0};  // per-device constant, filled on first use
  if (dev >= 0 && dev < 64 && cache[dev] > 0) return cache[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64) cache[dev] = n;
  return n;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int k_per_step(int dtype) { return dtype == JSV_F32 ? 16 : 32; }
// Bytes per element of the hidden states and RMSNorm weight (bf16 for an fp8 head).
size_t act_bytes(int dtype) { return dtype == JSV_F32 ? 4 : 2; }

// Validates the head; on success *nks is hidden / (waves * k per MFMA step).
jsv_status check_head(const jsv_lm_head* h, int* nks) {
  if (h == nullptr || h->weight == nullptr || h->norm_weight == nullptr) return JSV_EINVAL;
  if (h->dtype != JSV_BF16 && h->dtype != JSV_F32 && h->dtype != JSV_FP8) return JSV_EINVAL;
  if (h->dtype == JSV_FP8 && (h->weight_scale == nullptr ||
                              (reinterpret_cast<uintptr_t>(h->weight_scale) & 3u) != 0))
    return JSV_EINVAL;
  if (h->vocab < 1 || h->hidden < 1) return JSV_EINVAL;
  if (!(h->eps >= 0.f) || !isfinite(h->eps)) return JSV_EINVAL;
  if (!aligned16(h->weight) || !aligned16(h->norm_weight)) return JSV_EINVAL;
  if (h->vocab > kMaxVocab) return JSV_EUNSUPPORTED;
  const int64_t step = int64_t(kWaves) * k_per_step(h->dtype);
  if (h->hidden % step != 0) return JSV_EUNSUPPORTED;
  const int64_t n = h->hidden / step;
  if (n > 64 || !stats_supported(h->dtype, int(n))) return JSV_EUNSUPPORTED;
  *nks = int(n);
  return JSV_OK;
}

jsv_status check_block(int32_t B, int32_t K, float T, int32_t mode) {
  if (B < 1 || B > kMaxB || K < 1 || K > kMaxK) return JSV_EINVAL;
  if (!(T >= 0.f) || !isfinite(T)) return JSV_EINVAL;
  if (mode != JSV_PROPOSAL_SOFTMAX && mode != JSV_PROPOSAL_POINT) return JSV_EINVAL;
  return JSV_OK;
}

// Workgroups of the LM-head kernel: one per CU, at most one per 16-row vocabulary group.
jsv_status run_stats(const jsv_lm_head* head, int nks, const void* hidden, int M, float* logits,
                     const float* G, int B, int K, float T, int mode, int stats, RowStat* partial,
                     float* rnorm, char* ws, hipStream_t stream) {
  const int cus = device_cu_count();
  if (cus <= 0) return JSV_EHIP;
  if (stats && ws != nullptr && wide_eligible(head->dtype, head->hidden, M)) {
    // More rows than one pass holds: split d instead of the rows (W is read once).
    const WsLayout L = ws_layout(head->vocab, B, K, 0, head->hidden, head->dtype);
    WideArgs w{};
    w.W = head->weight;
    w.gamma = head->norm_weight;
    w.hidden = hidden;
    w.V = head->vocab;
    w.d = int(head->hidden);
    w.M = M;
    w.eps = head->eps;
    w.pl = plan_wide(head->vocab, head->hidden, M, cus);
    w.xhat = reinterpret_cast<uint16_t*>(ws + L.xhat);
    w.planes = reinterpret_cast<float*>(ws + L.planes);
    w.rnorm = rnorm;
    w.logits = logits;
    w.G = G;
    w.B = B;
    w.K = K;
    w.T = T;
    w.c = T > 0.f ? kLog2e / T : 0.f;
    w.want_q = (mode == JSV_PROPOSAL_SOFTMAX && T > 0.f && G != nullptr) ? 1 : 0;
    w.quad = ((head->vocab & 3) == 0 && aligned16(logits) && (G == nullptr || aligned16(G))) ? 1 : 0;
    w.partial = partial;
    return launch_wide(w, stream) == hipSuccess ? JSV_OK : JSV_EHIP;
  }
  StatsArgs a{};
  a.W = head->weight;
  a.wscale = head->dtype == JSV_FP8 ? head->weight_scale : nullptr;
  a.gamma = head->norm_weight;
  a.V = head->vocab;
  a.d = int(head->hidden);
  a.eps = head->eps;
  a.G = G;
  a.B = B;
  a.K = K;
  a.T = T;
  a.c = T > 0.f ? kLog2e / T : 0.f;
  a.stats = stats;
  a.want_q = (stats && mode == JSV_PROPOSAL_SOFTMAX && T > 0.f && G != nullptr) ? 1 : 0;
  a.partial = partial;
  a.rnorm = rnorm;
  // Verification and scoring fit one launch; plain logits of many rows take several.
  const size_t rowbytes = size_t(head->hidden) * act_bytes(head->dtype);
  for (int m0 = 0; m0 < M; m0 += kMaxPlanRows) {
    const int m = (M - m0) < kMaxPlanRows ? (M - m0) : kMaxPlanRows;
    if (stats && m0 > 0) return JSV_EUNSUPPORTED;
    const StatsPlan pl = plan_stats(head->vocab, m, cus);
    a.hidden = static_cast<const char*>(hidden) + size_t(m0) * rowbytes;
    a.logits = logits + size_t(m0) * size_t(head->vocab);
    a.M = m;
    a.rp = pl.rp;
    a.npass = pl.npass;
    a.nchunk = pl.nchunk;
    if (launch_stats(head->dtype, nks, pl.nchunk * pl.npass, a, stream) != hipSuccess) return JSV_EHIP;
  }
  return JSV_OK;
}

FinalArgs final_args(const jsv_lm_head* head, const void* hidden, const int32_t* drafts,
                     const float* G, int B, int K, float T, int mode, int kind, char* ws,
                     const WsLayout& L) {
  FinalArgs f{};
  f.W = head->weight;
  f.wscale = head->dtype == JSV_FP8 ? head->weight_scale : nullptr;
  f.gamma = head->norm_weight;
  f.hidden = hidden;
  f.V = head->vocab;
  f.d = int(head->hidden);
  f.dtype = head->dtype;
  f.G = G;
  f.drafts = drafts;
  f.B = B;
  f.K = K;
  f.T = T;
  f.mode = mode;
  f.kind = kind;
  const int cus = device_cu_count();
  const int M = B * (K + 1);
  f.P = cus <= 0 ? 0
        : wide_eligible(head->dtype, head->hidden, M) ? plan_wide(head->vocab, head->hidden, M, cus).ncomb
                                                      : plan_stats(head->vocab, M, cus).nchunk;
  f.partial = reinterpret_cast<const RowStat*>(ws + L.partial);
  f.rowstat = reinterpret_cast<RowStat*>(ws + L.rowstat);
  f.dlog = reinterpret_cast<DraftLogit*>(ws + L.dlog);
  f.rnorm = reinterpret_cast<const float*>(ws + L.rnorm);
  f.rowfinal = reinterpret_cast<RowFinal*>(ws + L.rowfinal);
  f.req = reinterpret_cast<ReqState*>(ws + L.req);
  return f;
}

size_t needed_bytes(const jsv_lm_head* head, int B, int K, int top_n, bool logits_in_ws) {
  const WsLayout L = ws_layout(head->vocab, B, K, top_n, head->hidden, head->dtype);
  return logits_in_ws ? L.total : L.logits;
}

}  // namespace

extern "C" {

int32_t jsv_version(void) { return 100; }

const char* jsv_status_string(jsv_status s) {
  switch (s) {
    case JSV_OK: return "ok";
    case JSV_EINVAL: return "invalid argument";
    case JSV_EUNSUPPORTED: return "unsupported shape or dtype";
    case JSV_EWORKSPACE: return "workspace too small";
    case JSV_EHIP: return "HIP runtime error";
  }
  return "unknown status";
}

size_t jsv_workspace_bytes(const jsv_lm_head* head, int32_t batch, int32_t K, int32_t top_n) {
  int nks = 0;
  if (check_head(head, &nks) != JSV_OK) return 0;
  if (batch < 1 || batch > kMaxB || K < 1 || K > kMaxK || top_n < 0 || top_n > kMaxTopN) return 0;
  // Any call with at most `batch` requests and `K` drafts: a smaller block can need more
  // (34..144 rows take the split-d LM head and its partial-product planes).
  size_t most = 0;
  for (int b = 1; b <= batch; ++b)
    for (int k = 1; k <= K; ++k) {
      const size_t n = needed_bytes(head, b, k, top_n, true);
      if (n > most) most = n;
    }
  return most;
}

jsv_status jsv_lmhead_logits(const jsv_lm_head* head, const void* hidden, int64_t rows,
                             float* logits, void* ws, size_t ws_bytes, void* hip_stream) {
  (void)ws;
  (void)ws_bytes;
  int nks = 0;
  jsv_status st = check_head(head, &nks);
  if (st != JSV_OK) return st;
  if (rows < 0) return JSV_EINVAL;
  if (rows == 0) return JSV_OK;
  if (hidden == nullptr || logits == nullptr || !aligned16(hidden)) return JSV_EINVAL;
  if (rows > INT32_MAX / 2) return JSV_EUNSUPPORTED;
  (void)hipGetLastError();
  return run_stats(head, nks, hidden, int(rows), logits, nullptr, 0, -1, 0.f, JSV_PROPOSAL_POINT,
                   0, nullptr, nullptr, nullptr, static_cast<hipStream_t>(hip_stream));
}

static jsv_status verify_prepare(const jsv_lm_head* head, const void* hidden,
                                 const int32_t* draft_tokens, const float* draft_logits,
                                 int32_t B, int32_t K, float T, int32_t mode, int32_t* n_accepted,
                                 int32_t* committed, const float* logits_out, void* ws,
                                 size_t ws_bytes, int* nks) {
  jsv_status st = check_head(head, nks);
  if (st != JSV_OK) return st;
  st = check_block(B, K, T, mode);
  if (st != JSV_OK) return st;
  if (hidden == nullptr || !aligned16(hidden)) return JSV_EINVAL;
  if (draft_tokens == nullptr || committed == nullptr || ws == nullptr) return JSV_EINVAL;
  if (n_accepted == nullptr) return JSV_EINVAL;
  if (mode == JSV_PROPOSAL_SOFTMAX && T > 0.f && draft_logits == nullptr) return JSV_EINVAL;
  if (!aligned16(ws)) return JSV_EINVAL;
  if (ws_bytes < needed_bytes(head, B, K, 0, logits_out == nullptr)) return JSV_EWORKSPACE;
  return JSV_OK;
}

jsv_status jsv_verify_stats(const jsv_lm_head* head, const void* hidden,
                            const int32_t* draft_tokens, const float* draft_logits, int32_t B,
                            int32_t K, float temperature, int32_t mode, uint64_t seed,
                            uint64_t offset, int32_t* n_accepted, int32_t* committed,
                            uint32_t* flags, float* logits_out, void* ws, size_t ws_bytes,
                            void* hip_stream) {
  (void)seed;
  (void)offset;
  (void)flags;
  int nks = 0;
  jsv_status st = verify_prepare(head, hidden, draft_tokens, draft_logits, B, K, temperature, mode,
                                 n_accepted, committed, logits_out, ws, ws_bytes, &nks);
  if (st != JSV_OK) return st;
  (void)hipGetLastError();
  const WsLayout L = ws_layout(head->vocab, B, K, 0, head->hidden, head->dtype);
  char* w = static_cast<char*>(ws);
  float* logits = logits_out ? logits_out : reinterpret_cast<float*>(w + L.logits);
  return run_stats(head, nks, hidden, B * (K + 1), logits, draft_logits, B, K, temperature, mode, 1,
                   reinterpret_cast<RowStat*>(w + L.partial), reinterpret_cast<float*>(w + L.rnorm),
                   w, static_cast<hipStream_t>(hip_stream));
}

jsv_status jsv_verify_sample(const jsv_lm_head* head, const void* hidden,
                             const int32_t* draft_tokens, const float* draft_logits, int32_t B,
                             int32_t K, float temperature, int32_t mode, uint64_t seed,
                             uint64_t offset, int32_t* n_accepted, int32_t* committed,
                             uint32_t* flags, const float* logits_out, void* ws, size_t ws_bytes,
                             void* hip_stream) {
  int nks = 0;
  jsv_status st = verify_prepare(head, hidden, draft_tokens, draft_logits, B, K, temperature, mode,
                                 n_accepted, committed, logits_out, ws, ws_bytes, &nks);
  if (st != JSV_OK) return st;
  (void)hipGetLastError();
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  const WsLayout L = ws_layout(head->vocab, B, K, 0, head->hidden, head->dtype);
  char* w = static_cast<char*>(ws);
  FinalArgs f = final_args(head, hidden, draft_tokens, draft_logits, B, K, temperature, mode,
                           kFinalizeVerify, w, L);
  f.seed = seed;
  f.offset = offset;
  f.n_accepted = n_accepted;
  f.committed = committed;
  f.flags = flags;
  if (f.P <= 0 || launch_rowstat(f, stream) != hipSuccess) return JSV_EHIP;
  if (!(temperature > 0.f)) {  // greedy: the scan writes the argmax bonus
    return launch_scan(f, stream) == hipSuccess ? JSV_OK : JSV_EHIP;
  }
  SampleArgs a{};
  a.f = f;
  a.c = kLog2e / temperature;
  a.logits = logits_out ? logits_out : reinterpret_cast<const float*>(w + L.logits);
  a.G = draft_logits;
  a.zs = reinterpret_cast<double*>(w + L.zs);
  return launch_sample(a, stream) == hipSuccess ? JSV_OK : JSV_EHIP;
}

jsv_status jsv_verify_block(const jsv_lm_head* head, const void* hidden,
                            const int32_t* draft_tokens, const float* draft_logits, int32_t B,
                            int32_t K, float temperature, int32_t mode, uint64_t seed,
                            uint64_t offset, int32_t* n_accepted, int32_t* committed,
                            uint32_t* flags, float* logits_out, void* ws, size_t ws_bytes,
                            void* hip_stream) {
  jsv_status st = jsv_verify_stats(head, hidden, draft_tokens, draft_logits, B, K, temperature,
                                   mode, seed, offset, n_accepted, committed, flags, logits_out,
                                   ws, ws_bytes, hip_stream);
  if (st != JSV_OK) return st;
  return jsv_verify_sample(head, hidden, draft_tokens, draft_logits, B, K, temperature, mode, seed,
                           offset, n_accepted, committed, flags, logits_out, ws, ws_bytes,
                           hip_stream);
}

jsv_status jsv_score_outcomes(const jsv_lm_head* head, const void* hidden_pred,
                              const int32_t* draft_tokens, const float* draft_logits, int32_t B,
                              int32_t K, float temperature, int32_t mode, int32_t top_n,
                              int32_t* out_len, int32_t* out_token, float* out_prob,
                              double* len_marginal, uint32_t* flags, void* ws, size_t ws_bytes,
                              void* hip_stream) {
  int nks = 0;
  jsv_status st = check_head(head, &nks);
  if (st != JSV_OK) return st;
  st = check_block(B, K, temperature, mode);
  if (st != JSV_OK) return st;
  if (top_n < 1 || top_n > kMaxTopN) return JSV_EINVAL;
  if (hidden_pred == nullptr || !aligned16(hidden_pred) || draft_tokens == nullptr) return JSV_EINVAL;
  if (out_len == nullptr || out_token == nullptr || out_prob == nullptr) return JSV_EINVAL;
  if (ws == nullptr || !aligned16(ws)) return JSV_EINVAL;
  if (mode == JSV_PROPOSAL_SOFTMAX && temperature > 0.f && draft_logits == nullptr) return JSV_EINVAL;
  if (ws_bytes < needed_bytes(head, B, K, top_n, true)) return JSV_EWORKSPACE;
  (void)hipGetLastError();
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  const WsLayout L = ws_layout(head->vocab, B, K, top_n, head->hidden, head->dtype);
  char* w = static_cast<char*>(ws);
  float* logits = reinterpret_cast<float*>(w + L.logits);
  st = run_stats(head, nks, hidden_pred, B * (K + 1), logits, draft_logits, B, K, temperature, mode,
                 1, reinterpret_cast<RowStat*>(w + L.partial), reinterpret_cast<float*>(w + L.rnorm),
                 w, stream);
  if (st != JSV_OK) return st;
  FinalArgs f = final_args(head, hidden_pred, draft_tokens, draft_logits, B, K, temperature, mode,
                           kFinalizeScore, w, L);
  f.flags = flags;
  f.top_n = top_n;
  f.out_len = out_len;
  f.out_token = out_token;
  f.out_prob = out_prob;
  f.len_marginal = len_marginal;
  if (f.P <= 0 || launch_rowstat(f, stream) != hipSuccess || launch_scan(f, stream) != hipSuccess)
    return JSV_EHIP;
  if (!(temperature > 0.f)) return JSV_OK;
  ScoreArgs a{};
  a.V = head->vocab;
  a.B = B;
  a.K = K;
  a.T = temperature;
  a.c = kLog2e / temperature;
  a.mode = mode;
  a.top_n = top_n;
  a.logits = logits;
  a.G = draft_logits;
  a.drafts = draft_tokens;
  a.rowfinal = reinterpret_cast<const RowFinal*>(w + L.rowfinal);
  a.req = reinterpret_cast<const ReqState*>(w + L.req);
  a.zs = reinterpret_cast<double*>(w + L.zs);
  a.cand = reinterpret_cast<Cand*>(w + L.cand);
  a.out_len = out_len;
  a.out_token = out_token;
  a.out_prob = out_prob;
  a.flags = flags;
  return launch_score(a, stream) == hipSuccess ? JSV_OK : JSV_EHIP;
}

jsv_status jsv_anchor_replace(const jsv_lm_head* head, const void* hidden_pred,
                              const int32_t* draft_tokens, int32_t B, int32_t K,
                              int32_t* position, int32_t* token, uint32_t* flags, void* ws,
                              size_t ws_bytes, void* hip_stream) {
  int nks = 0;
  jsv_status st = check_head(head, &nks);
  if (st != JSV_OK) return st;
  st = check_block(B, K, 0.f, JSV_PROPOSAL_POINT);
  if (st != JSV_OK) return st;
  if (hidden_pred == nullptr || !aligned16(hidden_pred) || draft_tokens == nullptr ||
      position == nullptr || token == nullptr || ws == nullptr || !aligned16(ws))
    return JSV_EINVAL;
  if (ws_bytes < needed_bytes(head, B, K, 0, true)) return JSV_EWORKSPACE;
  (void)hipGetLastError();
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  const WsLayout L = ws_layout(head->vocab, B, K, 0, head->hidden, head->dtype);
  char* w = static_cast<char*>(ws);
  st = run_stats(head, nks, hidden_pred, B * (K + 1), reinterpret_cast<float*>(w + L.logits),
                 nullptr, B, K, 0.f, JSV_PROPOSAL_POINT, 1, reinterpret_cast<RowStat*>(w + L.partial),
                 reinterpret_cast<float*>(w + L.rnorm), w, stream);
  if (st != JSV_OK) return st;
  FinalArgs f = final_args(head, hidden_pred, draft_tokens, nullptr, B, K, 0.f, JSV_PROPOSAL_POINT,
                           kFinalizeAnchor, w, L);
  f.n_accepted = position;
  f.committed = token;
  f.flags = flags;
  if (f.P <= 0 || launch_rowstat(f, stream) != hipSuccess || launch_scan(f, stream) != hipSuccess)
    return JSV_EHIP;
  return JSV_OK;
}

jsv_status jsv_cache_lookup(const int32_t* n_accepted, const int32_t* committed, int32_t B,
                            int32_t K, const int32_t* out_len, const int32_t* out_token,
                            int32_t top_n, int32_t* hit_index, void* hip_stream) {
  if (B < 1 || B > 65535 || K < 1 || K > kMaxK || top_n < 1 || top_n > kMaxTopN) return JSV_EINVAL;
  if (!n_accepted || !committed || !out_len || !out_token || !hit_index) return JSV_EINVAL;
  (void)hipGetLastError();
  return launch_lookup(n_accepted, committed, B, K, out_len, out_token, top_n, hit_index,
                       static_cast<hipStream_t>(hip_stream)) == hipSuccess ? JSV_OK : JSV_EHIP;
}

jsv_status jsv_calibrated_lengths(const double* p_tilde, int32_t B, int32_t K, double* len_score,
                                  uint32_t* flags, void* hip_stream) {
  if (B < 1 || B > 65535 || K < 1 || K > kMaxK || p_tilde == nullptr || len_score == nullptr)
    return JSV_EINVAL;
  (void)hipGetLastError();
  return launch_lengths(p_tilde, B, K, len_score, flags, static_cast<hipStream_t>(hip_stream)) ==
                 hipSuccess ? JSV_OK : JSV_EHIP;
}

// Host computation: the candidates of the surrogate problem are the M most likely lengths
// for M = 1..gamma+1 (paper App. F.2, proof of Proposition 2(a)).
jsv_status jsv_geometric_fanout(double alpha, double rho, int32_t gamma, int32_t B,
                                double* F_real, int32_t* F_int, double* hit_mass) {
  if (!(alpha > 0.0 && alpha < 1.0) || !(rho > 0.0) || gamma < 1 || gamma > 64 || B < 2 ||
      B > 1000000 || F_real == nullptr || F_int == nullptr)
    return JSV_EINVAL;
  const int n = gamma + 1;
  double P[65], w[65], bestF[65];
  int order[65];
  for (int k = 0; k < n; ++k) {
    P[k] = (k < gamma) ? pow(alpha, k) * (1.0 - alpha) : pow(alpha, gamma);
    w[k] = pow(P[k], 1.0 / (1.0 + rho));
    order[k] = k;
  }
  // lengths by P descending, ties to the lower k (insertion sort: n <= 65)
  for (int i = 1; i < n; ++i) {
    const int x = order[i];
    int j = i - 1;
    while (j >= 0 && (P[order[j]] < P[x] || (P[order[j]] == P[x] && order[j] > x))) {
      order[j + 1] = order[j];
      --j;
    }
    order[j + 1] = x;
  }
  double best = -1.0;
  for (int M = 1; M <= n; ++M) {
    double F[65] = {0.0}, ws = 0.0;
    for (int i = 0; i < M; ++i) ws += w[order[i]];
    bool feasible = true;
    for (int i = 0; i < M; ++i) {
      const int k = order[i];
      F[k] = double(B) * w[k] / ws;
      if (F[k] < 1.0) feasible = false;
    }
    if (!feasible) continue;
    double obj = 0.0;
    for (int k = 0; k < n; ++k)
      if (F[k] >= 1.0) obj += P[k] * (1.0 - pow(F[k], -rho));
    if (obj > best) {
      best = obj;
      memcpy(bestF, F, sizeof(double) * n);
    }
  }
  if (best < 0.0) return JSV_EINVAL;  // unreachable for B >= 2: M = 1 gives F = B
  int total = 0;
  double rem[65];
  for (int k = 0; k < n; ++k) {
    F_real[k] = bestF[k];
    F_int[k] = int(floor(bestF[k]));
    rem[k] = bestF[k] - F_int[k];
    total += F_int[k];
  }
  for (int left = B - total; left > 0; --left) {  // largest remainders, ties to the lower k
    int kb = -1;
    for (int k = 0; k < n; ++k)
      if (rem[k] >= 0.0 && (kb < 0 || rem[k] > rem[kb])) kb = k;
    F_int[kb] += 1;
    rem[kb] = -1.0;
  }
  if (hit_mass) *hit_mass = best;
  return JSV_OK;
}

}  // extern "C"
