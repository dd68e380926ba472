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

int k_per_step(int dtype) { return dtype == JSV_BF16 ? 32 : 16; }

// Validates the head; on success *nks is hidden / (waves * k per MFMA step).
jsv_status check_head(const jsv_lm_head* h, int* nks) {
  if (h == nullptr || h->weight == nullptr || h->norm_weight == nullptr) return JSV_EINVAL;
  if (h->dtype != JSV_BF16 && h->dtype != JSV_F32) return JSV_EINVAL;
  if (h->vocab < 1 || h->hidden < 1) return JSV_EINVAL;
  if (!(h->eps >= 0.f) || !isfinite(h->eps)) return JSV_EINVAL;
  if (!aligned16(h->weight) || !aligned16(h->norm_weight)) return JSV_EINVAL;
  if (h->vocab > INT32_MAX) return JSV_EUNSUPPORTED;
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

struct StatsCall {
  const jsv_lm_head* head;
  int nks;
  const void* hidden;
  int M;
  float* logits;
  const float* G;
  const int32_t* drafts;
  int B, K;
  float T;
  int mode;
  int stats;
  int finalize;
  uint64_t seed, offset;
  int32_t* n_accepted;
  int32_t* committed;
  uint32_t* flags;
  int top_n;
  int32_t* out_len;
  int32_t* out_token;
  float* out_prob;
  double* len_marginal;
  char* ws;
  WsLayout L;
};

jsv_status run_stats(const StatsCall& c, hipStream_t stream) {
  const int64_t V = c.head->vocab;
  const int64_t ngroups = (V + 15) / 16;
  const int cus = device_cu_count();
  if (cus <= 0) return JSV_EHIP;
  int64_t grid = cus < kMaxGrid ? cus : kMaxGrid;
  if (grid > ngroups) grid = ngroups;

  StatsArgs a{};
  a.W = c.head->weight;
  a.gamma = c.head->norm_weight;
  a.hidden = c.hidden;
  a.V = V;
  a.d = int(c.head->hidden);
  a.M = c.M;
  a.eps = c.head->eps;
  a.logits = c.logits;
  a.G = c.G;
  a.drafts = c.drafts;
  a.B = c.B;
  a.K = c.K;
  a.T = c.T;
  a.c = c.T > 0.f ? kLog2e / c.T : 0.f;
  a.stats = c.stats;
  a.want_q = (c.stats && c.mode == JSV_PROPOSAL_SOFTMAX && c.T > 0.f && c.G != nullptr) ? 1 : 0;
  a.mode = c.mode;
  a.seed = c.seed;
  a.offset = c.offset;
  a.n_accepted = c.n_accepted;
  a.committed = c.committed;
  a.flags = c.flags;
  a.top_n = c.top_n;
  a.out_len = c.out_len;
  a.out_token = c.out_token;
  a.out_prob = c.out_prob;
  a.len_marginal = c.len_marginal;
  if (c.ws != nullptr) {
    a.counter = reinterpret_cast<uint32_t*>(c.ws + c.L.counters);
    a.req = reinterpret_cast<ReqState*>(c.ws + c.L.req);
    a.rowfinal = reinterpret_cast<RowFinal*>(c.ws + c.L.rowfinal);
    a.zd = reinterpret_cast<double*>(c.ws + c.L.zd);
    a.partial = reinterpret_cast<RowStat*>(c.ws + c.L.partial);
  }
  for (int row0 = 0; row0 < c.M; row0 += kRowsPerPass) {
    a.row0 = row0;
    a.rows = (c.M - row0) < kRowsPerPass ? (c.M - row0) : kRowsPerPass;
    a.finalize = (row0 + kRowsPerPass >= c.M) ? c.finalize : kFinalizeNone;
    if (launch_stats(c.head->dtype, c.nks, a.rows, int(grid), a, stream) != hipSuccess) return JSV_EHIP;
  }
  return JSV_OK;
}

size_t needed_bytes(int64_t V, int B, int K, int top_n, bool logits_in_ws) {
  const WsLayout L = ws_layout(V, B, K, top_n);
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
  return needed_bytes(head->vocab, batch, K, top_n, true);
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
  StatsCall c{};
  c.head = head; c.nks = nks; c.hidden = hidden; c.M = int(rows); c.logits = logits;
  c.K = -1; c.B = 0; c.T = 0.f; c.stats = 0; c.finalize = kFinalizeNone; c.ws = nullptr;
  return run_stats(c, static_cast<hipStream_t>(hip_stream));
}

static jsv_status verify_prepare(const jsv_lm_head* head, const void* hidden,
                                 const int32_t* draft_tokens, const float* draft_logits,
                                 int32_t B, int32_t K, float T, int32_t mode, int32_t* n_accepted,
                                 int32_t* committed, const float* logits_out, void* ws,
                                 size_t ws_bytes, int* nks, bool need_hidden) {
  jsv_status st = check_head(head, nks);
  if (st != JSV_OK) return st;
  st = check_block(B, K, T, mode);
  if (st != JSV_OK) return st;
  if (need_hidden && (hidden == nullptr || !aligned16(hidden))) return JSV_EINVAL;
  if (draft_tokens == nullptr || committed == nullptr || ws == nullptr) return JSV_EINVAL;
  if (need_hidden && n_accepted == nullptr) return JSV_EINVAL;
  if (mode == JSV_PROPOSAL_SOFTMAX && T > 0.f && draft_logits == nullptr) return JSV_EINVAL;
  if (!aligned16(ws)) return JSV_EINVAL;
  if (ws_bytes < needed_bytes(head->vocab, B, K, 0, logits_out == nullptr)) return JSV_EWORKSPACE;
  return JSV_OK;
}

jsv_status jsv_verify_stats(const jsv_lm_head* head, const void* hidden,
                            const int32_t* draft_tokens, const float* draft_logits, int32_t B,
                            int32_t K, float temperature, int32_t mode, uint64_t seed,
                            uint64_t offset, int32_t* n_accepted, int32_t* committed,
                            uint32_t* flags, float* logits_out, void* ws, size_t ws_bytes,
                            void* hip_stream) {
  int nks = 0;
  jsv_status st = verify_prepare(head, hidden, draft_tokens, draft_logits, B, K, temperature, mode,
                                 n_accepted, committed, logits_out, ws, ws_bytes, &nks, true);
  if (st != JSV_OK) return st;
  (void)hipGetLastError();
  StatsCall c{};
  c.head = head; c.nks = nks; c.hidden = hidden; c.M = B * (K + 1);
  c.L = ws_layout(head->vocab, B, K, 0);
  c.ws = static_cast<char*>(ws);
  c.logits = logits_out ? logits_out : reinterpret_cast<float*>(c.ws + c.L.logits);
  c.G = draft_logits; c.drafts = draft_tokens; c.B = B; c.K = K; c.T = temperature; c.mode = mode;
  c.stats = 1; c.finalize = kFinalizeVerify; c.seed = seed; c.offset = offset;
  c.n_accepted = n_accepted; c.committed = committed; c.flags = flags;
  return run_stats(c, static_cast<hipStream_t>(hip_stream));
}

jsv_status jsv_verify_sample(const jsv_lm_head* head, const int32_t* draft_tokens,
                             const float* draft_logits, int32_t B, int32_t K, float temperature,
                             int32_t mode, int32_t* committed, uint32_t* flags,
                             const float* logits_out, void* ws, size_t ws_bytes,
                             void* hip_stream) {
  int nks = 0;
  jsv_status st = verify_prepare(head, nullptr, draft_tokens, draft_logits, B, K, temperature, mode,
                                 nullptr, committed, logits_out, ws, ws_bytes, &nks, false);
  if (st != JSV_OK) return st;
  if (!(temperature > 0.f)) return JSV_OK;  // greedy: the bonus is the argmax, already written
  (void)hipGetLastError();
  const WsLayout L = ws_layout(head->vocab, B, K, 0);
  char* w = static_cast<char*>(ws);
  SampleArgs a{};
  a.V = head->vocab;
  a.B = B;
  a.K = K;
  a.T = temperature;
  a.c = kLog2e / temperature;
  a.mode = mode;
  a.logits = logits_out ? logits_out : reinterpret_cast<const float*>(w + L.logits);
  a.G = draft_logits;
  a.drafts = draft_tokens;
  a.rowfinal = reinterpret_cast<const RowFinal*>(w + L.rowfinal);
  a.req = reinterpret_cast<const ReqState*>(w + L.req);
  a.zs = reinterpret_cast<double*>(w + L.zs);
  a.counter = reinterpret_cast<uint32_t*>(w + L.counters) + 8;
  a.committed = committed;
  a.flags = flags;
  return launch_sample(a, static_cast<hipStream_t>(hip_stream)) == hipSuccess ? JSV_OK : JSV_EHIP;
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
  return jsv_verify_sample(head, draft_tokens, draft_logits, B, K, temperature, mode, committed,
                           flags, logits_out, ws, ws_bytes, hip_stream);
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
  if (ws_bytes < needed_bytes(head->vocab, B, K, top_n, true)) return JSV_EWORKSPACE;
  (void)hipGetLastError();
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  StatsCall c{};
  c.head = head; c.nks = nks; c.hidden = hidden_pred; c.M = B * (K + 1);
  c.L = ws_layout(head->vocab, B, K, top_n);
  c.ws = static_cast<char*>(ws);
  c.logits = reinterpret_cast<float*>(c.ws + c.L.logits);
  c.G = draft_logits; c.drafts = draft_tokens; c.B = B; c.K = K; c.T = temperature; c.mode = mode;
  c.stats = 1; c.finalize = kFinalizeScore;
  c.flags = flags; c.top_n = top_n; c.out_len = out_len; c.out_token = out_token;
  c.out_prob = out_prob; c.len_marginal = len_marginal;
  st = run_stats(c, stream);
  if (st != JSV_OK || !(temperature > 0.f)) return st;
  ScoreArgs a{};
  a.V = head->vocab;
  a.B = B;
  a.K = K;
  a.T = temperature;
  a.c = kLog2e / temperature;
  a.mode = mode;
  a.top_n = top_n;
  a.logits = c.logits;
  a.G = draft_logits;
  a.drafts = draft_tokens;
  a.rowfinal = reinterpret_cast<const RowFinal*>(c.ws + c.L.rowfinal);
  a.req = reinterpret_cast<const ReqState*>(c.ws + c.L.req);
  a.zs = reinterpret_cast<double*>(c.ws + c.L.zs);
  a.cand = reinterpret_cast<Cand*>(c.ws + c.L.cand);
  a.counter = reinterpret_cast<uint32_t*>(c.ws + c.L.counters) + 16;
  a.out_len = out_len;
  a.out_token = out_token;
  a.out_prob = out_prob;
  a.flags = flags;
  return launch_score(a, stream) == hipSuccess ? JSV_OK : JSV_EHIP;
}

}  // extern "C"
