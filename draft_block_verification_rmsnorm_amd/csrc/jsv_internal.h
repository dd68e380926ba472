// Internal declarations shared by the host API (jsv_api.hip) and the kernels
// (jsv_kernels.hip) of libjsverify.  Not installed; the public ABI is include/jsverify.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace jsv {

constexpr int kWave = 64;
constexpr int kWaves = 8;                  // waves per workgroup of the LM-head kernel
constexpr int kThreads = kWaves * kWave;   // 512
constexpr int kRowsPerPass = 33;           // two 16-token MFMA tiles + one VALU row per pass over W
constexpr int kMaxGrid = 1024;             // LM-head workgroups (= partial records per row)
constexpr int kSampleSlices = 64;          // vocabulary slices of the bonus sampler
constexpr int kScoreSlices = 64;           // vocabulary slices per row of the scorer
constexpr int kSliceThreads = 256;
constexpr int kMaxB = 8;
constexpr int kMaxK = 32;
constexpr int kMaxTopN = 64;
constexpr int kSampleMaxSlice = 4096;      // columns staged in LDS by one sampler workgroup
constexpr int kScoreMaxSlice = 2048;       // columns staged in LDS by one scorer workgroup
constexpr int64_t kMaxVocab = int64_t(1) << 22;

// Per (LM-head workgroup, row) partial statistics of the logits and draft logits.
struct alignas(16) RowStat {
  double s;        // sum over this workgroup's columns of exp((z - m) / T)       (T > 0)
  double sq;       // same for the draft logits of this row (draft rows, softmax, T > 0)
  float m;         // max logit
  float top2;      // second largest logit (equal to m when the max is shared)
  float mq;        // max draft logit
  int idx;         // argmax, lowest token id among equal maxima
  uint32_t flags;  // JSV_FLAG_INVALID when a non-finite logit or draft logit was seen
  int pad[3];
};

// Per-row statistics after combining every workgroup's partial.
struct alignas(16) RowFinal {
  double s, sq;    // softmax normalisers of logits and draft logits
  double alpha;    // acceptance probability of this row's draft token (rows < K)
  double A;        // probability that verification reaches this row (A_0 = 1)
  float m, top2, mq;
  int idx;
  uint32_t flags;
  int pad[3];
};

// Per-request result of the acceptance scan, read by the bonus sampler and scorer.
struct alignas(16) ReqState {
  double vk;       // bonus uniform of row k
  int k;           // first rejection (K if none); -1 for an invalid request
  uint32_t flags;
  int pad[4];
};

// One top-N candidate of a (request, row, slice) of the scorer.
struct alignas(8) Cand {
  double r;        // residual value (ranking key), -1 for an empty slot
  double p;        // target probability (second key; used when the residual mass is 0)
  int tok;
  int pad;
};

__host__ __device__ inline int sample_slices(int64_t V) {
  const int64_t need = (V + kSampleMaxSlice - 1) / kSampleMaxSlice;
  return int(need > kSampleSlices ? need : kSampleSlices);
}
__host__ __device__ inline int score_slices(int64_t V) {
  const int64_t need = (V + kScoreMaxSlice - 1) / kScoreMaxSlice;
  return int(need > kScoreSlices ? need : kScoreSlices);
}

struct WsLayout {
  size_t req, rowfinal, rnorm, partial, zs, cand, logits, total;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace carve-up for B requests of K drafts over vocabulary V, top_n outcomes.
inline WsLayout ws_layout(int64_t V, int B, int K, int top_n) {
  const size_t M = size_t(B) * size_t(K + 1);
  WsLayout L{};
  size_t off = 0;
  L.req = off;      off = align256(off + kMaxB * sizeof(ReqState));
  L.rowfinal = off; off = align256(off + M * sizeof(RowFinal));
  L.rnorm = off;    off = align256(off + M * sizeof(float));
  L.partial = off;  off = align256(off + size_t(kMaxGrid) * M * sizeof(RowStat));
  const size_t zs_sample = size_t(B) * size_t(sample_slices(V)) * 2 * sizeof(double);
  const size_t zs_score = M * size_t(score_slices(V)) * sizeof(double);
  L.zs = off;       off = align256(off + (zs_sample > zs_score ? zs_sample : zs_score));
  L.cand = off;     off = align256(off + M * size_t(score_slices(V)) * size_t(top_n + 1) * sizeof(Cand));
  L.logits = off;   off = align256(off + M * size_t(V) * sizeof(float));
  L.total = off;
  return L;
}

// Fused RMSNorm + LM head + statistics, one pass over W for rows [row0, row0 + rows).
struct StatsArgs {
  const void* W;          // [V][d]
  const void* gamma;      // [d]
  const void* hidden;     // [M][d]
  int64_t V;
  int d;
  int row0, rows;         // rows handled by this pass (rows <= kRowsPerPass)
  int M;                  // total rows
  float eps;
  float* logits;          // [M][V]
  const float* G;         // [B][K][V] draft logits, or null
  int B, K;               // block structure (K = -1: plain rows, no statistics)
  float T, c;             // temperature and log2(e) / T
  int stats;              // write per-row partial statistics
  int want_q;             // also draft-logit statistics (softmax proposal, T > 0)
  RowStat* partial;       // [gridDim][M]
  float* rnorm;           // [M] RMSNorm factor of every row (written by workgroup 0), or null
};

enum FinalizeKind { kFinalizeVerify = 1, kFinalizeScore = 2 };

// Combine the partials of a request, then the acceptance scan (verify) or the outcome
// marginals (score).  One workgroup per request.
struct FinalArgs {
  const void* W;
  const void* gamma;
  const void* hidden;
  int64_t V;
  int d;
  int dtype;
  const float* G;
  const int* drafts;
  int B, K;
  float T;
  int mode;
  int kind;               // FinalizeKind
  uint64_t seed, offset;
  int P;                  // partial records per row
  const RowStat* partial;
  const float* rnorm;
  int* n_accepted;
  int* committed;
  uint32_t* flags;        // may be null
  RowFinal* rowfinal;
  ReqState* req;
  int top_n;
  int* out_len;
  int* out_token;
  float* out_prob;
  double* len_marginal;   // may be null
};

struct SampleArgs {
  int64_t V;
  int B, K;
  float T, c;
  int mode;
  const float* logits;
  const float* G;
  const int* drafts;
  const RowFinal* rowfinal;
  const ReqState* req;
  double* zs;             // [B][slices][2]
  int* committed;
  uint32_t* flags;        // may be null
};

struct ScoreArgs {
  int64_t V;
  int B, K;
  float T, c;
  int mode;
  int top_n;
  const float* logits;
  const float* G;
  const int* drafts;
  const RowFinal* rowfinal;
  const ReqState* req;
  double* zs;             // [B][K+1][slices]
  Cand* cand;             // [B][K+1][slices][top_n+1]
  int* out_len;
  int* out_token;
  float* out_prob;
  uint32_t* flags;        // may be null
};

// Host-side launchers (jsv_kernels.hip).  Return hipSuccess or the launch error.
// `nks` is hidden / (kWaves * elements per k-step); the launcher picks the instance.
bool stats_supported(int dtype, int nks);
hipError_t launch_stats(int dtype, int nks, int grid, const StatsArgs& a, hipStream_t stream);
hipError_t launch_finalize(const FinalArgs& a, hipStream_t stream);
hipError_t launch_sample(const SampleArgs& a, hipStream_t stream);
hipError_t launch_score(const ScoreArgs& a, hipStream_t stream);

}  // namespace jsv
