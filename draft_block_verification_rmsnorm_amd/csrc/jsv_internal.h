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
constexpr int kScoreSlices = 64;           // vocabulary slices per row of the scorer
constexpr int kSliceThreads = 256;
constexpr int kSampleCols = 4;             // columns per thread of the bonus sampler
constexpr int kSampleSlice = kSliceThreads * kSampleCols;  // columns per sampler slice
constexpr int kMaxB = 8;
constexpr int kMaxK = 32;
constexpr int kMaxTopN = 64;
constexpr int kScoreMaxSlice = 2048;       // columns staged in LDS by one scorer workgroup
constexpr int64_t kMaxVocab = int64_t(1) << 22;

// Per (row, LM-head workgroup) partial statistics of the logits and draft logits,
// stored row-major: partial[row * P + workgroup].
struct alignas(16) RowStat {
  double s;        // sum over this workgroup's columns of exp((z - m) / T)       (T > 0)
  double sq;       // same for the draft logits of this row (draft rows, softmax, T > 0)
  float m;         // max logit
  float top2;      // second largest logit (equal to m when the max is shared)
  float mq;        // max draft logit
  uint32_t idxf;   // argmax (lowest token id among equal maxima) in bits 0..30; bit 31 set
                   // when a non-finite logit or draft logit was seen
};
constexpr uint32_t kIdxMask = 0x7fffffffu;
constexpr uint32_t kBadBit = 0x80000000u;

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

// Float64 logit of a draft row at its draft token, and the draft logit there.
struct alignas(16) DraftLogit {
  double z;
  float g;
  int pad;
};

// Per-request result of the acceptance scan, read by the bonus sampler and scorer,
// with the statistics of row k that the residual there needs.
struct alignas(16) ReqState {
  double vk;       // bonus uniform of row k
  double s, sq;    // softmax normalisers of row k (logits, draft logits)
  float m, mq;     // maxima of row k
  int k;           // first rejection (K if none); -1 for an invalid request
  int dk;          // point-mass proposal: the draft token removed from the residual, else -1
  int use_q;       // residual max(p - q, 0) with the softmax proposal q of row k
  uint32_t flags;
};

// One top-N candidate of a (request, row, slice) of the scorer.
struct alignas(8) Cand {
  double r;        // residual value (ranking key), -1 for an empty slot
  double p;        // target probability (second key; used when the residual mass is 0)
  int tok;
  int pad;
};

__host__ __device__ inline int sample_slices(int64_t V) {
  return int((V + kSampleSlice - 1) / kSampleSlice);
}
__host__ __device__ inline int score_slices(int64_t V) {
  const int64_t need = (V + kScoreMaxSlice - 1) / kScoreMaxSlice;
  return int(need > kScoreSlices ? need : kScoreSlices);
}

struct WsLayout {
  size_t req, rowfinal, rowstat, dlog, rnorm, partial, zs, cand, xhat, planes, logits, total;
};

// LM head for more rows than one pass holds (bf16 W, 34..144 rows, d a multiple of 1024,
// at most 5120): the reduction dimension is split into blocks of 1024 columns instead of
// the rows into passes, so W is read once.  Workgroup (vocabulary chunk, block) holds
// every row's normalised states over its block, one 16-row tile per wave, and writes fp32
// partial products; a second kernel sums the blocks, writes the logits and forms the
// per-row partial statistics.
constexpr int kWideBlock = 1024;     // columns of d per block
constexpr int kWideMaxRows = 144;    // nine 16-row tiles
constexpr int kWideMaxD = 5120;      // at most five blocks
inline bool wide_eligible(int dtype, int64_t d, int M) {
  return dtype == 0 /* JSV_BF16 */ && M > kRowsPerPass && M <= kWideMaxRows &&
         d % kWideBlock == 0 && d <= kWideMaxD;
}
struct WidePlan {
  int nw;      // waves (tiles) of the product kernel: 8 or 9
  int mp;      // rows of a partial plane: M rounded up to whole tiles
  int S;       // blocks of d
  int nchunk;  // vocabulary chunks of the product kernel
  int ncomb;   // column chunks of the combine kernel (= partial statistics per row)
};
inline WidePlan plan_wide(int64_t V, int64_t d, int M, int cus) {
  WidePlan p{};
  p.nw = M <= 128 ? 8 : 9;  // eight waves move the eight quarters of a W group
  p.mp = 16 * ((M + 15) / 16);
  p.S = int(d / kWideBlock);
  const int64_t ngroups = (V + 15) / 16;
  int64_t nc = (cus > 0 ? cus : 1) / p.S;
  if (nc < 1) nc = 1;
  if (nc > ngroups) nc = ngroups;
  p.nchunk = int(nc);
  // combine: (column chunks) x (row groups) workgroups of 256 threads, about four per CU
  int64_t cb = (4 * int64_t(cus) + (M + 15) / 16 - 1) / ((M + 15) / 16);
  if (cb > kMaxGrid) cb = kMaxGrid;
  const int64_t ntiles = (V + 63) / 64;
  if (cb > ntiles) cb = ntiles;
  p.ncomb = int(cb > 0 ? cb : 1);
  return p;
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace carve-up for B requests of K drafts over vocabulary V, top_n outcomes.
inline WsLayout ws_layout(int64_t V, int B, int K, int top_n, int64_t d, int dtype) {
  const size_t M = size_t(B) * size_t(K + 1);
  WsLayout L{};
  size_t off = 0;
  L.req = off;      off = align256(off + kMaxB * sizeof(ReqState));
  L.rowfinal = off; off = align256(off + M * sizeof(RowFinal));
  L.rowstat = off;  off = align256(off + M * sizeof(RowStat));
  L.dlog = off;     off = align256(off + M * sizeof(DraftLogit));
  L.rnorm = off;    off = align256(off + M * sizeof(float));
  L.partial = off;  off = align256(off + size_t(kMaxGrid) * M * sizeof(RowStat));
  // Wide LM head only; before the sections whose size depends on top_n.
  const bool wide = wide_eligible(dtype, d, int(M));
  const WidePlan wp = plan_wide(V, d > 0 ? d : kWideBlock, int(M), 1);
  L.xhat = off;     off = align256(off + (wide ? M * size_t(d) * 2 : 0));
  L.planes = off;   off = align256(off + (wide ? size_t(wp.S) * size_t((V + 3) & ~int64_t(3)) * size_t(wp.mp) * 4 : 0));
  const size_t zs_sample = size_t(B) * size_t(sample_slices(V)) * 2 * sizeof(double);
  const size_t zs_score = M * size_t(score_slices(V)) * sizeof(double);
  L.zs = off;       off = align256(off + (zs_sample > zs_score ? zs_sample : zs_score));
  L.cand = off;     off = align256(off + M * size_t(score_slices(V)) * size_t(top_n + 1) * sizeof(Cand));
  L.logits = off;   off = align256(off + M * size_t(V) * sizeof(float));
  L.total = off;
  return L;
}

// Fused RMSNorm + LM head + statistics of M rows in one launch of nchunk * npass
// workgroups: the rows are split into npass passes of rp rows (rp <= kRowsPerPass) and
// the vocabulary into nchunk chunks.
struct StatsArgs {
  const void* W;          // [V][d]
  const float* wscale;    // [V] row scales of an fp8 head, else null
  const void* gamma;      // [d]
  const void* hidden;     // [M][d]
  int64_t V;
  int d;
  int rp, npass, nchunk;  // rows per pass, passes, vocabulary chunks
  int M;                  // total rows
  float eps;
  float* logits;          // [M][V]
  const float* G;         // [B][K][V] draft logits, or null
  int B, K;               // block structure (K = -1: plain rows, no statistics)
  float T, c;             // temperature and log2(e) / T
  int stats;              // write per-row partial statistics
  int want_q;             // also draft-logit statistics (softmax proposal, T > 0)
  RowStat* partial;       // [M][nchunk]
  float* rnorm;           // [M] RMSNorm factor of every row (written by workgroup 0), or null
};

// Launch plan of the LM-head kernel for M <= 8 * kRowsPerPass rows: the fewest passes
// (a power of two, so that the passes of a chunk share an XCD) and as many vocabulary
// chunks as leave one workgroup per compute unit.
struct StatsPlan {
  int npass, rp, nchunk;
};
inline StatsPlan plan_stats(int64_t V, int M, int cus) {
  StatsPlan p{1, M, 1};
  while ((M + p.npass - 1) / p.npass > kRowsPerPass) p.npass *= 2;
  p.rp = (M + p.npass - 1) / p.npass;
  int64_t base = cus < kMaxGrid ? cus : kMaxGrid;
  const int64_t ngroups = (V + 15) / 16;
  if (base > ngroups) base = ngroups;
  p.nchunk = int(base / p.npass > 0 ? base / p.npass : 1);
  return p;
}
constexpr int kMaxPlanRows = 8 * kRowsPerPass;  // verification and scoring: B (K + 1) <= 264

enum FinalizeKind { kFinalizeVerify = 1, kFinalizeScore = 2, kFinalizeAnchor = 3 };

// Finalize, in two launches: per-row tasks (combine the partials of a row; the exact
// logit of a draft row at its draft token) over a grid of one-wave workgroups, then per
// request the acceptance scan (verify) or the outcome marginals (score).
struct FinalArgs {
  const void* W;
  const float* wscale;    // [V] row scales of an fp8 head, else null
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
  int P;                  // partial records per row (LM-head workgroups)
  const RowStat* partial; // [M][P]
  RowStat* rowstat;       // [M] combined statistics
  DraftLogit* dlog;       // [M] (rows < K of each request)
  const float* rnorm;
  int* n_accepted;         // verify: k; anchor replacement: the position
  int* committed;          // verify: committed tokens; anchor replacement: the token [B]
  uint32_t* flags;        // may be null
  RowFinal* rowfinal;
  ReqState* req;
  int top_n;
  int* out_len;
  int* out_token;
  float* out_prob;
  double* len_marginal;   // may be null
};

// Bonus sampler (T > 0 verification): both kernels run the acceptance scan of `f`
// themselves, so the scan needs no launch of its own on this path.
struct SampleArgs {
  FinalArgs f;
  float c;                // log2(e) / T
  const float* logits;
  const float* G;
  double* zs;             // [B][slices][2]
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

// The wide LM head (see wide_eligible): three launches on `stream`.
struct WideArgs {
  const void* W;          // [V][d] bf16
  const void* gamma;      // [d]
  const void* hidden;     // [M][d]
  int64_t V;
  int d, M;
  float eps;
  WidePlan pl;
  uint16_t* xhat;         // [M][d] normalised rows (workspace)
  float* planes;          // [S][mp / 16][16][V rounded up to 4] partial products (workspace)
  float* rnorm;           // [M]
  float* logits;          // [M][V]
  const float* G;         // [B][K][V] draft logits, or null
  int B, K;
  float T, c;             // temperature and log2(e) / T
  int want_q;
  int quad;               // V % 4 == 0 and logits, G 16-byte aligned: 16-byte accesses
  RowStat* partial;       // [M][ncomb]
};
hipError_t launch_wide(const WideArgs& a, hipStream_t stream);
hipError_t launch_rowstat(const FinalArgs& a, hipStream_t stream);
hipError_t launch_scan(const FinalArgs& a, hipStream_t stream);
hipError_t launch_sample(const SampleArgs& a, hipStream_t stream);
hipError_t launch_score(const ScoreArgs& a, hipStream_t stream);
hipError_t launch_lookup(const int* n_accepted, const int* committed, int B, int K, const int* out_len,
                         const int* out_token, int top_n, int* hit, hipStream_t stream);
hipError_t launch_lengths(const double* p, int B, int K, double* out, uint32_t* flags,
                          hipStream_t stream);

}  // namespace jsv
