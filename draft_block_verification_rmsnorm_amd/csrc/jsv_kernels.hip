// HIP kernels of libjsverify for gfx950 (MI355X).
//
//   stats_kernel     fused final RMSNorm + LM head (bf16 MFMA 16x16x32, or f32 MFMA
//                    16x16x4) whose epilogue writes the logits and per-row online softmax
//                    statistics of its vocabulary range (JetSpec++ paper §4.2 "Decoder").
//   rowstat_kernel   per row: combine the partial statistics, and the exact logit at
//                    each draft token (one wave per task, spread over the chip).
//   scan_kernel      per request: the acceptance scan (paper §3, App. F.3) or the
//                    outcome marginals (§4.2 Eq. 6).
//   slice_sum_kernel / locate_kernel
//                    bonus token by inverse CDF over the residual of the rejected row
//                    (§3): residual mass per vocabulary slice, then the CDF step.
//   score_slice_kernel / score_merge_kernel
//                    residual mass and top-(N+1) columns per (row, slice), then the top-N
//                    outcomes of the request (§4.2 Eq. 7, App. B.1).
// Kernels hand results to each other only through kernel boundaries on one stream.
#include <float.h>
#include <limits.h>
#include <math.h>

#include "jsv_internal.h"
#include "jsverify.h"

namespace jsv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr double kAcceptTie = 1e-4;
constexpr float kLogitGapTie = 1e-3f;
constexpr double kCdfTie = 1e-8;  // absolute, in probability mass (C and t are unnormalised)
constexpr double kTopNTie = 1e-3;
constexpr double kLog2eD = 1.4426950408889634074;
constexpr uint32_t kOutOfRange = 0x80000000u;  // buffer offset past every resource used here
constexpr int kRsrcWord3 = 0x00020000;         // raw 32-bit-element buffer, gfx9 family

// ------------------------------------------------------------------------------------
// Philox4x32-10, from the SC'11 paper by Salmon, Moraes, Dror and Shaw.
// Counter (row i, request b, lo32(offset), hi32(offset)), key (lo32(seed), hi32(seed)).
__device__ inline void philox4x32_10(uint32_t ctr[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t lo0 = 0xD2511F53u * ctr[0], hi0 = __umulhi(0xD2511F53u, ctr[0]);
    const uint32_t lo1 = 0xCD9E8D57u * ctr[2], hi1 = __umulhi(0xCD9E8D57u, ctr[2]);
    const uint32_t n0 = hi1 ^ ctr[1] ^ k0;
    const uint32_t n2 = hi0 ^ ctr[3] ^ k1;
    ctr[0] = n0; ctr[1] = lo1; ctr[2] = n2; ctr[3] = lo0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
}

// u: acceptance uniform (x0 / 2^32); v: bonus uniform with 53 random bits.
__device__ inline void row_uniforms(uint64_t seed, uint64_t offset, int b, int i, double& u,
                                    double& v) {
  uint32_t c[4] = {uint32_t(i), uint32_t(b), uint32_t(offset), uint32_t(offset >> 32)};
  philox4x32_10(c, uint32_t(seed), uint32_t(seed >> 32));
  u = double(c[0]) * 0x1p-32;
  v = double((uint64_t(c[1]) << 21) | uint64_t(c[2] >> 11)) * 0x1p-53;
}

// ------------------------------------------------------------------------------------
// Memory helpers.  Buffer accesses past num_records return zero (loads) or are dropped
// (stores), so the streaming loops need no branches around their memory operations.
__device__ inline rsrc_t make_rsrc(const void* base, uint64_t bytes) {
  const uint32_t n = bytes > 0xffffffffull ? 0xffffffffu : uint32_t(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, kRsrcWord3);
}
__device__ inline uint4 bload16(rsrc_t r, uint32_t voff, uint32_t soff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
// The 32-bit buffer builtins move integer words: floats cross them as bit patterns.
__device__ inline float bload4f(rsrc_t r, uint32_t voff) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, 0, 0));
}
__device__ inline void bstore4f(float x, rsrc_t r, uint32_t voff) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, (int)voff, 0, 0);
}
__device__ inline void bstore16(const uint4& x, rsrc_t r, uint32_t voff) {
  __builtin_amdgcn_raw_buffer_store_b128(u32x4{x.x, x.y, x.z, x.w}, r, (int)voff, 0, 0);
}
// Same, marked non-temporal (streaming data the writer does not read again).
__device__ inline void bstore4f_nt(float x, rsrc_t r, uint32_t voff) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, (int)voff, 0, 2);
}

// Loads from a buffer straight into LDS.  The lanes' data land lane-linearly at the LDS
// byte address `lds` (wave-uniform), whatever addresses the lanes read; completion is
// counted by vmcnt.  They are written as inline assembly on purpose: the compiler then
// never sees LDS written by DMA, so it adds no wait-for-everything before each LDS read
// or barrier, and the kernel waits for exactly the loads it needs (waits below).  The
// descriptor is a raw buffer in SGPRs; the offset is range-checked (zeros past the end).
struct Srd { u32x4 v; };
__device__ inline Srd make_srd(const void* base, uint64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  Srd r;
  r.v.x = __builtin_amdgcn_readfirstlane(uint32_t(a));
  r.v.y = __builtin_amdgcn_readfirstlane(uint32_t(a >> 32) & 0xffffu);
  r.v.z = __builtin_amdgcn_readfirstlane(bytes > 0xffffffffull ? 0xffffffffu : uint32_t(bytes));
  r.v.w = uint32_t(kRsrcWord3);
  return r;
}
__device__ inline uint32_t lds_addr(const void* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_readfirstlane(
      uint32_t(uintptr_t((const __attribute__((address_space(3))) char*)p)));
#else
  (void)p;
  return 0;
#endif
}
// m0 is listed as clobbered although the compiler reserves it: none of these kernels uses
// m0 otherwise (gfx9 LDS instructions do not read it).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16 bytes per lane (1 KB per wave), non-temporal.
__device__ inline void dma16_nt(Srd r, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
               ::"s"(lds), "v"(voff), "s"(r.v) : "memory", "m0");
}
// 4 bytes per lane (256 B per wave).
__device__ inline void dma4(Srd r, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               ::"s"(lds), "v"(voff), "s"(r.v) : "memory", "m0");
}
#pragma clang diagnostic pop
// Waits that also order the compiler's memory accesses around them.
template <int N>
__device__ inline void wait_vmcnt() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }
__device__ inline void wait_lgkmcnt0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ inline double u2d(uint32_t lo, uint32_t hi) {
  return __builtin_bit_cast(double, (uint64_t(hi) << 32) | uint64_t(lo));
}

// ------------------------------------------------------------------------------------
// Cross-lane moves on the DPP path (a VALU operand modifier, no LDS round trip), and
// lane reads into scalar registers for wave-uniform lane indices.
//   0xB1 / 0x4E   quad_perm [1,0,3,2] / [2,3,0,1]   (lane ^ 1, lane ^ 2)
//   0x111..0x118  row_shr:1..8                     (within 16-lane rows)
//   0x124, 0x128  row_ror:4, row_ror:8
//   0x142, 0x143  row_bcast:15, row_bcast:31       (last lane of a row into later rows)
// Lanes whose source is outside the pattern, or whose row is masked off, read zero.
template <int CTRL, int ROWS = 0xf>
__device__ inline uint32_t dpp32(uint32_t x) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(x), CTRL, ROWS, 0xf, false));
}
template <int CTRL, int ROWS = 0xf>
__device__ inline float dppf(float x) {
  return __uint_as_float(dpp32<CTRL, ROWS>(__float_as_uint(x)));
}
template <int CTRL, int ROWS = 0xf>
__device__ inline double dppd(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint64_t lo = dpp32<CTRL, ROWS>(uint32_t(u)), hi = dpp32<CTRL, ROWS>(uint32_t(u >> 32));
  return __builtin_bit_cast(double, (hi << 32) | lo);
}
__device__ inline float readlane_f(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
__device__ inline int readlane_i(int x, int l) { return __builtin_amdgcn_readlane(x, l); }
__device__ inline double readlane_d(double x, int l) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint64_t lo = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(u)), l));
  const uint64_t hi = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(u >> 32)), l));
  return __builtin_bit_cast(double, (hi << 32) | lo);
}

// Inclusive prefix sum over the 64 lanes of a wave: row shifts, then row broadcasts.
__device__ inline double wave_incl_scan(double x) {
  x += dppd<0x111>(x);
  x += dppd<0x112>(x);
  x += dppd<0x114>(x);
  x += dppd<0x118>(x);
  x += dppd<0x142, 0xa>(x);
  x += dppd<0x143, 0xc>(x);
  return x;
}
// Sum over the 64 lanes (the last lane of the inclusive scan), in every lane.
__device__ inline double wave_sum(double x) { return readlane_d(wave_incl_scan(x), kWave - 1); }

// Lane l receives the sum of lanes l mod 16 + 16 i, i = 0..3 (the four 16-lane rows, in
// the order (r0 + r1) + (r2 + r3)), through gfx950's row-swapping permlanes.
__device__ inline uint2 swap16(uint32_t x) {
  const auto v = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return make_uint2(v[0], v[1]);
}
__device__ inline uint2 swap32(uint32_t x) {
  const auto v = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return make_uint2(v[0], v[1]);
}
__device__ inline float rows_sum(float y) {
  const uint2 a = swap16(__float_as_uint(y));
  const float z = __uint_as_float(a.x) + __uint_as_float(a.y);
  const uint2 b = swap32(__float_as_uint(z));
  return __uint_as_float(b.x) + __uint_as_float(b.y);
}
__device__ inline double rows_sum(double y) {
  const uint64_t u = __builtin_bit_cast(uint64_t, y);
  const uint2 lo = swap16(uint32_t(u)), hi = swap16(uint32_t(u >> 32));
  const double z = u2d(lo.x, hi.x) + u2d(lo.y, hi.y);
  const uint64_t w = __builtin_bit_cast(uint64_t, z);
  const uint2 lo2 = swap32(uint32_t(w)), hi2 = swap32(uint32_t(w >> 32));
  return u2d(lo2.x, hi2.x) + u2d(lo2.y, hi2.y);
}

// ------------------------------------------------------------------------------------
// Element helpers.
__device__ inline float bf16_to_f32(uint32_t h16) { return __uint_as_float(h16 << 16); }

// Two floats to packed bf16, round to nearest even (v_cvt_pk_bf16_f32; NaN stays NaN).
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  const floatx2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

template <int DT> struct Elem;
template <> struct Elem<JSV_BF16> { static constexpr int EPL = 8, ESZ = 2; };
template <> struct Elem<JSV_F32> { static constexpr int EPL = 4, ESZ = 4; };
// Element type of the hidden states, gamma and the normalised rows: an fp8 head keeps
// them in bf16 (weight-only quantisation).
template <int DT> struct Act { static constexpr int value = DT == JSV_FP8 ? JSV_BF16 : DT; };

// W operand of MFMA k-step half h from a 16-byte W load: unchanged for bf16 and f32; for
// an fp8 head the load holds 16 E4M3 codes, of which half h (8 codes) is widened to bf16
// (exact: every E4M3 value is a bf16 value) with v_cvt_scalef32_pk_bf16_fp8.
template <bool HI>
__device__ inline uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
template <int DT>
__device__ inline uint4 wfrag(const uint4& f, int h) {
  if constexpr (DT == JSV_FP8) {
    const uint32_t w0 = h ? f.z : f.x, w1 = h ? f.w : f.y;
    return make_uint4(fp8x2_to_bf16x2<false>(w0), fp8x2_to_bf16x2<true>(w0),
                      fp8x2_to_bf16x2<false>(w1), fp8x2_to_bf16x2<true>(w1));
  } else {
    return f;
  }
}

template <int DT>
__device__ inline void unpack(const uint4& q, float* x) {
  if constexpr (DT == JSV_BF16) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = bf16_to_f32(w[e] & 0xffffu);
      x[2 * e + 1] = bf16_to_f32(w[e] >> 16);
    }
  } else {
    x[0] = __uint_as_float(q.x); x[1] = __uint_as_float(q.y);
    x[2] = __uint_as_float(q.z); x[3] = __uint_as_float(q.w);
  }
}

// Sum of squares of one 16-byte group, in float64 (exact for bf16 inputs).
template <int DT>
__device__ inline double sumsq16(const uint4& q) {
  constexpr int EPL = Elem<DT>::EPL;
  float x[EPL];
  unpack<DT>(q, x);
  double s = 0.0;
#pragma unroll
  for (int e = 0; e < EPL; ++e) s = fma(double(x[e]), double(x[e]), s);
  return s;
}

// RMSNorm factor r = fp32(1 / sqrt(mean(h^2) + eps)) from the float64 sum of squares:
// r decides the rounding of every normalised element, so it is taken at a precision
// where a different summation order cannot move it.
__device__ inline float rms_factor(double ss, int d, float eps) {
  return float(1.0 / sqrt(ss / double(d) + double(eps)));
}

// x = round_dtype( fp32( fp32(h * r) * gamma ) ) for one 16-byte group of elements.
template <int DT>
__device__ inline uint4 norm_pack(const uint4& hq, const uint4& gq, float r) {
  constexpr int EPL = Elem<DT>::EPL;
  float h[EPL], g[EPL];
  unpack<DT>(hq, h);
  unpack<DT>(gq, g);
  float y[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const float t = __fmul_rn(h[e], r);
    y[e] = __fmul_rn(t, g[e]);
  }
  if constexpr (DT == JSV_BF16) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(y[2 * e], y[2 * e + 1]);
    return make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    return make_uint4(__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]),
                      __float_as_uint(y[3]));
  }
}

// acc += A(16 x k-step) * B(k-step x 16).  Lane l holds row l%16 of A and column l%16 of
// B over the same k positions (lane group l/16 owns its 16 bytes of the k-step; for f32
// the four elements feed four 16x16x4 steps), so any hardware k order gives the same sum.
template <int DT>
__device__ inline floatx4 mfma_step(const uint4& a, const uint4& b, floatx4 acc) {
  if constexpr (DT == JSV_BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  } else {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
    return acc;
  }
}

// x += W(16 B of one row) . xhat(16 B of one hidden row) on the VALU.
template <int DT>
__device__ inline float dot16(const uint4& wq, const uint4& xq, float acc) {
  if constexpr (DT == JSV_BF16) {
    const uint32_t a[4] = {wq.x, wq.y, wq.z, wq.w};
    const uint32_t b[4] = {xq.x, xq.y, xq.z, xq.w};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a[e]),
                                            __builtin_bit_cast(bf16x2, b[e]), acc, false);
    return acc;
  } else {
    acc = fmaf(__uint_as_float(wq.x), __uint_as_float(xq.x), acc);
    acc = fmaf(__uint_as_float(wq.y), __uint_as_float(xq.y), acc);
    acc = fmaf(__uint_as_float(wq.z), __uint_as_float(xq.z), acc);
    acc = fmaf(__uint_as_float(wq.w), __uint_as_float(xq.w), acc);
    return acc;
  }
}

// ------------------------------------------------------------------------------------
// Online softmax statistics.  (m, s) means s = sum exp((z - m)/T); top2 is the second
// largest value; idx the argmax with the lowest id among equal maxima.
struct Stat {
  float m, top2, mq;
  int idx;
  double s, sq;
  uint32_t flags;
};

__device__ inline void stat_init(Stat& st) {
  st.m = -INFINITY; st.top2 = -INFINITY; st.mq = -INFINITY;
  st.idx = INT_MAX; st.s = 0.0; st.sq = 0.0; st.flags = 0;
}

__device__ inline void ms_merge(float& m, double& s, float mo, double so, float c) {
  const float nm = fmaxf(m, mo);
  if (nm == -INFINITY) { m = nm; s = 0.0; return; }
  s = s * double(exp2f((m - nm) * c)) + so * double(exp2f((mo - nm) * c));
  m = nm;
}

__device__ inline void stat_merge(Stat& a, const Stat& b, float c, bool soft) {
  const bool take = (b.m > a.m) || (b.m == a.m && b.idx < a.idx);
  const float top2 = take ? fmaxf(b.top2, a.m) : fmaxf(a.top2, b.m);
  if (soft) {
    ms_merge(a.m, a.s, b.m, b.s, c);
    ms_merge(a.mq, a.sq, b.mq, b.sq, c);
  }
  if (take) { a.m = b.m; a.idx = b.idx; }
  a.top2 = top2;
  a.flags |= b.flags;
}

template <int CTRL>
__device__ inline Stat stat_dpp(const Stat& a) {
  Stat o;
  o.m = dppf<CTRL>(a.m);
  o.top2 = dppf<CTRL>(a.top2);
  o.mq = dppf<CTRL>(a.mq);
  o.idx = int(dpp32<CTRL>(uint32_t(a.idx)));
  o.s = dppd<CTRL>(a.s);
  o.sq = dppd<CTRL>(a.sq);
  o.flags = dpp32<CTRL>(a.flags);
  return o;
}

__device__ inline Stat stat_readlane(const Stat& a, int l) {
  Stat o;
  o.m = readlane_f(a.m, l);
  o.top2 = readlane_f(a.top2, l);
  o.mq = readlane_f(a.mq, l);
  o.idx = readlane_i(a.idx, l);
  o.s = readlane_d(a.s, l);
  o.sq = readlane_d(a.sq, l);
  o.flags = uint32_t(readlane_i(int(a.flags), l));
  return o;
}

// Merge over each 16-lane row; every lane of the row ends with the row's merge.  All
// 16 sources are read in every step, so the result does not depend on what the other
// lanes hold outside this row.
__device__ inline void stat_row_reduce(Stat& st, float c, bool soft) {
  stat_merge(st, stat_dpp<0xB1>(st), c, soft);
  stat_merge(st, stat_dpp<0x4E>(st), c, soft);
  stat_merge(st, stat_dpp<0x124>(st), c, soft);
  stat_merge(st, stat_dpp<0x128>(st), c, soft);
}

// Merge over the whole wave, in every lane.
__device__ inline void stat_wave_reduce(Stat& st, float c, bool soft) {
  stat_row_reduce(st, c, soft);
  Stat r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = stat_readlane(st, 16 * i);
  st = r[0];
#pragma unroll
  for (int i = 1; i < 4; ++i) stat_merge(st, r[i], c, soft);
}

__device__ inline Stat stat_load(const RowStat& r) {
  Stat s;
  s.m = r.m; s.top2 = r.top2; s.mq = r.mq; s.s = r.s; s.sq = r.sq;
  s.idx = int(r.idxf & kIdxMask);
  s.flags = (r.idxf & kBadBit) ? uint32_t(JSV_FLAG_INVALID) : 0u;
  return s;
}

// Fold one value into (max, sum exp) without branches; ze = -inf contributes nothing.
__device__ inline void fold(float& m, double& s, float ze, float c) {
  const float nm = fmaxf(m, ze);
  const double sc = nm == -INFINITY ? 0.0 : double(exp2f((m - nm) * c));
  const double ad = nm == -INFINITY ? 0.0 : double(exp2f((ze - nm) * c));
  s = s * sc + ad;
  m = nm;
}

// Prefetch window in k-steps: half a group of W ahead for one tile (measured faster than
// a whole group, whose registers crowd the rest of the loop), at most 8 steps for two.
constexpr int pick_window(int NT, int NKS) {
  const int cap = NT <= 1 ? NKS / 2 : 8;
  for (int D = cap; D >= 1; --D)
    if (NKS % D == 0) return D;
  return 1;
}

// ------------------------------------------------------------------------------------
template <bool B> struct Tag { static constexpr bool value = B; };

// Logit groups staged in LDS between write-outs: at most 96 KB of staging, and no more
// than the LDS left over by the other arrays (`used` bytes of the 160 KB).
constexpr int stage_groups(int NTOK, int used) {
  const int room = 160 * 1024 - 512 - used;
  const int budget = room < 96 * 1024 ? room : 96 * 1024;
  const int g = budget / (NTOK * 16 * 4);
  return g > 64 ? 64 : g;
}

// Fused RMSNorm + LM head + statistics.  Workgroup wg owns the vocabulary rows [r0, r1),
// an equal share taken 16 rows (one group) at a time; its 8 waves split d into equal
// k-slices.  Each wave keeps the normalised
// hidden states of its slice for the NT full 16-token tiles in registers (MFMA B
// operand) and streams the same slice of W straight into MFMA A operands, D k-steps
// ahead, through a buffer resource over the workgroup's rows (rows past the vocabulary
// read as zero).  NX further rows (at most one) are dotted on the VALU against their
// normalised state in LDS.  Per group the 8 partial tiles are summed through LDS (in
// fp64, fixed order); thread (token jj, column ii) folds its logit into running
// statistics and parks it in LDS, and every SF groups the staged logits go out as whole
// row runs (64-byte stores scattered between the W reads cost far more).  At the end
// the 16 threads of a token merge their statistics into one partial.
template <int DT, int NT, int NX, int NKS>
__global__ __launch_bounds__(kThreads) void stats_kernel(StatsArgs a) {
  constexpr int XD = Act<DT>::value;                    // element type of h, gamma, x
  constexpr int EPL = Elem<XD>::EPL, ESZ = Elem<XD>::ESZ, KS = 4 * EPL;
  constexpr int SPL = DT == JSV_FP8 ? 2 : 1;            // MFMA k-steps per 16-byte W load
  constexpr int WSZ = DT == JSV_FP8 ? 1 : ESZ;          // bytes per W element
  constexpr int NL = NKS / SPL;                         // W loads per group and lane
  constexpr int D = DT == JSV_FP8 ? NL : pick_window(NT, NKS);  // W loads in flight
  static_assert(NL * SPL == NKS && NL >= 1, "fp8 needs an even number of k-steps");
  // bf16 and fp8 heads with whole quarters (4 loads of 16 bytes per lane: 4 k-steps of
  // bf16, 8 of fp8; 256 bytes of each row) in a wave's slice: W goes to LDS by DMA loads
  // that each read 4 rows x 256 contiguous bytes, whole cache lines and non-temporal, RQ
  // quarters ahead; the MFMA fragments are read back from LDS.
  constexpr bool LDSW = (DT == JSV_BF16 || DT == JSV_FP8) && NL % 4 == 0;
  constexpr int NQ = NL / 4 > 0 ? NL / 4 : 1;   // quarters per slice
  constexpr int NSC = DT == JSV_FP8 ? 1 : 0;    // row-scale DMA loads per group
  constexpr int RQ = NT <= 1 ? 3 : 2;           // 4 KB quarter slots per wave
  constexpr int NTOK = NT * 16 + NX;
  constexpr int NGI = (NTOK + 3) / 4;       // 256-byte DMA loads of a group's draft logits
  constexpr int NEP = (NTOK + 31) / 32;     // tokens per epilogue thread
  constexpr int XLEN = kWaves * NKS * 4;    // 16-byte groups per hidden row
  constexpr int XPT = (XLEN + kThreads - 1) / kThreads;
  constexpr int NT1 = NT > 0 ? NT : 1, NX1 = NX > 0 ? NX : 1;
  constexpr int RING = LDSW ? kWaves * RQ * 256 : 1;  // uint4 entries
  constexpr int SF = stage_groups(NTOK, 2 * kWaves * NT1 * kWave * 16 + 2 * kWaves * NX1 * 16 * 4 +
                                            NX1 * XLEN * 16 + XLEN * 16 + kWaves * kRowsPerPass * 8 +
                                            kRowsPerPass * 4 + 16 + RING * 16 +
                                            (LDSW ? 2 * NGI * 4 * 16 * 4 : 64) + 512);
  static_assert(SF >= 1, "LDS");
  static_assert(NTOK >= 1 && NTOK <= kRowsPerPass && NX <= 1, "tiling");
  __shared__ floatx4 red[2][kWaves][NT1][kWave];
  __shared__ float redx[2][kWaves][NX1][16];
  __shared__ uint4 xrow[NX1][XLEN];
  __shared__ uint4 gsh[XLEN];
  __shared__ float zst[NTOK][SF * 16];
  __shared__ double ssq[kWaves][kRowsPerPass];
  __shared__ float rnorm[kRowsPerPass];
  __shared__ uint4 wring[RING];
  __shared__ float gvs[LDSW ? 2 : 1][LDSW ? NGI * 4 : 1][16];
  __shared__ float wss[LDSW && NSC ? 2 : 1][64];  // fp8 row scales of a group (16 used)

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  // Workgroup -> (vocabulary chunk, pass of rows).  The passes of one chunk sit on the
  // same XCD (workgroups are dealt to the 8 XCDs round robin), so W is read from HBM once
  // and the other passes find it in that XCD's L2.
  int pass, chunk;
  {
    const int x = blockIdx.x, grid = gridDim.x, np = a.npass;
    if (grid % (8 * np) == 0) {
      const int slot = x >> 3, cpx = (grid >> 3) / np;
      chunk = (x & 7) * cpx + slot / np;
      pass = slot % np;
    } else {
      chunk = x / np;
      pass = x % np;
    }
  }
  const int row0 = pass * a.rp;
  const int rows = min(a.rp, a.M - row0);
  if (rows <= 0) return;
  const int P = a.nchunk, wg = chunk;
  const int64_t V = a.V;
  const int d = a.d;
  const int64_t r0 = V * wg / P, r1 = V * (wg + 1) / P;  // this workgroup's vocabulary rows
  const int ng = int((r1 - r0 + 15) >> 4);                // 16-row groups, the last may be partial
  const uint32_t rowbytes = uint32_t(d) * ESZ;   // hidden-state row
  const uint32_t wrowbytes = uint32_t(d) * WSZ;  // W row
  // Element offset in the row of the 8 (bf16) or 4 (f32) elements this lane feeds to
  // MFMA k-step s; the W load u of the lane covers steps u*SPL .. u*SPL+SPL-1.
  auto kofs = [&](int s) -> int {
    if constexpr (DT == JSV_FP8)
      return w * (NKS * KS) + (s >> 1) * (2 * KS) + (lane >> 4) * 16 + (s & 1) * 8;
    else
      return w * (NKS * KS) + s * KS + (lane >> 4) * EPL;
  };

  // W rows [r0, r1) as one buffer.  Every offset goes in the range-checked voffset (the
  // soffset is not range-checked), so rows past r1 read as zero and cost no traffic.
  const rsrc_t wr = make_rsrc(static_cast<const char*>(a.W) + (size_t)r0 * wrowbytes,
                              (uint64_t)(r1 - r0) * wrowbytes);
  const uint32_t wvoff = uint32_t(lane & 15) * wrowbytes + uint32_t(kofs(0)) * WSZ;
  auto wload = [&](int g, int u) -> uint4 {  // every load advances 64 bytes along the row
    return bload16(wr, wvoff + uint32_t(g) * 16u * wrowbytes + uint32_t(u) * 64u, 0);
  };
  // LDS staging.  DMA instruction q of quarter c fills 1 KB of the wave's slot: lane p
  // reads row 4q + p/16, 16-byte chunk k = (p mod 16) xor row of the quarter's 256 bytes
  // of that row.  The fragment of lane l for k-step 4c + t (row r = l mod 16, chunk
  // k = 4t + l/16, i.e. elements 32(4c+t) + 8(l/16), the same k mapping as the VGPR path)
  // is at 1024 (r/4) + 16 (16 (r mod 4) + (k xor r)): the xor spreads the 16 rows that
  // read together over all the banks.
  uint32_t vq[4], rdo[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = 4 * q + (lane >> 4);
    vq[q] = uint32_t(row) * wrowbytes + uint32_t(w * NL * 64) + uint32_t((lane & 15) ^ row) * 16u;
    const int r = lane & 15, k = 4 * q + (lane >> 4);
    rdo[q] = uint32_t((r >> 2) * 1024 + ((r & 3) * 16 + (k ^ r)) * 16);
  }
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const char* const ring_w = reinterpret_cast<const char*>(wring) + wu * (RQ * 4096);
  const uint32_t ring_lds = lds_addr(ring_w);
  const Srd wsrd = make_srd(static_cast<const char*>(a.W) + (size_t)r0 * wrowbytes,
                            (uint64_t)(r1 - r0) * wrowbytes);
  auto issue_quarter = [&](int slot, int n) {  // quarter n of this workgroup's stream
    const int g = n / NQ, c = n - g * NQ;
    const uint32_t base = uint32_t(g) * 16u * wrowbytes + uint32_t(c) * 256u;
    const uint32_t sb = ring_lds + uint32_t(slot) * 4096u;
#pragma unroll
    for (int q = 0; q < 4; ++q) dma16_nt(wsrd, sb + q * 1024u, vq[q] + base);
  };

  // ---- RMSNorm of the rows of this pass ----------------------------------------------
  // The hidden-state and gamma loads are issued before the first W loads: a wave's
  // loads return in issue order, so the norm does not wait behind W.
  const char* Hb = static_cast<const char*>(a.hidden) + (size_t)row0 * rowbytes;
  const rsrc_t hr = make_rsrc(Hb, (uint64_t)rows * rowbytes);
  const rsrc_t gr = make_rsrc(a.gamma, rowbytes);
  uint4 gq[XPT];
#pragma unroll
  for (int j = 0; j < XPT; ++j) {
    const int q = tid + j * kThreads;
    gq[j] = bload16(gr, q < XLEN ? uint32_t(q) * 16u : kOutOfRange, 0);
  }
  uint32_t tokoff[NT1];
#pragma unroll
  for (int t = 0; t < NT1; ++t) {
    const int tok = t * 16 + (lane & 15);
    tokoff[t] = (t < NT && tok < rows) ? uint32_t(tok) * rowbytes : kOutOfRange;
  }
  uint4 xf[NT1][NKS];  // this wave's slice of the tile tokens (padding tokens read zeros)
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int s = 0; s < NKS; ++s) xf[t][s] = bload16(hr, tokoff[t] + uint32_t(kofs(s)) * ESZ, 0);
  uint4 xh[NX1][XPT];  // the VALU row, block-wide
#pragma unroll
  for (int x = 0; x < NX; ++x)
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const int q = tid + j * kThreads;
      xh[x][j] = bload16(hr, (q < XLEN) ? uint32_t(NT * 16 + x) * rowbytes + uint32_t(q) * 16u
                                        : kOutOfRange, 0);
    }
  asm volatile("" ::: "memory");  // keep the W loads behind the loads above
  // Every wave's hidden-state requests go out before any wave's W requests: the compute
  // unit's memory pipeline serves them in order, and the norm waits on the slowest wave.
  __syncthreads();
  uint4 fr[LDSW ? 1 : D];
  if constexpr (LDSW) {
#pragma unroll
    for (int j = 0; j < RQ; ++j) issue_quarter(j, j);
  } else {
#pragma unroll
    for (int j = 0; j < D; ++j) fr[j] = wload(0, j);
  }
  int slot = 0;  // ring slot of the next quarter

#pragma unroll
  for (int j = 0; j < XPT; ++j) {
    const int q = tid + j * kThreads;
    if (q < XLEN) gsh[q] = gq[j];
  }
  // Sums of squares of this wave's slice of every token.
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    double ps = 0.0;
#pragma unroll
    for (int s = 0; s < NKS; ++s) ps += sumsq16<XD>(xf[t][s]);
    ps = rows_sum(ps);
    if (lane < 16) ssq[w][t * 16 + lane] = ps;
  }
#pragma unroll
  for (int x = 0; x < NX; ++x) {
    double ps = 0.0;
#pragma unroll
    for (int j = 0; j < XPT; ++j) ps += sumsq16<XD>(xh[x][j]);
    ps = wave_sum(ps);
    if (lane == 0) ssq[w][NT * 16 + x] = ps;
  }
  __syncthreads();
  if (tid < rows) {
    double ss = 0.0;
#pragma unroll
    for (int w2 = 0; w2 < kWaves; ++w2) ss += ssq[w2][tid];  // fixed order over waves
    const float r = rms_factor(ss, d, a.eps);
    rnorm[tid] = r;
    if (wg == 0 && a.rnorm != nullptr) a.rnorm[row0 + tid] = r;
  }
  __syncthreads();

  // The tile tokens are normalised in place step by step inside the first group, where
  // the VALU work overlaps the W stream (padding tokens get r = 0; their output columns
  // are never used).  The VALU row is normalised into LDS here.
  float rt[NT1];
#pragma unroll
  for (int t = 0; t < NT1; ++t) {
    const int tok = t * 16 + (lane & 15);
    rt[t] = (t < NT && tok < rows) ? rnorm[tok] : 0.f;
  }
#pragma unroll
  for (int x = 0; x < NX; ++x) {
    const float r = rnorm[NT * 16 + x];
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const int q = tid + j * kThreads;
      if (q < XLEN) xrow[x][q] = norm_pack<XD>(xh[x][j], gsh[q], r);
    }
  }
  if (NX > 0) __syncthreads();

  // ---- epilogue identity: tokens jj = tid/16 (+32), vocabulary column ii ---------------
  const int ii = tid & 15;
  const bool soft = a.T > 0.f;
  const float c = a.c;
  // Logits rows of this pass, and the draft-logit rows of the requests it touches.
  const rsrc_t lr = make_rsrc(a.logits + (size_t)row0 * V, (uint64_t)rows * (uint64_t)V * 4u);
  const int qrow0 = a.want_q ? (row0 / (a.K + 1)) * a.K : 0;
  const int qrows = a.want_q ? ((row0 + rows - 1) / (a.K + 1)) * a.K + a.K - qrow0 : 0;
  const rsrc_t qr = make_rsrc(a.G + (size_t)qrow0 * V, (uint64_t)qrows * (uint64_t)V * 4u);
  // Row scales of an fp8 head for this workgroup's rows.
  const rsrc_t sr = make_rsrc(DT == JSV_FP8 ? a.wscale + r0 : a.logits,
                              DT == JSV_FP8 ? uint64_t(r1 - r0) * 4u : 0u);
  int jj[NEP];
  bool tok_ok[NEP], qrow[NEP];
  uint32_t qoff[NEP];
  Stat st[NEP];
#pragma unroll
  for (int e = 0; e < NEP; ++e) {
    jj[e] = (tid >> 4) + 32 * e;
    tok_ok[e] = jj[e] < NTOK && jj[e] < rows;
    const int row = row0 + (tok_ok[e] ? jj[e] : 0);
    qrow[e] = false;
    qoff[e] = kOutOfRange;
    if (a.want_q && tok_ok[e]) {
      const int b = row / (a.K + 1), i = row - b * (a.K + 1);
      if (i < a.K) { qrow[e] = true; qoff[e] = uint32_t(b * a.K + i - qrow0) * uint32_t(V) * 4u; }
    }
    stat_init(st[e]);
  }
  // Staged path: wave 0 moves a group's draft logits (softmax proposal) into LDS one
  // group ahead, NGI DMA loads in which lane p takes token 4i + p/16, column p mod 16.
  const bool gdma = LDSW && a.want_q;
  const bool w0 = wu == 0;
  const Srd qsrd = make_srd(a.G + (size_t)qrow0 * V, (uint64_t)qrows * (uint64_t)V * 4u);
  uint32_t gqo[LDSW ? NGI : 1];
#pragma unroll
  for (int i = 0; i < (LDSW ? NGI : 1); ++i) {
    const int jt = 4 * i + (lane >> 4);
    gqo[i] = kOutOfRange;
    if (a.want_q && jt < NTOK && jt < rows) {
      const int row = row0 + jt, b = row / (a.K + 1), ir = row - b * (a.K + 1);
      if (ir < a.K) gqo[i] = uint32_t(b * a.K + ir - qrow0) * uint32_t(V) * 4u + uint32_t(lane & 15) * 4u;
    }
  }
  const Srd ssrd = make_srd(DT == JSV_FP8 ? a.wscale + r0 : a.logits,
                            DT == JSV_FP8 ? uint64_t(r1 - r0) * 4u : 0u);
  // Wave 0's per-group side loads, one group ahead: the draft logits (softmax proposal,
  // NGI loads) and an fp8 head's 16 row scales (one load, lanes 0-15).
  auto issue_side = [&](int g) {
    if (gdma) {
      const uint32_t cb = uint32_t(r0 + int64_t(g) * 16) * 4u;
      const uint32_t dst = lds_addr(&gvs[g & 1][0][0]);
#pragma unroll
      for (int i = 0; i < (LDSW ? NGI : 1); ++i) dma4(qsrd, dst + uint32_t(i) * 256u, gqo[i] + cb);
    }
    if constexpr (NSC > 0)
      dma4(ssrd, lds_addr(&wss[g & 1][0]), lane < 16 ? uint32_t(g * 16 + lane) * 4u : kOutOfRange);
  };
  const bool side = gdma || NSC > 0;  // wave 0 issues side loads

  int buf = 0;
  int gb = 0;  // first group of the staged run
  auto group = [&](int g, auto first) {
    constexpr bool FIRST = decltype(first)::value;
    const int64_t v = r0 + g * 16 + ii;
    const bool vok = v < r1;
    float gv[NEP];
    if constexpr (!LDSW) {
#pragma unroll
      for (int e = 0; e < NEP; ++e) gv[e] = bload4f(qr, qoff[e] + uint32_t(v) * 4u);
    }
    float wsc = 1.f;
    if constexpr (DT == JSV_FP8 && !LDSW) wsc = bload4f(sr, uint32_t(g * 16 + ii) * 4u);
    floatx4 acc[NT1];
    float xacc[NX1];
#pragma unroll
    for (int t = 0; t < NT1; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int x = 0; x < NX1; ++x) xacc[x] = 0.f;
    if constexpr (LDSW) {
#pragma unroll
      for (int c = 0; c < NQ; ++c) {
        // This quarter's 4 DMA loads have landed: 4 (RQ - 1) loads of later quarters were
        // issued after them, and on wave 0 in the first RQ quarters also this group's side
        // loads.
        if (side && w0 && c < RQ) {
          if (gdma) wait_vmcnt<4 * (RQ - 1) + NGI + NSC>();
          else wait_vmcnt<4 * (RQ - 1) + NSC>();
        } else {
          wait_vmcnt<4 * (RQ - 1)>();
        }
        const char* sb = ring_w + slot * 4096;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint4 fw = *reinterpret_cast<const uint4*>(sb + rdo[t]);
#pragma unroll
          for (int h = 0; h < SPL; ++h) {
            const int s = (4 * c + t) * SPL + h;
            if constexpr (FIRST) {
              const uint4 gq = gsh[kofs(s) / EPL];
#pragma unroll
              for (int tt = 0; tt < NT; ++tt) xf[tt][s] = norm_pack<XD>(xf[tt][s], gq, rt[tt]);
            }
            const uint4 f = wfrag<DT>(fw, h);
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) acc[tt] = mfma_step<XD>(f, xf[tt][s], acc[tt]);
#pragma unroll
            for (int x = 0; x < NX; ++x) xacc[x] = dot16<XD>(f, xrow[x][kofs(s) / EPL], xacc[x]);
          }
        }
        wait_lgkmcnt0();  // the slot has been read: refill it RQ quarters ahead
        issue_quarter(slot, g * NQ + c + RQ);
        slot = slot + 1 == RQ ? 0 : slot + 1;
      }
    } else {
#pragma unroll
      for (int u = 0; u < NL; ++u) {
        const uint4 fw = fr[u % D];
#pragma unroll
        for (int h = 0; h < SPL; ++h) {
          const int s = u * SPL + h;
          if constexpr (FIRST) {
            const uint4 gq = gsh[kofs(s) / EPL];
#pragma unroll
            for (int t = 0; t < NT; ++t) xf[t][s] = norm_pack<XD>(xf[t][s], gq, rt[t]);
          }
          const uint4 f = wfrag<DT>(fw, h);
#pragma unroll
          for (int t = 0; t < NT; ++t) acc[t] = mfma_step<XD>(f, xf[t][s], acc[t]);
#pragma unroll
          for (int x = 0; x < NX; ++x) xacc[x] = dot16<XD>(f, xrow[x][kofs(s) / EPL], xacc[x]);
        }
        // refill this slot D loads ahead (past the last group the loads read zeros)
        const bool nxt = (u + D) >= NL;
        fr[u % D] = wload(nxt ? g + 1 : g, nxt ? (u + D - NL) : (u + D));
      }
    }
#pragma unroll
    for (int x = 0; x < NX; ++x) {
      const float y = rows_sum(xacc[x]);
      if (lane < 16) redx[buf][w][x][lane] = y;
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) red[buf][w][t][lane] = acc[t];
    if constexpr (LDSW) {
      if (side && w0) wait_vmcnt<NL>();  // this group's side loads: NL W loads since
    }
    __syncthreads();
    if constexpr (LDSW) {
      if (side && w0) issue_side(g + 1);
#pragma unroll
      for (int e = 0; e < NEP; ++e) gv[e] = qrow[e] ? gvs[g & 1][jj[e]][ii] : 0.f;
      if constexpr (NSC > 0) wsc = wss[g & 1][ii];
    }
#pragma unroll
    for (int e = 0; e < NEP; ++e) {
      if (jj[e] >= NTOK) continue;
      double zz = 0.0;
      if (jj[e] < NT * 16) {
        const int t = jj[e] >> 4, src = ((ii >> 2) << 4) + (jj[e] & 15), r = ii & 3;
#pragma unroll
        for (int w2 = 0; w2 < kWaves; ++w2) zz += double(red[buf][w2][t][src][r]);
      } else {
        const int x = jj[e] - NT * 16;
#pragma unroll
        for (int w2 = 0; w2 < kWaves; ++w2) zz += double(redx[buf][w2][x][ii]);
      }
      const float z = DT == JSV_FP8 ? float(zz * double(wsc)) : float(zz);
      const bool valid = tok_ok[e] && vok;
      zst[jj[e]][(g - gb) * 16 + ii] = z;
      if (a.stats) {
        Stat& S = st[e];
        const bool fin = fabsf(z) <= FLT_MAX;
        if (valid && !fin) S.flags |= JSV_FLAG_INVALID;
        const float ze = (valid && fin) ? z : -INFINITY;
        if (ze > S.m) { S.top2 = S.m; S.idx = int(v); } else { S.top2 = fmaxf(S.top2, ze); }
        if (soft) fold(S.m, S.s, ze, c); else S.m = fmaxf(S.m, ze);
        if (qrow[e]) {
          const float q = gv[e];
          const bool qf = fabsf(q) <= FLT_MAX;
          if (vok && !qf) S.flags |= JSV_FLAG_INVALID;
          fold(S.mq, S.sq, (vok && qf) ? q : -INFINITY, c);
        }
      }
    }
    if (g + 1 == ng || g + 1 - gb == SF) {  // write out the staged run
      __syncthreads();
      const int64_t c0l = r0 + gb * 16;
      const int ncol = int(min<int64_t>((g + 1 - gb) * 16, r1 - c0l));
      const uint32_t c0 = uint32_t(c0l);
#pragma unroll
      for (int rr = 0; rr < NTOK; ++rr) {
        if (rr >= rows) break;
        for (int cc = tid; cc < ncol; cc += kThreads) {
          const uint32_t vv = c0 + uint32_t(cc);
          bstore4f_nt(zst[rr][cc], lr, vv < uint32_t(V) ? uint32_t(rr) * uint32_t(V) * 4u + vv * 4u : kOutOfRange);
        }
      }
      gb = g + 1;
    }
    buf ^= 1;
  };
  if constexpr (LDSW) {
    if (side && w0) issue_side(0);
  }
  group(0, Tag<true>{});
  for (int g = 1; g < ng; ++g) group(g, Tag<false>{});
  if constexpr (LDSW) wait_vmcnt<0>();  // no DMA write into LDS may outlive the workgroup

  if (!a.stats) return;
#pragma unroll
  for (int e = 0; e < NEP; ++e) {
    stat_row_reduce(st[e], c, soft);
    if (ii == 0 && tok_ok[e]) {
      RowStat rs;
      rs.s = st[e].s; rs.sq = st[e].sq; rs.m = st[e].m; rs.top2 = st[e].top2; rs.mq = st[e].mq;
      rs.idxf = (uint32_t(st[e].idx) & kIdxMask) | (st[e].flags ? kBadBit : 0u);
      a.partial[(size_t)(row0 + jj[e]) * P + wg] = rs;
    }
  }
}

// ------------------------------------------------------------------------------------
// Wide LM head (bf16, 34..144 rows).  Part 1: the normalised rows, one workgroup of 256
// threads per row: r from the float64 sum of squares, x = bf16(fp32(fp32(h r) gamma)).
__global__ __launch_bounds__(kSliceThreads) void xhat_kernel(WideArgs a) {
  constexpr int PER = (kWideMaxD / 8 + kSliceThreads - 1) / kSliceThreads;  // 16-byte groups per thread
  const int m = blockIdx.x, tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const uint32_t rowbytes = uint32_t(a.d) * 2u;
  const int n16 = a.d / 8;
  const rsrc_t hr = make_rsrc(static_cast<const char*>(a.hidden) + (size_t)m * rowbytes, rowbytes);
  const rsrc_t gr = make_rsrc(a.gamma, rowbytes);
  uint4 hq[PER], gq[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int q = tid + j * kSliceThreads;
    hq[j] = bload16(hr, q < n16 ? uint32_t(q) * 16u : kOutOfRange, 0);
    gq[j] = bload16(gr, q < n16 ? uint32_t(q) * 16u : kOutOfRange, 0);
  }
  double ss = 0.0;
#pragma unroll
  for (int j = 0; j < PER; ++j) ss += sumsq16<JSV_BF16>(hq[j]);
  ss = wave_sum(ss);
  __shared__ double wsum[kSliceThreads / kWave];
  if (lane == 0) wsum[w] = ss;
  __syncthreads();
  double tot = 0.0;
#pragma unroll
  for (int i = 0; i < kSliceThreads / kWave; ++i) tot += wsum[i];  // fixed order
  const float r = rms_factor(tot, a.d, a.eps);
  if (tid == 0) a.rnorm[m] = r;
  uint4* xo = reinterpret_cast<uint4*>(a.xhat + (size_t)m * a.d);
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int q = tid + j * kSliceThreads;
    if (q < n16) xo[q] = norm_pack<JSV_BF16>(hq[j], gq[j], r);
  }
}

// Part 2: partial products.  Workgroup (vocabulary chunk, block q of 1024 columns of d);
// wave w holds tile w (rows 16w .. 16w + 15) of the normalised states over the block in
// registers (32 MFMA k-steps) and every wave multiplies the same W group (16 vocabulary
// rows x 1024 columns, 32 KB) from LDS.  The group is staged by DMA in eight quarters of
// 4 k-steps, wave w < 8 moving quarter w in the layout of the LM-head kernel (4 rows x
// 256 contiguous bytes per load, row-XOR swizzle), three groups ahead.  The products go to
// plane q in [row group][row][vocabulary] order straight from the accumulators, one
// 16-byte store per lane (its four values are consecutive vocabulary rows of one row).
template <int NW>
__global__ __launch_bounds__(NW * kWave) void wide_kernel(WideArgs a) {
  constexpr int NQ = kWideBlock / 128;  // quarters of a group (4 k-steps of 32 columns)
  constexpr int KS = kWideBlock / 32;   // k-steps of a block
  constexpr int RG = 4;                 // groups in the LDS ring (RG - 1 ahead)
  __shared__ uint4 ring[RG][NQ][256];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int S = a.pl.S, P = a.pl.nchunk, mp = a.pl.mp;
  const int q = blockIdx.x % S, chunk = blockIdx.x / S;
  const int64_t V = a.V, Vp = (V + 3) & ~int64_t(3);
  const int64_t ngroups = (V + 15) >> 4;  // chunks start on whole 16-row groups
  const int64_t r0 = 16 * (ngroups * chunk / P);
  const int64_t r1 = min(V, 16 * (ngroups * (chunk + 1) / P));
  const int ng = int((r1 - r0 + 15) >> 4);
  const uint32_t wrowbytes = uint32_t(a.d) * 2u;

  // DMA of quarter wu of group g into ring slot g % RG (waves 0..7).
  const Srd wsrd = make_srd(static_cast<const char*>(a.W) + (size_t)r0 * wrowbytes,
                            (uint64_t)(r1 - r0) * wrowbytes);
  uint32_t vq[4], rdo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * i + (lane >> 4);
    vq[i] = uint32_t(row) * wrowbytes + uint32_t(q) * (kWideBlock * 2u) + uint32_t(wu < NQ ? wu : 0) * 256u +
            uint32_t((lane & 15) ^ row) * 16u;
    const int r = lane & 15, k = 4 * i + (lane >> 4);
    rdo[i] = uint32_t((r >> 2) * 1024 + ((r & 3) * 16 + (k ^ r)) * 16);
  }
  const bool mover = wu < NQ;
  auto issue = [&](int g) {
    if (mover) {
      const uint32_t sb = lds_addr(&ring[g % RG][wu][0]);
      const uint32_t base = uint32_t(g) * 16u * wrowbytes;
#pragma unroll
      for (int i = 0; i < 4; ++i) dma16_nt(wsrd, sb + uint32_t(i) * 1024u, vq[i] + base);
    }
  };
#pragma unroll
  for (int j = 0; j < RG - 1; ++j) issue(j);

  // Tile w of the normalised rows over block q (rows past M read as zero).  Issued after
  // the DMA loads: the waits the compiler places for these then also cover the DMA.
  const int tok = 16 * wu + (lane & 15);
  const bool live = 16 * wu < a.M;
  const rsrc_t xr = make_rsrc(a.xhat, (uint64_t)a.M * wrowbytes);
  uint4 xf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s)
    xf[s] = bload16(xr, (live && tok < a.M) ? uint32_t(tok) * wrowbytes +
                            uint32_t(q * kWideBlock + 32 * s + 8 * (lane >> 4)) * 2u
                                            : kOutOfRange, 0);
  // Plane q, row group wu ([q][group][16 rows][Vp] layout, Vp = V rounded up to 4): lane
  // l holds the products of vocabulary rows v .. v + 3 (v = 16 g + 4 (l / 16) past r0) for
  // row l mod 16, stored as one 16-byte write; quads past Vp are not written.
  const int ngr = mp / 16;
  const rsrc_t pr = make_rsrc(a.planes + ((size_t)q * ngr + (live ? wu : 0)) * 16 * Vp,
                              live ? (uint64_t)16 * Vp * 4u : 0u);
  const uint32_t prow = uint32_t(lane & 15) * uint32_t(Vp);

  for (int g = 0; g < ng; ++g) {
    // this wave's quarter of group g has landed (RG - 2 later groups of DMA outstanding)
    wait_vmcnt<4 * (RG - 2)>();
    __syncthreads();  // every quarter of group g is in LDS; group g - 1's slot is free
    issue(g + RG - 1);
    if (live) {
      floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
      const char* sb = reinterpret_cast<const char*>(&ring[g % RG][0][0]);
#pragma unroll
      for (int c = 0; c < NQ; ++c) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint4 fw = *reinterpret_cast<const uint4*>(sb + c * 4096 + rdo[t]);
          acc = mfma_step<JSV_BF16>(fw, xf[4 * c + t], acc);
        }
      }
      const int64_t v = r0 + 16 * g + 4 * (lane >> 4);
      bstore16(make_uint4(__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]),
                          __float_as_uint(acc[3])),
               pr, v < Vp ? (prow + uint32_t(v)) * 4u : kOutOfRange);
    }
  }
  wait_vmcnt<0>();  // no DMA write into LDS may outlive the workgroup
}

// Part 3: logits and partial statistics.  Workgroup (wg, group rg) of 256 threads takes the
// 16 rows of row group rg over its share of the vocabulary (whole tiles of 64 columns):
// per tile the S plane tiles (16 rows x 256 B each) are summed in float64 in block order
// into an LDS tile [column][row], then the 16 threads of row m take four consecutive
// columns each: they write the logits and fold them (and the draft logits) into running
// statistics, merged over the 16 lanes into the row's partial record at the end.  With V
// a multiple of 4 every logit store and draft-logit load is one 16-byte access.
constexpr int kWideCombineThreads = 256;
template <int NS>  // blocks of d (= a.pl.S)
__global__ __launch_bounds__(kWideCombineThreads) void wide_stats_kernel(WideArgs a) {
  constexpr int TC = 64;
  __shared__ float zt[TC][17];
  const int tid = threadIdx.x;
  const int ngr = a.pl.mp / 16, P = a.pl.ncomb, M = a.M;
  const int wg = blockIdx.x, rg = blockIdx.y;
  const int64_t V = a.V, Vp = (V + 3) & ~int64_t(3);
  const int64_t ntiles = (V + TC - 1) / TC;
  const int64_t c0 = TC * (ntiles * wg / P), c1 = min(V, TC * (ntiles * (wg + 1) / P));
  const int ml = tid >> 4, u = tid & 15, m = 16 * rg + ml;
  const bool rowok = m < M;
  const bool soft = a.T > 0.f;
  const bool quad = a.quad != 0;  // rows of the logits and draft logits are 16-byte aligned
  const float c = a.c;
  int grow = -1;
  if (rowok && a.want_q) {
    const int b = m / (a.K + 1), i = m - b * (a.K + 1);
    if (i < a.K) grow = b * a.K + i;
  }
  const rsrc_t gr = make_rsrc(a.G, a.want_q ? (uint64_t)a.B * a.K * (uint64_t)V * 4u : 0u);
  const rsrc_t lr = make_rsrc(a.logits, (uint64_t)M * (uint64_t)V * 4u);
  rsrc_t pr[NS];
#pragma unroll
  for (int qq = 0; qq < NS; ++qq)
    pr[qq] = make_rsrc(a.planes + ((size_t)qq * ngr + rg) * 16 * Vp, (uint64_t)16 * Vp * 4u);
  // plane element of this thread in the tile: row tid / 16, columns 4 (tid mod 16) .. + 3
  const uint32_t prow = uint32_t(tid >> 4) * uint32_t(Vp);
  Stat st;
  stat_init(st);
  for (int64_t v0 = c0; v0 < c1; v0 += TC) {
    const int64_t vq = v0 + 4 * u;  // this thread's four columns in the fold
    float gv[4];
    if (quad) {
      const uint4 g4 = bload16(gr, (grow >= 0 && vq < c1) ? uint32_t((int64_t)grow * V + vq) * 4u : kOutOfRange, 0);
      gv[0] = __uint_as_float(g4.x); gv[1] = __uint_as_float(g4.y);
      gv[2] = __uint_as_float(g4.z); gv[3] = __uint_as_float(g4.w);
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        gv[k] = bload4f(gr, (grow >= 0 && vq + k < c1) ? uint32_t((int64_t)grow * V + vq + k) * 4u : kOutOfRange);
    }
    uint4 x[NS];
    const uint32_t off = (prow + uint32_t(v0) + 4u * uint32_t(tid & 15)) * 4u;
#pragma unroll
    for (int qq = 0; qq < NS; ++qq) x[qq] = bload16(pr[qq], off, 0);
    double sum[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int qq = 0; qq < NS; ++qq) {
      sum[0] += double(__uint_as_float(x[qq].x));
      sum[1] += double(__uint_as_float(x[qq].y));
      sum[2] += double(__uint_as_float(x[qq].z));
      sum[3] += double(__uint_as_float(x[qq].w));
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) zt[4 * (tid & 15) + k][tid >> 4] = float(sum[k]);
    __syncthreads();  // zt holds tile v0
    if (rowok) {
      float z[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) z[k] = zt[4 * u + k][ml];
      if (quad) {
        bstore16(make_uint4(__float_as_uint(z[0]), __float_as_uint(z[1]), __float_as_uint(z[2]),
                            __float_as_uint(z[3])),
                 lr, vq < c1 ? uint32_t((int64_t)m * V + vq) * 4u : kOutOfRange);
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) bstore4f(z[k], lr, vq + k < c1 ? uint32_t((int64_t)m * V + vq + k) * 4u : kOutOfRange);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int64_t v = vq + k;
        const bool vok = v < c1;
        const bool fin = fabsf(z[k]) <= FLT_MAX;
        if (vok && !fin) st.flags |= JSV_FLAG_INVALID;
        const float ze = (vok && fin) ? z[k] : -INFINITY;
        if (ze > st.m) { st.top2 = st.m; st.idx = int(v); } else { st.top2 = fmaxf(st.top2, ze); }
        if (soft) fold(st.m, st.s, ze, c); else st.m = fmaxf(st.m, ze);
        if (grow >= 0) {
          const float gq = gv[k];
          const bool qf = fabsf(gq) <= FLT_MAX;
          if (vok && !qf) st.flags |= JSV_FLAG_INVALID;
          fold(st.mq, st.sq, (vok && qf) ? gq : -INFINITY, c);
        }
      }
    }
    __syncthreads();  // the readers are done with zt
  }
  stat_row_reduce(st, c, soft);  // the 16 lanes of a row, in a fixed order
  if (rowok && u == 0) {
    RowStat rs;
    rs.s = st.s; rs.sq = st.sq; rs.m = st.m; rs.top2 = st.top2; rs.mq = st.mq;
    rs.idxf = (uint32_t(st.idx) & kIdxMask) | (st.flags ? kBadBit : 0u);
    a.partial[(size_t)m * P + wg] = rs;
  }
}

// ------------------------------------------------------------------------------------
// Finalize, part 1 (rowstat_kernel): grid (tasks, B) of one-wave workgroups, so that
// the reads spread over the chip.  Task i < K (T > 0 only): the float64 logit of draft
// row i at its draft token, from the normalised row and W[d_i], so that alpha and
// 1 - alpha keep their digits when alpha is close to 1 (paper §3, acceptance rule).  The
// other tasks merge the partial statistics of one row over every LM-head workgroup.
// Part 2 (scan_kernel): grid B, one wave, lane i = row i: acceptance probabilities and
// the scan to the first rejection with the Philox uniforms (verify: paper §3, App. F.3),
// or the outcome marginals (score: §4.2 Eq. 6).

// Float64 logit of hidden row `row` at vocabulary row `dt`, returned on every lane.  The
// normalised row is rebuilt from h, gamma and the stored RMSNorm factor the way the
// LM-head kernel builds it; all loads of a batch are in flight together.
template <int DT>
__device__ double exact_logit(const FinalArgs& a, int row, int dt, float r) {
  constexpr int EPL = Elem<DT>::EPL;
  constexpr int NJ = 8;  // 16-byte groups per lane and operand per batch
  const int lane = threadIdx.x & (kWave - 1);
  const uint32_t bytes = uint32_t(a.d) * uint32_t(Elem<DT>::ESZ);
  const rsrc_t hr = make_rsrc(static_cast<const char*>(a.hidden) + (size_t)row * bytes, bytes);
  const rsrc_t gr = make_rsrc(a.gamma, bytes);
  const rsrc_t wr = make_rsrc(static_cast<const char*>(a.W) + (size_t)dt * bytes, bytes);
  double acc = 0.0;
  for (uint32_t base = 0; base < bytes; base += NJ * kWave * 16) {
    uint4 hq[NJ], gq[NJ], wq[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const uint32_t off = base + uint32_t(j * kWave + lane) * 16u;
      hq[j] = bload16(hr, off, 0);
      gq[j] = bload16(gr, off, 0);
      wq[j] = bload16(wr, off, 0);
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      float xv[EPL], wv[EPL];
      unpack<DT>(norm_pack<DT>(hq[j], gq[j], r), xv);
      unpack<DT>(wq[j], wv);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc = fma(double(xv[e]), double(wv[e]), acc);
    }
  }
  return wave_sum(acc);
}

// The same for an fp8 head: W row dt holds E4M3 codes (one byte each) and a row scale;
// h and gamma are bf16.  Each lane takes 16 consecutive elements per load of codes.
__device__ double exact_logit_fp8(const FinalArgs& a, int row, int dt, float r) {
  constexpr int NJ = 4;  // 16-code loads per lane per batch
  const int lane = threadIdx.x & (kWave - 1);
  const uint32_t wbytes = uint32_t(a.d), xbytes = uint32_t(a.d) * 2u;
  const rsrc_t hr = make_rsrc(static_cast<const char*>(a.hidden) + (size_t)row * xbytes, xbytes);
  const rsrc_t gr = make_rsrc(a.gamma, xbytes);
  const rsrc_t wr = make_rsrc(static_cast<const char*>(a.W) + (size_t)dt * wbytes, wbytes);
  double acc = 0.0;
  for (uint32_t base = 0; base < wbytes; base += NJ * kWave * 16) {
    uint4 wq[NJ], hq[2 * NJ], gq[2 * NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const uint32_t e0 = base + uint32_t(j * kWave + lane) * 16u;  // first element
      wq[j] = bload16(wr, e0, 0);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        hq[2 * j + h] = bload16(hr, (e0 + 8u * h) * 2u, 0);
        gq[2 * j + h] = bload16(gr, (e0 + 8u * h) * 2u, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float xv[8], wv[8];
        unpack<JSV_BF16>(norm_pack<JSV_BF16>(hq[2 * j + h], gq[2 * j + h], r), xv);
        unpack<JSV_BF16>(wfrag<JSV_FP8>(wq[j], h), wv);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fma(double(xv[e]), double(wv[e]), acc);
      }
  }
  return wave_sum(acc) * double(a.wscale[dt]);
}

// Merge of the P partial records of one row, returned on every lane.
__device__ Stat combine_row(const FinalArgs& a, int row, float c, bool soft) {
  const int lane = threadIdx.x & (kWave - 1), P = a.P;
  const rsrc_t pr = make_rsrc(a.partial + (size_t)row * P, uint64_t(P) * sizeof(RowStat));
  Stat acc;
  stat_init(acc);
  for (int p0 = 0; p0 < P; p0 += 4 * kWave) {
    uint4 lo[4], hi[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t off = uint32_t(p0 + j * kWave + lane) * uint32_t(sizeof(RowStat));
      lo[j] = bload16(pr, off, 0);
      hi[j] = bload16(pr, off + 16u, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      Stat o;
      stat_init(o);
      if (p0 + j * kWave + lane < P) {
        o.s = u2d(lo[j].x, lo[j].y);
        o.sq = u2d(lo[j].z, lo[j].w);
        o.m = __uint_as_float(hi[j].x);
        o.top2 = __uint_as_float(hi[j].y);
        o.mq = __uint_as_float(hi[j].z);
        o.idx = int(hi[j].w & kIdxMask);
        o.flags = (hi[j].w & kBadBit) ? uint32_t(JSV_FLAG_INVALID) : 0u;
      }
      stat_merge(acc, o, c, soft);
    }
  }
  stat_wave_reduce(acc, c, soft);
  return acc;
}

__global__ __launch_bounds__(kWave) void rowstat_kernel(FinalArgs a) {
  const int t = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int K = a.K, R = K + 1;
  const int64_t V = a.V;
  const bool soft = a.T > 0.f;
  const int nx = soft ? K : 0;
  if (t < nx) {
    const int row = b * R + t;
    const int dt = a.drafts[b * K + t];
    const float r = a.rnorm[row];
    DraftLogit o{};
    if (dt >= 0 && (int64_t)dt < V) {
      if (a.mode == JSV_PROPOSAL_SOFTMAX) o.g = a.G[(size_t)(b * K + t) * V + dt];
      o.z = (a.dtype == JSV_BF16) ? exact_logit<JSV_BF16>(a, row, dt, r)
            : (a.dtype == JSV_FP8)  ? exact_logit_fp8(a, row, dt, r)
                                    : exact_logit<JSV_F32>(a, row, dt, r);
    }
    if (lane == 0) a.dlog[row] = o;
  } else {
    const float c = soft ? float(kLog2eD / double(a.T)) : 0.f;
    const int row = b * R + (t - nx);
    const Stat st = combine_row(a, row, c, soft);
    if (lane == 0) {
      RowStat rs;
      rs.s = st.s; rs.sq = st.sq; rs.m = st.m; rs.top2 = st.top2; rs.mq = st.mq;
      rs.idxf = (uint32_t(st.idx) & kIdxMask) | (st.flags ? kBadBit : 0u);
      a.rowstat[row] = rs;
    }
  }
}

// The acceptance scan of request b on one wave, lane i = row i (i <= K).  Every kernel
// that runs it on the same inputs gets the same k: the rule is positional and the
// uniforms are counter-based.
struct Scan {
  Stat st;        // this lane's row statistics
  int di;         // this lane's draft token (-1 past the drafts)
  double alpha;   // this lane's acceptance probability
  bool bad;       // the request is invalid (same on every lane)
  int k;          // first rejection, K if none (same on every lane)
  double vk;      // bonus uniform of row k
  uint32_t f;     // decision flags
};

__device__ Scan scan_request(const FinalArgs& a, int b) {
  const int lane = threadIdx.x & (kWave - 1);
  const int K = a.K, R = K + 1;
  const int64_t V = a.V;
  const bool soft = a.T > 0.f;
  const double cd = soft ? kLog2eD / double(a.T) : 0.0;
  Scan sc;
  sc.di = (lane < K) ? a.drafts[b * K + lane] : -1;
  DraftLogit dl{};
  if (soft && lane < K) dl = a.dlog[b * R + lane];
  const bool act = lane <= K;
  stat_init(sc.st);
  if (act) sc.st = stat_load(a.rowstat[b * R + lane]);
  const Stat& st = sc.st;
  const int di = sc.di;
  sc.bad = __ballot(act && ((st.flags & JSV_FLAG_INVALID) || (lane < K && (di < 0 || (int64_t)di >= V)))) != 0;
  sc.alpha = 0.0;
  sc.k = K;
  sc.vk = 0.0;
  sc.f = 0;
  if (sc.bad) return sc;
  if (!soft) {
    // Greedy verification: accept while the draft equals the row's argmax.
    sc.alpha = (lane < K && di == st.idx) ? 1.0 : 0.0;
  } else if (lane < K) {
    const double pd = exp2((dl.z - double(st.m)) * cd) / st.s;
    if (a.mode == JSV_PROPOSAL_POINT) {
      sc.alpha = pd;
    } else {
      const double qd = exp2((double(dl.g) - double(st.mq)) * cd) / st.sq;
      sc.alpha = (pd == 0.0) ? 0.0 : (pd >= qd ? 1.0 : pd / qd);
    }
  }
  if (!soft) {
    const uint64_t rej = __ballot(lane < K && sc.alpha == 0.0);
    sc.k = rej ? __builtin_ctzll(rej) : K;
    const bool gap = act && lane <= sc.k && (st.m - st.top2) < kLogitGapTie;
    if (__ballot(gap)) sc.f |= JSV_FLAG_LOGIT_GAP;
  } else if (a.kind == kFinalizeVerify) {
    double u = 0.0, v = 0.0;
    if (act) row_uniforms(a.seed, a.offset, b, lane, u, v);
    const uint64_t rej = __ballot(lane < K && !(u < sc.alpha));
    sc.k = rej ? __builtin_ctzll(rej) : K;
    const bool tie = lane < K && lane <= sc.k && fabs(u - sc.alpha) < kAcceptTie;
    if (__ballot(tie)) sc.f |= JSV_FLAG_ACCEPT_TIE;
    sc.vk = readlane_d(v, sc.k);
  }
  return sc;
}

// Row k's statistics with the scan result (what the bonus sampler needs of the rule).
__device__ inline ReqState req_state(const FinalArgs& a, const Scan& sc) {
  ReqState rq{};
  if (sc.bad) {
    rq.k = -1; rq.dk = -1; rq.flags = JSV_FLAG_INVALID;
    return rq;
  }
  const int k = sc.k, K = a.K;
  rq.vk = sc.vk; rq.k = k; rq.flags = sc.f;
  rq.s = readlane_d(sc.st.s, k); rq.sq = readlane_d(sc.st.sq, k);
  rq.m = readlane_f(sc.st.m, k); rq.mq = readlane_f(sc.st.mq, k);
  const int dk = readlane_i(sc.di, k);
  rq.use_q = (a.mode == JSV_PROPOSAL_SOFTMAX && k < K) ? 1 : 0;
  rq.dk = (a.mode == JSV_PROPOSAL_POINT && k < K) ? dk : -1;
  return rq;
}

// Per-request outputs of verification: committed = d_0..d_{k-1}, bonus, then -1.
__device__ inline void write_verify(const FinalArgs& a, int b, const Scan& sc, int bonus, uint32_t f) {
  const int lane = threadIdx.x & (kWave - 1), K = a.K, row = b * (K + 1) + lane;
  if (lane <= K) a.committed[row] = sc.bad ? -1 : ((lane < sc.k) ? sc.di : (lane == sc.k ? bonus : -1));
  if (lane == 0) {
    a.n_accepted[b] = sc.bad ? -1 : sc.k;
    if (a.flags) a.flags[b] = sc.bad ? uint32_t(JSV_FLAG_INVALID) : f;
  }
}

__global__ __launch_bounds__(kWave) void scan_kernel(FinalArgs a) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int K = a.K, R = K + 1;
  const bool soft = a.T > 0.f;
  const bool act = lane <= K;
  const int row = b * R + lane;
  const Scan sc = scan_request(a, b);
  const ReqState rq = req_state(a, sc);
  if (lane == 0) a.req[b] = rq;
  if (sc.bad) {
    if (a.kind == kFinalizeVerify) write_verify(a, b, sc, -1, 0u);
    if (a.kind == kFinalizeAnchor && lane == 0) {
      a.n_accepted[b] = -1;
      a.committed[b] = -1;
      if (a.flags) a.flags[b] = JSV_FLAG_INVALID;
    }
    if (a.kind == kFinalizeScore) {
      if (lane < a.top_n) {
        a.out_len[b * a.top_n + lane] = -1;
        a.out_token[b * a.top_n + lane] = -1;
        a.out_prob[b * a.top_n + lane] = 0.f;
      }
      if (act && a.len_marginal) a.len_marginal[row] = 0.0;
      if (lane == 0 && a.flags) a.flags[b] = JSV_FLAG_INVALID;
    }
    return;
  }
  const int k = sc.k;
  const double alpha = sc.alpha;
  const int bonus = readlane_i(sc.st.idx, k);

  // A_i = prod_{j<i} alpha_j (probability of reaching row i).
  double A = 1.0;
  for (int j = 0; j < K; ++j) {
    const double aj = readlane_d(alpha, j);
    if (j < lane) A *= aj;
  }
  if (act) {
    const Stat& st = sc.st;
    RowFinal rf{};
    rf.s = st.s; rf.sq = st.sq; rf.alpha = alpha; rf.A = A;
    rf.m = st.m; rf.top2 = st.top2; rf.mq = st.mq; rf.idx = st.idx; rf.flags = st.flags;
    a.rowfinal[row] = rf;
  }
  if (a.kind == kFinalizeAnchor) {  // greedy rule on decoder logits: position and token
    if (lane == 0) {
      a.n_accepted[b] = k;
      a.committed[b] = bonus;
      if (a.flags) a.flags[b] = sc.f;
    }
    return;
  }
  if (a.kind == kFinalizeVerify) {
    // T = 0: the bonus is the argmax of row k.  T > 0 verification draws it in the
    // sampler kernels, which run this scan themselves.
    write_verify(a, b, sc, soft ? -1 : bonus, sc.f);
  } else {  // score
    if (act && a.len_marginal) {
      a.len_marginal[row] = soft ? ((lane < K) ? A * (1.0 - alpha) : A) : (lane == k ? 1.0 : 0.0);
    }
    if (!soft && lane < a.top_n) {  // all mass on the greedy outcome
      a.out_len[b * a.top_n + lane] = (lane == 0) ? k : -1;
      a.out_token[b * a.top_n + lane] = (lane == 0) ? bonus : -1;
      a.out_prob[b * a.top_n + lane] = (lane == 0) ? 1.f : 0.f;
    }
    if (lane == 0 && a.flags) a.flags[b] = sc.f;
  }
}

// ------------------------------------------------------------------------------------
// Block-level helpers for the slice kernels (kSliceThreads = 256 = 4 waves).
__device__ inline double block_sum(double x, double* sh) {
  x = wave_sum(x);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) sh[w] = x;
  __syncthreads();
  double t = 0.0;
  for (int i = 0; i < kSliceThreads / kWave; ++i) t += sh[i];
  __syncthreads();
  return t;
}

// Residual value r(v) and target probability p(v) of row k (paper §3; App. F.3).
struct RowModel {
  float m, mq, c;
  double s, sq;
  bool use_q;
  int dk;
  __device__ inline void eval(int64_t v, float z, float g, double& r, double& p) const {
    p = double(exp2f((z - m) * c)) / s;
    if (use_q) {
      const double q = double(exp2f((g - mq) * c)) / sq;
      r = p > q ? p - q : 0.0;
    } else {
      r = (v == dk) ? 0.0 : p;
    }
  }
};

__device__ inline RowModel row_model(const RowFinal& rf, float c, int mode, int k, int K, int dk) {
  RowModel rm;
  rm.m = rf.m; rm.mq = rf.mq; rm.c = c; rm.s = rf.s; rm.sq = rf.sq;
  rm.use_q = (mode == JSV_PROPOSAL_SOFTMAX) && k < K;
  rm.dk = (mode == JSV_PROPOSAL_POINT && k < K) ? dk : -1;
  return rm;
}

__device__ inline RowModel req_model(const ReqState& rq, float c) {
  RowModel rm;
  rm.m = rq.m; rm.mq = rq.mq; rm.c = c; rm.s = rq.s; rm.sq = rq.sq;
  rm.use_q = rq.use_q != 0;
  rm.dk = rq.dk;
  return rm;
}

// ------------------------------------------------------------------------------------
// Bonus sampler, part 1: grid (slices of kSampleSlice columns, B).  Residual mass (and
// target mass, for the zero-residual fallback) of row k over each slice.
__global__ __launch_bounds__(kSliceThreads) void slice_sum_kernel(SampleArgs a) {
  const int b = blockIdx.y, j = blockIdx.x, tid = threadIdx.x, NB = gridDim.x;
  __shared__ ReqState rq_sh;
  if (tid < kWave) {
    const ReqState r = req_state(a.f, scan_request(a.f, b));
    if (tid == 0) rq_sh = r;
  }
  __syncthreads();
  const ReqState rq = rq_sh;
  if (rq.k < 0) return;
  const int K = a.f.K, k = rq.k, row = b * (K + 1) + k;
  const RowModel rm = req_model(rq, a.c);
  const int64_t V = a.f.V;
  const uint32_t rowbytes = uint32_t(V) * 4u;
  const rsrc_t zr = make_rsrc(a.logits + (size_t)row * V, rowbytes);
  const rsrc_t gr = make_rsrc(rm.use_q ? a.G + (size_t)(b * K + k) * V : a.logits,
                              rm.use_q ? rowbytes : 0u);
  const int64_t v0 = (int64_t)j * kSampleSlice + tid;
  float z[kSampleCols], g[kSampleCols];
#pragma unroll
  for (int e = 0; e < kSampleCols; ++e) {
    const uint32_t off = uint32_t(v0 + e * kSliceThreads) * 4u;
    z[e] = bload4f(zr, off);
    g[e] = bload4f(gr, off);
  }
  double rs = 0.0, ps = 0.0;
#pragma unroll
  for (int e = 0; e < kSampleCols; ++e) {
    const int64_t v = v0 + e * kSliceThreads;
    if (v < V) {
      double r, p;
      rm.eval(v, z[e], g[e], r, p);
      rs += r;
      ps += p;
    }
  }
  __shared__ double dsh[8];
  rs = block_sum(rs, dsh);
  ps = block_sum(ps, dsh);
  if (tid == 0) {
    a.zs[((size_t)b * NB + j) * 2 + 0] = rs;
    a.zs[((size_t)b * NB + j) * 2 + 1] = ps;
  }
}

// Bonus sampler, part 2: grid B, one wave.  t = v_k * Z is located among the slice
// totals (rounds of 64 slices: a running base plus a wave prefix sum), then inside the
// chosen slice (16 consecutive columns per lane): the token is the first column whose
// CDF exceeds t.  Both passes over the slice totals form every sum in the same order,
// so the CDF they walk ends exactly at the Z that t was taken from.
constexpr int kLocRounds = 4;  // slice-total rounds kept in registers (V <= 262144)

__global__ __launch_bounds__(kWave) void locate_kernel(SampleArgs a) {
  constexpr int CR = kSampleSlice / kWave;  // columns per lane inside a slice
  const int b = blockIdx.x, lane = threadIdx.x;
  const int NB = sample_slices(a.f.V), rounds = (NB + kWave - 1) / kWave;
  const rsrc_t zsr = make_rsrc(a.zs + (size_t)b * NB * 2, uint64_t(NB) * 16u);
  uint4 pre[kLocRounds];
#pragma unroll
  for (int q = 0; q < kLocRounds; ++q) pre[q] = bload16(zsr, uint32_t(q * kWave + lane) * 16u, 0);
  auto totals = [&](int q) {
    uint4 x = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int i = 0; i < kLocRounds; ++i)
      if (q == i) x = pre[i];
    if (q >= kLocRounds) x = bload16(zsr, uint32_t(q * kWave + lane) * 16u, 0);
    return x;
  };
  const Scan sc = scan_request(a.f, b);
  if (sc.bad) {
    write_verify(a.f, b, sc, -1, 0u);
    return;
  }
  const ReqState rq = req_state(a.f, sc);
  const int K = a.f.K, k = rq.k, row = b * (K + 1) + k;
  const RowModel rm = req_model(rq, a.c);
  const int64_t V = a.f.V;

  // pass 1: both totals
  double Zr = 0.0, Zp = 0.0;
  for (int q = 0; q < rounds; ++q) {
    const uint4 x = totals(q);
    Zr += wave_sum(u2d(x.x, x.y));
    Zp += wave_sum(u2d(x.z, x.w));
  }
  const int zero = (Zr > 0.0) ? 0 : 1;  // no residual mass: draw from p_k (flagged)
  const double Z = zero ? Zp : Zr;
  const double t = rq.vk * Z;

  // pass 2: the slice whose CDF step holds t
  double base = 0.0, sbase = 0.0, slast_base = 0.0;
  int s = -1, slast = -1;
  for (int q = 0; q < rounds && s < 0; ++q) {
    const uint4 x4 = totals(q);
    const double x = zero ? u2d(x4.z, x4.w) : u2d(x4.x, x4.y);
    const double inc = wave_incl_scan(x);
    const double hi = base + inc, lo = hi - x;
    const uint64_t hit = __ballot(x > 0.0 && hi > t);
    const uint64_t pos = __ballot(x > 0.0);
    if (hit) {
      const int l = __builtin_ctzll(hit);
      s = q * kWave + l;
      sbase = readlane_d(lo, l);
    } else if (pos) {
      const int l = 63 - __builtin_clzll(pos);
      slast = q * kWave + l;
      slast_base = readlane_d(lo, l);
    }
    base += readlane_d(inc, kWave - 1);
  }
  bool fall = s < 0;  // rounding left t at or above the last step: take the last mass
  if (fall) { s = slast; sbase = slast_base; }

  // Inside slice s, lane l takes the CR consecutive columns c0 + CR l + j: each lane sums
  // its own columns in order, one wave scan places the lanes, and every lane walks its
  // columns against t in parallel; the token is the first (lane, column) whose CDF
  // exceeds t.
  const uint32_t rowbytes = uint32_t(V) * 4u;
  const rsrc_t zr = make_rsrc(a.logits + (size_t)row * V, rowbytes);
  const rsrc_t gr = make_rsrc(rm.use_q ? a.G + (size_t)(b * K + k) * V : a.logits,
                              rm.use_q ? rowbytes : 0u);
  const int64_t c0 = (int64_t)s * kSampleSlice, cl = c0 + int64_t(lane) * CR;
  float z[CR], g[CR];
#pragma unroll
  for (int e = 0; e < CR; ++e) {
    const uint32_t off = uint32_t(cl + e) * 4u;
    z[e] = bload4f(zr, off);
    g[e] = bload4f(gr, off);
  }
  double x[CR];
  double own = 0.0;  // this lane's columns, summed in column order
#pragma unroll
  for (int e = 0; e < CR; ++e) {
    const int64_t v = cl + e;
    double r = 0.0, p = 0.0;
    if (s >= 0 && v < V) rm.eval(v, z[e], g[e], r, p);
    x[e] = zero ? p : r;
    own += x[e];
  }
  const double lbase = sbase + (wave_incl_scan(own) - own);  // CDF before this lane's columns
  int je = -1, jl = -1;  // first column whose CDF exceeds t; last column with mass
  double C = lbase, clo = 0.0, chi = 0.0;
#pragma unroll
  for (int e = 0; e < CR; ++e) {
    const double lo = C;
    C += x[e];
    if (x[e] > 0.0) {
      jl = e;
      if (je < 0 && C > t) { je = e; clo = lo; chi = C; }
    }
  }
  int tok = -1, lastpos = -1;
  const uint64_t hit = fall ? 0ull : __ballot(je >= 0);
  if (hit) {
    const int l = __builtin_ctzll(hit);
    tok = int(c0) + l * CR + readlane_i(je, l);
    clo = readlane_d(clo, l);
    chi = readlane_d(chi, l);
  }
  const uint64_t pos = __ballot(jl >= 0);
  if (pos) {
    const int l = 63 - __builtin_clzll(pos);
    lastpos = int(c0) + l * CR + readlane_i(jl, l);
  }
  uint32_t f = zero ? uint32_t(JSV_FLAG_ZERO_RESIDUAL) : 0u;
  if (tok >= 0) {
    if ((t - clo) < kCdfTie || (chi - t) < kCdfTie) f |= JSV_FLAG_CDF_TIE;
  } else {
    tok = lastpos;
    f |= JSV_FLAG_CDF_TIE;
  }
  write_verify(a.f, b, sc, tok, sc.f | f);
}

// ------------------------------------------------------------------------------------
// Cache hit test (paper §4.1): grid B, one wave; lane i compares cached entry i (and
// i + 64 beyond) with the realised (k, a).
__global__ __launch_bounds__(kWave) void lookup_kernel(const int* n_accepted, const int* committed,
                                                       int K, const int* out_len, const int* out_token,
                                                       int top_n, int* hit) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int k = n_accepted[b];
  const int a = (k >= 0 && k <= K) ? committed[b * (K + 1) + k] : -1;
  int found = -1;
  for (int i0 = 0; i0 < top_n && found < 0; i0 += kWave) {
    const int i = i0 + lane;
    const bool m = k >= 0 && k <= K && i < top_n && out_len[b * top_n + i] == k &&
                   out_token[b * top_n + i] == a;
    const uint64_t mask = __ballot(m);
    if (mask) found = i0 + __builtin_ctzll(mask);
  }
  if (lane == 0) hit[b] = found;
}

// Calibrated length score (paper App. B.1): grid B, one wave; lane k forms
// G(k) = prod_{i<=k} p_i from the estimates read into scalar registers in order.
__global__ __launch_bounds__(kWave) void lengths_kernel(const double* p, int K, double* out,
                                                        uint32_t* flags) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const double pl = (lane < K) ? p[b * K + lane] : 1.0;
  const bool bad = __ballot(lane < K && !(pl >= 0.0 && pl <= 1.0)) != 0;
  double G = 1.0, Gn = 1.0;  // G(lane), G(lane + 1)
  for (int i = 0; i < K; ++i) {
    const double pi = readlane_d(pl, i);
    if (i < lane) G *= pi;
    if (i <= lane) Gn *= pi;
  }
  if (lane == K) Gn = 0.0;
  if (lane <= K) out[b * (K + 1) + lane] = bad ? 0.0 : G - Gn;
  if (lane == 0 && flags) flags[b] = bad ? uint32_t(JSV_FLAG_INVALID) : 0u;
}

// ------------------------------------------------------------------------------------
// Outcome scorer, part 1: grid (slices, K+1, B).  Residual mass of (row k, slice) and its
// top-(N+1) columns by (r desc, p desc, token asc).
struct Key {
  double r, p;
  int v;
};
__device__ inline bool key_better(const Key& x, const Key& y) {
  if (x.r != y.r) return x.r > y.r;
  if (x.p != y.p) return x.p > y.p;
  return x.v < y.v;
}

template <int CTRL>
__device__ inline void key_dpp_max(Key& k) {
  Key o;
  o.r = dppd<CTRL>(k.r); o.p = dppd<CTRL>(k.p); o.v = int(dpp32<CTRL>(uint32_t(k.v)));
  if (key_better(o, k)) k = o;
}

__device__ inline Key block_best(Key k, Key* sh) {
  key_dpp_max<0xB1>(k);
  key_dpp_max<0x4E>(k);
  key_dpp_max<0x124>(k);
  key_dpp_max<0x128>(k);
  Key r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // the four row winners, in every lane
    r[i].r = readlane_d(k.r, 16 * i); r[i].p = readlane_d(k.p, 16 * i); r[i].v = readlane_i(k.v, 16 * i);
  }
  k = r[0];
#pragma unroll
  for (int i = 1; i < 4; ++i)
    if (key_better(r[i], k)) k = r[i];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) sh[w] = k;
  __syncthreads();
  Key best = sh[0];
  for (int i = 1; i < kSliceThreads / kWave; ++i)
    if (key_better(sh[i], best)) best = sh[i];
  __syncthreads();
  return best;
}

__global__ __launch_bounds__(kSliceThreads) void score_slice_kernel(ScoreArgs a) {
  const int b = blockIdx.z, k = blockIdx.y, j = blockIdx.x, NB = gridDim.x, tid = threadIdx.x;
  const ReqState rq = a.req[b];
  if (!(a.T > 0.f) || rq.k < 0) return;
  const int K = a.K, R = K + 1, row = b * R + k, N1 = a.top_n + 1;
  const RowFinal rf = a.rowfinal[row];
  const int64_t V = a.V;
  const double Pk = (k < K) ? rf.A * (1.0 - rf.alpha) : rf.A;
  const RowModel rm = row_model(rf, a.c, a.mode, k, K, k < K ? a.drafts[b * K + k] : -1);
  const float* zr = a.logits + (size_t)row * V;
  const float* gr = rm.use_q ? a.G + (size_t)(b * K + k) * V : nullptr;
  const int64_t L = (V + NB - 1) / NB;
  const int64_t v0 = (int64_t)j * L;
  const int n = (int)max<int64_t>(0, min<int64_t>(V, v0 + L) - v0);

  __shared__ double rsh[kScoreMaxSlice];
  __shared__ double psh[kScoreMaxSlice];
  __shared__ double dsh[8];
  __shared__ Key ksh[8];

  Cand* cand = a.cand + ((size_t)row * NB + j) * N1;
  if (!(Pk > 0.0)) {  // the row contributes no outcome
    if (tid == 0) a.zs[(size_t)row * NB + j] = 0.0;
    for (int q = tid; q < N1; q += kSliceThreads) {
      Cand cd{};
      cd.r = -1.0; cd.p = -1.0; cd.tok = -1;
      cand[q] = cd;
    }
    return;
  }
  for (int e = tid; e < n; e += kSliceThreads) {
    double r, p;
    rm.eval(v0 + e, zr[v0 + e], gr ? gr[v0 + e] : 0.f, r, p);
    rsh[e] = r;
    psh[e] = p;
  }
  __syncthreads();
  const int E = (n + kSliceThreads - 1) / kSliceThreads;
  const int e0 = tid * E, e1 = min(n, e0 + E);
  double rs = 0.0;
  for (int e = e0; e < e1; ++e) rs += rsh[e];
  rs = block_sum(rs, dsh);
  if (tid == 0) a.zs[(size_t)row * NB + j] = rs;
  Key thr{INFINITY, INFINITY, -1};
  for (int q = 0; q < N1; ++q) {
    Key best{-1.0, -1.0, INT_MAX};
    for (int e = e0; e < e1; ++e) {
      const Key x{rsh[e], psh[e], int(v0 + e)};
      if (key_better(thr, x) && key_better(x, best)) best = x;
    }
    best = block_best(best, ksh);
    if (tid == 0) {
      Cand cd{};
      cd.r = best.r; cd.p = best.p; cd.tok = (best.v == INT_MAX) ? -1 : best.v;
      cand[q] = cd;
    }
    thr = best;
  }
}

// Outcome scorer, part 2: grid (B).  Residual mass per row, then P(k, a) of every
// candidate and the top-N by (P desc, k asc, a asc).
__global__ __launch_bounds__(kSliceThreads) void score_merge_kernel(ScoreArgs a) {
  const int b = blockIdx.x, tid = threadIdx.x, NB = score_slices(a.V);
  const ReqState rq = a.req[b];
  if (!(a.T > 0.f) || rq.k < 0) return;
  const int K = a.K, R = K + 1, N1 = a.top_n + 1;
  __shared__ double scale_sh[kMaxK + 1];
  __shared__ double zk_sh[kMaxK + 1];
  __shared__ int usep_sh[kMaxK + 1];
  __shared__ uint32_t flag_sh;
  __shared__ Key ksh[8];
  if (tid == 0) flag_sh = 0u;
  {
    const int w = tid >> 6, lane = tid & 63;
    for (int kk = w; kk < R; kk += kSliceThreads / kWave) {
      double x = 0.0;
      for (int q = lane; q < NB; q += kWave) x += a.zs[((size_t)(b * R + kk)) * NB + q];
      x = wave_sum(x);
      if (lane == 0) zk_sh[kk] = x;
    }
  }
  __syncthreads();
  for (int kk = tid; kk < R; kk += kSliceThreads) {
    const RowFinal f2 = a.rowfinal[b * R + kk];
    const double P2 = (kk < K) ? f2.A * (1.0 - f2.alpha) : f2.A;
    const double Zk = zk_sh[kk];
    double sc = 0.0;
    int usep = 0;
    if (P2 > 0.0) {
      if (kk == K) { sc = P2; usep = 1; }
      else if (Zk > 0.0) { sc = P2 / Zk; }
      else { sc = P2; usep = 1; atomicOr(&flag_sh, JSV_FLAG_ZERO_RESIDUAL); }
    }
    scale_sh[kk] = sc;
    usep_sh[kk] = usep;
  }
  __syncthreads();

  const int total = R * NB * N1;
  const Cand* cb = a.cand + (size_t)b * R * NB * N1;
  // Merge key: r := P, p := -row, v := token (larger P, then smaller row, then smaller token).
  Key thr{INFINITY, INFINITY, -1};
  double prev = -1.0;
  for (int q = 0; q < N1; ++q) {
    Key best{-1.0, -1.0, INT_MAX};
    for (int e = tid; e < total; e += kSliceThreads) {
      const Cand cd = cb[e];
      if (cd.tok < 0) continue;
      const int kk = e / (NB * N1);
      const double P = scale_sh[kk] * (usep_sh[kk] ? cd.p : cd.r);
      if (!(P > 0.0)) continue;
      const Key x{P, -double(kk), cd.tok};
      if (key_better(thr, x) && key_better(x, best)) best = x;
    }
    best = block_best(best, ksh);
    thr = best;
    if (tid == 0) {
      const bool have = best.v != INT_MAX;
      if (q < a.top_n) {
        a.out_len[b * a.top_n + q] = have ? int(-best.p) : -1;
        a.out_token[b * a.top_n + q] = have ? best.v : -1;
        a.out_prob[b * a.top_n + q] = have ? float(best.r) : 0.f;
      }
      if (have && q > 0 && prev - best.r < kTopNTie * prev) flag_sh |= JSV_FLAG_TOPN_TIE;
      if (have) prev = best.r;
    }
  }
  __syncthreads();
  if (tid == 0 && a.flags) a.flags[b] |= flag_sh;
}

// ------------------------------------------------------------------------------------
// Launchers.
template <int DT, int NT, int NX, int NKS>
static hipError_t launch_stats_t(int grid, const StatsArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((stats_kernel<DT, NT, NX, NKS>), dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

#define JSV_NKS_LIST(X) X(1) X(2) X(4) X(8) X(12) X(16) X(20)

bool stats_supported(int dtype, int nks) {
  if (dtype != JSV_BF16 && dtype != JSV_F32 && dtype != JSV_FP8) return false;
  if (dtype == JSV_FP8 && (nks & 1)) return false;  // a 16-byte fp8 load spans two k-steps
  switch (nks) {
#define JSV_CASE(n) case n: return true;
    JSV_NKS_LIST(JSV_CASE)
#undef JSV_CASE
    default: return false;
  }
}

template <int DT, int NT, int NX>
static hipError_t dispatch_nks(int nks, int grid, const StatsArgs& a, hipStream_t s) {
  switch (nks) {
#define JSV_CASE(n)                                                          \
  case n:                                                                    \
    if constexpr (DT == JSV_FP8 && (n & 1)) return hipErrorInvalidValue;   \
    else return launch_stats_t<DT, NT, NX, n>(grid, a, s);
    JSV_NKS_LIST(JSV_CASE)
#undef JSV_CASE
    default: return hipErrorInvalidValue;
  }
}

// Tiling of `rows` (1..33) tokens: full 16-token MFMA tiles, plus one row on the VALU
// when exactly one row is left over.
template <int DT>
static hipError_t dispatch_rows(int nks, int grid, const StatsArgs& a, hipStream_t s) {
  const int rows = a.rp;
  if (rows <= 1) return dispatch_nks<DT, 0, 1>(nks, grid, a, s);
  if (rows <= 16) return dispatch_nks<DT, 1, 0>(nks, grid, a, s);
  if (rows == 17) return dispatch_nks<DT, 1, 1>(nks, grid, a, s);
  if (rows <= 32) return dispatch_nks<DT, 2, 0>(nks, grid, a, s);
  return dispatch_nks<DT, 2, 1>(nks, grid, a, s);
}

hipError_t launch_stats(int dtype, int nks, int grid, const StatsArgs& a, hipStream_t stream) {
  if (a.rp < 1 || a.rp > kRowsPerPass || a.npass < 1 || a.nchunk < 1 || grid != a.nchunk * a.npass ||
      a.M > a.rp * a.npass)
    return hipErrorInvalidValue;
  if (dtype == JSV_FP8) return dispatch_rows<JSV_FP8>(nks, grid, a, stream);
  return dtype == JSV_BF16 ? dispatch_rows<JSV_BF16>(nks, grid, a, stream)
                           : dispatch_rows<JSV_F32>(nks, grid, a, stream);
}

hipError_t launch_wide(const WideArgs& a, hipStream_t stream) {
  if (!wide_eligible(JSV_BF16, a.d, a.M) || a.pl.mp % 16 != 0 || a.pl.mp < a.M ||
      a.pl.mp > 16 * a.pl.nw || a.pl.mp > kWideMaxRows ||
      a.pl.S * kWideBlock != a.d || a.pl.nchunk < 1 || a.pl.ncomb < 1 || a.pl.ncomb > kMaxGrid)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(xhat_kernel, dim3(a.M), dim3(kSliceThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.pl.nw == 8)
    hipLaunchKernelGGL(wide_kernel<8>, dim3(a.pl.nchunk * a.pl.S), dim3(8 * kWave), 0, stream, a);
  else
    hipLaunchKernelGGL(wide_kernel<9>, dim3(a.pl.nchunk * a.pl.S), dim3(9 * kWave), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (a.pl.S) {
#define JSV_WIDE_S(n)                                                                            \
  case n:                                                                                        \
    hipLaunchKernelGGL(wide_stats_kernel<n>, dim3(a.pl.ncomb, a.pl.mp / 16), dim3(kWideCombineThreads), 0, \
                       stream, a);                                                              \
    break;
    JSV_WIDE_S(1) JSV_WIDE_S(2) JSV_WIDE_S(3) JSV_WIDE_S(4) JSV_WIDE_S(5)
#undef JSV_WIDE_S
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_rowstat(const FinalArgs& a, hipStream_t stream) {
  const int tasks = (a.T > 0.f ? a.K : 0) + a.K + 1;
  hipLaunchKernelGGL(rowstat_kernel, dim3(tasks, a.B), dim3(kWave), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_scan(const FinalArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(scan_kernel, dim3(a.B), dim3(kWave), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_lookup(const int* n_accepted, const int* committed, int B, int K, const int* out_len,
                         const int* out_token, int top_n, int* hit, hipStream_t stream) {
  hipLaunchKernelGGL(lookup_kernel, dim3(B), dim3(kWave), 0, stream, n_accepted, committed, K,
                     out_len, out_token, top_n, hit);
  return hipGetLastError();
}

hipError_t launch_lengths(const double* p, int B, int K, double* out, uint32_t* flags,
                          hipStream_t stream) {
  hipLaunchKernelGGL(lengths_kernel, dim3(B), dim3(kWave), 0, stream, p, K, out, flags);
  return hipGetLastError();
}

hipError_t launch_sample(const SampleArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(slice_sum_kernel, dim3(sample_slices(a.f.V), a.f.B), dim3(kSliceThreads), 0,
                     stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(locate_kernel, dim3(a.f.B), dim3(kWave), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_score(const ScoreArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(score_slice_kernel, dim3(score_slices(a.V), a.K + 1, a.B),
                     dim3(kSliceThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(score_merge_kernel, dim3(a.B), dim3(kSliceThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace jsv
