// Sampled verification from raw logits ("Inference Engineering Part 5/8",
// opening section for the sampling settings and section "Exactness Means
// Different Things For Greedy And Sampled Output" for the rule: accept with
// probability min(1, p(x)/q(x)), replace from normalize(max(0, p - q)), bonus
// from the target after the full draft; the draft and the target use the same
// sampling settings).  p and q are softmax(logits / temperature) of the target
// and draft rows, formed on the fly: e(v) = exp((l(v) - M) * (1/T)) with M the
// row maximum, p(v) = e(v) * (1/Z), the exponent reduced in fp64 and the
// exponential of its fraction taken by the hardware's fp32 exp2 (exp2_fast:
// about 1e-7 relative error, ten times inside the 1e-6 tolerance the decisions
// are held to).  Sums and every comparison are in fp64.
//
// With top-p the distribution is cut to its nucleus first: every id whose
// logit is at least t, where t is the largest logit value such that the ids at
// or above it hold at least top_p of the row's mass; ties at t are all kept,
// and p is renormalised over the nucleus.
//
// Three launches (four with top-p); the workspace keeps nothing between calls:
//  1. k_sl_stats: one workgroup per (split of kSlStatChunk logits, row, batch row)
//     writes the split's maximum and its exp-sum relative to that maximum; the
//     split that holds the row's draft token also leaves that token's logit.
//  1b. k_sl_nucleus (top-p only): one workgroup per (row, batch row) selects t
//     level by level, each level one read of the row: the first bins the
//     logits by (M - l) / T, the second the chosen bin's logits more finely,
//     the later ones the order keys of the chosen bin's interval; masses are
//     2^-41 fixed-point integers, so every sum is exact and order-free, and Z
//     is the fixed-point mass at or above t.
//  2. k_sl_mass: one workgroup per (split, batch row) evaluates every
//     acceptance test (the same result in every workgroup of a batch row) and
//     sums the stop row's residual mass max(0, p - q) (or p at position D) over
//     its split and over each thread's run of kSlRun ids.
//  3. k_sl_draw: one workgroup per (split, batch row); the one whose split
//     holds the crossing of u * T finds the run, then the id.
#include <math.h>
#include <limits.h>
#include "device_common.h"
#include "launch.h"
#include "wave_dpp.h"
#include "specdec.h"

// p and q are each rounded before p - q is formed (as the definition has it):
// no multiply-add contraction, which would leave p's rounding error in a
// residual that is exactly 0 when p = q.
#pragma clang fp contract(off)

namespace sd {

constexpr int kSlRun = kSlChunk / kSlThreads;  // ids of one thread's run of the stop row
static_assert(kSlChunk % kSlThreads == 0 && kSlRun <= kWave, "a thread run must fit one wave");
static_assert(kSlThreads >= 256 && kSlThreads % kWave == 0, "one thread per draft position, D <= 255");
static_assert(kSlStatThreads % kWave == 0, "whole waves");

// Logits per 16-byte vector, and whether PER logits of a thread are whole vectors.
template <int DT, int PER>
struct SlVec {
  static constexpr int E = DT == SPECDEC_F32 ? 4 : 8;
  static constexpr bool ok = PER % E == 0;
};
constexpr int kSlMaxRows = 2 * 255 + 1;     // 2D + 1 rows per batch row, D <= 255
constexpr int kSlMaxSplits = (1 << 22) / kSlChunk;  // V <= 2^22

template <int DT>
__device__ __forceinline__ float logit_at(const void *base, int64_t i) {
  if (DT == SPECDEC_F32) return static_cast<const float *>(base)[i];
  const uint32_t h = static_cast<const uint16_t *>(base)[i];
  return DT == SPECDEC_F16 ? f16_bits_to_f32(h) : bf16_bits_to_f32(h);
}

// 2^t for t <= 0 with about 1e-7 relative error, t = y log2(e) for e^y: t =
// n + f in fp64 with n an integer and |f| <= 1/2; 2^f by the hardware's fp32
// exp2 (f rounded to fp32 costs at most 2e-8 relative, the instruction a few
// times 6e-8 on [2^-1/2, 2^1/2]); then scaled by 2^n.  t is clamped at -1100
// first, where the scaling underflows to 0, so -inf and NaN give 0 with no
// branch or select (the exponentials of a thread's ids then interleave), and
// anything below about -1074 gives 0 as well.  Callers form t from an exact
// fp64 difference times (1/T) log2(e), one rounding.  About a third of the fp64
// instructions of the library exp.
constexpr double kLog2e = 0x1.71547652b82fep+0;

__device__ __forceinline__ double exp2_fast(double t) {
  const double tc = fmax(t, -1100.0);
  const double n = rint(tc);
  const float f = (float)(tc - n);
  return ldexp((double)__builtin_amdgcn_exp2f(f), (int)n);
}

// Row maximum M and 1/Z from the per-split statistics (split order).  Loads
// are issued kBatch splits at a time, and the first kBatch are kept for the
// sum, so a row of up to kBatch splits costs one round trip.
constexpr int kBatch = 8;

// c2 = (1/T) log2(e).
__device__ __forceinline__ void merge_row(const double *st, int S, double c2, double &M, double &inv_z) {
  double m0[kBatch], z0[kBatch];
#pragma unroll
  for (int k = 0; k < kBatch; ++k) {
    m0[k] = k < S ? st[2 * k] : -INFINITY;
    z0[k] = k < S ? st[2 * k + 1] : 0.0;
  }
  double m = -INFINITY;
#pragma unroll
  for (int k = 0; k < kBatch; ++k) m = fmax(m, m0[k]);
  for (int s0 = kBatch; s0 < S; s0 += kBatch) {
    double ms[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) ms[k] = s0 + k < S ? st[2 * (s0 + k)] : -INFINITY;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) m = fmax(m, ms[k]);
  }
  double z = 0.0;
#pragma unroll
  for (int k = 0; k < kBatch; ++k) {
    const double e = z0[k] * exp2_fast((m0[k] - m) * c2);
    z += m0[k] > -INFINITY ? e : 0.0;
  }
  for (int s0 = kBatch; s0 < S; s0 += kBatch) {
    double ms[kBatch], zs[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      ms[k] = s0 + k < S ? st[2 * (s0 + k)] : -INFINITY;
      zs[k] = s0 + k < S ? st[2 * (s0 + k) + 1] : 0.0;
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const double e = zs[k] * exp2_fast((ms[k] - m) * c2);
      z += ms[k] > -INFINITY ? e : 0.0;
    }
  }
  M = m;
  inv_z = 1.0 / z;
}

__device__ __forceinline__ int64_t target_row(const SampleLogitsParams &p, int b, int i) {
  return ((int64_t)b * (p.D + 1) + i) * p.V;
}
__device__ __forceinline__ int64_t draft_row(const SampleLogitsParams &p, int b, int i) {
  return ((int64_t)b * p.D + i) * p.V;
}

// Logits are streamed with non-temporal loads: read once, they do not
// allocate in the caches, and so they do not evict the dirty lines a preceding
// write-heavy kernel leaves in the Infinity Cache, whose write-back made
// ordinary loads twice as slow (statistics on the stoch logits: 28.9 against
// 16.1 us after a 512 MiB fill; alike after a read).
#define SL_LOAD(ptr) __builtin_nontemporal_load(ptr)
// kSlStatPer logits of one statistics split for this thread: id
// threadIdx.x + k * kSlStatThreads (scalar loads) or, with 16-byte vectors of
// E = 16 / esize logits, ids (threadIdx.x + j * kSlStatThreads) * E + e for
// vector j and lane e.  Ids at or past n read as -inf.  Every vector load is
// issued before any is used (an index past the split's whole vectors re-reads
// its last one, never used); the ragged end of a split, if any, is read by
// scalar loads afterwards.
template <int DT, bool VEC>
__device__ __forceinline__ void load_split(const void *base, int64_t off, int n, float *x) {
  if (VEC && SlVec<DT, kSlStatPer>::ok) {
    constexpr int E = SlVec<DT, kSlStatPer>::E;
    constexpr int NV = kSlStatPer / E;
    const int nv = n / E;  // whole vectors of the split
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 *vp = DT == SPECDEC_F32
                          ? reinterpret_cast<const u32x4 *>(static_cast<const float *>(base) + off)
                          : reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(base) + off);
    u32x4 v[NV];
    if (nv > 0) {
#pragma unroll
      for (int j = 0; j < NV; ++j) v[j] = SL_LOAD(vp + min((int)threadIdx.x + j * kSlStatThreads, nv - 1));
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int vi = threadIdx.x + j * kSlStatThreads;
      const uint32_t w[4] = {v[j][0], v[j][1], v[j][2], v[j][3]};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (DT == SPECDEC_F32) {
          x[j * E + e] = __uint_as_float(w[e]);
        } else {
          x[j * E + 2 * e] = DT == SPECDEC_F16 ? f16_bits_to_f32(w[e] & 0xFFFFu) : bf16_bits_to_f32(w[e] & 0xFFFFu);
          x[j * E + 2 * e + 1] = DT == SPECDEC_F16 ? f16_bits_to_f32(w[e] >> 16) : bf16_bits_to_f32(w[e] >> 16);
        }
      }
      if (vi >= nv) {
#pragma unroll
        for (int e = 0; e < E; ++e) x[j * E + e] = vi * E + e < n ? logit_at<DT>(base, off + vi * E + e) : -INFINITY;
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < kSlStatPer; ++k) {
      const int i = threadIdx.x + k * kSlStatThreads;
      x[k] = i < n ? logit_at<DT>(base, off + i) : -INFINITY;
    }
  }
}

// Thread and slot of load_split's x[] that hold the split's id lx.
template <int DT, bool VEC>
__device__ __forceinline__ void split_owner(int lx, int &thread, int &slot) {
  if (VEC && SlVec<DT, kSlStatPer>::ok) {
    constexpr int E = SlVec<DT, kSlStatPer>::E;
    const int vi = lx / E;
    thread = vi % kSlStatThreads;
    slot = (vi / kSlStatThreads) * E + lx % E;
  } else {
    thread = lx % kSlStatThreads;
    slot = lx / kSlStatThreads;
  }
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kSlStatThreads) void k_sl_stats(SampleLogitsParams p) {
  __shared__ float s_f[kSlStatThreads / kWave];
  __shared__ double s_d[kSlStatThreads / kWave];
  const int s = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
  const int D = p.D, R = 2 * D + 1;
  const void *base = r <= D ? p.target : p.draftl;
  const int64_t off = (r <= D ? target_row(p, b, r) : draft_row(p, b, r - D - 1)) + (int64_t)s * kSlStatChunk;
  const int n = min(kSlStatChunk, p.V - s * kSlStatChunk);
  // the draft token this row is tested at: target rows i < D and draft rows
  const int gi = r < D ? r : r - D - 1;
  const int gx = r != D ? p.draft[(int64_t)b * D + gi] : -1;
  float x[kSlStatPer];
  load_split<DT, VEC>(base, off, n, x);
  // the split that holds the token leaves its logit for the acceptance test
  const int lx = gx - s * kSlStatChunk;
  if (r != D && lx >= 0 && lx < n) {
    int owner, slot;
    split_owner<DT, VEC>(lx, owner, slot);
    if ((int)threadIdx.x == owner) {
      float v = x[0];
#pragma unroll
      for (int k = 1; k < kSlStatPer; ++k) v = k == slot ? x[k] : v;
      p.gath[((int64_t)b * D + gi) * 2 + (r > D ? 1 : 0)] = v;
    }
  }
  const double c2 = p.inv_t * kLog2e;
  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < kSlStatPer; ++k) m = fmaxf(m, x[k]);
  m = block_max_f32<kSlStatThreads>(m, s_f);
  double z = 0.0;
  if (m > -INFINITY) {
    const double md = (double)m;
#pragma unroll
    for (int k = 0; k < kSlStatPer; ++k) z += exp2_fast(((double)x[k] - md) * c2);  // -inf past n: 0
  }
  z = block_sum_d<kSlStatThreads>(z, s_d);
  if (threadIdx.x == 0) {
    double *st = p.stats + (((int64_t)b * R + r) * p.Ss + s) * 2;
    st[0] = (double)m;
    st[1] = z;
  }
}

// ------------------------------------------------------------------ top-p
#ifndef SPECDEC_NUC_THREADS
#define SPECDEC_NUC_THREADS 512
#endif
constexpr int kNucThreads = SPECDEC_NUC_THREADS;  // threads per nucleus workgroup
constexpr int kNucBins = 2048;      // first level: bins in u = -kNucScale t
constexpr int kNucSub = 1024;       // later levels: bins in the order key
constexpr int kNucUnroll = 3;       // 16-byte vectors in flight per thread (4 spills under the VGPR cap)
// three workgroups per CU (their LDS fits; 768 rows resident at once): at
// most 80 VGPRs
#ifndef SPECDEC_NUC_WAVES
#define SPECDEC_NUC_WAVES 6
#endif
constexpr int kNucWavesPerSimd = SPECDEC_NUC_WAVES;
constexpr double kFix = 2199023255552.0;  // 2^41: V <= 2^22 masses <= 1 sum below 2^63
// 2^t * 2^41 rounds to a fixed-point mass of 0 for every t <= -kNucSpan: the
// first level's bins are units of u = -t kNucScale over (-kNucSpan, 0] (u <
// 2016, the top 2016 of the bins), and logits past it (with -inf and NaN) go to
// one spare slot per lane past the bins, which no selection reads
constexpr double kNucSpan = 42.0;
constexpr double kNucScale = 48.0;
constexpr int kNucSlots = kNucBins + kWave;
static_assert(kNucSpan * kNucScale < kNucBins, "u below the bin count");

// Order key of a logit: larger key = larger value; -0.0 is folded onto +0.0
// (by adding +0.0) so equal values share a key.
__device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t u = __float_as_uint(v + 0.0f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// The largest float at or below d, and the smallest at or above it.
__device__ __forceinline__ float float_below(double d) {
  const float f = (float)d;
  return (double)f > d ? nextafterf(f, -INFINITY) : f;
}
__device__ __forceinline__ float float_above(double d) {
  const float f = (float)d;
  return (double)f < d ? nextafterf(f, INFINITY) : f;
}

// The fixed-point mass round(2^t * 2^41) (ties to even) for -kNucSpan < t <= 0:
// 2^t = e 2^n as in exp2_fast, e the fp32 exp2 of the fraction; e 2^(n + 41) <
// 2^42 is exact in fp64, and adding 2^52 rounds it to an integer that the low
// 52 bits of the sum hold.
__device__ __forceinline__ unsigned long long fixed41(double t) {
  const double n = rint(t);
  const float e = __builtin_amdgcn_exp2f((float)(t - n));
  const double v = ldexp((double)e, (int)n + 41);
  return (unsigned long long)__double_as_longlong(v + 0x1p52) & 0xFFFFFFFFFFFFFull;
}

// The logits of one 16-byte vector, in order: f(x).
template <int DT, class F>
__device__ __forceinline__ void each_in_vector(const uint4 &v, F &&f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (DT == SPECDEC_F32) {
      f(__uint_as_float(w[e]));
    } else {
      f(DT == SPECDEC_F16 ? f16_bits_to_f32(w[e] & 0xFFFFu) : bf16_bits_to_f32(w[e] & 0xFFFFu));
      f(DT == SPECDEC_F16 ? f16_bits_to_f32(w[e] >> 16) : bf16_bits_to_f32(w[e] >> 16));
    }
  }
}

// Every logit of one row for this thread of kNucThreads, in any order: f(x).
// Vectors go kNucUnroll at a time, every load issued before any is used: whole
// batches with no test, then the last batch with clamped loads (a repeated
// load, never used) and a test per vector.
template <int DT, bool VEC, class F>
__device__ __forceinline__ void each_logit(const void *base, int64_t off, int V, F &&f) {
  if (VEC) {
    constexpr int E = DT == SPECDEC_F32 ? 4 : 8;
    const int nv = V / E;
    const uint4 *row = reinterpret_cast<const uint4 *>(static_cast<const char *>(base) + off * (16 / E));
    int j0 = threadIdx.x;
    for (; j0 + (kNucUnroll - 1) * kNucThreads < nv; j0 += kNucThreads * kNucUnroll) {
      uint4 v[kNucUnroll];
#pragma unroll
      for (int u = 0; u < kNucUnroll; ++u) v[u] = row[j0 + u * kNucThreads];
#pragma unroll
      for (int u = 0; u < kNucUnroll; ++u) each_in_vector<DT>(v[u], f);
    }
    if (j0 < nv) {
      uint4 v[kNucUnroll];
#pragma unroll
      for (int u = 0; u < kNucUnroll; ++u) v[u] = row[min(j0 + u * kNucThreads, nv - 1)];
#pragma unroll
      for (int u = 0; u < kNucUnroll; ++u)
        if (j0 + u * kNucThreads < nv) each_in_vector<DT>(v[u], f);
    }
  } else {
    for (int i = threadIdx.x; i < V; i += kNucThreads) f(logit_at<DT>(base, off + i));
  }
}

__device__ __forceinline__ unsigned long long wave_incl_scan_u64(unsigned long long x, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const unsigned long long y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// One level of the selection over NB bins, a higher bin holding larger
// logits: the largest bin d whose mass at or above it, plus `above` (the mass
// of everything above the level's interval), reaches `need` (at the first
// level need < 0 asks for top_p times the level's total, stored back).
// s_above receives the mass above bin d and s_cmass bin d's mass.
template <int NB>
__device__ __forceinline__ int nuc_select(const unsigned long long *hist, unsigned long long above, double &need,
                                          float top_p, unsigned long long *s_wt, int *s_i,
                                          unsigned long long *s_above, unsigned long long *s_cmass) {
  constexpr int PER = NB / kNucThreads;
  static_assert(PER * kNucThreads == NB, "every thread owns the same number of bins");
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  const int top = NB - 1 - (int)threadIdx.x * PER;  // this thread's bins: top, top - 1, ...
  unsigned long long h[PER], tsum = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    h[k] = hist[top - k];
    tsum += h[k];
  }
  unsigned long long incl = wave_incl_scan_u64(tsum, lane);
  if (lane == kWave - 1) s_wt[wv] = incl;
  __syncthreads();
  unsigned long long total = 0;
#pragma unroll
  for (int k = 0; k < kNucThreads / kWave; ++k) {
    if (k < wv) incl += s_wt[k];
    total += s_wt[k];
  }
  if (need < 0.0) need = (double)top_p * (double)total;
  unsigned long long run = incl - tsum;  // mass of the bins above this thread's
  int cand = -1;
  unsigned long long cand_above = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    if (cand < 0 && (double)(above + run + h[k]) >= need) {
      cand = top - k;
      cand_above = above + run;
    }
    run += h[k];
  }
  const int d = max(block_max_int<kNucThreads>(cand, s_i), 0);
  if (cand == d) {
    *s_above = cand_above;
    *s_cmass = h[top - d];
  }
  __syncthreads();
  return d;
}

// One workgroup per (row r of 2D+1, batch row b): the nucleus threshold t and
// 1/Z over the nucleus, written to nuc[(b R + r) * 4 + {0, 1, 2}] = (M, 1/Z, t).
// Masses are 2^t with t = (x - M) (1/T) log2(e), the exponent the other
// kernels form (2^f by the fp32 exp2 as in exp2_fast, about 1e-7 relative error
// like every mass of this path), rounded to 2^-41 fixed-point integers so
// every sum is exact and order-free.  The threshold is selected level by
// level, each level one read of the row:
//  - the first bins the logits by the integer part of u = -t kNucScale
//    (monotone in the logit, and spread over the bins whatever the logits'
//    exponents), with one LDS atomic per logit;
//  - the second takes the chosen bin's logits (the same test, repeated) and
//    bins them by the fraction of u, tracking each bin's smallest and largest
//    32-bit order key;
//  - the later ones bin the order keys of the chosen bin's interval in
//    power-of-two runs of keys, until the chosen bin holds a single key (each
//    shrinks the interval at least kNucSub / 2-fold, so at most four follow).
// Z is the exact sum of the masses at or above the threshold.
template <int DT, bool VEC>
__global__ __launch_bounds__(kNucThreads, kNucWavesPerSimd) void k_sl_nucleus(SampleLogitsParams p) {
  __shared__ unsigned long long hist[kNucSlots];
  __shared__ uint32_t s_bmin[kNucSub], s_bmax[kNucSub];
  __shared__ unsigned long long s_wt[kNucThreads / kWave];
  __shared__ double s_d[kNucThreads / kWave];
  __shared__ int s_i[kNucThreads / kWave];
  __shared__ unsigned long long s_above, s_cmass;
  const int r = blockIdx.x, b = blockIdx.y;
  const int D = p.D, V = p.V, R = 2 * D + 1;
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  const void *base = r <= D ? p.target : p.draftl;
  const int64_t off = r <= D ? target_row(p, b, r) : draft_row(p, b, r - D - 1);
  // row maximum from the split statistics
  double m = -INFINITY;
  for (int k = threadIdx.x; k < p.Ss; k += kNucThreads) m = fmax(m, p.stats[(((int64_t)b * R + r) * p.Ss + k) * 2]);
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) m = fmax(m, __shfl_xor(m, o));
  if (lane == 0) s_d[wv] = m;
  for (int k = threadIdx.x; k < kNucSlots; k += kNucThreads) hist[k] = 0;
  __syncthreads();
  double M = s_d[0];
#pragma unroll
  for (int k = 1; k < kNucThreads / kWave; ++k) M = fmax(M, s_d[k]);
  const double c2 = p.inv_t * kLog2e;
  auto for_each = [&](auto &&f) { each_logit<DT, VEC>(base, off, V, f); };
  // t of a logit, the exponent of its mass 2^t, as the other kernels form it
  auto t_of = [&](float x) { return ((double)x - M) * c2; };

  // first level: bins in u (larger logits in higher bins), with no branch
  for_each([&](float x) {
    const double t = t_of(x);
    const int k = t > -kNucSpan ? kNucBins - 1 - (int)(-t * kNucScale) : kNucBins + lane;  // NaN: spare
    atomicAdd(&hist[k], fixed41(t));  // a spare slot's sum is never read
  });
  __syncthreads();
  double need = -1.0;
  const int d0 = nuc_select<kNucBins>(hist, 0ull, need, p.top_p, s_wt, s_i, &s_above, &s_cmass);
  unsigned long long above = s_above;
  // second level: the logits of bin d0 (the same test as the first level's),
  // binned by the fraction of their u
  for (int k = threadIdx.x; k < kNucSub; k += kNucThreads) {
    hist[k] = 0;
    s_bmin[k] = 0xFFFFFFFFu;
    s_bmax[k] = 0;
  }
  __syncthreads();
  const int u0 = kNucBins - 1 - d0;
  // the bin's logits lie in [M - (u0 + 1) w, M - u0 w], w = 1 / (kNucScale c2);
  // a float interval a thousandth of w wider, rounded outwards, is tested first
  const double w = 1.0 / (kNucScale * c2);
  const float xlo = float_below(M - (double)(u0 + 1) * w - 1e-3 * w);
  const float xhi = float_above(M - (double)u0 * w + 1e-3 * w);
  for_each([&](float x) {
    if (!(x >= xlo && x <= xhi)) return;
    const double t = t_of(x);
    const double u = -t * kNucScale;
    const int ui = (int)u;
    if (t > -kNucSpan && ui == u0) {
      const int sb = kNucSub - 1 - (int)((u - (double)ui) * kNucSub);  // u - ui is exact, in [0, 1)
      atomicAdd(&hist[sb], fixed41(t));
      const uint32_t key = order_key(x);
      atomicMin(&s_bmin[sb], key);
      atomicMax(&s_bmax[sb], key);
    }
  });
  __syncthreads();
  const int d1 = nuc_select<kNucSub>(hist, above, need, p.top_p, s_wt, s_i, &s_above, &s_cmass);
  uint32_t lo = s_bmin[d1], hi = s_bmax[d1];
  above = s_above;
  __syncthreads();  // every thread has the interval before the bins are cleared
  // later levels: bins in the key over [lo, hi]
#pragma unroll 1
  for (int level = 0; level < 8 && lo != hi; ++level) {
    // bins of 2^sh keys: (hi - lo) >> sh < kNucSub, and the interval shrinks at least kNucSub / 2-fold
    const int sh = max(0, 32 - __clz(hi - lo) - 10);
    for (int k = threadIdx.x; k < kNucSub; k += kNucThreads) {
      hist[k] = 0;
      s_bmin[k] = 0xFFFFFFFFu;
      s_bmax[k] = 0;
    }
    __syncthreads();
    for_each([&](float x) {
      const uint32_t key = order_key(x);
      if (key >= lo && key <= hi) {
        const int sb = (int)((key - lo) >> sh);
        const unsigned long long fx = fixed41(t_of(x));  // in the interval: t > -kNucSpan
        if (fx) atomicAdd(&hist[sb], fx);
        atomicMin(&s_bmin[sb], key);
        atomicMax(&s_bmax[sb], key);
      }
    });
    __syncthreads();
    const int d = nuc_select<kNucSub>(hist, above, need, p.top_p, s_wt, s_i, &s_above, &s_cmass);
    lo = s_bmin[d];
    hi = s_bmax[d];
    above = s_above;
    __syncthreads();  // every thread has the interval before the bins are cleared
  }
  if (threadIdx.x == 0) {
    double *o = p.nuc + ((int64_t)b * R + r) * 4;
    o[0] = M;
    o[1] = kFix / (double)(above + s_cmass);
    o[2] = (double)key_value(hi);
  }
}

// This thread's kSlRun consecutive logits of a split, ids t * kSlRun + k (the
// mass and draw kernels scan ids in order); ids at or past n read as -inf.
template <int DT, bool VEC>
__device__ __forceinline__ void load_run(const void *base, int64_t off, int t, int n, float *x) {
  const int i0 = t * kSlRun;
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  if (VEC && SlVec<DT, kSlRun>::ok && i0 + kSlRun <= n) {
    if (DT == SPECDEC_F32) {
#pragma unroll
      for (int j = 0; j < kSlRun / 4; ++j) {
        const u32x4 v = SL_LOAD(reinterpret_cast<const u32x4 *>(static_cast<const float *>(base) + off + i0 + 4 * j));
        x[4 * j] = __uint_as_float(v[0]);
        x[4 * j + 1] = __uint_as_float(v[1]);
        x[4 * j + 2] = __uint_as_float(v[2]);
        x[4 * j + 3] = __uint_as_float(v[3]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < kSlRun / 8; ++j) {
        const u32x4 v = SL_LOAD(reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(base) + off + i0 + 8 * j));
        const uint32_t w[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[8 * j + 2 * e] = DT == SPECDEC_F16 ? f16_bits_to_f32(w[e] & 0xFFFFu) : bf16_bits_to_f32(w[e] & 0xFFFFu);
          x[8 * j + 2 * e + 1] = DT == SPECDEC_F16 ? f16_bits_to_f32(w[e] >> 16) : bf16_bits_to_f32(w[e] >> 16);
        }
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < kSlRun; ++k) x[k] = i0 + k < n ? logit_at<DT>(base, off + i0 + k) : -INFINITY;
  }
}

// Probability of a logit in a row with maximum M, 1/Z and nucleus threshold
// cut (-inf: every id): 0 below the cut and for -inf logits.
__device__ __forceinline__ double prob(float l, double M, double iz, float cut, double c2) {
  const double v = exp2_fast(((double)l - M) * c2) * iz;
  return l >= cut ? v : 0.0;
}

// The stop row's weight at one logit: max(0, p - q) at a < D (resid), else p.
__device__ __forceinline__ double weight(float lt, float lq, bool resid, const double *ri, double c2) {
  const double pv = prob(lt, ri[0], ri[1], (float)ri[4], c2);
  if (!resid) return pv;
  const double d = pv - prob(lq, ri[2], ri[3], (float)ri[5], c2);
  return d > 0.0 ? d : 0.0;
}

// One workgroup per (split, batch row).  Every load it needs before the stop
// position is known goes out in one round trip: the draft tokens, the two
// logits at each (left by the statistics kernel), the uniforms, and the rows'
// statistics (or nuclei).  Every workgroup of batch row b then evaluates every
// acceptance test and takes the same stop position a; the second round trip
// reads its split of the stop row.  Each thread sums its run of kSlRun
// consecutive ids in id order: the weights w (max(0, p - q) at a < D, p at
// a = D) and, for the fallback, p.  Run sums and the split's totals (wave
// sums, then the waves in order) go to the workspace; split 0 also leaves the
// stop row's (M, 1/Z, threshold), the draw's uniform and a.
template <int DT, bool VEC>
__global__ __launch_bounds__(kSlThreads) void k_sl_mass(SampleLogitsParams p) {
  constexpr int NW = kSlThreads / kWave;
  __shared__ double s_m[kSlMaxRows], s_iz[kSlMaxRows];
  __shared__ float s_cut[kSlMaxRows];
  __shared__ double s_w[NW], s_p[NW];
  __shared__ int s_i[NW];
  __shared__ float s_ud;
  const int s = blockIdx.x, b = blockIdx.y;
  const int S = p.S, D = p.D, V = p.V, R = 2 * D + 1;
  const int t = threadIdx.x, lane = t & (kWave - 1), wv = t / kWave;
  const double c2 = p.inv_t * kLog2e;

  int x = -1;
  float gt = 0.0f, gd = 0.0f, ua = 0.0f, ud = 0.0f;
  if (t < D) {
    x = p.draft[(int64_t)b * D + t];
    gt = p.gath[((int64_t)b * D + t) * 2];
    gd = p.gath[((int64_t)b * D + t) * 2 + 1];
    ua = p.u_accept[(int64_t)b * D + t];
  }
  if (t <= D) ud = p.u_draw[(int64_t)b * (D + 1) + t];
  for (int r = t; r < R; r += kSlThreads) {
    double M, iz;
    float cut = -INFINITY;
    if (p.nucleus) {
      const double *o = p.nuc + ((int64_t)b * R + r) * 4;
      M = o[0];
      iz = o[1];
      cut = (float)o[2];
    } else {
      merge_row(p.stats + ((int64_t)b * R + r) * p.Ss * 2, p.Ss, c2, M, iz);
    }
    s_m[r] = M;
    s_iz[r] = iz;
    s_cut[r] = cut;
    if (s == 0 && p.cutoff) p.cutoff[(int64_t)b * R + r] = cut;
  }
  __syncthreads();
  // u q(x) <= p(x); q(x) = 0 accepts iff p(x) > 0
  bool reject = false, bad = false;
  if (t < D) {
    if (x >= 0 && x < V) {
      const double pt = prob(gt, s_m[t], s_iz[t], s_cut[t], c2);
      const double qd = prob(gd, s_m[D + 1 + t], s_iz[D + 1 + t], s_cut[D + 1 + t], c2);
      reject = !(qd > 0.0 ? ((double)ua * qd <= pt) : (pt > 0.0));
    } else {
      reject = bad = true;
    }
  }
  const int a = min(block_first<kSlThreads>(reject, s_i), D);
  if (s == 0) {
    const bool any_bad = block_first<kSlThreads>(bad, s_i) != INT_MAX;
    if (t == 0 && any_bad) set_status(p.status, SPECDEC_S_DRAFT_RANGE);
  }
  if (s == 0 && t == a) s_ud = ud;

  // this thread's run of the stop row's split, and the split's totals
  const bool resid = a < D;
  const double ri[6] = {s_m[a], s_iz[a], resid ? s_m[D + 1 + a] : 0.0, resid ? s_iz[D + 1 + a] : 0.0,
                        (double)s_cut[a], resid ? (double)s_cut[D + 1 + a] : 0.0};
  float lt[kSlRun], lq[kSlRun];
  const int n = min(kSlChunk, V - s * kSlChunk);
  load_run<DT, VEC>(p.target, target_row(p, b, a) + (int64_t)s * kSlChunk, t, n, lt);
  if (resid) {
    load_run<DT, VEC>(p.draftl, draft_row(p, b, a) + (int64_t)s * kSlChunk, t, n, lq);
  } else {
#pragma unroll
    for (int k = 0; k < kSlRun; ++k) lq[k] = 0.0f;
  }
  double wsum = 0.0, psum = 0.0;
#pragma unroll
  for (int k = 0; k < kSlRun; ++k) {
    wsum += weight(lt[k], lq[k], resid, ri, c2);
    psum += prob(lt[k], ri[0], ri[1], (float)ri[4], c2);
  }
  double *thr = p.thr + (((int64_t)b * S + s) * kSlThreads + t) * 2;
  thr[0] = wsum;
  thr[1] = psum;
  wsum = wave_total_f64(wsum);
  psum = wave_total_f64(psum);
  if (lane == 0) {
    s_w[wv] = wsum;
    s_p[wv] = psum;
  }
  __syncthreads();
  if (t == 0) {
    double tw = s_w[0], tp = s_p[0];
#pragma unroll
    for (int k = 1; k < NW; ++k) {
      tw += s_w[k];
      tp += s_p[k];
    }
    p.part[((int64_t)b * S + s) * 2] = tw;
    p.part[((int64_t)b * S + s) * 2 + 1] = tp;
    if (s == 0) {
      double *o = p.rowinfo + (int64_t)b * 8;
#pragma unroll
      for (int k = 0; k < 6; ++k) o[k] = ri[k];
      o[6] = (double)s_ud;
      o[7] = (double)a;
    }
  }
}

// One workgroup per (split, batch row).  In one round trip every workgroup
// reads the batch row's split totals, its own split's run sums and the stop
// row's parameters; each then finds, alike, the split in which the running
// mass (split totals in split order) first exceeds u T.  Only that split's
// workgroup goes on: a block scan of its run sums in thread order picks the
// run that crosses, and the run's weights, formed again with the mass kernel's
// functions (one id per lane) and added in id order as the mass kernel added
// them, give the id; the partial sums end at the run's sum, so the crossing lies
// inside the run.  A zero residual falls back to p; when rounding leaves no
// crossing, the last id with positive weight is taken; an all-zero row gives id
// 0 and SPECDEC_S_PROB.
template <int DT, bool VEC>
__global__ __launch_bounds__(kSlThreads) void k_sl_draw(SampleLogitsParams p) {
  constexpr int NW = kSlThreads / kWave;
  __shared__ double s_part[2 * kSlMaxSplits];
  __shared__ double s_w[NW];
  __shared__ int s_i[NW];
  __shared__ double s_base, s_target, s_wt[kSlRun];
  __shared__ int s_split, s_flags;
  const int s = blockIdx.x, b = blockIdx.y;
  const int S = p.S, D = p.D, V = p.V;
  const int t = threadIdx.x, lane = t & (kWave - 1), wv = t / kWave;
  const double c2 = p.inv_t * kLog2e;
  // one round trip: this thread's run sums and the stop row's parameters are
  // issued before the split totals, whose LDS copy waits for all of them
  const double *thr = p.thr + (((int64_t)b * S + s) * kSlThreads + t) * 2;
  const double rw = thr[0], rp = thr[1];
  double ri[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) ri[k] = p.rowinfo[(int64_t)b * 8 + k];
  const double *part = p.part + (int64_t)b * S * 2;
  for (int k = t; k < S; k += kSlThreads) {
    s_part[2 * k] = part[2 * k];
    s_part[2 * k + 1] = part[2 * k + 1];
  }
  __syncthreads();
  if (t == 0) {
    double T = 0.0, Tp = 0.0;
    for (int k = 0; k < S; ++k) {
      T += s_part[2 * k];
      Tp += s_part[2 * k + 1];
    }
    int flags = 0;  // 1: draw from p, 2: no crossing (take the last positive id), 4: zero mass
    if (!(T > 0.0)) {
      flags |= 1;
      T = Tp;
    }
    const int e = flags & 1;
    int split = -1;
    double base = 0.0, target = 0.0;
    if (T > 0.0) {
      target = ri[6] * T;
      double c = 0.0;
      for (int k = 0; k < S; ++k) {
        const double cn = c + s_part[2 * k + e];
        if (cn > target) {
          split = k;
          base = c;
          break;
        }
        c = cn;
      }
      if (split < 0) {
        flags |= 2;
        for (int k = S - 1; k >= 0; --k)
          if (s_part[2 * k + e] > 0.0) {
            split = k;
            break;
          }
      }
    } else {
      flags |= 4;
      split = 0;
    }
    s_split = split;
    s_base = base;
    s_target = target;
    s_flags = flags;
  }
  __syncthreads();
  const int flags = s_flags, a = (int)ri[7];
  if (s_split != s) return;
  if (flags & 4) {
    if (t == 0) {
      p.accept_len[b] = a;
      p.next_token[b] = 0;
      set_status(p.status, SPECDEC_S_PROB);
    }
    return;
  }
  const bool use_p = flags & 1, resid = a < D && !use_p;
  const double target = s_target;
  // the runs of this split, scanned in thread order
  const double m = use_p ? rp : rw;
  const double incl = wave_scan_f64(m);
  if (lane == kWave - 1) s_w[wv] = incl;
  __syncthreads();
  double ex = 0.0;
#pragma unroll
  for (int k = 0; k < NW; ++k)
    if (k < wv) ex += s_w[k];
  const double before = s_base + (ex + (incl - m));
  const bool cross = !(flags & 2) && m > 0.0 && before + m > target;
  const int who = block_first<kSlThreads>(cross, s_i);
  const int run = who != INT_MAX ? who : block_last<kSlThreads>(m > 0.0, s_i);
  if (run < 0) {  // no run with mass: not reached when the split was chosen for its mass
    if (t == 0) {
      p.accept_len[b] = a;
      p.next_token[b] = 0;
    }
    return;
  }
  // the run's weights, one id per lane of the first wave
  const int v0 = s * kSlChunk + run * kSlRun;
  if (t < kSlRun) {
    double w = 0.0;
    if (v0 + t < V) {
      const float lt = logit_at<DT>(p.target, target_row(p, b, a) + v0 + t);
      const float lq = resid ? logit_at<DT>(p.draftl, draft_row(p, b, a) + v0 + t) : 0.0f;
      w = use_p ? prob(lt, ri[0], ri[1], (float)ri[4], c2) : weight(lt, lq, resid, ri, c2);
    }
    s_wt[t] = w;
  }
  if (t == run) s_base = before;  // the mass before the run
  __syncthreads();
  if (t == 0) {
    // the same additions, in the same order, as the run's sum
    const double bef = s_base;
    int j = -1, lastpos = -1;
    double c = 0.0;
    for (int k = 0; k < kSlRun; ++k) {
      const double w = s_wt[k];
      c += w;
      if (w > 0.0) {
        lastpos = k;
        if (j < 0 && who != INT_MAX && bef + c > target) j = k;
      }
    }
    j = j >= 0 ? j : lastpos;
    p.accept_len[b] = a;
    p.next_token[b] = j >= 0 ? v0 + j : 0;
  }
}

template <int DT, bool VEC>
static hipError_t launch_sl(const SampleLogitsParams &p, hipStream_t s) {
  hipLaunchKernelGGL((k_sl_stats<DT, VEC>), dim3((unsigned)p.Ss, (unsigned)(2 * p.D + 1), (unsigned)p.B),
                     dim3(kSlStatThreads), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.nucleus) {
    hipLaunchKernelGGL((k_sl_nucleus<DT, VEC>), dim3((unsigned)(2 * p.D + 1), (unsigned)p.B), dim3(kNucThreads), 0,
                       s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((k_sl_mass<DT, VEC>), dim3((unsigned)p.S, (unsigned)p.B), dim3(kSlThreads), 0, s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_sl_draw<DT, VEC>), dim3((unsigned)p.S, (unsigned)p.B), dim3(kSlThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_verify_sample_logits(const SampleLogitsParams &p, hipStream_t s) {
  if (p.dtype == SPECDEC_F32) return p.vec ? launch_sl<SPECDEC_F32, true>(p, s) : launch_sl<SPECDEC_F32, false>(p, s);
  if (p.dtype == SPECDEC_F16) return p.vec ? launch_sl<SPECDEC_F16, true>(p, s) : launch_sl<SPECDEC_F16, false>(p, s);
  return p.vec ? launch_sl<SPECDEC_BF16, true>(p, s) : launch_sl<SPECDEC_BF16, false>(p, s);
}

}  // namespace sd
