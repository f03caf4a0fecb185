// Sampled verification from raw logits ("Inference Engineering Part 5/8",
// opening section for the sampling settings and section "Exactness Means
// Different Things For Greedy And Sampled Output" for the rule: accept with
// probability min(1, p(x)/q(x)), replace from normalize(max(0, p - q)), bonus
// from the target after the full draft; the draft and the target use the same
// sampling settings).  p and q are softmax(logits / temperature) of the target
// and draft rows, formed on the fly in fp64: e(v) = exp((l(v) - M) * (1/T)) with
// M the row maximum, p(v) = e(v) * (1/Z).  Every decision compares fp64 values.
//
// Three launches, no state kept in the workspace between calls:
//  1. k_sl_stats: one workgroup per (split of kSlChunk logits, row, batch row)
//     writes the split's maximum and its exp-sum relative to that maximum.
//  2. k_sl_mass: one workgroup per (split, batch row) merges the statistics of
//     the 2D+1 rows, evaluates the acceptance test of every draft (the same
//     result in every workgroup of the batch row), and sums the stop row's
//     residual mass max(0, p - q) (or p at position D) and its target mass
//     over its split.
//  3. k_sl_draw: one workgroup per batch row finds the split in which the
//     running mass first exceeds u * T and scans that split with an fp64 block
//     scan for the smallest such id.
#include <math.h>
#include <limits.h>
#include "device_common.h"
#include "launch.h"
#include "specdec.h"

// p and q are each rounded before p - q is formed (as the definition has it):
// no multiply-add contraction, which would leave p's rounding error in a
// residual that is exactly 0 when p = q.
#pragma clang fp contract(off)

namespace sd {

constexpr int kSlPer = kSlChunk / kBlock;  // logits per thread per split
constexpr int kSlMaxRows = 2 * 255 + 1;     // 2D + 1 rows per batch row, D <= 255

template <int DT>
__device__ __forceinline__ float logit_at(const void *base, int64_t i) {
  if (DT == SPECDEC_F32) return static_cast<const float *>(base)[i];
  const uint32_t h = static_cast<const uint16_t *>(base)[i];
  return DT == SPECDEC_F16 ? f16_bits_to_f32(h) : bf16_bits_to_f32(h);
}

// Block sum in a fixed order: wave sums, then the wave totals in wave order.
__device__ __forceinline__ double block_sum_d(double x, double *scratch) {
  x = wave_sum(x);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[threadIdx.x / kWave] = x;
  __syncthreads();
  double r = scratch[0];
#pragma unroll
  for (int k = 1; k < kBlock / kWave; ++k) r += scratch[k];
  return r;
}

// Row maximum M and 1/Z from the per-split statistics (split order).
__device__ __forceinline__ void merge_row(const double *st, int S, double inv_t, double &M, double &inv_z) {
  double m = -INFINITY;
  for (int s = 0; s < S; ++s) m = fmax(m, st[2 * s]);
  double z = 0.0;
  for (int s = 0; s < S; ++s)
    if (st[2 * s] > -INFINITY) z += st[2 * s + 1] * exp((st[2 * s] - m) * inv_t);
  M = m;
  inv_z = 1.0 / z;
}

__device__ __forceinline__ int64_t target_row(const SampleLogitsParams &p, int b, int i) {
  return ((int64_t)b * (p.D + 1) + i) * p.V;
}
__device__ __forceinline__ int64_t draft_row(const SampleLogitsParams &p, int b, int i) {
  return ((int64_t)b * p.D + i) * p.V;
}

template <int DT>
__global__ __launch_bounds__(kBlock) void k_sl_stats(SampleLogitsParams p) {
  __shared__ float s_f[kBlock / kWave];
  __shared__ double s_d[kBlock / kWave];
  const int s = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
  const int D = p.D, R = 2 * D + 1;
  const void *base = r <= D ? p.target : p.draftl;
  const int64_t off = (r <= D ? target_row(p, b, r) : draft_row(p, b, r - D - 1)) + (int64_t)s * kSlChunk;
  const int n = min(kSlChunk, p.V - s * kSlChunk);
  float x[kSlPer];
#pragma unroll
  for (int k = 0; k < kSlPer; ++k) {
    const int i = threadIdx.x + k * kBlock;
    x[k] = i < n ? logit_at<DT>(base, off + i) : -INFINITY;
  }
  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < kSlPer; ++k) m = fmaxf(m, x[k]);
  m = block_max_float(m, s_f);
  double z = 0.0;
  if (m > -INFINITY) {
#pragma unroll
    for (int k = 0; k < kSlPer; ++k)
      if (threadIdx.x + k * kBlock < n) z += exp(((double)x[k] - (double)m) * p.inv_t);
  }
  z = block_sum_d(z, s_d);
  if (threadIdx.x == 0) {
    double *st = p.stats + (((int64_t)b * R + r) * p.S + s) * 2;
    st[0] = (double)m;
    st[1] = z;
  }
}

template <int DT>
__global__ __launch_bounds__(kBlock) void k_sl_mass(SampleLogitsParams p) {
  __shared__ double s_m[kSlMaxRows], s_iz[kSlMaxRows];
  __shared__ int s_i[kBlock / kWave];
  __shared__ double s_d[kBlock / kWave];
  const int s = blockIdx.x, b = blockIdx.y;
  const int D = p.D, V = p.V, R = 2 * D + 1;
  for (int r = threadIdx.x; r < R; r += kBlock) {
    double M, iz;
    merge_row(p.stats + ((int64_t)b * R + r) * p.S * 2, p.S, p.inv_t, M, iz);
    s_m[r] = M;
    s_iz[r] = iz;
  }
  __syncthreads();
  // acceptance of every draft: u * q(x) <= p(x); q(x) = 0 accepts iff p(x) > 0
  int first = D, bad = 0;
  for (int i = threadIdx.x; i < D; i += kBlock) {
    const int x = p.draft[(int64_t)b * D + i];
    bool ok = false;
    if (x >= 0 && x < V) {
      const double pt = exp(((double)logit_at<DT>(p.target, target_row(p, b, i) + x) - s_m[i]) * p.inv_t) * s_iz[i];
      const double qd =
          exp(((double)logit_at<DT>(p.draftl, draft_row(p, b, i) + x) - s_m[D + 1 + i]) * p.inv_t) * s_iz[D + 1 + i];
      const double u = (double)p.u_accept[(int64_t)b * D + i];
      ok = qd > 0.0 ? (u * qd <= pt) : (pt > 0.0);
    } else {
      bad = SPECDEC_S_DRAFT_RANGE;
    }
    if (!ok) first = min(first, i);
  }
  const int a = block_min_int(first, s_i);
  if (s == 0) set_status(p.status, block_or_int(bad, s_i));
  // residual (a < D) or target (a = D) mass of this split, and the target mass
  const int n = min(kSlChunk, V - s * kSlChunk);
  const int64_t to = target_row(p, b, a) + (int64_t)s * kSlChunk;
  const int64_t qo = a < D ? draft_row(p, b, a) + (int64_t)s * kSlChunk : 0;
  float lt[kSlPer], lq[kSlPer];
#pragma unroll
  for (int k = 0; k < kSlPer; ++k) {
    const int i = threadIdx.x + k * kBlock;
    lt[k] = i < n ? logit_at<DT>(p.target, to + i) : 0.0f;
    lq[k] = (i < n && a < D) ? logit_at<DT>(p.draftl, qo + i) : 0.0f;
  }
  const double Mt = s_m[a], izt = s_iz[a];
  const double Mq = a < D ? s_m[D + 1 + a] : 0.0, izq = a < D ? s_iz[D + 1 + a] : 0.0;
  double wsum = 0.0, psum = 0.0;
#pragma unroll
  for (int k = 0; k < kSlPer; ++k) {
    if (threadIdx.x + k * kBlock < n) {
      const double pv = exp(((double)lt[k] - Mt) * p.inv_t) * izt;
      double w = pv;
      if (a < D) {
        const double d = pv - exp(((double)lq[k] - Mq) * p.inv_t) * izq;
        w = d > 0.0 ? d : 0.0;
      }
      wsum += w;
      psum += pv;
    }
  }
  wsum = block_sum_d(wsum, s_d);
  psum = block_sum_d(psum, s_d);
  if (threadIdx.x == 0) {
    p.part[((int64_t)b * p.S + s) * 2] = wsum;
    p.part[((int64_t)b * p.S + s) * 2 + 1] = psum;
    if (s == 0) p.stop[b] = a;
  }
}

template <int DT>
__global__ __launch_bounds__(kBlock) void k_sl_draw(SampleLogitsParams p) {
  __shared__ double s_d[kBlock / kWave];
  __shared__ int s_i[kBlock / kWave];
  __shared__ double s_base, s_target, s_m[2], s_iz[2];
  __shared__ int s_split, s_flags;  // flags: 1 draw from p, 2 no crossing (take the last positive id), 4 zero mass
  const int b = blockIdx.x, D = p.D, V = p.V, S = p.S, R = 2 * D + 1;
  const int a = p.stop[b];
  const double *part = p.part + (int64_t)b * S * 2;
  if (threadIdx.x == 0) {
    double T = 0.0;
    for (int s = 0; s < S; ++s) T += part[2 * s];
    int flags = 0;
    if (!(T > 0.0)) {
      flags |= 1;
      T = 0.0;
      for (int s = 0; s < S; ++s) T += part[2 * s + 1];
    }
    const int e = flags & 1;
    int split = -1;
    double base = 0.0;
    if (T > 0.0) {
      const double target = (double)p.u_draw[(int64_t)b * (D + 1) + a] * T;
      double c = 0.0;
      for (int s = 0; s < S; ++s) {
        const double cn = c + part[2 * s + e];
        if (cn > target) { split = s; base = c; break; }
        c = cn;
      }
      if (split < 0) {
        flags |= 2;
        for (int s = S - 1; s >= 0; --s)
          if (part[2 * s + e] > 0.0) { split = s; break; }
      }
      s_target = target;
    } else {
      flags |= 4;
      split = 0;
      s_target = 0.0;
    }
    s_split = split;
    s_base = base;
    s_flags = flags;
  } else if (threadIdx.x == kWave) {
    double M, iz;
    merge_row(p.stats + ((int64_t)b * R + a) * S * 2, S, p.inv_t, M, iz);
    s_m[0] = M;
    s_iz[0] = iz;
  } else if (threadIdx.x == 2 * kWave && a < D) {
    double M, iz;
    merge_row(p.stats + ((int64_t)b * R + D + 1 + a) * S * 2, S, p.inv_t, M, iz);
    s_m[1] = M;
    s_iz[1] = iz;
  }
  __syncthreads();
  const int flags = s_flags, split = s_split;
  if (flags & 4) {
    if (threadIdx.x == 0) {
      p.accept_len[b] = a;
      p.next_token[b] = 0;
      set_status(p.status, SPECDEC_S_PROB);
    }
    return;
  }
  const bool resid = a < D && !(flags & 1);
  // this thread's contiguous logits of the split, for an in-order scan
  const int v0 = split * kSlChunk, n = min(kSlChunk, V - v0);
  const int i0 = threadIdx.x * kSlPer;
  const int64_t to = target_row(p, b, a) + v0, qo = resid ? draft_row(p, b, a) + v0 : 0;
  double w[kSlPer];
  double tsum = 0.0;
#pragma unroll
  for (int k = 0; k < kSlPer; ++k) {
    const int i = i0 + k;
    double x = 0.0;
    if (i < n) {
      const double pv = exp(((double)logit_at<DT>(p.target, to + i) - s_m[0]) * p.inv_t) * s_iz[0];
      x = pv;
      if (resid) {
        const double d = pv - exp(((double)logit_at<DT>(p.draftl, qo + i) - s_m[1]) * p.inv_t) * s_iz[1];
        x = d > 0.0 ? d : 0.0;
      }
    }
    w[k] = x;
    tsum += x;
  }
  // exclusive block scan of the thread sums, in thread order
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  const double incl = wave_incl_scan(tsum, lane);
  if (lane == kWave - 1) s_d[wv] = incl;
  __syncthreads();
  double run = s_base + incl - tsum;
  for (int k = 0; k < wv; ++k) run += s_d[k];
  int found = INT_MAX, last = -1;
#pragma unroll
  for (int k = 0; k < kSlPer; ++k) {
    run += w[k];
    if (w[k] > 0.0) last = v0 + i0 + k;
    if (found == INT_MAX && run > s_target && w[k] > 0.0) found = v0 + i0 + k;
  }
  if (flags & 2) found = INT_MAX;
  int j = block_min_int(found, s_i);
  if (j == INT_MAX) j = block_max_int(last, s_i);
  if (threadIdx.x == 0) {
    p.accept_len[b] = a;
    p.next_token[b] = j >= 0 ? j : 0;
  }
}

template <int DT>
static hipError_t launch_sl(const SampleLogitsParams &p, hipStream_t s) {
  hipLaunchKernelGGL(k_sl_stats<DT>, dim3((unsigned)p.S, (unsigned)(2 * p.D + 1), (unsigned)p.B), dim3(kBlock), 0,
                     s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_sl_mass<DT>, dim3((unsigned)p.S, (unsigned)p.B), dim3(kBlock), 0, s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_sl_draw<DT>, dim3((unsigned)p.B), dim3(kBlock), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_verify_sample_logits(const SampleLogitsParams &p, hipStream_t s) {
  if (p.dtype == SPECDEC_F32) return launch_sl<SPECDEC_F32>(p, s);
  if (p.dtype == SPECDEC_F16) return launch_sl<SPECDEC_F16>(p, s);
  return launch_sl<SPECDEC_BF16>(p, s);
}

}  // namespace sd
