// Verification kernels: greedy (split-vocabulary argmax with a single-pass
// finish) and sampled (acceptance test plus inverse-CDF draw).
//
// Greedy follows "Inference Engineering Part 5/8: When Speculative Decoding
// Backfires", sections "Draft Possible Tokens, Then Verify Them Together" and
// "One Verification Pass Can Commit Several Tokens": the target's choice at
// every verified position is its highest-scoring token; drafts are read left to
// right and kept until the first one that differs; that position's choice is
// the replacement, or the bonus token when all drafts are kept.  Sampled
// verification follows section "Exactness Means Different Things For Greedy
// And Sampled Output": accept with probability min(1, p/q), replace from
// normalize(max(0, p - q)), take the bonus from p after the full draft.
#include <math.h>
#include <limits.h>
#include "device_common.h"
#include "launch.h"
#include "specdec.h"

namespace sd {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int DT> struct Elem;
template <> struct Elem<0> { static constexpr int size = 4; };
template <> struct Elem<1> { static constexpr int size = 2; };
template <> struct Elem<2> { static constexpr int size = 2; };

template <int DT>
__device__ __forceinline__ float load_scalar(const char *row, int v) {
  if constexpr (DT == 0) return reinterpret_cast<const float *>(row)[v];
  else if constexpr (DT == 1) return f16_bits_to_f32(reinterpret_cast<const uint16_t *>(row)[v]);
  else return bf16_bits_to_f32(reinterpret_cast<const uint16_t *>(row)[v]);
}

// Fold one 16-byte vector whose first element has id `base` into (bv, bi).
template <int DT>
__device__ __forceinline__ void consume(u32x4 r, int base, float &bv, int &bi) {
  if constexpr (DT == 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x = __uint_as_float(r[e]);
      if (better(x, base + e, bv, bi)) { bv = x; bi = base + e; }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t w = r[e];
      const float lo = DT == 2 ? __uint_as_float(w << 16) : f16_bits_to_f32(w & 0xFFFFu);
      const float hi = DT == 2 ? __uint_as_float(w & 0xFFFF0000u) : f16_bits_to_f32(w >> 16);
      if (better(lo, base + 2 * e, bv, bi)) { bv = lo; bi = base + 2 * e; }
      if (better(hi, base + 2 * e + 1, bv, bi)) { bv = hi; bi = base + 2 * e + 1; }
    }
  }
}

// One workgroup scans `chunk` ids of one logit row (row = b*(D+1) + i), folds
// its (value, id) into the row's 64-bit key with an atomic max, and the last
// workgroup of row-block b to finish reads the D+1 keys and runs the
// first-mismatch scan.  The workspace keys/counters are left zeroed.
template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void k_verify_greedy(GreedyParams p, int splits, int chunk) {
  constexpr int ES = Elem<DT>::size;
  constexpr int VW = 16 / ES;
  constexpr int UNR = 4;
  const int wg = blockIdx.x;
  const int row = wg / splits;
  const int split = wg - row * splits;
  const int D1 = p.D + 1;
  const int b = row / D1;
  const int start = split * chunk;
  const int end = min(p.V, start + chunk);
  const char *rowp = static_cast<const char *>(p.logits) + (size_t)row * (size_t)p.row_stride * ES;

  float bv = -INFINITY;
  int bi = INT_MAX;
  if constexpr (VEC) {
    const int nvec = (end - start) / VW;
    const u32x4 *vp = reinterpret_cast<const u32x4 *>(rowp) + start / VW;
    int k = threadIdx.x;
    for (; k + (UNR - 1) * kBlock < nvec; k += UNR * kBlock) {
      u32x4 r[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) r[u] = __builtin_nontemporal_load(vp + k + u * kBlock);
#pragma unroll
      for (int u = 0; u < UNR; ++u) consume<DT>(r[u], start + (k + u * kBlock) * VW, bv, bi);
    }
    for (; k < nvec; k += kBlock) consume<DT>(__builtin_nontemporal_load(vp + k), start + k * VW, bv, bi);
    for (int v = start + nvec * VW + threadIdx.x; v < end; v += kBlock) {
      const float x = load_scalar<DT>(rowp, v);
      if (better(x, v, bv, bi)) { bv = x; bi = v; }
    }
  } else {
    for (int v = start + threadIdx.x; v < end; v += kBlock) {
      const float x = load_scalar<DT>(rowp, v);
      if (better(x, v, bv, bi)) { bv = x; bi = v; }
    }
  }

  wave_argmax(bv, bi);
  __shared__ float s_v[kBlock / kWave];
  __shared__ int s_i[kBlock / kWave];
  __shared__ int s_last;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  if (lane == 0) { s_v[w] = bv; s_i[w] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int k = 1; k < kBlock / kWave; ++k)
      if (better(s_v[k], s_i[k], bv, bi)) { bv = s_v[k]; bi = s_i[k]; }
    atomicMax(&p.keys[row], argmax_key(bv, bi));
    __threadfence();
    const unsigned prev = atomicAdd(&p.counters[b], 1u);
    s_last = (prev == (unsigned)(D1 * splits - 1));
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  if (threadIdx.x == 0) {
    int a = 0, stop = 0, bad = 0;
    int next = 0;
    for (int i = 0; i < D1; ++i) {
      unsigned long long *kp = &p.keys[(size_t)b * D1 + i];
      const int t = key_id(load_agent(kp));
      store_agent(kp, 0ull);
      if (p.target_tok) p.target_tok[(size_t)b * D1 + i] = t;
      if (i < p.D) {
        const int d = p.draft[(size_t)b * p.D + i];
        bad |= (d < 0 || d >= p.V);
        if (!stop && d == t) ++a;
        else if (!stop) { stop = 1; next = t; }
      } else if (!stop) {
        next = t;
      }
    }
    p.accept_len[b] = a;
    p.next_token[b] = next;
    store_agent(&p.counters[b], 0u);
    if (bad) set_status(p.status, SPECDEC_S_DRAFT_RANGE);
  }
}

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 256;
  return cus;
}

template <int DT>
static hipError_t launch_greedy_dt(const GreedyParams &p, hipStream_t s) {
  constexpr int VW = 16 / Elem<DT>::size;
  const int rows = p.B * (p.D + 1);
  // Enough workgroups to keep every CU busy: aim at ~8 per CU, but never give a
  // workgroup less than one vector per thread.
  const long target = 8L * device_cus();
  const int min_chunk = kBlock * VW;
  int max_splits = (p.V + min_chunk - 1) / min_chunk;
  int splits = (int)((target + rows - 1) / rows);
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  int chunk = (p.V + splits - 1) / splits;
  chunk = (chunk + VW - 1) / VW * VW;
  splits = (p.V + chunk - 1) / chunk;
  const dim3 grid((unsigned)(rows * splits));
  if (p.vec)
    hipLaunchKernelGGL((k_verify_greedy<DT, true>), grid, dim3(kBlock), 0, s, p, splits, chunk);
  else
    hipLaunchKernelGGL((k_verify_greedy<DT, false>), grid, dim3(kBlock), 0, s, p, splits, chunk);
  return hipGetLastError();
}

hipError_t launch_verify_greedy(const GreedyParams &p, hipStream_t s) {
  if (p.dtype == 0) return launch_greedy_dt<0>(p, s);
  if (p.dtype == 1) return launch_greedy_dt<1>(p, s);
  return launch_greedy_dt<2>(p, s);
}

// ---------------------------------------------------------------- sampled

__device__ __forceinline__ double resid(const float *pa, const float *qa, int v) {
  const double d = qa ? (double)pa[v] - (double)qa[v] : (double)pa[v];
  return d > 0.0 ? d : 0.0;
}

// One workgroup per row b.  Thread t owns the contiguous ids [t*K, t*K+K): its
// partial mass, an exclusive scan of the partials in id order, then the thread
// whose range crosses u*T walks its ids.
__global__ __launch_bounds__(kBlock) void k_verify_sample(SampleParams p) {
  const int b = blockIdx.x;
  const int D = p.D, D1 = p.D + 1, V = p.V;
  __shared__ int s_a, s_bad, s_j, s_lastpos;
  __shared__ double s_part[kBlock];
  __shared__ double s_T;
  if (threadIdx.x == 0) { s_a = D; s_bad = 0; s_j = INT_MAX; s_lastpos = -1; }
  __syncthreads();
  for (int i = threadIdx.x; i < D; i += kBlock) {
    const int x = p.draft[(size_t)b * D + i];
    bool ok = false;
    if (x >= 0 && x < V) {
      const double px = p.p[((size_t)b * D1 + i) * V + x];
      const double qx = p.q[((size_t)b * D + i) * V + x];
      const double u = p.u_accept[(size_t)b * D + i];
      ok = qx > 0.0 ? (u * qx <= px) : (px > 0.0);
    } else {
      atomicOr(&s_bad, SPECDEC_S_DRAFT_RANGE);
    }
    if (!ok) atomicMin(&s_a, i);
  }
  __syncthreads();
  const int a = s_a;
  const float *pa = p.p + ((size_t)b * D1 + a) * V;
  const float *qa = a < D ? p.q + ((size_t)b * D + a) * V : nullptr;
  const int K = (V + kBlock - 1) / kBlock;
  const int lo = min(V, (int)threadIdx.x * K), hi = min(V, lo + K);

  double T = 0.0, mine = 0.0, before = 0.0;
  for (int pass = 0; pass < 2; ++pass) {
    mine = 0.0;
    for (int v = lo; v < hi; ++v) mine += resid(pa, qa, v);
    s_part[threadIdx.x] = mine;
    __syncthreads();
    if (threadIdx.x == 0) {
      double run = 0.0;
      for (int t = 0; t < kBlock; ++t) {
        const double x = s_part[t];
        s_part[t] = run;
        run += x;
      }
      s_T = run;
    }
    __syncthreads();
    T = s_T;
    before = s_part[threadIdx.x];
    __syncthreads();
    if (T > 0.0 || qa == nullptr) break;
    qa = nullptr;  // zero residual mass: fall back to p at this position
  }

  int j = 0;
  if (T > 0.0) {
    const double target = (double)p.u_draw[(size_t)b * D1 + a] * T;
    if (before + mine > target) {
      double run = before;
      for (int v = lo; v < hi; ++v) {
        run += resid(pa, qa, v);
        if (run > target) { atomicMin(&s_j, v); break; }
      }
    }
    int lastpos = -1;
    for (int v = hi - 1; v >= lo; --v)
      if (resid(pa, qa, v) > 0.0) { lastpos = v; break; }
    if (lastpos >= 0) atomicMax(&s_lastpos, lastpos);
    __syncthreads();
    j = s_j != INT_MAX ? s_j : s_lastpos;
  } else if (threadIdx.x == 0) {
    atomicOr(&s_bad, SPECDEC_S_PROB);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    p.accept_len[b] = a;
    p.next_token[b] = j;
    set_status(p.status, s_bad);
  }
}

hipError_t launch_verify_sample(const SampleParams &p, hipStream_t s) {
  hipLaunchKernelGGL(k_verify_sample, dim3((unsigned)p.B), dim3(kBlock), 0, s, p);
  return hipGetLastError();
}

}  // namespace sd
