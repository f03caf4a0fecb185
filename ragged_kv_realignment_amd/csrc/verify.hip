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

// Element e of a 16-byte vector of type DT, widened exactly to fp32.
template <int DT>
__device__ __forceinline__ float elem(u32x4 r, int e) {
  if constexpr (DT == 0) return __uint_as_float(r[e]);
  else if constexpr (DT == 2) return (e & 1) ? __uint_as_float(r[e >> 1] & 0xFFFF0000u) : __uint_as_float(r[e >> 1] << 16);
  else return f16_bits_to_f32((e & 1) ? (r[e >> 1] >> 16) : (r[e >> 1] & 0xFFFFu));
}

// Largest value of a vector.
template <int DT>
__device__ __forceinline__ float vmax(u32x4 r) {
  constexpr int VW = 16 / Elem<DT>::size;
  float m = elem<DT>(r, 0);
#pragma unroll
  for (int e = 1; e < VW; ++e) m = fmaxf(m, elem<DT>(r, e));
  return m;
}

// Offset of the first element equal to M (-0.0 == +0.0), or VW if none.
template <int DT>
__device__ __forceinline__ int first_eq(u32x4 r, float M) {
  constexpr int VW = 16 / Elem<DT>::size;
  int at = VW;
#pragma unroll
  for (int e = VW - 1; e >= 0; --e)
    if (elem<DT>(r, e) == M) at = e;
  return at;
}

// Tuning: 16-byte vectors each thread loads at once.  The default is the
// measured best on MI355X.
#ifndef SPECDEC_VG_VPT
#define SPECDEC_VG_VPT 4
#endif

// max(x, the value DPP control CTRL brings from another lane); rows outside
// RMASK keep x.
template <int CTRL, int RMASK>
__device__ __forceinline__ float dpp_max(float x) {
  const int y = __builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, RMASK, 0xF, false);
  return fmaxf(x, __int_as_float(y));
}

// Largest value over the wave (NaN only where every lane holds NaN), as a
// wave-uniform value: swaps within quads, half-row and row mirrors, then the
// row broadcasts carry each row's maximum into the last row.
__device__ __forceinline__ float wave_max_uniform(float v) {
  v = dpp_max<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v = dpp_max<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v = dpp_max<0x141, 0xF>(v);  // row_half_mirror
  v = dpp_max<0x140, 0xF>(v);  // row_mirror
  v = dpp_max<0x142, 0xA>(v);  // row_bcast:15
  v = dpp_max<0x143, 0xC>(v);  // row_bcast:31
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), kWave - 1));
}

// One workgroup scans `chunk` ids of one logit row (row = b*(D+1) + i;
// workgroups are numbered split-major, so the splits of a row are spread over
// the launch and finish at different times).  Every thread issues all of its
// 16-byte loads before consuming any and keeps each vector's maximum.  Each
// wave then takes its maximum M and the lowest id holding it: ids grow with
// the vector slot across the whole workgroup, then with the lane, so the first
// slot whose ballot of "my vector's maximum is M" is non-empty, at its lowest
// lane, holds it, and one search of that lane's vector gives the id.  The
// waves' 64-bit (value, ~id) keys are combined by thread 0.
//
// Finish: thread 0 folds the key into the row's key with an atomic max, then
// counts the workgroup in batch row b's counter (D+1 rows x splits arrivals).
// The max's result is consumed before the count is issued, so the workgroup
// that sees the count complete also sees every key (both are device-scope
// atomics performed at the device's coherence point; the keys are read back
// with device-scope atomic loads).  That last workgroup reads the D+1 keys in
// parallel, runs the first-mismatch scan and leaves keys and counter zeroed.
// Each key and counter has a 128-byte line of its own.  With `partial` set
// the key is stored per workgroup instead and a consumer kernel finishes.
template <int DT, bool VEC, int NT, int VPT>
__global__ __launch_bounds__(NT) void k_verify_greedy(GreedyParams p, int splits, int chunk) {
  constexpr int ES = Elem<DT>::size;
  constexpr int VW = 16 / ES;
  const int rows = (int)gridDim.x / splits;
  const int split = (int)blockIdx.x / rows;
  const int row = (int)blockIdx.x - split * rows;
  const int D = p.D, D1 = p.D + 1;
  const int b = row / D1;
  const int start = split * chunk;
  const int end = min(p.V, start + chunk);
  const char *rowp = static_cast<const char *>(p.logits) + (size_t)row * (size_t)p.row_stride * ES;
  __shared__ unsigned long long s_k[NT / kWave];
  __shared__ int s_last, s_a, s_bad;
  __shared__ int s_t[NT];

  unsigned long long key = 0ull;  // the smallest key: no id (a thread or wave past the end)
  if constexpr (VEC) {
    // 1. loads (one workgroup pass covers the chunk: chunk <= VPT*NT*VW);
    //    slots past the end re-read the last vector and are ignored
    const int nvec = (end - start) / VW;
    const u32x4 *vp = reinterpret_cast<const u32x4 *>(rowp) + start / VW;
    u32x4 r[VPT];
    float vm[VPT];
    float m = -INFINITY;
    if (nvec > 0) {
#pragma unroll
      for (int u = 0; u < VPT; ++u)
        r[u] = __builtin_nontemporal_load(vp + min(u * NT + (int)threadIdx.x, nvec - 1));
#pragma unroll
      for (int u = 0; u < VPT; ++u) {
        vm[u] = u * NT + (int)threadIdx.x < nvec ? vmax<DT>(r[u]) : -INFINITY;
        m = fmaxf(m, vm[u]);
      }
    }
    float tail_x = -INFINITY;  // the ragged end of the chunk: one scalar per thread
    const int tv = start + nvec * VW + threadIdx.x;
    if (tv < end) {
      tail_x = load_scalar<DT>(rowp, tv);
      m = fmaxf(m, tail_x);
    }
    // 2. the wave's maximum and the lowest id holding it (all wave-uniform)
    const float M = wave_max_uniform(m);
    int wid = INT_MAX;
    if (nvec > 0) {
#pragma unroll
      for (int u = 0; u < VPT; ++u) {
        const unsigned long long hit = __ballot(u * NT + (int)threadIdx.x < nvec && vm[u] == M);
        if (wid == INT_MAX && hit) {
          const int at = start + (u * NT + (int)threadIdx.x) * VW + first_eq<DT>(r[u], M);
          wid = __builtin_amdgcn_readlane(at, __builtin_ctzll(hit));
        }
      }
    }
    if (wid == INT_MAX) {  // the tail's ids follow every vector's
      const unsigned long long hit = __ballot(tv < end && tail_x == M);
      if (hit) wid = __builtin_amdgcn_readlane(tv, __builtin_ctzll(hit));
    }
    if (wid != INT_MAX) key = argmax_key(M, wid);
  } else {
    float m = -INFINITY;
    for (int v = start + threadIdx.x; v < end; v += NT) m = fmaxf(m, load_scalar<DT>(rowp, v));
    int bi = INT_MAX;
    for (int v = start + threadIdx.x; v < end; v += NT)
      if (load_scalar<DT>(rowp, v) == m) { bi = v; break; }
    if (bi != INT_MAX) key = argmax_key(m, bi);
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
      const unsigned long long o = __shfl_xor(key, off);
      key = o > key ? o : key;
    }
  }
  if ((threadIdx.x & (kWave - 1)) == 0) s_k[threadIdx.x / kWave] = key;
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 1; w < NT / kWave; ++w) key = s_k[w] > key ? s_k[w] : key;
    key = s_k[0] > key ? s_k[0] : key;
    if (p.partial) {
      p.partial[(size_t)row * splits + split] = key;
      s_last = 0;
    } else {
      const unsigned long long old = atomicMax(&p.keys[(size_t)row * kKeyStride], key);
      // opaque zero computed from the atomic's result: the count below cannot
      // issue before the key update has completed
      uint32_t dep = (uint32_t)old;
      asm volatile("v_mov_b32 %0, 0" : "=v"(dep) : "v"(dep));
      s_last = atomicAdd(&p.counters[(size_t)(b + (int)dep) * kCountStride], 1u) == (unsigned)(D1 * splits - 1);
    }
    s_a = D;
    s_bad = 0;
  }
  __syncthreads();
  if (!s_last) return;
  // D + 1 <= NT (checked on the host): one position per thread
  const int i = threadIdx.x;
  if (i < D1) {
    unsigned long long *kp = &p.keys[((size_t)b * D1 + i) * kKeyStride];
    const int t = key_id(load_agent(kp));
    store_agent(kp, 0ull);
    s_t[i] = t;
    if (p.target_tok) p.target_tok[(size_t)b * D1 + i] = t;
    if (i < D) {
      const int d = p.draft[(size_t)b * D + i];
      if (d < 0 || d >= p.V) s_bad = 1;
      if (d != t) atomicMin(&s_a, i);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const int a = s_a;
    p.accept_len[b] = a;
    p.next_token[b] = s_t[a];
    store_agent(&p.counters[(size_t)b * kCountStride], 0u);
    if (s_bad) set_status(p.status, SPECDEC_S_DRAFT_RANGE);
  }
}

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 256;
  return cus;
}

// Ids per workgroup: aim at ~8 workgroups per CU; a workgroup covers between
// one and SPECDEC_VG_VPT vectors per thread, all loaded before any is consumed.
static long greedy_chunk(int B, int D, int V, int dtype) {
  const int VW = 16 / (dtype == 0 ? 4 : 2);
  const long rows = (long)B * (D + 1);
  const long step = (long)kBlock * VW;  // ids covered by one vector per thread
  const long want = (8L * device_cus() + rows - 1) / rows;
  long chunk = (V + want - 1) / want;
  chunk = (chunk + step - 1) / step * step;
  if (chunk > (long)SPECDEC_VG_VPT * step) chunk = (long)SPECDEC_VG_VPT * step;
  return chunk;
}

int greedy_splits(int B, int D, int V, int dtype) {
  const long chunk = greedy_chunk(B, D, V, dtype);
  return (int)((V + chunk - 1) / chunk);
}

template <int DT>
static hipError_t launch_greedy_dt(const GreedyParams &p, hipStream_t s) {
  const long rows = (long)p.B * (p.D + 1);
  const long chunk = greedy_chunk(p.B, p.D, p.V, DT);
  const int splits = (int)((p.V + chunk - 1) / chunk);
  const dim3 grid((unsigned)(rows * splits));
  if (p.vec)
    hipLaunchKernelGGL((k_verify_greedy<DT, true, kBlock, SPECDEC_VG_VPT>), grid, dim3(kBlock), 0, s, p, splits,
                       (int)chunk);
  else
    hipLaunchKernelGGL((k_verify_greedy<DT, false, kBlock, SPECDEC_VG_VPT>), grid, dim3(kBlock), 0, s, p, splits,
                       (int)chunk);
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

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Residual masses w of ids v0 .. v0+VW-1 (0 past V).  VW = 4 reads 16-byte vectors.
template <int VW>
__device__ __forceinline__ void load_w(const float *pa, const float *qa, int v0, int V, double *w) {
  if constexpr (VW == 4) {
    if (v0 + 4 <= V) {
      const f32x4 pp = *reinterpret_cast<const f32x4 *>(pa + v0);
      f32x4 qq = (f32x4)(0.0f);
      if (qa) qq = *reinterpret_cast<const f32x4 *>(qa + v0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double d = qa ? (double)pp[e] - (double)qq[e] : (double)pp[e];
        w[e] = d > 0.0 ? d : 0.0;
      }
      return;
    }
  }
#pragma unroll
  for (int e = 0; e < VW; ++e) w[e] = (v0 + e < V) ? resid(pa, qa, v0 + e) : 0.0;
}

// One workgroup per row b.  Each wave owns a contiguous quarter of the row and
// reads it in chunks of 64 lanes x VW consecutive ids (coalesced).  Pass 1: the
// fp64 mass of each quarter and the block total T; the draw target u*T falls in
// the quarter whose running mass first exceeds it, which that wave re-walks
// chunk by chunk with an fp64 wave scan.  Several waves may claim the crossing
// when rounding puts u*T at a quarter boundary; the lowest id wins.
template <int VW>
__global__ __launch_bounds__(kBlock) void k_verify_sample(SampleParams p) {
  constexpr int NW = kBlock / kWave;
  constexpr int CH = kWave * VW;
  const int b = blockIdx.x;
  const int D = p.D, D1 = p.D + 1, V = p.V;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  __shared__ int s_a, s_bad, s_j, s_lastpos;
  __shared__ double s_wt[NW];
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
  const int nchunks = (V + CH - 1) / CH;
  const int per = (nchunks + NW - 1) / NW;
  const int c0 = min(nchunks, wave * per), c1 = min(nchunks, c0 + per);

  double T = 0.0, before = 0.0, mine = 0.0;
  for (int pass = 0; pass < 2; ++pass) {
    double acc = 0.0;
    int lastpos = -1;
    for (int c = c0; c < c1; ++c) {
      double w[VW];
      const int v0 = c * CH + lane * VW;
      load_w<VW>(pa, qa, v0, V, w);
#pragma unroll
      for (int e = 0; e < VW; ++e) {
        acc += w[e];
        if (w[e] > 0.0) lastpos = v0 + e;
      }
    }
    mine = wave_sum(acc);
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) lastpos = max(lastpos, __shfl_xor(lastpos, off));
    if (lane == 0) {
      s_wt[wave] = mine;
      if (lastpos >= 0) atomicMax(&s_lastpos, lastpos);
    }
    __syncthreads();
    T = 0.0;
    before = 0.0;
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      if (k < wave) before += s_wt[k];
      T += s_wt[k];
    }
    __syncthreads();
    if (T > 0.0 || qa == nullptr) break;
    qa = nullptr;  // zero residual mass: fall back to p at this position
    if (threadIdx.x == 0) s_lastpos = -1;
    __syncthreads();
  }

  int j = 0;
  if (T > 0.0) {
    const double target = (double)p.u_draw[(size_t)b * D1 + a] * T;
    if (before + mine > target) {
      double run = before;
      for (int c = c0; c < c1; ++c) {
        double w[VW];
        const int v0 = c * CH + lane * VW;
        load_w<VW>(pa, qa, v0, V, w);
        double sl = 0.0;
#pragma unroll
        for (int e = 0; e < VW; ++e) sl += w[e];
        const double incl = wave_incl_scan(sl, lane);
        const double chunk_total = __shfl(incl, kWave - 1);
        if (run + chunk_total > target) {
          // the crossing lies in this chunk: the first lane whose ids reach past u*T
          double cum = run + incl - sl;
          int cand = INT_MAX;
#pragma unroll
          for (int e = 0; e < VW; ++e) {
            cum += w[e];
            if (cand == INT_MAX && cum > target) cand = v0 + e;
          }
#pragma unroll
          for (int off = kWave / 2; off > 0; off >>= 1) cand = min(cand, __shfl_xor(cand, off));
          if (lane == 0 && cand != INT_MAX) atomicMin(&s_j, cand);
          if (cand != INT_MAX) break;
        }
        run += chunk_total;
      }
    }
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
  const bool vec = p.V % 4 == 0 && reinterpret_cast<uintptr_t>(p.p) % 16 == 0 &&
                   (p.q == nullptr || reinterpret_cast<uintptr_t>(p.q) % 16 == 0);
  if (vec)
    hipLaunchKernelGGL(k_verify_sample<4>, dim3((unsigned)p.B), dim3(kBlock), 0, s, p);
  else
    hipLaunchKernelGGL(k_verify_sample<1>, dim3((unsigned)p.B), dim3(kBlock), 0, s, p);
  return hipGetLastError();
}

}  // namespace sd
