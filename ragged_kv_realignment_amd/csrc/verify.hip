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
#include "coherent.h"
#include "device_common.h"
#include "launch.h"
#include "wave_dpp.h"
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
// The workgroup whose count completes the row reads the D+1 keys in parallel,
// runs the first-mismatch scan and leaves keys and counter zeroed.  Each key
// and counter has a 128-byte line of its own.
//
// Ordering.  The HIP memory model would have every arrival be an agent-scope
// release and the last workgroup take an agent-scope acquire.  On gfx950 these
// compile to a write-back of the whole L2 before each count (buffer_wbl2) and
// an L2 invalidate (buffer_inv) in the last workgroup; measured on MI355X over
// the 8b-gqa logits, they cost 14 to 75 us per call (the call itself takes
// about 8.4 us).  The kernel relies instead on three properties of gfx950 that
// the ISA gives and the language model does not promise:
//  1. a returning atomic (the max) hands back its result only once it has been
//     performed at the device's coherence point, where every atomic on that
//     line is performed;
//  2. the count is a data dependency of that result (an opaque zero computed
//     from it is part of the counter's address), so it is issued only after
//     the max has been performed;
//  3. the last workgroup reads the keys with agent-scope loads, which bypass
//     the non-coherent L2 (the sc1 bit) and are issued only after its own count
//     has returned.
// Every max therefore precedes its count, every count precedes the last one,
// and the last workgroup's key loads observe all of them.  A compiler that
// moved the count ahead of the max would break property 2; the dependency
// through the inline asm is what forbids it.
template <int DT, bool VEC, int NT, int VPT>
__global__ __launch_bounds__(NT) void k_verify_greedy(GreedyParams p, int splits, int chunk, FastDiv rows_div,
                                                      FastDiv d1_div) {
  constexpr int ES = Elem<DT>::size;
  constexpr int VW = 16 / ES;
  // workgroup -> (split, row, batch row) by multiply-high division: the
  // generic integer division sits in front of every workgroup's loads and
  // cost 0.35 us per call (8b-gqa, 64 cold rounds)
  const int rows = (int)rows_div.d;
  const int split = (int)fdiv(blockIdx.x, rows_div);
  const int row = (int)blockIdx.x - split * rows;
  const int D = p.D, D1 = p.D + 1;
  const int b = (int)fdiv((uint32_t)row, d1_div);
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
    const unsigned long long old = atomicMax(&p.keys[(size_t)row * kKeyStride], key);
    // opaque zero computed from the atomic's result: the count below cannot
    // issue before the key update has completed
    uint32_t dep = (uint32_t)old;
    asm volatile("v_mov_b32 %0, 0" : "=v"(dep) : "v"(dep));
    s_last = atomicAdd(&p.counters[(size_t)(b + (int)dep) * kCountStride], 1u) == (unsigned)(D1 * splits - 1);
    s_a = D;
    s_bad = 0;
  }
  __syncthreads();
  if (!s_last) return;
  // D + 1 <= NT (checked on the host): one position per thread.  The draft
  // token and the key are loaded together (one round trip), and the keys are
  // cleared only after the outputs, so no wait covers those stores.
  const int i = threadIdx.x;
  unsigned long long *kp = &p.keys[((size_t)b * D1 + min(i, D)) * kKeyStride];
  if (i < D1) {
    const int d = i < D ? p.draft[(size_t)b * D + i] : 0;
    const int t = key_id(load_agent(kp));
    s_t[i] = t;
    if (p.target_tok) p.target_tok[(size_t)b * D1 + i] = t;
    if (i < D) {
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
  if (i < D1) store_agent(kp, 0ull);
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

template <int DT>
static hipError_t launch_greedy_dt(const GreedyParams &p, hipStream_t s) {
  const long rows = (long)p.B * (p.D + 1);
  const long chunk = greedy_chunk(p.B, p.D, p.V, DT);
  const int splits = (int)((p.V + chunk - 1) / chunk);
  const dim3 grid((unsigned)(rows * splits));
  const FastDiv rows_div = host_fast_div((uint32_t)rows), d1_div = host_fast_div((uint32_t)(p.D + 1));
  if (p.vec)
    hipLaunchKernelGGL((k_verify_greedy<DT, true, kBlock, SPECDEC_VG_VPT>), grid, dim3(kBlock), 0, s, p, splits,
                       (int)chunk, rows_div, d1_div);
  else
    hipLaunchKernelGGL((k_verify_greedy<DT, false, kBlock, SPECDEC_VG_VPT>), grid, dim3(kBlock), 0, s, p, splits,
                       (int)chunk, rows_div, d1_div);
  return hipGetLastError();
}

hipError_t launch_verify_greedy(const GreedyParams &p, hipStream_t s) {
  if (p.dtype == 0) return launch_greedy_dt<0>(p, s);
  if (p.dtype == 1) return launch_greedy_dt<1>(p, s);
  return launch_greedy_dt<2>(p, s);
}

// ---------------------------------------------------------------- sampled

constexpr int kSampleBatch = 8;  // 16-byte vectors (of p and of q) a thread has in flight

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Residual mass max(0, p - q) of one id in fp64 (q absent: p).
__device__ __forceinline__ double resid_w(float pv, float qv, bool has_q) {
  const double d = has_q ? (double)pv - (double)qv : (double)pv;
  return d > 0.0 ? d : 0.0;
}

// The fp64 sums of one run [lo, hi) of ids, in id order: of the residual
// weights w = max(0, p - q) (q absent: w = p) into mw, and of max(0, p) into mp
// (the fallback when the residual has no mass).  VW = 4: the run starts on a
// 16-byte boundary and is read as vectors, NB of p (and of q) in flight at once.
template <int VW, int NB>
__device__ __forceinline__ void run_mass(const float *pa, const float *qa, int lo, int hi, double &mw, double &mp) {
  mw = 0.0;
  mp = 0.0;
  if constexpr (VW == 4) {
    for (int v0 = lo; v0 < hi; v0 += 4 * NB) {
      f32x4 pp[NB], qq[NB];
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const int v = min(v0 + 4 * k, hi - 4);  // in range: a repeated load, never used
        pp[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(pa + v));
        qq[k] = qa ? __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(qa + v)) : (f32x4)(0.0f);
      }
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const bool in = v0 + 4 * k < hi;  // a repeated vector adds +0 (sums start at +0, terms are >= 0)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          mw += in ? resid_w(pp[k][e], qq[k][e], qa != nullptr) : 0.0;
          mp += in ? resid_w(pp[k][e], 0.0f, false) : 0.0;
        }
      }
    }
  } else {
    for (int v = lo; v < hi; ++v) {
      mw += resid_w(pa[v], qa ? qa[v] : 0.0f, qa != nullptr);
      mp += resid_w(pa[v], 0.0f, false);
    }
  }
}

// The first id of the run [lo, hi) at which before + (the run's weights summed
// in id order, as run_mass sums them) passes target; else the run's last id
// with a positive weight (-1 if none).  The same additions in the same order
// (loads in batches of NB vectors, as run_mass), so the partial sums end
// exactly at run_mass's result.
template <int VW, int NB>
__device__ __forceinline__ int run_walk(const float *pa, const float *qa, int lo, int hi, double before,
                                        double target) {
  double c = 0.0;
  int last = -1;
  if constexpr (VW == 4) {
    for (int v0 = lo; v0 < hi; v0 += 4 * NB) {
      f32x4 pp[NB], qq[NB];
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const int v = min(v0 + 4 * k, hi - 4);
        pp[k] = *reinterpret_cast<const f32x4 *>(pa + v);
        qq[k] = qa ? *reinterpret_cast<const f32x4 *>(qa + v) : (f32x4)(0.0f);
      }
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const int v = v0 + 4 * k;
        if (v >= hi) break;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const double w = resid_w(pp[k][e], qq[k][e], qa != nullptr);
          c += w;
          if (w > 0.0) last = v + e;
          if (before + c > target) return v + e;
        }
      }
    }
  } else {
    for (int v = lo; v < hi; ++v) {
      const double w = resid_w(pa[v], qa ? qa[v] : 0.0f, qa != nullptr);
      c += w;
      if (w > 0.0) last = v;
      if (before + c > target) return v;
    }
  }
  return last;
}

// A run of exactly 4 NB ids [lo, hi) loaded as run_mass loads it (NB vectors
// of p and of q, out-of-range vectors repeating the last one), for a walk from
// registers.  Without q the q loads re-read p (not used), so no branch splits
// the loads.
template <int NB>
__device__ __forceinline__ void run_load(const float *pa, const float *qa, int lo, int hi, f32x4 (&pp)[NB],
                                         f32x4 (&qq)[NB]) {
  const float *qs = qa ? qa : pa;
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    const int v = min(lo + 4 * k, hi - 4);
    pp[k] = *reinterpret_cast<const f32x4 *>(pa + v);
    qq[k] = *reinterpret_cast<const f32x4 *>(qs + v);
  }
}

// run_mass's two sums of a run held in registers by run_load: the same
// additions in the same order, so the same values.
template <int NB>
__device__ __forceinline__ void run_sums_regs(const f32x4 (&pp)[NB], const f32x4 (&qq)[NB], bool has_q, int lo,
                                              int hi, double &mw, double &mp) {
  mw = 0.0;
  mp = 0.0;
  if (lo >= hi) return;
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    const bool in = lo + 4 * k < hi;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      mw += in ? resid_w(pp[k][e], qq[k][e], has_q) : 0.0;
      mp += in ? resid_w(pp[k][e], 0.0f, false) : 0.0;
    }
  }
}

// run_walk over a run held in registers by run_load: the same additions in
// the same order as run_mass.
template <int NB>
__device__ __forceinline__ int run_walk_regs(const f32x4 (&pp)[NB], const f32x4 (&qq)[NB], bool has_q, int lo,
                                             int hi, double before, double target) {
  double c = 0.0;
  int last = -1;
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    const int v = lo + 4 * k;
    if (v >= hi) break;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const double w = resid_w(pp[k][e], qq[k][e], has_q);
      c += w;
      if (w > 0.0) last = v + e;
      if (before + c > target) return v + e;
    }
  }
  return last;
}

// Sampled verification spread over the chip: batch row b's stop row is cut
// into S splits of kSampleThreads runs of R consecutive ids (run g = split *
// kSampleThreads + thread covers ids [g R, g R + R)); one workgroup per (split,
// batch row), numbered split-major.
//  1. Every workgroup of row b evaluates the acceptance of each draft (u q(x)
//     <= p(x), exactly, in fp64) and takes the first rejection a (the stop
//     position); it is the same in every workgroup.
//  2. Each thread sums its run of the stop row in id order in fp64: the
//     residual weights max(0, p_a - q_a) (p_D for the bonus) and, for the
//     fallback, p_a.  The workgroup adds its runs' sums in a fixed order into
//     the split's totals, which go to row b's workspace block.
//  3. The workgroup counts itself in row b's counter; the last of the S to
//     arrive draws.  Each wave scans the split totals across its lanes, lane k
//     holding split k (the same arithmetic in every wave): the total T, and
//     the first split with mass whose end passes the target u_draw[a] * T.
//     That split's run sums, one per thread, are scanned in thread order; the
//     first run whose end passes the target is walked again, id by id in the
//     order step 2 summed it, from its starting mass, so the partial sums end
//     exactly at the run's sum and the crossing id lies inside it.  Rounding
//     that leaves no crossing takes the last id with positive weight.  A zero
//     residual falls back to p_a; an all-zero row gives id 0 and
//     SPECDEC_S_PROB.
// The run sums of step 3: with PRE (runs of exactly 4 NB ids, e.g. 8) each
// thread of the drawing workgroup loads its run of the chosen split and forms
// its sums again, with step 2's additions in step 2's order (so the same
// values), and the crossing run is walked from the registers that hold it;
// step 2 then stores only the split totals.  Otherwise step 2 also stores every
// run's sums in the workspace block and step 3 loads the chosen split's.
// Ordering.  Sums are stored and loaded with the sc1 cache policy (written
// through to, and read from, the device's coherence point, past the
// non-coherent L2); every store waits to complete (vmcnt) before the count,
// which thread 0 issues after the workgroup's barrier, and the last workgroup
// loads the sums only after its own count has returned.  As with greedy
// verification's finish, this rests on gfx950's ordering, not on a
// release/acquire pair, whose L2 write-back and invalidate would cost more
// than the whole call.
template <int VW, int NB, bool PRE>
__global__ __launch_bounds__(kSampleThreads) void k_verify_sample(SampleParams p, FastDiv b_div) {
  constexpr int NW = kSampleThreads / kWave;
  const int B = p.B, S = p.S, R = p.R;
  const int split = (int)fdiv(blockIdx.x, b_div);
  const int b = (int)blockIdx.x - split * B;
  const int D = p.D, D1 = p.D + 1, V = p.V;
  const int t = threadIdx.x, lane = t & (kWave - 1), wv = t / kWave;
  __shared__ int s_bad, s_last, s_sel;
  __shared__ double s_w[NW], s_p[NW];
  __shared__ int s_i[NW];
  __shared__ float s_ud;
  if (t == 0) s_bad = 0;
  // the draw's uniform at every possible stop position, loaded with the
  // acceptance inputs (D + 1 <= kSampleThreads, one position per thread) and
  // kept for the stop position
  const float ud = t <= D ? p.u_draw[(size_t)b * D1 + t] : 0.0f;
  bool reject = false, bad = false;
  if (t < D) {
    // the uniform is loaded with the draft token, not behind the gather that
    // depends on the token (the empty asm keeps the compiler from sinking it)
    const int x = p.draft[(size_t)b * D + t];
    float uf = p.u_accept[(size_t)b * D + t];
    asm volatile("" : "+v"(uf));
    if (x >= 0 && x < V) {
      const double px = p.p[((size_t)b * D1 + t) * V + x];
      const double qx = p.q[((size_t)b * D + t) * V + x];
      const double u = uf;
      reject = !(qx > 0.0 ? (u * qx <= px) : (px > 0.0));
    } else {
      reject = bad = true;
    }
  }
  const int a = min(block_first<kSampleThreads>(reject, s_i), D);
  if (block_first<kSampleThreads>(bad, s_i) != INT_MAX && t == 0) s_bad = SPECDEC_S_DRAFT_RANGE;
  if (t == a) s_ud = ud;
  const float *pa = p.p + ((size_t)b * D1 + a) * V;
  const float *qa = a < D ? p.q + ((size_t)b * D + a) * V : nullptr;
  char *blk = p.ws + (size_t)b * kSampleRowBytes;
  unsigned int *counter = reinterpret_cast<unsigned int *>(blk);
  // (residual, p) totals of every split, then of every run: 16 bytes each
  const __amdgpu_buffer_rsrc_t rt = coherent_rsrc(blk + kAtomicLine, kSampleSplits * 16);
  const __amdgpu_buffer_rsrc_t rr = coherent_rsrc(blk + kAtomicLine + kSampleSplits * 16,
                                                  kSampleSplits * kSampleThreads * 16);

  // 2. this thread's run of the stop row, and the split's totals
  {
    const int g = split * kSampleThreads + t;
    const int lo = min(V, g * R), hi = min(V, lo + R);
    double mw, mp;
    run_mass<VW, NB>(pa, qa, lo, hi, mw, mp);
    if constexpr (!PRE) st_pair(rr, (uint32_t)g * 16u, mw, mp);
    const double ww = wave_total_f64(mw), wp = wave_total_f64(mp);
    if (lane == 0) {
      s_w[wv] = ww;
      s_p[wv] = wp;
    }
    if constexpr (!PRE) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (t == 0) {
      double tw = 0.0, tp = 0.0;
#pragma unroll
      for (int k = 0; k < NW; ++k) {
        tw += s_w[k];
        tp += s_p[k];
      }
      st_pair(rt, (uint32_t)split * 16u, tw, tp);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      s_last = atomicAdd(counter, 1u) == (unsigned)(S - 1);
    }
  }
  __syncthreads();
  if (!s_last) return;

  // 3. the draw, by the last of row b's workgroups.  Lane k of every wave holds
  // split k's totals (k < S <= 64); a DPP scan in lane order gives each split's
  // running mass and, in the last lane, the totals, alike in every wave.
  double mw, mp;
  ld_pair(rt, (uint32_t)min(lane, S - 1) * 16u, mw, mp);
  if (lane >= S) mw = mp = 0.0;
  const double iw = wave_scan_f64(mw), ip = wave_scan_f64(mp);
  const double Tw = lane_f64(iw, kWave - 1), Tp = lane_f64(ip, kWave - 1);
  const bool use_p = !(Tw > 0.0);  // zero residual: fall back to p at the stop position
  const double T = use_p ? Tp : Tw;
  const float *qw = use_p ? nullptr : qa;
  int j = 0;
  if (T > 0.0) {
    const double target = (double)s_ud * T;
    // the first split with mass whose end passes the target (else the last
    // split with mass) and the mass before it
    const double ms = use_p ? mp : mw, is = use_p ? ip : iw;
    const unsigned long long hit = __ballot(ms > 0.0 && is > target), pos = __ballot(ms > 0.0);
    const bool found = hit != 0;
    const int ss = found ? __builtin_ctzll(hit) : 63 - __builtin_clzll(pos);
    const double P = lane_f64(is - ms, ss);
    const double tgt = found ? target : INFINITY;  // no crossing: walk to the last id with mass
    // that split's runs, one per thread, scanned in thread order
    const int g = ss * kSampleThreads + t;
    const int lo = min(V, g * R), hi = min(V, lo + R);
    f32x4 pp[NB], qq[NB];
    double rw, rp;
    if constexpr (PRE) {
      run_load<NB>(pa, qa, lo, hi, pp, qq);
      run_sums_regs<NB>(pp, qq, qa != nullptr, lo, hi, rw, rp);
    } else {
      ld_pair(rr, (uint32_t)g * 16u, rw, rp);
    }
    const double m = use_p ? rp : rw;
    const double incl = wave_scan_f64(m);
    if (lane == kWave - 1) s_w[wv] = incl;
    __syncthreads();
    double before = P + (incl - m);
    {
      double e = 0.0;
#pragma unroll
      for (int k = 0; k < NW; ++k)
        if (k < wv) e += s_w[k];
      before = P + (e + (incl - m));
    }
    const bool cross = m > 0.0 && before + m > tgt;
    const int who = block_first<kSampleThreads>(cross, s_i);
    const int me = who != INT_MAX ? who : block_last<kSampleThreads>(m > 0.0, s_i);
    if (t == me) {
      const double tw = who != INT_MAX ? tgt : INFINITY;
      int hit;
      if constexpr (PRE)
        hit = run_walk_regs<NB>(pp, qq, !use_p && qa != nullptr, lo, hi, before, tw);
      else
        hit = run_walk<VW, NB>(pa, qw, lo, hi, before, tw);
      s_sel = hit >= 0 ? hit : 0;
    }
    __syncthreads();
    j = s_sel;
  } else if (t == 0) {
    atomicOr(&s_bad, SPECDEC_S_PROB);
  }
  __syncthreads();
  if (t == 0) {
    p.accept_len[b] = a;
    p.next_token[b] = j;
    store_agent(counter, 0u);
    set_status(p.status, s_bad);
  }
}

// Ids per run and splits per row of sampled verification: runs of at least 8
// ids (a multiple of 4), long enough that a row needs at most kSampleSplits
// workgroups (R >= V / (kSampleSplits * kSampleThreads), so S <= kSampleSplits).
void sample_shape(int V, int &R, int &S) {
  const long per = ((long)V + (long)kSampleSplits * kSampleThreads - 1) / ((long)kSampleSplits * kSampleThreads);
  R = (int)((per < 8 ? 8 : per) + 3) / 4 * 4;
  S = (int)(((long)V + (long)kSampleThreads * R - 1) / ((long)kSampleThreads * R));
  if (S < 1) S = 1;
}

hipError_t launch_verify_sample(const SampleParams &p, hipStream_t s) {
  const bool vec = p.V % 4 == 0 && reinterpret_cast<uintptr_t>(p.p) % 16 == 0 &&
                   (p.q == nullptr || reinterpret_cast<uintptr_t>(p.q) % 16 == 0);
  const dim3 grid((unsigned)((long)p.B * p.S));
  // vectors in flight per batch of a run: all of a run of 8 ids, else 8
  const FastDiv b_div = host_fast_div((uint32_t)p.B);
  if (vec && p.R == 8)
    hipLaunchKernelGGL((k_verify_sample<4, 2, true>), grid, dim3(kSampleThreads), 0, s, p, b_div);
  else if (vec)
    hipLaunchKernelGGL((k_verify_sample<4, kSampleBatch, false>), grid, dim3(kSampleThreads), 0, s, p, b_div);
  else
    hipLaunchKernelGGL((k_verify_sample<1, 1, false>), grid, dim3(kSampleThreads), 0, s, p, b_div);
  return hipGetLastError();
}

}  // namespace sd
