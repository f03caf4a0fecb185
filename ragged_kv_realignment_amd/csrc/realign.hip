// Realignment kernels: EQSPEC unpad-append-repad of a left-padded rectangle,
// and the pool gather / in-place append used by equal-length scheduling.
//
// "Batch Speculative Decoding Done Right", section 2.1: after a round every row
// must have the same pad + content length (rectangular alignment) and position
// ids 0.. over its content (position-id contiguity).  Section 2.2 (EQSPEC):
// unpad each row, append its accepted tokens and bonus token, left-pad all rows
// to the longest, recompute position ids and shift the KV cache.  Section 2.3
// (EXSPEC): same-length groups need no realignment; only mixed-length groups
// are resynchronised.  "Inference Engineering Part 5/8", section "Acceptance
// changes across the workload": committed KV is kept and speculative entries
// are committed or discarded once acceptance is known.
//
// Every KV move is a copy of whole positions (head_dim * element bytes, a
// multiple of 16): each (layer, K|V, row, head) sequence is contiguous, so a
// row's shift is a whole number of positions and every load and store is a
// naturally aligned 16-byte vector.  Threads of a workgroup cover
// kBlock / units consecutive positions per pass, so a wave reads and writes
// contiguous bytes; pad positions are store-only.
#include <limits.h>
#include "device_common.h"
#include "launch.h"
#include "specdec.h"

namespace sd {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kMaxB = 1024;
constexpr int kPasses = 4;  // positions per thread per tile

__device__ __forceinline__ u32x4 ld(const u32x4 *p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st(u32x4 v, u32x4 *p) { __builtin_nontemporal_store(v, p); }

// Contiguous share [t0, t1) of `ntiles` tiles for this workgroup.
__device__ __forceinline__ void my_tiles(long ntiles, long &t0, long &t1) {
  const long per = (ntiles + gridDim.x - 1) / gridDim.x;
  t0 = (long)blockIdx.x * per;
  t1 = t0 + per < ntiles ? t0 + per : ntiles;
}

// ------------------------------------------------------------------ EQSPEC
__global__ __launch_bounds__(kBlock) void k_realign_eqspec(RealignParams p) {
  __shared__ int s_c[kMaxB];
  __shared__ int s_n[kMaxB];
  __shared__ int s_red[kBlock / kWave];
  const int B = p.B, D = p.D, U = p.units, H = p.heads;
  const int S = p.width_in[0];
  int mx = 0, bad = (S < 0 || S > p.cap_in) ? SPECDEC_S_LEN_RANGE : 0;
  for (int b = threadIdx.x; b < B; b += kBlock) {
    const int c = p.len_in[b], a = p.accept_len[b];
    if (c < 0 || c > S || a < 0 || a > D) bad = SPECDEC_S_LEN_RANGE;
    s_c[b] = c;
    s_n[b] = a + 1;
    mx = max(mx, c + a + 1);
  }
  const int Snew = block_max_int(mx, s_red);
  bad = block_or_int(bad, s_red);
  if (!bad && Snew > p.cap_out) bad = SPECDEC_S_CAPACITY;
  if (bad) {
    if (blockIdx.x == 0 && threadIdx.x == 0) set_status(p.status, bad);
    return;
  }

  const int PP = kBlock / U;             // positions per pass
  const int TP = PP * kPasses;           // positions per tile
  const int chunks = (Snew + TP - 1) / TP;
  const long nseg = (long)p.layers * 2 * B * H;
  const int poff = threadIdx.x / U, u = threadIdx.x - poff * U;
  const bool active = poff < PP;
  const u32x4 *in = static_cast<const u32x4 *>(p.kv_in);
  u32x4 *out = static_cast<u32x4 *>(p.kv_out);
  const u32x4 *nw = static_cast<const u32x4 *>(p.kv_new);

  long t0, t1;
  my_tiles(nseg * chunks, t0, t1);
  if (t0 < t1 && active) {
    long seg = t0 / chunks;
    int chunk = (int)(t0 - seg * chunks);
    int b = (int)((seg / H) % B);
    for (long t = t0; t < t1; ++t) {
      const int c = s_c[b], n = s_n[b];
      const int pin = S - c, pout = Snew - c - n;
      const u32x4 *src = in + (size_t)seg * p.cap_in * U + u;
      const u32x4 *srcn = nw + (size_t)seg * (D + 1) * U + u;
      u32x4 *dst = out + (size_t)seg * p.cap_out * U + u;
      const int j0 = chunk * TP + poff;
      u32x4 v[kPasses];
#pragma unroll
      for (int k = 0; k < kPasses; ++k) {
        const int j = j0 + k * PP;
        const int cj = j - pout;
        v[k] = (u32x4)(0u);
        if (j < Snew && cj >= 0) v[k] = cj < c ? ld(src + (size_t)(pin + cj) * U) : ld(srcn + (size_t)(cj - c) * U);
      }
#pragma unroll
      for (int k = 0; k < kPasses; ++k) {
        const int j = j0 + k * PP;
        if (j < Snew) st(v[k], dst + (size_t)j * U);
      }
      if (++chunk == chunks) {
        chunk = 0;
        ++seg;
        b = (int)((seg / H) % B);
      }
    }
  }

  // token ids, position ids and mask of every row, on [0, Snew)
  for (int b = blockIdx.x; b < B; b += gridDim.x) {
    const int c = s_c[b], n = s_n[b], a = n - 1;
    const int pin = S - c, pout = Snew - c - n;
    const int32_t *ti = p.tok_in + (size_t)b * p.cap_in;
    int32_t *to = p.tok_out + (size_t)b * p.cap_out;
    int32_t *po = p.pos_out + (size_t)b * p.cap_out;
    int8_t *mo = p.mask_out + (size_t)b * p.cap_out;
    for (int j = threadIdx.x; j < Snew; j += kBlock) {
      const int cj = j - pout;
      int32_t tok;
      if (cj < 0) tok = p.pad_token;
      else if (cj < c) tok = ti[pin + cj];
      else if (cj - c < a) tok = p.draft[(size_t)b * D + (cj - c)];
      else tok = p.next_token[b];
      to[j] = tok;
      po[j] = cj < 0 ? 0 : cj;
      mo[j] = (int8_t)(cj >= 0);
    }
    if (threadIdx.x == 0) {
      p.len_out[b] = c + n;
      if (b == 0) p.width_out[0] = Snew;
    }
  }
}

// ------------------------------------------------------------------ GATHER
// Pool rows (content at [0, len)) -> one left-padded rectangle per group of
// `group` batch entries, for every group not marked in skip_group.
__global__ __launch_bounds__(kBlock) void k_gather(RealignParams p) {
  __shared__ int s_r[kMaxB];
  __shared__ int s_c[kMaxB];
  __shared__ int s_W[kMaxB];
  __shared__ int s_act[kMaxB];
  __shared__ int s_nact;
  __shared__ int s_red[kBlock / kWave];
  const int B = p.B, G = p.group, U = p.units, H = p.heads;
  const int ng = (B + G - 1) / G;
  int bad = 0;
  for (int j = threadIdx.x; j < B; j += kBlock) {
    const int r = p.rows ? p.rows[j] : j;
    int c = 0;
    if (r < 0 || r >= p.rows_in) bad = SPECDEC_S_LEN_RANGE;
    else c = p.len_in[r];
    if (c < 0 || c > p.cap_in) bad = SPECDEC_S_LEN_RANGE;
    s_r[j] = r;
    s_c[j] = c;
  }
  __syncthreads();
  int wmax = 0;
  for (int g = threadIdx.x; g < ng; g += kBlock) {
    int W = 0;
    for (int j = g * G; j < min(B, g * G + G); ++j) W = max(W, s_c[j]);
    const bool skip = p.skip_group && p.skip_group[g];
    s_W[g] = skip ? -1 : W;
    if (!skip) {
      wmax = max(wmax, W);
      if (W > p.cap_out) bad |= SPECDEC_S_CAPACITY;
    }
  }
  const int Wmax = block_max_int(wmax, s_red);
  bad = block_or_int(bad, s_red);
  if (bad) {
    if (blockIdx.x == 0 && threadIdx.x == 0) set_status(p.status, bad);
    return;
  }
  if (threadIdx.x == 0) {
    int k = 0;
    for (int j = 0; j < B; ++j)
      if (s_W[j / G] >= 0) s_act[k++] = j;
    s_nact = k;
  }
  __syncthreads();
  const int nact = s_nact;

  const int PP = kBlock / U;
  const int TP = PP * kPasses;
  const int chunks = (Wmax + TP - 1) / TP;
  const long nseg = (long)p.layers * 2 * nact * H;
  const int poff = threadIdx.x / U, u = threadIdx.x - poff * U;
  const bool active = poff < PP;
  const u32x4 *in = static_cast<const u32x4 *>(p.kv_in);
  u32x4 *out = static_cast<u32x4 *>(p.kv_out);

  long t0 = 0, t1 = 0;
  if (chunks > 0) my_tiles(nseg * chunks, t0, t1);
  if (t0 < t1 && active) {
    long seg = t0 / chunks;
    int chunk = (int)(t0 - seg * chunks);
    for (long t = t0; t < t1; ++t) {
      const long lk = seg / ((long)nact * H);
      const int rem = (int)(seg - lk * nact * H);
      const int k = rem / H, h = rem - k * H;
      const int j = s_act[k], r = s_r[j], c = s_c[j], W = s_W[j / G];
      const int pad = W - c;
      const u32x4 *src = in + ((size_t)(lk * p.rows_in + r) * H + h) * p.cap_in * U + u;
      u32x4 *dst = out + ((size_t)(lk * p.rows_out + j) * H + h) * p.cap_out * U + u;
      const int j0 = chunk * TP + poff;
      u32x4 v[kPasses];
#pragma unroll
      for (int q = 0; q < kPasses; ++q) {
        const int x = j0 + q * PP;
        v[q] = (u32x4)(0u);
        if (x < W && x >= pad) v[q] = ld(src + (size_t)(x - pad) * U);
      }
#pragma unroll
      for (int q = 0; q < kPasses; ++q) {
        const int x = j0 + q * PP;
        if (x < W) st(v[q], dst + (size_t)x * U);
      }
      if (++chunk == chunks) {
        chunk = 0;
        ++seg;
      }
    }
  }

  for (int k = blockIdx.x; k < nact; k += gridDim.x) {
    const int j = s_act[k], r = s_r[j], c = s_c[j], W = s_W[j / G];
    const int pad = W - c;
    const int32_t *ti = p.tok_in ? p.tok_in + (size_t)r * p.cap_in : nullptr;
    int32_t *to = p.tok_out ? p.tok_out + (size_t)j * p.cap_out : nullptr;
    int32_t *po = p.pos_out ? p.pos_out + (size_t)j * p.cap_out : nullptr;
    int8_t *mo = p.mask_out ? p.mask_out + (size_t)j * p.cap_out : nullptr;
    for (int x = threadIdx.x; x < W; x += kBlock) {
      const int cj = x - pad;
      if (to) to[x] = (cj >= 0 && ti) ? ti[cj] : p.pad_token;
      if (po) po[x] = cj < 0 ? 0 : cj;
      if (mo) mo[x] = (int8_t)(cj >= 0);
    }
    if (threadIdx.x == 0) {
      if (p.len_out) p.len_out[j] = c;
      if (p.width_out && j % G == 0) p.width_out[j / G] = W;
    }
  }
}

// ------------------------------------------------------------------ APPEND
// Validation shared by both append kernels: returns status bits (0 = valid).
__device__ int append_check(const RealignParams &p, int *s_r, int *s_c, int *s_n, int *s_red) {
  int bad = 0;
  for (int b = threadIdx.x; b < p.B; b += kBlock) {
    const int r = p.rows ? p.rows[b] : b;
    const int a = p.accept_len[b];
    int c = 0;
    if (r < 0 || r >= p.rows_in || a < 0 || a > p.D) bad |= SPECDEC_S_LEN_RANGE;
    else {
      c = p.len_in[r];
      if (c < 0 || c > p.cap_in) bad |= SPECDEC_S_LEN_RANGE;
      else if (c + a + 1 > p.cap_in) bad |= SPECDEC_S_CAPACITY;
    }
    s_r[b] = r;
    s_c[b] = c;
    s_n[b] = a + 1;
  }
  return block_or_int(bad, s_red);
}

// KV entries: tile = one (layer, K|V, entry, head) sequence, n_b positions.
__global__ __launch_bounds__(kBlock) void k_append_kv(RealignParams p) {
  __shared__ int s_r[kMaxB];
  __shared__ int s_c[kMaxB];
  __shared__ int s_n[kMaxB];
  __shared__ int s_red[kBlock / kWave];
  if (append_check(p, s_r, s_c, s_n, s_red)) return;  // reported by k_append_meta
  const int B = p.B, U = p.units, H = p.heads, D1 = p.D + 1;
  const long nseg = (long)p.layers * 2 * B * H;
  long t0, t1;
  my_tiles(nseg, t0, t1);
  const u32x4 *nw = static_cast<const u32x4 *>(p.kv_new);
  u32x4 *pool = static_cast<u32x4 *>(p.kv_out);
  for (long seg = t0; seg < t1; ++seg) {
    const long lk = seg / ((long)B * H);
    const int rem = (int)(seg - lk * B * H);
    const int b = rem / H, h = rem - b * H;
    const int r = s_r[b], c = s_c[b], n = s_n[b];
    const u32x4 *src = nw + (size_t)seg * D1 * U;
    u32x4 *dst = pool + ((size_t)(lk * p.rows_in + r) * H + h) * p.cap_in * U + (size_t)c * U;
    for (int f = threadIdx.x; f < n * U; f += kBlock) st(ld(src + f), dst + f);
  }
}

// Token ids and lengths, after the KV copy (stream order keeps len stable
// while k_append_kv reads it).
__global__ __launch_bounds__(kBlock) void k_append_meta(RealignParams p) {
  __shared__ int s_r[kMaxB];
  __shared__ int s_c[kMaxB];
  __shared__ int s_n[kMaxB];
  __shared__ int s_red[kBlock / kWave];
  const int bad = append_check(p, s_r, s_c, s_n, s_red);
  if (bad) {
    if (threadIdx.x == 0) set_status(p.status, bad);
    return;
  }
  const int B = p.B;
  int dup = 0;
  for (int b = threadIdx.x; b < B; b += kBlock)
    for (int o = 0; o < b; ++o) dup |= (s_r[o] == s_r[b]);
  dup = block_or_int(dup, s_red);
  for (int b = threadIdx.x; b < B; b += kBlock) {
    const int r = s_r[b], c = s_c[b], n = s_n[b], a = n - 1;
    if (p.tok_out) {
      int32_t *to = p.tok_out + (size_t)r * p.cap_in + c;
      for (int k = 0; k < a; ++k) to[k] = p.draft[(size_t)b * p.D + k];
      to[a] = p.next_token[b];
    }
    p.len_out[r] = c + n;
  }
  if (dup && threadIdx.x == 0) set_status(p.status, SPECDEC_S_ROWS_DUP);
}

hipError_t launch_realign(const RealignParams &p, hipStream_t s) {
  const int grid = 8 * device_cus();
  if (p.mode == SPECDEC_EQSPEC) {
    hipLaunchKernelGGL(k_realign_eqspec, dim3(grid), dim3(kBlock), 0, s, p);
  } else if (p.mode == SPECDEC_GATHER) {
    hipLaunchKernelGGL(k_gather, dim3(grid), dim3(kBlock), 0, s, p);
  } else {
    const long nseg = (long)p.layers * 2 * p.B * p.heads;
    const long g = nseg < grid ? nseg : grid;
    hipLaunchKernelGGL(k_append_kv, dim3((unsigned)(g > 0 ? g : 1)), dim3(kBlock), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_append_meta, dim3(1), dim3(kBlock), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace sd
