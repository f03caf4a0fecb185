// In-place EQSPEC realignment ("Batch Speculative Decoding Done Right",
// section 2.2): the unpad-append-repad of a left-padded rectangle written back
// into the same buffers.  Every row's content keeps its order and moves as a
// whole, so instead of rewriting the full new rectangle only the bytes that
// change are moved: a row's content when its pad width changes, its committed
// entries, and pad that appears where content or unused capacity was.
#include "buffer_io.h"
#include "device_common.h"
#include "launch.h"
#include "specdec.h"

namespace sd {

// The same result as EQSPEC on positions [0, S') of a single rectangle.  Row b's
// content moves by shift = pout - pin positions (|shift| <= D+1): one workgroup
// per (layer, K|V, row, head) sequence walks it in chunks, in ascending order
// for a move to lower positions and descending order otherwise, so a chunk's
// stores only overlap its own sources (a barrier separates its loads from its
// stores) and the next chunk's sources, which it prefetches, are never written
// by the current one.  Positions vacated by a move to higher positions become
// pad (zero bytes); the committed entries follow the content.  Sequences whose
// shift is 0 only append.  The old pad is taken to hold zero bytes, as every
// realignment leaves it.  Token ids, position ids and mask of row b are rebuilt
// by workgroup nseg + b; lengths and width are written by k_inplace_meta.
constexpr int kIpBlock = 256;
constexpr int kIpPasses = 4;

__device__ __forceinline__ void ip_load(const char *base, int pin, int k0, int c, int PP, int U, int poff, int u,
                                        bool act, size_t pos_bytes, i32x4 *v) {
  const __amdgpu_buffer_rsrc_t r = rsrc(base + (size_t)pin * pos_bytes, (uint32_t)(c * pos_bytes));
#pragma unroll
  for (int q = 0; q < kIpPasses; ++q) {
    const int k = k0 + poff + q * PP;
    v[q] = bld(r, (act && k >= 0 && k < c) ? (uint32_t)(k * U + u) * 16u : kOOB);
  }
}

__device__ __forceinline__ void ip_store(char *base, int pout, int k0, int c, int PP, int U, int poff, int u,
                                         bool act, size_t pos_bytes, const i32x4 *v) {
  const __amdgpu_buffer_rsrc_t r = rsrc(base + (size_t)pout * pos_bytes, (uint32_t)(c * pos_bytes));
#pragma unroll
  for (int q = 0; q < kIpPasses; ++q) {
    const int k = k0 + poff + q * PP;
    bst(v[q], r, (act && k >= 0 && k < c) ? (uint32_t)(k * U + u) * 16u : kOOB);
  }
}

__global__ __launch_bounds__(kIpBlock) void k_realign_inplace(RealignParams p) {
  __shared__ int s_c[kMaxRealignRows];
  __shared__ int s_n[kMaxRealignRows];
  __shared__ int s_red[kIpBlock / kWave];
  __shared__ int s_red2[kIpBlock / kWave];
  const int B = p.B, D = p.D, U = p.units, H = p.heads;
  const int S = p.width_in[0];
  int mx = 0, bad = (S < 0 || S > p.cap_in) ? SPECDEC_S_LEN_RANGE : 0;
  for (int b = threadIdx.x; b < B; b += kIpBlock) {
    const int c = p.len_in[b], a = p.accept_len[b];
    if (c < 0 || c > S || a < 0 || a > D) bad = SPECDEC_S_LEN_RANGE;
    s_c[b] = c;
    s_n[b] = a + 1;
    mx = max(mx, c + a + 1);
  }
  int Snew;
  {
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
      mx = max(mx, __shfl_xor(mx, off));
      bad |= __shfl_xor(bad, off);
    }
    if ((threadIdx.x & (kWave - 1)) == 0) {
      s_red[threadIdx.x / kWave] = mx;
      s_red2[threadIdx.x / kWave] = bad;
    }
    __syncthreads();
    Snew = s_red[0];
    bad = s_red2[0];
#pragma unroll
    for (int k = 1; k < kIpBlock / kWave; ++k) {
      Snew = max(Snew, s_red[k]);
      bad |= s_red2[k];
    }
  }
  if (!bad && Snew > p.cap_out) bad = SPECDEC_S_CAPACITY;
  if (bad) {
    if (blockIdx.x == 0 && threadIdx.x == 0) set_status(p.status, bad);
    return;
  }
  const long nseg = (long)p.layers * 2 * B * H;
  const size_t pos_bytes = (size_t)U * 16;
  const int PP = kIpBlock / U, TP = PP * kIpPasses;
  const int poff = threadIdx.x / U, u = threadIdx.x - poff * U;
  const bool act = poff < PP;
  char *kv = static_cast<char *>(p.kv_out);
  const char *nw = static_cast<const char *>(p.kv_new);

  for (long w = blockIdx.x; w < nseg + B; w += gridDim.x) {
    if (w < nseg) {
      const int b = (int)((w / H) % B);
      const int c = s_c[b], n = s_n[b];
      const int pin = S - c, pout = Snew - c - n, shift = pout - pin;
      char *base = kv + (size_t)w * p.cap_in * pos_bytes;
      if (shift != 0 && c > 0) {
        const int nch = (c + TP - 1) / TP;
        // chunk order: ascending for a move to lower positions, descending otherwise
        const int first = shift < 0 ? 0 : nch - 1, step = shift < 0 ? 1 : -1;
        i32x4 v[kIpPasses], nv[kIpPasses];
        ip_load(base, pin, first * TP, c, PP, U, poff, u, act, pos_bytes, v);
        for (int i = 0, ch = first; i < nch; ++i, ch += step) {
          // every thread holds chunk ch (its loads have returned) before any of it
          // is overwritten: consuming the registers makes the wait explicit
#pragma unroll
          for (int q = 0; q < kIpPasses; ++q) asm volatile("" ::"v"(v[q]));
          __syncthreads();
          const int nx = ch + step;
          ip_load(base, pin, nx * TP, (i + 1 < nch) ? c : 0, PP, U, poff, u, act, pos_bytes, nv);
          ip_store(base, pout, ch * TP, c, PP, U, poff, u, act, pos_bytes, v);
#pragma unroll
          for (int q = 0; q < kIpPasses; ++q) v[q] = nv[q];
        }
      }
      if (shift > 0) {
        // positions [pin, pout) become pad: zero bytes (vacated content, or for a
        // short row positions past the old width)
        const __amdgpu_buffer_rsrc_t rz = rsrc(base + (size_t)pin * pos_bytes, (uint32_t)(shift * pos_bytes));
        for (int f = threadIdx.x; f < shift * U; f += kIpBlock) bst((i32x4)(0), rz, (uint32_t)f * 16u);
      }
      // committed entries at [pout + c, Snew)
      const __amdgpu_buffer_rsrc_t ra = rsrc(nw + (size_t)w * (D + 1) * pos_bytes, (uint32_t)(n * pos_bytes));
      const __amdgpu_buffer_rsrc_t rd = rsrc(base + (size_t)(pout + c) * pos_bytes, (uint32_t)(n * pos_bytes));
      for (int f = threadIdx.x; f < (D + 1) * U; f += kIpBlock) {
        const uint32_t off = f < n * U ? (uint32_t)f * 16u : kOOB;
        bst(bld(ra, off), rd, off);
      }
    } else {
      // token ids, position ids and mask of row b
      const int b = (int)(w - nseg);
      const int c = s_c[b], n = s_n[b], a = n - 1;
      const int pin = S - c, pout = Snew - c - n, shift = pout - pin;
      int32_t *tok = p.tok_out + (size_t)b * p.cap_in;
      if (shift != 0 && c > 0) {
        constexpr int E = kIpBlock * 4;  // ids per chunk
        const int nch = (c + E - 1) / E;
        const int first = shift < 0 ? 0 : nch - 1, step = shift < 0 ? 1 : -1;
        for (int i = 0, ch = first; i < nch; ++i, ch += step) {
          int t[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int k = ch * E + q * kIpBlock + (int)threadIdx.x;
            t[q] = k < c ? tok[pin + k] : 0;
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) asm volatile("" ::"v"(t[q]));
          __syncthreads();
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int k = ch * E + q * kIpBlock + (int)threadIdx.x;
            if (k < c) tok[pout + k] = t[q];
          }
          __syncthreads();
        }
      }
      for (int j = threadIdx.x; j < Snew; j += kIpBlock) {
        const int cj = j - pout;
        if (cj < 0) tok[j] = p.pad_token;
        else if (cj >= c) tok[j] = (cj - c < a) ? p.draft[(size_t)b * D + (cj - c)] : p.next_token[b];
        p.pos_out[(size_t)b * p.cap_in + j] = cj < 0 ? 0 : cj;
        p.mask_out[(size_t)b * p.cap_in + j] = (int8_t)(cj >= 0);
      }
    }
  }
}

// Lengths and width of the in-place realignment, after k_realign_inplace (which
// reads them in every workgroup).
__global__ __launch_bounds__(kIpBlock) void k_inplace_meta(RealignParams p) {
  const int B = p.B, D = p.D;
  const int S = p.width_in[0];
  __shared__ int s_mx, s_bad;
  if (threadIdx.x == 0) { s_mx = 0; s_bad = (S < 0 || S > p.cap_in) ? 1 : 0; }
  __syncthreads();
  int mx = 0, bad = 0;
  for (int b = threadIdx.x; b < B; b += kIpBlock) {
    const int c = p.len_in[b], a = p.accept_len[b];
    if (c < 0 || c > S || a < 0 || a > D) bad = 1;
    mx = max(mx, c + a + 1);
  }
  atomicMax(&s_mx, mx);
  if (bad) atomicOr(&s_bad, 1);
  __syncthreads();
  if (s_bad || s_mx > p.cap_out) return;
  __syncthreads();
  for (int b = threadIdx.x; b < B; b += kIpBlock) p.len_out[b] = p.len_in[b] + p.accept_len[b] + 1;
  __syncthreads();
  if (threadIdx.x == 0) p.width_out[0] = s_mx;
}

hipError_t launch_realign_inplace(const RealignParams &p, hipStream_t s) {
  const long g = (long)p.layers * 2 * p.B * p.heads + p.B;
  hipLaunchKernelGGL(k_realign_inplace, dim3((unsigned)(g < (1L << 30) ? g : (1L << 30))), dim3(kIpBlock), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_inplace_meta, dim3(1), dim3(kIpBlock), 0, s, p);
  return hipGetLastError();
}

}  // namespace sd
