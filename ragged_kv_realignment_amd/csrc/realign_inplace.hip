// In-place EQSPEC realignment ("Batch Speculative Decoding Done Right",
// section 2.2): the unpad-append-repad of a left-padded rectangle written back
// into the same buffers.  Every row's content keeps its order and moves as a
// whole, so instead of rewriting the full new rectangle only the bytes that
// change are moved: a row's content when its pad width changes, its committed
// entries, and pad that appears where content or unused capacity was.
#include "buffer_io.h"
#include "device_common.h"
#include "realign_params.h"
#include "specdec.h"

namespace sd {

// The same result as EQSPEC on positions [0, S') of a single rectangle.  Row b's
// content moves by shift = pout - pin positions.  One workgroup per (layer,
// K|V, row, head) sequence walks the move in chunks of 16-byte units, in
// ascending order for a move to lower positions and descending order
// otherwise: a chunk's stores then overlap only its own sources and those of
// chunks already moved, never the sources of chunks still to come, which are
// loaded (two chunks ahead) before the current chunk is stored.  Every thread
// has its loads of a chunk back (the registers are consumed) before a barrier,
// and the chunk is stored after it.  Positions vacated by a move to higher
// positions become pad (zero bytes); the committed entries follow the content.
// Sequences whose shift is 0 only append.  The old pad is taken to hold zero
// bytes, as every realignment leaves it; with SPECDEC_EQSPEC_INPLACE_ZERO_PAD
// the whole new pad is written with zeros instead (for an input whose pad holds
// other bytes, as a left-padded prefill leaves it).  Token ids, position ids
// and mask of row b are rebuilt by workgroup nseg + b; lengths and width are
// written by k_inplace_meta.
#ifndef SPECDEC_IP_BLOCK
#define SPECDEC_IP_BLOCK 1024  // threads per workgroup (one sequence)
#endif
#ifndef SPECDEC_IP_PASSES
#define SPECDEC_IP_PASSES 6   // 16-byte units per thread per chunk (measured best of 2-8)
#endif
constexpr int kIpBlock = SPECDEC_IP_BLOCK;
constexpr int kIpWaves = kIpBlock / kWave;
constexpr int kIpPasses = SPECDEC_IP_PASSES;
constexpr int kIpChunk = kIpBlock * kIpPasses;  // 16-byte units per chunk

__device__ __forceinline__ void ip_load(__amdgpu_buffer_rsrc_t r, int f0, i32x4 *v) {
#pragma unroll
  for (int q = 0; q < kIpPasses; ++q) v[q] = bld(r, (uint32_t)(f0 + q * kIpBlock) * 16u);
}

__device__ __forceinline__ void ip_store(__amdgpu_buffer_rsrc_t r, int f0, const i32x4 *v) {
#pragma unroll
  for (int q = 0; q < kIpPasses; ++q) bst(v[q], r, (uint32_t)(f0 + q * kIpBlock) * 16u);
}

// Walk step k: every load of chunk k (in `cur`) has returned in every thread
// before the first store; chunk k + 2 is loaded into `ahead`; chunk k is
// stored.  Steps past the last chunk use zero-range descriptors: no access.
__device__ __forceinline__ void ip_step(int k, int nch, int first, int step, int t, __amdgpu_buffer_rsrc_t rs,
                                        __amdgpu_buffer_rsrc_t rd, __amdgpu_buffer_rsrc_t r0, i32x4 *cur,
                                        i32x4 *ahead) {
#pragma unroll
  for (int q = 0; q < kIpPasses; ++q) asm volatile("" ::"v"(cur[q]));
  __syncthreads();
  ip_load(k + 2 < nch ? rs : r0, (first + (k + 2) * step) * kIpChunk + t, ahead);
  ip_store(k < nch ? rd : r0, (first + k * step) * kIpChunk + t, cur);
}

__global__ __launch_bounds__(kIpBlock) void k_realign_inplace(RealignParams p) {
  __shared__ int s_c[kMaxRealignRows];
  __shared__ int s_n[kMaxRealignRows];
  __shared__ int s_red[kIpWaves];
  __shared__ int s_red2[kIpWaves];
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
    for (int k = 1; k < kIpWaves; ++k) {
      Snew = max(Snew, s_red[k]);
      bad |= s_red2[k];
    }
  }
  Snew = uni(Snew);
  bad = uni(bad);
  if (!bad && Snew > p.cap_out) bad = SPECDEC_S_CAPACITY;
  if (bad) {
    if (blockIdx.x == 0 && threadIdx.x == 0) set_status(p.status, bad);
    return;
  }
  const long nseg = (long)p.layers * 2 * B * H;
  const bool zero_pad = p.mode == SPECDEC_EQSPEC_INPLACE_ZERO_PAD;
  const uint32_t pos_bytes = (uint32_t)U * 16u;
  const int t = threadIdx.x;
  char *kv = static_cast<char *>(p.kv_out);
  const char *nw = static_cast<const char *>(p.kv_new);

  for (long x = blockIdx.x; x < nseg + B; x += gridDim.x) {
    if (x < nseg) {
      // Sequence w of this workgroup.  The dispatcher deals workgroups to the
      // 8 XCDs in turn (x mod 8) and, within an XCD, to its 4 shader engines in
      // turn ((x / 8) mod 4), whichever has a free CU; a row's sequences are
      // all moved or all append-only, so with the heads innermost (w = x) every
      // sequence of row b lands on one engine per XCD (b mod 4 when H = 8) and
      // the engines carry unequal loads.  Rotating each (layer, K|V) block of
      // B*H sequences by lk*H spreads every row over all 32 (XCD, engine)
      // streams.
      const long BH = (long)B * H, lk = x / BH;
      long bh = x - lk * BH - (lk * H) % BH;
      if (bh < 0) bh += BH;
      const long w = lk * BH + bh;
      const int b = (int)(bh / H);
      const int c = uni(s_c[b]), n = uni(s_n[b]);
      const int pin = S - c, pout = Snew - c - n, shift = pout - pin;
      char *base = kv + (size_t)w * p.cap_in * pos_bytes;
      // committed entries go to [pout + c, Snew); their first kIpBlock units are
      // loaded now, so storing them at the end waits for nothing still in flight
      const __amdgpu_buffer_rsrc_t ra = rsrc(nw + (size_t)w * (D + 1) * pos_bytes, (uint32_t)n * pos_bytes);
      const __amdgpu_buffer_rsrc_t rc = rsrc(base + (size_t)(pout + c) * pos_bytes, (uint32_t)n * pos_bytes);
      i32x4 e0 = bld(ra, (uint32_t)t * 16u);
      if (shift != 0 && c > 0) {
        const uint32_t cb = (uint32_t)c * pos_bytes;
        const __amdgpu_buffer_rsrc_t rs = rsrc(base + (size_t)pin * pos_bytes, cb);
        const __amdgpu_buffer_rsrc_t rd = rsrc(base + (size_t)pout * pos_bytes, cb);
        const __amdgpu_buffer_rsrc_t r0 = rsrc(base, 0);
        const int nch = (c * U + kIpChunk - 1) / kIpChunk;
        const int first = shift < 0 ? 0 : nch - 1, step = shift < 0 ? 1 : -1;
        i32x4 v0[kIpPasses], v1[kIpPasses], v2[kIpPasses];
#pragma unroll
        for (int q = 0; q < kIpPasses; ++q) v2[q] = (i32x4)(0);
        // the prologue issues loads and (empty) stores in the order of a
        // steady-state step, so the loop starts with the same loads in flight
        ip_load(rs, first * kIpChunk + t, v0);
        ip_store(r0, t, v2);
        ip_load(nch > 1 ? rs : r0, (first + step) * kIpChunk + t, v1);
        ip_store(r0, t, v2);
        // arrived before the first chunk, so this wait costs nothing; redefining
        // the register leaves no load pending on it at the store below
        asm volatile("" : "+v"(e0));
        for (int k = 0; k < nch; k += 3) {
          ip_step(k, nch, first, step, t, rs, rd, r0, v0, v2);
          ip_step(k + 1, nch, first, step, t, rs, rd, r0, v1, v0);
          ip_step(k + 2, nch, first, step, t, rs, rd, r0, v2, v1);
        }
      } else {
        asm volatile("" : "+v"(e0));
      }
      // positions [z0, pout) become pad: zero bytes.  z0 = pin: what the content
      // vacates, or for a short row positions past the old width (nothing when
      // shift <= 0).  z0 = 0 when the input pad may hold other bytes.
      const int z0 = zero_pad ? 0 : pin;
      if (pout > z0) {
        const __amdgpu_buffer_rsrc_t rz = rsrc(base + (size_t)z0 * pos_bytes, (uint32_t)(pout - z0) * pos_bytes);
        for (int f = t; f < (pout - z0) * U; f += kIpBlock) bst((i32x4)(0), rz, (uint32_t)f * 16u);
      }
      bst(e0, rc, (uint32_t)t * 16u);
      for (int f = t + kIpBlock; f < n * U; f += kIpBlock) bst(bld(ra, (uint32_t)f * 16u), rc, (uint32_t)f * 16u);
    } else {
      // token ids, position ids and mask of row b
      const int b = (int)(x - nseg);
      const int c = uni(s_c[b]), n = uni(s_n[b]), a = n - 1;
      const int pin = S - c, pout = Snew - c - n, shift = pout - pin;
      int32_t *tok = p.tok_out + (size_t)b * p.cap_in;
      if (shift != 0 && c > 0) {
        constexpr int E = kIpBlock * 4;  // ids per chunk
        const int nch = (c + E - 1) / E;
        const int first = shift < 0 ? 0 : nch - 1, step = shift < 0 ? 1 : -1;
        for (int i = 0, ch = first; i < nch; ++i, ch += step) {
          int v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int k = ch * E + q * kIpBlock + t;
            v[q] = k < c ? tok[pin + k] : 0;
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) asm volatile("" ::"v"(v[q]));
          __syncthreads();
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int k = ch * E + q * kIpBlock + t;
            if (k < c) tok[pout + k] = v[q];
          }
        }
      }
      for (int j = t; j < Snew; j += kIpBlock) {
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
  // one workgroup per sequence and per row
  const long g = (long)p.layers * 2 * p.B * p.heads + p.B;
  hipLaunchKernelGGL(k_realign_inplace, dim3((unsigned)(g < (1L << 30) ? g : (1L << 30))), dim3(kIpBlock), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_inplace_meta, dim3(1), dim3(kIpBlock), 0, s, p);
  return hipGetLastError();
}

}  // namespace sd
