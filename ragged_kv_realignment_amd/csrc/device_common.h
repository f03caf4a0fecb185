// Device helpers shared by the library's kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sd {

constexpr int kBlock = 256;     // threads per workgroup of the verify kernels: 4 waves of 64
constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Monotone 64-bit key of (value, id) for the argmax: a larger key is a larger
// value, then a lower id on equal values.  -0.0 is folded onto +0.0 first so
// the key order matches float comparison.
__device__ __forceinline__ unsigned long long argmax_key(float v, int id) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)ord << 32) | (unsigned long long)(~(uint32_t)id);
}

__device__ __forceinline__ int key_id(unsigned long long k) { return (int)(~(uint32_t)(k & 0xFFFFFFFFull)); }

__device__ __forceinline__ unsigned long long load_agent(const unsigned long long *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(unsigned long long *p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(unsigned int *p, unsigned int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void set_status(int32_t *status, int32_t bits) {
  if (status && bits) atomicOr(status, bits);
}

// Block-wide reductions over NT threads; `scratch` holds NT/kWave ints.
template <int NT = kBlock>
__device__ __forceinline__ int block_max_int(int v, int *scratch) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) v = max(v, __shfl_xor(v, off));
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[w] = v;
  __syncthreads();
  int r = scratch[0];
#pragma unroll
  for (int k = 1; k < NT / kWave; ++k) r = max(r, scratch[k]);
  return r;
}

template <int NT = kBlock>
__device__ __forceinline__ int block_or_int(int v, int *scratch) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) v |= __shfl_xor(v, off);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[w] = v;
  __syncthreads();
  int r = 0;
#pragma unroll
  for (int k = 0; k < NT / kWave; ++k) r |= scratch[k];
  return r;
}

// Whether two of the n non-negative values v[0..n) are equal (n <= TAB / 2,
// TAB a power of two): each value is inserted into an open-addressing table
// of TAB ints in LDS by compare-and-swap (multiplicative hash, linear
// probing); an insert that meets its own value has found a duplicate.  At most
// half the table fills, so every probe sequence ends at an empty slot.  Every
// thread of the workgroup calls it; the result is the same in all of them.
template <int NT, int TAB>
__device__ __forceinline__ int block_any_duplicate(const int *v, int n, int *tab, int *scratch) {
  static_assert((TAB & (TAB - 1)) == 0, "the table size is a power of two");
  constexpr int kShift = 32 - __builtin_ctz(TAB);
  for (int i = threadIdx.x; i < TAB; i += NT) tab[i] = -1;
  __syncthreads();
  int dup = 0;
  for (int i = threadIdx.x; i < n; i += NT) {
    const int x = v[i];
    uint32_t h = ((uint32_t)x * 2654435761u) >> kShift;
    while (true) {
      const int old = atomicCAS(&tab[h], -1, x);
      if (old == -1) break;
      if (old == x) {
        dup = 1;
        break;
      }
      h = (h + 1) & (TAB - 1);
    }
  }
  return block_or_int<NT>(dup, scratch);
}

template <int NT = kBlock>
__device__ __forceinline__ float block_max_float(float v, float *scratch) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[w] = v;
  __syncthreads();
  float r = scratch[0];
#pragma unroll
  for (int k = 1; k < NT / kWave; ++k) r = fmaxf(r, scratch[k]);
  return r;
}

template <int NT = kBlock>
__device__ __forceinline__ int block_min_int(int v, int *scratch) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) v = min(v, __shfl_xor(v, off));
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[w] = v;
  __syncthreads();
  int r = scratch[0];
#pragma unroll
  for (int k = 1; k < NT / kWave; ++k) r = min(r, scratch[k]);
  return r;
}

// fp64 wave reductions (a fixed order of additions for a given lane mapping).
__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

__device__ __forceinline__ double wave_incl_scan(double x, int lane) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const double y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

// Division by a runtime-invariant divisor d (1 <= d < 2^31) for n < 2^31 with a
// multiply-high: with s = ceil(log2 d) and m = floor(2^32 (2^s - d) / d) + 1,
// n / d = (mulhi(n, m) + n) >> s (Granlund and Montgomery, "Division by
// invariant integers using multiplication", PLDI 1994).
struct FastDiv {
  uint32_t d, m, s;
};

__device__ __forceinline__ FastDiv fast_div(uint32_t d) {
  FastDiv f;
  f.d = d;
  f.s = d > 1 ? 32u - (uint32_t)__clz((int)(d - 1)) : 0u;
  f.m = (uint32_t)(((1ull << 32) * ((1ull << f.s) - d)) / d + 1ull);
  return f;
}

// The same s and m computed on the host, for divisors fixed per launch.
inline FastDiv host_fast_div(uint32_t d) {
  FastDiv f;
  f.d = d;
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  f.s = s;
  f.m = (uint32_t)(((1ull << 32) * ((1ull << s) - d)) / d + 1ull);
  return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv &f) {
  return (uint32_t)(((unsigned long long)__umulhi(n, f.m) + n) >> f.s);
}

}  // namespace sd
