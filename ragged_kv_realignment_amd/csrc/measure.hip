// Measurement kernels for the benchmark, built into their own library
// (libspecdec_measure.so) and not part of the C ABI: bare streaming reads of
// logits with exactly the launch shape and loads of a library kernel, and no
// arithmetic.  Their durations are the floors that the kernel's loads alone
// take on the same cold buffers; the benchmark reports the kernel against them.
//  - k_read_floor: greedy verification's grid, 256-thread workgroups, four
//    16-byte non-temporal loads per thread, the same split of each row.
//  - k_read_stats_floor: the sampling statistics kernel's grid (a split of
//    4096 logits of each target and draft row per workgroup), 256 threads of
//    16 logits, all 16-byte non-temporal loads issued before any is used, the
//    ragged end of a split by scalar loads.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;  // as greedy verification
constexpr int kVpt = 4;        // 16-byte vectors per thread, as greedy verification

// Ids per workgroup, by greedy verification's rule: about 8 workgroups per CU,
// between one and kVpt vectors per thread.
long chunk_for(int B, int D, int V, int es) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  const int vw = 16 / es;
  const long rows = (long)B * (D + 1);
  const long step = (long)kThreads * vw;
  const long want = (8L * cus + rows - 1) / rows;
  long chunk = (V + want - 1) / want;
  chunk = (chunk + step - 1) / step * step;
  if (chunk > (long)kVpt * step) chunk = (long)kVpt * step;
  return chunk;
}

// Division by a divisor fixed per launch with a multiply-high (Granlund and
// Montgomery, PLDI 1994), as greedy verification numbers its workgroups.
struct Div {
  uint32_t d, m, s;
};
Div make_div(uint32_t d) {
  Div f;
  f.d = d;
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  f.s = s;
  f.m = (uint32_t)(((1ull << 32) * ((1ull << s) - d)) / d + 1ull);
  return f;
}
__device__ __forceinline__ uint32_t div_by(uint32_t n, const Div &f) {
  return (uint32_t)(((unsigned long long)__umulhi(n, f.m) + n) >> f.s);
}

__global__ __launch_bounds__(kThreads) void k_read_floor(const char *logits, int64_t row_bytes, int V, int es,
                                                         int chunk, Div rows_div, uint32_t *sink) {
  const int vw = 16 / es;
  const int rows = (int)rows_div.d;
  const int split = (int)div_by(blockIdx.x, rows_div);
  const int row = (int)blockIdx.x - split * rows;
  const int start = split * chunk;
  const int end = min(V, start + chunk);
  const char *rowp = logits + (size_t)row * (size_t)row_bytes;
  const int nvec = (end - start) / vw;
  const u32x4 *vp = reinterpret_cast<const u32x4 *>(rowp) + start / vw;
  uint32_t x = 0;
  if (nvec > 0) {
    u32x4 r[kVpt];
#pragma unroll
    for (int u = 0; u < kVpt; ++u)
      r[u] = __builtin_nontemporal_load(vp + min(u * kThreads + (int)threadIdx.x, nvec - 1));
#pragma unroll
    for (int u = 0; u < kVpt; ++u) x ^= r[u][0] ^ r[u][1] ^ r[u][2] ^ r[u][3];
  }
  const int tv = start + nvec * vw + threadIdx.x;
  if (tv < end) x ^= es == 4 ? reinterpret_cast<const uint32_t *>(rowp)[tv]
                             : (uint32_t)reinterpret_cast<const uint16_t *>(rowp)[tv];
  // never true in practice; keeps the loads
  if (x == 0x9E3779B9u) sink[blockIdx.x] = x;
}

constexpr int kStatChunk = 4096;  // logits per split, as the sampling statistics kernel
constexpr int kStatPer = kStatChunk / kThreads;

__global__ __launch_bounds__(kThreads) void k_read_stats_floor(const char *target, const char *draft, int es, int D,
                                                               int V, uint32_t *sink) {
  const int s = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
  const char *rowp = r <= D ? target + ((size_t)b * (D + 1) + r) * (size_t)V * es
                            : draft + ((size_t)b * D + (r - D - 1)) * (size_t)V * es;
  const int start = s * kStatChunk, n = min(kStatChunk, V - start);
  const int vw = 16 / es;
  const int nv = n / vw;
  const u32x4 *vp = reinterpret_cast<const u32x4 *>(rowp + (size_t)start * es);
  uint32_t x = 0;
  if (es == 4) {
    constexpr int NV = kStatPer / 4;
    u32x4 v[NV];
    if (nv > 0) {
#pragma unroll
      for (int j = 0; j < NV; ++j) v[j] = __builtin_nontemporal_load(vp + min((int)threadIdx.x + j * kThreads, nv - 1));
#pragma unroll
      for (int j = 0; j < NV; ++j) x ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
    }
  } else {
    constexpr int NV = kStatPer / 8;
    u32x4 v[NV];
    if (nv > 0) {
#pragma unroll
      for (int j = 0; j < NV; ++j) v[j] = __builtin_nontemporal_load(vp + min((int)threadIdx.x + j * kThreads, nv - 1));
#pragma unroll
      for (int j = 0; j < NV; ++j) x ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
    }
  }
  for (int i = nv * vw + threadIdx.x; i < n; i += kThreads)
    x ^= es == 4 ? reinterpret_cast<const uint32_t *>(rowp)[start + i]
                 : (uint32_t)reinterpret_cast<const uint16_t *>(rowp)[start + i];
  // never true in practice; keeps the loads
  if (x == 0x9E3779B9u) sink[((size_t)b * gridDim.y + r) * gridDim.x + s] = x;
}

}  // namespace

// Launches the bare read over rows (b, i), b < B, i <= D, of `logits` (16-byte
// aligned rows of row_stride elements of es bytes).  sink: device uint32
// [grid], written only on a 2^-32 chance.  Returns the grid size, or -1.
extern "C" __attribute__((visibility("default"))) int specdec_measure_read_floor(
    const void *logits, int es, int64_t row_stride, int B, int D, int V, uint32_t *sink, int sink_words,
    void *stream) {
  if (!logits || !sink || (es != 2 && es != 4) || B < 1 || D < 0 || V < 1 || row_stride < V) return -1;
  if (reinterpret_cast<uintptr_t>(logits) % 16 != 0 || ((size_t)row_stride * es) % 16 != 0) return -1;
  const long chunk = chunk_for(B, D, V, es);
  const long splits = (V + chunk - 1) / chunk;
  const long grid = (long)B * (D + 1) * splits;
  if (grid > sink_words || grid > 0x7FFFFFFFL) return -1;
  hipLaunchKernelGGL(k_read_floor, dim3((unsigned)grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const char *>(logits), (int64_t)row_stride * es, V, es, (int)chunk,
                     make_div((uint32_t)((long)B * (D + 1))), sink);
  return hipGetLastError() == hipSuccess ? (int)grid : -1;
}

// Launches the bare read of the sampling statistics kernel over target logits
// [B][D+1][V] and draft logits [B][D][V] (both of es bytes per element,
// rows contiguous, 16-byte aligned, V a whole number of 16-byte vectors).
// sink: device uint32 [B (2D+1) ceil(V/4096)], written only on a 2^-32
// chance.  Returns the grid size, or -1.
extern "C" __attribute__((visibility("default"))) int specdec_measure_stats_floor(
    const void *target, const void *draft, int es, int B, int D, int V, uint32_t *sink, int sink_words,
    void *stream) {
  if (!target || (D > 0 && !draft) || !sink || (es != 2 && es != 4) || B < 1 || B > 65535 || D < 0 || D > 255 ||
      V < 1)
    return -1;
  if (reinterpret_cast<uintptr_t>(target) % 16 != 0 || (D > 0 && reinterpret_cast<uintptr_t>(draft) % 16 != 0) ||
      ((size_t)V * es) % 16 != 0)
    return -1;
  const long splits = (V + kStatChunk - 1) / kStatChunk;
  const long grid = splits * (2L * D + 1) * B;
  if (grid > sink_words || splits > 0x7FFFFFFFL) return -1;
  hipLaunchKernelGGL(k_read_stats_floor, dim3((unsigned)splits, (unsigned)(2 * D + 1), (unsigned)B), dim3(kThreads),
                     0, static_cast<hipStream_t>(stream), static_cast<const char *>(target),
                     static_cast<const char *>(draft), es, D, V, sink);
  return hipGetLastError() == hipSuccess ? (int)grid : -1;
}
