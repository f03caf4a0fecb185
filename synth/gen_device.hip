// Device side of the seeded input generator: the same values as gen_host.c,
// written straight into device memory so multi-GB workloads never cross PCIe.
// Untimed set-up only; nothing here belongs to the verify or realign path.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "gen_core.h"

#define EXPORT extern "C" __attribute__((visibility("default")))

static int g_grid = 0;
static int grid_size() {
  if (!g_grid) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
      g_grid = cus * 8;
    else
      g_grid = 2048;
  }
  return g_grid;
}

__global__ void k_fill_normal(int dtype, uint64_t key, uint64_t start, uint64_t count, float sigma, void *out) {
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += (uint64_t)gridDim.x * blockDim.x)
    syn_store(dtype, out, i, sigma * syn_normal(key, start + i));
}

__global__ void k_fill_logits(int dtype, uint64_t key, int64_t row0, int64_t nrows, int64_t V, int64_t row_stride,
                              float sigma, void *out) {
  const uint64_t total = (uint64_t)nrows * (uint64_t)V;
  const size_t es = dtype == SYN_F32 ? 4 : 2;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (uint64_t)gridDim.x * blockDim.x) {
    const uint64_t r = i / (uint64_t)V, v = i % (uint64_t)V;
    char *row = (char *)out + (size_t)(r * (uint64_t)row_stride) * es;
    syn_store(dtype, row, v, sigma * syn_normal(key, (uint64_t)(row0 * V) + i));
  }
}

__global__ void k_plant(int dtype, int64_t row0, int64_t nrows, int64_t row_stride, const int32_t *plant,
                        float plant_value, void *out) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= nrows) return;
  const size_t es = dtype == SYN_F32 ? 4 : 2;
  char *row = (char *)out + (size_t)(r * row_stride) * es;
  for (int s = 0; s < 3; ++s) {
    const int32_t id = plant[(row0 + r) * 3 + s];
    if (id >= 0) syn_store(dtype, row, (uint64_t)id, plant_value);
  }
}

__global__ void k_fill_kv(int dtype, uint64_t key, int rows, int H, int cap, int Dh, const int32_t *len, int width,
                          int left_pad, int layer0, uint64_t nelem, void *out) {
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nelem; i += (uint64_t)gridDim.x * blockDim.x) {
    const uint64_t d = i % (uint64_t)Dh;
    const uint64_t p = (i / (uint64_t)Dh) % (uint64_t)cap;
    const uint64_t s = i / ((uint64_t)Dh * (uint64_t)cap);
    const uint64_t gseg = (uint64_t)layer0 * 2 * rows * H + s;
    const int b = (int)((gseg / (uint64_t)H) % (uint64_t)rows);
    const int off = left_pad ? width - len[b] : 0;
    const int64_t j = (int64_t)p - off;
    float v = 0.0f;
    if (j >= 0 && j < len[b]) v = syn_normal(key, (gseg * (uint64_t)cap + (uint64_t)j) * (uint64_t)Dh + d);
    syn_store(dtype, out, i, v);
  }
}

EXPORT int synth_dev_fill_normal(int dtype, uint64_t seed, uint32_t stream, uint32_t round, uint64_t start,
                                 uint64_t count, float sigma, void *out, void *hstream) {
  if (!count) return 0;
  hipLaunchKernelGGL(k_fill_normal, dim3(grid_size()), dim3(256), 0, (hipStream_t)hstream, dtype,
                     syn_key(seed, stream, round), start, count, sigma, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

EXPORT int synth_dev_fill_logits(int dtype, uint64_t seed, uint32_t round, int64_t row0, int64_t nrows, int64_t V,
                                 int64_t row_stride, float sigma, const int32_t *plant_dev, float plant_value,
                                 void *out, void *hstream) {
  hipStream_t st = (hipStream_t)hstream;
  hipLaunchKernelGGL(k_fill_logits, dim3(grid_size()), dim3(256), 0, st, dtype, syn_key(seed, SYN_S_LOGIT, round),
                     row0, nrows, V, row_stride, sigma, out);
  if (plant_dev)
    hipLaunchKernelGGL(k_plant, dim3((unsigned)((nrows + 255) / 256)), dim3(256), 0, st, dtype, row0, nrows,
                       row_stride, plant_dev, plant_value, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

EXPORT int synth_dev_fill_kv(int dtype, uint64_t seed, int rows, int H, int cap, int Dh, const int32_t *len_dev,
                             int width, int left_pad, int layer0, int nlayers, void *out, void *hstream) {
  const uint64_t nelem = (uint64_t)nlayers * 2 * rows * H * cap * Dh;
  hipLaunchKernelGGL(k_fill_kv, dim3(grid_size()), dim3(256), 0, (hipStream_t)hstream, dtype,
                     syn_key(seed, SYN_S_KV0, 0), rows, H, cap, Dh, len_dev, width, left_pad, layer0, nelem, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
