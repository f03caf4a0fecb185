// Equal-length grouping of a sequence pool ("Batch Speculative Decoding Done
// Right", section 2.3: a pool of active sequences is scheduled in batches of
// equal length, which need no realignment; only mixed batches are realigned).
//
// One workgroup.  Entry i's length is len[i], or len[ids[i]] for a list of
// pool rows (and then the order lists those rows).  The entries are ranked by
// (length, i): their 64-bit keys (length with its sign bit flipped, then i) are
// sorted in LDS by a bitonic network, so entry i sits at its rank k.  In sorted
// order a length's entries are contiguous: a prefix maximum over the class
// starts gives each rank the first rank of its length, lb; the last rank of
// each length records the class size eq at lb; k - lb entries of its length
// come before k, and the first floor(eq / G) * G of a length are full-batch
// members.  Full members are listed first in rank order, the others after them
// in the same order, so rank k goes to slot fb (the full members ranked before
// it, by a block prefix sum) if it is one, else total_full + (k - fb).  Both
// segments are sorted by length and the full segment holds a multiple of G
// ids, so no batch straddles the two: a batch's shortest and longest lengths
// are those of its first and last ids.  The workgroup has 256 threads for up
// to 1024 entries, else 1024 (four ranks per thread in the scans), so a small
// pool's barriers span few waves.
#include "device_common.h"
#include "launch.h"
#include "specdec.h"

namespace sd {

constexpr int kRanksPerThread = 4;
static_assert(kRanksPerThread * 1024 >= kMaxPoolSlots, "the largest workgroup ranks a full pool");

// Inclusive scan of x over the wave's lanes with the combine op (sum or max)
// and its identity: DPP row shifts, then row broadcasts.
template <bool MAX>
__device__ __forceinline__ int wave_scan_i32(int x, int id) {
#define SD_GRP_STEP(CTRL, RM)                                              \
  {                                                                        \
    const int y = __builtin_amdgcn_update_dpp(id, x, CTRL, RM, 0xF, false); \
    x = MAX ? max(x, y) : x + y;                                           \
  }
  SD_GRP_STEP(0x111, 0xF)  // row_shr:1
  SD_GRP_STEP(0x112, 0xF)  // row_shr:2
  SD_GRP_STEP(0x114, 0xF)  // row_shr:4
  SD_GRP_STEP(0x118, 0xF)  // row_shr:8
  SD_GRP_STEP(0x142, 0xA)  // row_bcast:15
  SD_GRP_STEP(0x143, 0xC)  // row_bcast:31
#undef SD_GRP_STEP
  return x;
}

// Exclusive scan of v over the workgroup's threads in thread order (sum or
// max, with identity id), and the total: wave scans, then the wave totals
// through LDS.  The value one lane down comes from a wave shift.
template <int NT, bool MAX>
__device__ __forceinline__ int block_excl_scan_i32(int v, int id, int *red, int &total) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int x = wave_scan_i32<MAX>(v, id);
  int before = __builtin_amdgcn_update_dpp(id, x, 0x138, 0xF, 0xF, false);  // wave_shr:1
  __syncthreads();
  if (lane == kWave - 1) red[w] = x;
  __syncthreads();
  total = id;
#pragma unroll
  for (int k = 0; k < NW; ++k) {
    if (k < w) before = MAX ? max(before, red[k]) : before + red[k];
    total = MAX ? max(total, red[k]) : total + red[k];
  }
  return before;
}

template <int NT>
__global__ __launch_bounds__(NT) void k_group_by_len(GroupParams p) {
  constexpr int MC = kRanksPerThread * NT;  // keys at most
  __shared__ unsigned long long s_key[MC];
  __shared__ int s_aux[MC];  // class sizes by first rank, then lengths by output slot
  __shared__ int s_red[NT / kWave];
  __shared__ int s_nu;
  const int N = p.N, G = p.group, t = threadIdx.x;
  int M = 2;
  while (M < N) M <<= 1;
  if (t == 0) s_nu = 0;
  // the keys, positions past N padding (every load at once, indices clamped
  // into range)
  const int k0 = t * kRanksPerThread;
  {
    unsigned long long v[kRanksPerThread];
#pragma unroll
    for (int e = 0; e < kRanksPerThread; ++e) v[e] = ~0ull;  // padding sorts last
    if (N > 0) {
      int id[kRanksPerThread], l[kRanksPerThread];
#pragma unroll
      for (int e = 0; e < kRanksPerThread; ++e) id[e] = p.ids ? p.ids[min(k0 + e, N - 1)] : min(k0 + e, N - 1);
#pragma unroll
      for (int e = 0; e < kRanksPerThread; ++e) l[e] = p.len[id[e]];
#pragma unroll
      for (int e = 0; e < kRanksPerThread; ++e)
        if (k0 + e < N) v[e] = ((unsigned long long)((uint32_t)l[e] ^ 0x80000000u) << 32) | (uint32_t)(k0 + e);
    }
#pragma unroll
    for (int e = 0; e < kRanksPerThread; ++e) s_key[k0 + e] = v[e];
  }
  __syncthreads();
  // bitonic sort of the M keys in LDS, ascending
  for (int k = 2; k <= M; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int q = t; q < M / 2; q += NT) {
        const int x = ((q & ~(j - 1)) << 1) | (q & (j - 1)), y = x + j;
        const unsigned long long a = s_key[x], b = s_key[y];
        if ((a > b) == ((x & k) == 0)) {
          s_key[x] = b;
          s_key[y] = a;
        }
      }
      __syncthreads();
    }
  }
  // ranks k = t * 4 + e: the length's first rank lb (prefix maximum of the
  // class starts), then its size, recorded at lb by its last rank
  uint32_t h[kRanksPerThread + 2];  // lengths of ranks k0 - 1 .. k0 + 4 (keys' high words)
#pragma unroll
  for (int e = 0; e < kRanksPerThread + 2; ++e) {
    const int k = k0 - 1 + e;
    h[e] = (uint32_t)(s_key[k < 0 ? 0 : (k < MC ? k : MC - 1)] >> 32);
  }
  int lbl[kRanksPerThread], run = 0;
#pragma unroll
  for (int e = 0; e < kRanksPerThread; ++e) {
    const int k = k0 + e;
    if (k < N && (k == 0 || h[e + 1] != h[e])) run = k;
    lbl[e] = run;
  }
  int tot;
  const int lbx = block_excl_scan_i32<NT, true>(run, 0, s_red, tot);
  int lb[kRanksPerThread];
#pragma unroll
  for (int e = 0; e < kRanksPerThread; ++e) {
    const int k = k0 + e;
    lb[e] = max(lbx, lbl[e]);
    if (k < N && (k == N - 1 || h[e + 2] != h[e + 1])) s_aux[lb[e]] = k + 1 - lb[e];
  }
  __syncthreads();
  int full[kRanksPerThread], fsum = 0;
#pragma unroll
  for (int e = 0; e < kRanksPerThread; ++e) {
    const int k = k0 + e;
    full[e] = 0;
    if (k >= N) continue;
    const int eq = s_aux[lb[e]], eqb = k - lb[e];
    full[e] = eqb < (eq / G) * G;
    fsum += full[e];
  }
  int fb = block_excl_scan_i32<NT, false>(fsum, 0, s_red, tot);  // (its barriers also end the reads above)
#pragma unroll
  for (int e = 0; e < kRanksPerThread; ++e) {
    const int k = k0 + e;
    if (k >= N) continue;
    const int i = (int)(uint32_t)s_key[k], slot = full[e] ? fb : tot + (k - fb);
    fb += full[e];
    s_aux[slot] = (int)(h[e + 1] ^ 0x80000000u);
    p.order[slot] = p.ids ? p.ids[i] : i;
  }
  __syncthreads();
  const int nb = (N + G - 1) / G;
  int nu = 0;
  for (int g = t; g < nb; g += NT) {
    const int mn = s_aux[g * G], mx = s_aux[min(N, g * G + G) - 1];
    p.uniform[g] = mn == mx;
    p.width[g] = mx;
    nu += mn == mx;
  }
  if (nu) atomicAdd(&s_nu, nu);
  __syncthreads();
  if (t == 0) p.n_uniform[0] = s_nu;
}

hipError_t launch_group_by_len(const GroupParams &p, hipStream_t s) {
  if (p.N <= 4 * 256)
    hipLaunchKernelGGL(k_group_by_len<256>, dim3(1), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(k_group_by_len<1024>, dim3(1), dim3(1024), 0, s, p);
  return hipGetLastError();
}

__global__ void k_zero(uint32_t *p, size_t words) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += (size_t)gridDim.x * blockDim.x) p[i] = 0u;
}

hipError_t launch_zero(void *ptr, size_t bytes, hipStream_t s) {
  const size_t words = bytes / 4;
  if (!words) return hipSuccess;
  size_t blocks = (words + kBlock - 1) / kBlock;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(k_zero, dim3((unsigned)blocks), dim3(kBlock), 0, s, static_cast<uint32_t *>(ptr), words);
  return hipGetLastError();
}

}  // namespace sd
