// Equal-length grouping of a sequence pool ("Batch Speculative Decoding Done
// Right", section 2.3: a pool of active sequences is scheduled in batches of
// equal length, which need no realignment; only mixed batches are realigned).
//
// One workgroup of 1024 threads ranks N <= 4096 lengths held in LDS (entry i's
// length is len[i], or len[ids[i]] for a list of pool rows, and then the order
// lists those rows).  With
// lt_i = #{len < len_i}, eq_i = #{len == len_i} and eqb_i = #{j < i, len_j ==
// len_i}, id i sits at position lt_i + eqb_i of the (length, id) order; the
// first floor(eq_i / G) * G ids of each length are full-batch members.  Full
// members are listed first in (length, id) order, the others after them in the
// same order, so i's output slot is the number of full members ranked before it
// (if it is one) or total_full + (its rank - full members before it).
#include "device_common.h"
#include "launch.h"
#include "specdec.h"

namespace sd {

constexpr int kGroupThreads = 1024;
constexpr int kMaxPool = kMaxPoolSlots;

__global__ __launch_bounds__(kGroupThreads) void k_group_by_len(GroupParams p) {
  __shared__ int s_len[kMaxPool];
  __shared__ unsigned char s_full[kMaxPool];
  __shared__ int s_order[kMaxPool];
  __shared__ int s_tot;
  __shared__ int s_nu;
  const int N = p.N, G = p.group;
  if (threadIdx.x == 0) { s_tot = 0; s_nu = 0; }
  for (int i = threadIdx.x; i < N; i += kGroupThreads) s_len[i] = p.len[p.ids ? p.ids[i] : i];
  __syncthreads();
  int myfull = 0;
  for (int i = threadIdx.x; i < N; i += kGroupThreads) {
    const int li = s_len[i];
    int eq = 0, eqb = 0;
    for (int j = 0; j < N; ++j) {
      const int e = s_len[j] == li;
      eq += e;
      eqb += e & (j < i);
    }
    const int full = eqb < (eq / G) * G;
    s_full[i] = (unsigned char)full;
    myfull += full;
  }
  atomicAdd(&s_tot, myfull);
  __syncthreads();
  const int tot = s_tot;
  for (int i = threadIdx.x; i < N; i += kGroupThreads) {
    const int li = s_len[i];
    int lt = 0, eqb = 0, fb = 0;  // fb: full members ranked before i
    for (int j = 0; j < N; ++j) {
      const int lj = s_len[j];
      const int less = lj < li, e = lj == li;
      lt += less;
      eqb += e & (j < i);
      fb += s_full[j] & (less | (e & (j < i)));
    }
    const int rank = lt + eqb;
    s_order[s_full[i] ? fb : tot + (rank - fb)] = i;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < N; i += kGroupThreads) p.order[i] = p.ids ? p.ids[s_order[i]] : s_order[i];
  const int nb = (N + G - 1) / G;
  int nu = 0;
  for (int g = threadIdx.x; g < nb; g += kGroupThreads) {
    int mn = s_len[s_order[g * G]], mx = mn;
    for (int k = g * G + 1; k < min(N, g * G + G); ++k) {
      const int l = s_len[s_order[k]];
      mn = min(mn, l);
      mx = max(mx, l);
    }
    p.uniform[g] = mn == mx;
    p.width[g] = mx;
    nu += mn == mx;
  }
  atomicAdd(&s_nu, nu);
  __syncthreads();
  if (threadIdx.x == 0) p.n_uniform[0] = s_nu;
}

hipError_t launch_group_by_len(const GroupParams &p, hipStream_t s) {
  hipLaunchKernelGGL(k_group_by_len, dim3(1), dim3(kGroupThreads), 0, s, p);
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
