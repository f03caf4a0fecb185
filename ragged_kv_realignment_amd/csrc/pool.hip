// Lifecycle of a sequence pool ("Batch Speculative Decoding Done Right",
// section 2.3: EXSPEC keeps a pool of active sequences instead of a fixed batch
// and regroups them every round).  Around the per-round step (group, gather the
// mixed batches, verify, append) sequences finish and new prompts take their
// slots.  Policies (the pages name the pool, not its policies):
//  - every active sequence runs every round; `active` lists their slots in
//    schedule order;
//  - finish: after the append, a sequence finishes at the first newly committed
//    position p that holds the end-of-sequence id or has p + 1 >= max_len; its
//    length becomes p + 1, it leaves the active list (the others keep their
//    order), and its slot joins the free slots, kept in ascending order;
//  - admit: queued prompts, in queue order, go to the lowest free slots and
//    join the end of the active list; a prompt's content and token ids are
//    copied into its slot (the pool is left-aligned: content at [0, len)).
//
// Finish is one workgroup (slots <= 4096 fit LDS).  Admit is a one-workgroup
// plan that updates every list, length and token id and names the admitted
// slots, then a copy of the admitted prompts' KV by many workgroups.
#include "device_common.h"
#include "launch.h"
#include "specdec.h"

namespace sd {

constexpr int kPoolThreads = 1024;
constexpr int kPoolPer = kMaxPoolSlots / kPoolThreads;  // slots per thread in the scans
static_assert(kPoolPer * kPoolThreads == kMaxPoolSlots, "the scans cover every slot");

typedef int i32x4q __attribute__((ext_vector_type(4)));

// Exclusive prefix over the workgroup (thread order) of v, and the total.
__device__ __forceinline__ int pool_excl_scan(int v, int *red, int &total) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  int x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  __syncthreads();
  if (lane == kWave - 1) red[w] = x;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int k = 0; k < kPoolThreads / kWave; ++k) {
    if (k < w) before += red[k];
    total += red[k];
  }
  __syncthreads();
  return before + x - v;
}

__global__ __launch_bounds__(kPoolThreads) void k_pool_finish(PoolParams p) {
  __shared__ int s_inb[kMaxPoolSlots];     // 1 + batch index of each slot in this round's batch, 0 if absent
  __shared__ int s_newlen[kMaxPoolSlots];  // length after finishing, -1 if the slot goes on
  __shared__ unsigned char s_free[kMaxPoolSlots];
  __shared__ int s_act[kMaxPoolSlots];
  __shared__ int s_red[kPoolThreads / kWave];
  const int S = p.slots, B = p.B;
  const int na = *p.n_active, nf = *p.n_free;
  int bad = (na != B || nf < 0 || na + nf > S) ? SPECDEC_S_LEN_RANGE : 0;
  for (int s = threadIdx.x; s < S; s += kPoolThreads) {
    s_inb[s] = 0;
    s_newlen[s] = -1;
    s_free[s] = 0;
  }
  __syncthreads();
  // the round's batch: every entry an active slot, once; its committed tokens
  for (int j = threadIdx.x; j < B; j += kPoolThreads) {
    const int s = p.rows[j], a = p.accept_len[j];
    if (s < 0 || s >= S || a < 0 || a > p.D) {
      bad |= SPECDEC_S_LEN_RANGE;
      continue;
    }
    if (atomicCAS(&s_inb[s], 0, j + 1) != 0) bad |= SPECDEC_S_ROWS_DUP;
    const int cn = p.len[s], c = cn - (a + 1);
    if (c < 0 || cn > p.cap) {
      bad |= SPECDEC_S_LEN_RANGE;
      continue;
    }
    for (int q = c; q < cn; ++q)
      if (p.tokens[(size_t)s * p.cap + q] == p.eos_id || q + 1 >= p.max_len) {
        s_newlen[s] = q + 1;
        break;
      }
  }
  __syncthreads();
  if (!bad) {
    for (int j = threadIdx.x; j < na; j += kPoolThreads) {
      const int s = p.active[j];
      if (s < 0 || s >= S || s_inb[s] == 0) bad |= SPECDEC_S_LEN_RANGE;
      else s_act[j] = s;
    }
    for (int i = threadIdx.x; i < nf; i += kPoolThreads) {
      const int s = p.free_slots[i];
      if (s < 0 || s >= S) bad |= SPECDEC_S_LEN_RANGE;
      else s_free[s] = 1;
    }
  }
  bad = block_or_int<kPoolThreads>(bad, s_red);
  if (bad) {
    if (threadIdx.x == 0) set_status(p.status, bad);
    return;
  }
  // stable split of the active list into those going on and those finishing
  int keep[kPoolPer], nk = 0, nr = 0;
#pragma unroll
  for (int e = 0; e < kPoolPer; ++e) {
    const int j = threadIdx.x * kPoolPer + e;
    keep[e] = j < na ? (s_newlen[s_act[j]] < 0) : -1;
    nk += keep[e] == 1;
    nr += keep[e] == 0;
  }
  int tk, tr;
  int ok = pool_excl_scan(nk, s_red, tk);
  int orr = pool_excl_scan(nr, s_red, tr);
#pragma unroll
  for (int e = 0; e < kPoolPer; ++e) {
    const int j = threadIdx.x * kPoolPer + e;
    if (keep[e] == 1) p.active[ok++] = s_act[j];
    if (keep[e] == 0) {
      const int s = s_act[j];
      p.retired[orr++] = s;
      p.len[s] = s_newlen[s];
      s_free[s] = 1;
    }
  }
  __syncthreads();
  // the free slots in ascending order
  int fl = 0;
#pragma unroll
  for (int e = 0; e < kPoolPer; ++e) {
    const int s = threadIdx.x * kPoolPer + e;
    fl += s < S && s_free[s];
  }
  int tf;
  int of = pool_excl_scan(fl, s_red, tf);
#pragma unroll
  for (int e = 0; e < kPoolPer; ++e) {
    const int s = threadIdx.x * kPoolPer + e;
    if (s < S && s_free[s]) p.free_slots[of++] = s;
  }
  if (threadIdx.x == 0) {
    *p.n_active = tk;
    *p.n_free = tf;
    *p.n_retired = tr;
  }
}

// Admit, part 1 (one workgroup): k = min(free slots, queued prompts left)
// prompts go to the k lowest free slots; every list, the lengths and the token
// ids are updated, and admitted / n_admitted name the slots.  A prompt longer
// than the pool's rows admits nothing and sets SPECDEC_S_CAPACITY.
__global__ __launch_bounds__(kPoolThreads) void k_pool_admit_plan(PoolParams p) {
  __shared__ int s_red[kPoolThreads / kWave];
  __shared__ int s_fr[kMaxPoolSlots];
  const int S = p.slots;
  const int na = *p.n_active, nf = *p.n_free, qh = *p.q_head;
  int bad = (na < 0 || nf < 0 || na + nf > S || qh < 0 || qh > p.Q) ? SPECDEC_S_LEN_RANGE : 0;
  const int k = bad ? 0 : min(nf, p.Q - qh);
  for (int i = threadIdx.x; i < k; i += kPoolThreads) {
    const int n = p.plen[qh + i], s = p.free_slots[i];
    if (n < 0 || n > p.pcap || s < 0 || s >= S) bad |= SPECDEC_S_LEN_RANGE;
    else if (n > p.cap) bad |= SPECDEC_S_CAPACITY;
  }
  for (int i = threadIdx.x; i < nf && !bad; i += kPoolThreads) s_fr[i] = p.free_slots[i];
  bad = block_or_int<kPoolThreads>(bad, s_red);
  if (bad) {
    if (threadIdx.x == 0) {
      *p.n_admitted = 0;
      set_status(p.status, bad);
    }
    return;
  }
  for (int i = threadIdx.x; i < k; i += kPoolThreads) {
    const int s = s_fr[i], q = qh + i;
    p.active[na + i] = s;
    p.admitted[i] = s;
    p.len[s] = p.plen[q];
  }
  for (int i = k + (int)threadIdx.x; i < nf; i += kPoolThreads) p.free_slots[i - k] = s_fr[i];
  // token ids of the admitted prompts: one wave per prompt, the waves over
  // the prompts at once, eight loads per lane in flight (positions past the
  // prompt re-read its first token and are not stored)
  {
    constexpr int kR = 8;
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    for (int i = w; i < k; i += kPoolThreads / kWave) {
      const int q = qh + i, n = p.plen[q];
      int32_t *to = p.tokens + (size_t)s_fr[i] * p.cap;
      const int32_t *from = p.ptok + (size_t)q * p.pcap;
      for (int j0 = lane; j0 < n; j0 += kWave * kR) {
        int v[kR];
#pragma unroll
        for (int r = 0; r < kR; ++r) {
          const int j = j0 + r * kWave;
          v[r] = from[j < n ? j : 0];
        }
#pragma unroll
        for (int r = 0; r < kR; ++r) {
          const int j = j0 + r * kWave;
          if (j < n) to[j] = v[r];
        }
      }
    }
  }
  if (threadIdx.x == 0) {
    *p.n_active = na + k;
    *p.n_free = nf - k;
    *p.q_head = qh + k;
    *p.n_admitted = k;
  }
}

// Admit, part 2: the KV of admitted prompt i (queue entry q_head - k + i,
// q_head already advanced) into slot admitted[i], positions [0, plen).
// Workgroups stride over (prompt, layer, K|V, head) sequences.
__global__ __launch_bounds__(256) void k_pool_admit_copy(PoolParams p) {
  const int k = *p.n_admitted;
  const int q0 = *p.q_head - k;
  const int H = p.heads, U = p.units;
  const long nseg = (long)k * p.layers * 2 * H;
  const i32x4q *src = static_cast<const i32x4q *>(p.pkv);
  i32x4q *dst = static_cast<i32x4q *>(p.kv);
  for (long seg = blockIdx.x; seg < nseg; seg += gridDim.x) {
    const int i = (int)(seg / ((long)p.layers * 2 * H));
    const int rem = (int)(seg - (long)i * p.layers * 2 * H);
    const int lk = rem / H, h = rem - lk * H;
    const int q = q0 + i, s = p.admitted[i], n = p.plen[q];
    const i32x4q *from = src + ((((size_t)lk * p.Q + q) * H + h) * p.pcap) * U;
    i32x4q *to = dst + ((((size_t)lk * p.slots + s) * H + h) * p.cap) * U;
    // four 16-byte units per thread per step, two steps in flight: a step's
    // loads are issued two steps ahead, each right after the stores of the
    // registers they refill, so (the vector-memory counter being in order) the
    // wait for a step's loads never covers earlier stores.  Units past the
    // sequence re-read its first unit and are not stored, so no load sits
    // behind a branch.
    const int nu = n * U;
    if (nu <= 0) continue;
    constexpr int kStep = 4 * 256;
    i32x4q a[4], b[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int ua = threadIdx.x + t * 256, ub = ua + kStep;
      a[t] = __builtin_nontemporal_load(from + (ua < nu ? ua : 0));
      b[t] = __builtin_nontemporal_load(from + (ub < nu ? ub : 0));
    }
    for (int u0 = threadIdx.x; u0 < nu; u0 += 2 * kStep) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int u = u0 + t * 256;
        if (u < nu) to[u] = a[t];
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int u = u0 + 2 * kStep + t * 256;
        a[t] = __builtin_nontemporal_load(from + (u < nu ? u : 0));
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int u = u0 + kStep + t * 256;
        if (u < nu) to[u] = b[t];
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int u = u0 + 3 * kStep + t * 256;
        b[t] = __builtin_nontemporal_load(from + (u < nu ? u : 0));
      }
    }
  }
}

hipError_t launch_pool_finish(const PoolParams &p, hipStream_t st) {
  hipLaunchKernelGGL(k_pool_finish, dim3(1), dim3(kPoolThreads), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_pool_admit(const PoolParams &p, hipStream_t st) {
  hipLaunchKernelGGL(k_pool_admit_plan, dim3(1), dim3(kPoolThreads), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // sequences of the widest possible admission; workgroups past the real count find none
  const int kmax = p.slots < p.Q ? p.slots : p.Q;
  const long seqs = (long)kmax * p.layers * 2 * p.heads;
  const long g = seqs < 16L * device_cus() ? seqs : 16L * device_cus();
  if (g > 0) hipLaunchKernelGGL(k_pool_admit_copy, dim3((unsigned)g), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace sd
