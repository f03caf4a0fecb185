// Paged KV cache: a row's content lives in pages of a shared pool, listed in
// the row's block table, so the left-padded rectangle that the alignment
// invariant asks for ("Batch Speculative Decoding Done Right", section 2.1:
// equal pad + content length for every row, position ids 0.. over the content)
// is metadata: row b's pad is S' - len'_b.  EQSPEC's unpad-append-repad
// (section 2.2) then writes only each row's committed entries at its length;
// the KV already in the pages never moves.  The arXiv abstract of the same
// paper ties the superlinear realignment cost to contiguous layouts; this is
// the layout that removes it.  Committed and discarded speculative entries:
// "Inference Engineering Part 5/8", section "Acceptance changes across the
// workload".
//
// Layout: pages [L][2][n_pages][H][page][units * 16 bytes]; block table
// int32 [rows][max_blocks] (-1 = none); a stack of free page ids whose entries
// [0, n_free) are free; token ids int32 [rows][max_blocks * page] from 0.
//
// Page allocation: batch entries in order take their new pages from the top of
// the free stack, an entry's first new block getting the topmost remaining id;
// retiring pushes a row's pages back in block order, entries in batch order.
//
// Every workgroup of a call first runs the same plan (lengths, page counts and
// their exclusive prefix over the batch, checks) on the unchanged inputs, so
// all of them agree on the outcome; a call that fails a check writes nothing.
// Append and admit are one launch each: the workgroup that arrives last at a
// counter (after every other workgroup has finished reading the inputs)
// updates the block table, the free stack, lengths and token ids, and resets
// the counter.
#include <limits.h>
#include "device_common.h"
#include "launch.h"
#include "specdec.h"

namespace sd {

constexpr int kPgBlock = 256;                   // threads per workgroup
constexpr int kAppendKvWgs = kPagedMaxGrid - 1024;  // an append's KV-copy workgroups at most
constexpr int kPgPer = kMaxRealignRows / kPgBlock;  // batch entries per thread in the plan
static_assert(kPgPer * kPgBlock == kMaxRealignRows, "the plan covers every batch entry");

typedef int i32x4p __attribute__((ext_vector_type(4)));

constexpr int kFreeLds = 2048;  // entries of the free stack a call pops that are staged in LDS
constexpr int kRectPer = 4;     // positions per thread of a rectangle-view workgroup
constexpr int kRectChunk = kRectPer * kPgBlock;

struct PagedPlan {
  int r[kMaxRealignRows];         // pool row of each batch entry
  int c[kMaxRealignRows];         // its length before the call (0 for admit)
  int n[kMaxRealignRows];         // positions it gains
  int k0[kMaxRealignRows];        // pages taken by the entries before it
  int first_pg[kMaxRealignRows];  // page of a partly filled block an append starts in
  int nxt[kMaxRealignRows];       // an append's next token of each batch entry
  int freep[kFreeLds];            // freep[i] = free_pages[n_free - 1 - i], the i-th page popped
  int red[4 * (kPgBlock / kWave)];
  int need, smax, flags, n_free, last;
};

__device__ __forceinline__ int blocks_for(int n, int page) { return (n + page - 1) / page; }

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_i32(int x, int old) {
  return __builtin_amdgcn_update_dpp(old, x, CTRL, ROW_MASK, 0xF, false);
}

// The plan's reductions over the workgroup in one LDS round: the exclusive
// prefix of ksum in thread order and its total, the maximum of mx, the OR of
// fl and the minimum of first.  Within a wave by DPP lane moves (the scan by
// row shifts and row broadcasts; the others by quad swaps, mirrors and row
// broadcasts, which leave the wave's value in its last lane), then across the
// waves through LDS.
struct PlanSums {
  int before, total, mx, fl, first;
};

__device__ __forceinline__ PlanSums plan_reduce(int ksum, int mx, int fl, int first, int *red) {
  constexpr int NW = kPgBlock / kWave;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  int x = ksum;
  x += dpp_i32<0x111, 0xF>(x, 0);  // row_shr:1
  x += dpp_i32<0x112, 0xF>(x, 0);  // row_shr:2
  x += dpp_i32<0x114, 0xF>(x, 0);  // row_shr:4
  x += dpp_i32<0x118, 0xF>(x, 0);  // row_shr:8
  x += dpp_i32<0x142, 0xA>(x, 0);  // row_bcast:15
  x += dpp_i32<0x143, 0xC>(x, 0);  // row_bcast:31
#define SD_PLAN_RED_STEP(CTRL, MASK)              \
  mx = max(mx, dpp_i32<CTRL, MASK>(mx, mx));      \
  fl |= dpp_i32<CTRL, MASK>(fl, fl);              \
  first = min(first, dpp_i32<CTRL, MASK>(first, first));
  SD_PLAN_RED_STEP(0xB1, 0xF)   // quad_perm [1,0,3,2]
  SD_PLAN_RED_STEP(0x4E, 0xF)   // quad_perm [2,3,0,1]
  SD_PLAN_RED_STEP(0x141, 0xF)  // row_half_mirror
  SD_PLAN_RED_STEP(0x140, 0xF)  // row_mirror
  SD_PLAN_RED_STEP(0x142, 0xA)  // row_bcast:15
  SD_PLAN_RED_STEP(0x143, 0xC)  // row_bcast:31
#undef SD_PLAN_RED_STEP
  if (lane == kWave - 1) {
    red[w] = x;
    red[NW + w] = mx;
    red[2 * NW + w] = fl;
    red[3 * NW + w] = first;
  }
  __syncthreads();
  PlanSums r;
  r.before = x - ksum;
  r.total = 0;
  r.mx = INT_MIN;
  r.fl = 0;
  r.first = INT_MAX;
#pragma unroll
  for (int k = 0; k < NW; ++k) {
    if (k < w) r.before += red[k];
    r.total += red[k];
    r.mx = max(r.mx, red[NW + k]);
    r.fl |= red[2 * NW + k];
    r.first = min(r.first, red[3 * NW + k]);
  }
  return r;
}

// Exclusive prefix of v over the workgroup's threads (thread order) and the total.
__device__ __forceinline__ int block_excl_scan(int v, int *red, int &total) {
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
  for (int k = 0; k < kPgBlock / kWave; ++k) {
    if (k < w) before += red[k];
    total += red[k];
  }
  return before + x - v;
}

// The plan of an append (ADMIT = false: entry b gains accept_len[b] + 1
// positions at its length) or an admit (entry b's row must be empty and gains
// in_len[b] positions), from the call's unchanged inputs.  Returns the status
// bits of a failed check (0 = go).
template <bool ADMIT>
__device__ int paged_plan(const PagedParams &p, PagedPlan &s) {
  const int B = p.B, tcap = p.max_blocks * p.page;
  int bad = 0, cap = 0, mx = 0, ksum = 0;
  int kloc[kPgPer];
  // Three dependent round trips, each issuing all of its loads before any is
  // used (indices clamped into range, so no load waits behind a branch): the
  // entries' rows, gains and next tokens with the free-stack count; then the
  // rows' lengths with the top of the free stack; then the partly filled
  // blocks' pages.  Without a row map the lengths load in the first trip.
  // Results of out-of-range entries are not used.
  const int nf = *p.n_free;
  int width_in = 0;
  if (ADMIT) width_in = *p.in_width;
  int rr[kPgPer], cc[kPgPer], nn[kPgPer], xx[kPgPer], fpl[kPgPer];
  if (p.rowmap == nullptr) {  // entry b is row b: its length loads with the rest
#pragma unroll
    for (int e = 0; e < kPgPer; ++e) {
      const int b = min((int)threadIdx.x * kPgPer + e, B - 1);
      rr[e] = b;
      nn[e] = ADMIT ? p.in_len[b] : p.accept_len[b] + 1;
      xx[e] = ADMIT ? 0 : p.next_token[b];
      cc[e] = p.len[b < p.rows ? b : 0];
    }
  } else {
#pragma unroll
    for (int e = 0; e < kPgPer; ++e) {
      const int b = min((int)threadIdx.x * kPgPer + e, B - 1);
      rr[e] = p.rowmap[b];
      nn[e] = ADMIT ? p.in_len[b] : p.accept_len[b] + 1;
      xx[e] = ADMIT ? 0 : p.next_token[b];
    }
#pragma unroll
    for (int e = 0; e < kPgPer; ++e) {
      const int r = rr[e];
      cc[e] = p.len[r >= 0 && r < p.rows ? r : 0];
    }
  }
  // the top of the free stack, one entry per thread, before it is known how
  // many entries the call pops
  const bool nf_ok = nf >= 0 && nf <= p.n_pages;
  const int top = nf_ok && (int)threadIdx.x < nf ? p.free_pages[nf - 1 - (int)threadIdx.x] : -1;
#pragma unroll
  for (int e = 0; e < kPgPer; ++e) {
    // the block an append starts in, when partly filled (a safe index otherwise)
    const int r = rr[e], c = cc[e];
    const bool part = !ADMIT && r >= 0 && r < p.rows && c > 0 && c < tcap && c % p.page != 0;
    fpl[e] = p.bt[part ? (size_t)r * p.max_blocks + c / p.page : 0];
  }
#pragma unroll
  for (int e = 0; e < kPgPer; ++e) {
    const int b = threadIdx.x * kPgPer + e;
    if (b >= B) {
      rr[e] = cc[e] = nn[e] = 0;
      continue;
    }
    if (rr[e] < 0 || rr[e] >= p.rows) {
      bad |= SPECDEC_S_LEN_RANGE;
      rr[e] = 0;
    }
    if (!ADMIT) s.nxt[b] = xx[e];
  }
  if (ADMIT && (width_in < 0 || width_in > p.rect_cap)) bad |= SPECDEC_S_LEN_RANGE;
#pragma unroll
  for (int e = 0; e < kPgPer; ++e) {
    const int b = threadIdx.x * kPgPer + e;
    kloc[e] = 0;
    if (b >= B) continue;
    const int r = rr[e];
    int c = cc[e];
    const int n = nn[e];
    if (ADMIT) {
      if (c != 0 || n < 0 || n > width_in) bad |= SPECDEC_S_LEN_RANGE;
      c = 0;
    } else if (n < 1 || n > p.D + 1 || c < 0 || c > tcap) {
      bad |= SPECDEC_S_LEN_RANGE;
    }
    if (bad) continue;
    const int cn = c + n;
    if (cn > tcap) {
      cap = SPECDEC_S_CAPACITY;
      continue;
    }
    // a partly filled block an append starts in must already be a valid page
    int fp = -1;
    if (!ADMIT && c % p.page != 0) {
      fp = fpl[e];
      if (fp < 0 || fp >= p.n_pages) bad |= SPECDEC_S_LEN_RANGE;
    }
    s.r[b] = r;
    s.c[b] = c;
    s.n[b] = n;
    s.first_pg[b] = fp;
    kloc[e] = blocks_for(cn, p.page) - blocks_for(c, p.page);
    ksum += kloc[e];
    mx = max(mx, cn);
  }
  if (!nf_ok) bad |= SPECDEC_S_LEN_RANGE;
  // The pages about to be popped must be valid ids; the first kFreeLds are
  // staged in LDS.  The top kPgBlock entries are staged and checked before the
  // count the call pops is known (the lowest thread holding an invalid one),
  // any deeper ones after it.
  static_assert(kFreeLds >= kPgBlock, "the top of the free stack is staged whole");
  s.freep[threadIdx.x] = top;
  const bool top_bad = (int)threadIdx.x < nf && (top < 0 || top >= p.n_pages);
  const PlanSums red = plan_reduce(ksum, mx, bad | cap, top_bad ? (int)threadIdx.x : INT_MAX, s.red);
  const int total = red.total, smax = red.mx;
  int flags = red.fl | (red.first < total ? SPECDEC_S_LEN_RANGE : 0);
  int base = red.before;
#pragma unroll
  for (int e = 0; e < kPgPer; ++e) {
    const int b = threadIdx.x * kPgPer + e;
    if (b < B) s.k0[b] = base;
    base += kloc[e];
  }
  if (nf_ok && total > kPgBlock) {  // the call pops more pages than the staged top
    int deep = 0;
    for (int i = kPgBlock + (int)threadIdx.x; i < total && i < nf; i += kPgBlock) {
      const int pg = p.free_pages[nf - 1 - i];
      if (pg < 0 || pg >= p.n_pages) deep |= SPECDEC_S_LEN_RANGE;
      if (i < kFreeLds) s.freep[i] = pg;
    }
    flags |= block_or_int<kPgBlock>(deep, s.red);
  }
  if (!(flags & SPECDEC_S_LEN_RANGE)) {
    if (total > nf) flags |= SPECDEC_S_CAPACITY;
    if (!ADMIT && p.rect_tok && smax > p.rect_cap) flags |= SPECDEC_S_CAPACITY;
  }
  if (threadIdx.x == 0) {
    s.need = total;
    s.smax = smax;
    s.flags = flags;
    s.n_free = nf;
  }
  __syncthreads();
  return flags;
}

// Page id of block `blk` of batch entry b after the call's allocation (blk at
// or after the entry's first block touched).
// nb_old: the blocks entry b held before the call.  The free-stack entries
// past the staged ones are read with a non-temporal load, so the compiler
// keeps the two reads apart instead of merging them into one flat load (whose
// wait would also wait for every global load in flight).
__device__ __forceinline__ int page_at(const PagedParams &p, const PagedPlan &s, int b, int blk, int nb_old) {
  if (blk < nb_old) return s.first_pg[b];  // only the partly filled block an append starts in
  const int i = s.k0[b] + blk - nb_old;
  if (i < kFreeLds) return s.freep[i];
  return __builtin_nontemporal_load(p.free_pages + (s.n_free - 1 - i));
}

__device__ __forceinline__ int page_of(const PagedParams &p, const PagedPlan &s, int b, int blk) {
  return page_at(p, s, b, blk, blocks_for(s.c[b], p.page));
}

// Divisors of an append's KV copy, fixed per launch (computed on the host).
struct AppendDivs {
  FastDiv ups, u, h, b, page;
};

__device__ __forceinline__ size_t page_unit(const PagedParams &p, int lk, int pg, int h, int slot) {
  return ((((size_t)lk * p.n_pages + pg) * p.heads + h) * p.page + slot) * (size_t)p.units;
}

// Every workgroup of a call counts its arrival once, after all of its reads
// of the cache's metadata; the last one to arrive then commits the counts
// (lengths, free-stack count).  No fence is needed: a workgroup's reads have
// returned their values before its arrival is counted, so the commit's later
// writes cannot reach them, and the commit reads nothing another workgroup
// wrote.  Arrivals are counted in two levels so that no counter takes more than
// a few dozen atomics: workgroups in groups of kArriveGroup consecutive ids
// count in their group's counter; the last of each group counts in the root
// counter sync[0].  The counts are wrapping increments (atomicInc), so the
// last arrival at each counter returns it to zero for the next call.  Counters
// sit kSyncStride words apart, one per 128-byte line.  The count is split in
// two so that its first level overlaps the copy: arrive_issue (thread 0, right
// after the plan, whose barrier has seen every metadata read return) issues the
// group count and keeps the returned value; arrive_finish, after the copy,
// reads that value and, in the group's last workgroup, counts the group at the
// root.  (A wrapping increment is also left alone by the compiler's atomic
// optimizer, which would otherwise wait for an add's result right after issuing
// it, before the copy.)
//
// Ordering.  The only hazard is a workgroup's read of the metadata meeting the
// commit's write of it.  In the HIP memory model the arrivals would be
// agent-scope releases and the last arrival an acquire; on gfx950 those are an
// L2 write-back before every count and an L2 invalidate in the committer, which
// cost tens of microseconds per call (the same fences measured 14 to 75 us on
// the verification kernel), against 17 us for the whole append.  The kernel
// relies instead on the hardware's order: a workgroup's metadata loads have
// returned their values (they fed its plan, and the plan's last barrier waits
// for that) before its count is issued; counts on one line are performed one
// after another at the device's coherence point; and the committer issues its
// writes only after its own count has returned the final value.  So every read
// has completed before any write of the counts is issued.  The block-table
// entries and token ids an append's tables workgroup writes early are never
// read by a plan, and the KV stores are not ordered against the commit either:
// they touch other addresses and are read only after the kernel completes.
static_assert(kArriveGroup * (kPagedSyncWords / kSyncStride - 1) >= kPagedMaxGrid, "every group has its counter");

__device__ __forceinline__ int arrive_issue(const PagedParams &p) {
  if (threadIdx.x != 0) return 0;
  const int g = blockIdx.x / kArriveGroup;
  const int in_group = min(kArriveGroup, (int)gridDim.x - g * kArriveGroup);
  return (int)atomicInc(reinterpret_cast<unsigned int *>(p.sync + (size_t)(1 + g) * kSyncStride),
                        (unsigned int)(in_group - 1));
}

__device__ __forceinline__ bool arrive_finish(const PagedParams &p, PagedPlan &s, int old) {
  __syncthreads();
  if (threadIdx.x == 0) {
    const int g = blockIdx.x / kArriveGroup;
    const int groups = ((int)gridDim.x + kArriveGroup - 1) / kArriveGroup;
    const int in_group = min(kArriveGroup, (int)gridDim.x - g * kArriveGroup);
    int last = 0;
    if (old == in_group - 1)
      last = (int)atomicInc(reinterpret_cast<unsigned int *>(p.sync), (unsigned int)(groups - 1)) == groups - 1;
    s.last = last;
  }
  __syncthreads();
  return s.last;
}

// The commit of an append or an admit, in two parts.
// paged_commit_tables: the block-table entries of the blocks each entry
// gains, its token ids, and the duplicate-row status.  No plan reads what it
// writes (a plan reads a row's length, the free-stack count and entries, and
// only the table entry of the block its length ends in, which is never one it
// gains; the rectangle view reads token ids below each length), so an append
// runs it in its own workgroup right after the plan, alongside the copy.
// paged_commit_counts, by the last workgroup to arrive, once every plan has
// read the metadata: the lengths, the free-stack count, the width of an
// append; or only the status bits of a failed plan.
template <bool ADMIT>
__device__ void paged_commit_tables(const PagedParams &p, PagedPlan &s) {
  const int B = p.B, tcap = p.max_blocks * p.page;
  __shared__ int s_tab[2 * kMaxRealignRows];
  const int dup = block_any_duplicate<kPgBlock, 2 * kMaxRealignRows>(s.r, B, s_tab, s.red);
  for (int b = threadIdx.x; b < B; b += kPgBlock) {
    const int r = s.r[b], c = s.c[b], n = s.n[b];
    const int nb0 = blocks_for(c, p.page), nb1 = blocks_for(c + n, p.page);
    for (int blk = nb0; blk < nb1; ++blk) p.bt[(size_t)r * p.max_blocks + blk] = page_of(p, s, b, blk);
  }
  if (ADMIT) {
    // token ids: positions [S - n, S) of each input row, all entries at once
    const int S = *p.in_width;
    for (long x = threadIdx.x; x < (long)B * S; x += kPgBlock) {
      const int b = (int)(x / S), j = (int)(x - (long)b * S), n = s.n[b];
      if (j >= S - n) p.tokens[(size_t)s.r[b] * tcap + j - (S - n)] = p.rect_tok[(size_t)b * p.rect_cap + j];
    }
  } else {
    const int D1 = p.D + 1;
    for (int x = threadIdx.x; x < B * D1; x += kPgBlock) {
      const int b = x / D1, k = x - b * D1, n = s.n[b];
      if (k < n) p.tokens[(size_t)s.r[b] * tcap + s.c[b] + k] = k < n - 1 ? p.draft[(size_t)b * p.D + k]
                                                                          : s.nxt[b];
    }
  }
  if (threadIdx.x == 0 && dup) set_status(p.status, SPECDEC_S_ROWS_DUP);
}

template <bool ADMIT>
__device__ void paged_commit_counts(const PagedParams &p, PagedPlan &s) {
  if (s.flags) {
    if (threadIdx.x == 0) set_status(p.status, s.flags);
    return;
  }
  for (int b = threadIdx.x; b < p.B; b += kPgBlock) p.len[s.r[b]] = s.c[b] + s.n[b];
  if (threadIdx.x == 0) {
    *p.n_free = s.n_free - s.need;
    if (!ADMIT && p.width_out) *p.width_out = s.smax;
  }
}

// Append, one launch: workgroups [0, kv_wgs) copy the committed KV entries of
// every (layer, K|V, entry, head) sequence into their page slots; those after
// them (when the rectangle view is asked for) write row b's token ids,
// position ids and mask over [0, S'), kRectChunk positions each; the grid's
// last workgroup writes the block-table entries and token ids; the last
// workgroup to finish commits the lengths and the free-stack count.
__global__ __launch_bounds__(kPgBlock) void k_paged_append(PagedParams p, AppendDivs dv) {
  __shared__ PagedPlan s;
  const int flags = paged_plan<false>(p, s);
  const int arrived = arrive_issue(p);
  const int B = p.B, U = p.units, H = p.heads, D1 = p.D + 1;
  if (!flags && (int)blockIdx.x == (int)gridDim.x - 1) {
    paged_commit_tables<false>(p, s);
  } else if (!flags && (int)blockIdx.x >= p.kv_wgs) {
    // rectangle view: item (b, chunk) covers positions [chunk * kRectChunk, +kRectChunk) of row b
    const int chunks = (p.rect_cap + kRectChunk - 1) / kRectChunk;
    const int rect_wgs = (int)gridDim.x - 1 - p.kv_wgs;
    const int tcap = p.max_blocks * p.page, W = s.smax;
    for (int item = blockIdx.x - p.kv_wgs; item < p.B * chunks; item += rect_wgs) {
      const int b = item / chunks, j0 = (item - b * chunks) * kRectChunk;
      const int r = s.r[b], c = s.c[b], n = s.n[b], pad = W - c - n;
      int t[kRectPer];
#pragma unroll
      for (int k = 0; k < kRectPer; ++k) {  // every load of the chunk before any store
        const int j = j0 + k * kPgBlock + (int)threadIdx.x, x = j - pad;  // x: content index
        t[k] = p.pad_token;
        if (j < W && x >= 0)
          t[k] = x < c ? p.tokens[(size_t)r * tcap + x] : (x < c + n - 1 ? p.draft[(size_t)b * p.D + x - c]
                                                                           : s.nxt[b]);
      }
#pragma unroll
      for (int k = 0; k < kRectPer; ++k) {
        const int j = j0 + k * kPgBlock + (int)threadIdx.x, x = j - pad;
        if (j >= W) continue;
        p.rect_tok[(size_t)b * p.rect_cap + j] = t[k];
        if (p.rect_pos) p.rect_pos[(size_t)b * p.rect_cap + j] = x >= 0 ? x : 0;
        if (p.rect_mask) p.rect_mask[(size_t)b * p.rect_cap + j] = (int8_t)(x >= 0);
      }
    }
  } else if (!flags) {
    // flat unit q of kv_new [L*2][B][H][D+1][U] (the host keeps it below 2^31).
    // Every load of a pass is issued before any destination is worked out
    // (whose free-stack read would otherwise wait for the loads in flight).
    const uint32_t ups = (uint32_t)D1 * (uint32_t)U;
    const uint32_t total = (uint32_t)p.layers * 2u * (uint32_t)B * (uint32_t)H * ups;
    const i32x4p *nw = static_cast<const i32x4p *>(p.kv_new);
    i32x4p *pages = static_cast<i32x4p *>(p.pages);
    constexpr int kPer = 4;
    // one pass: kPer units per thread from unit q0 on
    auto pass = [&](uint32_t q0) {
      i32x4p v[kPer];
      uint32_t lk[kPer], bb[kPer], hh[kPer], ii[kPer], uu[kPer];
      bool ok[kPer];
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const uint32_t q = q0 + k * kPgBlock + threadIdx.x;
        const uint32_t seg = fdiv(q, dv.ups), rest = q - seg * ups;
        ii[k] = fdiv(rest, dv.u);
        uu[k] = rest - ii[k] * (uint32_t)U;
        const uint32_t t = fdiv(seg, dv.h);
        hh[k] = seg - t * (uint32_t)H;
        lk[k] = fdiv(t, dv.b);
        bb[k] = t - lk[k] * (uint32_t)B;
        ok[k] = q < total && (int)ii[k] < s.n[min(bb[k], (uint32_t)B - 1)];
        // a unit not copied re-reads the pass's first unit (one line per
        // wave), so no load sits behind a branch
        v[k] = __builtin_nontemporal_load(nw + (ok[k] ? q : q0));
      }
      // destinations, every page id read before the first store (a wait for a
      // page id read then covers no store)
      size_t at[kPer];
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int b = (int)min(bb[k], (uint32_t)B - 1), c = s.c[b], j = c + (int)ii[k];
        const int blk = (int)fdiv((uint32_t)j, dv.page), slot = j - blk * p.page;
        const int nb_old = (int)fdiv((uint32_t)(c + p.page - 1), dv.page);
        at[k] = ok[k] ? page_unit(p, (int)lk[k], page_at(p, s, b, blk, nb_old), (int)hh[k], slot) + uu[k] : 0;
      }
#pragma unroll
      for (int k = 0; k < kPer; ++k)
        if (ok[k]) pages[at[k]] = v[k];
    };
    // A grid that covers the units takes one pass with no loop around it, so
    // nothing in it waits for an earlier pass's stores.
    const uint32_t step = (uint32_t)p.kv_wgs * (kPgBlock * kPer), q0 = blockIdx.x * (uint32_t)(kPgBlock * kPer);
    if (step >= total) {
      if (q0 < total) pass(q0);  // (no units at all with zero layers)
    } else {
      for (uint32_t q = q0; q < total; q += step) pass(q);
    }
  }
  if (arrive_finish(p, s, arrived)) paged_commit_counts<false>(p, s);
}

// Admit, one launch: workgroups copy entry b's content, positions
// [S - in_len[b], S) of the input rectangle, into the pages the plan gives it;
// the last workgroup to finish commits.
__global__ __launch_bounds__(kPgBlock) void k_paged_admit(PagedParams p) {
  __shared__ PagedPlan s;
  const int flags = paged_plan<true>(p, s);
  const int arrived = arrive_issue(p);
  if (!flags) {
    const int B = p.B, U = p.units, H = p.heads;
    const int S = *p.in_width;
    const long nseg = (long)p.layers * 2 * B * H;
    const i32x4p *src = static_cast<const i32x4p *>(p.rect_kv);
    i32x4p *pages = static_cast<i32x4p *>(p.pages);
    const long per_seg = (long)S * U;
    const long total = nseg * per_seg;
    for (long q0 = (long)blockIdx.x * kPgBlock * 4; q0 < total; q0 += (long)gridDim.x * kPgBlock * 4) {
      i32x4p v[4];
      long dst[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const long q = q0 + k * kPgBlock + threadIdx.x;
        dst[k] = -1;
        if (q >= total) continue;
        const long seg = q / per_seg;
        const int w = (int)(q - seg * per_seg), pos = w / U, u = w - pos * U;
        const int lk = (int)(seg / ((long)B * H));
        const int rem = (int)(seg - (long)lk * B * H);
        const int b = rem / H, h = rem - b * H;
        const int j = pos - (S - s.n[b]);  // content index
        if (j < 0) continue;
        v[k] = __builtin_nontemporal_load(src + (((size_t)seg * p.rect_cap) + pos) * U + u);
        dst[k] = (long)page_unit(p, lk, page_of(p, s, b, j / p.page), h, j % p.page) + u;
      }
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (dst[k] >= 0) pages[dst[k]] = v[k];
    }
  }
  if (arrive_finish(p, s, arrived)) {
    if (!s.flags) paged_commit_tables<true>(p, s);
    paged_commit_counts<true>(p, s);
  }
}

// Gather: the batch's rows as a left-padded rectangle of width W = their
// longest length (zero KV bytes on the pad), read through the block table.
// Workgroups [0, kv_wgs) copy KV; the B after them write token ids, position
// ids, mask and length of one row each (and W).  A block-table entry outside
// [0, n_pages) is read as zero bytes and sets SPECDEC_S_LEN_RANGE.
__global__ __launch_bounds__(kPgBlock) void k_paged_gather(PagedParams p) {
  __shared__ int s_r[kMaxRealignRows], s_c[kMaxRealignRows];
  __shared__ int s_red[kPgBlock / kWave];
  const int B = p.B, U = p.units, H = p.heads, tcap = p.max_blocks * p.page;
  int bad = 0, mx = 0;
  for (int b = threadIdx.x; b < B; b += kPgBlock) {
    int r = p.rowmap ? p.rowmap[b] : b;
    if (r < 0 || r >= p.rows) {
      bad = 1;
      r = 0;
    }
    const int c = p.len[r];
    if (c < 0 || c > tcap) bad = 1;
    s_r[b] = r;
    s_c[b] = c;
    mx = max(mx, c);
  }
  const int W = block_max_int<kPgBlock>(mx, s_red);
  bad = block_or_int<kPgBlock>(bad, s_red);
  if (bad || W > p.rect_cap) {
    if (blockIdx.x == 0 && threadIdx.x == 0)
      set_status(p.status, bad ? SPECDEC_S_LEN_RANGE : SPECDEC_S_CAPACITY);
    return;
  }
  if ((int)blockIdx.x >= p.kv_wgs) {
    const int b = blockIdx.x - p.kv_wgs, r = s_r[b], c = s_c[b], pad = W - c;
    for (int j = threadIdx.x; j < W; j += kPgBlock) {
      const int k = j - pad;
      p.rect_tok[(size_t)b * p.rect_cap + j] = k >= 0 ? p.tokens[(size_t)r * tcap + k] : p.pad_token;
      if (p.rect_pos) p.rect_pos[(size_t)b * p.rect_cap + j] = k >= 0 ? k : 0;
      if (p.rect_mask) p.rect_mask[(size_t)b * p.rect_cap + j] = (int8_t)(k >= 0);
    }
    if (threadIdx.x == 0) {
      p.rect_len[b] = c;
      if (b == 0) *p.rect_width = W;
    }
    return;
  }
  const long nseg = (long)p.layers * 2 * B * H;
  const long per_seg = (long)W * U;
  const long total = nseg * per_seg;
  const i32x4p *pages = static_cast<const i32x4p *>(p.pages);
  i32x4p *dst = static_cast<i32x4p *>(p.rect_kv);
  int oob = 0;
  for (long q0 = (long)blockIdx.x * kPgBlock * 4; q0 < total; q0 += (long)p.kv_wgs * kPgBlock * 4) {
    i32x4p v[4];
    long at[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const long q = q0 + k * kPgBlock + threadIdx.x;
      at[k] = -1;
      v[k] = i32x4p{0, 0, 0, 0};
      if (q >= total) continue;
      const long seg = q / per_seg;
      const int w = (int)(q - seg * per_seg), pos = w / U, u = w - pos * U;
      const int lk = (int)(seg / ((long)B * H));
      const int rem = (int)(seg - (long)lk * B * H);
      const int b = rem / H, h = rem - b * H;
      at[k] = ((long)seg * p.rect_cap + pos) * U + u;
      const int j = pos - (W - s_c[b]);
      if (j < 0) continue;  // pad: zero
      const int pg = p.bt[(size_t)s_r[b] * p.max_blocks + j / p.page];
      if (pg < 0 || pg >= p.n_pages) {
        oob = 1;
        continue;
      }
      v[k] = __builtin_nontemporal_load(pages + page_unit(p, lk, pg, h, j % p.page) + u);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (at[k] >= 0) dst[at[k]] = v[k];
  }
  if (oob) set_status(p.status, SPECDEC_S_LEN_RANGE);
}

// Retire: the batch's rows push their pages on the free stack (block order,
// entries in batch order), their table entries become -1, their lengths 0.
// One workgroup.
__global__ __launch_bounds__(kPgBlock) void k_paged_retire(PagedParams p) {
  __shared__ int s_r[kMaxRealignRows], s_k0[kMaxRealignRows];
  __shared__ int s_red[kPgBlock / kWave];
  const int B = p.B, tcap = p.max_blocks * p.page;
  int bad = 0, ksum = 0;
  int kloc[kPgPer];
#pragma unroll
  for (int e = 0; e < kPgPer; ++e) {
    const int b = threadIdx.x * kPgPer + e;
    kloc[e] = 0;
    if (b >= B) continue;
    int r = p.rowmap ? p.rowmap[b] : b;
    if (r < 0 || r >= p.rows) {
      bad = 1;
      r = 0;
    }
    const int c = p.len[r];
    if (c < 0 || c > tcap) bad = 1;
    s_r[b] = r;
    kloc[e] = bad ? 0 : blocks_for(c, p.page);
    ksum += kloc[e];
  }
  int total;
  int base = block_excl_scan(ksum, s_red, total);
#pragma unroll
  for (int e = 0; e < kPgPer; ++e) {
    const int b = threadIdx.x * kPgPer + e;
    if (b < B) s_k0[b] = base;
    base += kloc[e];
  }
  int dup = 0;
  for (int b = threadIdx.x; b < B; b += kPgBlock)
    for (int o = 0; o < b; ++o) dup |= (s_r[o] == s_r[b]);
  const int nf = *p.n_free;
  if (nf < 0 || nf + total > p.n_pages) bad = 1;
  bad = block_or_int<kPgBlock>(bad | (dup << 1), s_red);
  if (bad) {
    if (threadIdx.x == 0) set_status(p.status, (bad & 1 ? SPECDEC_S_LEN_RANGE : 0) | (bad & 2 ? SPECDEC_S_ROWS_DUP : 0));
    return;
  }
  for (int b = threadIdx.x; b < B; b += kPgBlock) {
    const int r = s_r[b], nb = blocks_for(p.len[r], p.page);
    for (int blk = 0; blk < nb; ++blk) {
      p.free_pages[nf + s_k0[b] + blk] = p.bt[(size_t)r * p.max_blocks + blk];
      p.bt[(size_t)r * p.max_blocks + blk] = -1;
    }
  }
  __syncthreads();  // every length read above before any is cleared
  for (int b = threadIdx.x; b < B; b += kPgBlock) p.len[s_r[b]] = 0;
  if (threadIdx.x == 0) *p.n_free = nf + total;
}

hipError_t launch_paged(const PagedParams &q, hipStream_t st) {
  PagedParams p = q;
  const int cus = device_cus() < 1024 ? device_cus() : 1024;
  if (p.op == kPagedAppend) {
    // one pass of the copy per workgroup up to kAppendKvWgs workgroups (a grid
    // of at most kAppendKvWgs + 1024 workgroups)
    const long units = (long)p.layers * 2 * p.B * p.heads * (p.D + 1) * p.units;
    const long g = (units + kPgBlock * 4 - 1) / (kPgBlock * 4);
    p.kv_wgs = (int)(g < kAppendKvWgs ? (g > 0 ? g : 1) : kAppendKvWgs);
    const long items = p.rect_tok ? (long)p.B * ((p.rect_cap + kRectChunk - 1) / kRectChunk) : 0;
    const int extra = (int)(items < 1023 ? items : 1023) + 1;  // rectangle view, then the tables
    AppendDivs dv;
    dv.ups = host_fast_div((uint32_t)((p.D + 1) * p.units));
    dv.u = host_fast_div((uint32_t)p.units);
    dv.h = host_fast_div((uint32_t)p.heads);
    dv.b = host_fast_div((uint32_t)p.B);
    dv.page = host_fast_div((uint32_t)p.page);
    hipLaunchKernelGGL(k_paged_append, dim3((unsigned)(p.kv_wgs + extra)), dim3(kPgBlock), 0, st, p, dv);
  } else if (p.op == kPagedAdmit) {
    // units of the widest input the buffer allows; workgroups past the real count find none
    const long units = (long)p.layers * 2 * p.B * p.heads * p.rect_cap * p.units;
    const long g = (units + kPgBlock * 4 - 1) / (kPgBlock * 4);
    p.kv_wgs = (int)(g < 8L * cus ? (g > 0 ? g : 1) : 8L * cus);
    if (p.kv_wgs > kPagedMaxGrid) p.kv_wgs = kPagedMaxGrid;
    hipLaunchKernelGGL(k_paged_admit, dim3((unsigned)p.kv_wgs), dim3(kPgBlock), 0, st, p);
  } else if (p.op == kPagedGather) {
    const long units = (long)p.layers * 2 * p.B * p.heads * p.rect_cap * p.units;
    const long g = (units + kPgBlock * 4 - 1) / (kPgBlock * 4);
    p.kv_wgs = (int)(g < 16L * cus ? (g > 0 ? g : 1) : 16L * cus);
    hipLaunchKernelGGL(k_paged_gather, dim3((unsigned)(p.kv_wgs + p.B)), dim3(kPgBlock), 0, st, p);
  } else {
    hipLaunchKernelGGL(k_paged_retire, dim3(1), dim3(kPgBlock), 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace sd
