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
// (workgroup size / units) consecutive positions per pass, so a wave reads and writes
// contiguous bytes.  Loads and stores are raw buffer operations on one
// descriptor per source and destination sequence (buffer_io.h).  Pad positions are
// thereby store-only, the tile body is straight-line code, and each thread
// keeps all of its loads in flight before its stores.
#include <limits.h>
#include "buffer_io.h"
#include "device_common.h"
#include "realign_params.h"
#include "specdec.h"

namespace sd {

constexpr int kMaxB = kMaxRealignRows;

// Tuning knobs (defaults are the measured best on MI355X).
#ifndef SPECDEC_RA_BLOCK
#define SPECDEC_RA_BLOCK 1024    // threads per realign workgroup
#endif
#ifndef SPECDEC_RA_TILES_PER_WG
#define SPECDEC_RA_TILES_PER_WG 2  // EQSPEC grid: tiles of the widest possible output per workgroup
#endif
#ifndef SPECDEC_AP_WGS_PER_CU
#define SPECDEC_AP_WGS_PER_CU 2  // in-place append: workgroups per CU at most
#endif
#ifndef SPECDEC_GA_TILES_PER_WG
#define SPECDEC_GA_TILES_PER_WG 8  // GATHER grid: tiles per workgroup if every group were gathered
#endif
// Positions per thread per tile: short rows take small tiles, rows that hold
// at least two large tiles take large ones (see launch_realign).
#ifndef SPECDEC_RA_PASSES
#define SPECDEC_RA_PASSES 4
#endif
#ifndef SPECDEC_RA_PASSES_LONG
#define SPECDEC_RA_PASSES_LONG 12
#endif
#ifndef SPECDEC_RA_INTERLEAVE
#define SPECDEC_RA_INTERLEAVE 1  // tile t -> workgroup t mod grid (1) or contiguous ranges (0)
#endif
constexpr int kPassesShort = SPECDEC_RA_PASSES, kPassesLong = SPECDEC_RA_PASSES_LONG;
constexpr int kRaBlock = SPECDEC_RA_BLOCK;

// A destination tile of the pipelined copy: positions [j_lo, j_lo + TP) of one
// sequence; position j < a_hi takes source position j - a_lo when j >= a_lo and
// zero otherwise (pad); positions at or past a_hi are not written here.
struct Tile {
  __amdgpu_buffer_rsrc_t ra, rd;
  int j_lo, a_lo, a_hi;
};

__device__ __forceinline__ Tile empty_tile() {
  Tile t;
  t.ra = rsrc(nullptr, 0);
  t.rd = rsrc(nullptr, 0);
  t.j_lo = 0;
  t.a_lo = 0;
  t.a_hi = 0;
  return t;
}

template <int kPasses>
__device__ __forceinline__ void load_tile(const Tile &t, i32x4 *v, int poff, int PP, int U, int u, bool act) {
#pragma unroll
  for (int k = 0; k < kPasses; ++k) {
    const int j = t.j_lo + poff + k * PP;
    const bool in = act && j >= t.a_lo && j < t.a_hi;
    v[k] = bld(t.ra, in ? (uint32_t)((j - t.a_lo) * U + u) * 16u : kOOB);
  }
}

template <int kPasses>
__device__ __forceinline__ void store_tile(const Tile &t, const i32x4 *v, int poff, int PP, int U, int u, bool act) {
#pragma unroll
  for (int k = 0; k < kPasses; ++k) {
    const int j = t.j_lo + poff + k * PP;
    bst(v[k], t.rd, (act && j < t.a_hi) ? (uint32_t)(j * U + u) * 16u : kOOB);
  }
}

// Block-wide max of `mx` and OR of `bits` with a single barrier (scratch arrays
// hold one entry per wave and are not reused before the barrier).
__device__ __forceinline__ void block_max_or(int mx, int bits, int *s_m, int *s_o, int &out_mx, int &out_bits) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) {
    mx = max(mx, __shfl_xor(mx, off));
    bits |= __shfl_xor(bits, off);
  }
  if ((threadIdx.x & (kWave - 1)) == 0) {
    s_m[threadIdx.x / kWave] = mx;
    s_o[threadIdx.x / kWave] = bits;
  }
  __syncthreads();
  out_mx = s_m[0];
  out_bits = s_o[0];
#pragma unroll
  for (int k = 1; k < kRaBlock / kWave; ++k) {
    out_mx = max(out_mx, s_m[k]);
    out_bits |= s_o[k];
  }
}

// This workgroup's tiles: t = first, first + step, ... < end.  Interleaved
// (t mod grid) keeps all resident workgroups within one window of consecutive
// tiles, so the pages they touch stay few; contiguous ranges are the
// alternative.
struct Sched {
  uint32_t first, end, step;
};

__device__ __forceinline__ Sched my_tiles(uint32_t ntiles) {
  Sched s;
#if SPECDEC_RA_INTERLEAVE
  s.first = blockIdx.x;
  s.end = ntiles;
  s.step = gridDim.x;
#else
  const uint32_t per = (ntiles + gridDim.x - 1) / gridDim.x;
  s.first = blockIdx.x * per;
  s.end = min(ntiles, s.first + per);
  s.step = 1;
#endif
  return s;
}

// Software-pipelined copy over this workgroup's tiles: a tile's loads are
// issued before the previous tile's stores, so waiting for loads never waits
// for stores (the gfx9 vector-memory counter is in order).
template <int kPasses, typename TileAt>
__device__ __forceinline__ void run_tiles(uint32_t ntiles, TileAt tile_at, int poff, int PP, int U, int u,
                                          bool act) {
  const Sched sc = my_tiles(ntiles);
  if (sc.first >= sc.end) return;
  Tile cur = tile_at(sc.first);
  i32x4 v[kPasses];
  load_tile<kPasses>(cur, v, poff, PP, U, u, act);
  for (uint32_t t = sc.first; t < sc.end; t += sc.step) {
    const uint32_t tn = t + sc.step;
    Tile nxt = tn < sc.end ? tile_at(tn) : empty_tile();
    i32x4 w[kPasses];
    load_tile<kPasses>(nxt, w, poff, PP, U, u, act);
    store_tile<kPasses>(cur, v, poff, PP, U, u, act);
    cur = nxt;
#pragma unroll
    for (int k = 0; k < kPasses; ++k) v[k] = w[k];
  }
}

// EQSPEC tile (seg, chunk): old content [pin, S) of the input sequence lands at
// [pout, pout + c) of the output; the committed entries after it are copied
// separately.
__device__ __forceinline__ Tile eq_tile(const char *in, char *out, const RealignParams &p, long seg, int chunk, int b,
                                        const int *s_c, const int *s_n, int S, int Snew, int TP, size_t pos_bytes) {
  const int c = uni(s_c[b]), n = uni(s_n[b]);
  const int pin = S - c, pout = Snew - c - n;
  Tile t;
  t.ra = rsrc(in + ((size_t)seg * p.cap_in + pin) * pos_bytes, (uint32_t)(c * pos_bytes));
  t.rd = rsrc(out + (size_t)seg * p.cap_out * pos_bytes, (uint32_t)((pout + c) * pos_bytes));
  t.j_lo = chunk * TP;
  t.a_lo = pout;
  t.a_hi = pout + c;
  return t;
}

// ------------------------------------------------------------------ EQSPEC
template <int kPasses>
__global__ __launch_bounds__(kRaBlock) void k_realign_eqspec(RealignParams p) {
  __shared__ int s_c[kMaxB];
  __shared__ int s_n[kMaxB];
  __shared__ int s_red[kRaBlock / kWave];
  __shared__ int s_red2[kRaBlock / kWave];
  const int B = p.B, D = p.D, U = p.units, H = p.heads;
  const int S = p.width_in[0];
  int mx = 0, bad = (S < 0 || S > p.cap_in) ? SPECDEC_S_LEN_RANGE : 0;
  for (int b = threadIdx.x; b < B; b += kRaBlock) {
    const int c = p.len_in[b], a = p.accept_len[b];
    if (c < 0 || c > S || a < 0 || a > D) bad = SPECDEC_S_LEN_RANGE;
    s_c[b] = c;
    s_n[b] = a + 1;
    mx = max(mx, c + a + 1);
  }
  // one fused reduction (new width, error bits) with a single barrier
  int Snew;
  block_max_or(mx, bad, s_red, s_red2, Snew, bad);
  if (!bad && Snew > p.cap_out) bad = SPECDEC_S_CAPACITY;
  if (bad) {
    if (blockIdx.x == 0 && threadIdx.x == 0) set_status(p.status, bad);
    return;
  }

  const int PP = kRaBlock / U;             // positions per pass
  const int TP = PP * kPasses;           // positions per tile
  const int chunks = (Snew + TP - 1) / TP;
  const long nseg = (long)p.layers * 2 * B * H;
  const int poff = threadIdx.x / U, u = threadIdx.x - poff * U;
  const bool active = poff < PP;
  const char *in = static_cast<const char *>(p.kv_in);
  char *out = static_cast<char *>(p.kv_out);
  const char *nw = static_cast<const char *>(p.kv_new);
  const size_t pos_bytes = (size_t)U * 16;

  // 1. the n committed entries of every sequence: positions [Snew - n, Snew);
  // a workgroup pass covers kRaBlock / ((D+1)*U) sequences
  {
    const int ups = (D + 1) * U;
    const int spp = max(1, kRaBlock / ups);
    const int sq = threadIdx.x / ups, f = threadIdx.x - sq * ups;
    for (long s0 = (long)blockIdx.x * spp; s0 < nseg; s0 += (long)gridDim.x * spp) {
      const long sg = s0 + sq;
      if (sq < spp && sg < nseg) {
        const int b = (int)((sg / H) % B);
        const int n = s_n[b];
        const char *src = nw + (size_t)sg * (D + 1) * pos_bytes;
        char *dst = out + ((size_t)sg * p.cap_out + (Snew - n)) * pos_bytes;
        for (int g = f; g < n * U; g += ups)
          *reinterpret_cast<i32x4 *>(dst + (size_t)g * 16) = __builtin_nontemporal_load(
              reinterpret_cast<const i32x4 *>(src + (size_t)g * 16));
      }
    }
  }

  // 2. pad and old content, positions [0, Snew - n): tiles of TP positions,
  // software-pipelined so a tile's loads are issued before the previous tile's
  // stores (waiting for loads then never waits for stores)
  const FastDiv fd_chunks = fast_div(chunks), fd_h = fast_div(H), fd_b = fast_div(B);
  auto tile_at = [&](uint32_t t) {
    const uint32_t seg = fdiv(t, fd_chunks);
    const int chunk = (int)(t - seg * chunks);
    const uint32_t sh = fdiv(seg, fd_h);
    const int b = (int)(sh - fdiv(sh, fd_b) * B);
    return eq_tile(in, out, p, seg, chunk, b, s_c, s_n, S, Snew, TP, pos_bytes);
  };
  run_tiles<kPasses>((uint32_t)(nseg * chunks), tile_at, poff, PP, U, u, active);

  // token ids, position ids and mask of every row, on [0, Snew)
  for (int b = blockIdx.x; b < B; b += gridDim.x) {
    const int c = s_c[b], n = s_n[b], a = n - 1;
    const int pin = S - c, pout = Snew - c - n;
    const int32_t *ti = p.tok_in + (size_t)b * p.cap_in;
    int32_t *to = p.tok_out + (size_t)b * p.cap_out;
    int32_t *po = p.pos_out + (size_t)b * p.cap_out;
    int8_t *mo = p.mask_out + (size_t)b * p.cap_out;
    for (int j = threadIdx.x; j < Snew; j += kRaBlock) {
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
template <int kPasses>
__global__ __launch_bounds__(kRaBlock) void k_gather(RealignParams p) {
  __shared__ int s_r[kMaxB];
  __shared__ int s_c[kMaxB];
  __shared__ int s_W[kMaxB];
  __shared__ int s_act[kMaxB];
  __shared__ int s_gpre[kMaxB];
  __shared__ int s_nact;
  __shared__ int s_red[kRaBlock / kWave];
  __shared__ int s_red2[kRaBlock / kWave];
  const int B = p.B, G = p.group, U = p.units, H = p.heads;
  const int ng = (B + G - 1) / G;
  int bad = 0;
  for (int j = threadIdx.x; j < B; j += kRaBlock) {
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
  for (int g = threadIdx.x; g < ng; g += kRaBlock) {
    int W = 0;
    for (int j = g * G; j < min(B, g * G + G); ++j) W = max(W, s_c[j]);
    const bool skip = p.skip_group && p.skip_group[g];
    s_W[g] = skip ? -1 : W;
    if (!skip) {
      wmax = max(wmax, W);
      if (W > p.cap_out) bad |= SPECDEC_S_CAPACITY;
    }
  }
  int Wmax;
  block_max_or(wmax, bad, s_red, s_red2, Wmax, bad);
  if (bad) {
    if (blockIdx.x == 0 && threadIdx.x == 0) set_status(p.status, bad);
    return;
  }
  // compact the entries of the gathered groups: exclusive prefix of the groups'
  // entry counts (wave 0, 64 groups per step), then every entry places itself
  if (threadIdx.x < kWave) {
    int carry = 0;
    for (int g0 = 0; g0 < ng; g0 += kWave) {
      const int g = g0 + (int)threadIdx.x;
      const int cnt = (g < ng && s_W[g] >= 0) ? min(B, g * G + G) - g * G : 0;
      int incl = cnt;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if ((int)threadIdx.x >= off) incl += y;
      }
      if (g < ng) s_gpre[g] = carry + incl - cnt;
      carry += __shfl(incl, kWave - 1);
    }
    if (threadIdx.x == 0) s_nact = carry;
  }
  __syncthreads();
  for (int j = threadIdx.x; j < B; j += kRaBlock) {
    const int g = j / G;
    if (s_W[g] >= 0) s_act[s_gpre[g] + (j - g * G)] = j;
  }
  __syncthreads();
  const int nact = s_nact;

  const int PP = kRaBlock / U;
  const int TP = PP * kPasses;
  const int chunks = (Wmax + TP - 1) / TP;
  const long nseg = (long)p.layers * 2 * nact * H;
  const int poff = threadIdx.x / U, u = threadIdx.x - poff * U;
  const bool active = poff < PP;
  const char *in = static_cast<const char *>(p.kv_in);
  char *out = static_cast<char *>(p.kv_out);
  const size_t pos_bytes = (size_t)U * 16;

  // tile (seg, chunk) of active entry k: the pool row's content [0, c) lands at
  // [W - c, W) of the rectangle row; the same pipelined copy as EQSPEC
  if (chunks > 0) {
    const FastDiv fd_chunks = fast_div(chunks), fd_kh = fast_div(nact * H), fd_h = fast_div(H);
    auto tile_at = [&](uint32_t t) {
      const uint32_t seg = fdiv(t, fd_chunks);
      const int chunk = (int)(t - seg * chunks);
      const uint32_t lk = fdiv(seg, fd_kh);
      const uint32_t rem = seg - lk * (uint32_t)(nact * H);
      const uint32_t k = fdiv(rem, fd_h), h = rem - k * H;
      const int j = uni(s_act[k]);
      const int r = uni(s_r[j]), c = uni(s_c[j]), W = uni(s_W[j / G]);
      Tile t2;
      t2.ra = rsrc(in + ((size_t)(lk * p.rows_in + r) * H + h) * p.cap_in * pos_bytes, (uint32_t)(c * pos_bytes));
      t2.rd = rsrc(out + ((size_t)(lk * p.rows_out + j) * H + h) * p.cap_out * pos_bytes, (uint32_t)(W * pos_bytes));
      t2.j_lo = chunk * TP;
      t2.a_lo = W - c;
      t2.a_hi = W;
      return t2;
    };
    run_tiles<kPasses>((uint32_t)(nseg * chunks), tile_at, poff, PP, U, u, active);
  }

  for (int k = blockIdx.x; k < nact; k += gridDim.x) {
    const int j = s_act[k], r = s_r[j], c = s_c[j], W = s_W[j / G];
    const int pad = W - c;
    const int32_t *ti = p.tok_in ? p.tok_in + (size_t)r * p.cap_in : nullptr;
    int32_t *to = p.tok_out ? p.tok_out + (size_t)j * p.cap_out : nullptr;
    int32_t *po = p.pos_out ? p.pos_out + (size_t)j * p.cap_out : nullptr;
    int8_t *mo = p.mask_out ? p.mask_out + (size_t)j * p.cap_out : nullptr;
    for (int x = threadIdx.x; x < W; x += kRaBlock) {
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
  for (int b = threadIdx.x; b < p.B; b += kRaBlock) {
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
  return block_or_int<kRaBlock>(bad, s_red);
}

// Divisors of the append's sequence numbering, fixed per launch (computed on
// the host): seg = (lk * B + b) * H + h.
struct AppendKvDivs {
  FastDiv bh, h;
};

// KV entries: tile = one (layer, K|V, entry, head) sequence, n_b positions.
// A workgroup pass covers kRaBlock / ((D+1) U) sequences, one 16-byte unit per
// thread (unit g of a sequence, g < (D+1) U, copied when g < n_b U).  Each
// workgroup takes passes s0, s0 + step, ... in two alternating registers: a
// pass's load is issued two passes ahead, right after the store of the
// register it refills.  A unit not copied re-reads the sequence's first unit
// and is not stored, so no load sits behind a branch.  Few workgroups (two per
// CU) carry many passes: each one first checks the whole batch (two round
// trips and a reduction), which a pass-per-workgroup grid paid over and over.
__global__ __launch_bounds__(kRaBlock) void k_append_kv(RealignParams p, AppendKvDivs dv) {
  __shared__ int s_r[kMaxB];
  __shared__ int s_c[kMaxB];
  __shared__ int s_n[kMaxB];
  __shared__ int s_red[kRaBlock / kWave];
  if (append_check(p, s_r, s_c, s_n, s_red)) return;  // reported by k_append_meta
  const int B = p.B, U = p.units, H = p.heads, D1 = p.D + 1;
  const uint32_t nseg = (uint32_t)p.layers * 2u * (uint32_t)B * (uint32_t)H;
  const i32x4 *nw = static_cast<const i32x4 *>(p.kv_new);
  i32x4 *pool = static_cast<i32x4 *>(p.kv_out);
  const int ups = D1 * U;
  const int spp = max(1, kRaBlock / ups);
  const int sq = threadIdx.x / ups, f = threadIdx.x - sq * ups;
  const uint32_t step = gridDim.x * (uint32_t)spp;
  // this thread's unit of pass s0: its source, and its destination or SIZE_MAX
  auto unit = [&](uint32_t s0, size_t &src, size_t &dst) {
    const uint32_t seg = s0 + (uint32_t)sq;
    src = 0;
    dst = SIZE_MAX;
    if (sq >= spp || seg >= nseg) return;
    const uint32_t lk = fdiv(seg, dv.bh), rem = seg - lk * (uint32_t)(B * H);
    const uint32_t b = fdiv(rem, dv.h), h = rem - b * (uint32_t)H;
    src = (size_t)seg * ups;
    if (f >= s_n[b] * U) return;
    src += f;
    dst = (((size_t)lk * p.rows_in + s_r[b]) * H + h) * (size_t)p.cap_in * U + (size_t)s_c[b] * U + f;
  };
  size_t sa, da, sb, db;
  const uint32_t s0 = blockIdx.x * (uint32_t)spp;
  unit(s0, sa, da);
  unit(s0 + step, sb, db);
  i32x4 a = __builtin_nontemporal_load(nw + sa), b = __builtin_nontemporal_load(nw + sb);
  for (uint32_t s = s0; s < nseg; s += 2 * step) {
    if (da != SIZE_MAX) pool[da] = a;
    unit(s + 2 * step, sa, da);
    a = __builtin_nontemporal_load(nw + sa);
    if (db != SIZE_MAX) pool[db] = b;
    unit(s + 3 * step, sb, db);
    b = __builtin_nontemporal_load(nw + sb);
  }
}

// Token ids and lengths, after the KV copy (stream order keeps len stable
// while k_append_kv reads it).
__global__ __launch_bounds__(kRaBlock) void k_append_meta(RealignParams p) {
  __shared__ int s_r[kMaxB];
  __shared__ int s_c[kMaxB];
  __shared__ int s_n[kMaxB];
  __shared__ int s_red[kRaBlock / kWave];
  const int bad = append_check(p, s_r, s_c, s_n, s_red);
  if (bad) {
    if (threadIdx.x == 0) set_status(p.status, bad);
    return;
  }
  const int B = p.B;
  __shared__ int s_tab[2 * kMaxB];
  const int dup = block_any_duplicate<kRaBlock, 2 * kMaxB>(s_r, B, s_tab, s_red);
  for (int b = threadIdx.x; b < B; b += kRaBlock) {
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
  const int cus = device_cus();
  // Large tiles when the output rows hold at least two of them: measured on
  // MI355X, 12 positions per thread were 10-20% faster than 4 for rows of
  // 2,057-4,256 positions (and even at 2,432) and 5% slower at 1,344.
  const long pp = kRaBlock / p.units;  // positions per pass
  const bool long_rows = p.cap_out >= 2 * pp * kPassesLong;
  const long tp = pp * (long_rows ? kPassesLong : kPassesShort);
  // tiles of the widest output the buffers allow (the true width is known only
  // on the device); workgroups past the real tile count find no tile
  const long seqs = (long)p.layers * 2 * p.B * p.heads;
  const long tiles_max = seqs * ((p.cap_out + tp - 1) / tp);
  int grid = 8 * cus;
  if (p.mode == SPECDEC_EQSPEC) {
    const long g = (tiles_max + SPECDEC_RA_TILES_PER_WG - 1) / SPECDEC_RA_TILES_PER_WG;
    if (g > grid) grid = (int)(g < (1L << 30) ? g : (1L << 30));
    if (long_rows)
      hipLaunchKernelGGL(k_realign_eqspec<kPassesLong>, dim3(grid), dim3(kRaBlock), 0, s, p);
    else
      hipLaunchKernelGGL(k_realign_eqspec<kPassesShort>, dim3(grid), dim3(kRaBlock), 0, s, p);
  } else if (p.mode == SPECDEC_GATHER) {
    const long g = (tiles_max + SPECDEC_GA_TILES_PER_WG - 1) / SPECDEC_GA_TILES_PER_WG;
    if (g > grid) grid = (int)(g < (1L << 30) ? g : (1L << 30));
    if (long_rows)
      hipLaunchKernelGGL(k_gather<kPassesLong>, dim3(grid), dim3(kRaBlock), 0, s, p);
    else
      hipLaunchKernelGGL(k_gather<kPassesShort>, dim3(grid), dim3(kRaBlock), 0, s, p);
  } else {
    // a few workgroups per CU, each carrying many passes
    const long ups = (long)(p.D + 1) * p.units;
    const long spp = ups < kRaBlock ? kRaBlock / ups : 1;
    const long passes = ((long)p.layers * 2 * p.B * p.heads + spp - 1) / spp;
    const long g = passes < SPECDEC_AP_WGS_PER_CU * (long)cus ? passes : SPECDEC_AP_WGS_PER_CU * (long)cus;
    AppendKvDivs dv;
    dv.bh = host_fast_div((uint32_t)(p.B * p.heads));
    dv.h = host_fast_div((uint32_t)p.heads);
    hipLaunchKernelGGL(k_append_kv, dim3((unsigned)(g > 0 ? g : 1)), dim3(kRaBlock), 0, s, p, dv);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_append_meta, dim3(1), dim3(kRaBlock), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace sd
