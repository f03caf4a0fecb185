/* Host side of the seeded input generator (gcc, OpenMP).  Every function
 * fills caller-owned host memory; values are defined in gen_core.h and are
 * bit-identical to the device fills in gen_device.hip.  Nothing here computes
 * an argmax, an acceptance decision or a realignment: the greedy plan states
 * by construction which id is each row's maximum (it writes a value above the
 * support of the normal draws there) and which draft position first differs. */
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#include "gen_core.h"

#define EXPORT __attribute__((visibility("default")))

static size_t esize_of(int dtype) { return dtype == SYN_F32 ? 4 : 2; }

/* out[i] = sigma * normal(stream key, start + i), encoded as dtype. */
EXPORT void synth_fill_normal(int dtype, uint64_t seed, uint32_t stream, uint32_t round,
                              uint64_t start, uint64_t count, float sigma, void *out) {
  const uint64_t k = syn_key(seed, stream, round);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)count; ++i)
    syn_store(dtype, out, (uint64_t)i, sigma * syn_normal(k, start + (uint64_t)i));
}

EXPORT void synth_fill_uniform(uint64_t seed, uint32_t stream, uint32_t round, uint64_t start,
                               uint64_t count, float *out) {
  const uint64_t k = syn_key(seed, stream, round);
  for (uint64_t i = 0; i < count; ++i) out[i] = syn_uniform24(k, start + i);
}

/* out[i] = lo + (draw mod (hi - lo + 1)), inclusive range. */
EXPORT void synth_fill_int(uint64_t seed, uint32_t stream, uint32_t round, uint64_t start,
                           uint64_t count, int64_t lo, int64_t hi, int32_t *out) {
  const uint64_t k = syn_key(seed, stream, round);
  const uint64_t span = (uint64_t)(hi - lo + 1);
  for (uint64_t i = 0; i < count; ++i) out[i] = (int32_t)(lo + (int64_t)(syn_u64(k, start + i) % span));
}

/* Pool lengths: nvals distinct values in [lo, hi], each given to n/nvals
 * sequences; the value-to-sequence assignment is a seeded Fisher-Yates shuffle. */
EXPORT int synth_pool_lengths(uint64_t seed, int n, int nvals, int lo, int hi, int32_t *out) {
  if (nvals <= 0 || n % nvals != 0 || hi - lo + 1 < nvals) return -1;
  const uint64_t k = syn_key(seed, SYN_S_LEN, 0);
  int32_t vals[4096];
  if (nvals > 4096) return -1;
  uint64_t draw = 0;
  for (int v = 0; v < nvals;) {
    int32_t c = lo + (int32_t)(syn_u64(k, draw++) % (uint64_t)(hi - lo + 1));
    int dup = 0;
    for (int w = 0; w < v; ++w) dup |= (vals[w] == c);
    if (!dup) vals[v++] = c;
  }
  const int per = n / nvals;
  for (int i = 0; i < n; ++i) out[i] = vals[i / per];
  const uint64_t ks = syn_key(seed, SYN_S_LEN, 1);
  for (int i = n - 1; i > 0; --i) {
    int j = (int)(syn_u64(ks, (uint64_t)i) % (uint64_t)(i + 1));
    int32_t t = out[i]; out[i] = out[j]; out[j] = t;
  }
  return 0;
}

/* Greedy round plan for B rows, D drafts, D+1 verified positions per row.
 *   plant[(b*(D+1)+i)*3 + s]: ids that receive the planted maximum in logit row
 *     (b,i); slot 0 is the lowest and is the row's designed argmax, slots 1-2
 *     (or -1) are extra copies at higher ids that create exact ties.
 *   mode 0: each draft position matches its row's designed argmax with
 *     probability p independently (otherwise a different id);
 *   mode 1: the number k of leading matching drafts is geometric, P(k) =
 *     p (1-p)^k capped at D; position k (if < D) holds a different id and
 *     positions after it hold uniform ids.
 *   first_miss[b]: the designed position of the first non-matching draft (D if
 *     none), i.e. the accepted length the plan was built to produce.
 *   draft[b*D + i]: the draft ids. */
EXPORT void synth_plan_greedy(uint64_t seed, uint32_t round, int B, int D, int V, int mode, double p,
                              double tie_frac, int32_t *plant, int32_t *first_miss, int32_t *draft) {
  const uint64_t k = syn_key(seed, SYN_S_PLANT, round);
  const int D1 = D + 1;
  for (int r = 0; r < B * D1; ++r) {
    const uint64_t base = (uint64_t)r * 8;
    int32_t t = (int32_t)(syn_u64(k, base) % (uint64_t)V);
    plant[r * 3 + 0] = t;
    plant[r * 3 + 1] = -1;
    plant[r * 3 + 2] = -1;
    const uint64_t h = syn_u64(k, base + 1);
    const float u = (float)(uint32_t)(h >> 40) * (1.0f / 16777216.0f);
    if ((double)u < tie_frac && t < V - 1) {
      int extra = 1 + (int)(h & 1);
      for (int c = 0; c < extra; ++c)
        plant[r * 3 + 1 + c] = t + 1 + (int32_t)(syn_u64(k, base + 2 + (uint64_t)c) % (uint64_t)(V - 1 - t));
    }
  }
  const uint64_t kd = syn_key(seed, SYN_S_PLANT, round + 0x10000u);
  for (int b = 0; b < B; ++b) {
    const uint64_t base = (uint64_t)b * 64;
    int match[256];
    int kk = D;
    if (mode == 1) {
      kk = 0;
      while (kk < D && (double)syn_uniform24(kd, base + (uint64_t)kk) >= p) ++kk;
      for (int i = 0; i < D; ++i) match[i] = (i < kk) ? 1 : (i == kk ? 0 : 2);
    } else {
      for (int i = 0; i < D; ++i) match[i] = (double)syn_uniform24(kd, base + (uint64_t)i) < p;
      for (int i = 0; i < D; ++i)
        if (!match[i]) { kk = i; break; }
    }
    first_miss[b] = kk;
    for (int i = 0; i < D; ++i) {
      const int32_t t = plant[(b * D1 + i) * 3];
      const uint64_t h = syn_u64(kd, base + 32 + (uint64_t)i);
      if (match[i] == 1) draft[b * D + i] = t;
      else if (match[i] == 0) draft[b * D + i] = (V > 1) ? (int32_t)((t + 1 + (int64_t)(h % (uint64_t)(V - 1))) % V) : t;
      else draft[b * D + i] = (int32_t)(h % (uint64_t)V);
    }
  }
}

/* Logit rows [row0, row0+nrows) of a round: sigma * normal at logical index
 * row*V + v, then the planted maximum written at the plan's ids.  Row r of the
 * output starts at out + (r-row0)*row_stride elements. */
EXPORT void synth_fill_logits(int dtype, uint64_t seed, uint32_t round, int64_t row0, int64_t nrows,
                              int64_t V, int64_t row_stride, float sigma, const int32_t *plant,
                              float plant_value, void *out) {
  const uint64_t k = syn_key(seed, SYN_S_LOGIT, round);
  const size_t es = esize_of(dtype);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < nrows; ++r) {
    char *row = (char *)out + (size_t)(r * row_stride) * es;
    const uint64_t base = (uint64_t)((row0 + r) * V);
    for (int64_t v = 0; v < V; ++v) syn_store(dtype, row, (uint64_t)v, sigma * syn_normal(k, base + (uint64_t)v));
    if (plant)
      for (int s = 0; s < 3; ++s) {
        int32_t id = plant[(row0 + r) * 3 + s];
        if (id >= 0) syn_store(dtype, row, (uint64_t)id, plant_value);
      }
  }
}

/* KV content of a sequence buffer [L][2][rows][H][cap][Dh]; this call fills the
 * layer range [layer0, layer0+nlayers) into out (which starts at layer0).
 * Content element (l, kv, b, h, j, d), j < len[b], is normal at index
 * ((((l*2+kv)*rows + b)*H + h)*cap + j)*Dh + d of stream SYN_S_KV0.
 * left_pad != 0: content sits at positions [width-len[b], width) (a left-padded
 * rectangle); otherwise at [0, len[b]) (a pool row).  Every other position is 0. */
EXPORT void synth_fill_kv(int dtype, uint64_t seed, int L, int rows, int H, int cap, int Dh,
                          const int32_t *len, int width, int left_pad, int layer0, int nlayers,
                          void *out) {
  (void)L;
  const uint64_t k = syn_key(seed, SYN_S_KV0, 0);
  const size_t es = esize_of(dtype);
  const int64_t nseg = (int64_t)nlayers * 2 * rows * H;
#pragma omp parallel for schedule(static)
  for (int64_t s = 0; s < nseg; ++s) {
    const int64_t gseg = (int64_t)layer0 * 2 * rows * H + s;
    const int b = (int)((gseg / H) % rows);
    const int off = left_pad ? width - len[b] : 0;
    char *seg = (char *)out + (size_t)s * cap * Dh * es;
    memset(seg, 0, (size_t)cap * Dh * es);
    for (int j = 0; j < len[b]; ++j)
      for (int d = 0; d < Dh; ++d)
        syn_store(dtype, seg, (uint64_t)(off + j) * Dh + d,
                  syn_normal(k, ((uint64_t)gseg * cap + (uint64_t)j) * Dh + (uint64_t)d));
  }
}

/* Initial token ids of the same buffer: uniform ids in [0,V) at content
 * positions, pad_token elsewhere.  pos/mask (nullable) describe the same
 * layout: mask 1 on content, position ids 0..len-1 over content, 0 on pad. */
EXPORT void synth_fill_tokens(uint64_t seed, int rows, int cap, int V, const int32_t *len, int width,
                              int left_pad, int32_t pad_token, int32_t *tokens, int32_t *pos,
                              int8_t *mask) {
  const uint64_t k = syn_key(seed, SYN_S_TOK0, 0);
  for (int b = 0; b < rows; ++b) {
    const int off = left_pad ? width - len[b] : 0;
    for (int j = 0; j < cap; ++j) {
      const int c = j - off;
      const int in = (c >= 0 && c < len[b]);
      tokens[(size_t)b * cap + j] = in ? (int32_t)(syn_u64(k, (uint64_t)b * cap + (uint64_t)c) % (uint64_t)V) : pad_token;
      if (pos) pos[(size_t)b * cap + j] = in ? c : 0;
      if (mask) mask[(size_t)b * cap + j] = (int8_t)in;
    }
  }
}
