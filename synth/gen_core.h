/* Counter-based synthetic input generator: the single definition of every
 * seeded value used by the workloads, compiled for the host (gcc) and for the
 * device (hipcc).  It produces inputs only: it never computes an argmax, an
 * acceptance decision, a residual draw or a realignment.
 *
 * Randomness: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014).  Output n of a stream keyed by k is the
 * SplitMix64 finaliser applied to k + (n+1)*0x9E3779B97F4A7C15, so any element
 * of any tensor is computable on its own from (seed, stream, round, index).
 *
 * Value shapes:
 *   uniform24  = top 24 bits * 2^-24, in [0,1), exact in fp32
 *   normal     = Irwin-Hall of twelve 16-bit uniforms, centred and scaled:
 *                z = (sum - 393210) / 65536, exact in fp32, |z| < 6, var ~= 1
 *   bf16/fp16  = round-to-nearest-even of the fp32 value, done with integer
 *                operations so host and device agree bit for bit.
 */
#ifndef SYNTH_GEN_CORE_H
#define SYNTH_GEN_CORE_H

#include <stdint.h>

#ifdef __HIPCC__
#define SYN_FN __host__ __device__ static inline
#else
#define SYN_FN static inline
#endif

#define SYN_GAMMA 0x9E3779B97F4A7C15ULL

SYN_FN uint64_t syn_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* Stream key for (seed, stream id, round). */
SYN_FN uint64_t syn_key(uint64_t seed, uint32_t stream, uint32_t round) {
  uint64_t k = syn_mix(seed * SYN_GAMMA + 0x2545F4914F6CDD1DULL);
  k = syn_mix(k ^ ((uint64_t)stream * 0xD1B54A32D192ED03ULL));
  k = syn_mix(k ^ ((uint64_t)round * 0xABC98388FB8FAC03ULL));
  return k;
}

/* n-th SplitMix64 output of the stream keyed by k. */
SYN_FN uint64_t syn_u64(uint64_t k, uint64_t n) { return syn_mix(k + (n + 1) * SYN_GAMMA); }

SYN_FN float syn_uniform24(uint64_t k, uint64_t n) {
  return (float)(uint32_t)(syn_u64(k, n) >> 40) * (1.0f / 16777216.0f);
}

/* Irwin-Hall(12) normal: three 64-bit draws give twelve 16-bit uniforms. */
SYN_FN float syn_normal(uint64_t k, uint64_t n) {
  int32_t s = 0;
  for (int w = 0; w < 3; ++w) {
    uint64_t r = syn_u64(k, 3 * n + (uint64_t)w);
    s += (int32_t)(r & 0xFFFF) + (int32_t)((r >> 16) & 0xFFFF) + (int32_t)((r >> 32) & 0xFFFF) +
         (int32_t)(r >> 48);
  }
  return (float)(s - 393210) * (1.0f / 65536.0f);
}

SYN_FN uint32_t syn_f32_bits(float f) {
  union { float f; uint32_t u; } c;
  c.f = f;
  return c.u;
}

/* fp32 -> bf16, round to nearest even (finite inputs). */
SYN_FN uint16_t syn_to_bf16(float f) {
  uint32_t x = syn_f32_bits(f);
  x += 0x7FFFu + ((x >> 16) & 1u);
  return (uint16_t)(x >> 16);
}

/* fp32 -> IEEE binary16, round to nearest even, subnormals included. */
SYN_FN uint16_t syn_to_f16(float f) {
  uint32_t x = syn_f32_bits(f);
  uint32_t sign = (x >> 16) & 0x8000u;
  uint32_t ax = x & 0x7FFFFFFFu;
  if (ax >= 0x47800000u) return (uint16_t)(sign | 0x7C00u | (ax > 0x7F800000u ? 0x200u : 0u));
  if (ax < 0x38800000u) {               /* below 2^-14: binary16 subnormal or zero */
    uint32_t e = ax >> 23;
    if (e < 102u) return (uint16_t)sign; /* below 2^-25 */
    uint32_t m = (ax & 0x7FFFFFu) | 0x800000u;
    uint32_t shift = 126u - e;           /* 14..24 */
    uint32_t q = m >> shift, rem = m & ((1u << shift) - 1u), half = 1u << (shift - 1u);
    if (rem > half || (rem == half && (q & 1u))) ++q;
    return (uint16_t)(sign | q);
  }
  uint32_t r = ax - 0x38000000u;         /* rebias exponent 127 -> 15 */
  r += 0xFFFu + ((r >> 13) & 1u);
  return (uint16_t)(sign | (r >> 13));
}

/* Stream ids shared by every recipe. */
enum {
  SYN_S_LEN = 1,     /* content lengths */
  SYN_S_KV0 = 2,     /* initial KV content */
  SYN_S_TOK0 = 3,    /* initial token ids */
  SYN_S_LOGIT = 4,   /* target logits of a round */
  SYN_S_PLANT = 5,   /* planted argmax positions, ties, drafts */
  SYN_S_KVNEW = 6,   /* KV of the D+1 verified positions of a round */
  SYN_S_UNIF = 7,    /* acceptance / draw uniforms */
  SYN_S_NOISE = 8    /* draft-logit noise */
};

enum { SYN_F32 = 0, SYN_F16 = 1, SYN_BF16 = 2 };

/* Encode a normal draw scaled by sigma into the element type; writes esize bytes. */
SYN_FN void syn_store(int dtype, void *dst, uint64_t i, float v) {
  if (dtype == SYN_F32) ((float *)dst)[i] = v;
  else if (dtype == SYN_F16) ((uint16_t *)dst)[i] = syn_to_f16(v);
  else ((uint16_t *)dst)[i] = syn_to_bf16(v);
}

#endif
