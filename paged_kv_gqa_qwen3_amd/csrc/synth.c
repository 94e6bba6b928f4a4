/*
 * Seeded synthetic inputs for the decode step: weights, norm gains and
 * paged K/V contents, produced as bf16 bit patterns (uint16).
 *
 * This file is an input generator only.  It holds none of the decode step's
 * arithmetic; both the CPU oracle's tests and the GPU path read the bytes it
 * writes, so they see identical inputs.
 *
 * Generator (counter based, so any element can be produced independently and
 * the work splits over threads without changing the result):
 *   key      = mix64(seed ^ fnv1a64(tensor name))
 *   word(i)  = mix64(key + (i + 1) * 0x9E3779B97F4A7C15)
 *   mix64    = the SplitMix64 output finaliser (Steele, Lea, Flood,
 *              "Fast splittable pseudorandom number generators", OOPSLA 2014)
 * Normal deviates use the Box-Muller transform on the pair of words
 * (2j, 2j+1): u1 = (word >> 11 + 1) * 2^-53 in (0, 1], u2 = (word >> 11) * 2^-53;
 * element 2j gets r*cos(2*pi*u2), element 2j+1 gets r*sin(2*pi*u2),
 * r = sqrt(-2 ln u1).  value = mean + std * z, rounded to nearest-even bf16.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t word_at(uint64_t key, uint64_t i) {
  return mix64(key + (i + 1ULL) * 0x9E3779B97F4A7C15ULL);
}

uint64_t synth_key(uint64_t seed, const char* name) {
  uint64_t h = 0xCBF29CE484222325ULL; /* FNV-1a 64 */
  for (const unsigned char* p = (const unsigned char*)name; *p; ++p) {
    h ^= *p;
    h *= 0x100000001B3ULL;
  }
  return mix64(seed ^ h);
}

/* float -> bf16 bits, round to nearest, ties to even (inputs here are finite). */
static inline uint16_t f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

/* n bf16 values ~ N(mean, std^2).  The double result is first rounded to
 * fp32, then to bf16; the distribution, not the rounding path, is what the
 * workloads specify. */
void synth_normal_bf16(uint64_t key, double mean, double stdv, uint16_t* out,
                       int64_t n) {
  const double two_pi = 6.283185307179586476925286766559;
  int64_t npairs = (n + 1) / 2;
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < npairs; ++j) {
    uint64_t a = word_at(key, (uint64_t)(2 * j));
    uint64_t b = word_at(key, (uint64_t)(2 * j + 1));
    double u1 = ((double)(a >> 11) + 1.0) * 0x1.0p-53;
    double u2 = (double)(b >> 11) * 0x1.0p-53;
    double r = sqrt(-2.0 * log(u1));
    double z0 = r * cos(two_pi * u2);
    double z1 = r * sin(two_pi * u2);
    out[2 * j] = f32_to_bf16((float)(mean + stdv * z0));
    if (2 * j + 1 < n) out[2 * j + 1] = f32_to_bf16((float)(mean + stdv * z1));
  }
}

/* n integers uniform on [0, hi) (hi < 2^31), by the multiply-shift map. */
void synth_uniform_int(uint64_t key, int32_t hi, int32_t* out, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    uint64_t w = word_at(key, (uint64_t)i);
    out[i] = (int32_t)(((__uint128_t)w * (uint64_t)hi) >> 64); /* floor(w * hi / 2^64) */
  }
}

/* Fill the K/V contents of a paged pool for a set of logical token slots.
 * pool layout: [L][P][2][Hkv][page][D] bf16.  For sequence s, logical token t
 * (0 <= t < ctx[s]) lives in page table[s*maxp + t/page], slot t%page.  The
 * value of (layer, kv, head, seq, t, d) is the normal deviate with counter
 * ((((layer*2 + kv)*Hkv + head)*nseq + s)*tmax + t)*D + d, so the content of a
 * logical token does not depend on which physical page holds it. */
void synth_fill_pool(uint64_t key, double stdv, uint16_t* pool, int L, int P,
                     int Hkv, int page, int D, int nseq, const int32_t* ctx,
                     const int32_t* table, int maxp, int tmax) {
  const double two_pi = 6.283185307179586476925286766559;
  int64_t rows = (int64_t)L * 2 * Hkv * nseq * tmax;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    int64_t rr = r;
    int t = (int)(rr % tmax); rr /= tmax;
    int s = (int)(rr % nseq); rr /= nseq;
    int hd = (int)(rr % Hkv); rr /= Hkv;
    int kv = (int)(rr % 2); rr /= 2;
    int l = (int)rr;
    if (t >= ctx[s]) continue;
    int pg = table[(int64_t)s * maxp + t / page];
    uint16_t* dst = pool + ((((((int64_t)l * P + pg) * 2 + kv) * Hkv + hd) * page +
                             (t % page)) * D);
    int64_t base = r * D;
    for (int d = 0; d < D; d += 2) {
      uint64_t a = word_at(key, (uint64_t)(base + d));
      uint64_t b = word_at(key, (uint64_t)(base + d + 1));
      double u1 = ((double)(a >> 11) + 1.0) * 0x1.0p-53;
      double u2 = (double)(b >> 11) * 0x1.0p-53;
      double rad = sqrt(-2.0 * log(u1));
      dst[d] = f32_to_bf16((float)(stdv * rad * cos(two_pi * u2)));
      if (d + 1 < D) dst[d + 1] = f32_to_bf16((float)(stdv * rad * sin(two_pi * u2)));
    }
  }
}

/* The same slots of an 8-bit pool (OCP E4M3 codes) filled with random codes
 * drawn directly as bit fields: a random sign, an exponent field in 3..8 and
 * a random 3-bit mantissa, i.e. magnitudes 2^-4 .. 3.75 and never a NaN
 * code.  (No rounding: the codes themselves are the random draw.) */
void synth_fill_pool_fp8(uint64_t key, uint8_t* pool, int L, int P, int Hkv, int page, int D,
                         int nseq, const int32_t* ctx, const int32_t* table, int maxp,
                         int tmax) {
  int64_t rows = (int64_t)L * 2 * Hkv * nseq * tmax;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    int64_t rr = r;
    int t = (int)(rr % tmax); rr /= tmax;
    int s = (int)(rr % nseq); rr /= nseq;
    int hd = (int)(rr % Hkv); rr /= Hkv;
    int kv = (int)(rr % 2); rr /= 2;
    int l = (int)rr;
    if (t >= ctx[s]) continue;
    int pg = table[(int64_t)s * maxp + t / page];
    uint8_t* dst = pool + ((((((int64_t)l * P + pg) * 2 + kv) * Hkv + hd) * page +
                            (t % page)) * D);
    int64_t base = r * D;
    for (int d = 0; d < D; ++d) {
      uint64_t w = word_at(key, (uint64_t)(base + d));
      unsigned sign = (unsigned)(w >> 63) << 7;
      unsigned e = 3 + (unsigned)((w >> 8) % 6);
      unsigned m = (unsigned)(w >> 32) & 7;
      dst[d] = (uint8_t)(sign | (e << 3) | m);
    }
  }
}

/* Fill n bytes with a constant (the NaN poison page of an 8-bit pool). */
void synth_fill_u8(uint8_t* out, uint8_t v, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = v;
}

/* Fill n bf16 slots with a constant bit pattern (used for the NaN poison page). */
void synth_fill_u16(uint16_t* out, uint16_t v, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = v;
}
