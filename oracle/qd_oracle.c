/*
 * CPU oracle for one batched decode step of a Qwen3-style GQA decoder.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this code.  The GPU library shares
 * no code with it and never calls it.
 *
 * Plain, slow, obviously correct: every quantity is held and accumulated in
 * fp64.  The only roundings are the ones the method fixes: weights and the KV
 * pool are bf16 ("qwen3-runtime" blog, Part 1: BF16 model; Part 4: bf16 paged
 * pool), so appended K/V are rounded to nearest-even bf16 before they enter
 * the pool and attention reads them back from the pool.
 *
 * Steps and the passages they follow (pages named by title, sections as on
 * the page):
 *   embedding lookup              "推理引擎里面发生了什么", Prefill, step 1
 *   pre-norm layer x += Attn(RMSNorm(x)); x += MLP(RMSNorm(x))
 *                                 rkmt "从零构建 Qwen3-8B", section 4.2.2
 *   RMSNorm x*rsqrt(mean(x^2)+eps)*w, eps 1e-6
 *                                 blog Part 6, native RMSNorm listing
 *   q/k RMSNorm after projection, then NeoX RoPE (rotate_half = cat(-x2, x1),
 *   non-interleaved)              blog Part 6, bullet list and item 2
 *   GQA: query head g*G+h reads KV head g, scores scaled by 1/sqrt(d_head)
 *                                 rkmt page, section 4.4.2
 *   paged KV: 16-token pages found through a per-sequence block table
 *                                 "推理引擎里面发生了什么", KV Cache /
 *                                 PagedAttention; blog Part 4
 *   SwiGLU silu(gate)*up          blog Part 6, bullet list
 *   greedy next token = argmax of the logits on the last position
 *                                 blog Part 3 item 1, Part 7
 *   FP8 KV pool (optional): K and V quantised to 8-bit floating point
 *                                 "推理引擎里面发生了什么", Tensor Core：精度即吞吐
 *                                 and Quantization 对 Kernel 的影响
 * Readings where the pages are silent: a final RMSNorm before the LM head;
 * no projection biases; q/k norm gains of length head_dim shared by all
 * heads, eps 1e-6; RoPE inverse frequency theta^(-2i/D) for pair (i, i+D/2);
 * the current token attends to itself (context = position + 1); argmax ties
 * go to the lowest index.  The FP8 pool's format is not named: it is read as
 * OCP E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no
 * infinities, NaN = S.1111.111, largest finite 448), one scale for all of K
 * and one for all of V (stored code = E4M3(value / scale), round to nearest
 * even, saturating at +-448; read value = code * scale).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_PAGE 16

double or_bf16_to_f64(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Round a double to the nearest bf16 value, ties to even, in one step (no
 * intermediate rounding to fp32).  bf16 has 8 significant bits and the fp32
 * exponent range, so the spacing of bf16 values near |v| = m*2^e (m in
 * [0.5,1)) is 2^(e-8), and 2^-133 in the subnormal range.  Dividing by that
 * power of two is exact; nearbyint rounds half to even in the default mode. */
uint16_t or_f64_to_bf16(double v) {
  if (isnan(v)) return 0x7FC0;
  if (v == 0.0) return signbit(v) ? 0x8000 : 0x0000;
  if (isinf(v)) return signbit(v) ? 0xFF80 : 0x7F80;
  int e;
  frexp(fabs(v), &e);
  int qexp = e - 8;
  if (qexp < -133) qexp = -133;
  double r = nearbyint(ldexp(v, -qexp));
  double q = ldexp(r, qexp);
  const double max_bf16 = ldexp(255.0, 120); /* 0x7F7F = (2 - 2^-7) * 2^127 */
  if (fabs(q) > max_bf16) return signbit(v) ? 0xFF80 : 0x7F80;
  float f = (float)q; /* exact: q is a bf16 value */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

/* OCP E4M3 code -> exact value.  Exponent field e (bias 7), mantissa m:
 * e = 0 is subnormal, m * 2^-9; e = 15 with m = 7 is NaN; otherwise
 * (1 + m/8) * 2^(e-7). */
double or_e4m3_to_f64(uint8_t c) {
  const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

/* Nearest E4M3 code of v, ties to even, in one rounding step; magnitudes
 * beyond the largest finite value (448) saturate to it; NaN gives 0x7F.
 * Near |v| = f*2^x (f in [0.5,1)) the spacing of E4M3 values is 2^(x-4) for
 * normal results and 2^-9 below 2^-6 (subnormals), so v divided by that
 * spacing is rounded to an integer with nearbyint (half to even in the
 * default mode) and multiplied back, exactly. */
uint8_t or_f64_to_e4m3(double v) {
  if (isnan(v)) return 0x7F;
  const uint8_t sign = signbit(v) ? 0x80 : 0x00;
  double a = fabs(v);
  if (a == 0.0) return sign;
  if (a >= 448.0) return sign | 0x7E;
  int x;
  frexp(a, &x);
  int qexp = x - 4;
  if (qexp < -9) qexp = -9;
  double q = ldexp(nearbyint(ldexp(a, -qexp)), qexp);
  if (q > 448.0) q = 448.0; /* (cannot happen below 464; kept for clarity) */
  /* q is now an E4M3 value: find its code */
  if (q < ldexp(1.0, -6)) return sign | (uint8_t)(q * 512.0);  /* subnormal, or 2^-6 as m = 8 */
  int e2;
  double f = frexp(q, &e2);  /* q = f * 2^e2, f in [0.5, 1) */
  const int e = e2 - 1 + 7;
  const int m = (int)((2.0 * f - 1.0) * 8.0);
  return sign | (uint8_t)((e << 3) | m);
}

/* y = x / sqrt(mean(x^2) + eps) * g */
void or_rmsnorm(const double* x, int n, const uint16_t* g, double eps, double* y) {
  double ss = 0.0;
  for (int i = 0; i < n; ++i) ss += x[i] * x[i];
  double inv = 1.0 / sqrt(ss / n + eps);
  for (int i = 0; i < n; ++i) y[i] = x[i] * inv * or_bf16_to_f64(g[i]);
}

/* y[b][n] = sum_k W[n][k] * x[b][k];  W is [N][K] row-major bf16 ([out, in]). */
void or_linear(const double* x, int B, int K, const uint16_t* W, int N, double* y) {
#pragma omp parallel for schedule(static)
  for (int n = 0; n < N; ++n) {
    const uint16_t* w = W + (int64_t)n * K;
    for (int b = 0; b < B; ++b) {
      const double* xb = x + (int64_t)b * K;
      double acc = 0.0;
      for (int k = 0; k < K; ++k) acc += or_bf16_to_f64(w[k]) * xb[k];
      y[(int64_t)b * N + n] = acc;
    }
  }
}

/* NeoX rotary embedding at position pos, in place on one head vector of
 * length D: for i < D/2, angle a = pos * theta^(-2i/D) and
 * (x_i, x_{i+D/2}) <- (x_i cos a - x_{i+D/2} sin a, x_{i+D/2} cos a + x_i sin a),
 * i.e. x*cos + rotate_half(x)*sin with rotate_half(x) = cat(-x2, x1). */
void or_rope_neox(double* v, int D, int pos, double theta) {
  int half = D / 2;
  for (int i = 0; i < half; ++i) {
    double inv_freq = pow(theta, -2.0 * i / D);
    double a = (double)pos * inv_freq;
    double c = cos(a), s = sin(a);
    double x1 = v[i], x2 = v[i + half];
    v[i] = x1 * c - x2 * s;
    v[i + half] = x2 * c + x1 * s;
  }
}

/* Element type of the pool: NULL or fp8 = 0 is bf16; fp8 = 1 is OCP E4M3
 * with one scale for K and one for V. */
typedef struct or_kv {
  int fp8;
  double k_scale, v_scale;
} or_kv;

/* Element index of the first of the D values of (layer, page, K|V, head, slot). */
static inline int64_t pool_index(int num_pages, int Hkv, int D, int layer, int page, int kv,
                                 int head, int slot) {
  return ((((int64_t)layer * num_pages + page) * 2 + kv) * Hkv + head) * OR_PAGE * D +
         (int64_t)slot * D;
}

/* The value the pool holds at element i (which = 0 for K, 1 for V). */
static inline double pool_get(const void* pool, const or_kv* kv, int64_t i, int which) {
  if (!kv || !kv->fp8) return or_bf16_to_f64(((const uint16_t*)pool)[i]);
  return or_e4m3_to_f64(((const uint8_t*)pool)[i]) * (which ? kv->v_scale : kv->k_scale);
}

/* Store v at element i, rounded to the pool's type. */
static inline void pool_put(void* pool, const or_kv* kv, int64_t i, int which, double v) {
  if (!kv || !kv->fp8)
    ((uint16_t*)pool)[i] = or_f64_to_bf16(v);
  else
    ((uint8_t*)pool)[i] = or_f64_to_e4m3(v / (which ? kv->v_scale : kv->k_scale));
}

/* Paged GQA decode attention for one sequence.
 * q: [Hq][D]; the sequence's tokens 0..ctx-1 are read from the pool through
 * its block-table row (token t: page table_row[t/16], slot t%16).  Query head
 * h uses KV head h / (Hq/Hkv).  o: [Hq][D].  kv: the pool's element type
 * (NULL: bf16). */
void or_attention(const double* q, int Hq, int Hkv, int D, const void* pool,
                  int num_pages, int layer, const int32_t* table_row, int ctx,
                  double* o, const or_kv* kv) {
  int G = Hq / Hkv;
  double scale = 1.0 / sqrt((double)D);
#pragma omp parallel for schedule(static)
  for (int h = 0; h < Hq; ++h) {
    int g = h / G;
    double* s = (double*)malloc(sizeof(double) * (ctx > 0 ? ctx : 1));
    const double* qh = q + (int64_t)h * D;
    double mx = -INFINITY;
    for (int t = 0; t < ctx; ++t) {
      const int64_t kr = pool_index(num_pages, Hkv, D, layer, table_row[t / OR_PAGE], 0, g,
                                    t % OR_PAGE);
      double acc = 0.0;
      for (int d = 0; d < D; ++d) acc += qh[d] * pool_get(pool, kv, kr + d, 0);
      s[t] = acc * scale;
      if (s[t] > mx) mx = s[t];
    }
    double den = 0.0;
    for (int t = 0; t < ctx; ++t) {
      s[t] = exp(s[t] - mx);
      den += s[t];
    }
    double* oh = o + (int64_t)h * D;
    for (int d = 0; d < D; ++d) oh[d] = 0.0;
    for (int t = 0; t < ctx; ++t) {
      const int64_t vr = pool_index(num_pages, Hkv, D, layer, table_row[t / OR_PAGE], 1, g,
                                    t % OR_PAGE);
      double w = s[t] / den;
      for (int d = 0; d < D; ++d) oh[d] += w * pool_get(pool, kv, vr + d, 1);
    }
    free(s);
  }
}

double or_silu(double z) { return z / (1.0 + exp(-z)); }

/* Element-wise forms of or_f64_to_bf16 and or_silu over arrays (the same
 * scalar functions applied in a loop, so that callers need not cross into
 * C once per element). */
void or_f64_to_bf16_n(const double* x, int64_t n, uint16_t* y) {
  for (int64_t i = 0; i < n; ++i) y[i] = or_f64_to_bf16(x[i]);
}

void or_f64_to_e4m3_n(const double* x, int64_t n, uint8_t* y) {
  for (int64_t i = 0; i < n; ++i) y[i] = or_f64_to_e4m3(x[i]);
}

void or_e4m3_to_f64_n(const uint8_t* c, int64_t n, double* y) {
  for (int64_t i = 0; i < n; ++i) y[i] = or_e4m3_to_f64(c[i]);
}

void or_silu_n(const double* z, int64_t n, double* y) {
  for (int64_t i = 0; i < n; ++i) y[i] = or_silu(z[i]);
}

/* Index of the largest value, lowest index among equals; -1 if any NaN. */
int or_argmax(const double* v, int n) {
  int best = -1;
  for (int i = 0; i < n; ++i) {
    if (isnan(v[i])) return -1;
    if (best < 0 || v[i] > v[best]) best = i;
  }
  return best;
}

typedef struct or_config {
  int num_layers, hidden, num_q_heads, num_kv_heads, head_dim, intermediate, vocab;
  int tie_embeddings;
  double rms_eps, rope_theta;
} or_config;

/* Per-layer weight pointers (bf16, HF [out, in] layout). */
typedef struct or_layer {
  const uint16_t *in_norm, *wq, *wk, *wv, *wo, *q_norm, *k_norm, *post_norm, *wgate,
      *wup, *wdown;
} or_layer;

typedef struct or_weights {
  const uint16_t* embed;      /* [V][H] */
  const uint16_t* final_norm; /* [H] */
  const uint16_t* lm_head;    /* [V][H]; NULL when tied to embed */
  const or_layer* layers;     /* [L] */
} or_weights;

/* Intermediate values of one chosen layer (any pointer may be NULL). */
typedef struct or_taps {
  int layer;
  double* x_in;   /* [B][H] residual entering the layer */
  double* qkv;    /* [B][(Hq+2Hkv)D] projections q | k | v */
  double* q_rot;  /* [B][Hq][D] after q-norm and RoPE */
  double* k_rot;  /* [B][Hkv][D] after k-norm and RoPE, before rounding to the pool type */
  double* attn;   /* [B][Hq][D] attention output */
  double* x_mid;  /* [B][H] residual after the attention block */
  double* act;    /* [B][I] silu(gate) * up */
  double* x_out;  /* [B][H] residual after the MLP block */
  double* final_h;/* [B][H] final normalised hidden state */
} or_taps;

/* One decode step for B sequences.  Sequence b decodes token tokens[b] at
 * position positions[b]; its K/V for that position are appended to the pool
 * and attention spans positions 0..positions[b].  logits: [B][V] (may be
 * NULL), next: [B].  kv: the pool's element type (NULL: bf16).  Returns 0,
 * or -1 on bad arguments. */
int or_decode_step(const or_config* c, const or_weights* w, int B, const int32_t* tokens,
                   const int32_t* positions, const int32_t* block_tables, int max_pages,
                   void* pool, int num_pages, double* logits, int32_t* next,
                   const or_taps* taps, const or_kv* kv) {
  const int L = c->num_layers, H = c->hidden, Hq = c->num_q_heads, Hkv = c->num_kv_heads;
  const int D = c->head_dim, I = c->intermediate, V = c->vocab;
  if (B <= 0 || Hq % Hkv != 0 || D % 2 != 0) return -1;
  for (int b = 0; b < B; ++b) {
    if (tokens[b] < 0 || tokens[b] >= V) return -1;
    if (positions[b] < 0 || positions[b] / OR_PAGE >= max_pages) return -1;
  }
  const int QD = Hq * D, KD = Hkv * D;
  double* x = calloc((size_t)B * H, sizeof(double));
  double* h = calloc((size_t)B * H, sizeof(double));
  double* q = calloc((size_t)B * QD, sizeof(double));
  double* k = calloc((size_t)B * KD, sizeof(double));
  double* v = calloc((size_t)B * KD, sizeof(double));
  double* att = calloc((size_t)B * QD, sizeof(double));
  double* tmp = calloc((size_t)B * H, sizeof(double));
  double* gt = calloc((size_t)B * I, sizeof(double));
  double* up = calloc((size_t)B * I, sizeof(double));
  double* headbuf = calloc((size_t)D, sizeof(double));

  for (int b = 0; b < B; ++b)
    for (int i = 0; i < H; ++i)
      x[(int64_t)b * H + i] = or_bf16_to_f64(w->embed[(int64_t)tokens[b] * H + i]);

  for (int l = 0; l < L; ++l) {
    const or_layer* ly = &w->layers[l];
    int tap = taps && taps->layer == l;
    if (tap && taps->x_in) memcpy(taps->x_in, x, sizeof(double) * B * H);

    /* attention block */
    for (int b = 0; b < B; ++b) or_rmsnorm(x + (int64_t)b * H, H, ly->in_norm, c->rms_eps,
                                           h + (int64_t)b * H);
    or_linear(h, B, H, ly->wq, QD, q);
    or_linear(h, B, H, ly->wk, KD, k);
    or_linear(h, B, H, ly->wv, KD, v);
    if (tap && taps->qkv)
      for (int b = 0; b < B; ++b) {
        double* dst = taps->qkv + (int64_t)b * (QD + 2 * KD);
        memcpy(dst, q + (int64_t)b * QD, sizeof(double) * QD);
        memcpy(dst + QD, k + (int64_t)b * KD, sizeof(double) * KD);
        memcpy(dst + QD + KD, v + (int64_t)b * KD, sizeof(double) * KD);
      }
    for (int b = 0; b < B; ++b) {
      for (int hh = 0; hh < Hq; ++hh) {
        double* qh = q + (int64_t)b * QD + (int64_t)hh * D;
        or_rmsnorm(qh, D, ly->q_norm, c->rms_eps, headbuf);
        memcpy(qh, headbuf, sizeof(double) * D);
        or_rope_neox(qh, D, positions[b], c->rope_theta);
      }
      for (int g = 0; g < Hkv; ++g) {
        double* kh = k + (int64_t)b * KD + (int64_t)g * D;
        or_rmsnorm(kh, D, ly->k_norm, c->rms_eps, headbuf);
        memcpy(kh, headbuf, sizeof(double) * D);
        or_rope_neox(kh, D, positions[b], c->rope_theta);
      }
    }
    if (tap && taps->q_rot) memcpy(taps->q_rot, q, sizeof(double) * B * QD);
    if (tap && taps->k_rot) memcpy(taps->k_rot, k, sizeof(double) * B * KD);
    /* append this step's K/V (rounded to the pool's type) at each sequence's position */
    for (int b = 0; b < B; ++b) {
      int pos = positions[b];
      int page = block_tables[(int64_t)b * max_pages + pos / OR_PAGE];
      if (page < 0 || page >= num_pages) goto bad;
      for (int g = 0; g < Hkv; ++g) {
        const int64_t kd = pool_index(num_pages, Hkv, D, l, page, 0, g, pos % OR_PAGE);
        const int64_t vd = pool_index(num_pages, Hkv, D, l, page, 1, g, pos % OR_PAGE);
        for (int d = 0; d < D; ++d) {
          pool_put(pool, kv, kd + d, 0, k[(int64_t)b * KD + (int64_t)g * D + d]);
          pool_put(pool, kv, vd + d, 1, v[(int64_t)b * KD + (int64_t)g * D + d]);
        }
      }
    }
    for (int b = 0; b < B; ++b) {
      int ctx = positions[b] + 1;
      const int32_t* row = block_tables + (int64_t)b * max_pages;
      for (int t = 0; t < (ctx + OR_PAGE - 1) / OR_PAGE; ++t)
        if (row[t] < 0 || row[t] >= num_pages) goto bad;
      or_attention(q + (int64_t)b * QD, Hq, Hkv, D, pool, num_pages, l, row, ctx,
                   att + (int64_t)b * QD, kv);
    }
    if (tap && taps->attn) memcpy(taps->attn, att, sizeof(double) * B * QD);
    or_linear(att, B, QD, ly->wo, H, tmp);
    for (int64_t i = 0; i < (int64_t)B * H; ++i) x[i] += tmp[i];
    if (tap && taps->x_mid) memcpy(taps->x_mid, x, sizeof(double) * B * H);

    /* MLP block */
    for (int b = 0; b < B; ++b) or_rmsnorm(x + (int64_t)b * H, H, ly->post_norm, c->rms_eps,
                                           h + (int64_t)b * H);
    or_linear(h, B, H, ly->wgate, I, gt);
    or_linear(h, B, H, ly->wup, I, up);
    for (int64_t i = 0; i < (int64_t)B * I; ++i) gt[i] = or_silu(gt[i]) * up[i];
    if (tap && taps->act) memcpy(taps->act, gt, sizeof(double) * B * I);
    or_linear(gt, B, I, ly->wdown, H, tmp);
    for (int64_t i = 0; i < (int64_t)B * H; ++i) x[i] += tmp[i];
    if (tap && taps->x_out) memcpy(taps->x_out, x, sizeof(double) * B * H);
  }

  for (int b = 0; b < B; ++b) or_rmsnorm(x + (int64_t)b * H, H, w->final_norm, c->rms_eps,
                                         h + (int64_t)b * H);
  if (taps && taps->final_h) memcpy(taps->final_h, h, sizeof(double) * B * H);
  {
    double* lg = logits ? logits : calloc((size_t)B * V, sizeof(double));
    or_linear(h, B, H, w->lm_head ? w->lm_head : w->embed, V, lg);
    for (int b = 0; b < B; ++b) next[b] = or_argmax(lg + (int64_t)b * V, V);
    if (!logits) free(lg);
  }
  free(x); free(h); free(q); free(k); free(v); free(att); free(tmp); free(gt); free(up);
  free(headbuf);
  return 0;
bad:
  free(x); free(h); free(q); free(k); free(v); free(att); free(tmp); free(gt); free(up);
  free(headbuf);
  return -1;
}
