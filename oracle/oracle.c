/*
 * oracle.c -- CPU oracle for the continuous-batching decode forward step.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this library. The product path (the HIP library)
 * never calls, links or includes anything here, and nothing here includes
 * or calls the product's code.
 *
 * What it computes, and from where:
 *  - The decoder: a pre-norm transformer with grouped-query attention,
 *    RMSNorm, RoPE and a SwiGLU feed-forward. The pages never define the
 *    model ("batched GQA / normalisation workers" on the Kestrel page,
 *    "0.8MB 跑通 Qwen" 14-1, section 2); the structure is the plainest
 *    reading of the workload description (RMSNorm gains, RoPE base 10000,
 *    SwiGLU FFN, GQA head counts).
 *  - Serial mode decodes one sequence alone, one token per forward, over a
 *    dense per-sequence KV store. This is the ground truth: the Kestrel page
 *    (section 3) reports batched outputs byte-identical to serial ones, and
 *    section 1 states that only the compute is merged, never the per-request
 *    state.
 *  - Paged-batched mode applies the method: one step over many sequences,
 *    rows taken in order, KV read and appended through per-sequence block
 *    tables into a shared pool of fixed-size blocks (Go under the hood,
 *    section 20.3.2: PagedAttention's fixed-size blocks; prefill chunks and
 *    decode rows share one step). Its per-row arithmetic is the serial
 *    mode's, so the two agree byte for byte.
 *  - The sampler (temperature, top-k, top-p, frequency/presence penalty with
 *    decay) follows the Albatross worker description (RWKV-Runner Albatross
 *    article, "Worker main loop" and adapter defaults). Its per-id values
 *    (penalised logit, z, e, counts) are fp32, the precision of the GPU
 *    sampler, because they decide an integer token; the masses summed over
 *    the vocabulary are accumulated in double so that each decision is the
 *    one the exact sum of those fp32 values makes.
 *  - The draw: Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11,
 *    "Parallel random numbers: as easy as 1, 2, 3"), counter = (request id,
 *    step id, 0, 0), key = (seed, 0).
 *
 * Arithmetic: every dot product accumulates in double, in ascending index
 * order, and every activation inside the layers stays a double: the norm
 * outputs, the projections, the rotated query, the attention output, the
 * SwiGLU product and the residual stream are never rounded. bf16 appears
 * where the model stores values in memory that the step streams: the
 * weights (given) and the KV cache, where each appended K (after RoPE) and
 * V is rounded to bf16 (round to nearest even, directly from the double);
 * and at the LM head, a bf16 contraction whose input (the final norm's
 * output) is rounded to bf16 the same way. Logits are doubles; the greedy id is the lowest id of the maximum of the logits
 * rounded to binary32, the precision in which the GPU takes that decision.
 * OpenMP runs only across independent rows, heads or output elements,
 * never inside a reduction.
 *
 * Storage formats beyond bf16 (follow-ups the pages name): an 8-bit KV cache
 * (OCP E4M3 codes of value / scale, the "Continuous Batching" practice
 * article, section 6) and int8 weights (codes q with one scale per matrix
 * row, read as q * scale; the RWKV-Runner Albatross article's follow-up
 * list). Both are defined here by their decoded values, in double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_OK 0
#define OR_EINVAL -1

/* ------------------------------------------------------------------ bf16 */

/* bf16 bits -> double: bf16 is the top half of an IEEE binary32. */
double or_bf16_to_f64(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* double -> bf16, round to nearest even from the exact double value.
 * bf16 keeps 8 significant bits. For normal results the rounding is done
 * on the double's 52-bit fraction at bit 45; results below the smallest
 * normal float go through binary32 (those magnitudes never arise here). */
uint16_t or_f64_to_bf16(double x) {
  if (isnan(x)) return 0x7fc0;
  double ax = fabs(x);
  if (ax != 0.0 && ax < 1.1754943508222875e-38) {
    float f = (float)x;
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
  }
  uint64_t b;
  memcpy(&b, &x, 8);
  uint64_t lsb = (b >> 45) & 1u;
  b += ((uint64_t)1 << 44) - 1 + lsb;
  b &= ~(((uint64_t)1 << 45) - 1);
  double r;
  memcpy(&r, &b, 8);
  if (fabs(r) > 3.3895313892515355e38) /* beyond the largest finite bf16 */
    return (uint16_t)(x < 0 ? 0xff80 : 0x7f80);
  float f = (float)r; /* exact: r has 8 significant bits and a float exponent */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

static inline double bf(uint16_t h) { return or_bf16_to_f64(h); }
static inline uint16_t tobf(double x) { return or_f64_to_bf16(x); }

/* ------------------------------------------------------------ fp8 e4m3 */

/* The OCP 8-bit float E4M3 (the KV-cache quantisation the "Continuous
 * Batching" practice article recommends, section 6): 1 sign bit, 4 exponent
 * bits (bias 7), 3 mantissa bits. Exponent field 0 holds the subnormals
 * m * 2^-9; exponent field 15 with mantissa 7 is NaN; there is no infinity,
 * and the largest magnitude is 1.75 * 2^8 = 448. */
double or_e4m3_to_f64(uint8_t c) {
  int e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = m * ldexp(1.0, -9);
  else
    v = (1.0 + m / 8.0) * ldexp(1.0, e - 7);
  return (c & 0x80) ? -v : v;
}

/* double -> E4M3: the finite code nearest to x (on a tie the code with an
 * even mantissa), so magnitudes beyond 448 saturate to 448; NaN -> 0x7f.
 * Found by comparing |x| with every non-negative finite code. */
uint8_t or_f64_to_e4m3(double x) {
  if (isnan(x)) return 0x7f;
  const uint8_t sign = signbit(x) ? 0x80 : 0;
  const double a = fabs(x);
  int best = 0;
  double bd = INFINITY;
  for (int c = 0; c < 0x7f; ++c) {
    const double d = fabs(a - or_e4m3_to_f64((uint8_t)c));
    if (d < bd || (d == bd && (c & 1) == 0)) {
      bd = d;
      best = c;
    }
  }
  return (uint8_t)(sign | best);
}

/* ------------------------------------------------------------ the model */

typedef struct {
  int32_t n_layers, d_model, n_heads, n_kv_heads, head_dim, ffn_dim, vocab;
  int32_t kv_fp8; /* 0: the KV cache holds bf16; 1: E4M3 codes of value / scale */
  double rms_eps, rope_base;
  const uint16_t* embed;      /* [vocab][d_model] */
  const uint16_t* final_norm; /* [d_model] */
  const uint16_t* lm_head;    /* [vocab][d_model] */
  const uint16_t* const* attn_norm; /* per layer [d_model] */
  const uint16_t* const* w_qkv;     /* per layer [(Hq+2Hkv)*hd][d_model] */
  const uint16_t* const* w_o;       /* per layer [d_model][Hq*hd] */
  const uint16_t* const* ffn_norm;  /* per layer [d_model] */
  const uint16_t* const* w_gate;    /* per layer [ffn][d_model] */
  const uint16_t* const* w_up;      /* per layer [ffn][d_model] */
  const uint16_t* const* w_down;    /* per layer [d_model][ffn] */
  double k_scale, v_scale;          /* fp8 cache: value = decode(code) * scale */
  /* w_int8: the projection matrices (QKV, O, gate, up, down, LM head) hold
   * int8 codes q (the pointers above point at int8 [rows][cols]) read as
   * q * scale[row]; the embedding and the norm gains stay bf16. */
  int32_t w_int8;
  int32_t pad_;
  const float* lm_head_scale;       /* [vocab] */
  const float* const* s_qkv;        /* per layer, one scale per matrix row */
  const float* const* s_o;
  const float* const* s_gate;
  const float* const* s_up;
  const float* const* s_down;
} or_model;

/* RMSNorm: y_i = x_i / sqrt(mean(x^2) + eps) * g_i. */
void or_rmsnorm(const double* x, const uint16_t* g, int32_t d, double eps, double* y) {
  double ss = 0.0;
  for (int32_t i = 0; i < d; ++i) ss += x[i] * x[i];
  double inv = 1.0 / sqrt(ss / (double)d + eps);
  for (int32_t i = 0; i < d; ++i) y[i] = x[i] * inv * bf(g[i]);
}

/* y[n] = sum_k x[k] * W[n][k], W row-major [N][K] bf16. */
void or_linear(const double* x, int32_t K, const uint16_t* W, int32_t N, double* y) {
  for (int32_t n = 0; n < N; ++n) {
    const uint16_t* w = W + (size_t)n * K;
    double s = 0.0;
    for (int32_t k = 0; k < K; ++k) s += x[k] * bf(w[k]);
    y[n] = s;
  }
}

/* Weight-only int8 (the RWKV-Runner Albatross article lists int8 weights
 * as a follow-up): y[n] = scale[n] * sum_k x[k] * Q[n][k], Q row-major
 * [N][K] int8, one scale per output row. */
void or_linear_i8(const double* x, int32_t K, const int8_t* Q, const float* scale, int32_t N,
                  double* y) {
  for (int32_t n = 0; n < N; ++n) {
    const int8_t* q = Q + (size_t)n * K;
    double s = 0.0;
    for (int32_t k = 0; k < K; ++k) s += x[k] * (double)q[k];
    y[n] = (double)scale[n] * s;
  }
}

/* A projection of the model: bf16 weights, or int8 codes with row scales. */
static void project(const or_model* m, const uint16_t* W, const float* scale, const double* x,
                    int32_t K, int32_t N, double* y) {
  if (m->w_int8)
    or_linear_i8(x, K, (const int8_t*)(const void*)W, scale, N, y);
  else
    or_linear(x, K, W, N, y);
}

/* RoPE, rotate-half pairing: element i pairs with i + hd/2, angle
 * pos * base^(-2i/hd). (a, b) -> (a cos - b sin, b cos + a sin). */
void or_rope(double* v, int32_t hd, int32_t pos, double base) {
  int32_t half = hd / 2;
  for (int32_t i = 0; i < half; ++i) {
    double inv_freq = pow(base, -2.0 * (double)i / (double)hd);
    double th = (double)pos * inv_freq;
    double c = cos(th), s = sin(th);
    double a = v[i], b = v[i + half];
    v[i] = a * c - b * s;
    v[i + half] = b * c + a * s;
  }
}

/* How the cache stores one K or V vector: bf16 values, or E4M3 codes of
 * value / scale. */
typedef struct {
  int32_t fp8;
  double k_scale, v_scale;
} or_kvfmt;

static inline double kv_elem(const void* p, int32_t i, int32_t fp8, double scale) {
  if (fp8) return or_e4m3_to_f64(((const uint8_t*)p)[i]) * scale;
  return bf(((const uint16_t*)p)[i]);
}

/* One query head over n keys: softmax(q.k_j / sqrt(hd)) weighted sum of v_j.
 * keys[j] / vals[j] point at hd stored values each (format f). */
static void attend_head(const double* q, const void* const* keys, const void* const* vals,
                        int32_t n, int32_t hd, or_kvfmt f, double* s /* scratch [n] */,
                        double* out) {
  double scale = 1.0 / sqrt((double)hd);
  double m = -INFINITY;
  for (int32_t j = 0; j < n; ++j) {
    double dot = 0.0;
    for (int32_t i = 0; i < hd; ++i) dot += q[i] * kv_elem(keys[j], i, f.fp8, f.k_scale);
    s[j] = dot * scale;
    if (s[j] > m) m = s[j];
  }
  double den = 0.0;
  for (int32_t j = 0; j < n; ++j) {
    s[j] = exp(s[j] - m);
    den += s[j];
  }
  for (int32_t i = 0; i < hd; ++i) {
    double acc = 0.0;
    for (int32_t j = 0; j < n; ++j) acc += s[j] * kv_elem(vals[j], i, f.fp8, f.v_scale);
    out[i] = acc / den;
  }
}

/* Dense attention for tests: q [Hq][hd] (double), K/V [n][Hkv][hd] stored
 * values (fp8 = 0: bf16; 1: E4M3 codes of value / scale); query head h
 * reads KV head h*Hkv/Hq (query heads grouped contiguously). */
int or_attention_dense_kv(const double* q, const void* K, const void* V, int32_t n,
                          int32_t n_heads, int32_t n_kv_heads, int32_t hd, int32_t fp8,
                          double k_scale, double v_scale, double* out) {
  if (n <= 0 || n_heads % n_kv_heads) return OR_EINVAL;
  const size_t esz = fp8 ? 1 : 2;
  or_kvfmt f = {fp8, k_scale, v_scale};
  const void** kp = malloc(sizeof(*kp) * (size_t)n);
  const void** vp = malloc(sizeof(*vp) * (size_t)n);
  double* s = malloc(sizeof(double) * (size_t)n);
  for (int32_t h = 0; h < n_heads; ++h) {
    int32_t g = h * n_kv_heads / n_heads;
    for (int32_t j = 0; j < n; ++j) {
      kp[j] = (const uint8_t*)K + ((size_t)j * n_kv_heads + g) * hd * esz;
      vp[j] = (const uint8_t*)V + ((size_t)j * n_kv_heads + g) * hd * esz;
    }
    attend_head(q + (size_t)h * hd, kp, vp, n, hd, f, s, out + (size_t)h * hd);
  }
  free(kp);
  free(vp);
  free(s);
  return OR_OK;
}

int or_attention_dense(const double* q, const uint16_t* K, const uint16_t* V, int32_t n,
                       int32_t n_heads, int32_t n_kv_heads, int32_t hd, double* out) {
  return or_attention_dense_kv(q, K, V, n, n_heads, n_kv_heads, hd, 0, 1.0, 1.0, out);
}

/* ------------------------------------------------------- KV addressing */

/* Where the K (kind 0) or V (kind 1) vector of one position lives.
 * Dense store:  [L][2][max_pos][Hkv][hd], one per sequence.
 * Paged pool:   [L][2][num_blocks][bs][Hkv][hd], shared; a sequence's
 *               position p lives in block table[p / bs], slot p % bs. */
typedef struct {
  int32_t paged;
  int32_t max_pos;    /* dense */
  void* base;         /* dense store or pool (bf16 values, or fp8 codes) */
  int32_t num_blocks; /* paged */
  int32_t block_size; /* paged */
  const int32_t* table;
  int32_t table_len;
} or_kv;

static void* kv_at(const or_model* m, const or_kv* kv, int32_t layer, int32_t kind,
                   int32_t pos, int32_t g) {
  size_t vec = (size_t)m->n_kv_heads * m->head_dim;
  const size_t esz = m->kv_fp8 ? 1 : 2;  /* bytes per stored value */
  if (pos < 0) return NULL;
  if (!kv->paged) {
    if (pos >= kv->max_pos) return NULL;
    size_t off = (((size_t)layer * 2 + kind) * kv->max_pos + pos) * vec +
                 (size_t)g * m->head_dim;
    return (uint8_t*)kv->base + off * esz;
  }
  int32_t bi = pos / kv->block_size;
  if (bi >= kv->table_len) return NULL;
  int32_t blk = kv->table[bi];
  if (blk < 0 || blk >= kv->num_blocks) return NULL;
  size_t off = ((((size_t)layer * 2 + kind) * kv->num_blocks + blk) *
                    kv->block_size + (size_t)(pos % kv->block_size)) * vec +
               (size_t)g * m->head_dim;
  return (uint8_t*)kv->base + off * esz;
}

static or_kvfmt kv_format(const or_model* m) {
  or_kvfmt f = {m->kv_fp8, m->k_scale, m->v_scale};
  return f;
}

/* ----------------------------------------------------- one decoder row */

static int32_t qkv_width(const or_model* m) {
  return (m->n_heads + 2 * m->n_kv_heads) * m->head_dim;
}

/* Stage A of a layer for one row: norm, QKV projection, RoPE at `pos`,
 * then append this row's K and V at `pos` (rounded to bf16, the cache's
 * storage type). Leaves the rotated query in q. */
static int row_pre_attention(const or_model* m, int32_t layer, const or_kv* kv,
                             const double* x, int32_t pos, double* q, double* hbuf,
                             double* acc) {
  int32_t d = m->d_model, hd = m->head_dim, hq = m->n_heads, hkv = m->n_kv_heads;
  or_rmsnorm(x, m->attn_norm[layer], d, m->rms_eps, hbuf);
  project(m, m->w_qkv[layer], m->w_int8 ? m->s_qkv[layer] : NULL, hbuf, d, qkv_width(m), acc);
  memcpy(q, acc, sizeof(double) * (size_t)hq * hd);
  for (int32_t h = 0; h < hq; ++h) or_rope(q + (size_t)h * hd, hd, pos, m->rope_base);
  for (int32_t g = 0; g < hkv; ++g) {
    void* kd = kv_at(m, kv, layer, 0, pos, g);
    void* vd = kv_at(m, kv, layer, 1, pos, g);
    if (!kd || !vd) return OR_EINVAL;
    double* k = acc + (size_t)(hq + g) * hd;
    const double* v = acc + (size_t)(hq + hkv + g) * hd;
    or_rope(k, hd, pos, m->rope_base);
    for (int32_t i = 0; i < hd; ++i) {
      if (m->kv_fp8) {  /* the cache's E4M3 code of value / scale */
        ((uint8_t*)kd)[i] = or_f64_to_e4m3(k[i] / m->k_scale);
        ((uint8_t*)vd)[i] = or_f64_to_e4m3(v[i] / m->v_scale);
      } else {
        ((uint16_t*)kd)[i] = tobf(k[i]);
        ((uint16_t*)vd)[i] = tobf(v[i]);
      }
    }
  }
  return OR_OK;
}

/* Stage B: every query head of the row attends over positions 0..pos. */
static int row_attention(const or_model* m, int32_t layer, const or_kv* kv,
                         const double* q, int32_t pos, double* o) {
  int32_t n = pos + 1, hd = m->head_dim;
  const void** kp = malloc(sizeof(*kp) * (size_t)n);
  const void** vp = malloc(sizeof(*vp) * (size_t)n);
  double* s = malloc(sizeof(double) * (size_t)n);
  int rc = OR_OK;
  for (int32_t h = 0; h < m->n_heads && rc == OR_OK; ++h) {
    int32_t g = h * m->n_kv_heads / m->n_heads;
    for (int32_t j = 0; j < n; ++j) {
      kp[j] = kv_at(m, kv, layer, 0, j, g);
      vp[j] = kv_at(m, kv, layer, 1, j, g);
      if (!kp[j] || !vp[j]) {
        rc = OR_EINVAL;
        break;
      }
    }
    if (rc == OR_OK)
      attend_head(q + (size_t)h * hd, kp, vp, n, hd, kv_format(m), s, o + (size_t)h * hd);
  }
  free(kp);
  free(vp);
  free(s);
  return rc;
}

/* Stage C: O projection + residual, norm, SwiGLU FFN + residual. */
static void row_post_attention(const or_model* m, int32_t layer, double* x, const double* o,
                               double* hbuf, double* acc, double* acc2) {
  int32_t d = m->d_model, f = m->ffn_dim, qd = m->n_heads * m->head_dim;
  project(m, m->w_o[layer], m->w_int8 ? m->s_o[layer] : NULL, o, qd, d, acc);
  for (int32_t i = 0; i < d; ++i) x[i] += acc[i];
  or_rmsnorm(x, m->ffn_norm[layer], d, m->rms_eps, hbuf);
  project(m, m->w_gate[layer], m->w_int8 ? m->s_gate[layer] : NULL, hbuf, d, f, acc);
  project(m, m->w_up[layer], m->w_int8 ? m->s_up[layer] : NULL, hbuf, d, f, acc2);
  for (int32_t i = 0; i < f; ++i) {
    double g = acc[i];
    acc[i] = g / (1.0 + exp(-g)) * acc2[i]; /* silu(gate) * up */
  }
  project(m, m->w_down[layer], m->w_int8 ? m->s_down[layer] : NULL, acc, f, d, acc2);
  for (int32_t i = 0; i < d; ++i) x[i] += acc2[i];
}

/* Final RMSNorm and LM head: logits[v] = sum_k bf16(norm(x)[k]) * W_lm[v][k].
 * The LM head is a bf16 contraction: its input, the final norm's output, is
 * rounded once to bf16 like its weights, and the products accumulate in
 * double. No stage follows it whose own rounding could turn this one's
 * last-bit differences into larger ones. */
static void row_logits(const or_model* m, const double* x, double* logits) {
  int32_t d = m->d_model;
  double* h = malloc(sizeof(double) * (size_t)d);
  or_rmsnorm(x, m->final_norm, d, m->rms_eps, h);
  for (int32_t k = 0; k < d; ++k) h[k] = bf(tobf(h[k]));
#pragma omp parallel for schedule(static)
  for (int32_t v = 0; v < m->vocab; ++v) {
    double s = 0.0;
    if (m->w_int8) {
      const int8_t* q = (const int8_t*)(const void*)m->lm_head + (size_t)v * d;
      for (int32_t k = 0; k < d; ++k) s += h[k] * (double)q[k];
      s *= (double)m->lm_head_scale[v];
    } else {
      const uint16_t* w = m->lm_head + (size_t)v * d;
      for (int32_t k = 0; k < d; ++k) s += h[k] * bf(w[k]);
    }
    logits[v] = s;
  }
  free(h);
}

/* The greedy decision: lowest id of the maximum of the logits rounded to
 * binary32. */
static int32_t greedy_id(const double* lg, int32_t V) {
  int32_t best = 0;
  float bv = (float)lg[0];
  for (int32_t v = 1; v < V; ++v)
    if ((float)lg[v] > bv) {
      bv = (float)lg[v];
      best = v;
    }
  return best;
}

typedef struct {
  double *q, *h, *o, *acc, *acc2;
} scratch_t;

static int scratch_alloc(const or_model* m, scratch_t* s) {
  int32_t w = qkv_width(m);
  int32_t big = w > m->ffn_dim ? w : m->ffn_dim;
  if (m->d_model > big) big = m->d_model;
  s->q = malloc(sizeof(double) * (size_t)m->n_heads * m->head_dim);
  s->o = malloc(sizeof(double) * (size_t)m->n_heads * m->head_dim);
  s->h = malloc(sizeof(double) * (size_t)m->d_model);
  s->acc = malloc(sizeof(double) * (size_t)big);
  s->acc2 = malloc(sizeof(double) * (size_t)big);
  return (s->q && s->o && s->h && s->acc && s->acc2) ? OR_OK : OR_EINVAL;
}

static void scratch_free(scratch_t* s) {
  free(s->q);
  free(s->o);
  free(s->h);
  free(s->acc);
  free(s->acc2);
}

static int model_ok(const or_model* m) {
  return m && (m->kv_fp8 == 0 || (m->kv_fp8 == 1 && m->k_scale > 0 && m->v_scale > 0)) &&
         (m->w_int8 == 0 || (m->w_int8 == 1 && m->lm_head_scale && m->s_qkv && m->s_o &&
                             m->s_gate && m->s_up && m->s_down)) &&
         m->n_layers > 0 && m->d_model > 0 && m->n_heads > 0 &&
         m->n_kv_heads > 0 && m->n_heads % m->n_kv_heads == 0 &&
         m->head_dim > 0 && m->head_dim % 2 == 0 && m->ffn_dim > 0 &&
         m->vocab > 0;
}

static void embed_row(const or_model* m, int32_t tok, double* x) {
  const uint16_t* e = m->embed + (size_t)tok * m->d_model;
  for (int32_t i = 0; i < m->d_model; ++i) x[i] = bf(e[i]);
}

/* ------------------------------------------------------------ serial mode */

/* Decode one sequence alone: feed tokens[0..n) one per forward at positions
 * start_pos.., appending to the dense store kv[L][2][max_pos][Hkv][hd].
 * If logits is non-NULL it receives [n][vocab] (or only the last token's
 * [vocab] when last_only is set). Returns 0 or OR_EINVAL. */
int or_serial_forward(const or_model* m, void* kv_dense, int32_t max_pos,
                      const int32_t* tokens, int32_t n, int32_t start_pos,
                      int32_t last_only, double* logits) {
  if (!model_ok(m) || n <= 0 || start_pos < 0 || start_pos + n > max_pos)
    return OR_EINVAL;
  or_kv kv = {0, max_pos, kv_dense, 0, 0, NULL, 0};
  scratch_t s;
  double* x = malloc(sizeof(double) * (size_t)m->d_model);
  if (scratch_alloc(m, &s) != OR_OK || !x) return OR_EINVAL;
  int rc = OR_OK;
  for (int32_t t = 0; t < n && rc == OR_OK; ++t) {
    int32_t tok = tokens[t], pos = start_pos + t;
    if (tok < 0 || tok >= m->vocab) {
      rc = OR_EINVAL;
      break;
    }
    embed_row(m, tok, x);
    for (int32_t l = 0; l < m->n_layers && rc == OR_OK; ++l) {
      rc = row_pre_attention(m, l, &kv, x, pos, s.q, s.h, s.acc);
      if (rc == OR_OK) rc = row_attention(m, l, &kv, s.q, pos, s.o);
      if (rc == OR_OK) row_post_attention(m, l, x, s.o, s.h, s.acc, s.acc2);
    }
    if (rc == OR_OK && logits && (!last_only || t == n - 1))
      row_logits(m, x, logits + (last_only ? 0 : (size_t)t * m->vocab));
  }
  free(x);
  scratch_free(&s);
  return rc;
}

/* ------------------------------------------------------ paged-batched mode */

/* One continuous-batching step. Sequences are taken in order; sequence s
 * contributes n_new[s] consecutive rows of `tokens` at positions
 * ctx_lens[s] .. ctx_lens[s]+n_new[s]-1 (ctx_lens = positions already in the
 * pool before the step). Each layer runs in three stages over all rows:
 * (A) norm, QKV, RoPE, append every row's K/V into the pool; (B) attention of
 * each row over its own positions 0..pos through its block table, which
 * makes a prefill chunk causal; (C) the rest of the layer. Sequences with
 * want_token[s] != 0 emit logits for their last row, in sequence order,
 * into logits_out [n_out][vocab]; greedy_out (optional) gets the greedy id.
 * pool: [L][2][num_blocks][bs][Hkv][hd]. */
int or_paged_step(const or_model* m, void* pool, int32_t num_blocks,
                  int32_t block_size, int32_t n_seqs, const int32_t* block_tables,
                  int32_t max_blocks_per_seq, const int32_t* ctx_lens,
                  const int32_t* n_new, const int32_t* tokens,
                  const int32_t* want_token, double* logits_out,
                  int32_t* greedy_out) {
  if (!model_ok(m) || n_seqs <= 0 || block_size <= 0 || num_blocks <= 0)
    return OR_EINVAL;
  int32_t R = 0;
  for (int32_t s = 0; s < n_seqs; ++s) {
    if (n_new[s] <= 0 || ctx_lens[s] < 0) return OR_EINVAL;
    if (ctx_lens[s] + n_new[s] > max_blocks_per_seq * block_size) return OR_EINVAL;
    R += n_new[s];
  }
  int32_t d = m->d_model, qd = m->n_heads * m->head_dim;
  double* X = malloc(sizeof(double) * (size_t)R * d);
  double* Q = malloc(sizeof(double) * (size_t)R * qd);
  double* O = malloc(sizeof(double) * (size_t)R * qd);
  int32_t* row_seq = malloc(sizeof(int32_t) * (size_t)R);
  int32_t* row_pos = malloc(sizeof(int32_t) * (size_t)R);
  or_kv* kvs = malloc(sizeof(or_kv) * (size_t)n_seqs);
  if (!X || !Q || !O || !row_seq || !row_pos || !kvs) return OR_EINVAL;
  int rc = OR_OK;
  for (int32_t s = 0, r = 0; s < n_seqs; ++s) {
    or_kv k = {1, 0, pool, num_blocks, block_size,
               block_tables + (size_t)s * max_blocks_per_seq, max_blocks_per_seq};
    kvs[s] = k;
    for (int32_t i = 0; i < n_new[s]; ++i, ++r) {
      row_seq[r] = s;
      row_pos[r] = ctx_lens[s] + i;
      if (tokens[r] < 0 || tokens[r] >= m->vocab) rc = OR_EINVAL;
    }
  }
  for (int32_t r = 0; r < R && rc == OR_OK; ++r) embed_row(m, tokens[r], X + (size_t)r * d);

  for (int32_t l = 0; l < m->n_layers && rc == OR_OK; ++l) {
#pragma omp parallel
    {
      scratch_t sc;
      int lrc = scratch_alloc(m, &sc);
#pragma omp for schedule(static)
      for (int32_t r = 0; r < R; ++r) {
        int e = row_pre_attention(m, l, &kvs[row_seq[r]], X + (size_t)r * d, row_pos[r],
                                  Q + (size_t)r * qd, sc.h, sc.acc);
        if (e != OR_OK) lrc = e;
      }
#pragma omp for schedule(dynamic)
      for (int32_t r = 0; r < R; ++r) {
        int e = row_attention(m, l, &kvs[row_seq[r]], Q + (size_t)r * qd, row_pos[r],
                              O + (size_t)r * qd);
        if (e != OR_OK) lrc = e;
      }
#pragma omp for schedule(static)
      for (int32_t r = 0; r < R; ++r)
        row_post_attention(m, l, X + (size_t)r * d, O + (size_t)r * qd, sc.h, sc.acc, sc.acc2);
      if (lrc != OR_OK) {
#pragma omp atomic write
        rc = lrc;
      }
      scratch_free(&sc);
    }
  }
  if (rc == OR_OK) {
    int32_t o = 0;
    for (int32_t s = 0, r = 0; s < n_seqs; ++s) {
      r += n_new[s];
      if (!want_token[s]) continue;
      double* lg = logits_out + (size_t)o * m->vocab;
      row_logits(m, X + (size_t)(r - 1) * d, lg);
      if (greedy_out) greedy_out[o] = greedy_id(lg, m->vocab);
      ++o;
    }
  }
  free(X);
  free(Q);
  free(O);
  free(row_seq);
  free(row_pos);
  free(kvs);
  return rc;
}

/* ------------------------------------------------------------- argmax */

/* Lowest id among the maxima. */
int32_t or_argmax_f32(const float* x, int32_t n) {
  int32_t best = 0;
  for (int32_t i = 1; i < n; ++i)
    if (x[i] > x[best]) best = i;
  return best;
}

int32_t or_argmax_f64(const double* x, int32_t n) {
  int32_t best = 0;
  for (int32_t i = 1; i < n; ++i)
    if (x[i] > x[best]) best = i;
  return best;
}

/* ------------------------------------------------------------- Philox */

static inline void mulhilo64(uint64_t a, uint64_t b, uint64_t* hi, uint64_t* lo) {
  unsigned __int128 p = (unsigned __int128)a * b;
  *hi = (uint64_t)(p >> 64);
  *lo = (uint64_t)p;
}

/* Philox4x64 with 10 rounds: each round multiplies words 0 and 2 by the two
 * round multipliers, recombines the halves with words 1 and 3 and the key,
 * then bumps the key by the two Weyl constants. */
void or_philox4x64_10(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4]) {
  uint64_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
  uint64_t k0 = key[0], k1 = key[1];
  for (int r = 0; r < 10; ++r) {
    uint64_t hi0, lo0, hi1, lo1;
    mulhilo64(0xD2E7470EE14C6C93ull, x0, &hi0, &lo0);
    mulhilo64(0xCA5A826395121157ull, x2, &hi1, &lo1);
    uint64_t y0 = hi1 ^ x1 ^ k0, y1 = lo1, y2 = hi0 ^ x3 ^ k1, y3 = lo0;
    x0 = y0;
    x1 = y1;
    x2 = y2;
    x3 = y3;
    k0 += 0x9E3779B97F4A7C15ull;
    k1 += 0xBB67AE8584CAA73Bull;
  }
  out[0] = x0;
  out[1] = x1;
  out[2] = x2;
  out[3] = x3;
}

/* The sampler's uniform: the top 24 bits of word 0 of
 * Philox4x64-10(counter = (request_id, step_id, 0, 0), key = (seed, 0)),
 * times 2^-24, exactly representable in fp32, in [0, 1). */
float or_uniform24(uint64_t seed, uint64_t request_id, uint32_t step_id) {
  uint64_t c[4] = {request_id, (uint64_t)step_id, 0, 0}, k[2] = {seed, 0}, o[4];
  or_philox4x64_10(c, k, o);
  return (float)(o[0] >> 40) * (1.0f / 16777216.0f);
}

/* ------------------------------------------------------------ sampler */

#define OR_MAX_FORBIDDEN 8
typedef struct {
  float temperature, top_p;
  int32_t top_k;
  float freq_penalty, presence_penalty, penalty_decay;
  uint64_t seed;
  int32_t n_forbidden;               /* ids never drawn: their l' is -inf */
  int32_t forbidden[OR_MAX_FORBIDDEN];
} or_sampling;

/* What decided the draw; lets a comparison skip rows whose outcome sits
 * within rounding of a boundary. Masses are unnormalised (exp(z - max z)). */
typedef struct {
  int32_t token;
  int32_t n_kept;         /* ids surviving top-k and top-p */
  float sum_all;          /* sum of e over the vocabulary */
  float sum_topk;         /* sum of e over the top-k set */
  float target;           /* top_p * sum_topk */
  float cum_before;       /* top-p running mass before the crossing id */
  float cum_after;        /* ... including it */
  float sum_kept;         /* mass of the final kept set */
  float r;                /* u * sum_kept */
  float cdf_lo, cdf_hi;   /* chosen id's interval of the ascending-id CDF */
  float p1, p2;           /* two largest e / sum_all */
  float u;
  int32_t n_cut;          /* ids summed before the top-p crossing id */
  int32_t n_before;       /* kept ids before the chosen one (ascending id) */
} or_sample_info;

typedef struct {
  float e;
  int32_t id;
} ev_t;

static int cmp_desc(const void* a, const void* b) {
  const ev_t* x = a;
  const ev_t* y = b;
  if (x->e > y->e) return -1;
  if (x->e < y->e) return 1;
  return (x->id > y->id) - (x->id < y->id);
}

/* One row of the batched sampler, in this order:
 *  S1 penalty   l' = l - f*c - q*[c > 0]                       (fp32);
 *               a forbidden id's l' is -inf (the Albatross worker masks
 *               forbidden tokens before the penalties and the draw)
 *  S2 T == 0    greedy on l' (lowest id); else z = l' / T       (fp32)
 *  S3 softmax   e = exp(z - max z), unnormalised               (fp32)
 *  S4 top-k     keep the k largest by (e desc, id asc) when 0 < k < V
 *  S5 top-p     when p < 1: in (e desc, id asc) order keep the shortest
 *               prefix whose mass reaches p * (mass kept by S4); the
 *               crossing id is kept
 *  S6 draw      u from Philox; r = u * kept mass; the first kept id in
 *               ascending id order whose running kept mass exceeds r
 *  S7 counts    c = c * decay for every id, then c[token] += 1  (fp32)
 * The masses in S4-S6 are sums of the fp32 values e; they are accumulated
 * exactly enough (double) that the decisions are those of the mathematical
 * sums (a sequential fp32 sum over a large vocabulary loses every term below
 * half an ulp of the running total and drifts by ~1e-4).
 * counts (in/out, [V]) may be NULL: then no penalty and no update. */
int32_t or_sample_f32(const float* logits, int32_t V, float* counts,
                      const or_sampling* sp, uint64_t request_id,
                      uint32_t step_id, or_sample_info* info) {
  or_sample_info di;
  memset(&di, 0, sizeof(di));
  float* lp = malloc(sizeof(float) * (size_t)V);
  float* e = malloc(sizeof(float) * (size_t)V);
  unsigned char* kept = malloc((size_t)V);
  ev_t* ord = malloc(sizeof(ev_t) * (size_t)V);
  for (int32_t v = 0; v < V; ++v) {
    float l = logits[v];
    if (counts) {
      float c = counts[v];
      float t = sp->freq_penalty * c;
      l = l - t;
      if (c > 0.0f) l = l - sp->presence_penalty;
    }
    lp[v] = l;
  }
  for (int32_t f = 0; f < sp->n_forbidden && f < OR_MAX_FORBIDDEN; ++f)
    if (sp->forbidden[f] >= 0 && sp->forbidden[f] < V) lp[sp->forbidden[f]] = -INFINITY;
  int32_t token;
  if (sp->temperature == 0.0f) {
    token = or_argmax_f32(lp, V);
    di.n_kept = 1;
  } else {
    float zmax = -INFINITY;
    for (int32_t v = 0; v < V; ++v) {
      float z = lp[v] / sp->temperature;
      e[v] = z;
      if (z > zmax) zmax = z;
    }
    double sum_all = 0.0;
    for (int32_t v = 0; v < V; ++v) {
      e[v] = expf(e[v] - zmax);
      sum_all += e[v];
      kept[v] = 1;
    }
    di.sum_all = (float)sum_all;
    for (int32_t v = 0; v < V; ++v) {
      ord[v].e = e[v];
      ord[v].id = v;
    }
    qsort(ord, (size_t)V, sizeof(ev_t), cmp_desc);
    di.p1 = (float)(ord[0].e / sum_all);
    di.p2 = V > 1 ? (float)(ord[1].e / sum_all) : 0.0f;
    int32_t nk = V;
    if (sp->top_k > 0 && sp->top_k < V) {
      nk = sp->top_k;
      for (int32_t i = nk; i < V; ++i) kept[ord[i].id] = 0;
    }
    double sum_topk = 0.0;
    for (int32_t v = 0; v < V; ++v)
      if (kept[v]) sum_topk += e[v];
    di.sum_topk = (float)sum_topk;
    if (sp->top_p < 1.0f) {
      double target = (double)sp->top_p * sum_topk;
      double run = 0.0;
      int32_t cut = nk - 1;
      for (int32_t i = 0; i < nk; ++i) {
        double before = run;
        run += ord[i].e;
        if (run >= target) {
          cut = i;
          di.n_cut = i;
          di.cum_before = (float)before;
          di.cum_after = (float)run;
          break;
        }
      }
      for (int32_t i = cut + 1; i < nk; ++i) kept[ord[i].id] = 0;
      di.target = (float)target;
    }
    double sum_kept = 0.0;
    int32_t n_kept = 0;
    for (int32_t v = 0; v < V; ++v)
      if (kept[v]) {
        sum_kept += e[v];
        ++n_kept;
      }
    float u = or_uniform24(sp->seed, request_id, step_id);
    double r = (double)u * sum_kept;
    double run = 0.0;
    token = -1;
    int32_t last = -1, seen = 0;
    for (int32_t v = 0; v < V; ++v) {
      if (!kept[v]) continue;
      double lo = run;
      run += e[v];
      last = v;
      di.n_before = seen++;
      if (run > r) {
        token = v;
        di.cdf_lo = (float)lo;
        di.cdf_hi = (float)run;
        break;
      }
    }
    if (token < 0) { /* r reached the total: take the last kept id */
      token = last;
      di.cdf_lo = (float)(run - e[last]);
      di.cdf_hi = (float)run;
    }
    di.n_kept = n_kept;
    di.sum_kept = (float)sum_kept;
    di.r = (float)r;
    di.u = u;
  }
  if (counts) {
    for (int32_t v = 0; v < V; ++v) counts[v] = counts[v] * sp->penalty_decay;
    counts[token] = counts[token] + 1.0f;
  }
  di.token = token;
  if (info) *info = di;
  free(lp);
  free(e);
  free(kept);
  free(ord);
  return token;
}

int32_t or_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads the oracle's parallel loops use from now on (n >= 1). */
void or_set_num_threads(int32_t n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
