/*
 * oracle.c -- CPU reference of the KV-cached decode forward pass.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h). Plain loops, one thread, no BLAS.
 * Every reduction accumulates in double in index order; every tensor is float.
 *
 * Sources (the three pages this method is described on):
 *   [BML]  "bare-metal-llm: GPT-2 inference on hand-written Metal kernels",
 *          sections "Picking the model", "What got built", "The bug worth telling".
 *   [BF]   "batch_forge" README: component status table, the GELU/tanh paragraph,
 *          the KV-cache roadmap item.
 *   [RVM]  "rvllm Metal backend" post: "What the kernels do", "Things that were
 *          problematic", "How I know it's correct", "What's basic about it" and
 *          "What's next" (the F32 KV cache and 1-byte Q8_0 weights as next steps).
 *   [BF] status table also lists int8 dequantization and sampling (greedy,
 *          temperature, top-k), and the temperature 0.7 demo.
 * Where the pages give no formula, the reading used is stated at the function.
 */
#include "oracle.h"

#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static int g_mut = 0;
/* Planted mistakes, used only by the mutation tests of the pins:
 *  1 GELU without the argument clamp, tanh from float exp(2a) (the overflow bug in [BML])
 *  2 GELU without the cubic term
 *  3 LayerNorm without subtracting the mean
 *  4 attention scale 1/hd instead of 1/sqrt(hd)
 *  5 KV-cached attention leaves out the current position
 *  6 RoPE rotates the other way
 *  7 GQA maps query head h to KV head h mod n_kv
 *  8 argmax ties go to the highest index
 *  9 stateless causal mask lets each row see one future position
 * 10 linear layers drop the bias
 * 11 bfloat16 rounding of K/V truncates instead of rounding to nearest even
 * 12 8-bit quantization truncates toward zero instead of rounding
 * 13 8-bit quantization scale max|x| / 128
 * 14 sampling ignores the temperature
 * 15 sampling keeps one candidate more than top_k                                   */
void orc_set_mutation(int m) { g_mut = m; }

struct orc_model {
  orc_config c;
  const float* w;
  float* own;   /* weight_q8: the dequantized copy w points to */
  /* offsets (in floats) into w */
  size_t wte, wpe, lnf_g, lnf_b, rmsf, w_head;
  size_t* layer; /* n_layer entries: offset of the layer's first tensor */
};

struct orc_seq {
  int cap, len;
  int L, H, hd;
  float* K; /* [L][H][cap][hd] */
  float* V;
};

/* ------------------------------------------------------------------ sizes */

static int cfg_ok(const orc_config* c) {
  if (!c) return 0;
  if (c->arch != ORC_ARCH_GPT2 && c->arch != ORC_ARCH_LLAMA) return 0;
  if (c->n_layer < 0 || c->d_model <= 0 || c->n_head <= 0 || c->head_dim <= 0) return 0;
  if (c->d_ff <= 0 || c->vocab <= 0 || c->n_ctx <= 0) return 0;
  if (c->arch == ORC_ARCH_GPT2) {
    if (c->n_kv_head != c->n_head || c->n_head * c->head_dim != c->d_model) return 0;
  } else {
    if (c->n_kv_head <= 0 || c->n_head % c->n_kv_head != 0 || (c->head_dim % 2) != 0) return 0;
  }
  if (c->weight_q8 && (c->d_model % 32 || c->d_ff % 32 || (c->n_head * c->head_dim) % 32)) return 0;
  return 1;
}

static size_t layer_floats(const orc_config* c) {
  size_t d = (size_t)c->d_model, ff = (size_t)c->d_ff;
  if (c->arch == ORC_ARCH_GPT2) {
    return 2 * d + 3 * d * d + 3 * d + d * d + d + 2 * d + ff * d + ff + d * ff + d;
  }
  size_t hq = (size_t)c->n_head * c->head_dim, hk = (size_t)c->n_kv_head * c->head_dim;
  return d + hq * d + 2 * hk * d + d * hq + d + 2 * ff * d + d * ff;
}

size_t orc_weight_count(const orc_config* c) {
  if (!cfg_ok(c)) return 0;
  size_t d = (size_t)c->d_model, V = (size_t)c->vocab;
  size_t n = V * d + (size_t)c->n_layer * layer_floats(c);
  if (c->arch == ORC_ARCH_GPT2) n += (size_t)c->n_ctx * d + 2 * d;
  else n += d + V * d;
  return n;
}

/* In place: every row of the [rows][cols] matrix at w replaced by the dequantization
 * q * d of its 8-bit block quantization. */
static void q8_matrix(float* w, size_t rows, int cols) {
  signed char* q = (signed char*)malloc((size_t)cols);
  float* d = (float*)malloc(sizeof(float) * (size_t)(cols / 32));
  for (size_t r = 0; r < rows; ++r) {
    float* x = w + r * (size_t)cols;
    orc_quantize_q8(x, cols, q, d);
    for (int i = 0; i < cols; ++i) x[i] = (float)q[i] * d[i / 32];
  }
  free(q);
  free(d);
}

orc_model* orc_model_create(const orc_config* c, const float* w, size_t n) {
  if (!cfg_ok(c) || !w || n != orc_weight_count(c)) return NULL;
  orc_model* m = (orc_model*)calloc(1, sizeof(orc_model));
  if (!m) return NULL;
  m->c = *c;
  m->w = w;
  m->layer = (size_t*)calloc((size_t)(c->n_layer > 0 ? c->n_layer : 1), sizeof(size_t));
  size_t d = (size_t)c->d_model, V = (size_t)c->vocab, off = 0;
  m->wte = off; off += V * d;
  if (c->arch == ORC_ARCH_GPT2) { m->wpe = off; off += (size_t)c->n_ctx * d; }
  for (int l = 0; l < c->n_layer; ++l) { m->layer[l] = off; off += layer_floats(c); }
  if (c->arch == ORC_ARCH_GPT2) {
    m->lnf_g = off; off += d;
    m->lnf_b = off; off += d;
  } else {
    m->rmsf = off; off += d;
    m->w_head = off; off += V * d;
  }
  if (c->weight_q8) {
    /* every weight matrix (embeddings and head included) through the 8-bit blocks of
     * its rows; norm parameters and biases stay float */
    m->own = (float*)malloc(sizeof(float) * n);
    if (!m->own) { orc_model_free(m); return NULL; }
    memcpy(m->own, w, sizeof(float) * n);
    m->w = m->own;
    size_t ff = (size_t)c->d_ff, hq = (size_t)c->n_head * c->head_dim, hk = (size_t)c->n_kv_head * c->head_dim;
    q8_matrix(m->own + m->wte, V, (int)d);
    if (c->arch == ORC_ARCH_GPT2) {
      q8_matrix(m->own + m->wpe, (size_t)c->n_ctx, (int)d);
      for (int l = 0; l < c->n_layer; ++l) {
        float* p = m->own + m->layer[l] + 2 * d;   /* after ln1_g, ln1_b */
        q8_matrix(p, 3 * d, (int)d); p += 3 * d * d + 3 * d;
        q8_matrix(p, d, (int)d); p += d * d + d + 2 * d;
        q8_matrix(p, ff, (int)d); p += ff * d + ff;
        q8_matrix(p, d, (int)ff);
      }
    } else {
      for (int l = 0; l < c->n_layer; ++l) {
        float* p = m->own + m->layer[l] + d;       /* after rms1 */
        q8_matrix(p, hq, (int)d); p += hq * d;
        q8_matrix(p, hk, (int)d); p += hk * d;
        q8_matrix(p, hk, (int)d); p += hk * d;
        q8_matrix(p, d, (int)hq); p += d * hq + d;
        q8_matrix(p, ff, (int)d); p += ff * d;
        q8_matrix(p, ff, (int)d); p += ff * d;
        q8_matrix(p, d, (int)ff);
      }
      q8_matrix(m->own + m->w_head, V, (int)d);
    }
  }
  return m;
}

void orc_model_free(orc_model* m) {
  if (!m) return;
  free(m->own);
  free(m->layer);
  free(m);
}

orc_seq* orc_seq_create(const orc_model* m, int cap) {
  if (!m || cap <= 0) return NULL;
  orc_seq* s = (orc_seq*)calloc(1, sizeof(orc_seq));
  if (!s) return NULL;
  s->cap = cap;
  s->L = m->c.n_layer;
  s->H = m->c.n_kv_head;
  s->hd = m->c.head_dim;
  size_t n = (size_t)(s->L > 0 ? s->L : 1) * s->H * (size_t)cap * s->hd;
  s->K = (float*)calloc(n, sizeof(float));
  s->V = (float*)calloc(n, sizeof(float));
  if (!s->K || !s->V) { orc_seq_free(s); return NULL; }
  return s;
}

void orc_seq_free(orc_seq* s) {
  if (!s) return;
  free(s->K);
  free(s->V);
  free(s);
}

int orc_seq_len(const orc_seq* s) { return s ? s->len : -1; }

/* ------------------------------------------------------------- components */

/* [BML] "What got built" (layernorm); [BF] status table (layernorm). The pages print no
 * formula; the reading is the standard one: biased variance over the row, eps inside
 * the square root, then gain and shift. */
void orc_layernorm(const float* x, const float* g, const float* b, int n, double eps, float* y) {
  double mean = 0.0;
  for (int i = 0; i < n; ++i) mean += (double)x[i];
  mean /= n;
  if (g_mut == 3) mean = 0.0;
  double var = 0.0;
  for (int i = 0; i < n; ++i) {
    double t = (double)x[i] - mean;
    var += t * t;
  }
  var /= n;
  double r = 1.0 / sqrt(var + eps);
  for (int i = 0; i < n; ++i) y[i] = (float)(((double)x[i] - mean) * r * (double)g[i] + (double)b[i]);
}

/* [BF] status table (rmsnorm); [RVM] "What the kernels do" (RMSNorm the input):
 * y = x / sqrt(mean(x^2) + eps) * w. */
void orc_rmsnorm(const float* x, const float* w, int n, double eps, float* y) {
  double ms = 0.0;
  for (int i = 0; i < n; ++i) ms += (double)x[i] * (double)x[i];
  ms /= n;
  double r = 1.0 / sqrt(ms + eps);
  for (int i = 0; i < n; ++i) y[i] = (float)((double)x[i] * r * (double)w[i]);
}

/* tanh-GELU. [BML] "The bug worth telling": tanh overflowed through exp(2x) to Inf/Inf.
 * [BF] GELU paragraph: the fix clamps the tanh argument to +-15, where tanh is already
 * +-1 to float precision. The pages do not print the formula; the reading is GPT-2's
 * tanh approximation 0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3))). */
float orc_gelu(float u) {
  double x = (double)u;
  double c = sqrt(2.0 / 3.14159265358979323846);
  double a = (g_mut == 2) ? c * x : c * (x + 0.044715 * x * x * x);
  if (g_mut == 1) {
    /* the overflow-prone evaluation of tanh in float, no clamp */
    float af = (float)a;
    float e = expf(2.0f * af);
    float t = (e - 1.0f) / (e + 1.0f);
    return (float)(0.5 * x * (1.0 + (double)t));
  }
  if (a > 15.0) a = 15.0;
  if (a < -15.0) a = -15.0;
  return (float)(0.5 * x * (1.0 + tanh(a)));
}

/* [RVM] "What the kernels do": silu(gate) * up; silu(z) = z / (1 + e^-z). */
float orc_silu(float z) {
  double x = (double)z;
  return (float)(x / (1.0 + exp(-x)));
}

/* [BML] "What got built" (softmax); [RVM] "Things that were problematic": masked scores
 * are -inf and exp(-inf) is exactly 0. Max-subtracted for range safety. */
void orc_softmax(const float* s, int n, float* p) {
  double m = -INFINITY;
  for (int i = 0; i < n; ++i)
    if ((double)s[i] > m) m = (double)s[i];
  double sum = 0.0;
  for (int i = 0; i < n; ++i) sum += exp((double)s[i] - m);
  for (int i = 0; i < n; ++i) p[i] = (float)(exp((double)s[i] - m) / sum);
}

/* [RVM] "The matmul pain story": a linear layer is y = x . W^T with W stored [out][in]. */
void orc_linear(const float* x, const float* W, const float* b, int n_out, int n_in, float* y) {
  for (int o = 0; o < n_out; ++o) {
    const float* row = W + (size_t)o * n_in;
    double acc = 0.0;
    for (int i = 0; i < n_in; ++i) acc += (double)x[i] * (double)row[i];
    if (b && g_mut != 10) acc += (double)b[o];
    y[o] = (float)acc;
  }
}

/* One query against T cached rows. [BML] "What got built" (KV-cached causal attention):
 * the new token attends to every cached position, itself included. The scale 1/sqrt(hd)
 * is the standard scaled dot product (not printed on the pages). */
void orc_attend(const float* q, const float* K, const float* V, int T, int hd, int ld, float* o) {
  double scale = (g_mut == 4) ? 1.0 / hd : 1.0 / sqrt((double)hd);
  float* s = (float*)malloc(sizeof(float) * (size_t)(T > 0 ? T : 1));
  float* p = (float*)malloc(sizeof(float) * (size_t)(T > 0 ? T : 1));
  for (int j = 0; j < T; ++j) {
    double acc = 0.0;
    for (int i = 0; i < hd; ++i) acc += (double)q[i] * (double)K[(size_t)j * ld + i];
    s[j] = (float)(acc * scale);
  }
  orc_softmax(s, T, p);
  for (int i = 0; i < hd; ++i) {
    double acc = 0.0;
    for (int j = 0; j < T; ++j) acc += (double)p[j] * (double)V[(size_t)j * ld + i];
    o[i] = (float)acc;
  }
  free(s);
  free(p);
}

/* [BF] status table (rope); [RVM] "What the kernels do": RoPE rotates q and k by their
 * position, one pair of numbers at a time. Reading: rotate-half pairing (i, i + hd/2)
 * with angle pos * theta^(-2i/hd), angle evaluated in double. */
void orc_rope(float* v, int hd, int pos, double theta) {
  int h = hd / 2;
  for (int i = 0; i < h; ++i) {
    double ang = (double)pos * pow(theta, -2.0 * (double)i / (double)hd);
    if (g_mut == 6) ang = -ang;
    double c = cos(ang), s = sin(ang);
    double a = (double)v[i], b = (double)v[i + h];
    v[i] = (float)(a * c - b * s);
    v[i + h] = (float)(a * s + b * c);
  }
}

/* [RVM] "What the kernels do": GPU argmax returns one integer per sequence; "How I know
 * it's correct": argmax is tested with ties and NaN. Reading: NaN is larger than every
 * number (first NaN wins); ties go to the lowest index. */
int orc_argmax(const float* v, int n) {
  int best = 0;
  for (int i = 1; i < n; ++i) {
    float a = v[i], b = v[best];
    if (isnan(b)) continue;
    if (isnan(a)) { best = i; continue; }
    if (a > b || (g_mut == 8 && a == b)) best = i;
  }
  return n > 0 ? best : -1;
}

/* bfloat16 keeps the top 16 bits of a float. Rounding to nearest, ties to even, on the
 * bit pattern: add 0x7fff plus the lowest kept bit, then clear the low 16 bits (the
 * carry may round up into the exponent, which is the correct result up to infinity).
 * [RVM] "What's basic about it" names the F32 KV cache as the basic choice; the
 * 16-bit cache is the reading of the half-size KV step. */
float orc_round_bf16(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return x;   /* NaN */
  if (g_mut == 11) u &= 0xffff0000u;
  else u = (u + 0x7fffu + ((u >> 16) & 1u)) & 0xffff0000u;
  float y;
  memcpy(&y, &u, 4);
  return y;
}

/* 8-bit blocks as in the Q8_0 format [RVM] names ("What's basic about it": one byte
 * per weight; [BF] status table: int8 dequantization): per block of 32 values, the
 * scale d = max|x| / 127 and q = round(x / d), evaluated as x * (1 / d) in float and
 * rounded half away from zero; d is kept as a float. */
void orc_quantize_q8(const float* x, int n, signed char* q, float* d) {
  for (int b = 0; b < n / 32; ++b) {
    const float* xb = x + 32 * b;
    float amax = 0.0f;
    for (int i = 0; i < 32; ++i) {
      float a = fabsf(xb[i]);
      if (a > amax) amax = a;
    }
    float db = amax / (g_mut == 13 ? 128.0f : 127.0f);
    float id = db != 0.0f ? 1.0f / db : 0.0f;
    for (int i = 0; i < 32; ++i) {
      float t = xb[i] * id;
      float r = (g_mut == 12) ? truncf(t) : roundf(t);
      q[32 * b + i] = (signed char)r;
    }
    d[b] = db;
  }
}

/* Philox4x64-10 (Salmon, Moraes, Dror, Shaw: "Parallel random numbers: as easy as 1, 2,
 * 3", SC 2011): ten rounds of two 64 x 64 -> 128-bit products of counter words with
 * the round multipliers, the high halves xored with the other counter words and the
 * key, the key advanced by the Weyl increments after each round. */
void orc_philox4x64(const unsigned long long ctr[4], const unsigned long long key[2], unsigned long long out[4]) {
  const unsigned long long M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const unsigned long long W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
  unsigned long long c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3], k0 = key[0], k1 = key[1];
  for (int r = 0; r < 10; ++r) {
    unsigned __int128 p0 = (unsigned __int128)M0 * c0, p1 = (unsigned __int128)M1 * c2;
    unsigned long long hi0 = (unsigned long long)(p0 >> 64), lo0 = (unsigned long long)p0;
    unsigned long long hi1 = (unsigned long long)(p1 >> 64), lo1 = (unsigned long long)p1;
    c0 = hi1 ^ c1 ^ k0;
    c1 = lo1;
    c2 = hi0 ^ c3 ^ k1;
    c3 = lo0;
    k0 += W0;
    k1 += W1;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

double orc_uniform(unsigned long long seed, int seq, int pos) {
  unsigned long long ctr[4] = {(unsigned long long)pos, (unsigned long long)seq, 0, 0}, key[2] = {seed, 0};
  unsigned long long out[4];
  orc_philox4x64(ctr, key, out);
  return (double)(out[0] >> 40) * (1.0 / 16777216.0);
}

static const float* g_sort_keys;
/* descending logit, ties to the lower index */
static int by_logit_desc(const void* a, const void* b) {
  int i = *(const int*)a, j = *(const int*)b;
  float x = g_sort_keys[i], y = g_sort_keys[j];
  if (x > y) return -1;
  if (x < y) return 1;
  return i < j ? -1 : (i > j);
}

/* [BF] status table: sampling by greedy, temperature and top-k ("--temperature 0.7" in
 * its demo). The pages print no rule; the reading: keep the top_k largest logits
 * (ties to the lower index), weight them by exp((l - l_max) / temperature) and return
 * the first candidate, in that order, whose cumulative weight exceeds u times the
 * total. */
int orc_sample(const float* logits, int n, double temperature, int top_k, double u) {
  if (n <= 0) return -1;
  for (int i = 0; i < n; ++i)
    if (isnan(logits[i])) return i;
  if (temperature <= 0.0 || top_k == 1) return orc_argmax(logits, n);
  int k = (top_k <= 0 || top_k > n) ? n : top_k;
  if (g_mut == 15 && k < n) k += 1;
  int* idx = (int*)malloc(sizeof(int) * (size_t)n);
  for (int i = 0; i < n; ++i) idx[i] = i;
  g_sort_keys = logits;
  qsort(idx, (size_t)n, sizeof(int), by_logit_desc);
  double t = (g_mut == 14) ? 1.0 : temperature;
  double top = (double)logits[idx[0]];
  double* w = (double*)malloc(sizeof(double) * (size_t)k);
  double total = 0.0;
  for (int r = 0; r < k; ++r) {
    w[r] = exp(((double)logits[idx[r]] - top) / t);
    total += w[r];
  }
  double target = u * total, cum = 0.0;
  int pick = idx[k - 1];
  for (int r = 0; r < k; ++r) {
    cum += w[r];
    if (target < cum) { pick = idx[r]; break; }
  }
  free(w);
  free(idx);
  return pick;
}

/* ---------------------------------------------------------- layer tensors */

typedef struct {
  const float *ln1_g, *ln1_b, *w_qkv, *b_qkv, *w_o, *b_o, *ln2_g, *ln2_b, *w_fc, *b_fc, *w_proj, *b_proj;
} gpt2_layer;

typedef struct {
  const float *rms1, *w_q, *w_k, *w_v, *w_o, *rms2, *w_gate, *w_up, *w_down;
} llama_layer;

static gpt2_layer gpt2_at(const orc_model* m, int l) {
  const orc_config* c = &m->c;
  size_t d = (size_t)c->d_model, ff = (size_t)c->d_ff;
  const float* p = m->w + m->layer[l];
  gpt2_layer t;
  t.ln1_g = p; p += d;
  t.ln1_b = p; p += d;
  t.w_qkv = p; p += 3 * d * d;
  t.b_qkv = p; p += 3 * d;
  t.w_o = p; p += d * d;
  t.b_o = p; p += d;
  t.ln2_g = p; p += d;
  t.ln2_b = p; p += d;
  t.w_fc = p; p += ff * d;
  t.b_fc = p; p += ff;
  t.w_proj = p; p += d * ff;
  t.b_proj = p;
  return t;
}

static llama_layer llama_at(const orc_model* m, int l) {
  const orc_config* c = &m->c;
  size_t d = (size_t)c->d_model, ff = (size_t)c->d_ff;
  size_t hq = (size_t)c->n_head * c->head_dim, hk = (size_t)c->n_kv_head * c->head_dim;
  const float* p = m->w + m->layer[l];
  llama_layer t;
  t.rms1 = p; p += d;
  t.w_q = p; p += hq * d;
  t.w_k = p; p += hk * d;
  t.w_v = p; p += hk * d;
  t.w_o = p; p += d * hq;
  t.rms2 = p; p += d;
  t.w_gate = p; p += ff * d;
  t.w_up = p; p += ff * d;
  t.w_down = p;
  return t;
}

static int kv_head_of(const orc_config* c, int h) {
  int group = c->n_head / c->n_kv_head;
  if (g_mut == 7) return h % c->n_kv_head;
  return h / group;
}

/* Final norm and logits. GPT-2: LayerNorm then the tied embedding ([BML] "What got
 * built": the transposed linear for tied embeddings). Llama: RMSNorm then the untied
 * head ([RVM] "What the kernels do": final norm and output projection). */
static void head_logits(const orc_model* m, const float* x, float* logits) {
  const orc_config* c = &m->c;
  int d = c->d_model;
  float* h = (float*)malloc(sizeof(float) * (size_t)d);
  if (c->arch == ORC_ARCH_GPT2) {
    orc_layernorm(x, m->w + m->lnf_g, m->w + m->lnf_b, d, c->norm_eps, h);
    orc_linear(h, m->w + m->wte, NULL, c->vocab, d, logits);
  } else {
    orc_rmsnorm(x, m->w + m->rmsf, d, c->norm_eps, h);
    orc_linear(h, m->w + m->w_head, NULL, c->vocab, d, logits);
  }
  free(h);
}

/* --------------------------------------------------- KV-cached forward step */

int orc_forward(const orc_model* m, orc_seq* s, int token, float* logits_out) {
  const orc_config* c = &m->c;
  if (token < 0 || token >= c->vocab) return -1;
  int p = s->len;
  if (p >= s->cap) return -2;
  if (c->arch == ORC_ARCH_GPT2 && p >= c->n_ctx) return -2;
  int d = c->d_model, hd = c->head_dim, H = c->n_head, Hk = c->n_kv_head, ff = c->d_ff;
  int qdim = H * hd, kdim = Hk * hd;
  float* x = (float*)malloc(sizeof(float) * (size_t)d);
  float* a = (float*)malloc(sizeof(float) * (size_t)d);
  float* qkv = (float*)malloc(sizeof(float) * (size_t)(qdim + 2 * kdim));
  float* o = (float*)malloc(sizeof(float) * (size_t)qdim);
  float* t = (float*)malloc(sizeof(float) * (size_t)d);
  float* u = (float*)malloc(sizeof(float) * (size_t)ff);
  float* g = (float*)malloc(sizeof(float) * (size_t)ff);
  float* logits = logits_out ? logits_out : (float*)malloc(sizeof(float) * (size_t)c->vocab);

  /* embedding: [BML] "Picking the model" (learned position embeddings for GPT-2) */
  const float* e = m->w + m->wte + (size_t)token * d;
  if (c->arch == ORC_ARCH_GPT2) {
    const float* pe = m->w + m->wpe + (size_t)p * d;
    for (int i = 0; i < d; ++i) x[i] = e[i] + pe[i];
  } else {
    for (int i = 0; i < d; ++i) x[i] = e[i];
  }

  for (int l = 0; l < c->n_layer; ++l) {
    float* q = qkv;
    float* k = qkv + qdim;
    float* v = qkv + qdim + kdim;
    if (c->arch == ORC_ARCH_GPT2) {
      gpt2_layer w = gpt2_at(m, l);
      orc_layernorm(x, w.ln1_g, w.ln1_b, d, c->norm_eps, a);
      orc_linear(a, w.w_qkv, w.b_qkv, 3 * d, d, qkv);
    } else {
      llama_layer w = llama_at(m, l);
      orc_rmsnorm(x, w.rms1, d, c->norm_eps, a);
      orc_linear(a, w.w_q, NULL, qdim, d, q);
      orc_linear(a, w.w_k, NULL, kdim, d, k);
      orc_linear(a, w.w_v, NULL, kdim, d, v);
      for (int h = 0; h < H; ++h) orc_rope(q + h * hd, hd, p, c->rope_theta);
      for (int h = 0; h < Hk; ++h) orc_rope(k + h * hd, hd, p, c->rope_theta);
    }
    /* append this position's K and V: [BML] "What got built" (a real KV cache); with
     * kv_bf16 the cache holds them rounded to bfloat16 */
    for (int h = 0; h < Hk; ++h) {
      size_t base = (((size_t)l * Hk + h) * s->cap + p) * hd;
      for (int i = 0; i < hd; ++i) {
        float kk = k[h * hd + i], vv = v[h * hd + i];
        s->K[base + i] = c->kv_bf16 ? orc_round_bf16(kk) : kk;
        s->V[base + i] = c->kv_bf16 ? orc_round_bf16(vv) : vv;
      }
    }
    int T = (g_mut == 5) ? p : p + 1;
    for (int h = 0; h < H; ++h) {
      int kh = kv_head_of(c, h);
      size_t base = ((size_t)l * Hk + kh) * s->cap * hd;
      if (T > 0) {
        orc_attend(q + h * hd, s->K + base, s->V + base, T, hd, hd, o + h * hd);
      } else {
        for (int i = 0; i < hd; ++i) o[h * hd + i] = 0.0f;
      }
    }
    if (c->arch == ORC_ARCH_GPT2) {
      gpt2_layer w = gpt2_at(m, l);
      orc_linear(o, w.w_o, w.b_o, d, qdim, t);
      for (int i = 0; i < d; ++i) x[i] += t[i];
      orc_layernorm(x, w.ln2_g, w.ln2_b, d, c->norm_eps, a);
      orc_linear(a, w.w_fc, w.b_fc, ff, d, u);
      for (int j = 0; j < ff; ++j) u[j] = orc_gelu(u[j]);
      orc_linear(u, w.w_proj, w.b_proj, d, ff, t);
      for (int i = 0; i < d; ++i) x[i] += t[i];
    } else {
      llama_layer w = llama_at(m, l);
      orc_linear(o, w.w_o, NULL, d, qdim, t);
      for (int i = 0; i < d; ++i) x[i] += t[i];
      orc_rmsnorm(x, w.rms2, d, c->norm_eps, a);
      orc_linear(a, w.w_gate, NULL, ff, d, g);
      orc_linear(a, w.w_up, NULL, ff, d, u);
      for (int j = 0; j < ff; ++j) u[j] = (float)((double)orc_silu(g[j]) * (double)u[j]);
      orc_linear(u, w.w_down, NULL, d, ff, t);
      for (int i = 0; i < d; ++i) x[i] += t[i];
    }
  }
  s->len = p + 1;
  head_logits(m, x, logits);
  int best = orc_argmax(logits, c->vocab);
  free(x); free(a); free(qkv); free(o); free(t); free(u); free(g);
  if (!logits_out) free(logits);
  return best;
}

/* -------------------------------------------- stateless matrix-form forward */

/* The whole sequence recomputed at once ([BF] roadmap: each step recomputes the full
 * sequence; [BML] "What got built": stateless causal attention). Attention is written
 * in matrix form here: S = Q K^T / sqrt(hd) over all T x T pairs, an explicit -inf mask
 * above the diagonal, a row softmax, then P V. It shares the pinned component
 * functions (norms, linear, GELU, SiLU, RoPE) with the cached path, but none of its
 * cache or attention code. */
int orc_forward_stateless(const orc_model* m, const int* tokens, int T, float* logits) {
  const orc_config* c = &m->c;
  if (T <= 0) return -3;
  if (c->arch == ORC_ARCH_GPT2 && T > c->n_ctx) return -2;
  for (int i = 0; i < T; ++i)
    if (tokens[i] < 0 || tokens[i] >= c->vocab) return -1;
  int d = c->d_model, hd = c->head_dim, H = c->n_head, Hk = c->n_kv_head, ff = c->d_ff;
  int qdim = H * hd, kdim = Hk * hd, wq = qdim + 2 * kdim;
  float* X = (float*)malloc(sizeof(float) * (size_t)T * d);
  float* A = (float*)malloc(sizeof(float) * (size_t)T * d);
  float* QKV = (float*)malloc(sizeof(float) * (size_t)T * wq);
  float* O = (float*)malloc(sizeof(float) * (size_t)T * qdim);
  float* Tm = (float*)malloc(sizeof(float) * (size_t)d);
  float* U = (float*)malloc(sizeof(float) * (size_t)ff);
  float* G = (float*)malloc(sizeof(float) * (size_t)ff);
  float* S = (float*)malloc(sizeof(float) * (size_t)T * T);
  float* P = (float*)malloc(sizeof(float) * (size_t)T * T);

  for (int r = 0; r < T; ++r) {
    const float* e = m->w + m->wte + (size_t)tokens[r] * d;
    for (int i = 0; i < d; ++i) {
      float v = e[i];
      if (c->arch == ORC_ARCH_GPT2) v += m->w[m->wpe + (size_t)r * d + i];
      X[(size_t)r * d + i] = v;
    }
  }
  double scale = (g_mut == 4) ? 1.0 / hd : 1.0 / sqrt((double)hd);
  int group = H / Hk;
  for (int l = 0; l < c->n_layer; ++l) {
    for (int r = 0; r < T; ++r) {
      float* xr = X + (size_t)r * d;
      float* ar = A + (size_t)r * d;
      float* qr = QKV + (size_t)r * wq;
      if (c->arch == ORC_ARCH_GPT2) {
        gpt2_layer w = gpt2_at(m, l);
        orc_layernorm(xr, w.ln1_g, w.ln1_b, d, c->norm_eps, ar);
        orc_linear(ar, w.w_qkv, w.b_qkv, 3 * d, d, qr);
      } else {
        llama_layer w = llama_at(m, l);
        orc_rmsnorm(xr, w.rms1, d, c->norm_eps, ar);
        orc_linear(ar, w.w_q, NULL, qdim, d, qr);
        orc_linear(ar, w.w_k, NULL, kdim, d, qr + qdim);
        orc_linear(ar, w.w_v, NULL, kdim, d, qr + qdim + kdim);
        for (int h = 0; h < H; ++h) orc_rope(qr + h * hd, hd, r, c->rope_theta);
        for (int h = 0; h < Hk; ++h) orc_rope(qr + qdim + h * hd, hd, r, c->rope_theta);
      }
      /* the keys and values attention reads (bfloat16-rounded with kv_bf16) */
      if (c->kv_bf16)
        for (int i = qdim; i < wq; ++i) qr[i] = orc_round_bf16(qr[i]);
    }
    for (int h = 0; h < H; ++h) {
      int kh = (g_mut == 7) ? h % Hk : h / group;
      /* S = Q_h K_kh^T * scale with the causal mask */
      for (int i = 0; i < T; ++i) {
        for (int j = 0; j < T; ++j) {
          int masked = (g_mut == 9) ? (j > i + 1) : (j > i);
          if (masked) { S[(size_t)i * T + j] = -INFINITY; continue; }
          const float* qi = QKV + (size_t)i * wq + h * hd;
          const float* kj = QKV + (size_t)j * wq + qdim + kh * hd;
          double acc = 0.0;
          for (int t = 0; t < hd; ++t) acc += (double)qi[t] * (double)kj[t];
          S[(size_t)i * T + j] = (float)(acc * scale);
        }
        orc_softmax(S + (size_t)i * T, T, P + (size_t)i * T);
      }
      /* O_h = P V_kh */
      for (int i = 0; i < T; ++i) {
        for (int t = 0; t < hd; ++t) {
          double acc = 0.0;
          for (int j = 0; j < T; ++j)
            acc += (double)P[(size_t)i * T + j] * (double)QKV[(size_t)j * wq + qdim + kdim + kh * hd + t];
          O[(size_t)i * qdim + h * hd + t] = (float)acc;
        }
      }
    }
    for (int r = 0; r < T; ++r) {
      float* xr = X + (size_t)r * d;
      float* ar = A + (size_t)r * d;
      const float* orow = O + (size_t)r * qdim;
      if (c->arch == ORC_ARCH_GPT2) {
        gpt2_layer w = gpt2_at(m, l);
        orc_linear(orow, w.w_o, w.b_o, d, qdim, Tm);
        for (int i = 0; i < d; ++i) xr[i] += Tm[i];
        orc_layernorm(xr, w.ln2_g, w.ln2_b, d, c->norm_eps, ar);
        orc_linear(ar, w.w_fc, w.b_fc, ff, d, U);
        for (int j = 0; j < ff; ++j) U[j] = orc_gelu(U[j]);
        orc_linear(U, w.w_proj, w.b_proj, d, ff, Tm);
        for (int i = 0; i < d; ++i) xr[i] += Tm[i];
      } else {
        llama_layer w = llama_at(m, l);
        orc_linear(orow, w.w_o, NULL, d, qdim, Tm);
        for (int i = 0; i < d; ++i) xr[i] += Tm[i];
        orc_rmsnorm(xr, w.rms2, d, c->norm_eps, ar);
        orc_linear(ar, w.w_gate, NULL, ff, d, G);
        orc_linear(ar, w.w_up, NULL, ff, d, U);
        for (int j = 0; j < ff; ++j) U[j] = (float)((double)orc_silu(G[j]) * (double)U[j]);
        orc_linear(U, w.w_down, NULL, d, ff, Tm);
        for (int i = 0; i < d; ++i) xr[i] += Tm[i];
      }
    }
  }
  for (int r = 0; r < T; ++r) head_logits(m, X + (size_t)r * d, logits + (size_t)r * c->vocab);
  free(X); free(A); free(QKV); free(O); free(Tm); free(U); free(G); free(S); free(P);
  return 0;
}
