/*
 * oracle.h -- plain, slow, single-threaded CPU reference of the KV-cached decode
 * forward pass of a GPT-2-style decoder (and of the Llama-style variant).
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library may include, link or
 * call this code; only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark use it. It shares no code with the GPU path.
 *
 * What is computed (pages: "bare-metal-llm", section "What got built"; "batch_forge",
 * component status table; "rvllm Metal post", section "What the kernels do"):
 *   GPT-2 style: x = wte[t] + wpe[p]; per layer pre-LayerNorm attention block and
 *   pre-LayerNorm tanh-GELU MLP block with residual adds; final LayerNorm; logits
 *   through the tied embedding; greedy argmax.
 *   Llama style: x = wte[t]; per layer RMSNorm, Q/K/V projections, RoPE on q and k,
 *   grouped-query attention, output projection, residual, RMSNorm, SiLU-gated MLP,
 *   residual; final RMSNorm; untied output head; greedy argmax.
 *
 * Numerics: every tensor is float32; each reduction (dot products, norm moments,
 * softmax sums, attention sums) is accumulated in double in index order and rounded
 * to float once; nonlinear functions are evaluated in double on the float input and
 * rounded once.
 *
 * Weights: one packed float32 buffer in the canonical order documented in
 * synth/__init__.py (GPT-2: wte, wpe, per layer ln1_g ln1_b w_qkv b_qkv w_o b_o
 * ln2_g ln2_b w_fc b_fc w_proj b_proj, then lnf_g lnf_b; Llama: wte, per layer
 * rms1 w_q w_k w_v w_o rms2 w_gate w_up w_down, then rmsf w_head). Matrices are
 * [out][in], so a linear layer is y = x . W^T + b. The buffer is borrowed: it must
 * outlive the model.
 */
#ifndef GD_ORACLE_H
#define GD_ORACLE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORC_ARCH_GPT2 0
#define ORC_ARCH_LLAMA 1

typedef struct {
  int arch;
  int n_layer, d_model, n_head, n_kv_head, head_dim, d_ff, vocab, n_ctx;
  double norm_eps;
  double rope_theta;
  int kv_bf16;    /* 1: K and V are rounded to bfloat16 (nearest, ties to even) as they
                   * enter the cache; attention reads the rounded values */
  int weight_q8;  /* 1: every weight matrix is replaced by its 8-bit block quantization
                   * (orc_quantize_q8 on each row's blocks of 32), dequantized to float */
} orc_config;

typedef struct orc_model orc_model;
typedef struct orc_seq orc_seq;

/* Number of floats in the packed canonical weight buffer; 0 for an invalid config. */
size_t orc_weight_count(const orc_config* cfg);

/* Returns NULL if cfg is invalid or n != orc_weight_count(cfg). */
orc_model* orc_model_create(const orc_config* cfg, const float* weights, size_t n);
void orc_model_free(orc_model* m);

/* A sequence's KV cache (positions 0 .. capacity-1). */
orc_seq* orc_seq_create(const orc_model* m, int capacity);
void orc_seq_free(orc_seq* s);
int orc_seq_len(const orc_seq* s);

/* One KV-cached forward step of `token` at position orc_seq_len(s); appends its K/V.
 * Writes the vocab logits if `logits` is not NULL. Returns the greedy argmax, or
 * -1 for a token out of range, -2 when the sequence is full. */
int orc_forward(const orc_model* m, orc_seq* s, int token, float* logits);

/* Stateless matrix form over tokens[0..T): full T x T scores with an explicit -inf
 * causal mask. Writes logits [T][vocab] (every row). Returns 0, or <0 on bad input. */
int orc_forward_stateless(const orc_model* m, const int* tokens, int T, float* logits);

/* First index of the maximum; NaN counts as larger than every number (first NaN wins);
 * ties go to the lowest index. */
int orc_argmax(const float* v, int n);

/* Components (also the building blocks of the forward passes above). */
void orc_layernorm(const float* x, const float* g, const float* b, int n, double eps, float* y);
void orc_rmsnorm(const float* x, const float* w, int n, double eps, float* y);
float orc_gelu(float u);
float orc_silu(float z);
void orc_softmax(const float* s, int n, float* p);
void orc_linear(const float* x, const float* W, const float* b, int n_out, int n_in, float* y);
/* One query row against T cached rows (row stride `ld` floats): o = softmax(q.K^T/sqrt(hd)) V */
void orc_attend(const float* q, const float* K, const float* V, int T, int hd, int ld, float* o);
/* Rotate-half RoPE of one head vector v[hd] at position pos (pairs i, i + hd/2). */
void orc_rope(float* v, int hd, int pos, double theta);

/* bfloat16 rounding of a float (nearest, ties to even; NaN stays NaN), returned as float. */
float orc_round_bf16(float x);

/* 8-bit block quantization of n values (n a multiple of 32), blocks of 32: scale
 * d = max|x| / 127, q = round-half-away(x / d) in [-127, 127] (x * (1/d) in float),
 * d = 0 and q = 0 for an all-zero block. Writes q[n] and d[n / 32]. */
void orc_quantize_q8(const float* x, int n, signed char* q, float* d);

/* Philox4x64-10 block of counter ctr[4] and key key[2] into out[4]. */
void orc_philox4x64(const unsigned long long ctr[4], const unsigned long long key[2], unsigned long long out[4]);

/* The uniform number in [0, 1) that drives sampling of the token after position pos of
 * sequence slot seq: the top 24 bits of the first word of Philox4x64-10 with counter
 * (pos, seq, 0, 0) and key (seed, 0), times 2^-24. */
double orc_uniform(unsigned long long seed, int seq, int pos);

/* Temperature / top-k sampling of one row of logits with the uniform u: the top_k
 * largest logits (ties to the lower index; top_k <= 0 or > n: all), weights
 * exp((l - l_max) / temperature), the first candidate in that order whose cumulative
 * weight exceeds u times the total. temperature <= 0 or top_k == 1: the greedy argmax.
 * A NaN among the logits gives the first NaN's index. */
int orc_sample(const float* logits, int n, double temperature, int top_k, double u);

/* Planted mistakes for mutation tests of the pins (0 = none). See oracle.c. */
void orc_set_mutation(int m);

#ifdef __cplusplus
}
#endif
#endif
