/*
 * gd.h -- C ABI of the MI355X (gfx950) KV-cached transformer decode library.
 *
 * One library, libgptdecode.so, runs the decode forward pass of a GPT-2-style
 * decoder (LayerNorm, fused QKV with bias, causal multi-head attention against a
 * KV cache, output projection, tanh-GELU MLP, residual adds, tied-embedding logits,
 * greedy argmax) and of a Llama-style variant (RMSNorm, RoPE, grouped-query
 * attention over a paged KV cache, SiLU-gated MLP, untied head). Every step of the
 * pass runs in the library's HIP kernels; there is no CPU fallback.
 *
 * Sources for what is computed:
 *   "bare-metal-llm" (GPT-2 on hand-written Metal kernels): "What got built" lists
 *   the kernels of the pass and the KV cache; "The bug worth telling" is the GELU
 *   overflow; "What it taught me" asks for one submission per forward pass.
 *   "batch_forge" README: the op set (layernorm, rmsnorm, rope, gelu with the tanh
 *   argument clamped to +-15, attention, tiled matmul) and resident weights.
 *   "rvllm Metal backend" post: "What the kernels do" (the Llama-style layer, the
 *   paged cache addressed as block = pos / B, slot = pos mod B, GPU argmax returning
 *   one integer per sequence); "Memory is shared" (never read a buffer the GPU is
 *   still writing); "Things that were problematic" (-inf masks, NaN-aware argmax,
 *   tests must not skip when a kernel fails to load).
 *
 * Conventions
 *   - Device memory is owned by the caller (e.g. PyTorch tensors). The library only
 *     borrows the pointers given to gd_bind_memory / gd_decode_step / gd_prefill;
 *     they must stay valid while the model uses them.
 *   - Calls enqueue work on the model's HIP stream and return without waiting,
 *     except gd_load_weights (waits) and gd_device_errors (waits). Read results on
 *     the host only after synchronizing that stream.
 *   - Errors: every call returns a gd_status; gd_last_error() gives a message for
 *     the calling thread. A HIP failure poisons the model: every later call on it
 *     returns GD_ERR_HIP. A model is not thread-safe.
 *   - Activations and accumulation are float32; the KV cache float32 or bfloat16
 *     (kv_dtype). Weight matrices are stored float32 or bfloat16 (weight_dtype); norm
 *     parameters and biases float32.
 */
#ifndef GD_H
#define GD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GD_OK = 0,
  GD_ERR_INVALID = -1,   /* bad argument, shape or token id */
  GD_ERR_NO_DEVICE = -2, /* no HIP device, or not a gfx950 device */
  GD_ERR_HIP = -3,       /* a HIP call or kernel launch failed; the model is poisoned */
  GD_ERR_OOM = -4,       /* bound memory too small */
  GD_ERR_CTX_FULL = -5,  /* a sequence has no room for another position */
  GD_ERR_STATE = -6      /* call out of order (e.g. memory not bound, weights not loaded) */
} gd_status;

#define GD_ARCH_GPT2 0  /* LayerNorm, learned positions, tanh-GELU MLP, biases, tied head */
#define GD_ARCH_LLAMA 1 /* RMSNorm, RoPE, GQA, SiLU-gated MLP, no biases, untied head */

#define GD_WEIGHT_F32 0
#define GD_WEIGHT_BF16 1
#define GD_WEIGHT_Q8 2 /* 8-bit blocks: every weight matrix quantized at gd_load_weights, per
                        * row and block of 32 inputs, as in the Q8_0 format (scale
                        * max|x| / 127 kept as float32, codes round(x / scale), half away
                        * from zero): one byte per weight plus 4 bytes per 32 ("rvllm Metal
                        * backend", "What's basic about it" and "What's next": Q8_0 weights
                        * as the decode speed-up; "batch_forge" README, status table: int8
                        * dequantization). The linear layers run on the VALU GEMV (launches
                        * of up to 4 rows); d_model, d_ff and n_head*head_dim must be
                        * multiples of 32 */

#define GD_KV_F32 0   /* the KV cache holds float32 */
#define GD_KV_BF16 1  /* K and V are rounded to bfloat16 (nearest, ties to even) as they enter
                       * the cache and widened to float32 when attention reads them: half the
                       * cache bytes ("rvllm Metal backend", "What's basic about it": the F32
                       * KV cache as the basic choice) */

typedef struct {
  int32_t arch;           /* GD_ARCH_* */
  int32_t n_layer, d_model, n_head, n_kv_head, head_dim, d_ff, vocab;   /* d_model, d_ff: multiples of 8, <= 2^20 */
  int32_t n_ctx;          /* positions per sequence (GPT-2: rows of the position table) */
  float norm_eps;         /* LayerNorm / RMSNorm epsilon */
  float rope_theta;       /* Llama only */
  int32_t weight_dtype;   /* GD_WEIGHT_* */
  int32_t max_seqs;       /* sequence slots 0 .. max_seqs-1 */
  int32_t max_batch;      /* rows of one decode step (<= 32) */
  int32_t kv_block_size;  /* 0: contiguous cache, n_ctx positions per slot; else paged */
  int32_t kv_num_blocks;  /* paged: blocks in the pool */
  int32_t kv_dtype;       /* GD_KV_* */
} gd_config;

typedef struct gd_model gd_model;

/* Checks the config and the device (must be gfx950) and binds `hip_stream`
 * (a hipStream_t; NULL = the null stream). Allocates no device memory except a few
 * bytes of HIP objects.
 * Defines: the model shapes this engine runs -- GPT-2 with LayerNorm, learned positions
 * and plain multi-head attention ("bare-metal-llm", "Picking the model") and the
 * Llama-style layer with RMSNorm, RoPE, grouped K/V heads and a gated MLP ("rvllm Metal
 * backend", "What the kernels do").
 * Errors: GD_ERR_INVALID for a bad config (nothing created); GD_ERR_NO_DEVICE when no
 * gfx950 device is present -- a backend that is asked for and missing is an error, never
 * a silent fallback ("batch_forge" README, the generate binary's usage notes). *out
 * is NULL on any error. */
gd_status gd_create(const gd_config* cfg, void* hip_stream, gd_model** out);

/* Bytes of device memory the caller must provide: packed weights, KV cache and
 * scratch (activations, attention partials, argmax partials, row metadata, block
 * tables). The weights stay resident in the first buffer for the model's life
 * ("batch_forge" README, roadmap: resident weights instead of a re-upload per call).
 * Errors: GD_ERR_INVALID if m is NULL; NULL size pointers are skipped. */
gd_status gd_memory_requirements(const gd_model* m, size_t* weights_bytes, size_t* kv_bytes,
                                 size_t* scratch_bytes);

/* Binds caller-owned device buffers of at least the required sizes (256-byte aligned).
 * Clears the scratch, the sequence lengths and (contiguous cache) installs identity
 * block tables; waits for that. The caller keeps ownership and must keep the buffers
 * alive while the model uses them ("rvllm Metal backend", "Memory is shared": buffers
 * are the caller's, read only after the GPU is done with them).
 * Errors: GD_ERR_INVALID (NULL or misaligned pointer), GD_ERR_HIP. Unloads any weights
 * loaded before (GD_ERR_STATE until gd_load_weights runs again). */
gd_status gd_bind_memory(gd_model* m, void* weights_dev, void* kv_dev, void* scratch_dev);

/* Uploads the weights from one host float32 buffer in the canonical order (resident
 * weights: "batch_forge" README, roadmap; the tied output head reads wte transposed:
 * "bare-metal-llm", "What got built"):
 *   GPT-2: wte[V][d], wpe[n_ctx][d], then per layer ln1_g[d], ln1_b[d],
 *          w_qkv[3d][d], b_qkv[3d], w_o[d][d], b_o[d], ln2_g[d], ln2_b[d],
 *          w_fc[ff][d], b_fc[ff], w_proj[d][ff], b_proj[d]; then lnf_g[d], lnf_b[d].
 *   Llama: wte[V][d], then per layer rms1[d], w_q[Hq*hd][d], w_k[Hkv*hd][d],
 *          w_v[Hkv*hd][d], w_o[d][Hq*hd], rms2[d], w_gate[ff][d], w_up[ff][d],
 *          w_down[d][ff]; then rmsf[d], w_head[V][d].
 * Matrices are [out][in] (y = x . W^T + b). With GD_WEIGHT_BF16 the matrices are
 * rounded to bfloat16 (nearest, ties to even); with GD_WEIGHT_Q8 quantized to 8-bit blocks
 * (see GD_WEIGHT_Q8). Repacks into the device layout and
 * waits for the copy. n_floats must equal the canonical count (else GD_ERR_INVALID);
 * GD_ERR_STATE before gd_bind_memory. The host buffer is only read during the call. */
gd_status gd_load_weights(gd_model* m, const float* host_weights, size_t n_floats);

/* Paged cache only: installs the block table of sequence slot `seq` (n entries,
 * each in [0, kv_num_blocks)). Position p of the sequence lives in block
 * blocks[p / kv_block_size], slot p mod kv_block_size ("rvllm Metal backend", "What the
 * kernels do": the paged cache addressed by integer division and modulo). Capacity =
 * min(n * block size, n_ctx). Errors: GD_ERR_STATE for a contiguous cache,
 * GD_ERR_INVALID for an entry out of range. The host array is copied before return. */
gd_status gd_set_block_table(gd_model* m, int32_t seq, const int32_t* blocks_host, int32_t n);

/* Empties sequence slot `seq` (length 0): the KV cache of a sequence holds only what
 * it has run ("bare-metal-llm", "What got built": a real KV cache, each step computes
 * only the new token). GD_ERR_INVALID for a slot out of range. */
gd_status gd_reset_seq(gd_model* m, int32_t seq);

/* Shortens sequence slot `seq` to `len` positions (0 <= len <= current length); the
 * positions past it are dropped and later overwritten (rewind, e.g. to replay a
 * generation from the end of its prompt, as the same KV cache of "bare-metal-llm",
 * "What got built"). GD_ERR_INVALID outside 0..length. */
gd_status gd_truncate_seq(gd_model* m, int32_t seq, int32_t len);

/* Host-side length of a sequence slot (positions filled, as enqueued; the device copy
 * is advanced by the decode step itself). GD_ERR_INVALID for a bad slot. */
gd_status gd_seq_len(const gd_model* m, int32_t seq, int32_t* len);

/* Runs tokens_host[0..n) of one sequence at positions len .. len+n-1 (causal within
 * the prompt), appends their K/V, and writes the greedy argmax of the last position
 * to *next_token_dev (device int32) and, if logits_dev is not NULL, its vocab logits
 * (device float[vocab]) ("rvllm Metal backend", "Numbers": the prompt is processed
 * before the first token; "bare-metal-llm", "What got built": the KV cache filled for
 * later steps). n >= 1 and every id in [0, vocab), else GD_ERR_INVALID; GD_ERR_CTX_FULL
 * past the slot's capacity. Enqueued, not waited for. */
gd_status gd_prefill(gd_model* m, int32_t seq, const int32_t* tokens_host, int32_t n,
                     int32_t* next_token_dev, float* logits_dev);

/* One decode step for `batch` sequences ("bare-metal-llm", "What got built" and "What
 * it taught me": one token per step against the KV cache, the whole forward pass in
 * one submission; "rvllm Metal backend", "What the kernels do": the GPU argmax returns
 * one integer per sequence). Row b runs token tokens_dev[b] (device int32)
 * of sequence seq_ids_host[b] at its current length, appends K/V, and writes
 * next_tokens_dev[b] (device int32) and, if logits_dev is not NULL, logits_dev[b][vocab].
 * seq ids must be distinct. tokens_dev may alias next_tokens_dev (greedy decode fed on
 * the device). The step is one hipGraph launch, captured on first use for each
 * (batch, pointers, short/long context) combination; the 16 most recently used graphs
 * are kept (an evicted graph costs one stream synchronization). Token ids produced on
 * the device are checked by the kernels: an out-of-range id sets a device error flag
 * (gd_device_errors) and is replaced by 0. Host-checked errors: GD_ERR_INVALID (batch,
 * ids), GD_ERR_STATE (an empty sequence), GD_ERR_CTX_FULL (a full one). */
gd_status gd_decode_step(gd_model* m, int32_t batch, const int32_t* seq_ids_host,
                         const int32_t* tokens_dev, int32_t* next_tokens_dev, float* logits_dev);

/* Temperature / top-k sampling instead of the greedy argmax for every later prefill
 * and decode step ("batch_forge" README, status table: greedy, temperature and top-k
 * sampling; its demo samples at temperature 0.7). The token after position p of
 * sequence slot s keeps the top_k largest logits (ties to the lower index), weights
 * them by exp((l - l_max) / temperature) in that order, and takes the first whose
 * cumulative weight exceeds u times the total, u being the top 24 bits of the first
 * word of Philox4x64-10 (counter (p, s, 0, 0), key (seed, 0)) times 2^-24; a NaN logit
 * gives the first NaN's index. temperature <= 0 or top_k == 1: greedy (the default).
 * Otherwise 2 <= top_k <= min(256, vocab) and vocab <= 65536, else GD_ERR_INVALID.
 * Drops the captured graphs; host-side only. */
gd_status gd_set_sampling(gd_model* m, float temperature, int32_t top_k, uint64_t seed);

/* Waits for the stream and returns the device error flags (bit 0: token id out of
 * range; bit 1: position beyond a sequence's capacity; bit 2: block table entry out
 * of range), then clears them. Waiting first is the rule of "rvllm Metal backend",
 * "Memory is shared": no buffer is read while the GPU may still write it. */
gd_status gd_device_errors(gd_model* m, int32_t* flags);

/* Tuning/testing switches (per shape, the pages' engines pick among kernel variants:
 * "bare-metal-llm", "What it taught me"; "rvllm Metal backend", "The matmul pain story").
 * GD_OPT_LINEAR_VARIANT: 0 auto (VALU GEMV for <= 4 rows, MFMA otherwise), 1 force VALU
 * GEMV, 2 force MFMA. GD_OPT_USE_GRAPH: 1 (default) capture decode steps in hipGraphs,
 * 0 launch kernels directly. Every call drops the captured graphs. GD_ERR_INVALID for
 * an unknown option or a value outside its set. */
#define GD_OPT_LINEAR_VARIANT 1
#define GD_OPT_USE_GRAPH 2
#define GD_OPT_FUSE_ATTN_O 4 /* 1 (default): attention runs fused with the output
                              * projection (+ bias + residual) when the projection is the
                              * VALU GEMV (up to 4 rows by default, any row count with
                              * GD_OPT_LINEAR_VARIANT = 1) and every context holds at most
                              * 256 positions, and for the one-chunk split-context case
                              * (GD_OPT_ATTN_CHUNKS) with a contiguous cache, head_dim 64,
                              * one query head per KV head and d_model <= 768; 0: attention
                              * and projection always run as separate launches */
#define GD_OPT_FOLD_NORM 7 /* 1 (default): with fp32 weights a layer behind a pre-norm
                           * (QKV, MLP up, head) reads copies of its weights with the
                           * norm's gain folded in (and the shift in its bias), made at
                           * gd_load_weights, and applies the row statistics in its
                           * epilogue; the tiled prompt pass applies its pre-norms inside
                           * the QKV and MLP-up GEMMs (LayerNorm through those folded
                           * copies, RMSNorm with any weights: gains applied as the rows
                           * are staged, the row scale in the epilogue). 0: the norm's
                           * gain and shift are applied to the rows first */
#define GD_OPT_ATTN_CHUNKS 9 /* context chunks per row of the split-context attention
                             * (rows that do not take the short-context fused attention):
                             * 1 (one workgroup per row and KV head over the whole context:
                             * normalized output written directly, or the output
                             * projection applied in the same launch, see
                             * GD_OPT_FUSE_ATTN_O) or 8 (partials merged by the output
                             * projection's prologue or a merge launch); 0 (default): 1
                             * when rows x KV heads >= the CU count and the output
                             * projection would be a matrix-core launch, 32 (merged by a
                             * launch of their own) when some row attends to 1024 or more
                             * positions and rows x KV heads x 8 < the CU count, else 8.
                             * Below that context length, when the output projection is
                             * the VALU GEMV (at most 4 rows, or any row count with
                             * GD_OPT_LINEAR_VARIANT = 1) the split-context attention
                             * always uses 8 (the GEMV's prologue merges them) */
#define GD_OPT_TILED_PREFILL 10 /* 1 (default): prompts of at least 64 tokens run the tiled
                                * prompt pass (512 rows at a time: 64 x 64 matrix-core GEMM
                                * tiles with the decode epilogues, tiled causal attention with
                                * K/V tiles in LDS) when the weights are float or bf16 and
                                * head_dim is 64; 0: every prompt runs the decode kernels over
                                * 32 rows at a time */
#define GD_OPT_PREFILL_BF16_PARTS 11 /* how the tiled prompt pass computes its GEMM
                                      * products. 1 (default): with bf16 weights on the
                                      * bf16 matrix cores, every fp32 activation split into
                                      * three bf16 parts (exact: three products per
                                      * weight); with fp32 weights the same for the GEMMs
                                      * not split in K (QKV and MLP up: the weights split
                                      * too, the six largest of the nine part products, the
                                      * dropped ones below 2^-24 of the product) and the
                                      * fp32 matrix cores for the split ones. 2: bf16 parts
                                      * for every fp32 GEMM. 0: fp32 matrix cores for all.
                                      * GD_ERR_INVALID for other values */
#define GD_OPT_PROFILE 3 /* launch eagerly and time every kernel with a HIP event pair.
                          * 1: as enqueued (host enqueue gaps fall inside short pairs);
                          * 2: each decode step waits behind a 3 ms hold on a helper
                          * stream while the host enqueues it whole, so its launches run
                          * back to back */
gd_status gd_set_option(gd_model* m, int32_t option, int32_t value);

/* Per-kernel profile gathered while GD_OPT_PROFILE is on ("rvllm Metal backend",
 * "The matmul pain story": GPU time summed per kernel). Waits for the stream
 * ("Memory is shared": read only after the GPU is done). One
 * entry per role (e.g. "linear.qkv", "attention"); `kernel` is the HIP kernel it ran;
 * `bytes` is the algorithmic traffic of those launches (every weight, bias and norm
 * parameter once, activations in and out, K/V of every attended position once).
 * Fills up to `max` entries, sets *n to the number of roles, and clears the profile
 * if reset != 0. */
typedef struct {
  char role[32];
  char kernel[64];
  int64_t launches;
  double total_us;
  double bytes;
} gd_kernel_stat;
gd_status gd_profile_read(gd_model* m, gd_kernel_stat* out, int32_t max, int32_t* n, int32_t reset);

/* Waits for the model's stream, releases its graphs, events and pinned staging; the
 * caller's device buffers are untouched. NULL is ignored. */
void gd_destroy(gd_model* m);
/* Message of the calling thread's last error (empty if none). A kernel that fails to
 * load or launch is reported as GD_ERR_HIP with this message and poisons the model --
 * a hard failure, never a quiet skip ("rvllm Metal backend", "Things that were
 * problematic"). The string is valid until the thread's next call. */
const char* gd_last_error(void);

/* ------------------------------------------------------------------ op level
 * Single kernels on caller buffers, for kernel tests and tools. All pointers are
 * device pointers; `hip_stream` is a hipStream_t (NULL = null stream). */

#define GD_NORM_NONE 0
#define GD_NORM_LAYER 1 /* (x - mean) / sqrt(var + eps) * g + b, biased variance */
#define GD_NORM_RMS 2   /* x / sqrt(mean(x^2) + eps) * g */
#define GD_ACT_NONE 0
#define GD_ACT_GELU 1   /* 0.5 u (1 + tanh(clamp(sqrt(2/pi)(u + 0.044715 u^3), -15, 15))) */

/* Workspace bytes gd_linear needs for (M, N, K) with the given variant.
 * GD_ERR_INVALID for shapes gd_linear refuses. */
gd_status gd_linear_workspace(int32_t M, int32_t N, int32_t K, int32_t variant, size_t* bytes);

/* One linear layer y = x . W^T with W stored [out][in] ("rvllm Metal backend", "The
 * matmul pain story"), with its pre-norm and epilogue ("batch_forge" README: layernorm,
 * rmsnorm and gelu with the tanh argument clamped to +-15):
 * y[m][n] = act(norm(x[m]) . W[n]^T + bias[n]) (+ resid[m][n]) for m < M, n < N.
 * x: float [M][ldx] (K used); W: [N][K] float32 or bf16 bits (weight_dtype); bias,
 * norm_g, norm_b: float or NULL; resid: float [M][ldr] or NULL; y: float [M][ldy].
 * 1 <= M <= 32, N >= 1, 8 <= K <= 2^20 and K % 8 == 0; W must be 16-byte aligned.
 * variant: 0 auto, 1 VALU GEMV, 2 MFMA. workspace: gd_linear_workspace bytes, zeroed
 * once before first use. Its first part (a zero vector) is never written; the rest
 * receives, on each call that runs the MFMA kernel, the tile-major copy of W that
 * kernel reads, so calls sharing one workspace must not overlap. */
gd_status gd_linear(const float* x, int32_t ldx, const void* W, int32_t weight_dtype,
                    const float* bias, int32_t norm, const float* norm_g, const float* norm_b,
                    float eps, int32_t act, const float* resid, int32_t ldr, float* y, int32_t ldy,
                    int32_t M, int32_t N, int32_t K, int32_t variant, void* workspace,
                    size_t workspace_bytes, void* hip_stream);

/* Greedy argmax of each row of logits [rows][vocab] (device) into out[rows] (device
 * int32), on the GPU so that one integer per row comes back ("rvllm Metal backend",
 * "What the kernels do"). NaN is larger than every number (first NaN wins; the
 * argmax is defined by its NaN handling: "Things that were problematic"); ties go to
 * the lowest index. 1 <= rows <= 32, else GD_ERR_INVALID. workspace:
 * gd_argmax_workspace bytes, zeroed once; calls sharing one workspace must not overlap. */
gd_status gd_argmax_workspace(int32_t rows, int32_t vocab, size_t* bytes);
gd_status gd_argmax(const float* logits, int32_t rows, int32_t vocab, int32_t* out, void* workspace,
                    size_t workspace_bytes, void* hip_stream);

/* gd_argmax without a workspace, for callers that cannot allocate device memory
 * (code under stream capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same result as gd_argmax. Its partials and counters live in a static device array
 * of the library (64 KiB per GPU, kept until the process ends), so it allocates
 * nothing: 1 <= rows <= 32 and 1 <= vocab <= 2^20, else GD_ERR_INVALID. Every call on
 * one GPU shares that array: calls that overlap on one GPU (other streams or threads)
 * race and must not be issued. Enqueued on hip_stream of the current device. */
gd_status gd_argmax_static(const float* logits, int32_t rows, int32_t vocab, int32_t* out, void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif
