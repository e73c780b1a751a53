// linear.h -- y = epilogue(prologue(x) . W^T) for 1..32 activation rows.
//
// A linear layer is y = x . W^T with W stored [out][in] ("rvllm Metal backend",
// "The matmul pain story"). One decode step streams every weight once and does
// little arithmetic per byte, so both kernels are built around streaming W with
// 16-byte loads issued before anything that depends on the activations.
//
// No workgroup waits for another inside a launch: an agent-scope release costs tens
// of microseconds per launch here (each workgroup's release writes back its XCD's
// L2), so there are no last-arriver reductions. The only cross-workgroup sums are
// the matrix-core kernel's split-K float atomics into an in-place residual, which
// only the next launch reads.
//
// k_gemv (1..4 rows, VALU): each wave owns RW weight rows; lane l holds chunks
//   c = l + 64 i (16 bytes each: 4 fp32 or 8 bf16 weights) of each row in registers,
//   loaded first. Meanwhile the workgroup stages the activation rows in LDS through a
//   prologue (a copy, the merge of split-context attention partials, or, in the first
//   QKV launch of a decode step, the rows' input embeddings formed from the step's
//   tokens and positions, so that the step needs no set-up launch). A pre-norm
//   (LayerNorm or RMSNorm) is taken per wave in registers, either applied to the row
//   (gain and shift loaded) or folded into the weights (see NRM_FOLDED). Dot products
//   are reduced across the wave.
// k_mm (5..32 rows): matrix-core tiles of 16 columns (fp32 products, or exact bf16
//   parts where a workgroup streams several tiles), activation rows held in registers in
//   the MFMA operand layout; its prologue copies the rows or (output projection, up to 16
//   rows) merges the split-context attention partials into them; see the MFMA section
//   below.
//
// Epilogues: bias, clamped tanh-GELU, residual add; SiLU-gated pairs (gate and up
// rows interleaved, gate at even rows); QKV scatter (q to a buffer, k and v into the
// KV cache at the row's (sequence, position), with rotate-half RoPE for the Llama
// layout whose q/k rows are packed as adjacent (i, i + hd/2) pairs); greedy argmax
// partials per workgroup (reduced by k_argmax_finalize).
#pragma once
#include "common.h"
#include "attention.h"
#include "misc.h"

// Source of the activation rows.
#define PRO_COPY 0    // x rows as given
#define PRO_ATTN 3    // merge of split-context attention partials
#define PRO_EMBED 4   // the decode rows' input embeddings (k_gemv, QKV: the step's set-up folded in)
// Row normalization applied after the source (LinParams::norm).
#define NORM_NONE 0
#define NORM_LN 1    // (x - mean) / sqrt(var + eps) * g + b, biased variance
#define NORM_RMS 2   // x / sqrt(mean(x^2) + eps) * g

// How k_gemv applies a pre-norm.
#define NRM_NONE 0
#define NRM_EXPLICIT 1   // gain and shift loaded and applied to the row
#define NRM_FOLDED 2     // gain and shift folded into W, bias and row sums (LinParams::fs)

// Epilogues (a template parameter of the kernels, so that the loads of their
// operands compile to straight-line code).
#define EPI_PLAIN 0     // y = v + bias + resid
#define EPI_GELU 1      // y = gelu(v + bias) + resid
#define EPI_SWIGLU 2    // y[n / 2] = silu(v_n) * v_(n+1): gate rows even, up rows odd
#define EPI_ARGMAX 3    // logits (optional) and per-workgroup greedy argmax partials
#define EPI_QKV 4       // q to y, k and v into the cache slot, + bias
#define EPI_QKV_ROPE 5  // as EPI_QKV with rotate-half RoPE on adjacent (q, k) row pairs

#define GEMV_MAX_ROWS 4

struct LinParams {
  // ---- input rows
  int pro, norm;
  const float* x; int ldx;                  // COPY (and MFMA input)
  const float* ng; const float* nb; float eps;
  const float* apart; int Hq, nch;          // ATTN: partials [M][Hq][nch][gd_apart_stride(hd)] (k_gemv: nch = GD_ATT_NCH)
  int* err;
  const long long* row_kvoff;               // element offset of each row's K/V slot in a layer pool (-1: none)
  // ---- weights
  const void* w; int M, N, K;               // [N][K] row-major (VALU kernel)
  const float* wsc;                         // 8-bit weights: the block scales [N][K / 32]
  const void* wtl;                          // the same, tile-major (matrix-core kernel; see k_pack_tiles)
  // ---- the pre-norm folded into the layer (fp32 weights; NULL: not available). With
  // LN(x)_k = (x_k - mu) r g_k + b_k the layer is y_n = r sum_k (x_k - mu) g_k W_nk +
  // (bias_n + sum_k b_k W_nk): wf holds g_k W_nk, bf the bracket, fs the row sums of wf.
  const void* wf; const float* bf; const float* fs;
  const void* wfl;                          // wf, tile-major (matrix-core kernel)
  // ---- epilogue
  int epi;
  const float* bias;                        // never NULL: a zero vector when the layer has none
  const float* resid; int ldr;              // never NULL for PLAIN/GELU: zeros with ldr = 0 when none
  float* y; int ldy;
  float* am_val; int* am_idx;               // [gridDim.x][M]
  float* logits; int ldl;
  int qdim, kdim, hd, kv_hstride;           // QKV: head g of a slot at + g * kv_hstride
  const float* rope_cs;                     // [M][hd]: each row's cos | sin of pair i (NULL: no RoPE)
  void* kc; void* vc;                       // K / V pools of the layer: float, or bf16 bits if kv16
  int kv16;
};

// The embedding prologue's sources (PRO_EMBED): row b < M is token tok[b] of sequence
// slot sids[b] at that sequence's length len[.], as k_setup_decode takes it; erp
// addresses the tables, the cache's block table and the rows' metadata that workgroup
// 0 stores. A kernel argument type of its own, so that every other launch keeps the
// smaller argument block of LinParams.
struct EmbSrc {
  RowParams erp;
  const int* sids; const int* tok; const int* len; const int* cap;
};
struct LinEmbParams : LinParams {
  EmbSrc e;
};
// Every linear launch passes a LinParams by value, and the matrix-core kernels read
// hidden arguments placed after it: with the embedding sources inside LinParams their
// argument blocks grew from 536 to 744 bytes and the batched steps measured 0.8-0.9 %
// slower, so it stays this size.
static_assert(sizeof(LinParams) <= 280, "LinParams: keep the launch argument block small");
template <int PRO>
struct GemvArgs { typedef LinParams T; };
template <>
struct GemvArgs<PRO_EMBED> { typedef LinEmbParams T; };

// ------------------------------------------------------------ shared pieces

// Stores QKV output column n of row m: q columns go to y, k and v columns into this
// layer's cache slot of the row (nothing if the slot is invalid), as float or, with a
// bf16 cache, rounded to bf16.
__device__ __forceinline__ void qkv_store(const LinParams& p, int m, int n, long long kvoff, float v) {
  if (n < p.qdim) { p.y[(size_t)m * p.ldy + n] = v; return; }
  if (kvoff < 0) return;
  int kn = n - p.qdim;
  void* base = p.kc;
  if (kn >= p.kdim) { kn -= p.kdim; base = p.vc; }
  const int g = kn / p.hd, d = kn - g * p.hd;
  const size_t e = (size_t)kvoff + (size_t)g * p.kv_hstride + d;
  if (p.kv16) reinterpret_cast<uint16_t*>(base)[e] = bf16_rne(v);
  else reinterpret_cast<float*>(base)[e] = v;
}

template <int EPI>
struct EpiTraits { static constexpr bool pair = EPI == EPI_SWIGLU || EPI == EPI_QKV_ROPE; };

// Epilogue operands of one output column n (or adjacent pair n, n + 1) of row m. They
// are plain loads whose addresses depend only on kernel arguments and indices, issued
// at kernel start so that their latency overlaps the weight stream; every decision
// that depends on a loaded value is taken in epi_store.
struct EpiOps {
  float b0, b1, r0;   // bias of n and n + 1, residual of n
  float f0, f1;       // row sums of the folded weights of n and n + 1 (NRM_FOLDED)
  float c, s;         // RoPE cos/sin of the pair
  long long kvoff;    // the row's cache slot (QKV)
};

// META: the row's cache slot and RoPE row come from p.row_kvoff / p.rope_cs (else the
// caller fills them in).
template <int EPI, bool FOLD = false, bool META = true>
__device__ __forceinline__ EpiOps epi_prefetch(const LinParams& p, int m, int n) {
  EpiOps e;
  e.b0 = e.b1 = e.r0 = 0.f;
  e.f0 = e.f1 = 0.f;
  if (FOLD) {
    e.f0 = p.fs[n];
    if (EpiTraits<EPI>::pair) e.f1 = p.fs[n + 1];
    if (EPI == EPI_ARGMAX) e.b0 = p.bias[n];
  }
  e.c = 1.f; e.s = 0.f;
  e.kvoff = 0;
  if (EPI == EPI_PLAIN || EPI == EPI_GELU) {
    e.b0 = p.bias[n];
    e.r0 = p.resid[(size_t)m * p.ldr + n];
  } else if (EPI == EPI_QKV) {
    e.b0 = p.bias[n];
    if (META) e.kvoff = p.row_kvoff[m];
  } else if (EPI == EPI_QKV_ROPE) {
    e.b0 = p.bias[n];
    e.b1 = p.bias[n + 1];
    if (META) {
      e.kvoff = p.row_kvoff[m];
      const int i = (n % p.hd) >> 1;
      const float* cs = p.rope_cs + (size_t)m * p.hd;
      e.c = cs[i];
      e.s = cs[(p.hd >> 1) + i];
    }
  }
  return e;
}

// Applies the epilogue to output (m, n) = v0, or to the adjacent pair (v0, v1).
template <int EPI>
__device__ __forceinline__ void epi_store(const LinParams& p, const EpiOps& e, int m, int n, float v0, float v1) {
  if (EPI == EPI_SWIGLU) {
    p.y[(size_t)m * p.ldy + (n >> 1)] = silu(v0) * v1;
  } else if (EPI == EPI_QKV || EPI == EPI_QKV_ROPE) {
    v0 += e.b0;
    if (EPI == EPI_QKV_ROPE) {
      v1 += e.b1;
      if (n < p.qdim + p.kdim) {   // rotate-half RoPE on q and k; v is stored as is
        const float a = v0, b = v1;
        v0 = a * e.c - b * e.s;
        v1 = a * e.s + b * e.c;
      }
      qkv_store(p, m, n + 1, e.kvoff, v1);
    }
    qkv_store(p, m, n, e.kvoff, v0);
  } else {
    v0 += e.b0;
    if (EPI == EPI_GELU) v0 = gelu_clamped(v0);
    p.y[(size_t)m * p.ldy + n] = e.r0 + v0;
  }
}

// Activation rows are staged into LDS xs[m * K + k] as they are. stage_issue loads
// the first XPT float4 chunks of this thread; it runs before the weight loads, so that
// waiting for the rows does not wait for the weight stream (vector loads complete in
// issue order). stage_finish stores them and copies any remaining chunks. A pre-norm
// is applied later, in the dot products (k_gemv).
template <int XPT>
struct RowRegs {
  f32x4 x[XPT];
};

template <int XPT, int PRO>
__device__ __forceinline__ void stage_issue(const LinParams& p, RowRegs<XPT>& rr) {
  // Loads are unconditional (clamped to the last valid chunk; stage_finish stores only
  // valid ones) and the prologue is fixed at compile time, so the compiler can count
  // them and wait for these alone later, not for the weight loads issued after them.
  if (PRO != PRO_COPY) return;
  const int tid = threadIdx.x, K4 = p.K >> 2;
#pragma unroll
  for (int j = 0; j < XPT; ++j) {
    const int i = min(tid + GD_WG * j, p.M * K4 - 1);
    const int m = i / K4, k = (i - m * K4) << 2;
    rr.x[j] = *reinterpret_cast<const f32x4*>(p.x + (size_t)m * p.ldx + k);
  }
}

// Attention merge prologue: its loads are issued with the other row loads, before the
// weights.
template <int PRO>
__device__ __forceinline__ void stage_issue_attn(const LinParams& p, MergeRegs<4>& ar) {
  if (PRO != PRO_ATTN) return;
  attn_merge_issue<4>(p.apart, p.Hq, p.hd, p.M, ar, GD_WG);
}

template <int XPT, int PRO>
__device__ __forceinline__ void stage_finish(const LinParams& p, float* xs, const RowRegs<XPT>& rr,
                                             const MergeRegs<4>& ar, float* s_aw) {
  const int tid = threadIdx.x;
  const int M = p.M, K = p.K;
  if (PRO == PRO_ATTN) {
    attn_merge_finish<4>(p.apart, p.Hq, p.hd, M, ar, xs, K, s_aw, GD_WG);
    return;
  }
  // Every thread stores its (clamped) chunks: threads past the rows rewrite the last
  // chunk with the value its owner writes. A conditional store would let the compiler
  // sink the row loads into the branch, behind the weight loads, and wait for those.
  const int K4 = K >> 2;
#pragma unroll
  for (int j = 0; j < XPT; ++j) {
    const int i = min(tid + GD_WG * j, M * K4 - 1);
    const int m = i / K4, k = (i - m * K4) << 2;
    *reinterpret_cast<f32x4*>(xs + m * K + k) = rr.x[j];
  }
  for (int i = tid + GD_WG * XPT; i < M * K4; i += GD_WG) {   // rows beyond the register share
    const int m = i / K4, k = (i - m * K4) << 2;
    *reinterpret_cast<f32x4*>(xs + m * K + k) = *reinterpret_cast<const f32x4*>(p.x + (size_t)m * p.ldx + k);
  }
}

// ---- PRO_EMBED: the decode step's set-up done by its first QKV launch (a GEMV).
// Every workgroup takes the rows' (sequence, position, token) as k_setup_decode does
// (the position is the sequence's length, kept below its capacity; a token or learned
// position out of range is replaced by 0) and forms x_b = wte[t] (+ wpe[p]) itself
// ("bare-metal-llm", "What got built": token and learned position embeddings).
// Workgroup 0 also stores the rows, their metadata and the error flags for the later
// launches of the step. The step's argmax finalize advances the lengths, after every
// workgroup here has read them.
struct EmbMeta {
  int vseq, vtok;   // lane m < M: row m's sequence slot and token as loaded
  int seq[GEMV_MAX_ROWS], pos[GEMV_MAX_ROWS], tok[GEMV_MAX_ROWS], ppos[GEMV_MAX_ROWS], flags[GEMV_MAX_ROWS];
};

// v[m] of a row index m < GEMV_MAX_ROWS held in a register (no indexed register array)
__device__ __forceinline__ int sel_row(int m, const int (&v)[GEMV_MAX_ROWS]) {
  return m == 0 ? v[0] : m == 1 ? v[1] : m == 2 ? v[2] : v[3];
}

// Issued before the weights (vector loads complete in issue order, so waiting for
// these does not wait for the weight stream): lane m loads row m's sequence slot and
// token.
__device__ __forceinline__ void emb_meta_issue(const LinEmbParams& p, EmbMeta& em) {
  const int lm = min((int)(threadIdx.x & 63), p.M - 1);
  em.vseq = p.e.sids[lm];
  em.vtok = p.e.tok[lm];
}

// After the weights: the tokens (an out-of-range one is replaced by 0) ...
__device__ __forceinline__ void emb_meta_tokens(const LinEmbParams& p, EmbMeta& em) {
#pragma unroll
  for (int m = 0; m < GEMV_MAX_ROWS; ++m) {
    const int tok = __builtin_amdgcn_readlane(em.vtok, m);
    const bool ok = tok >= 0 && tok < p.e.erp.vocab;
    em.tok[m] = ok ? tok : 0;
    em.flags[m] = ok ? 0 : GD_DERR_TOKEN;
    em.seq[m] = __builtin_amdgcn_readlane(em.vseq, m);
  }
}

// ... then the sequences' lengths and capacities (scalar loads), clamped as
// k_setup_decode does.
__device__ __forceinline__ void emb_meta_finish(const LinEmbParams& p, EmbMeta& em) {
  const RowParams& r = p.e.erp;
  int len[GEMV_MAX_ROWS], cap[GEMV_MAX_ROWS];
#pragma unroll
  for (int m = 0; m < GEMV_MAX_ROWS; ++m) {
    len[m] = p.e.len[em.seq[m]];
    cap[m] = p.e.cap[em.seq[m]];
  }
#pragma unroll
  for (int m = 0; m < GEMV_MAX_ROWS; ++m) {
    int pos = len[m];
    int fl = em.flags[m];
    if (pos >= cap[m]) { fl |= GD_DERR_POS; pos = cap[m] - 1; }
    int ppos = pos;
    if (r.wpe && (ppos < 0 || ppos >= r.n_pos)) { fl |= GD_DERR_POS; ppos = 0; }
    em.pos[m] = pos;
    em.ppos[m] = ppos;
    em.flags[m] = fl;
  }
}

// Four consecutive elements of an embedding table (the weights' type): float4, four
// bf16, four int8 codes (with their block scale).
template <int WT>
struct EmbChunk;
template <>
struct EmbChunk<0> { typedef f32x4 T; };
template <>
struct EmbChunk<1> { typedef uint2 T; };
template <>
struct EmbChunk<2> { typedef uint32_t T; };

template <int WT>
struct EmbLoad {
  typename EmbChunk<WT>::T a, b;   // wte, wpe
  float sa, sb;                    // 8-bit: block scales
};

// Chunk (m, k) of wte[t] (needs the tokens only) ...
template <int WT>
__device__ __forceinline__ void emb_load_te(const LinEmbParams& p, const EmbMeta& em, int m, int k, EmbLoad<WT>& l) {
  typedef typename EmbChunk<WT>::T ET;
  constexpr int ES = WT == 0 ? 4 : WT == 1 ? 2 : 1;
  const RowParams& r = p.e.erp;
  const size_t et = (size_t)sel_row(m, em.tok) * r.d + k;
  l.a = *reinterpret_cast<const ET*>(reinterpret_cast<const char*>(r.wte) + et * ES);
  l.sa = 1.f;
  if constexpr (WT == 2) l.sa = r.wte_sc[et >> 5];
}

// ... and of wpe[p] (the positions).
template <int WT>
__device__ __forceinline__ void emb_load_pe(const LinEmbParams& p, const EmbMeta& em, int m, int k, EmbLoad<WT>& l) {
  typedef typename EmbChunk<WT>::T ET;
  constexpr int ES = WT == 0 ? 4 : WT == 1 ? 2 : 1;
  const RowParams& r = p.e.erp;
  const size_t ep = (size_t)sel_row(m, em.ppos) * r.d + k;
  l.b = *reinterpret_cast<const ET*>(reinterpret_cast<const char*>(r.wpe) + ep * ES);
  l.sb = 1.f;
  if constexpr (WT == 2) l.sb = r.wpe_sc[ep >> 5];
}

// x = wte[t][k..k+3] (+ wpe[p][k..k+3]), as k_setup_decode sums them.
template <int WT>
__device__ __forceinline__ f32x4 emb_value(const EmbLoad<WT>& l, bool pe) {
  f32x4 v;
  if constexpr (WT == 0) {
    v = l.a;
    if (pe) { v.x += l.b.x; v.y += l.b.y; v.z += l.b.z; v.w += l.b.w; }
  } else if constexpr (WT == 1) {
    v = (f32x4){bf16_lo(l.a.x), bf16_hi(l.a.x), bf16_lo(l.a.y), bf16_hi(l.a.y)};
    if (pe) { v.x += bf16_lo(l.b.x); v.y += bf16_hi(l.b.x); v.z += bf16_lo(l.b.y); v.w += bf16_hi(l.b.y); }
  } else {
    v = (f32x4){q8_at(l.a, 0) * l.sa, q8_at(l.a, 1) * l.sa, q8_at(l.a, 2) * l.sa, q8_at(l.a, 3) * l.sa};
    if (pe) {
      v.x += q8_at(l.b, 0) * l.sb; v.y += q8_at(l.b, 1) * l.sb;
      v.z += q8_at(l.b, 2) * l.sb; v.w += q8_at(l.b, 3) * l.sb;
    }
  }
  return v;
}

// This thread's chunks of all rows: chunk j is i = tid + GD_WG j of the M K / 4; XE
// covers GEMV_MAX_ROWS rows, and the chunks past the M rows are not loaded.
template <int WT, int XE>
__device__ __forceinline__ void emb_issue_te(const LinEmbParams& p, const EmbMeta& em, EmbLoad<WT> (&el)[XE]) {
  const int tid = threadIdx.x, K4 = p.K >> 2, MK4 = p.M * K4;
#pragma unroll
  for (int j = 0; j < XE; ++j) {
    const int i = tid + GD_WG * j;
    if (i < MK4) {
      const int m = i / K4, k = (i - m * K4) << 2;
      emb_load_te<WT>(p, em, m, k, el[j]);
    }
  }
}

template <int WT, int XE>
__device__ __forceinline__ void emb_issue_pe(const LinEmbParams& p, const EmbMeta& em, EmbLoad<WT> (&el)[XE]) {
  const int tid = threadIdx.x, K4 = p.K >> 2, MK4 = p.M * K4;
#pragma unroll
  for (int j = 0; j < XE; ++j) {
    const int i = tid + GD_WG * j;
    if (i < MK4) {
      const int m = i / K4, k = (i - m * K4) << 2;
      emb_load_pe<WT>(p, em, m, k, el[j]);
    }
  }
}

// The rows into LDS xs[m * K + k].
template <int WT, int XE>
__device__ __forceinline__ void emb_finish(const LinEmbParams& p, const EmbLoad<WT> (&el)[XE], float* xs) {
  const int tid = threadIdx.x, K = p.K, K4 = K >> 2, MK4 = p.M * K4;
  const bool pe = p.e.erp.wpe != nullptr;
#pragma unroll
  for (int j = 0; j < XE; ++j) {
    const int i = tid + GD_WG * j;
    if (i < MK4) {
      const int m = i / K4, k = (i - m * K4) << 2;
      *reinterpret_cast<f32x4*>(xs + m * K + k) = emb_value<WT>(el[j], pe);
    }
  }
}

// The row's K/V slot (kv_slot_offset with the block-table load unconditional).
__device__ __forceinline__ long long emb_kvoff(const RowParams& r, int seq, int pos) {
  const int bi = max(pos, 0) / r.block_size;
  const int blk = r.table[(size_t)seq * r.max_blocks + min(bi, r.max_blocks - 1)];
  if (pos < 0 || bi >= r.max_blocks || (unsigned)blk >= (unsigned)r.nblk) return -1;
  return ((long long)blk * r.Hkv * r.block_size + (pos - bi * r.block_size)) * r.hd;
}

// The QKV epilogue's row metadata of output (m, n) from the embedding prologue.
template <int EPI>
__device__ __forceinline__ void emb_epi_ops(const LinEmbParams& p, const EmbMeta& em, int m, int n, EpiOps& e) {
  const RowParams& r = p.e.erp;
  const int pos = sel_row(m, em.pos);
  e.kvoff = emb_kvoff(r, sel_row(m, em.seq), pos);
  if constexpr (EPI == EPI_QKV_ROPE) {
    const int i = (n % p.hd) >> 1;
    const float* cs = r.rope + (size_t)min(max(pos, 0), r.n_pos - 1) * p.hd;
    e.c = cs[i];
    e.s = cs[(p.hd >> 1) + i];
  }
}

// Workgroup 0: the rows' metadata (lane m < M of wave 0, which owns row m's output and
// holds its slot in e), error flags and RoPE rows, as k_setup_decode leaves them.
template <int EPI>
__device__ __forceinline__ void emb_publish(const LinEmbParams& p, const EmbMeta& em, const EpiOps& e) {
  const RowParams& r = p.e.erp;
  const int tid = threadIdx.x;
  if (tid < p.M) {
    r.row_seq[tid] = sel_row(tid, em.seq);
    r.row_pos[tid] = sel_row(tid, em.pos);
    r.row_tok[tid] = sel_row(tid, em.tok);
    r.row_kvoff[tid] = e.kvoff;
    const int fl = sel_row(tid, em.flags) | (e.kvoff < 0 ? GD_DERR_BLOCK : 0);
    if (fl) atomicOr(p.err, fl);
  }
  if constexpr (EPI == EPI_QKV_ROPE) {
    for (int i = tid; i < p.M * p.hd; i += GD_WG) {
      const int m = i / p.hd, j = i - m * p.hd;
      r.row_cs[i] = r.rope[(size_t)min(max(sel_row(m, em.pos), 0), r.n_pos - 1) * p.hd + j];
    }
  }
}

template <int WT>
struct WChunk;
template <>
struct WChunk<0> { typedef f32x4 T; static constexpr int CE = 4; };
template <>
struct WChunk<1> { typedef u32x4 T; static constexpr int CE = 8; };
template <>
struct WChunk<2> { typedef u32x4 T; static constexpr int CE = 16; };   // 16 int8 codes, one block scale

// The sum over one 16-code chunk of 8-bit weights against its 16 activations a[0..3],
// times the chunk's block scale.
__device__ __forceinline__ float q8_chunk_dot(const u32x4& w, const f32x4* a, float sc) {
  float t = 0.f;
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    t = fmaf(q8_at(ws[j], 0), a[j].x, t);
    t = fmaf(q8_at(ws[j], 1), a[j].y, t);
    t = fmaf(q8_at(ws[j], 2), a[j].z, t);
    t = fmaf(q8_at(ws[j], 3), a[j].w, t);
  }
  return t * sc;
}

// ------------------------------------------------------------------ GEMV

// PRO: source of the rows (PRO_COPY or PRO_ATTN); NRM: how a pre-norm (p.norm:
// LayerNorm or RMSNorm) is applied (NRM_NONE, NRM_EXPLICIT, NRM_FOLDED). Both are
// compile-time so that every path issues a fixed number of loads and the waits for the
// rows do not cover the weight stream.
//
// NRM_FOLDED (fp32 weights): p.w holds g_k W_nk, p.bias the folded bias, p.fs the row
// sums of p.w. A wave shifts its row by the row's first element, d = x - x_0, and
// forms the moments of d; the dot products use d as is, so they do not wait for the
// statistics, and the result is r (d . w_n - a s_n) + bias_n with a = mean(d) (this
// equals r (x - mu) . w_n) and r = 1 / sqrt(var + eps). RMSNorm: no shift, a = 0.
template <int WT, int NC, int RW, int EPI, int PRO, int NRM>
__global__ __launch_bounds__(GD_WG) void k_gemv(typename GemvArgs<PRO>::T p) {
  typedef typename WChunk<WT>::T VT;
  constexpr int CE = WChunk<WT>::CE;
  extern __shared__ __align__(16) float xs[];   // [M][K] rows
  __shared__ float s_am[GEMV_MAX_ROWS][4 * RW];
  __shared__ float s_aw[GEMV_MAX_ROWS * GD_MAX_HEADS * GD_ATT_NCH];   // attention chunk weights
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int M = p.M, N = p.N, K = p.K;
  const int nw0 = (blockIdx.x * 4 + wave) * RW;              // first row of this wave

  // 0. this thread's share of the activation rows (M = 1 rows fit entirely)
  constexpr int XPT = (NC * CE + 15) / 16;
  RowRegs<XPT> rr;
  stage_issue<XPT, PRO>(p, rr);
  MergeRegs<4> ar;
  stage_issue_attn<PRO>(p, ar);
  const float* bsrc = p.nb ? p.nb : p.ng;
  EmbMeta em;
  if constexpr (PRO == PRO_EMBED) {
    emb_meta_issue(p, em);
    __builtin_amdgcn_sched_barrier(0);
  }
  // the norm's gain and shift at this lane's chunks (RMSNorm: no shift; the gain is
  // loaded in its place so that the number of loads stays fixed)
  f32x4 gn[NC][CE / 4], bn[NC][CE / 4];
  if constexpr (NRM == NRM_EXPLICIT) {
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int k = min((lane + 64 * i) * CE, K - CE);
#pragma unroll
      for (int h = 0; h < CE / 4; ++h) {
        gn[i][h] = *reinterpret_cast<const f32x4*>(p.ng + k + 4 * h);
        bn[i][h] = *reinterpret_cast<const f32x4*>(bsrc + k + 4 * h);
      }
    }
  }
  // 1. weights: they do not depend on anything
  VT w[RW][NC];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int n = nw0 + r;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      // unconditional load of a clamped chunk: chunks past K are never used (the dot
      // products skip them) and rows past N are never stored
      const int k = min((lane + 64 * i) * CE, K - CE);
      w[r][i] = __builtin_nontemporal_load(reinterpret_cast<const VT*>(
          reinterpret_cast<const char*>(p.w) + ((size_t)min(n, N - 1) * K + k) * (WT == 0 ? 4 : WT == 1 ? 2 : 1)));
    }
  }
  // 8-bit weights: each chunk's block scale (blocks of 32: two chunks per scale)
  float wsc[RW][NC];
  if constexpr (WT == 2) {
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        const int k = min((lane + 64 * i) * CE, K - CE);
        wsc[r][i] = p.wsc[(size_t)min(nw0 + r, N - 1) * (K >> 5) + (k >> 5)];
      }
  }
  // embedding rows (PRO_EMBED), loaded after the weights: the token rows once the rows'
  // slots and tokens (loaded before the weights) are in, the position rows after one
  // more scalar round trip (the sequences' lengths); both overlap the weight stream
  constexpr int XE = PRO == PRO_EMBED ? GEMV_MAX_ROWS * XPT : 1;
  EmbLoad<WT> el[XE];
  if constexpr (PRO == PRO_EMBED) {
    __builtin_amdgcn_sched_barrier(0);
    emb_meta_tokens(p, em);
    emb_issue_te<WT, XE>(p, em, el);
    emb_meta_finish(p, em);
    if (p.e.erp.wpe) emb_issue_pe<WT, XE>(p, em, el);
  }
  // 2. epilogue operands of this lane's output (lane m * RW + r), or pair (lane m)
  constexpr bool PAIR = EpiTraits<EPI>::pair;
  static_assert(!PAIR || RW == 2, "pair epilogues need both rows of the pair in one wave");
  static_assert(PRO != PRO_EMBED || EPI == EPI_QKV || EPI == EPI_QKV_ROPE, "embedding rows: the QKV launch only");
  const int om = PAIR ? lane : lane / RW, orr = PAIR ? 0 : lane % RW;
  const int on = nw0 + orr;
  const bool own = EPI != EPI_ARGMAX && om < M && (PAIR ? nw0 + 1 < N : (lane < M * RW && on < N));
  // argmax: lane m * RW + r finishes output (m, nw0 + r)
  const int an = min(nw0 + lane % RW, N - 1);
  constexpr bool META = PRO != PRO_EMBED;
  EpiOps eo = EPI == EPI_ARGMAX ? epi_prefetch<EPI, NRM == NRM_FOLDED, META>(p, 0, an)
                                : epi_prefetch<EPI, NRM == NRM_FOLDED, META>(p, own ? om : 0, own ? on : 0);
  if constexpr (PRO == PRO_EMBED) emb_epi_ops<EPI>(p, em, own ? om : 0, own ? on : 0, eo);
  // every load above is issued here, in this order: the scheduler may not move any of
  // them below the waits for the rows
  __builtin_amdgcn_sched_barrier(0);
  // 3. activation rows into LDS
  if constexpr (PRO == PRO_EMBED) emb_finish<WT, XE>(p, el, xs);
  else stage_finish<XPT, PRO>(p, xs, rr, ar, s_aw);
  __syncthreads();
  if constexpr (PRO == PRO_EMBED) {
    if (blockIdx.x == 0) {   // the residual rows for the rest of the step
      const int K4 = K >> 2;
      for (int i = tid; i < M * K4; i += GD_WG) {
        const int m = i / K4, k = (i - m * K4) << 2;
        *reinterpret_cast<f32x4*>(p.e.erp.x + (size_t)m * p.e.erp.d + k) = *reinterpret_cast<const f32x4*>(xs + m * K + k);
      }
    }
  }
  // 4. dot products. With a pre-norm every row is normalized on the fly: the lanes of a
  //    wave hold the row's whole K range (chunks lane + 64 i), so each wave forms the
  //    row's statistics itself (one-pass moments shifted by the row's first element,
  //    summed with wave-level reductions) and no workgroup exchange is needed.
  float acc[RW][GEMV_MAX_ROWS];
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int m = 0; m < GEMV_MAX_ROWS; ++m) acc[r][m] = 0.f;
  // acc[.][m] += w . xv over this lane's chunks (xv: the row's chunks in registers)
  auto dot_row = [&](int m, const f32x4 (&xv)[NC][CE / 4]) {
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      if constexpr (WT == 2) {
        if ((lane + 64 * i) * CE < K) {
#pragma unroll
          for (int r = 0; r < RW; ++r) acc[r][m] += q8_chunk_dot(w[r][i], xv[i], wsc[r][i]);
        }
        continue;
      }
      if ((lane + 64 * i) * CE < K) {
        const f32x4 a = xv[i][0];
#pragma unroll
        for (int r = 0; r < RW; ++r) {
          float s = acc[r][m];
          if (WT == 0) {
            s = fmaf(w[r][i].x, a.x, s); s = fmaf(w[r][i].y, a.y, s);
            s = fmaf(w[r][i].z, a.z, s); s = fmaf(w[r][i].w, a.w, s);
          } else {
            s = fmaf(bf16_lo(w[r][i].x), a.x, s); s = fmaf(bf16_hi(w[r][i].x), a.y, s);
            s = fmaf(bf16_lo(w[r][i].y), a.z, s); s = fmaf(bf16_hi(w[r][i].y), a.w, s);
          }
          acc[r][m] = s;
        }
        if constexpr (WT == 1) {
          const f32x4 b = xv[i][CE / 4 - 1];
#pragma unroll
          for (int r = 0; r < RW; ++r) {
            float s = acc[r][m];
            s = fmaf(bf16_lo(w[r][i].z), b.x, s); s = fmaf(bf16_hi(w[r][i].z), b.y, s);
            s = fmaf(bf16_lo(w[r][i].w), b.z, s); s = fmaf(bf16_hi(w[r][i].w), b.w, s);
            acc[r][m] = s;
          }
        }
      }
    }
  };
  // the row's chunks from LDS into registers (zeros past K)
  auto load_row = [&](int m, f32x4 (&xv)[NC][CE / 4]) {
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int k = (lane + 64 * i) * CE;
#pragma unroll
      for (int h = 0; h < CE / 4; ++h)
        xv[i][h] = k < K ? *reinterpret_cast<const f32x4*>(xs + m * K + k + 4 * h) : (f32x4){0.f, 0.f, 0.f, 0.f};
    }
  };
  float rsv[GEMV_MAX_ROWS], av[GEMV_MAX_ROWS];   // NRM_FOLDED: per-row 1/sqrt(var + eps), mean of d
  const float invK = 1.0f / (float)K;
  if (NRM == NRM_NONE && M > 1) {
    // several rows as staged: chunk-outer, so that each weight chunk meets every row
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int k = (lane + 64 * i) * CE;
      if (k < K) {
#pragma unroll
        for (int m = 0; m < GEMV_MAX_ROWS; ++m) {
          if (m < M) {
            const float* xr = xs + m * K + k;
            if constexpr (WT == 2) {
              const f32x4 a4[4] = {*reinterpret_cast<const f32x4*>(xr), *reinterpret_cast<const f32x4*>(xr + 4),
                                   *reinterpret_cast<const f32x4*>(xr + 8), *reinterpret_cast<const f32x4*>(xr + 12)};
#pragma unroll
              for (int r = 0; r < RW; ++r) acc[r][m] += q8_chunk_dot(w[r][i], a4, wsc[r][i]);
              continue;
            }
            const f32x4 a = *reinterpret_cast<const f32x4*>(xr);
#pragma unroll
            for (int r = 0; r < RW; ++r) {
              float s = acc[r][m];
              if (WT == 0) {
                s = fmaf(w[r][i].x, a.x, s); s = fmaf(w[r][i].y, a.y, s);
                s = fmaf(w[r][i].z, a.z, s); s = fmaf(w[r][i].w, a.w, s);
              } else {
                s = fmaf(bf16_lo(w[r][i].x), a.x, s); s = fmaf(bf16_hi(w[r][i].x), a.y, s);
                s = fmaf(bf16_lo(w[r][i].y), a.z, s); s = fmaf(bf16_hi(w[r][i].y), a.w, s);
              }
              acc[r][m] = s;
            }
            if constexpr (WT == 1) {
              const f32x4 b = *reinterpret_cast<const f32x4*>(xr + 4);
#pragma unroll
              for (int r = 0; r < RW; ++r) {
                float s = acc[r][m];
                s = fmaf(bf16_lo(w[r][i].z), b.x, s); s = fmaf(bf16_hi(w[r][i].z), b.y, s);
                s = fmaf(bf16_lo(w[r][i].w), b.z, s); s = fmaf(bf16_hi(w[r][i].w), b.w, s);
                acc[r][m] = s;
              }
            }
          }
        }
      }
    }
  } else {
    // row by row with the row's chunks in registers (a single row, or a pre-norm that
    // needs each row's statistics before its products)
#pragma unroll
    for (int m = 0; m < GEMV_MAX_ROWS; ++m) {
      if (m < M) {
        f32x4 xv[NC][CE / 4];
        load_row(m, xv);
        if constexpr (NRM != NRM_NONE) {
          const bool ln = p.norm == NORM_LN;
          const float sh = ln ? xs[m * K] : 0.f;
          float st[2] = {0.f, 0.f};
#pragma unroll
          for (int i = 0; i < NC; ++i) {
            if ((lane + 64 * i) * CE < K) {
#pragma unroll
              for (int h = 0; h < CE / 4; ++h) {
                f32x4& v = xv[i][h];
                v.x -= sh; v.y -= sh; v.z -= sh; v.w -= sh;
                st[0] += (v.x + v.y) + (v.z + v.w);
                st[1] += fmaf(v.x, v.x, v.y * v.y) + fmaf(v.z, v.z, v.w * v.w);
              }
            }
          }
          wave_sum_n<2>(st);
          const float a = ln ? st[0] * invK : 0.f;   // mean of the shifted values
          const float var = fmaxf(st[1] * invK - a * a, 0.f);
          const float rs = rsqrtf(var + p.eps);
          if constexpr (NRM == NRM_FOLDED) {
            rsv[m] = rs;
            av[m] = a;
          } else {
            // (x - mu) r g + b with x - mu = d - a
#pragma unroll
            for (int i = 0; i < NC; ++i)
#pragma unroll
              for (int h = 0; h < CE / 4; ++h) {
                f32x4& v = xv[i][h];
                const f32x4 g = gn[i][h], b = bn[i][h];
                v.x = fmaf((v.x - a) * rs, g.x, ln ? b.x : 0.f);
                v.y = fmaf((v.y - a) * rs, g.y, ln ? b.y : 0.f);
                v.z = fmaf((v.z - a) * rs, g.z, ln ? b.z : 0.f);
                v.w = fmaf((v.w - a) * rs, g.w, ln ? b.w : 0.f);
              }
          }
        }
        dot_row(m, xv);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int m = 0; m < GEMV_MAX_ROWS; ++m)
      if (m < M) acc[r][m] = wave_sum(acc[r][m]);
  // 5. epilogue
  if (EPI == EPI_ARGMAX) {
    if (lane < M * RW) {
      const int am = lane / RW, ar = lane % RW;
      float v = 0.f;
#pragma unroll
      for (int m = 0; m < GEMV_MAX_ROWS; ++m)
#pragma unroll
        for (int r = 0; r < RW; ++r)
          if (m == am && r == ar) {
            v = acc[r][m];
            if (NRM == NRM_FOLDED) v = fmaf(rsv[m], v - av[m] * eo.f0, eo.b0);
          }
      s_am[am][wave * RW + ar] = v;
      if (p.logits && nw0 + ar < N) p.logits[(size_t)am * p.ldl + nw0 + ar] = v;
    }
    __syncthreads();
    if (tid < M) {
      const int nb0 = blockIdx.x * 4 * RW;
      float bv = s_am[tid][0];
      int bi = nb0;
      for (int j = 1; j < 4 * RW && nb0 + j < N; ++j)
        if (am_better(s_am[tid][j], nb0 + j, bv, bi)) { bv = s_am[tid][j]; bi = nb0 + j; }
      p.am_val[(size_t)blockIdx.x * M + tid] = bv;
      p.am_idx[(size_t)blockIdx.x * M + tid] = bi;
    }
    return;
  }
  if constexpr (PRO == PRO_EMBED) {
    if (blockIdx.x == 0) emb_publish<EPI>(p, em, eo);
  }
  if (!own) return;
  float v0 = 0.f, v1 = 0.f;
#pragma unroll
  for (int m = 0; m < GEMV_MAX_ROWS; ++m) {
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      if (m == om && r == orr) v0 = acc[r][m];
      if (m == om && r == orr + 1) v1 = acc[r][m];
    }
    if (NRM == NRM_FOLDED && m == om) {
      v0 = rsv[m] * (v0 - av[m] * eo.f0);
      v1 = rsv[m] * (v1 - av[m] * eo.f1);
    }
  }
  epi_store<EPI>(p, eo, om, on, v0, v1);
}

// ------------------------------------------------------------------- MFMA
//
// k_mm (1..32 rows): 16-column tiles on v_mfma_f32_16x16x4f32 (bf16 weights widened to
// fp32 in registers) or, for workgroups that stream several tiles (PT), on the bf16
// matrix cores (v_mfma_f32_16x16x32_bf16, 16 times the fp32 rate) in exact parts: the
// staged activations are split once into three bf16 parts, fp32 weights as they arrive
// (per block) as well; a product is then the sum of the part products with i + j <= 2
// (six for fp32 weights: the dropped terms lie below 2^-24 of the product; three for
// bf16 weights, which are one part: exact), smallest first, accumulated in fp32. With
// one tile per workgroup the split of the activations outweighs the faster products.
// Grid (G, S): workgroup (g, s) owns the 32-column K blocks
// [s nb / S, (s + 1) nb / S) and the column tiles g, g + G, g + 2G, ...; S > 1 only for
// a linear epilogue whose output is the residual, updated in place: each split adds
// its partial sums to it with float atomics, the bias coming from split 0.
//
// Operand layout: lane l = 16 q + c holds W[n0 + c][kk + 8q .. +8] and
// X[m0 + c][kk + 8q .. +8] for the 32-column block kk; fp32 MFMA step t of 8 feeds
// element t of both, so one instruction contracts the k-values kk + 8q + t for A and B
// alike (PT: eight bf16 values per part, one MFMA per part pair for the whole block).
// D[i][j]: lane l holds column j = l % 16 and rows 4q + v.
//
// Loads are shaped for the memory pipeline rather than for that layout: a load
// instruction that spreads over 16 rows reaches a CU at well under half the rate of
// one that reads 1 KB of contiguous bytes. Hence
//  - the weights are read from a tile-major copy (k_pack_tiles) in which every 16 x 32
//    block is stored in operand order, so each instruction reads 1 KB contiguously;
//  - the activation rows of the K range are loaded a whole row per wave (lane l: 16
//    bytes at 16 l + 1 KB j), normalized there (two-pass mean and variance from
//    registers), written to LDS once and read back in operand layout; each wave then
//    keeps its K blocks (block = range start + wave + MM_NW j) in registers for all of
//    its tiles.
// Padding is zero on both sides (weight rows past N and columns past K in the packed
// copy; LDS columns past the K range and rows past M), so no lane needs masking.
// The next tile's weights are issued (into a second register set) before a tile's
// MFMAs; the waves' partial tiles are summed through a double-buffered LDS array
// placed over the (by then unused) row staging area, and each thread applies the epilogue to its own output
// (row tid / 16, column tid % 16). The head's argmax keeps a running best per output
// thread across tiles and writes one partial per workgroup and row.

#define MM_NW 8                       // waves per workgroup
#define MM_JB 4                       // K blocks per wave and pass held in registers
#define MM_KC (MM_NW * MM_JB * 32)    // K columns per pass
static_assert(64 * MM_JB * 4 <= MM_KC, "a lane's staging slots stay inside a row's MM_KC columns");
#define MM_LDX (MM_KC + 4)            // LDS row stride: 16 rows read at one column fall in distinct banks

// Bytes of one packed 16 x 32 block.
__host__ __device__ constexpr int mm_block_bytes(int wt) { return wt == 0 ? 2048 : 1024; }
// Bytes of the packed copy of an [N][K] matrix.
__host__ __device__ inline size_t mm_packed_bytes(int wt, int N, int K) {
  return (size_t)((N + 15) / 16) * ((K + 31) / 32) * mm_block_bytes(wt);
}

// Tile-major copy of W [N][K]: block (t, b) (t = column tile of 16 rows, b = 32-column
// K block) at ((t * nb + b) * block bytes); inside it, fp32: two 1 KB halves h, lane l's
// 16 bytes at h * 1024 + 16 l hold W[16t + l%16][32b + 8(l/16) + 4h .. +4]; bf16: lane
// l's 16 bytes at 16 l hold W[16t + l%16][32b + 8(l/16) .. +8]. Rows >= N and columns
// >= K are zero. One thread per 16-byte unit.
__global__ __launch_bounds__(GD_WG) void k_pack_tiles(const void* __restrict__ W, int wt, int N, int K,
                                                      void* __restrict__ dst, size_t units) {
  const size_t u = (size_t)blockIdx.x * GD_WG + threadIdx.x;
  if (u >= units) return;
  const int nb = (K + 31) >> 5;
  u32x4 v = {0u, 0u, 0u, 0u};
  if (wt == 0) {
    const int l = (int)(u & 63), h = (int)((u >> 6) & 1);
    const size_t blk = u >> 7;
    const int t = (int)(blk / nb), b = (int)(blk % nb);
    const int n = 16 * t + (l & 15), k = 32 * b + 8 * (l >> 4) + 4 * h;
    if (n < N && k < K) v = *reinterpret_cast<const u32x4*>(reinterpret_cast<const float*>(W) + (size_t)n * K + k);
  } else {
    const int l = (int)(u & 63);
    const size_t blk = u >> 6;
    const int t = (int)(blk / nb), b = (int)(blk % nb);
    const int n = 16 * t + (l & 15), k = 32 * b + 8 * (l >> 4);
    if (n < N && k < K) v = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(W) + (size_t)n * K + k);
  }
  reinterpret_cast<u32x4*>(dst)[u] = v;
}

// bf16 parts of fp32 values (the matrix-core kernels): an fp32 value is the exact sum of
// three bf16 parts, each the nearest bf16 to what the previous ones left (8 + 8 + 8
// significant bits), and a product of two bf16 values is exact in fp32.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two floats to packed bf16 bits, rounded to nearest even (element 0 in the low half).
__device__ __forceinline__ uint32_t pk_bf16(float x, float y) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((float __attribute__((ext_vector_type(2)))){x, y}, bf16x2_t));
}

// Four floats as three packed bf16 parts: a = hi + mid + lo.
__device__ __forceinline__ void split3(const f32x4& a, uint2& hi, uint2& mid, uint2& lo) {
  hi = make_uint2(pk_bf16(a.x, a.y), pk_bf16(a.z, a.w));
  float r0 = a.x - bf16_lo(hi.x), r1 = a.y - bf16_hi(hi.x), r2 = a.z - bf16_lo(hi.y), r3 = a.w - bf16_hi(hi.y);
  mid = make_uint2(pk_bf16(r0, r1), pk_bf16(r2, r3));
  r0 -= bf16_lo(mid.x); r1 -= bf16_hi(mid.x); r2 -= bf16_lo(mid.y); r3 -= bf16_hi(mid.y);
  lo = make_uint2(pk_bf16(r0, r1), pk_bf16(r2, r3));
}

// Eight consecutive fp32 values (two float4) as three bf16x8 parts.
__device__ __forceinline__ void split3x8(const f32x4& a, const f32x4& b, u32x4 (&pt)[3]) {
  uint2 ha, ma, la, hb, mb, lb;
  split3(a, ha, ma, la);
  split3(b, hb, mb, lb);
  pt[0] = (u32x4){ha.x, ha.y, hb.x, hb.y};
  pt[1] = (u32x4){ma.x, ma.y, mb.x, mb.y};
  pt[2] = (u32x4){la.x, la.y, lb.x, lb.y};
}

template <int WT> struct W8;   // eight weights of one lane and block, as stored
template <> struct W8<0> { f32x4 a, b; };
template <> struct W8<1> { u32x4 a; };

// Lane's eight weights of packed block blk (byte offset blk * block bytes).
template <int WT>
__device__ __forceinline__ W8<WT> load_w8tile(const void* __restrict__ Wt, size_t blk, int lane) {
  W8<WT> r;
  const char* base = reinterpret_cast<const char*>(Wt) + blk * mm_block_bytes(WT) + 16 * lane;
  if constexpr (WT == 0) {
    r.a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(base));
    r.b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(base + 1024));
  } else {
    r.a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base));
  }
  return r;
}

template <int WT>
__device__ __forceinline__ float w8_at(const W8<WT>& r, int t) {
  if constexpr (WT == 0) {
    const f32x4 v = t < 4 ? r.a : r.b;
    const int u = t & 3;
    return u == 0 ? v.x : u == 1 ? v.y : u == 2 ? v.z : v.w;
  } else {
    const int u = t >> 1;
    const uint32_t x = u == 0 ? r.a.x : u == 1 ? r.a.y : u == 2 ? r.a.z : r.a.w;
    return (t & 1) ? bf16_hi(x) : bf16_lo(x);
  }
}

struct F8 { f32x4 a, b; };   // eight consecutive fp32 values

__device__ __forceinline__ float f8_at(const F8& r, int t) {
  const f32x4 v = t < 4 ? r.a : r.b;
  const int u = t & 3;
  return u == 0 ? v.x : u == 1 ? v.y : u == 2 ? v.z : v.w;
}

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}

// Keeps the loads that produced v in flight no longer than this point: the compiler
// waits for them here (where they have long arrived) rather than at their use, which
// may follow loads issued later.
__device__ __forceinline__ void settle(float v) { asm volatile("" ::"v"(v)); }

__device__ __forceinline__ f32x4 f4_zero() { return (f32x4){0.f, 0.f, 0.f, 0.f}; }

// LDS floats of k_mm with R activation rows.
__host__ __device__ constexpr int mm_lds_floats(int R) { return R * MM_LDX; }

// NRM: how a pre-norm (LayerNorm or RMSNorm by p.norm; S == 1, one pass) is applied,
// as in k_gemv: NRM_EXPLICIT normalizes the staged rows with the loaded gain and shift;
// NRM_FOLDED (fp32) stages the rows shifted by their first element, d = x - x_0, keeps
// each row's r = 1 / sqrt(var + eps) and a = mean(d) in LDS and applies
// r (acc - a s_n) + bias_n in the epilogue, with the folded weights, row sums and bias.
// MP: the K range of a split may exceed one pass (no norm): rows and weights are then
// staged per pass and tile. Without MP the weight loads are unconditional, so the
// compiler's wait counts stay exact and nothing waits for the next tile's weights.
//
// Staging costs VALU time (two waves per SIMD hide little), so only NRM_EXPLICIT masks
// element by element. Elsewhere the slots past a row's range hold a copy of its last
// chunk, which only ever meets zero weight columns (the packed copy is zero past K), and
// rows >= M hold copies of row M - 1, whose outputs are never stored.
//
// PRO: PRO_COPY stages the rows of p.x; PRO_ATTN (the output projection behind
// split-context attention, no norm, one register pass) forms them from the attention
// partials p.apart [M][Hq][nch][gd_apart_stride(hd)] (per chunk: running max, sum of
// weights and the unnormalized weighted sum of V), so that no merge launch precedes the
// projection. Each lane loads, for its float4 of every real staged row, the float4 of
// all nch (<= GD_ATT_NCH) chunks, and lane c of each aligned group of 8 the (max, sum)
// of chunk c (the group's 32 columns lie in one head: hd is a multiple of 32); all at
// once, before the weights (one memory round trip). The chunk weights e_c = exp(max_c -
// max) / sum_c' e_c' sum_c' are formed as k_attn_merge forms them and shared within the
// group by lane exchanges. A split spans at most 256 columns (one float4 slot per lane);
// the host plans the splits so.
template <int WT, int MT, int EPI, int NRM, bool MP, int PRO, bool PT>
__global__ __launch_bounds__(64 * MM_NW) void k_mm(LinParams p) {
  static_assert(!(NRM != NRM_NONE && MP), "the norm needs whole rows in one pass");
  static_assert(PRO == PRO_COPY || (NRM == NRM_NONE && !MP && EPI == EPI_PLAIN), "merged rows: projection only");
  constexpr int R = MT * 16;          // activation rows of the tile (rows >= M discarded)
  constexpr int RPW = R / MM_NW;      // rows staged per wave
  constexpr int RS = 17;              // padded row stride of a partial tile in LDS
  constexpr bool PAIR = EpiTraits<EPI>::pair;
  static_assert(2 * MM_NW * R * RS <= mm_lds_floats(R), "partial tiles fit over the staging area");
  __shared__ __align__(16) float xs[mm_lds_floats(R)];   // staged rows [R][MM_LDX], later s_red[2]
  __shared__ float s_rs[R], s_mu[R];   // NRM_FOLDED: each row's r and a
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, c = lane & 15;
  const int M = p.M, N = p.N, K = p.K;
  // Workgroups are placed round-robin over the 8 XCDs in launch order; the G column
  // tiles of one K split read the same slice of the activation rows, so the launch index
  // is renumbered to put consecutive tiles of a split on one XCD (the slice then comes
  // from HBM about once per split rather than once per XCD): L = 8 k + x (x < 8) becomes
  // x per + k for the first 8 per indices, per = total / 8; the remainder keeps its index.
  const int S = gridDim.y, G = gridDim.x;
  const int wgid = [&] {
    const int total = G * S, L = blockIdx.x + G * blockIdx.y, per = total >> 3;
    return L < 8 * per ? (L & 7) * per + (L >> 3) : L;
  }();
  const int s = wgid / G, wg = wgid - s * G;
  const int nb = (K + 31) >> 5;
  const int b0 = s * nb / S, b1 = (s + 1) * nb / S;   // 32-bit: S <= 256, nb <= 2^16
  const int ntiles = (N + GD_TILE_N - 1) / GD_TILE_N;
  // this thread's output in the epilogue (threads >= R * 16 own none)
  const int om = tid >> 4, oc = tid & 15;
  const bool orow = tid < R * 16 && om < M;

  // ---- staging of blocks [cb, ce). stage_issue loads this wave's rows (and the norm's
  // gain and shift); it runs before the weight loads, so that waiting for the rows does
  // not wait for the weights (vector loads complete in issue order). stage_finish
  // normalizes, writes the rows to LDS and reads this wave's operand blocks into xr.
  F8 xr[MM_JB][MT];          // this wave's operand blocks (fp32 products)
  u32x4 xp[MM_JB][MT][3];    // the same as three bf16 parts (PT)
  f32x4 v[RPW][MM_JB], g[MM_JB], bb[MM_JB];
  f32x4 ao[RPW][GD_ATT_NCH];    // PRO_ATTN: the chunks' values of this lane's float4
  float2 aml[RPW];              // and chunk (lane & 7)'s (max, sum)
  auto stage_issue = [&](int cb, int ce) {
    const int ka = cb * 32;
    const int kq = (min(ce * 32, K) - ka) >> 2;   // float4 chunks of real columns per row
    const int pc = ((ce - cb) * 8 + 63) >> 6;     // chunks per lane (padded range)
    if constexpr (PRO == PRO_ATTN) {
      // slot 0 only (a split spans <= 256 columns); rows >= M (wave-uniform) are not
      // loaded; chunks past nch repeat the last one and get weight 0
      const int hd = p.hd, stride = gd_apart_stride(hd), C = p.nch;
      const int col = ka + 4 * min(lane, kq - 1);
      const int hh = col / hd, dd = col - hh * hd;
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        if (wave + MM_NW * i < M) {
          const float* pp = p.apart + ((size_t)(wave + MM_NW * i) * p.Hq + hh) * C * stride;
          aml[i] = *reinterpret_cast<const float2*>(pp + (size_t)min(lane & 7, C - 1) * stride);
#pragma unroll
          for (int c = 0; c < GD_ATT_NCH; ++c)
            ao[i][c] = *reinterpret_cast<const f32x4*>(pp + (size_t)min(c, C - 1) * stride + GD_APART_O + dd);
        }
      }
      return;
    }
    // Without a norm only the slots of the range's padded blocks are loaded (j < pc, a
    // wave-uniform test: the load pipeline of a CU is the bottleneck there); with a
    // norm every slot is, which keeps the statistics free of branches. Lanes past the
    // range read a clamped chunk of the same row. No load is under a per-lane
    // condition: such a load would be compiled as a branch of its own, waiting for
    // everything issued before it. NRM_EXPLICIT zeroes the lanes past the range (by a
    // product: a select would let the compiler sink the load again).
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int m = min(wave + MM_NW * i, M - 1);
#pragma unroll
      for (int j = 0; j < MM_JB; ++j) {
        if (NRM != NRM_NONE || j < pc) {
          const int ch = lane + 64 * j;
          const f32x4 t = *reinterpret_cast<const f32x4*>(p.x + (size_t)m * p.ldx + ka + 4 * min(ch, kq - 1));
          if constexpr (NRM == NRM_EXPLICIT) {
            const float keep = ch < kq ? 1.f : 0.f;
            v[i][j] = (f32x4){t.x * keep, t.y * keep, t.z * keep, t.w * keep};
          } else {
            v[i][j] = t;
          }
        }
      }
    }
    if constexpr (NRM == NRM_EXPLICIT) {
      const float* bsrc = p.norm == NORM_LN ? p.nb : p.ng;   // RMSNorm: shift 0 (bsel below)
#pragma unroll
      for (int j = 0; j < MM_JB; ++j) {
        const int ch = lane + 64 * j, cc = 4 * min(ch, kq - 1);
        const float keep = ch < kq ? 1.f : 0.f;
        const f32x4 tg = *reinterpret_cast<const f32x4*>(p.ng + cc);
        const f32x4 tb = *reinterpret_cast<const f32x4*>(bsrc + cc);
        g[j] = (f32x4){tg.x * keep, tg.y * keep, tg.z * keep, tg.w * keep};
        bb[j] = (f32x4){tb.x * keep, tb.y * keep, tb.z * keep, tb.w * keep};
      }
    }
  };
  // NRM_FOLDED: each staged row's r = 1 / sqrt(var + eps) and a = mean of the shifted
  // row, into LDS (read by the epilogue after the partial-tile barrier). Lanes past the
  // range are masked by selects (no branches).
  auto fold_stats = [&](int pc, int kq) {
    (void)pc;
    const bool ln = p.norm == NORM_LN;
    const float invK = 1.0f / (float)K;
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      float st[2] = {0.f, 0.f};
#pragma unroll
      for (int j = 0; j < MM_JB; ++j) {
        const f32x4 d = v[i][j];
        const bool in = lane + 64 * j < kq;
        const float cs = (d.x + d.y) + (d.z + d.w);
        const float cq = fmaf(d.x, d.x, d.y * d.y) + fmaf(d.z, d.z, d.w * d.w);
        st[0] += in ? cs : 0.f;
        st[1] += in ? cq : 0.f;
      }
      wave_sum_n<2>(st);
      const float a = ln ? st[0] * invK : 0.f;
      const float var = fmaxf(st[1] * invK - a * a, 0.f);
      if (lane == 0) {
        s_rs[wave + MM_NW * i] = rsqrtf(var + p.eps);
        s_mu[wave + MM_NW * i] = a;
      }
    }
  };
  auto stage_finish = [&](int cb, int ce) {
    const int kq = (min(ce * 32, K) - cb * 32) >> 2;
    const int kqp = (ce - cb) * 8;
    const int pc = (kqp + 63) >> 6;
    if constexpr (PRO == PRO_ATTN) {
      // each real row: chunk weights within each 8-lane group (lane c: chunk c), then
      // the weighted values in chunk order; rows >= M stage zeros
      static_assert(GD_ATT_NCH == 8, "one chunk per lane of an 8-lane group");
      const int gb = lane & ~7;
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        f32x4 o = f4_zero();
        if (wave + MM_NW * i < M) {
          const bool live = (lane & 7) < p.nch;
          const float mc = live ? aml[i].x : -INFINITY;
          const float mx = group_max<GD_ATT_NCH>(mc);
          const float e = expf(mc - mx);
          const float l = group_sum<GD_ATT_NCH>((live ? aml[i].y : 0.f) * e);
          const float w = e / l;
#pragma unroll
          for (int c = 0; c < GD_ATT_NCH; ++c) {
            const float wc = __shfl(w, gb + c);
            o.x = fmaf(wc, ao[i][c].x, o.x);
            o.y = fmaf(wc, ao[i][c].y, o.y);
            o.z = fmaf(wc, ao[i][c].z, o.z);
            o.w = fmaf(wc, ao[i][c].w, o.w);
          }
        }
        v[i][0] = o;
      }
    }
    if constexpr (NRM == NRM_FOLDED) {
      // shift each row by its first element (lane 0, slot 0): the shifted row is what the
      // MFMAs see; then its moments
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        const float shf =
            p.norm == NORM_LN ? __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v[i][0].x))) : 0.f;
#pragma unroll
        for (int j = 0; j < MM_JB; ++j) {
          f32x4& d = v[i][j];
          d.x -= shf; d.y -= shf; d.z -= shf; d.w -= shf;
        }
      }
      fold_stats(pc, kq);
    }
    if constexpr (NRM == NRM_EXPLICIT) {
      // two-pass moments of each whole row (S == 1: the range is the row)
      const bool ln = p.norm == NORM_LN;
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        float s1 = 0.f;
#pragma unroll
        for (int j = 0; j < MM_JB; ++j) s1 += (v[i][j].x + v[i][j].y) + (v[i][j].z + v[i][j].w);   // zeros past K
        const float mu = ln ? wave_sum(s1) / (float)K : 0.f;
        float s2 = 0.f;
#pragma unroll
        for (int j = 0; j < MM_JB; ++j) {
          const int ch = lane + 64 * j;
          if (j < pc && ch < kq) {
            const float d0 = v[i][j].x - mu, d1 = v[i][j].y - mu, d2 = v[i][j].z - mu, d3 = v[i][j].w - mu;
            s2 += fmaf(d0, d0, d1 * d1) + fmaf(d2, d2, d3 * d3);
          }
        }
        const float r = 1.0f / sqrtf(wave_sum(s2) / (float)K + p.eps);
        const float bsel = ln ? 1.f : 0.f;
#pragma unroll
        for (int j = 0; j < MM_JB; ++j) {
          v[i][j].x = (v[i][j].x - mu) * r * g[j].x + bsel * bb[j].x;
          v[i][j].y = (v[i][j].y - mu) * r * g[j].y + bsel * bb[j].y;
          v[i][j].z = (v[i][j].z - mu) * r * g[j].z + bsel * bb[j].z;
          v[i][j].w = (v[i][j].w - mu) * r * g[j].w + bsel * bb[j].w;
        }
      }
    }
    // Slots of the range's padded 32-column blocks are stored, the rest skipped by a
    // wave-uniform test (the loads cannot sink into it: a scheduling barrier separates
    // them). Slots past the range are never read as operands.
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int m = wave + MM_NW * i;
#pragma unroll
      for (int j = 0; j < MM_JB; ++j) {
        const int ch = lane + 64 * j;
        if (j < pc && (PRO == PRO_COPY || j == 0)) *reinterpret_cast<f32x4*>(xs + m * MM_LDX + 4 * ch) = v[i][j];
      }
    }
    (void)kqp;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < MM_JB; ++j) {
      // block within the range (clamped: slots past the range are never multiplied)
      const int blk = min(wave + MM_NW * j, ce - cb - 1);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const float* src = xs + (mt * 16 + c) * MM_LDX + blk * 32 + 8 * q;
        if constexpr (PT) {
          split3x8(*reinterpret_cast<const f32x4*>(src), *reinterpret_cast<const f32x4*>(src + 4), xp[j][mt]);
        } else {
          xr[j][mt].a = *reinterpret_cast<const f32x4*>(src);
          xr[j][mt].b = *reinterpret_cast<const f32x4*>(src + 4);
        }
      }
    }
    __syncthreads();   // the staging area is reused for the partial tiles
  };
  // weights of tile t for this wave's blocks of [cb, ce) (unused slots repeat the last
  // block: loads stay unconditional); more = false reads 16 bytes at the base instead
  auto load_w = [&](W8<WT> (&w)[MM_JB], int t, int cb, int ce, bool more) {
#pragma unroll
    for (int j = 0; j < MM_JB; ++j) {
      const int blk = min(cb + wave + MM_NW * j, ce - 1);
      w[j] = load_w8tile<WT>(p.wtl, more ? (size_t)t * nb + blk : 0, more ? lane : 0);
    }
  };

  // every kernel argument the launch reads, loaded at once (left to itself the compiler
  // loads each just before its first use, inside the branch that uses it)
  asm volatile("" ::"s"(p.x), "s"(p.ldx), "s"(p.ng), "s"(p.nb), "s"(p.norm), "s"(p.eps), "s"(p.wtl), "s"(p.bias),
               "s"(p.resid), "s"(p.ldr), "s"(p.y), "s"(p.ldy));
  if constexpr (PRO == PRO_ATTN) asm volatile("" ::"s"(p.apart), "s"(p.Hq), "s"(p.hd), "s"(p.nch));
  W8<WT> wa[MM_JB], wb[MM_JB];   // this tile's weights and the next tile's
  int t = wg;
  if constexpr (!MP) {
    stage_issue(b0, b1);
    load_w(wa, t, b0, b1, true);   // the first tile's weights stream while the rows are staged
    // keep every load above issued here: the scheduler would otherwise move the weight
    // loads below the waits for the rows, adding a memory round trip
    __builtin_amdgcn_sched_barrier(0);
    stage_finish(b0, b1);
  }

  float bv = -INFINITY;   // argmax: running best of this thread's columns
  int bi = 0x7fffffff;
  // One tile with its weights in w; the next tile's weights go to wn before this tile's
  // MFMAs (unconditional: past the last tile they read 16 bytes at the base).
  auto tile = [&](int t, int it, W8<WT> (&w)[MM_JB], W8<WT> (&wn)[MM_JB]) {
    // epilogue operands of this thread's output(s) of the tile
    const int n = t * GD_TILE_N + oc;
    const bool own = orow && (PAIR ? n + 1 < N : n < N);
    const EpiOps eo = epi_prefetch<EPI, NRM == NRM_FOLDED>(p, own ? om : 0, own ? n : 0);
    if constexpr (!MP) load_w(wn, t + G, b0, b1, t + G < ntiles);
    __builtin_amdgcn_sched_barrier(0);   // the loads above go out before this tile's MFMAs
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f4_zero();
    for (int cb = b0; cb < b1; cb += MM_NW * MM_JB) {
      const int ce = min(b1, cb + MM_NW * MM_JB);
      if constexpr (MP) {
        __syncthreads();   // the previous tile's partials have been read
        stage_issue(cb, ce);
        load_w(w, t, cb, ce, true);
        stage_finish(cb, ce);
      }
#pragma unroll
      for (int j = 0; j < MM_JB; ++j) {
        if (cb + wave + MM_NW * j < ce && !PT) {   // wave-uniform: MFMAs run with the whole wave
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int u = 0; u < 8; ++u)
              acc[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(f8_at(xr[j][mt], u), w8_at<WT>(w[j], u), acc[mt], 0, 0, 0);
        }
        if (cb + wave + MM_NW * j < ce && PT) {
          constexpr int NW = WT == 0 ? 3 : 1;   // parts of a weight
          u32x4 wp[3];
          if constexpr (WT == 0) split3x8(w[j].a, w[j].b, wp);
          else wp[0] = w[j].a;
          // the part pairs (pa, pw) with pa + pw <= 2, smallest terms first
#pragma unroll
          for (int sp = 2; sp >= 0; --sp)
#pragma unroll
            for (int pa = 0; pa <= sp; ++pa) {
              const int pw = sp - pa;
              if (pw >= NW) continue;
#pragma unroll
              for (int mt = 0; mt < MT; ++mt)
                acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xp[j][mt][pa]),
                                                                  __builtin_bit_cast(bf16x8_t, wp[pw]), acc[mt], 0, 0, 0);
            }
        }
      }
    }
    settle(eo.b0); settle(eo.b1); settle(eo.r0); settle(eo.c); settle(eo.s); settle(eo.f0);
    settle(__int_as_float((int)eo.kvoff)); settle(__int_as_float((int)(eo.kvoff >> 32)));
    float* red = xs + (it & 1) * (MM_NW * R * RS);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      float* rw = red + (wave * R + mt * 16 + 4 * q) * RS + c;
      rw[0] = acc[mt].x;
      rw[RS] = acc[mt].y;
      rw[2 * RS] = acc[mt].z;
      rw[3 * RS] = acc[mt].w;
    }
    __syncthreads();   // the other buffer is rewritten only after the next tile's barrier
    if (tid < R * 16) {
      float v = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < MM_NW; ++w2) v += red[(w2 * R + om) * RS + oc];
      if (NRM == NRM_FOLDED) {
        v = s_rs[om] * (v - s_mu[om] * eo.f0);
        if (EPI == EPI_ARGMAX) v += eo.b0;   // the folded bias (other epilogues add it)
      }
      if (EPI == EPI_ARGMAX) {
        if (own) {
          if (p.logits) p.logits[(size_t)om * p.ldl + n] = v;
          if (am_better(v, n, bv, bi)) { bv = v; bi = n; }
        }
      } else if (PAIR) {
        const float v1 = dpp_f<DPP_QUAD_1032>(v);   // the odd neighbour's column
        if (own && (oc & 1) == 0) epi_store<EPI>(p, eo, om, n, v, v1);
      } else if (own) {
        if (EPI == EPI_PLAIN && S > 1)
          __hip_atomic_fetch_add(p.y + (size_t)om * p.ldy + n, v + (s == 0 ? eo.b0 : 0.f), __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
        else
          epi_store<EPI>(p, eo, om, n, v, 0.f);
      }
    }
  };
  // the two weight buffers alternate between consecutive tiles
  for (int it = 0; t < ntiles;) {
    tile(t, it, wa, wb);
    t += G; ++it;
    if (t >= ntiles) break;
    tile(t, it, wb, wa);
    t += G; ++it;
  }
  if (EPI == EPI_ARGMAX && tid < R * 16) {
    // best of the 16 threads of each row (one 16-lane DPP row)
#define MM_AM_STEP(CTRL)                                   \
    {                                                      \
      const float ov = dpp_f<CTRL>(bv);                    \
      const int oi = dpp_i<CTRL>(bi);                      \
      if (am_better(ov, oi, bv, bi)) { bv = ov; bi = oi; } \
    }
    MM_AM_STEP(DPP_QUAD_1032)
    MM_AM_STEP(DPP_QUAD_2301)
    MM_AM_STEP(DPP_ROW_HALF_MIRROR)
    MM_AM_STEP(DPP_ROW_MIRROR)
#undef MM_AM_STEP
    if (oc == 0 && om < M) {
      p.am_val[(size_t)wg * M + om] = bv;
      p.am_idx[(size_t)wg * M + om] = bi;
    }
  }
}

// Greedy argmax over the per-workgroup partials of one row (one workgroup per row).
// Every thread loads all of its partials before comparing, so the reduction costs
// one memory round trip. nparts <= GD_WG * AM_FIN_PER.
#define AM_FIN_PER 16
// With adv_len (a decode step whose set-up ran in its QKV launch) it also advances the
// row's sequence length: adv_len[adv_seq[m]] = adv_pos[m] + 1.
__global__ __launch_bounds__(GD_WG) void k_argmax_finalize(const float* __restrict__ val, const int* __restrict__ idx,
                                                           int nparts, int M, int* out, const int* __restrict__ adv_seq,
                                                           const int* __restrict__ adv_pos, int* adv_len) {
  __shared__ float sv[GD_WG / 64];
  __shared__ int si[GD_WG / 64];
  const int m = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float v[AM_FIN_PER];
  int ix[AM_FIN_PER];
#pragma unroll
  for (int j = 0; j < AM_FIN_PER; ++j) {
    const int q = tid + GD_WG * j;
    v[j] = q < nparts ? val[(size_t)q * M + m] : 0.f;
    ix[j] = q < nparts ? idx[(size_t)q * M + m] : 0x7fffffff;
  }
  // the row's slot and position after the partials are issued (a wait for them then
  // does not hold the partials back)
  __builtin_amdgcn_sched_barrier(0);
  int aseq = 0, apos = 0;
  if (adv_len) {
    aseq = adv_seq[m];
    apos = adv_pos[m];
  }
  float bv = v[0];
  int bi = ix[0];
#pragma unroll
  for (int j = 1; j < AM_FIN_PER; ++j)
    if (ix[j] != 0x7fffffff && (bi == 0x7fffffff || am_better(v[j], ix[j], bv, bi))) { bv = v[j]; bi = ix[j]; }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (oi != 0x7fffffff && (bi == 0x7fffffff || am_better(ov, oi, bv, bi))) { bv = ov; bi = oi; }
  }
  if (lane == 0) { sv[wave] = bv; si[wave] = bi; }
  __syncthreads();
  if (tid == 0) {
    float v0 = sv[0];
    int i0 = si[0];
    for (int w = 1; w < GD_WG / 64; ++w)
      if (si[w] != 0x7fffffff && (i0 == 0x7fffffff || am_better(sv[w], si[w], v0, i0))) { v0 = sv[w]; i0 = si[w]; }
    out[m] = i0;
    if (adv_len) adv_len[aseq] = apos + 1;
  }
}
