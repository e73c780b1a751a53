// runtime.hip -- host runtime and C ABI of libgptdecode.so (see include/gd.h).
//
// The decode step is one hipGraph launch (one submission per forward pass:
// "bare-metal-llm", "What it taught me"; "rvllm Metal backend", "You record work,
// then you submit it"). Per-step state (positions, lengths, tokens) lives on the
// device, so a captured step replays without host work beyond the launch.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "gd.h"
#include "common.h"
#include "linear.h"
#include "attention.h"
#include "misc.h"
#include "prefill.h"

// ------------------------------------------------------------------ errors

static thread_local std::string g_err;

static gd_status set_err(gd_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

extern "C" const char* gd_last_error(void) { return g_err.c_str(); }

#define HIP_TRY(m, call)                                                                   \
  do {                                                                                     \
    hipError_t e_ = (call);                                                                \
    if (e_ != hipSuccess) {                                                                \
      if (m) (m)->poisoned = true;                                                         \
      return set_err(GD_ERR_HIP, "%s failed: %s (%s:%d)", #call, hipGetErrorString(e_), __FILE__, __LINE__); \
    }                                                                                      \
  } while (0)

static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
static int iceil(int a, int b) { return (a + b - 1) / b; }

// ------------------------------------------------------- launch profiling
//
// While a profiling scope is open on this thread, every launch takes its own start
// and stop events (hipExtLaunchKernelGGL): the events carry the kernel's execution
// timestamps, so a scope's time is the sum of its kernels' execution with no queue or
// host time in it.

static hipEvent_t prof_event(gd_model* m);
static thread_local gd_model* t_prof_m = nullptr;
static thread_local std::vector<std::pair<hipEvent_t, hipEvent_t>>* t_prof_pairs = nullptr;
// where the argmax finalize launches of a profiled head are timed (their own role)
static thread_local std::vector<std::pair<hipEvent_t, hipEvent_t>>* t_prof_fin = nullptr;

#define GD_LAUNCH(K, G, B, L, S, ...)                                     \
  do {                                                                     \
    if (t_prof_pairs) {                                                    \
      hipEvent_t a_ = prof_event(t_prof_m), b_ = prof_event(t_prof_m);     \
      hipExtLaunchKernelGGL(K, G, B, L, S, a_, b_, 0, __VA_ARGS__);        \
      t_prof_pairs->push_back({a_, b_});                                   \
    } else {                                                               \
      hipLaunchKernelGGL(K, G, B, L, S, __VA_ARGS__);                      \
    }                                                                      \
  } while (0)

// ---------------------------------------------------------- linear planning
//
// var 0: k_gemv, VALU dot products with the weight rows held in registers; at most
//        GEMV_MAX_ROWS activation rows per launch (more rows run as several launches).
// var 1: k_mm, 16-column tiles on the fp32 matrix cores; 1..32 rows per launch.

struct LinPlan {
  int var;     // 0 gemv, 1 mm
  int nc, rw;  // gemv: 16-byte weight chunks per lane and row, weight rows per wave
  int mt, nw;  // mm: 16-row activation tiles, waves per workgroup
  int splits;  // mm: K splits (grid.y), > 1 only for in-place residual outputs
  int passes;  // mm: register passes over the K range of one split (MM_KC columns each)
  int rows;    // activation rows per launch
  int grid;
  int parts;   // argmax partials per row (gemv: workgroups; mm: column tiles)
  size_t lds;  // dynamic LDS bytes
};

static const int kNcChoices[] = {1, 2, 3, 4, 6, 8, 12};

// Smallest instantiated chunk count covering K (-1: K too long for the gemv kernel).
static int gemv_nc(int K, int wt) {
  const int ce = wt == GD_WEIGHT_F32 ? 4 : wt == GD_WEIGHT_BF16 ? 8 : 16;
  const int need = iceil(iceil(K, ce), 64);
  for (int c : kNcChoices)
    if (c >= need) return c;
  return -1;
}

// variant: 0 auto (gemv for <= GEMV_MAX_ROWS rows), 1 gemv, 2 mfma.
// norm: the prologue normalizes the rows (LDS for statistics, gain and shift).
static int gemv_rows_per_wave(int epi, int N) {
  if (epi == EPI_SWIGLU || epi == EPI_QKV_ROPE) return 2;   // both rows of a pair in one wave
  // a wide head: four rows per wave (8-bit heads with 16 rows per wave measured 61 us
  // against 21 us at GPT-2 124M: each wave then serializes 16 cross-lane sums)
  if (epi == EPI_ARGMAX && N >= 16384) return 4;
  return 1;
}

static const size_t kGemvLdsMax = 64 * 1024;
// Widest reduction (K) of a linear layer: keeps the matrix-core kernel's split bounds
// (split index x 32-column blocks) in 32-bit arithmetic.
static const int kMaxK = 1 << 20;
static const int kMmTargetWgs = 256;   // one matrix-core workgroup per CU

// splittable: linear epilogue whose output is the residual, updated in place (the
// K splits are then summed with atomics into it). attn_rows: the rows are merged from
// split-context attention partials (PRO_ATTN), which the matrix-core kernel does for
// up to 16 rows with splits of at most 256 columns (head_dim a multiple of 32).
static LinPlan plan_linear(int M, int N, int K, int wt, int variant, int epi, bool norm, bool splittable = false,
                           bool attn_rows = false) {
  LinPlan p;
  memset(&p, 0, sizeof(p));
  p.var = variant == 1 ? 0 : variant == 2 ? 1 : (M <= GEMV_MAX_ROWS ? 0 : 1);
  if (wt == GD_WEIGHT_Q8) p.var = 0;   // 8-bit weights: the VALU kernel only (launches of <= 4 rows)
  p.nc = gemv_nc(K, wt);
  if (p.var == 1 && norm && K > MM_KC) p.var = 0;   // the norm needs whole rows in one register pass
  if (p.var == 0 && p.nc < 0 && wt != GD_WEIGHT_Q8) p.var = 1;
  if (p.var == 0) {
    p.rw = gemv_rows_per_wave(epi, N);
    p.rows = std::min(M, GEMV_MAX_ROWS);
    p.grid = iceil(N, 4 * p.rw);
    p.parts = p.grid;
    // the activation rows (a pre-norm is applied in registers)
    const size_t xs = ((size_t)p.rows * K + 3) & ~(size_t)3;
    p.lds = xs * sizeof(float);
    if (p.lds > kGemvLdsMax && !(norm && K > MM_KC) && wt != GD_WEIGHT_Q8) p.var = 1;   // rows too long to stage
  }
  if (p.var == 1) {
    const int ntiles = iceil(N, GD_TILE_N), nb = iceil(K, 32);
    p.mt = M <= 16 ? 1 : 2;
    p.nw = MM_NW;
    p.rows = M;
    p.splits = 1;
    // split K only as far as one workgroup per CU allows (a second round of workgroups
    // would double the kernel's time)
    if (splittable && !norm && epi == EPI_PLAIN) {
      p.splits = std::max(1, std::min(nb, kMmTargetWgs / ntiles));
      p.splits = std::max(p.splits, iceil(nb, MM_KC / 32));   // one register pass per split
      if (attn_rows) p.splits = std::max(p.splits, iceil(nb, 8));   // one float4 slot per lane
    }
    p.passes = iceil(iceil(nb, p.splits) * 32, MM_KC);
    // at most one workgroup per CU; wider layers stream several tiles per workgroup
    p.grid = std::min(ntiles, kMmTargetWgs);
    p.parts = p.grid;
    p.lds = 0;
  }
  return p;
}

// With a pre-norm whose folded form is given (fp32 weights, prm.wf), the folded
// weights, bias and row sums replace the layer's own (NRM_FOLDED). es: the embedding
// prologue's sources (prm.pro == PRO_EMBED).
template <int WT, int NC>
static hipError_t launch_gemv_nc(const LinPlan& lp, const LinParams& prm0, hipStream_t st, const EmbSrc* es) {
  const dim3 g(lp.grid), b(GD_WG);
  const bool nrm = prm0.norm != NORM_NONE;
  const bool fold = WT == 0 && nrm && prm0.wf;
  LinParams prm = prm0;
  if (fold) {
    prm.w = prm0.wf;
    prm.bias = prm0.bf;
  }
#define GD_GEMV(RW, EPI, PRO, NRM) GD_LAUNCH((k_gemv<WT, NC, RW, EPI, PRO, NRM>), g, b, lp.lds, st, prm)
#define GD_GEMV_N(RW, EPI)                                                   \
  do {                                                                       \
    if (fold) GD_GEMV(RW, EPI, PRO_COPY, NRM_FOLDED);                        \
    else GD_GEMV(RW, EPI, PRO_COPY, NRM_EXPLICIT);                           \
  } while (0)
  if (prm.pro == PRO_ATTN) {   // the output projection behind split-context attention
    if (prm.epi != EPI_PLAIN || nrm) return hipErrorNotSupported;
    GD_GEMV(1, EPI_PLAIN, PRO_ATTN, NRM_NONE);
    return hipSuccess;
  }
  if (prm.pro == PRO_EMBED) {   // the decode step's first QKV launch, its set-up included
    if (!nrm || !es || lp.rows < prm.M) return hipErrorNotSupported;
    LinEmbParams eprm;
    static_cast<LinParams&>(eprm) = prm;
    eprm.e = *es;
#define GD_GEMV_E(RW, EPI, NRM) GD_LAUNCH((k_gemv<WT, NC, RW, EPI, PRO_EMBED, NRM>), g, b, lp.lds, st, eprm)
    if (prm.epi == EPI_QKV) {
      if (fold) GD_GEMV_E(1, EPI_QKV, NRM_FOLDED);
      else GD_GEMV_E(1, EPI_QKV, NRM_EXPLICIT);
    } else if (prm.epi == EPI_QKV_ROPE) {
      if (fold) GD_GEMV_E(2, EPI_QKV_ROPE, NRM_FOLDED);
      else GD_GEMV_E(2, EPI_QKV_ROPE, NRM_EXPLICIT);
    } else {
      return hipErrorNotSupported;
    }
#undef GD_GEMV_E
    return hipSuccess;
  }
  switch (prm.epi) {
    case EPI_PLAIN: if (nrm) GD_GEMV_N(1, EPI_PLAIN); else GD_GEMV(1, EPI_PLAIN, PRO_COPY, NRM_NONE); break;
    case EPI_GELU: if (nrm) GD_GEMV_N(1, EPI_GELU); else GD_GEMV(1, EPI_GELU, PRO_COPY, NRM_NONE); break;
    // the remaining epilogues always follow a pre-norm
    case EPI_QKV: if (!nrm) return hipErrorNotSupported; GD_GEMV_N(1, EPI_QKV); break;
    case EPI_SWIGLU: if (!nrm) return hipErrorNotSupported; GD_GEMV_N(2, EPI_SWIGLU); break;
    case EPI_QKV_ROPE: if (!nrm) return hipErrorNotSupported; GD_GEMV_N(2, EPI_QKV_ROPE); break;
    default:
      if (!nrm) return hipErrorNotSupported;
      if (lp.rw == 4) GD_GEMV_N(4, EPI_ARGMAX);
      else GD_GEMV_N(1, EPI_ARGMAX);
      break;
  }
#undef GD_GEMV_N
#undef GD_GEMV
  return hipSuccess;
}

template <int WT>
static hipError_t launch_gemv(const LinPlan& lp, const LinParams& prm, hipStream_t st, const EmbSrc* es) {
  switch (lp.nc) {
    case 1: return launch_gemv_nc<WT, 1>(lp, prm, st, es);
    case 2: return launch_gemv_nc<WT, 2>(lp, prm, st, es);
    case 3: return launch_gemv_nc<WT, 3>(lp, prm, st, es);
    case 4: return launch_gemv_nc<WT, 4>(lp, prm, st, es);
    case 6: return launch_gemv_nc<WT, 6>(lp, prm, st, es);
    case 8: return launch_gemv_nc<WT, 8>(lp, prm, st, es);
    default: return launch_gemv_nc<WT, 12>(lp, prm, st, es);
  }
}

// Whether a matrix-core launch multiplies on the bf16 matrix cores in parts: when its
// workgroups stream several tiles (the head; the SwiGLU up-projection with the norm
// applied to the rows), where the faster products outweigh splitting the activations
// (with one tile per workgroup they measured slower).
static bool mm_parts(const LinPlan& lp, int N, int epi, bool fold) {
  if (lp.var != 1 || lp.passes != 1 || iceil(N, GD_TILE_N) <= lp.grid) return false;
  return epi == EPI_ARGMAX || (epi == EPI_SWIGLU && !fold);
}

// A pre-norm whose folded form is given (fp32 weights, prm.wfl) runs as NRM_FOLDED on
// the folded tile-major weights, bias and row sums.
template <int WT, int MT>
static hipError_t launch_mm_mt(const LinPlan& lp, const LinParams& prm0, hipStream_t st) {
  const dim3 g(lp.grid, lp.splits), b(64 * MM_NW);
  const bool nrm = prm0.norm != NORM_NONE;
  const bool fold = WT == 0 && nrm && prm0.wfl;
  LinParams prm = prm0;
  if (fold) {
    prm.wtl = prm0.wfl;
    prm.bias = prm0.bf;
  }
#define GD_MM(EPI, NRM, MP) GD_LAUNCH((k_mm<WT, MT, EPI, NRM, MP, PRO_COPY, false>), g, b, 0, st, prm)
  const bool pt = mm_parts(lp, prm.N, prm.epi, fold);
#define GD_MM_PT(EPI, NRM) GD_LAUNCH((k_mm<WT, MT, EPI, NRM, false, PRO_COPY, true>), g, b, 0, st, prm)
#define GD_MM_N(EPI)                                   \
  do {                                                 \
    if (fold) GD_MM(EPI, NRM_FOLDED, false);           \
    else GD_MM(EPI, NRM_EXPLICIT, false);              \
  } while (0)
  if (prm.pro == PRO_EMBED) return hipErrorNotSupported;   // embedding rows: the GEMV only
  if (prm.pro == PRO_ATTN) {   // the output projection behind split-context attention (<= 16 rows)
    if constexpr (MT == 1) {
      if (nrm || prm.epi != EPI_PLAIN || lp.passes > 1 || prm.nch < 1 || prm.nch > GD_ATT_NCH || prm.hd % 32 ||
          iceil(iceil(prm.K, 32), lp.splits) > 8)
        return hipErrorNotSupported;
      GD_LAUNCH((k_mm<WT, MT, EPI_PLAIN, NRM_NONE, false, PRO_ATTN, false>), g, b, 0, st, prm);
      return hipSuccess;
    }
    return hipErrorNotSupported;
  }
  if (lp.passes > 1) {   // K range wider than one pass: plain or GELU epilogue, no norm
    if (nrm) return hipErrorNotSupported;
    if (prm.epi == EPI_PLAIN) GD_MM(EPI_PLAIN, NRM_NONE, true);
    else if (prm.epi == EPI_GELU) GD_MM(EPI_GELU, NRM_NONE, true);
    else return hipErrorNotSupported;
    return hipSuccess;
  }
  switch (prm.epi) {
    case EPI_PLAIN: if (nrm) GD_MM_N(EPI_PLAIN); else GD_MM(EPI_PLAIN, NRM_NONE, false); break;
    case EPI_GELU: if (nrm) GD_MM_N(EPI_GELU); else GD_MM(EPI_GELU, NRM_NONE, false); break;
    // the remaining epilogues always follow a pre-norm
    case EPI_SWIGLU:
      if (!nrm) return hipErrorNotSupported;
      if (pt) GD_MM_PT(EPI_SWIGLU, NRM_EXPLICIT);
      else GD_MM_N(EPI_SWIGLU);
      break;
    case EPI_ARGMAX:
      if (!nrm) return hipErrorNotSupported;
      if (pt && fold) GD_MM_PT(EPI_ARGMAX, NRM_FOLDED);
      else if (pt) GD_MM_PT(EPI_ARGMAX, NRM_EXPLICIT);
      else GD_MM_N(EPI_ARGMAX);
      break;
    case EPI_QKV: if (!nrm) return hipErrorNotSupported; GD_MM_N(EPI_QKV); break;
    case EPI_QKV_ROPE: if (!nrm) return hipErrorNotSupported; GD_MM_N(EPI_QKV_ROPE); break;
    default: return hipErrorNotSupported;
  }
#undef GD_MM_N
#undef GD_MM_PT
#undef GD_MM
  return hipSuccess;
}

template <int WT>
static hipError_t launch_mm(const LinPlan& lp, const LinParams& prm, hipStream_t st) {
  return lp.mt == 1 ? launch_mm_mt<WT, 1>(lp, prm, st) : launch_mm_mt<WT, 2>(lp, prm, st);
}

// One launch of one plan over prm.M rows (prm.M <= lp.rows).
static hipError_t launch_linear(int wt, const LinPlan& lp, const LinParams& prm, hipStream_t st, const EmbSrc* es) {
  if (lp.var == 0) {
    const hipError_t e = wt == GD_WEIGHT_F32    ? launch_gemv<0>(lp, prm, st, es)
                         : wt == GD_WEIGHT_BF16 ? launch_gemv<1>(lp, prm, st, es)
                                                : launch_gemv<2>(lp, prm, st, es);
    if (e != hipSuccess) return e;
  } else {
    const hipError_t e = wt == GD_WEIGHT_F32 ? launch_mm<0>(lp, prm, st) : launch_mm<1>(lp, prm, st);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

// A decode step whose set-up ran in its first QKV launch: the head's argmax finalize
// advances len[seq[b]] to pos[b] + 1 for its rows b.
struct AdvLen {
  int* len; const int* seq; const int* pos;
};

// Runs a linear layer over prm.M rows, as several launches of at most lp.rows rows when
// needed (every per-row pointer advances with the row group). With EPI_ARGMAX each
// group's per-workgroup partials are reduced into am_out[rows of the group].
static hipError_t run_linear_rows(int wt, const LinPlan& lp, const LinParams& prm, hipStream_t st, int* am_out,
                                  const EmbSrc* es, const AdvLen* adv) {
  for (int r0 = 0; r0 < prm.M; r0 += lp.rows) {
    LinParams p = prm;
    p.M = std::min(lp.rows, prm.M - r0);
    if (r0 && prm.pro == PRO_EMBED) return hipErrorNotSupported;   // its rows' arrays do not advance
    if (r0) {
      if (p.x) p.x += (size_t)r0 * p.ldx;
      p.resid += (size_t)r0 * p.ldr;
      if (p.y) p.y += (size_t)r0 * p.ldy;
      if (p.logits) p.logits += (size_t)r0 * p.ldl;
      if (p.row_kvoff) p.row_kvoff += r0;
      if (p.rope_cs) p.rope_cs += (size_t)r0 * p.hd;
      if (p.apart) p.apart += (size_t)r0 * p.Hq * p.nch * gd_apart_stride(p.hd);
    }
    hipError_t e = launch_linear(wt, lp, p, st, es);
    if (e != hipSuccess) return e;
    if (p.epi == EPI_ARGMAX) {
      auto* keep = t_prof_pairs;
      if (t_prof_pairs) t_prof_pairs = t_prof_fin;
      GD_LAUNCH(k_argmax_finalize, dim3(p.M), dim3(GD_WG), 0, st, p.am_val, p.am_idx, lp.parts, p.M, am_out + r0,
                adv ? adv->seq + r0 : nullptr, adv ? adv->pos + r0 : nullptr, adv ? adv->len : nullptr);
      t_prof_pairs = keep;
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

// ------------------------------------------------------------------- model

struct LayerOff {
  size_t n1g, n1b, wqkv, bqkv, wo, bo, n2g, n2b, wfc, bfc, wproj, bproj;
  size_t sqkv, so, sfc, sproj;   // 8-bit weights: block scales of the matrices (0: none)
  size_t tqkv, to, tfc, tproj;   // tile-major copies of the matrices (matrix-core kernel)
  // pre-norm folded into QKV and MLP-up (fp32): weights, bias, row sums (0: none)
  size_t fqkv, fqkv_b, fqkv_s, ffc, ffc_b, ffc_s;
  size_t tfqkv, tffc;   // their tile-major copies
};

struct GraphKey {
  int batch;
  const void* tok;
  void* next;
  void* logits;
  bool short_ctx;   // every row attends to at most kFusedAttnOMaxT positions
  bool long_ctx;    // some row attends to at least kLongCtxT positions
  bool operator<(const GraphKey& o) const {
    return std::tie(batch, tok, next, logits, short_ctx, long_ctx) <
           std::tie(o.batch, o.tok, o.next, o.logits, o.short_ctx, o.long_ctx);
  }
};

// Rows of at most this many positions (and few rows) run attention fused with the output
// projection: every projection slice recomputes the attention from K/V in cache.
static const int kFusedAttnOMaxT = 256;
// From this many attended positions, launches with few (row, KV head) pairs split each
// context into GD_ATT_NCH_LONG chunks (merged by k_attn_merge_n) instead of GD_ATT_NCH.
static const int kLongCtxT = 1024;
// Decode-step graphs kept per model.
static const size_t kMaxGraphs = 16;
// Prompts of at least kPrefillMinRows tokens run the tiled prompt pass, kPrefillChunk
// rows at a time; shorter ones run the decode kernels over <= 32 rows per pass.
static const int kPrefillMinRows = 64;
static const int kPrefillChunk = 512;

struct gd_model {
  gd_config c;
  hipStream_t stream = nullptr;
  hipStream_t cap_stream = nullptr;
  bool poisoned = false;
  int variant = 0;
  bool use_graph = true;
  bool fuse_attn_o = true;
  int attn_chunks = 0;   // split-context chunks per row: 0 auto, 1 or GD_ATT_NCH (GD_OPT_ATTN_CHUNKS)
  bool use_fold = true;  // GEMV pre-norms folded into the weights when available (GD_OPT_FOLD_NORM)
  bool use_pf = true;    // long prompts take the tiled prompt pass (GD_OPT_TILED_PREFILL)
  int pf_parts = 1;      // prompt GEMMs on the bf16 matrix cores in parts (GD_OPT_PREFILL_BF16_PARTS)
  // temperature / top-k sampling instead of the greedy argmax (gd_set_sampling)
  bool sample = false;
  int top_k = 1;
  float inv_temp = 1.f;
  unsigned long long seed = 0;
  int dev = 0;
  int n_cu = 0;         // compute units

  // derived shapes
  int qdim, kdim, qkvdim, fcN, hdim, wt;
  int nblk, bsize, max_blocks;
  size_t elt;  // bytes per weight element
  bool kv16 = false;   // the KV cache holds bf16 (GD_KV_BF16)
  size_t kv_elt = 4;   // bytes per KV cache element

  // sizes
  size_t w_bytes = 0, kv_bytes = 0, s_bytes = 0;
  size_t w_rowmajor_bytes = 0;   // the row-major part of the weights (what the caller's values fill)
  size_t am_parts = 0;  // argmax partials per row (workgroups of the head's widest plan)

  // bound memory
  char* w = nullptr;
  char* kv = nullptr;
  char* s = nullptr;
  bool bound = false, loaded = false;

  // weight offsets (bytes)
  size_t o_wte = 0, o_wpe = 0, o_nfg = 0, o_nfb = 0, o_head = 0, o_thead = 0;
  size_t o_swte = 0, o_swpe = 0, o_shead = 0;   // 8-bit weights: block scales of the tables and head
  size_t o_fhead = 0, o_fhead_b = 0, o_fhead_s = 0, o_fold = 0;   // folded final norm + head
  size_t o_tfhead = 0, o_fold_end = 0;   // tile-major folded head; end of the row-major folded part
  bool folded = false;   // the folded copies exist (fp32 weights)
  std::vector<LayerOff> L;

  // scratch offsets (bytes)
  size_t o_x, o_q, o_attn, o_h, o_amv, o_ami, o_apart, o_zero;
  size_t o_slog = 0;   // logits rows the sampler reads when the caller asks for none
  // the tiled prompt pass (kPrefillChunk rows): residual, normalized rows, queries,
  // attention output, MLP hidden
  bool pf_ok = false;
  size_t o_px = 0, o_pxn = 0, o_pq = 0, o_pattn = 0, o_ph = 0, o_ppart = 0;
  size_t o_rseq, o_rpos, o_rtok, o_rkv, o_rcs, o_pseq, o_ppos, o_ptok, o_pkv, o_pcs, o_len, o_cap, o_sids, o_table, o_err, o_rope;

  // host mirror
  std::vector<int> len, cap;
  std::vector<int> last_sids;
  int* staging = nullptr;  // pinned
  size_t staging_ints = 0;
  hipEvent_t staging_evt = nullptr;
  bool staging_pending = false;

  // Captured decode steps, keyed by (batch, step pointers, context bucket), at most
  // kMaxGraphs of them: the least recently launched one is dropped first.
  struct GraphEntry { hipGraphExec_t exec; unsigned long long last_use; };
  std::map<GraphKey, GraphEntry> graphs;
  unsigned long long graph_clock = 0;

  // per-kernel profiling (GD_OPT_PROFILE)
  bool profile = false;
  bool profile_gated = false;   // profiled decode steps wait behind k_gate while enqueued
  hipEvent_t gate_evt = nullptr;
  struct ProfRec { int stat; std::vector<std::pair<hipEvent_t, hipEvent_t>> pairs; double bytes; };
  std::vector<hipEvent_t> ev_free;
  std::vector<ProfRec> prof_pending;
  std::vector<gd_kernel_stat> prof_stats;
  std::vector<int> prof_T;   // attended positions per row of the launch being enqueued

  template <class T>
  T* sp(size_t off) const { return reinterpret_cast<T*>(s + off); }
  template <class T>
  const T* wp(size_t off) const { return reinterpret_cast<const T*>(w + off); }
  const float* wf(size_t off) const { return reinterpret_cast<const float*>(w + off); }
  // K pools of all layers, then V pools; elements of kv_elt bytes (float or bf16)
  void* kpool(int l) const { return kv + (size_t)l * layer_kv_elems() * kv_elt; }
  void* vpool(int l) const { return kv + (size_t)(c.n_layer + l) * layer_kv_elems() * kv_elt; }
  size_t layer_kv_elems() const { return (size_t)nblk * c.n_kv_head * bsize * c.head_dim; }
};

static gd_status check_cfg(const gd_config* c) {
  if (!c) return set_err(GD_ERR_INVALID, "config is NULL");
  if (c->arch != GD_ARCH_GPT2 && c->arch != GD_ARCH_LLAMA) return set_err(GD_ERR_INVALID, "bad arch %d", c->arch);
  if (c->n_layer < 1 || c->d_model < 8 || c->n_head < 1 || c->n_kv_head < 1 || c->d_ff < 8 || c->vocab < 1 ||
      c->n_ctx < 1)
    return set_err(GD_ERR_INVALID, "bad model sizes");
  if (c->head_dim != 16 && c->head_dim != 64) return set_err(GD_ERR_INVALID, "head_dim must be 16 or 64");
  if (c->d_model % 8 || c->d_ff % 8) return set_err(GD_ERR_INVALID, "d_model and d_ff must be multiples of 8");
  if (c->d_model > kMaxK || c->d_ff > kMaxK) return set_err(GD_ERR_INVALID, "d_model and d_ff must be at most %d", kMaxK);
  if (c->arch == GD_ARCH_GPT2 && (c->n_kv_head != c->n_head || c->n_head * c->head_dim != c->d_model))
    return set_err(GD_ERR_INVALID, "GPT-2 arch needs n_kv_head == n_head and n_head*head_dim == d_model");
  if (c->n_head % c->n_kv_head) return set_err(GD_ERR_INVALID, "n_head must be a multiple of n_kv_head");
  if (c->n_head > GD_MAX_HEADS) return set_err(GD_ERR_INVALID, "at most %d query heads", GD_MAX_HEADS);
  int G = c->n_head / c->n_kv_head;
  if (G != 1 && G != 3) return set_err(GD_ERR_INVALID, "query heads per KV head must be 1 or 3");
  if ((c->n_head * c->head_dim) % 8) return set_err(GD_ERR_INVALID, "n_head*head_dim must be a multiple of 8");
  if (c->weight_dtype != GD_WEIGHT_F32 && c->weight_dtype != GD_WEIGHT_BF16 && c->weight_dtype != GD_WEIGHT_Q8)
    return set_err(GD_ERR_INVALID, "bad weight_dtype");
  if (c->weight_dtype == GD_WEIGHT_Q8 && (c->d_model % 32 || c->d_ff % 32 || (c->n_head * c->head_dim) % 32))
    return set_err(GD_ERR_INVALID, "8-bit weights need d_model, d_ff and n_head*head_dim multiples of 32");
  if (c->kv_dtype != GD_KV_F32 && c->kv_dtype != GD_KV_BF16) return set_err(GD_ERR_INVALID, "bad kv_dtype");
  if (c->max_seqs < 1 || c->max_batch < 1 || c->max_batch > GD_MAX_ROWS)
    return set_err(GD_ERR_INVALID, "max_seqs >= 1 and 1 <= max_batch <= 32 required");
  if (c->kv_block_size < 0 || (c->kv_block_size > 0 && c->kv_num_blocks < 1))
    return set_err(GD_ERR_INVALID, "bad paged cache sizes");
  if (!(c->norm_eps > 0.f)) return set_err(GD_ERR_INVALID, "norm_eps must be > 0");
  return GD_OK;
}

static void layout(gd_model* m) {
  const gd_config& c = m->c;
  const size_t d = c.d_model, ff = c.d_ff, V = c.vocab;
  m->wt = c.weight_dtype;
  m->elt = m->wt == GD_WEIGHT_F32 ? 4 : m->wt == GD_WEIGHT_BF16 ? 2 : 1;
  const bool q8 = m->wt == GD_WEIGHT_Q8;
  m->kv16 = c.kv_dtype == GD_KV_BF16;
  m->kv_elt = m->kv16 ? 2 : 4;
  m->qdim = c.n_head * c.head_dim;
  m->kdim = c.n_kv_head * c.head_dim;
  m->qkvdim = m->qdim + 2 * m->kdim;
  m->fcN = c.arch == GD_ARCH_GPT2 ? c.d_ff : 2 * c.d_ff;
  m->hdim = c.d_ff;
  if (c.kv_block_size > 0) {
    m->bsize = c.kv_block_size;
    m->nblk = c.kv_num_blocks;
    m->max_blocks = iceil(c.n_ctx, c.kv_block_size);
  } else {
    m->bsize = c.n_ctx;
    m->nblk = c.max_seqs;
    m->max_blocks = 1;
  }

  // weights
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes, 256); return o; };
  const size_t e = m->elt;
  // a matrix of R rows by K: its elements, then (8-bit weights) its block scales
  auto mat = [&](size_t R, size_t K, size_t& sc) {
    const size_t o = take(R * K * e);
    sc = q8 ? take(R * (K / 32) * 4) : 0;
    return o;
  };
  m->o_wte = mat(V, d, m->o_swte);
  if (c.arch == GD_ARCH_GPT2) m->o_wpe = mat((size_t)c.n_ctx, d, m->o_swpe);
  m->L.resize(c.n_layer);
  for (int l = 0; l < c.n_layer; ++l) {
    LayerOff& t = m->L[l];
    t.n1g = take(d * 4);
    t.n1b = c.arch == GD_ARCH_GPT2 ? take(d * 4) : 0;
    t.wqkv = mat((size_t)m->qkvdim, d, t.sqkv);
    t.bqkv = c.arch == GD_ARCH_GPT2 ? take((size_t)m->qkvdim * 4) : 0;
    t.wo = mat(d, (size_t)m->qdim, t.so);
    t.bo = c.arch == GD_ARCH_GPT2 ? take(d * 4) : 0;
    t.n2g = take(d * 4);
    t.n2b = c.arch == GD_ARCH_GPT2 ? take(d * 4) : 0;
    t.wfc = mat((size_t)m->fcN, d, t.sfc);
    t.bfc = c.arch == GD_ARCH_GPT2 ? take(ff * 4) : 0;
    t.wproj = mat(d, ff, t.sproj);
    t.bproj = c.arch == GD_ARCH_GPT2 ? take(d * 4) : 0;
  }
  m->o_nfg = take(d * 4);
  if (c.arch == GD_ARCH_GPT2) m->o_nfb = take(d * 4);
  else m->o_head = mat(V, d, m->o_shead);
  // tile-major copies for the matrix-core kernel (filled from the row-major matrices;
  // none for 8-bit weights, which run on the VALU kernel only)
  m->w_rowmajor_bytes = off;
  const int wt = m->wt == GD_WEIGHT_F32 ? 0 : 1;
  if (!q8) {
    for (int l = 0; l < c.n_layer; ++l) {
      LayerOff& t = m->L[l];
      t.tqkv = take(mm_packed_bytes(wt, m->qkvdim, (int)d));
      t.to = take(mm_packed_bytes(wt, (int)d, m->qdim));
      t.tfc = take(mm_packed_bytes(wt, m->fcN, (int)d));
      t.tproj = take(mm_packed_bytes(wt, (int)d, (int)ff));
    }
    m->o_thead = take(mm_packed_bytes(wt, (int)V, (int)d));
  }
  // the pre-norms folded into the layers that follow them (fp32 weights only: a bf16
  // copy of g_k W_nk would round the weights a second time)
  m->folded = m->wt == GD_WEIGHT_F32;
  m->o_fold = off;
  if (m->folded) {
    for (int l = 0; l < c.n_layer; ++l) {
      LayerOff& t = m->L[l];
      t.fqkv = take((size_t)m->qkvdim * d * 4);
      t.fqkv_b = take((size_t)m->qkvdim * 4);
      t.fqkv_s = take((size_t)m->qkvdim * 4);
      t.ffc = take((size_t)m->fcN * d * 4);
      t.ffc_b = take((size_t)m->fcN * 4);
      t.ffc_s = take((size_t)m->fcN * 4);
    }
    m->o_fhead = take(V * d * 4);
    m->o_fhead_b = take(V * 4);
    m->o_fhead_s = take(V * 4);
  }
  m->o_fold_end = off;   // the host fills [o_fold, o_fold_end); k_pack_tiles the rest
  if (m->folded) {
    for (int l = 0; l < c.n_layer; ++l) {
      LayerOff& t = m->L[l];
      t.tfqkv = take(mm_packed_bytes(0, m->qkvdim, (int)d));
      t.tffc = take(mm_packed_bytes(0, m->fcN, (int)d));
    }
    m->o_tfhead = take(mm_packed_bytes(0, (int)V, (int)d));
  }
  m->w_bytes = off;

  // KV cache: K pools for all layers, then V pools
  m->kv_bytes = 2 * (size_t)c.n_layer * m->layer_kv_elems() * m->kv_elt;

  // argmax partials: the head's widest grid over both kernels
  m->am_parts = 0;
  for (int v = 1; v <= 2; ++v)
    for (int M = 1; M <= GD_MAX_ROWS; ++M)
      m->am_parts = std::max(m->am_parts, (size_t)plan_linear(M, c.vocab, c.d_model, m->wt, v, EPI_ARGMAX, true).parts);

  // scratch
  off = 0;
  const size_t R = GD_MAX_ROWS;
  m->o_x = take(R * d * 4);
  m->o_q = take(R * m->qdim * 4);
  m->o_attn = take(R * m->qdim * 4);
  m->o_h = take(R * ff * 4);
  m->o_amv = take(m->am_parts * R * 4);
  m->o_ami = take(m->am_parts * R * 4);
  m->o_apart = take(R * c.n_head * GD_ATT_NCH_LONG * gd_apart_stride(c.head_dim) * 4);
  m->o_slog = take(R * (size_t)c.vocab * 4);
  // the tiled prompt pass: float or bf16 weights, head_dim 64, widths multiples of 32
  m->pf_ok = m->wt != GD_WEIGHT_Q8 && c.head_dim == 64 && c.d_model % 32 == 0 && c.d_ff % 32 == 0 &&
             m->qdim % 32 == 0 && c.d_model <= PF_NT * 16 && (c.n_head % c.n_kv_head) == 0;
  if (m->pf_ok) {
    const size_t P = kPrefillChunk;
    m->o_px = take(P * d * 4);
    m->o_pxn = take(P * d * 4);
    m->o_pq = take(P * (size_t)m->qdim * 4);
    m->o_pattn = take(P * (size_t)m->qdim * 4);
    m->o_ph = take(P * ff * 4);
    m->o_ppart = take(P * c.n_head * PF_MAXS * PF_PSTRIDE * 4);
  }
  // zeros (cleared at bind, never written): the bias or residual of layers that have none
  m->o_zero = take((size_t)std::max({m->qkvdim, m->fcN, (int)d, (int)ff}) * 4);
  m->o_rseq = take(R * 4);
  m->o_rpos = take(R * 4);
  m->o_rtok = take(R * 4);
  m->o_rkv = take(R * 8);
  m->o_rcs = c.arch == GD_ARCH_LLAMA ? take(R * c.head_dim * 4) : 0;
  m->o_pseq = take((size_t)c.n_ctx * 4);
  m->o_ppos = take((size_t)c.n_ctx * 4);
  m->o_ptok = take((size_t)c.n_ctx * 4);
  m->o_pkv = take((size_t)c.n_ctx * 8);
  m->o_pcs = c.arch == GD_ARCH_LLAMA ? take((size_t)c.n_ctx * c.head_dim * 4) : 0;
  m->o_len = take((size_t)c.max_seqs * 4);
  m->o_cap = take((size_t)c.max_seqs * 4);
  m->o_sids = take(R * 4);
  m->o_table = take((size_t)c.max_seqs * m->max_blocks * 4);
  m->o_err = take(4);
  m->o_rope = c.arch == GD_ARCH_LLAMA ? take((size_t)c.n_ctx * c.head_dim * 4) : 0;
  m->s_bytes = off;
}

extern "C" gd_status gd_create(const gd_config* cfg, void* hip_stream, gd_model** out) {
  if (!out) return set_err(GD_ERR_INVALID, "out is NULL");
  *out = nullptr;
  gd_status st = check_cfg(cfg);
  if (st != GD_OK) return st;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) return set_err(GD_ERR_NO_DEVICE, "no HIP device");
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return set_err(GD_ERR_NO_DEVICE, "hipGetDevice failed");
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return set_err(GD_ERR_NO_DEVICE, "no device properties");
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return set_err(GD_ERR_NO_DEVICE, "device %d is %s, this library is built for gfx950", dev, prop.gcnArchName);
  gd_model* m = new gd_model();
  m->c = *cfg;
  m->dev = dev;
  m->n_cu = prop.multiProcessorCount;
  m->stream = reinterpret_cast<hipStream_t>(hip_stream);
  layout(m);
  if (hipStreamCreateWithFlags(&m->cap_stream, hipStreamNonBlocking) != hipSuccess ||
      hipEventCreateWithFlags(&m->staging_evt, hipEventDisableTiming) != hipSuccess) {
    delete m;
    return set_err(GD_ERR_HIP, "stream/event creation failed");
  }
  m->staging_ints = 3 * (size_t)cfg->n_ctx + 64;
  if (hipHostMalloc(reinterpret_cast<void**>(&m->staging), m->staging_ints * sizeof(int), hipHostMallocDefault) !=
      hipSuccess) {
    (void)hipStreamDestroy(m->cap_stream);
    delete m;
    return set_err(GD_ERR_HIP, "pinned staging allocation failed");
  }
  if (m->am_parts > (size_t)GD_WG * AM_FIN_PER) {
    (void)hipHostFree(m->staging);
    (void)hipEventDestroy(m->staging_evt);
    (void)hipStreamDestroy(m->cap_stream);
    delete m;
    return set_err(GD_ERR_INVALID, "vocab %d too large for the argmax reduction", cfg->vocab);
  }
  m->len.assign(cfg->max_seqs, 0);
  m->cap.assign(cfg->max_seqs, cfg->kv_block_size > 0 ? 0 : cfg->n_ctx);
  *out = m;
  return GD_OK;
}

extern "C" void gd_destroy(gd_model* m) {
  if (!m) return;
  if (m->stream) (void)hipStreamSynchronize(m->stream);
  for (auto& kv : m->graphs) (void)hipGraphExecDestroy(kv.second.exec);
  for (auto& r : m->prof_pending)
    for (auto& pr : r.pairs) { (void)hipEventDestroy(pr.first); (void)hipEventDestroy(pr.second); }
  if (m->gate_evt) (void)hipEventDestroy(m->gate_evt);
  for (auto e : m->ev_free) (void)hipEventDestroy(e);
  if (m->cap_stream) (void)hipStreamDestroy(m->cap_stream);
  if (m->staging_evt) (void)hipEventDestroy(m->staging_evt);
  if (m->staging) (void)hipHostFree(m->staging);
  delete m;
}

extern "C" gd_status gd_memory_requirements(const gd_model* m, size_t* wb, size_t* kb, size_t* sb) {
  if (!m) return set_err(GD_ERR_INVALID, "model is NULL");
  if (wb) *wb = m->w_bytes;
  if (kb) *kb = m->kv_bytes;
  if (sb) *sb = m->s_bytes;
  return GD_OK;
}

// Waits until the pinned staging buffer is no longer read by an enqueued copy.
static gd_status staging_wait(gd_model* m) {
  if (m->staging_pending) {
    HIP_TRY(m, hipEventSynchronize(m->staging_evt));
    m->staging_pending = false;
  }
  return GD_OK;
}

static gd_status staging_done(gd_model* m) {
  HIP_TRY(m, hipEventRecord(m->staging_evt, m->stream));
  m->staging_pending = true;
  return GD_OK;
}

extern "C" gd_status gd_bind_memory(gd_model* m, void* wdev, void* kvdev, void* sdev) {
  if (!m) return set_err(GD_ERR_INVALID, "model is NULL");
  if (m->poisoned) return set_err(GD_ERR_HIP, "model is poisoned by an earlier HIP error");
  if (!wdev || !kvdev || !sdev) return set_err(GD_ERR_INVALID, "NULL device buffer");
  if ((reinterpret_cast<uintptr_t>(wdev) | reinterpret_cast<uintptr_t>(kvdev) | reinterpret_cast<uintptr_t>(sdev)) & 255)
    return set_err(GD_ERR_INVALID, "device buffers must be 256-byte aligned");
  m->w = static_cast<char*>(wdev);
  m->kv = static_cast<char*>(kvdev);
  m->s = static_cast<char*>(sdev);
  HIP_TRY(m, hipMemsetAsync(m->s, 0, m->s_bytes, m->stream));
  const gd_config& c = m->c;
  // sequence capacities and (contiguous cache) identity block tables
  HIP_TRY(m, staging_wait(m) == GD_OK ? hipSuccess : hipErrorUnknown);
  std::vector<int> tab((size_t)c.max_seqs * m->max_blocks, -1);
  if (c.kv_block_size == 0)
    for (int s = 0; s < c.max_seqs; ++s) tab[s] = s;
  HIP_TRY(m, hipMemcpyAsync(m->sp<int>(m->o_table), tab.data(), tab.size() * 4, hipMemcpyHostToDevice, m->stream));
  HIP_TRY(m, hipMemcpyAsync(m->sp<int>(m->o_cap), m->cap.data(), m->cap.size() * 4, hipMemcpyHostToDevice, m->stream));
  if (c.arch == GD_ARCH_LLAMA) {
    const int hd = c.head_dim, half = hd / 2;
    std::vector<float> cs((size_t)c.n_ctx * hd);
    for (int p = 0; p < c.n_ctx; ++p)
      for (int j = 0; j < half; ++j) {
        double ang = (double)p * std::pow((double)c.rope_theta, -2.0 * j / (double)hd);
        cs[(size_t)p * hd + j] = (float)std::cos(ang);
        cs[(size_t)p * hd + half + j] = (float)std::sin(ang);
      }
    HIP_TRY(m, hipMemcpyAsync(m->sp<float>(m->o_rope), cs.data(), cs.size() * 4, hipMemcpyHostToDevice, m->stream));
  }
  HIP_TRY(m, hipStreamSynchronize(m->stream));
  std::fill(m->len.begin(), m->len.end(), 0);
  m->last_sids.clear();
  for (auto& kv : m->graphs) (void)hipGraphExecDestroy(kv.second.exec);
  m->graphs.clear();
  m->bound = true;
  m->loaded = false;
  return GD_OK;
}

static uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static void put_mat(const gd_model* m, std::vector<char>& dst, size_t off, const float* src, size_t n) {
  if (m->wt == GD_WEIGHT_F32) {
    memcpy(dst.data() + off, src, n * 4);
  } else {
    uint16_t* d = reinterpret_cast<uint16_t*>(dst.data() + off);
    for (size_t i = 0; i < n; ++i) d[i] = to_bf16(src[i]);
  }
}

// 8-bit blocks of one row of K values (K a multiple of 32), as in the Q8_0 format: per
// block of 32, the scale s = max|x| / 127 and the codes round(x * (1 / s)), rounded half
// away from zero, in [-127, 127]; s = 0 and codes 0 for an all-zero block.
static void quantize_q8_row(const float* x, size_t K, int8_t* q, float* sc) {
  for (size_t b = 0; b < K / 32; ++b) {
    float amax = 0.f;
    for (size_t i = 0; i < 32; ++i) amax = std::max(amax, std::fabs(x[32 * b + i]));
    const float s = amax / 127.0f;
    const float inv = s != 0.f ? 1.0f / s : 0.f;
    for (size_t i = 0; i < 32; ++i) q[32 * b + i] = (int8_t)std::round(x[32 * b + i] * inv);
    sc[b] = s;
  }
}

// Rows [row0, row0 + nrows) of a [rows][K] matrix stored at byte offset off (8-bit
// weights: its block scales at sc_off), from nrows float rows at src.
static void put_rows(const gd_model* m, std::vector<char>& dst, size_t off, size_t sc_off, size_t row0,
                     const float* src, size_t nrows, size_t K) {
  if (m->wt == GD_WEIGHT_Q8) {
    int8_t* q = reinterpret_cast<int8_t*>(dst.data() + off) + row0 * K;
    float* sc = reinterpret_cast<float*>(dst.data() + sc_off) + row0 * (K / 32);
    for (size_t r = 0; r < nrows; ++r) quantize_q8_row(src + r * K, K, q + r * K, sc + r * (K / 32));
    return;
  }
  put_mat(m, dst, off + row0 * K * m->elt, src, nrows * K);
}

static void put_vec(std::vector<char>& dst, size_t off, const float* src, size_t n) {
  memcpy(dst.data() + off, src, n * 4);
}

// Fills the tile-major copy of an [N][K] matrix (k_pack_tiles).
static hipError_t launch_pack(const void* W, int wt, int N, int K, void* dst, hipStream_t st) {
  const int w = wt == GD_WEIGHT_F32 ? 0 : 1;
  const size_t units = mm_packed_bytes(w, N, K) / 16;
  GD_LAUNCH(k_pack_tiles, dim3((unsigned)((units + GD_WG - 1) / GD_WG)), dim3(GD_WG), 0, st, W, w, N, K, dst,
                     units);
  return hipGetLastError();
}

static size_t canonical_count(const gd_config& c) {
  size_t d = c.d_model, ff = c.d_ff, V = c.vocab;
  size_t hq = (size_t)c.n_head * c.head_dim, hk = (size_t)c.n_kv_head * c.head_dim;
  if (c.arch == GD_ARCH_GPT2)
    return V * d + (size_t)c.n_ctx * d + (size_t)c.n_layer * (2 * d + 3 * d * d + 3 * d + d * d + d + 2 * d + ff * d + ff + d * ff + d) + 2 * d;
  return V * d + (size_t)c.n_layer * (d + hq * d + 2 * hk * d + d * hq + d + 2 * ff * d + d * ff) + d + V * d;
}

extern "C" gd_status gd_load_weights(gd_model* m, const float* hw, size_t n) {
  if (!m || !hw) return set_err(GD_ERR_INVALID, "NULL argument");
  if (m->poisoned) return set_err(GD_ERR_HIP, "model is poisoned by an earlier HIP error");
  if (!m->bound) return set_err(GD_ERR_STATE, "memory not bound");
  const gd_config& c = m->c;
  if (n != canonical_count(c)) return set_err(GD_ERR_INVALID, "weight count %zu, expected %zu", n, canonical_count(c));
  const size_t d = c.d_model, ff = c.d_ff, V = c.vocab;
  std::vector<char> buf(m->w_rowmajor_bytes, 0);
  const float* p = hw;
  put_rows(m, buf, m->o_wte, m->o_swte, 0, p, V, d);
  p += V * d;
  if (c.arch == GD_ARCH_GPT2) {
    put_rows(m, buf, m->o_wpe, m->o_swpe, 0, p, (size_t)c.n_ctx, d);
    p += (size_t)c.n_ctx * d;
    for (int l = 0; l < c.n_layer; ++l) {
      const LayerOff& t = m->L[l];
      put_vec(buf, t.n1g, p, d); p += d;
      put_vec(buf, t.n1b, p, d); p += d;
      put_rows(m, buf, t.wqkv, t.sqkv, 0, p, 3 * d, d); p += 3 * d * d;
      put_vec(buf, t.bqkv, p, 3 * d); p += 3 * d;
      put_rows(m, buf, t.wo, t.so, 0, p, d, d); p += d * d;
      put_vec(buf, t.bo, p, d); p += d;
      put_vec(buf, t.n2g, p, d); p += d;
      put_vec(buf, t.n2b, p, d); p += d;
      put_rows(m, buf, t.wfc, t.sfc, 0, p, ff, d); p += ff * d;
      put_vec(buf, t.bfc, p, ff); p += ff;
      put_rows(m, buf, t.wproj, t.sproj, 0, p, d, ff); p += d * ff;
      put_vec(buf, t.bproj, p, d); p += d;
    }
    put_vec(buf, m->o_nfg, p, d); p += d;
    put_vec(buf, m->o_nfb, p, d); p += d;
  } else {
    const size_t hq = m->qdim, hk = m->kdim, hd = c.head_dim, half = hd / 2;
    // q and k rows are stored so that each RoPE pair (i, i + hd/2) of a head sits in
    // adjacent rows (2i, 2i + 1); q.k is unchanged because both use the same order.
    auto put_rope_rows = [&](const LayerOff& t, size_t row_base, const float* src, size_t heads) {
      for (size_t h = 0; h < heads; ++h)
        for (size_t i = 0; i < half; ++i) {
          put_rows(m, buf, t.wqkv, t.sqkv, row_base + h * hd + 2 * i, src + (h * hd + i) * d, 1, d);
          put_rows(m, buf, t.wqkv, t.sqkv, row_base + h * hd + 2 * i + 1, src + (h * hd + half + i) * d, 1, d);
        }
    };
    for (int l = 0; l < c.n_layer; ++l) {
      const LayerOff& t = m->L[l];
      put_vec(buf, t.n1g, p, d); p += d;
      // fused [w_q; w_k; w_v]
      put_rope_rows(t, 0, p, c.n_head); p += hq * d;
      put_rope_rows(t, hq, p, c.n_kv_head); p += hk * d;
      put_rows(m, buf, t.wqkv, t.sqkv, hq + hk, p, hk, d); p += hk * d;
      put_rows(m, buf, t.wo, t.so, 0, p, d, hq); p += d * hq;
      put_vec(buf, t.n2g, p, d); p += d;
      // gate and up interleaved by row: row 2j = gate j, row 2j + 1 = up j
      const float* g = p;
      const float* u = p + ff * d;
      for (size_t j = 0; j < ff; ++j) {
        put_rows(m, buf, t.wfc, t.sfc, 2 * j, g + j * d, 1, d);
        put_rows(m, buf, t.wfc, t.sfc, 2 * j + 1, u + j * d, 1, d);
      }
      p += 2 * ff * d;
      put_rows(m, buf, t.wproj, t.sproj, 0, p, d, ff); p += d * ff;
    }
    put_vec(buf, m->o_nfg, p, d); p += d;
    put_rows(m, buf, m->o_head, m->o_shead, 0, p, V, d); p += V * d;
  }
  HIP_TRY(m, hipMemcpyAsync(m->w, buf.data(), buf.size(), hipMemcpyHostToDevice, m->stream));
  std::vector<char> fbuf;
  if (m->folded) {
    // W'_nk = g_k W_nk (one fp32 product), s_n = sum_k W'_nk, bias'_n = bias_n +
    // sum_k b_k W_nk, from the row-major matrices as stored (sums in double)
    fbuf.assign(m->o_fold_end - m->o_fold, 0);
    auto rf = [&](size_t off) { return reinterpret_cast<const float*>(buf.data() + off); };
    auto wf = [&](size_t off) { return reinterpret_cast<float*>(fbuf.data() + (off - m->o_fold)); };
    auto fold = [&](size_t w, int N, size_t g, size_t b, size_t bias, size_t fw, size_t fb, size_t fs) {
      const float* W = rf(w);
      const float* G = rf(g);
      const float* B = b ? rf(b) : nullptr;
      const float* bi = bias ? rf(bias) : nullptr;
      float* Wf = wf(fw);
      float* Bf = wf(fb);
      float* Sf = wf(fs);
      for (size_t n = 0; n < (size_t)N; ++n) {
        double sn = 0.0, bn = bi ? (double)bi[n] : 0.0;
        for (size_t k = 0; k < d; ++k) {
          const float v = W[n * d + k];
          const float f = G[k] * v;
          Wf[n * d + k] = f;
          sn += (double)f;
          if (B) bn += (double)B[k] * (double)v;
        }
        Sf[n] = (float)sn;
        Bf[n] = (float)bn;
      }
    };
    for (int l = 0; l < c.n_layer; ++l) {
      const LayerOff& t = m->L[l];
      fold(t.wqkv, m->qkvdim, t.n1g, t.n1b, t.bqkv, t.fqkv, t.fqkv_b, t.fqkv_s);
      fold(t.wfc, m->fcN, t.n2g, t.n2b, t.bfc, t.ffc, t.ffc_b, t.ffc_s);
    }
    fold(c.arch == GD_ARCH_GPT2 ? m->o_wte : m->o_head, (int)V, m->o_nfg, m->o_nfb, 0, m->o_fhead, m->o_fhead_b,
         m->o_fhead_s);
    HIP_TRY(m, hipMemcpyAsync(m->w + m->o_fold, fbuf.data(), fbuf.size(), hipMemcpyHostToDevice, m->stream));
  }
  auto pack = [&](size_t src, size_t dst, int N, int K) {
    return launch_pack(m->w + src, m->wt, N, K, m->w + dst, m->stream);
  };
  for (int l = 0; l < c.n_layer && m->wt != GD_WEIGHT_Q8; ++l) {
    const LayerOff& t = m->L[l];
    HIP_TRY(m, pack(t.wqkv, t.tqkv, m->qkvdim, (int)d));
    HIP_TRY(m, pack(t.wo, t.to, (int)d, m->qdim));
    HIP_TRY(m, pack(t.wfc, t.tfc, m->fcN, (int)d));
    HIP_TRY(m, pack(t.wproj, t.tproj, (int)d, (int)ff));
  }
  if (m->wt != GD_WEIGHT_Q8)
    HIP_TRY(m, pack(c.arch == GD_ARCH_GPT2 ? m->o_wte : m->o_head, m->o_thead, (int)V, (int)d));
  if (m->folded) {
    for (int l = 0; l < c.n_layer; ++l) {
      const LayerOff& t = m->L[l];
      HIP_TRY(m, pack(t.fqkv, t.tfqkv, m->qkvdim, (int)d));
      HIP_TRY(m, pack(t.ffc, t.tffc, m->fcN, (int)d));
    }
    HIP_TRY(m, pack(m->o_fhead, m->o_tfhead, (int)V, (int)d));
  }
  HIP_TRY(m, hipStreamSynchronize(m->stream));
  m->loaded = true;
  return GD_OK;
}

extern "C" gd_status gd_set_block_table(gd_model* m, int32_t seq, const int32_t* blocks, int32_t n) {
  if (!m) return set_err(GD_ERR_INVALID, "model is NULL");
  if (m->poisoned) return set_err(GD_ERR_HIP, "model is poisoned by an earlier HIP error");
  if (!m->bound) return set_err(GD_ERR_STATE, "memory not bound");
  if (m->c.kv_block_size == 0) return set_err(GD_ERR_STATE, "contiguous cache has no block tables");
  if (seq < 0 || seq >= m->c.max_seqs) return set_err(GD_ERR_INVALID, "seq %d out of range", seq);
  if (n < 0 || n > m->max_blocks || (n > 0 && !blocks)) return set_err(GD_ERR_INVALID, "bad block count %d", n);
  for (int i = 0; i < n; ++i)
    if (blocks[i] < 0 || blocks[i] >= m->nblk) return set_err(GD_ERR_INVALID, "block %d out of range", blocks[i]);
  gd_status st = staging_wait(m);
  if (st != GD_OK) return st;
  int* h = m->staging;
  for (int i = 0; i < m->max_blocks; ++i) h[i] = i < n ? blocks[i] : -1;
  int cp = std::min(n * m->bsize, m->c.n_ctx);
  h[m->max_blocks] = cp;
  HIP_TRY(m, hipMemcpyAsync(m->sp<int>(m->o_table) + (size_t)seq * m->max_blocks, h, m->max_blocks * 4,
                            hipMemcpyHostToDevice, m->stream));
  HIP_TRY(m, hipMemcpyAsync(m->sp<int>(m->o_cap) + seq, h + m->max_blocks, 4, hipMemcpyHostToDevice, m->stream));
  st = staging_done(m);
  if (st != GD_OK) return st;
  m->cap[seq] = cp;
  return GD_OK;
}

extern "C" gd_status gd_reset_seq(gd_model* m, int32_t seq) {
  if (!m) return set_err(GD_ERR_INVALID, "model is NULL");
  if (m->poisoned) return set_err(GD_ERR_HIP, "model is poisoned by an earlier HIP error");
  if (!m->bound) return set_err(GD_ERR_STATE, "memory not bound");
  if (seq < 0 || seq >= m->c.max_seqs) return set_err(GD_ERR_INVALID, "seq %d out of range", seq);
  HIP_TRY(m, hipMemsetAsync(m->sp<int>(m->o_len) + seq, 0, 4, m->stream));
  m->len[seq] = 0;
  return GD_OK;
}

extern "C" gd_status gd_truncate_seq(gd_model* m, int32_t seq, int32_t len) {
  if (!m) return set_err(GD_ERR_INVALID, "model is NULL");
  if (m->poisoned) return set_err(GD_ERR_HIP, "model is poisoned by an earlier HIP error");
  if (!m->bound) return set_err(GD_ERR_STATE, "memory not bound");
  if (seq < 0 || seq >= m->c.max_seqs) return set_err(GD_ERR_INVALID, "seq %d out of range", seq);
  if (len < 0 || len > m->len[seq]) return set_err(GD_ERR_INVALID, "length %d outside 0..%d", len, m->len[seq]);
  gd_status st = staging_wait(m);
  if (st != GD_OK) return st;
  m->staging[0] = len;
  HIP_TRY(m, hipMemcpyAsync(m->sp<int>(m->o_len) + seq, m->staging, 4, hipMemcpyHostToDevice, m->stream));
  if ((st = staging_done(m)) != GD_OK) return st;
  m->len[seq] = len;
  return GD_OK;
}

extern "C" gd_status gd_profile_read(gd_model* m, gd_kernel_stat* out, int32_t max, int32_t* n, int32_t reset) {
  if (!m || !n) return set_err(GD_ERR_INVALID, "NULL argument");
  HIP_TRY(m, hipStreamSynchronize(m->stream));
  for (auto& r : m->prof_pending) {
    double us = 0.0;
    for (auto& pr : r.pairs) {
      float ms = 0.f;
      HIP_TRY(m, hipEventElapsedTime(&ms, pr.first, pr.second));
      us += ms * 1000.0;
      m->ev_free.push_back(pr.first);
      m->ev_free.push_back(pr.second);
    }
    gd_kernel_stat& s = m->prof_stats[r.stat];
    s.launches += 1;
    s.total_us += us;
    s.bytes += r.bytes;
  }
  m->prof_pending.clear();
  *n = (int)m->prof_stats.size();
  for (int i = 0; i < std::min<int>(max, *n); ++i) out[i] = m->prof_stats[i];
  if (reset) m->prof_stats.clear();
  return GD_OK;
}

extern "C" gd_status gd_seq_len(const gd_model* m, int32_t seq, int32_t* len) {
  if (!m || !len) return set_err(GD_ERR_INVALID, "NULL argument");
  if (seq < 0 || seq >= m->c.max_seqs) return set_err(GD_ERR_INVALID, "seq %d out of range", seq);
  *len = m->len[seq];
  return GD_OK;
}

extern "C" gd_status gd_set_option(gd_model* m, int32_t opt, int32_t v) {
  if (!m) return set_err(GD_ERR_INVALID, "model is NULL");
  if (opt == GD_OPT_LINEAR_VARIANT) {
    if (v < 0 || v > 2) return set_err(GD_ERR_INVALID, "variant must be 0, 1 or 2");
    m->variant = v;
  } else if (opt == GD_OPT_USE_GRAPH) {
    m->use_graph = v != 0;
  } else if (opt == GD_OPT_FUSE_ATTN_O) {
    m->fuse_attn_o = v != 0;
  } else if (opt == GD_OPT_FOLD_NORM) {
    m->use_fold = v != 0;
  } else if (opt == GD_OPT_TILED_PREFILL) {
    m->use_pf = v != 0;
  } else if (opt == GD_OPT_PREFILL_BF16_PARTS) {
    if (v < 0 || v > 2) return set_err(GD_ERR_INVALID, "prefill bf16 parts must be 0, 1 or 2");
    m->pf_parts = v;
  } else if (opt == GD_OPT_ATTN_CHUNKS) {
    if (v != 0 && v != 1 && v != GD_ATT_NCH) return set_err(GD_ERR_INVALID, "attention chunks must be 0, 1 or %d", GD_ATT_NCH);
    m->attn_chunks = v;
  } else if (opt == GD_OPT_PROFILE) {
    if (v < 0 || v > 2) return set_err(GD_ERR_INVALID, "profile must be 0, 1 or 2");
    m->profile = v != 0;
    m->profile_gated = v == 2;
  } else {
    return set_err(GD_ERR_INVALID, "unknown option %d", opt);
  }
  for (auto& kv : m->graphs) (void)hipGraphExecDestroy(kv.second.exec);
  m->graphs.clear();
  return GD_OK;
}

extern "C" gd_status gd_set_sampling(gd_model* m, float temperature, int32_t top_k, uint64_t seed) {
  if (!m) return set_err(GD_ERR_INVALID, "model is NULL");
  if (!(temperature == temperature)) return set_err(GD_ERR_INVALID, "temperature is NaN");
  if (temperature <= 0.f || top_k == 1) {
    m->sample = false;
  } else {
    if (m->c.vocab > GD_SAMPLE_NT * GD_SAMPLE_VPT)
      return set_err(GD_ERR_INVALID, "sampling needs vocab <= %d", GD_SAMPLE_NT * GD_SAMPLE_VPT);
    if (top_k < 2 || top_k > GD_SAMPLE_MAX_K || top_k > m->c.vocab)
      return set_err(GD_ERR_INVALID, "top_k %d outside 1..min(%d, vocab)", top_k, GD_SAMPLE_MAX_K);
    m->sample = true;
    m->top_k = top_k;
    m->inv_temp = 1.0f / temperature;
    m->seed = seed;
  }
  for (auto& kv : m->graphs) (void)hipGraphExecDestroy(kv.second.exec);
  m->graphs.clear();
  return GD_OK;
}

extern "C" gd_status gd_device_errors(gd_model* m, int32_t* flags) {
  if (!m || !flags) return set_err(GD_ERR_INVALID, "NULL argument");
  if (!m->bound) return set_err(GD_ERR_STATE, "memory not bound");
  int h = 0;
  HIP_TRY(m, hipMemcpyAsync(&h, m->sp<int>(m->o_err), 4, hipMemcpyDeviceToHost, m->stream));
  HIP_TRY(m, hipStreamSynchronize(m->stream));
  HIP_TRY(m, hipMemsetAsync(m->sp<int>(m->o_err), 0, 4, m->stream));
  *flags = h;
  return GD_OK;
}

// ------------------------------------------------------ forward over rows

static int prof_stat_index(gd_model* m, const char* role, const char* kernel) {
  for (size_t i = 0; i < m->prof_stats.size(); ++i)
    if (!strcmp(m->prof_stats[i].role, role) && !strcmp(m->prof_stats[i].kernel, kernel)) return (int)i;
  gd_kernel_stat s;
  memset(&s, 0, sizeof(s));
  snprintf(s.role, sizeof(s.role), "%s", role);
  snprintf(s.kernel, sizeof(s.kernel), "%s", kernel);
  m->prof_stats.push_back(s);
  return (int)m->prof_stats.size() - 1;
}

static hipEvent_t prof_event(gd_model* m) {
  if (!m->ev_free.empty()) {
    hipEvent_t e = m->ev_free.back();
    m->ev_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  (void)hipEventCreate(&e);
  return e;
}

// One profiled unit (a role): the launches made while it is open are timed one by one
// (GD_LAUNCH) and summed into the role's statistics.
struct ProfScope {
  gd_model* m;
  int idx = -1;
  double bytes;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pairs;
  gd_model* save_m = nullptr;
  std::vector<std::pair<hipEvent_t, hipEvent_t>>* save_p = nullptr;
  ProfScope(gd_model* m_, hipStream_t, const char* role, const char* kernel, double b) : m(m_), bytes(b) {
    if (!m->profile) return;
    idx = prof_stat_index(m, role, kernel);
    save_m = t_prof_m;
    save_p = t_prof_pairs;
    t_prof_m = m;
    t_prof_pairs = &pairs;
  }
  ~ProfScope() {
    if (idx < 0) return;
    t_prof_m = save_m;
    t_prof_pairs = save_p;
    m->prof_pending.push_back({idx, std::move(pairs), bytes});
  }
};

static const char* linear_kernel_name(int wt, const LinPlan& lp, int N, int epi, bool norm, bool fold, int pro,
                                      char* buf, size_t n) {
  const int w = wt == GD_WEIGHT_F32 ? 0 : wt == GD_WEIGHT_BF16 ? 1 : 2;
  // as rocprofv3 prints the instantiation
  if (lp.var == 0)
    snprintf(buf, n, "k_gemv<%d, %d, %d, %d, %d, %d>", w, lp.nc, lp.rw, epi, pro,
             !norm ? NRM_NONE : (fold && w == 0) ? NRM_FOLDED : NRM_EXPLICIT);
  else
    snprintf(buf, n, "k_mm<%d, %d, %d, %d, %s, %d, %s>", w, lp.mt, epi,
             !norm ? NRM_NONE : (fold && w == 0) ? NRM_FOLDED : NRM_EXPLICIT, lp.passes > 1 ? "true" : "false", pro,
             mm_parts(lp, N, epi, norm && fold && w == 0) ? "true" : "false");
  return buf;
}

// Algorithmic bytes of one linear layer over p.M rows: every weight, bias and norm
// parameter once, the activation rows in, the outputs out (and the residual read).
static double linear_bytes(const gd_model* m, const LinParams& p) {
  const int n_out = p.epi == EPI_SWIGLU ? p.N / 2 : (p.epi == EPI_ARGMAX ? (p.logits ? p.N : 0) : p.N);
  // rows in: as given, the attention partials they are merged from, or the embedding
  // rows they are summed from (stored once as the residual rows)
  const double rows_in = p.pro == PRO_ATTN    ? (double)p.M * p.Hq * p.nch * (p.hd + 2) * 4
                         : p.pro == PRO_EMBED ? (double)p.M * p.K * (m->elt * (m->c.arch == GD_ARCH_GPT2 ? 2 : 1) + 4)
                                              : (double)p.M * p.K * 4;
  double b = (double)p.N * p.K * m->elt + rows_in + (double)p.M * n_out * 4;
  if (m->wt == GD_WEIGHT_Q8) b += (double)p.N * (p.K / 32) * 4;   // block scales
  const float* zero = m->sp<float>(m->o_zero);
  if (p.bias && p.bias != zero) b += (double)p.N * 4;
  if (p.norm) b += (double)p.K * 4 * (p.nb ? 2 : 1);
  if (p.resid && p.resid != zero) b += (double)p.M * p.N * 4;
  return b;
}

// Launches one linear layer (profiled when enabled). es: the embedding prologue's
// sources (p.pro == PRO_EMBED); adv: the lengths the argmax finalize advances.
static hipError_t run_linear(gd_model* m, hipStream_t st, const char* role, const LinParams& p,
                             int* am_out = nullptr, const EmbSrc* es = nullptr, const AdvLen* adv = nullptr) {
  const bool inplace = p.resid == p.y && p.ldr == p.ldy;
  LinPlan lp = plan_linear(p.M, p.N, p.K, m->wt, m->variant, p.epi, p.norm != NORM_NONE, inplace, p.pro == PRO_ATTN);
  char kn[64];
  std::vector<std::pair<hipEvent_t, hipEvent_t>> fin;
  hipError_t e;
  {
    ProfScope ps(m, st, role,
                 linear_kernel_name(m->wt, lp, p.N, p.epi, p.norm != NORM_NONE, p.wf != nullptr, p.pro, kn, sizeof(kn)),
                 m->profile ? linear_bytes(m, p) : 0);
    t_prof_fin = &fin;
    e = run_linear_rows(m->wt, lp, p, st, am_out, es, adv);
    t_prof_fin = nullptr;
  }
  if (m->profile && !fin.empty())
    m->prof_pending.push_back({prof_stat_index(m, "argmax", "k_argmax_finalize"), std::move(fin),
                               (double)lp.parts * p.M * 8 + p.M * 4.0});
  return e;
}

template <int HD, int G, bool KV16>
static void launch_attn_o_kv(hipStream_t st, const AttnParams& a, const AttnOParams& po, bool paged, int wt, int M,
                             int Hkv) {
  constexpr int PPG = HD == 64 ? 4 : 1;   // 64 positions per load round (measured: 8 and 2 slower)
  const dim3 grid(iceil(po.N, AttnORows<HD>::ROWS), Hkv, M), b(GD_WG);
  if (paged) {
    if (wt == GD_WEIGHT_F32) GD_LAUNCH((k_attn_o<HD, G, PPG, true, 0, KV16>), grid, b, 0, st, a, po);
    else if (wt == GD_WEIGHT_BF16) GD_LAUNCH((k_attn_o<HD, G, PPG, true, 1, KV16>), grid, b, 0, st, a, po);
    else GD_LAUNCH((k_attn_o<HD, G, PPG, true, 2, KV16>), grid, b, 0, st, a, po);
  } else {
    if (wt == GD_WEIGHT_F32) GD_LAUNCH((k_attn_o<HD, G, PPG, false, 0, KV16>), grid, b, 0, st, a, po);
    else if (wt == GD_WEIGHT_BF16) GD_LAUNCH((k_attn_o<HD, G, PPG, false, 1, KV16>), grid, b, 0, st, a, po);
    else GD_LAUNCH((k_attn_o<HD, G, PPG, false, 2, KV16>), grid, b, 0, st, a, po);
  }
}

template <int HD, int G>
static void launch_attn_o(hipStream_t st, const AttnParams& a, const AttnOParams& po, bool paged, int wt, int M,
                          int Hkv, bool kv16) {
  if (kv16) launch_attn_o_kv<HD, G, true>(st, a, po, paged, wt, M, Hkv);
  else launch_attn_o_kv<HD, G, false>(st, a, po, paged, wt, M, Hkv);
}

// Outputs of k_attn_proj: NP passes of 32 (512 threads, 16 lanes per output).
static const int kAttnProjPasses = 24;

static void launch_attn_proj(hipStream_t st, const AttnParams& a, const AttnOParams& po, int wt, int M, int Hkv,
                             bool kv16) {
  // 512 threads: 768 and 1024 (more positions per load round, one workgroup per CU)
  // measured 11 % and 16 % slower at batch 32
  constexpr int NT = 2 * GD_WG, NP = kAttnProjPasses;
  const dim3 grid(1, Hkv, M), b(NT);
  if (kv16) {
    if (wt == GD_WEIGHT_F32) GD_LAUNCH((k_attn_proj<64, false, 0, NT, NP, true>), grid, b, 0, st, a, po);
    else GD_LAUNCH((k_attn_proj<64, false, 1, NT, NP, true>), grid, b, 0, st, a, po);
  } else {
    if (wt == GD_WEIGHT_F32) GD_LAUNCH((k_attn_proj<64, false, 0, NT, NP, false>), grid, b, 0, st, a, po);
    else GD_LAUNCH((k_attn_proj<64, false, 1, NT, NP, false>), grid, b, 0, st, a, po);
  }
}

template <int HD, int G, bool KV16>
static void launch_attention_kv(dim3 grid, hipStream_t st, const AttnParams& a, bool paged) {
  static_assert(HD == 64 || HD == 16, "head_dim");
  // 64 positions per load round: at batch 32 the kernel runs 40 % faster than with 128
  // (fewer registers, more workgroups resident per CU); 32 and 16 measure slightly slower
  // One chunk per row: 512 threads, twice the positions in flight for the longest rows.
  constexpr int PPG = HD == 64 ? 4 : 1;
  if (grid.x == 1 && !paged)
    GD_LAUNCH((k_attention<HD, G, PPG, false, 2 * GD_WG, KV16>), grid, dim3(2 * GD_WG), 0, st, a);
  else if (paged) GD_LAUNCH((k_attention<HD, G, PPG, true, GD_WG, KV16>), grid, dim3(GD_WG), 0, st, a);
  else GD_LAUNCH((k_attention<HD, G, PPG, false, GD_WG, KV16>), grid, dim3(GD_WG), 0, st, a);
}

template <int HD, int G>
static void launch_attention(dim3 grid, hipStream_t st, const AttnParams& a, bool paged, bool kv16) {
  if (kv16) launch_attention_kv<HD, G, true>(grid, st, a, paged);
  else launch_attention_kv<HD, G, false>(grid, st, a, paged);
}

// Row set-up parameters over the row arrays starting at seq/pos/tok/kvoff.
static RowParams row_params(gd_model* m, int* rseq, int* rpos, int* rtok, long long* rkv, float* rcs) {
  const gd_config& c = m->c;
  RowParams r;
  memset(&r, 0, sizeof(r));
  r.table = m->sp<int>(m->o_table); r.max_blocks = m->max_blocks; r.block_size = m->bsize; r.nblk = m->nblk;
  r.Hkv = c.n_kv_head; r.hd = c.head_dim;
  r.wte = m->w + m->o_wte;
  r.wpe = c.arch == GD_ARCH_GPT2 ? (const void*)(m->w + m->o_wpe) : nullptr;
  r.vocab = c.vocab; r.n_pos = c.n_ctx; r.d = c.d_model; r.emb_bf16 = m->wt == GD_WEIGHT_BF16;
  r.emb_q8 = m->wt == GD_WEIGHT_Q8;
  if (r.emb_q8) {
    r.wte_sc = m->wf(m->o_swte);
    r.wpe_sc = c.arch == GD_ARCH_GPT2 ? m->wf(m->o_swpe) : nullptr;
  }
  r.x = m->sp<float>(m->o_x);
  r.row_seq = rseq; r.row_pos = rpos; r.row_tok = rtok; r.row_kvoff = rkv;
  r.rope = c.arch == GD_ARCH_LLAMA ? m->sp<float>(m->o_rope) : nullptr;
  r.row_cs = rcs;
  r.err = m->sp<int>(m->o_err);
  return r;
}

// Final norm + logits (tied embedding or untied head) + the greedy argmax (or the
// sampled token) of rows [head_row, head_row + head_rows) of the residual rows x.
// adv_len: the finalize advances the rows' sequence lengths (a decode step whose
// set-up ran in its first QKV launch).
static hipError_t enqueue_head(gd_model* m, hipStream_t st, const RowParams& rp, const float* x, int head_row,
                               int head_rows, int* head_out, float* logits, int* adv_len = nullptr) {
  const gd_config& c = m->c;
  const int d = c.d_model;
  const bool gpt2 = c.arch == GD_ARCH_GPT2;
  const int nrm = gpt2 ? NORM_LN : NORM_RMS;
  const bool fold = m->folded && m->use_fold;
  hipError_t e;
  LinParams base;
  memset(&base, 0, sizeof(base));
  base.eps = c.norm_eps;
  base.err = m->sp<int>(m->o_err);
  base.hd = c.head_dim;
  base.Hq = c.n_head;
  {
    // final norm + logits (tied embedding or untied head) + greedy argmax partials
    LinParams p = base;
    p.pro = PRO_COPY;
    p.x = x + (size_t)head_row * d; p.ldx = d;
    p.norm = nrm; p.ng = m->wf(m->o_nfg); p.nb = gpt2 ? m->wf(m->o_nfb) : nullptr;
    p.w = m->w + (gpt2 ? m->o_wte : m->o_head); p.wtl = m->w + m->o_thead; p.N = c.vocab; p.K = d;
    if (m->wt == GD_WEIGHT_Q8) p.wsc = m->wf(gpt2 ? m->o_swte : m->o_shead);
    if (fold) {
      p.wf = m->w + m->o_fhead; p.wfl = m->w + m->o_tfhead; p.bf = m->wf(m->o_fhead_b); p.fs = m->wf(m->o_fhead_s);
    }
    p.epi = EPI_ARGMAX;
    p.M = head_rows;
    p.row_kvoff = rp.row_kvoff + head_row;
    p.rope_cs = nullptr;
    p.am_val = m->sp<float>(m->o_amv); p.am_idx = m->sp<int>(m->o_ami);
    // the sampler reads whole logit rows: the caller's, or the scratch rows
    p.logits = logits ? logits : (m->sample ? m->sp<float>(m->o_slog) : nullptr);
    p.ldl = c.vocab;
    const AdvLen adv{adv_len, rp.row_seq + head_row, rp.row_pos + head_row};
    if ((e = run_linear(m, st, "linear.head", p, head_out, nullptr, adv_len ? &adv : nullptr)) != hipSuccess) return e;
    if (m->sample) {
      // temperature / top-k draw over each head row (replaces the greedy token)
      SampleParams sp;
      sp.logits = p.logits; sp.ldl = c.vocab; sp.V = c.vocab; sp.top_k = m->top_k;
      sp.inv_temp = m->inv_temp; sp.seed = m->seed;
      sp.row_seq = rp.row_seq + head_row; sp.row_pos = rp.row_pos + head_row;
      sp.out = head_out;
      ProfScope ps(m, st, "sample", "k_sample", (double)head_rows * c.vocab * 4);
      GD_LAUNCH(k_sample, dim3(head_rows), dim3(GD_SAMPLE_NT), 0, st, sp);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

// Enqueues the forward pass of M (<= 32) rows with device-resident row metadata.
// If head_out is not NULL, computes logits/argmax for rows [head_row, head_row + head_rows).
// The decode step's set-up folded into its first QKV launch: the rows' sequence slots
// and tokens, and the sequences' lengths (advanced by the step's argmax finalize) and
// capacities.
struct StepEmbed {
  const int* sids; const int* tok; int* len; const int* cap;
};

static hipError_t enqueue_rows(gd_model* m, hipStream_t st, const RowParams& rp, int M, int max_T, int head_row,
                               int head_rows, int* head_out, float* logits, const StepEmbed* se = nullptr) {
  const gd_config& c = m->c;
  const int d = c.d_model, ff = c.d_ff;
  float* x = m->sp<float>(m->o_x);
  float* q = m->sp<float>(m->o_q);
  float* attn = m->sp<float>(m->o_attn);
  float* h = m->sp<float>(m->o_h);
  float* apart = m->sp<float>(m->o_apart);
  const float* zero = m->sp<float>(m->o_zero);
  int* err = m->sp<int>(m->o_err);
  hipError_t e;
  // the gemv O-projection merges the attention partials in its prologue, and so does
  // the matrix-core one for up to 16 rows
  const bool o_gemv = plan_linear(M, c.d_model, m->qdim, m->wt, m->variant, EPI_PLAIN, false).var == 0;
  const bool o_mm_merge = !o_gemv && M <= 16 && c.head_dim % 32 == 0;
  // few rows at short contexts: attention fused with the output projection
  const bool fuse_ao = m->fuse_attn_o && o_gemv && max_T <= kFusedAttnOMaxT;
  // Split-context chunks per row: one when the rows and KV heads alone give every CU a
  // workgroup (the kernel then writes the normalized output and no merge launch
  // follows); else GD_ATT_NCH, whose partials the O-projection merges as it stages its
  // rows (gemv, or matrix-core up to 16 rows) or a merge launch does.
  // Long contexts with few (row, KV head) pairs: 32 chunks, so that the scan spreads over
  // the GPU (8 chunks of a 3700-position context leave 160 workgroups walking 460
  // positions each: 18.5 -> 11.7 us, plus a 4.2 us merge, while the projection no longer
  // merges in its prologue: 9.2 -> 4.1 us), merged by a launch of their own. With 8
  // chunks already giving the CUs a workgroup each (8 rows x 5 KV heads), 32 measured
  // slightly slower.
  const bool long_split = !m->attn_chunks && max_T >= kLongCtxT && !fuse_ao &&
                          M * c.n_kv_head * GD_ATT_NCH < m->n_cu;
  const int nch = long_split ? GD_ATT_NCH_LONG
                  : o_gemv ? GD_ATT_NCH
                  : m->attn_chunks ? m->attn_chunks
                  : (M * c.n_kv_head >= m->n_cu ? 1 : GD_ATT_NCH);
  // With one chunk per row (contiguous cache, head_dim 64, one query head per KV head,
  // d_model <= 768) the attention workgroups also apply the output projection.
  const bool fuse_ap = m->fuse_attn_o && !fuse_ao && nch == 1 && c.kv_block_size == 0 && c.head_dim == 64 &&
                       c.n_head == c.n_kv_head && c.d_model <= kAttnProjPasses * 32 && m->wt != GD_WEIGHT_Q8;
  const bool gpt2 = c.arch == GD_ARCH_GPT2;
  const int nrm = gpt2 ? NORM_LN : NORM_RMS;
  const int G = c.n_head / c.n_kv_head;
  const bool fold = m->folded && m->use_fold;   // pre-norms folded into QKV, MLP up and the head

  double kv_pos = 0;  // attended positions summed over rows (profiling only)
  for (int t : m->prof_T) kv_pos += t;

  LinParams base;
  memset(&base, 0, sizeof(base));
  base.eps = c.norm_eps;
  base.err = err;
  base.hd = c.head_dim;
  base.Hq = c.n_head;
  base.row_kvoff = rp.row_kvoff;
  base.M = M;

  for (int l = 0; l < c.n_layer; ++l) {
    const LayerOff& t = m->L[l];
    // pre-norm + QKV + bias; q to its buffer, k and v appended to the cache (RoPE first
    // for the Llama layout)
    {
      LinParams p = base;
      p.pro = PRO_COPY;
      p.x = x; p.ldx = d;
      p.norm = nrm; p.ng = m->wf(t.n1g); p.nb = t.n1b ? m->wf(t.n1b) : nullptr;
      p.w = m->w + t.wqkv; p.wtl = m->w + t.tqkv; p.N = m->qkvdim; p.K = d;
      if (m->wt == GD_WEIGHT_Q8) p.wsc = m->wf(t.sqkv);
      if (fold) { p.wf = m->w + t.fqkv; p.wfl = m->w + t.tfqkv; p.bf = m->wf(t.fqkv_b); p.fs = m->wf(t.fqkv_s); }
      p.epi = gpt2 ? EPI_QKV : EPI_QKV_ROPE;
      p.bias = t.bqkv ? m->wf(t.bqkv) : zero;
      p.y = q; p.ldy = m->qdim;
      p.qdim = m->qdim; p.kdim = m->kdim;
      p.rope_cs = rp.row_cs;
      p.kc = m->kpool(l); p.vc = m->vpool(l); p.kv16 = m->kv16;
      p.kv_hstride = m->bsize * c.head_dim;
      EmbSrc es;
      if (l == 0 && se) {
        // the rows are the step's input embeddings, formed by this launch
        p.pro = PRO_EMBED;
        p.x = nullptr;
        es = EmbSrc{rp, se->sids, se->tok, se->len, se->cap};
      }
      if ((e = run_linear(m, st, "linear.qkv", p, nullptr, p.pro == PRO_EMBED ? &es : nullptr)) != hipSuccess) return e;
    }
    AttnParams a;
    memset(&a, 0, sizeof(a));
    a.q = q; a.ldq = m->qdim;
    a.kc = m->kpool(l); a.vc = m->vpool(l);
    a.table = m->sp<int>(m->o_table); a.max_blocks = m->max_blocks; a.block_size = m->bsize; a.nblk = m->nblk;
    a.Hq = c.n_head; a.Hkv = c.n_kv_head; a.row_seq = rp.row_seq; a.row_pos = rp.row_pos;
    a.row_kvoff = rp.row_kvoff;
    a.M = M;
    a.scale = 1.0f / std::sqrt((float)c.head_dim);
    a.part = apart;
    a.out = attn; a.ldo = m->qdim;
    const bool paged = c.kv_block_size > 0;
    if (fuse_ao) {
      // attention + output projection + bias + residual (in place on x), one launch
      AttnOParams po;
      po.w = m->w + t.wo; po.bias = t.bo ? m->wf(t.bo) : zero;
      po.wsc = m->wt == GD_WEIGHT_Q8 ? m->wf(t.so) : nullptr;
      po.y = x; po.ldy = d; po.N = d; po.K = m->qdim;
      char kn[48];
      snprintf(kn, sizeof(kn), "k_attn_o<%d, %d>", c.head_dim, G);
      ProfScope ps(m, st, "attn_o", kn,
                   kv_pos * c.n_kv_head * c.head_dim * m->kv_elt * 2 + 2.0 * M * m->qdim * 4 +
                       (double)d * m->qdim * m->elt + (m->wt == GD_WEIGHT_Q8 ? d * (m->qdim / 32) * 4.0 : 0.0) + (t.bo ? d * 4.0 : 0.0) + 2.0 * M * d * 4);
      if (c.head_dim == 64 && G == 1) launch_attn_o<64, 1>(st, a, po, paged, m->wt, M, c.n_kv_head, m->kv16);
      else if (c.head_dim == 64) launch_attn_o<64, 3>(st, a, po, paged, m->wt, M, c.n_kv_head, m->kv16);
      else if (G == 1) launch_attn_o<16, 1>(st, a, po, paged, m->wt, M, c.n_kv_head, m->kv16);
      else launch_attn_o<16, 3>(st, a, po, paged, m->wt, M, c.n_kv_head, m->kv16);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    } else if (fuse_ap) {
      // attention + output projection + bias + residual (in place on x), one workgroup
      // per (KV head, row)
      AttnOParams po;
      po.w = m->w + t.wo; po.bias = t.bo ? m->wf(t.bo) : zero;
      po.wsc = m->wt == GD_WEIGHT_Q8 ? m->wf(t.so) : nullptr;
      po.y = x; po.ldy = d; po.N = d; po.K = m->qdim;
      ProfScope ps(m, st, "attn_proj", "k_attn_proj<64>",
                   kv_pos * c.n_kv_head * c.head_dim * m->kv_elt * 2 + M * m->qdim * 4.0 + (double)d * m->qdim * m->elt +
                       (t.bo ? d * 4.0 : 0.0) + 2.0 * M * d * 4);
      launch_attn_proj(st, a, po, m->wt, M, c.n_kv_head, m->kv16);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    } else {
      // causal attention of every row against its sequence's cache (split-context partials)
      dim3 grid(nch, c.n_kv_head, M);
      char kn[48];
      snprintf(kn, sizeof(kn), "k_attention<%d, %d>", c.head_dim, G);
      ProfScope ps(m, st, "attention", kn, kv_pos * c.n_kv_head * c.head_dim * m->kv_elt * 2 + 2.0 * M * m->qdim * 4);
      if (c.head_dim == 64 && G == 1) launch_attention<64, 1>(grid, st, a, paged, m->kv16);
      else if (c.head_dim == 64) launch_attention<64, 3>(grid, st, a, paged, m->kv16);
      else if (G == 1) launch_attention<16, 1>(grid, st, a, paged, m->kv16);
      else launch_attention<16, 3>(grid, st, a, paged, m->kv16);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // output projection + bias + residual (in place on x); the attention partials are
    // merged as the projection stages its rows (gemv; matrix-core up to 16 rows), else
    // by a merge launch first
    if (!fuse_ao && !fuse_ap) {
      LinParams p = base;
      if (long_split) {
        ProfScope ps(m, st, "attn_merge", "k_attn_merge_n",
                     (double)M * c.n_head * (GD_ATT_NCH_LONG * (c.head_dim + 2) + c.head_dim) * 4.0);
        GD_LAUNCH(k_attn_merge_n, dim3(c.n_head, M), dim3(64), 0, st, apart, c.n_head, c.head_dim, GD_ATT_NCH_LONG, attn,
                  m->qdim);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        p.pro = PRO_COPY;
        p.x = attn; p.ldx = m->qdim;
      } else if (o_gemv || (o_mm_merge && nch == GD_ATT_NCH)) {
        p.pro = PRO_ATTN;
        p.apart = apart;
        p.nch = GD_ATT_NCH;
      } else {
        if (nch > 1) {
          ProfScope ps(m, st, "attn_merge", "k_attn_merge", (double)M * c.n_head * (c.head_dim + 2) * 4.0 * 2);
          GD_LAUNCH(k_attn_merge, dim3(M), dim3(GD_WG), 0, st, apart, c.n_head, c.head_dim, attn, m->qdim);
          if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        p.pro = PRO_COPY;
        p.x = attn; p.ldx = m->qdim;
      }
      p.w = m->w + t.wo; p.wtl = m->w + t.to; p.N = d; p.K = m->qdim;
      if (m->wt == GD_WEIGHT_Q8) p.wsc = m->wf(t.so);
      p.epi = EPI_PLAIN;
      p.bias = t.bo ? m->wf(t.bo) : zero;
      p.resid = x; p.ldr = d; p.y = x; p.ldy = d;
      if ((e = run_linear(m, st, "linear.o", p)) != hipSuccess) return e;
    }
    // pre-norm + MLP up: GPT-2 FC + bias + clamped tanh-GELU; Llama gate|up + SiLU gate
    {
      LinParams p = base;
      p.pro = PRO_COPY;
      p.x = x; p.ldx = d;
      p.norm = nrm; p.ng = m->wf(t.n2g); p.nb = t.n2b ? m->wf(t.n2b) : nullptr;
      p.w = m->w + t.wfc; p.wtl = m->w + t.tfc; p.N = m->fcN; p.K = d;
      if (m->wt == GD_WEIGHT_Q8) p.wsc = m->wf(t.sfc);
      if (fold) { p.wf = m->w + t.ffc; p.wfl = m->w + t.tffc; p.bf = m->wf(t.ffc_b); p.fs = m->wf(t.ffc_s); }
      p.epi = gpt2 ? EPI_GELU : EPI_SWIGLU;
      p.bias = t.bfc ? m->wf(t.bfc) : zero;
      p.resid = zero; p.ldr = 0;
      p.y = h; p.ldy = ff;
      if ((e = run_linear(m, st, "linear.fc", p)) != hipSuccess) return e;
    }
    // MLP down + bias + residual (in place on x)
    {
      LinParams p = base;
      p.pro = PRO_COPY;
      p.x = h; p.ldx = ff;
      p.w = m->w + t.wproj; p.wtl = m->w + t.tproj; p.N = d; p.K = ff;
      if (m->wt == GD_WEIGHT_Q8) p.wsc = m->wf(t.sproj);
      p.epi = EPI_PLAIN;
      p.bias = t.bproj ? m->wf(t.bproj) : zero;
      p.resid = x; p.ldr = d; p.y = x; p.ldy = d;
      if ((e = run_linear(m, st, "linear.down", p)) != hipSuccess) return e;
    }
  }
  if (head_out) return enqueue_head(m, st, rp, x, head_row, head_rows, head_out, logits, se ? se->len : nullptr);
  return hipSuccess;
}

// ------------------------------------------------------------ tiled prompt pass

// K splits of a prompt-pass GEMM: the plain epilogue into the in-place residual is
// split until the launch has about two workgroups per CU (each split keeping at least
// four 32-wide K steps); every other GEMM runs unsplit.
static int gemm_pf_splits(const gd_model* m, const LinParams& p) {
  if (p.epi != EPI_PLAIN || p.y != p.resid || p.ldy != p.ldr) return 1;
  const int tiles = iceil(p.N, PF_BN) * iceil(p.M, PF_BM);
  const int want = iceil(2 * m->n_cu, tiles);
  return std::max(1, std::min({want, PF_MAXS, p.K / PF_BK / 4}));
}

// nrm: PFN_NONE, PFN_RMS (SwiGLU and QKV + RoPE: the Llama layout) or PFN_FOLD (GELU
// and QKV with fp32 weights).
template <int WT, bool SPLIT>
static void launch_gemm_pf(hipStream_t st, const LinParams& p, int S, int nrm) {
  const dim3 g(iceil(p.N, PF_BN), iceil(p.M, PF_BM), S), b(PF_NT);
#define PF_GO(E, N) GD_LAUNCH((k_gemm_pf<WT, E, SPLIT, N>), g, b, 0, st, p)
  switch (p.epi) {
    case EPI_PLAIN: PF_GO(EPI_PLAIN, PFN_NONE); break;
    case EPI_GELU:
    case EPI_QKV:
      if constexpr (WT == 0) {
        if (nrm == PFN_FOLD) {
          if (p.epi == EPI_GELU) PF_GO(EPI_GELU, PFN_FOLD);
          else PF_GO(EPI_QKV, PFN_FOLD);
          break;
        }
      }
      if (p.epi == EPI_GELU) PF_GO(EPI_GELU, PFN_NONE);
      else PF_GO(EPI_QKV, PFN_NONE);
      break;
    case EPI_SWIGLU:
      if (nrm == PFN_RMS) PF_GO(EPI_SWIGLU, PFN_RMS);
      else PF_GO(EPI_SWIGLU, PFN_NONE);
      break;
    default:
      if (nrm == PFN_RMS) PF_GO(EPI_QKV_ROPE, PFN_RMS);
      else PF_GO(EPI_QKV_ROPE, PFN_NONE);
      break;
  }
#undef PF_GO
}

// One GEMM of the prompt pass (profiled as role `role`: 2 M N K flops, the bytes of
// the weights, the rows in and out).
static hipError_t run_gemm_pf(gd_model* m, hipStream_t st, const char* role, const LinParams& p,
                              int nrm = PFN_NONE) {
  char kn[48];
  const int S = gemm_pf_splits(m, p);
  // bf16 parts: the default for bf16 weights (three products per weight, 1.3-1.8x
  // faster); for fp32 weights (six products, the weights split too) by default only
  // for the unsplit GEMMs (the wide QKV and MLP-up): the narrow split-K ones measured
  // slower that way
  const bool parts = m->wt == GD_WEIGHT_F32 ? (m->pf_parts == 2 || (m->pf_parts == 1 && S == 1)) : m->pf_parts >= 1;
  snprintf(kn, sizeof(kn), "k_gemm_pf<%d, %d, %s, %d>", m->wt == GD_WEIGHT_F32 ? 0 : 1, p.epi, parts ? "true" : "false",
           nrm);
  ProfScope ps(m, st, role, kn, (double)p.N * p.K * m->elt + 4.0 * p.M * (p.K + p.N));
  if (m->wt == GD_WEIGHT_F32) {
    if (parts) launch_gemm_pf<0, true>(st, p, S, nrm);
    else launch_gemm_pf<0, false>(st, p, S, nrm);
  } else {
    if (parts) launch_gemm_pf<1, true>(st, p, S, nrm);
    else launch_gemm_pf<1, false>(st, p, S, nrm);
  }
  return hipGetLastError();
}

static hipError_t run_rownorm(gd_model* m, hipStream_t st, const float* x, const float* g, const float* b, float* y,
                              int M) {
  const gd_config& c = m->c;
  ProfScope ps(m, st, "pf.norm", "k_rownorm", (double)M * c.d_model * 8.0);
  if (c.arch == GD_ARCH_GPT2)
    GD_LAUNCH(k_rownorm<NORM_LN>, dim3(M), dim3(PF_NT), 0, st, x, c.d_model, g, b, c.norm_eps, c.d_model, y, c.d_model);
  else
    GD_LAUNCH(k_rownorm<NORM_RMS>, dim3(M), dim3(PF_NT), 0, st, x, c.d_model, g, g, c.norm_eps, c.d_model, y,
              c.d_model);
  return hipGetLastError();
}

// The prompt pass over M (<= kPrefillChunk) rows of sequence `seq` at positions
// p0 .. p0 + M - 1, whose metadata rp holds (rp.x = the prompt pass's residual rows):
// pre-norm, QKV GEMM (K/V appended), tiled causal attention, output projection GEMM,
// pre-norm, MLP GEMMs; then, if head_out is given, the head of the last row.
static hipError_t enqueue_prefill_tiled(gd_model* m, hipStream_t st, const RowParams& rp, int seq, int M, int p0,
                                        int* head_out, float* logits) {
  const gd_config& c = m->c;
  const int d = c.d_model, ff = c.d_ff;
  const bool gpt2 = c.arch == GD_ARCH_GPT2;
  float* x = m->sp<float>(m->o_px);
  float* xn = m->sp<float>(m->o_pxn);
  float* q = m->sp<float>(m->o_pq);
  float* att = m->sp<float>(m->o_pattn);
  float* h = m->sp<float>(m->o_ph);
  const float* zero = m->sp<float>(m->o_zero);
  hipError_t e;
  LinParams base;
  memset(&base, 0, sizeof(base));
  base.err = m->sp<int>(m->o_err);
  base.hd = c.head_dim;
  base.Hq = c.n_head;
  base.row_kvoff = rp.row_kvoff;
  base.M = M;
  base.pro = PRO_COPY;
  base.eps = c.norm_eps;
  // the pre-norms inside the QKV and MLP-up GEMMs: RMSNorm (any weights), LayerNorm
  // through the folded fp32 weights; otherwise k_rownorm normalizes the rows first
  const int nrm = !m->use_fold ? PFN_NONE : !gpt2 ? PFN_RMS : m->folded ? PFN_FOLD : PFN_NONE;
  for (int l = 0; l < c.n_layer; ++l) {
    const LayerOff& t = m->L[l];
    if (nrm == PFN_NONE &&
        (e = run_rownorm(m, st, x, m->wf(t.n1g), t.n1b ? m->wf(t.n1b) : nullptr, xn, M)) != hipSuccess)
      return e;
    {
      LinParams p = base;
      p.x = nrm == PFN_NONE ? xn : x; p.ldx = d;
      p.w = m->w + (nrm == PFN_FOLD ? t.fqkv : t.wqkv); p.N = m->qkvdim; p.K = d;
      p.epi = gpt2 ? EPI_QKV : EPI_QKV_ROPE;
      p.bias = nrm == PFN_FOLD ? m->wf(t.fqkv_b) : t.bqkv ? m->wf(t.bqkv) : zero;
      p.fs = nrm == PFN_FOLD ? m->wf(t.fqkv_s) : nullptr;
      p.ng = m->wf(t.n1g);
      p.y = q; p.ldy = m->qdim;
      p.qdim = m->qdim; p.kdim = m->kdim;
      p.rope_cs = rp.row_cs;
      p.kc = m->kpool(l); p.vc = m->vpool(l); p.kv16 = m->kv16;
      p.kv_hstride = m->bsize * c.head_dim;
      if ((e = run_gemm_pf(m, st, "pf.qkv", p, nrm)) != hipSuccess) return e;
    }
    {
      PfAttnParams a;
      a.q = q; a.ldq = m->qdim;
      a.kc = m->kpool(l); a.vc = m->vpool(l);
      const bool paged = c.kv_block_size > 0;
      a.table = paged ? m->sp<int>(m->o_table) + (size_t)seq * m->max_blocks : nullptr;
      a.kv0 = paged ? 0 : (long long)seq * c.n_kv_head * m->bsize * c.head_dim;
      a.block_size = m->bsize; a.nblk = m->nblk; a.Hq = c.n_head; a.Hkv = c.n_kv_head; a.M = M; a.p0 = p0;
      a.scale = 1.0f / std::sqrt((float)c.head_dim);
      a.out = att; a.ldo = m->qdim;
      // key tiles of the last query tile, cut into at most PF_MAXS splits of kt tiles
      const int ntk = (p0 + M - 1) / 64 + 1;
      a.kt = iceil(ntk, PF_MAXS);
      a.S = iceil(ntk, a.kt);
      a.part = m->sp<float>(m->o_ppart);
      const dim3 g(iceil(M, 64), c.n_head, a.S), b(PF_NT);
      {
        // K/V of every attended position: each query tile reads its keys once; with
        // splits, each partial is written and read once more
        double kvb = 0;
        for (int r0 = 0; r0 < M; r0 += 64) kvb += (double)(p0 + std::min(r0 + 64, M)) * c.n_head * c.head_dim * m->kv_elt * 2;
        const double pb = a.S > 1 ? 4.0 * M * c.n_head * a.S * PF_PSTRIDE : 4.0 * M * m->qdim;
        ProfScope ps(m, st, "pf.attention", "k_attn_prefill", kvb + 4.0 * M * m->qdim + pb);
        if (paged && m->kv16) GD_LAUNCH((k_attn_prefill<64, true, true>), g, b, 0, st, a);
        else if (paged) GD_LAUNCH((k_attn_prefill<64, true, false>), g, b, 0, st, a);
        else if (m->kv16) GD_LAUNCH((k_attn_prefill<64, false, true>), g, b, 0, st, a);
        else GD_LAUNCH((k_attn_prefill<64, false, false>), g, b, 0, st, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
      }
      if (a.S > 1) {
        ProfScope ps(m, st, "pf.attn_merge", "k_attn_pf_merge", 4.0 * M * c.n_head * a.S * PF_PSTRIDE + 4.0 * M * m->qdim);
        GD_LAUNCH(k_attn_pf_merge, dim3(M), dim3(PF_NT), 0, st, a.part, c.n_head, a.S, att, m->qdim);
        if ((e = hipGetLastError()) != hipSuccess) return e;
      }
    }
    {
      LinParams p = base;
      p.x = att; p.ldx = m->qdim;
      p.w = m->w + t.wo; p.N = d; p.K = m->qdim;
      p.epi = EPI_PLAIN;
      p.bias = t.bo ? m->wf(t.bo) : zero;
      p.resid = x; p.ldr = d; p.y = x; p.ldy = d;
      if ((e = run_gemm_pf(m, st, "pf.o", p)) != hipSuccess) return e;
    }
    if (nrm == PFN_NONE &&
        (e = run_rownorm(m, st, x, m->wf(t.n2g), t.n2b ? m->wf(t.n2b) : nullptr, xn, M)) != hipSuccess)
      return e;
    {
      LinParams p = base;
      p.x = nrm == PFN_NONE ? xn : x; p.ldx = d;
      p.w = m->w + (nrm == PFN_FOLD ? t.ffc : t.wfc); p.N = m->fcN; p.K = d;
      p.epi = gpt2 ? EPI_GELU : EPI_SWIGLU;
      p.bias = nrm == PFN_FOLD ? m->wf(t.ffc_b) : t.bfc ? m->wf(t.bfc) : zero;
      p.fs = nrm == PFN_FOLD ? m->wf(t.ffc_s) : nullptr;
      p.ng = m->wf(t.n2g);
      p.resid = zero; p.ldr = 0;
      p.y = h; p.ldy = ff;
      if ((e = run_gemm_pf(m, st, "pf.fc", p, nrm)) != hipSuccess) return e;
    }
    {
      LinParams p = base;
      p.x = h; p.ldx = ff;
      p.w = m->w + t.wproj; p.N = d; p.K = ff;
      p.epi = EPI_PLAIN;
      p.bias = t.bproj ? m->wf(t.bproj) : zero;
      p.resid = x; p.ldr = d; p.y = x; p.ldy = d;
      if ((e = run_gemm_pf(m, st, "pf.down", p)) != hipSuccess) return e;
    }
  }
  if (head_out) return enqueue_head(m, st, rp, x, M - 1, 1, head_out, logits);
  return hipSuccess;
}

static gd_status ready(gd_model* m) {
  if (!m) return set_err(GD_ERR_INVALID, "model is NULL");
  if (m->poisoned) return set_err(GD_ERR_HIP, "model is poisoned by an earlier HIP error");
  if (!m->bound) return set_err(GD_ERR_STATE, "memory not bound");
  if (!m->loaded) return set_err(GD_ERR_STATE, "weights not loaded");
  return GD_OK;
}

extern "C" gd_status gd_prefill(gd_model* m, int32_t seq, const int32_t* tokens, int32_t n, int32_t* next_dev,
                                float* logits_dev) {
  gd_status st = ready(m);
  if (st != GD_OK) return st;
  const gd_config& c = m->c;
  if (seq < 0 || seq >= c.max_seqs) return set_err(GD_ERR_INVALID, "seq %d out of range", seq);
  if (!tokens || n < 1) return set_err(GD_ERR_INVALID, "prefill needs at least one token");
  if (!next_dev) return set_err(GD_ERR_INVALID, "next_token_dev is NULL");
  for (int i = 0; i < n; ++i)
    if (tokens[i] < 0 || tokens[i] >= c.vocab) return set_err(GD_ERR_INVALID, "token %d out of range at %d", tokens[i], i);
  const int p0 = m->len[seq];
  if (p0 + n > m->cap[seq])
    return set_err(GD_ERR_CTX_FULL, "sequence %d: %d + %d positions exceed capacity %d", seq, p0, n, m->cap[seq]);
  if ((st = staging_wait(m)) != GD_OK) return st;
  int* hs = m->staging;
  int* hp = hs + n;
  int* ht = hs + 2 * n;
  for (int i = 0; i < n; ++i) { hs[i] = seq; hp[i] = p0 + i; ht[i] = tokens[i]; }
  hs[3 * n] = p0 + n;
  hipStream_t s = m->stream;
  HIP_TRY(m, hipMemcpyAsync(m->sp<int>(m->o_pseq), hs, (size_t)n * 4, hipMemcpyHostToDevice, s));
  HIP_TRY(m, hipMemcpyAsync(m->sp<int>(m->o_ppos), hp, (size_t)n * 4, hipMemcpyHostToDevice, s));
  HIP_TRY(m, hipMemcpyAsync(m->sp<int>(m->o_ptok), ht, (size_t)n * 4, hipMemcpyHostToDevice, s));
  HIP_TRY(m, hipMemcpyAsync(m->sp<int>(m->o_len) + seq, hs + 3 * n, 4, hipMemcpyHostToDevice, s));
  if ((st = staging_done(m)) != GD_OK) return st;
  if (m->pf_ok && m->use_pf && n >= kPrefillMinRows) {
    for (int r0 = 0; r0 < n; r0 += kPrefillChunk) {
      const int M = std::min(kPrefillChunk, n - r0);
      const bool last = r0 + M == n;
      RowParams rp = row_params(m, m->sp<int>(m->o_pseq) + r0, m->sp<int>(m->o_ppos) + r0,
                                m->sp<int>(m->o_ptok) + r0, m->sp<long long>(m->o_pkv) + r0,
                                c.arch == GD_ARCH_LLAMA ? m->sp<float>(m->o_pcs) + (size_t)r0 * c.head_dim : nullptr);
      rp.x = m->sp<float>(m->o_px);
      hipError_t e;
      {
        ProfScope ps(m, s, "setup", "k_setup_rows", (double)M * c.d_model * (m->elt * 2 + 4));
        GD_LAUNCH(k_setup_rows, dim3(M), dim3(GD_WG), 0, s, rp);
        e = hipGetLastError();
      }
      if (e == hipSuccess)
        e = enqueue_prefill_tiled(m, s, rp, seq, M, p0 + r0, last ? next_dev : nullptr, last ? logits_dev : nullptr);
      if (e != hipSuccess) {
        m->poisoned = true;
        return set_err(GD_ERR_HIP, "prefill launch failed: %s", hipGetErrorString(e));
      }
    }
    m->len[seq] = p0 + n;
    return GD_OK;
  }
  for (int r0 = 0; r0 < n; r0 += GD_MAX_ROWS) {
    int M = std::min(GD_MAX_ROWS, n - r0);
    bool last = r0 + M == n;
    m->prof_T.clear();
    if (m->profile)
      for (int i = 0; i < M; ++i) m->prof_T.push_back(p0 + r0 + i + 1);
    RowParams rp = row_params(m, m->sp<int>(m->o_pseq) + r0, m->sp<int>(m->o_ppos) + r0,
                              m->sp<int>(m->o_ptok) + r0, m->sp<long long>(m->o_pkv) + r0,
                              c.arch == GD_ARCH_LLAMA ? m->sp<float>(m->o_pcs) + (size_t)r0 * c.head_dim : nullptr);
    hipError_t e;
    {
      ProfScope ps(m, s, "setup", "k_setup_rows", (double)M * c.d_model * (m->elt * 2 + 4));
      GD_LAUNCH(k_setup_rows, dim3(M), dim3(GD_WG), 0, s, rp);
      e = hipGetLastError();
    }
    if (e == hipSuccess)
      e = enqueue_rows(m, s, rp, M, p0 + r0 + M, M - 1, 1, last ? next_dev : nullptr, last ? logits_dev : nullptr);
    if (e != hipSuccess) {
      m->poisoned = true;
      return set_err(GD_ERR_HIP, "prefill launch failed: %s", hipGetErrorString(e));
    }
  }
  m->len[seq] = p0 + n;
  return GD_OK;
}

static hipError_t enqueue_decode(gd_model* m, hipStream_t st, int B, int max_T, const int* tok, int* next,
                                 float* logits) {
  RowParams rp = row_params(m, m->sp<int>(m->o_rseq), m->sp<int>(m->o_rpos), m->sp<int>(m->o_rtok),
                            m->sp<long long>(m->o_rkv),
                            m->c.arch == GD_ARCH_LLAMA ? m->sp<float>(m->o_rcs) : nullptr);
  // With a GEMV QKV launch (<= 4 rows) the set-up runs inside it (one launch fewer);
  // the matrix-core one stages its rows from the set-up launch's output.
  const gd_config& c = m->c;
  const int qkv_epi = c.arch == GD_ARCH_GPT2 ? EPI_QKV : EPI_QKV_ROPE;
  const StepEmbed se{m->sp<int>(m->o_sids), tok, m->sp<int>(m->o_len), m->sp<int>(m->o_cap)};
  const LinPlan qp = plan_linear(B, m->qkvdim, c.d_model, m->wt, m->variant, qkv_epi, true);
  const bool embed = next != nullptr && qp.var == 0 && qp.rows >= B;   // one launch over all rows
  if (!embed) {
    ProfScope ps(m, st, "setup", "k_setup_decode", (double)B * c.d_model * (m->elt * 2 + 4));
    GD_LAUNCH(k_setup_decode, dim3(B), dim3(GD_WG), 0, st, rp, se.sids, tok, se.len, se.cap);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return enqueue_rows(m, st, rp, B, max_T, 0, B, next, logits, embed ? &se : nullptr);
}

extern "C" gd_status gd_decode_step(gd_model* m, int32_t B, const int32_t* sids, const int32_t* tok_dev,
                                    int32_t* next_dev, float* logits_dev) {
  gd_status st = ready(m);
  if (st != GD_OK) return st;
  const gd_config& c = m->c;
  if (B < 1 || B > c.max_batch) return set_err(GD_ERR_INVALID, "batch %d outside 1..%d", B, c.max_batch);
  if (!sids || !tok_dev || !next_dev) return set_err(GD_ERR_INVALID, "NULL argument");
  for (int b = 0; b < B; ++b) {
    if (sids[b] < 0 || sids[b] >= c.max_seqs) return set_err(GD_ERR_INVALID, "seq id %d out of range", sids[b]);
    for (int b2 = 0; b2 < b; ++b2)
      if (sids[b2] == sids[b]) return set_err(GD_ERR_INVALID, "seq id %d repeated in the batch", sids[b]);
    if (m->len[sids[b]] < 1) return set_err(GD_ERR_STATE, "sequence %d has no prefilled context", sids[b]);
    if (m->len[sids[b]] >= m->cap[sids[b]])
      return set_err(GD_ERR_CTX_FULL, "sequence %d is full (%d positions)", sids[b], m->cap[sids[b]]);
  }
  hipStream_t s = m->stream;
  std::vector<int> want(sids, sids + B);
  if (want != m->last_sids) {
    if ((st = staging_wait(m)) != GD_OK) return st;
    memcpy(m->staging, sids, (size_t)B * 4);
    HIP_TRY(m, hipMemcpyAsync(m->sp<int>(m->o_sids), m->staging, (size_t)B * 4, hipMemcpyHostToDevice, s));
    if ((st = staging_done(m)) != GD_OK) return st;
    m->last_sids = want;
  }
  m->prof_T.clear();
  if (m->profile)
    for (int b = 0; b < B; ++b) m->prof_T.push_back(m->len[sids[b]] + 1);
  int max_T = 0;   // attended positions of the longest row
  for (int b = 0; b < B; ++b) max_T = std::max(max_T, m->len[sids[b]] + 1);
  if (m->profile && m->profile_gated) {
    // hold the stream (bounded) while the step is enqueued, then let it run whole
    if (!m->gate_evt) HIP_TRY(m, hipEventCreateWithFlags(&m->gate_evt, hipEventDisableTiming));
    hipLaunchKernelGGL(k_gate, dim3(1), dim3(64), 0, m->cap_stream, 300000LL);
    HIP_TRY(m, hipGetLastError());
    HIP_TRY(m, hipEventRecord(m->gate_evt, m->cap_stream));
    HIP_TRY(m, hipStreamWaitEvent(s, m->gate_evt, 0));
    hipError_t e = enqueue_decode(m, s, B, max_T, tok_dev, next_dev, logits_dev);
    if (e != hipSuccess) {
      m->poisoned = true;
      return set_err(GD_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
    }
  } else if (m->use_graph && !m->profile) {
    GraphKey key{B, tok_dev, next_dev, logits_dev, max_T <= kFusedAttnOMaxT, max_T >= kLongCtxT};
    auto it = m->graphs.find(key);
    if (it == m->graphs.end()) {
      if (m->graphs.size() >= kMaxGraphs) {
        // drop the least recently launched graph; it may still run on the stream
        auto lru = m->graphs.begin();
        for (auto g = m->graphs.begin(); g != m->graphs.end(); ++g)
          if (g->second.last_use < lru->second.last_use) lru = g;
        HIP_TRY(m, hipStreamSynchronize(s));
        HIP_TRY(m, hipGraphExecDestroy(lru->second.exec));
        m->graphs.erase(lru);
      }
      hipGraph_t g;
      HIP_TRY(m, hipStreamBeginCapture(m->cap_stream, hipStreamCaptureModeThreadLocal));
      hipError_t e = enqueue_decode(m, m->cap_stream, B, max_T, tok_dev, next_dev, logits_dev);
      hipError_t e2 = hipStreamEndCapture(m->cap_stream, &g);
      if (e != hipSuccess || e2 != hipSuccess) {
        m->poisoned = true;
        return set_err(GD_ERR_HIP, "decode capture failed: %s / %s", hipGetErrorString(e), hipGetErrorString(e2));
      }
      hipGraphExec_t ex;
      hipError_t e3 = hipGraphInstantiate(&ex, g, nullptr, nullptr, 0);
      (void)hipGraphDestroy(g);
      if (e3 != hipSuccess) {
        m->poisoned = true;
        return set_err(GD_ERR_HIP, "graph instantiate failed: %s", hipGetErrorString(e3));
      }
      it = m->graphs.emplace(key, gd_model::GraphEntry{ex, 0}).first;
    }
    it->second.last_use = ++m->graph_clock;
    HIP_TRY(m, hipGraphLaunch(it->second.exec, s));
  } else {
    hipError_t e = enqueue_decode(m, s, B, max_T, tok_dev, next_dev, logits_dev);
    if (e != hipSuccess) {
      m->poisoned = true;
      return set_err(GD_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
    }
  }
  for (int b = 0; b < B; ++b) m->len[sids[b]] += 1;
  return GD_OK;
}

// ---------------------------------------------------------------- op level

static gd_status linear_check(int M, int N, int K, int variant) {
  if (M < 1 || M > GD_MAX_ROWS || N < 1 || K < 8 || K % 8 || K > kMaxK)
    return set_err(GD_ERR_INVALID, "bad shape M=%d N=%d K=%d", M, N, K);
  if (variant < 0 || variant > 2) return set_err(GD_ERR_INVALID, "bad variant %d", variant);
  return GD_OK;
}

// The op-level linear's workspace: a zero vector read in place of an absent bias or
// residual, then room for the tile-major copy of W that the matrix-core kernel reads
// (sized for fp32, filled on every call that uses that kernel).
static size_t linear_ws_zero_bytes(int N) { return align_up((size_t)N * 4, 256); }
static size_t linear_ws_bytes(int N, int K) { return linear_ws_zero_bytes(N) + mm_packed_bytes(0, N, K); }

extern "C" gd_status gd_linear_workspace(int32_t M, int32_t N, int32_t K, int32_t variant, size_t* bytes) {
  if (!bytes) return set_err(GD_ERR_INVALID, "bytes is NULL");
  gd_status st = linear_check(M, N, K, variant);
  if (st != GD_OK) return st;
  *bytes = linear_ws_bytes(N, K);
  return GD_OK;
}

extern "C" gd_status gd_linear(const float* x, int32_t ldx, const void* W, int32_t wdt, const float* bias,
                               int32_t norm, const float* ng, const float* nb, float eps, int32_t act,
                               const float* resid, int32_t ldr, float* y, int32_t ldy, int32_t M, int32_t N, int32_t K,
                               int32_t variant, void* ws, size_t ws_bytes, void* stream) {
  gd_status st = linear_check(M, N, K, variant);
  if (st != GD_OK) return st;
  if (!x || !W || !y) return set_err(GD_ERR_INVALID, "NULL argument");
  if (wdt != GD_WEIGHT_F32 && wdt != GD_WEIGHT_BF16) return set_err(GD_ERR_INVALID, "bad weight dtype");
  if (norm < 0 || norm > 2 || (norm && !ng) || (norm == 1 && !nb)) return set_err(GD_ERR_INVALID, "bad norm");
  if (norm && !(eps > 0.f)) return set_err(GD_ERR_INVALID, "eps must be > 0");
  if (act != GD_ACT_NONE && act != GD_ACT_GELU) return set_err(GD_ERR_INVALID, "bad act");
  if (ldx < K || ldx % 4 || ldy < N || (resid && ldr < N)) return set_err(GD_ERR_INVALID, "bad leading dimensions");
  if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(W)) & 15)
    return set_err(GD_ERR_INVALID, "x and W must be 16-byte aligned");
  if (!ws || ws_bytes < linear_ws_bytes(N, K))
    return set_err(GD_ERR_OOM, "workspace %zu < %zu bytes", ws_bytes, linear_ws_bytes(N, K));
  const float* zero = static_cast<const float*>(ws);
  LinParams p;
  memset(&p, 0, sizeof(p));
  p.pro = PRO_COPY;
  p.norm = norm == GD_NORM_LAYER ? NORM_LN : norm == GD_NORM_RMS ? NORM_RMS : NORM_NONE;
  p.x = x; p.ldx = ldx; p.ng = ng; p.nb = nb; p.eps = eps;
  p.w = W; p.M = M; p.N = N; p.K = K;
  p.epi = act == GD_ACT_GELU ? EPI_GELU : EPI_PLAIN;
  p.bias = bias ? bias : zero;
  p.resid = resid ? resid : zero;
  p.ldr = resid ? ldr : 0;
  p.y = y; p.ldy = ldy;
  const bool inplace = resid && resid == y && ldr == ldy;
  LinPlan lp = plan_linear(M, N, K, wdt, variant, p.epi, p.norm != NORM_NONE, inplace);
  hipError_t e = hipSuccess;
  if (lp.var == 1) {
    void* packed = static_cast<char*>(ws) + linear_ws_zero_bytes(N);
    e = launch_pack(W, wdt, N, K, packed, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return set_err(GD_ERR_HIP, "linear launch failed: %s", hipGetErrorString(e));
    p.wtl = packed;
  }
  e = run_linear_rows(wdt, lp, p, reinterpret_cast<hipStream_t>(stream), nullptr, nullptr, nullptr);
  if (e != hipSuccess) return set_err(GD_ERR_HIP, "linear launch failed: %s", hipGetErrorString(e));
  return GD_OK;
}

extern "C" gd_status gd_argmax_workspace(int32_t rows, int32_t vocab, size_t* bytes) {
  if (!bytes || rows < 1 || rows > GD_MAX_ROWS || vocab < 1) return set_err(GD_ERR_INVALID, "bad argmax shape");
  int nch = iceil(vocab, 4096);
  *bytes = 2 * align_up((size_t)rows * nch * 4, 256) + align_up((size_t)rows * 4, 256);
  return GD_OK;
}

extern "C" gd_status gd_argmax(const float* logits, int32_t rows, int32_t vocab, int32_t* out, void* ws,
                               size_t ws_bytes, void* stream) {
  size_t need;
  gd_status st = gd_argmax_workspace(rows, vocab, &need);
  if (st != GD_OK) return st;
  if (!logits || !out || !ws) return set_err(GD_ERR_INVALID, "NULL argument");
  if (ws_bytes < need) return set_err(GD_ERR_OOM, "workspace %zu < %zu bytes", ws_bytes, need);
  int nch = iceil(vocab, 4096);
  char* b = static_cast<char*>(ws);
  float* pv = reinterpret_cast<float*>(b);
  int* pi = reinterpret_cast<int*>(b + align_up((size_t)rows * nch * 4, 256));
  int* ctr = reinterpret_cast<int*>(b + 2 * align_up((size_t)rows * nch * 4, 256));
  GD_LAUNCH(k_argmax_rows, dim3(nch, rows), dim3(GD_WG), 0, reinterpret_cast<hipStream_t>(stream), logits,
                     rows, vocab, nch, pv, pi, ctr, out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_err(GD_ERR_HIP, "argmax launch failed: %s", hipGetErrorString(e));
  return GD_OK;
}

// ------------------------------------------------- argmax without allocation
//
// gd_argmax_static keeps the per-chunk partials and the per-row arrival counters of
// k_argmax_rows in `scratch`, a file-scope device array: one copy per GPU, held until
// the process ends. Host code never passes `scratch` itself to a kernel (on the host
// it is only a stand-in for the symbol): the first call on each device looks up that
// device's copy with hipGetSymbolAddress and keeps the address.
static const int kStaticArgmaxMaxVocab = 1 << 20;
static const int kStaticArgmaxChunks = kStaticArgmaxMaxVocab / 4096;   // chunks of k_argmax_rows
static const size_t kStaticPartBytes = (size_t)GD_MAX_ROWS * kStaticArgmaxChunks * 4;
static const size_t kStaticScratchBytes = 2 * kStaticPartBytes + 256;   // values, indices, counters
static __device__ __align__(256) char scratch[kStaticScratchBytes];

static const int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// Clears n ints (a fill kernel rather than a memset, so that the call can be captured).
__global__ void k_zero_ints(int* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

extern "C" gd_status gd_argmax_static(const float* logits, int32_t rows, int32_t vocab, int32_t* out,
                                      void* hip_stream) {
  if (rows < 1 || rows > GD_MAX_ROWS)
    return set_err(GD_ERR_INVALID, "argmax_static: rows %d outside 1..%d", rows, GD_MAX_ROWS);
  if (vocab < 1 || vocab > kStaticArgmaxMaxVocab)
    return set_err(GD_ERR_INVALID, "argmax_static: vocab %d outside 1..%d (the static scratch holds %d chunks "
                   "per row)", vocab, kStaticArgmaxMaxVocab, kStaticArgmaxChunks);
  if (!logits || !out) return set_err(GD_ERR_INVALID, "NULL argument");
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return set_err(GD_ERR_NO_DEVICE, "argmax_static: no current device below %d", kMaxDevices);
  char* base;
  {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      void* ptr = nullptr;
      const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !ptr)
        return set_err(GD_ERR_HIP, "argmax_static: hipGetSymbolAddress failed on device %d: %s", dev,
                       hipGetErrorString(e));
      g_scratch_ptr[dev] = ptr;
    }
    base = static_cast<char*>(g_scratch_ptr[dev]);
  }
  float* pv = reinterpret_cast<float*>(base);
  int* pi = reinterpret_cast<int*>(base + kStaticPartBytes);
  int* ctr = reinterpret_cast<int*>(base + 2 * kStaticPartBytes);
  const hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
  const int nch = iceil(vocab, 4096);
  hipLaunchKernelGGL(k_zero_ints, dim3(1), dim3(64), 0, st, ctr, rows);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) {
    GD_LAUNCH(k_argmax_rows, dim3(nch, rows), dim3(GD_WG), 0, st, logits, rows, vocab, nch, pv, pi, ctr, out);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return set_err(GD_ERR_HIP, "argmax_static launch failed: %s", hipGetErrorString(e));
  return GD_OK;
}
