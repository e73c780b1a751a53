// linear.h -- y = epilogue(prologue(x) . W^T) for 1..32 activation rows.
//
// A linear layer is y = x . W^T with W stored [out][in] ("rvllm Metal backend",
// "The matmul pain story"). One decode step streams every weight once and does
// little arithmetic per byte, so both kernels are built around streaming W with
// 16-byte loads issued before anything that depends on the activations.
//
// Cross-workgroup communication happens only at kernel boundaries: an agent-scope
// fence costs tens of nanoseconds per workgroup and serializes, so no split-K or
// last-arriver reductions are used here.
//
// k_gemv (1..4 rows, VALU): each wave owns RW weight rows; lane l holds chunks
//   c = l + 64 i (16 bytes each: 4 fp32 or 8 bf16 weights) of each row in registers,
//   loaded first. Meanwhile the workgroup stages the activation rows in LDS through a
//   prologue (a copy or, for the first layer, the token + position embedding, or
//   the merge of split-context attention partials), then LayerNorm or RMSNorm of
//   each row. Dot products are reduced across the wave.
// k_mfma (5..32 rows): v_mfma_f32_16x16x4f32 on a 16-column tile. Lane l holds
//   W[n0 + l%16][k + 8(l/16) .. +8] and X[m0 + l%16][same k]; step t of 8 feeds
//   element t of both, so the four k-slots of one instruction are k + 8q + t
//   (q = l/16) for A and B alike. NW waves split K by 32-element blocks; X fragments
//   come straight from L2 with the row normalization applied on the fly.
//
// Epilogues: bias, clamped tanh-GELU, residual add; SiLU-gated pairs (gate and up
// rows interleaved, gate at even rows); QKV scatter (q to a buffer, k and v into the
// KV cache at the row's (sequence, position), with rotate-half RoPE for the Llama
// layout whose q/k rows are packed as adjacent (i, i + hd/2) pairs); greedy argmax
// partials per workgroup (reduced by k_argmax_finalize).
#pragma once
#include "common.h"
#include "attention.h"

// Source of the activation rows.
#define PRO_COPY 0   // x rows as given
#define PRO_ATTN 3   // merge of split-context attention partials
// Row normalization applied after the source (LinParams::norm).
#define NORM_NONE 0
#define NORM_LN 1    // (x - mean) / sqrt(var + eps) * g + b, biased variance
#define NORM_RMS 2   // x / sqrt(mean(x^2) + eps) * g

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
  const float* apart; int Hq;               // ATTN: partials [M][Hq][GD_ATT_NCH][hd + 2]
  int* err;
  const long long* row_kvoff;               // element offset of each row's K/V slot in a layer pool (-1: none)
  // ---- weights
  const void* w; int M, N, K;
  // ---- epilogue
  int epi;
  const float* bias;                        // never NULL: a zero vector when the layer has none
  const float* resid; int ldr;              // never NULL for PLAIN/GELU: zeros with ldr = 0 when none
  float* y; int ldy;
  float* am_val; int* am_idx;               // [gridDim.x][M]
  float* logits; int ldl;
  int qdim, kdim, hd, kv_hstride;           // QKV: head g of a slot at + g * kv_hstride
  const float* rope_cs;                     // [M][hd]: each row's cos | sin of pair i (NULL: no RoPE)
  float* kc; float* vc;
};

// ------------------------------------------------------------ shared pieces

// Destination of QKV output column n of row m: q columns go to y, k and v columns
// into this layer's cache slot of the row (none if the slot is invalid).
__device__ __forceinline__ float* qkv_dst(const LinParams& p, int m, int n, long long kvoff) {
  if (n < p.qdim) return p.y + (size_t)m * p.ldy + n;
  if (kvoff < 0) return nullptr;
  int kn = n - p.qdim;
  float* base = p.kc;
  if (kn >= p.kdim) { kn -= p.kdim; base = p.vc; }
  const int g = kn / p.hd, d = kn - g * p.hd;
  return base + kvoff + (size_t)g * p.kv_hstride + d;
}

template <int EPI>
struct EpiTraits { static constexpr bool pair = EPI == EPI_SWIGLU || EPI == EPI_QKV_ROPE; };

// Epilogue operands of one output column n (or adjacent pair n, n + 1) of row m. They
// are plain loads whose addresses depend only on kernel arguments and indices, issued
// at kernel start so that their latency overlaps the weight stream; every decision
// that depends on a loaded value is taken in epi_store.
struct EpiOps {
  float b0, b1, r0;   // bias of n and n + 1, residual of n
  float c, s;         // RoPE cos/sin of the pair
  long long kvoff;    // the row's cache slot (QKV)
};

template <int EPI>
__device__ __forceinline__ EpiOps epi_prefetch(const LinParams& p, int m, int n) {
  EpiOps e;
  e.b0 = e.b1 = e.r0 = 0.f;
  e.c = 1.f; e.s = 0.f;
  e.kvoff = 0;
  if (EPI == EPI_PLAIN || EPI == EPI_GELU) {
    e.b0 = p.bias[n];
    e.r0 = p.resid[(size_t)m * p.ldr + n];
  } else if (EPI == EPI_QKV) {
    e.b0 = p.bias[n];
    e.kvoff = p.row_kvoff[m];
  } else if (EPI == EPI_QKV_ROPE) {
    e.b0 = p.bias[n];
    e.b1 = p.bias[n + 1];
    e.kvoff = p.row_kvoff[m];
    const int i = (n % p.hd) >> 1;
    const float* cs = p.rope_cs + (size_t)m * p.hd;
    e.c = cs[i];
    e.s = cs[(p.hd >> 1) + i];
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
      float* d1 = qkv_dst(p, m, n + 1, e.kvoff);
      if (d1) *d1 = v1;
    }
    float* d0 = qkv_dst(p, m, n, e.kvoff);
    if (d0) *d0 = v0;
  } else {
    v0 += e.b0;
    if (EPI == EPI_GELU) v0 = gelu_clamped(v0);
    p.y[(size_t)m * p.ldy + n] = e.r0 + v0;
  }
}

// Activation rows are staged into LDS xs[m * K + k] in two parts. stage_issue loads
// the first XPT float4 chunks of this thread (rows, and the norm's gain and shift)
// into registers; it runs before the weight loads, so that waiting for the rows
// does not wait for the weight stream (vector loads complete in issue order).
// stage_finish stores them, loads any remaining chunks, and normalizes the rows.
template <int XPT>
struct RowRegs {
  f32x4 x[XPT], g[XPT], b[XPT];
  float x0[GEMV_MAX_ROWS];   // first element of each row (shift of the one-pass moments)
};

template <int XPT>
__device__ __forceinline__ void stage_issue(const LinParams& p, RowRegs<XPT>& rr) {
  // Loads are unconditional (clamped to the last valid chunk; stage_finish stores only
  // valid ones), so the compiler can count them and wait for these alone later.
  if (p.pro != PRO_COPY) return;
  const int tid = threadIdx.x, K4 = p.K >> 2;
  const float* gsrc = p.ng ? p.ng : p.x;
  const float* bsrc = p.nb ? p.nb : gsrc;
#pragma unroll
  for (int j = 0; j < XPT; ++j) {
    const int i = min(tid + GD_WG * j, p.M * K4 - 1);
    const int m = i / K4, k = (i - m * K4) << 2;
    rr.x[j] = *reinterpret_cast<const f32x4*>(p.x + (size_t)m * p.ldx + k);
    const int kg = min(tid + GD_WG * j, K4 - 1) << 2;
    rr.g[j] = *reinterpret_cast<const f32x4*>(gsrc + kg);
    rr.b[j] = *reinterpret_cast<const f32x4*>(bsrc + kg);
  }
#pragma unroll
  for (int m = 0; m < GEMV_MAX_ROWS; ++m) rr.x0[m] = p.x[(size_t)min(m, p.M - 1) * p.ldx];
}

// Sum over the workgroup of one value per row (rows < M), for every thread.
__device__ __forceinline__ void block_sum_rows(float v[GEMV_MAX_ROWS], int M, float (*red)[GEMV_MAX_ROWS]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int m = 0; m < GEMV_MAX_ROWS; ++m)
    if (m < M) v[m] = wave_sum(v[m]);
  if (lane == 0) {
#pragma unroll
    for (int m = 0; m < GEMV_MAX_ROWS; ++m) red[wave][m] = v[m];
  }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < GEMV_MAX_ROWS; ++m) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < GD_WG / 64; ++w) t += red[w][m];
    v[m] = t;
  }
}

template <int XPT>
__device__ void stage_finish(const LinParams& p, float* xs, float* s_gb, const RowRegs<XPT>& rr,
                             float (*red)[GD_WG / 64][GEMV_MAX_ROWS]) {
  const int tid = threadIdx.x;
  const int M = p.M, K = p.K;
  if (p.pro == PRO_ATTN) {
    const int hd = p.hd;
    for (int i = tid; i < M * K; i += GD_WG) {
      const int m = i / K, k = i - m * K;
      const int h = k / hd, d = k - h * hd;
      xs[i] = attn_merge_one(p.apart + ((size_t)m * p.Hq + h) * GD_ATT_NCH * (hd + 2), hd, d);
    }
    return;
  }
  const int K4 = K >> 2;
  float* s_g = s_gb;
  float* s_b = s_gb + K;
  if (p.norm != NORM_NONE && M * K4 <= GD_WG * XPT) {
    // Every row is in registers: moments from registers with one workgroup reduction,
    // shifted by the row's first element (sum d and sum d^2 with d = x - x0), then
    // normalize in registers and store. RMSNorm uses the unshifted sum of squares.
    float s1[GEMV_MAX_ROWS], s2[GEMV_MAX_ROWS];
#pragma unroll
    for (int m = 0; m < GEMV_MAX_ROWS; ++m) s1[m] = s2[m] = 0.f;
    const bool ln = p.norm == NORM_LN;
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const int i = tid + GD_WG * j;
      if (i < M * K4) {
        const int m = i / K4;
#pragma unroll
        for (int mm = 0; mm < GEMV_MAX_ROWS; ++mm)
          if (mm == m) {
            const float sh = ln ? rr.x0[mm] : 0.f;
            const float d0 = rr.x[j].x - sh, d1 = rr.x[j].y - sh, d2 = rr.x[j].z - sh, d3 = rr.x[j].w - sh;
            s1[mm] += (d0 + d1) + (d2 + d3);
            s2[mm] += fmaf(d0, d0, d1 * d1) + fmaf(d2, d2, d3 * d3);
          }
      }
    }
    block_sum_rows(s1, M, red[0]);
    block_sum_rows(s2, M, red[1]);
    float mu[GEMV_MAX_ROWS], rs[GEMV_MAX_ROWS];
#pragma unroll
    for (int m = 0; m < GEMV_MAX_ROWS; ++m) {
      const float a = s1[m] / (float)K;                  // mean of d
      const float var = ln ? fmaxf(s2[m] / (float)K - a * a, 0.f) : s2[m] / (float)K;
      mu[m] = ln ? rr.x0[m] + a : 0.f;
      rs[m] = 1.0f / sqrtf(var + p.eps);
    }
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const int i = tid + GD_WG * j;
      if (i < M * K4) {
        const int m = i / K4, k = (i - m * K4) << 2;
        float u = 0.f, r = 0.f;
#pragma unroll
        for (int mm = 0; mm < GEMV_MAX_ROWS; ++mm)
          if (mm == m) { u = mu[mm]; r = rs[mm]; }
        f32x4 v = rr.x[j];
        f32x4 gg, bb;
        if (m == 0) { gg = rr.g[j]; bb = rr.b[j]; }   // this thread's gain/shift chunk is column k
        else {
          gg = *reinterpret_cast<const f32x4*>(p.ng + k);
          bb = ln ? *reinterpret_cast<const f32x4*>(p.nb + k) : (f32x4){0.f, 0.f, 0.f, 0.f};
        }
        if (ln) {
          v.x = (v.x - u) * r * gg.x + bb.x; v.y = (v.y - u) * r * gg.y + bb.y;
          v.z = (v.z - u) * r * gg.z + bb.z; v.w = (v.w - u) * r * gg.w + bb.w;
        } else {
          v.x = v.x * r * gg.x; v.y = v.y * r * gg.y; v.z = v.z * r * gg.z; v.w = v.w * r * gg.w;
        }
        *reinterpret_cast<f32x4*>(xs + m * K + k) = v;
      }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < XPT; ++j) {
    const int i = tid + GD_WG * j;
    if (i < M * K4) {
      const int m = i / K4, k = (i - m * K4) << 2;
      *reinterpret_cast<f32x4*>(xs + m * K + k) = rr.x[j];
    }
    if (p.norm != NORM_NONE && i < K4) {
      *reinterpret_cast<f32x4*>(s_g + 4 * i) = rr.g[j];
      if (p.norm == NORM_LN) *reinterpret_cast<f32x4*>(s_b + 4 * i) = rr.b[j];
    }
  }
  for (int i = tid + GD_WG * XPT; i < M * K4; i += GD_WG) {   // rows beyond the register share
    const int m = i / K4, k = (i - m * K4) << 2;
    *reinterpret_cast<f32x4*>(xs + m * K + k) = *reinterpret_cast<const f32x4*>(p.x + (size_t)m * p.ldx + k);
    if (p.norm != NORM_NONE && i < K4) {
      *reinterpret_cast<f32x4*>(s_g + 4 * i) = *reinterpret_cast<const f32x4*>(p.ng + 4 * i);
      if (p.norm == NORM_LN) *reinterpret_cast<f32x4*>(s_b + 4 * i) = *reinterpret_cast<const f32x4*>(p.nb + 4 * i);
    }
  }
  if (p.norm == NORM_NONE) return;
  __syncthreads();
  // row statistics over the whole workgroup: mean, then the mean of squared deviations
  float mean[GEMV_MAX_ROWS], var[GEMV_MAX_ROWS];
#pragma unroll
  for (int m = 0; m < GEMV_MAX_ROWS; ++m) mean[m] = 0.f;
  if (p.norm == NORM_LN) {
#pragma unroll
    for (int m = 0; m < GEMV_MAX_ROWS; ++m)
      if (m < M)
        for (int k = tid; k < K; k += GD_WG) mean[m] += xs[m * K + k];
    block_sum_rows(mean, M, red[0]);
#pragma unroll
    for (int m = 0; m < GEMV_MAX_ROWS; ++m) mean[m] /= (float)K;
  }
#pragma unroll
  for (int m = 0; m < GEMV_MAX_ROWS; ++m) {
    var[m] = 0.f;
    if (m < M)
      for (int k = tid; k < K; k += GD_WG) {
        const float t = xs[m * K + k] - mean[m];
        var[m] = fmaf(t, t, var[m]);
      }
  }
  block_sum_rows(var, M, red[1]);
  float rs[GEMV_MAX_ROWS];
#pragma unroll
  for (int m = 0; m < GEMV_MAX_ROWS; ++m) rs[m] = 1.0f / sqrtf(var[m] / (float)K + p.eps);
#pragma unroll
  for (int m = 0; m < GEMV_MAX_ROWS; ++m)
    if (m < M)
      for (int k = tid; k < K; k += GD_WG) {
        const float v = xs[m * K + k];
        xs[m * K + k] = p.norm == NORM_RMS ? v * rs[m] * s_g[k] : (v - mean[m]) * rs[m] * s_g[k] + s_b[k];
      }
}

template <int WT>
struct WChunk;
template <>
struct WChunk<0> { typedef f32x4 T; static constexpr int CE = 4; };
template <>
struct WChunk<1> { typedef u32x4 T; static constexpr int CE = 8; };

// ------------------------------------------------------------------ GEMV

template <int WT, int NC, int RW, int EPI>
__global__ __launch_bounds__(GD_WG) void k_gemv(LinParams p) {
  typedef typename WChunk<WT>::T VT;
  constexpr int CE = WChunk<WT>::CE;
  extern __shared__ __align__(16) float xs[];   // [M][K] rows, then the norm's gain and shift [2][K]
  float* s_gb = xs + ((p.M * p.K + 3) & ~3);
  __shared__ float s_am[GEMV_MAX_ROWS][4 * RW];
  __shared__ float s_red[2][GD_WG / 64][GEMV_MAX_ROWS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int M = p.M, N = p.N, K = p.K;
  const int nw0 = (blockIdx.x * 4 + wave) * RW;              // first row of this wave

  // 0. this thread's share of the activation rows (M = 1 rows fit entirely)
  constexpr int XPT = (NC * CE + 15) / 16;
  RowRegs<XPT> rr;
  stage_issue<XPT>(p, rr);
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
          reinterpret_cast<const char*>(p.w) + ((size_t)min(n, N - 1) * K + k) * (WT == 0 ? 4 : 2)));
    }
  }
  // 2. epilogue operands of this lane's output (lane m * RW + r), or pair (lane m)
  constexpr bool PAIR = EpiTraits<EPI>::pair;
  static_assert(!PAIR || RW == 2, "pair epilogues need both rows of the pair in one wave");
  const int om = PAIR ? lane : lane / RW, orr = PAIR ? 0 : lane % RW;
  const int on = nw0 + orr;
  const bool own = EPI != EPI_ARGMAX && om < M && (PAIR ? nw0 + 1 < N : (lane < M * RW && on < N));
  EpiOps eo = epi_prefetch<EPI>(p, own ? om : 0, own ? on : 0);
  // 3. activations into LDS, normalized
  stage_finish<XPT>(p, xs, s_gb, rr, s_red);
  __syncthreads();
  // 4. dot products
  float acc[RW][GEMV_MAX_ROWS];
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int m = 0; m < GEMV_MAX_ROWS; ++m) acc[r][m] = 0.f;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int k = (lane + 64 * i) * CE;
    if (k < K) {
#pragma unroll
      for (int m = 0; m < GEMV_MAX_ROWS; ++m) {
        if (m < M) {
          const float* xr = xs + m * K + k;
          f32x4 a = *reinterpret_cast<const f32x4*>(xr);
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
          if (WT == 1) {
            f32x4 b = *reinterpret_cast<const f32x4*>(xr + 4);
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
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int m = 0; m < GEMV_MAX_ROWS; ++m)
      if (m < M) acc[r][m] = wave_sum(acc[r][m]);
  // 5. epilogue
  if (EPI == EPI_ARGMAX) {
    if (lane == 0) {
#pragma unroll
      for (int m = 0; m < GEMV_MAX_ROWS; ++m)
#pragma unroll
        for (int r = 0; r < RW; ++r)
          if (m < M) s_am[m][wave * RW + r] = acc[r][m];
    }
    if (p.logits && lane < M * RW) {
#pragma unroll
      for (int m = 0; m < GEMV_MAX_ROWS; ++m)
#pragma unroll
        for (int r = 0; r < RW; ++r)
          if (lane == m * RW + r && nw0 + r < N) p.logits[(size_t)m * p.ldl + nw0 + r] = acc[r][m];
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
  if (!own) return;
  float v0 = 0.f, v1 = 0.f;
#pragma unroll
  for (int m = 0; m < GEMV_MAX_ROWS; ++m)
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      if (m == om && r == orr) v0 = acc[r][m];
      if (m == om && r == orr + 1) v1 = acc[r][m];
    }
  epi_store<EPI>(p, eo, om, on, v0, v1);
}

// ------------------------------------------------------------------- MFMA

typedef float TileT[GD_MAX_ROWS][GD_TILE_N + 1];

template <int EPI>
__device__ void mfma_epi(const LinParams& p, TileT& tileT, int n0, int nthr) {
  const int tid = threadIdx.x;
  if (EpiTraits<EPI>::pair) {
    for (int i = tid; i < p.M * (GD_TILE_N / 2); i += nthr) {
      const int m = i >> 3, c = (i & 7) * 2;
      if (n0 + c + 1 < p.N) {
        const EpiOps e = epi_prefetch<EPI>(p, m, n0 + c);
        epi_store<EPI>(p, e, m, n0 + c, tileT[m][c], tileT[m][c + 1]);
      }
    }
  } else {
    for (int i = tid; i < p.M * GD_TILE_N; i += nthr) {
      const int m = i >> 4, c = i & 15;
      if (n0 + c < p.N) {
        const EpiOps e = epi_prefetch<EPI>(p, m, n0 + c);
        epi_store<EPI>(p, e, m, n0 + c, tileT[m][c], 0.f);
      }
    }
  }
}

__device__ void mfma_argmax(const LinParams& p, TileT& tileT, int n0, int nthr) {
  const int tid = threadIdx.x;
  if (p.logits)
    for (int i = tid; i < p.M * GD_TILE_N; i += nthr) {
      const int m = i >> 4, c = i & 15;
      if (n0 + c < p.N) p.logits[(size_t)m * p.ldl + n0 + c] = tileT[m][c];
    }
  if (tid < p.M) {
    float bv = tileT[tid][0];
    int bi = n0;
    for (int c = 1; c < GD_TILE_N && n0 + c < p.N; ++c)
      if (am_better(tileT[tid][c], n0 + c, bv, bi)) { bv = tileT[tid][c]; bi = n0 + c; }
    p.am_val[(size_t)blockIdx.x * p.M + tid] = bv;
    p.am_idx[(size_t)blockIdx.x * p.M + tid] = bi;
  }
}

template <int WT, int MT, int NW>
__global__ __launch_bounds__(64 * NW) void k_mfma(LinParams p) {
  __shared__ float s_stat[GD_MAX_ROWS * 2];
  __shared__ float red[NW][GD_MAX_ROWS][GD_TILE_N + 1];
  __shared__ TileT tileT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int M = p.M, N = p.N, K = p.K;
  const int n0 = blockIdx.x * GD_TILE_N;
  const int n = n0 + (lane & 15);
  const int q = lane >> 4;
  const bool norm = p.norm != NORM_NONE;

  if (norm) {
    for (int m = wave; m < M; m += NW) {
      const float* xr = p.x + (size_t)m * p.ldx;
      float mean = 0.f;
      if (p.norm == NORM_LN) {
        float s = 0.f;
        for (int k = lane; k < K; k += 64) s += xr[k];
        mean = wave_sum(s) / (float)K;
      }
      float v = 0.f;
      for (int k = lane; k < K; k += 64) { float t = xr[k] - mean; v = fmaf(t, t, v); }
      const float var = wave_sum(v) / (float)K;
      if (lane == 0) { s_stat[2 * m] = mean; s_stat[2 * m + 1] = 1.0f / sqrtf(var + p.eps); }
    }
    __syncthreads();
  }
  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const int nb = (K + 31) >> 5;
  for (int b = wave; b < nb; b += NW) {
    const int kk = b * 32 + q * 8;
    float w[8];
    if (n < N && kk < K) load_w8<WT>(p.w, (size_t)n * K, kk, w);
    else {
#pragma unroll
      for (int i = 0; i < 8; ++i) w[i] = 0.f;
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mt * 16 + (lane & 15);
      float xv[8];
      if (m < M && kk < K) {
        const float* xr = p.x + (size_t)m * p.ldx + kk;
        f32x4 a = *reinterpret_cast<const f32x4*>(xr), c = *reinterpret_cast<const f32x4*>(xr + 4);
        xv[0] = a.x; xv[1] = a.y; xv[2] = a.z; xv[3] = a.w; xv[4] = c.x; xv[5] = c.y; xv[6] = c.z; xv[7] = c.w;
        if (norm) {
          const float mu = s_stat[2 * m], r = s_stat[2 * m + 1];
#pragma unroll
          for (int i = 0; i < 8; ++i)
            xv[i] = p.norm == NORM_RMS ? xv[i] * r * p.ng[kk + i] : (xv[i] - mu) * r * p.ng[kk + i] + p.nb[kk + i];
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) xv[i] = 0.f;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[i], w[i], acc[mt], 0, 0, 0);
    }
  }
  // D[i][j]: lane holds column j = lane % 16, rows i = 4q + v
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    red[wave][mt * 16 + 4 * q + 0][lane & 15] = acc[mt].x;
    red[wave][mt * 16 + 4 * q + 1][lane & 15] = acc[mt].y;
    red[wave][mt * 16 + 4 * q + 2][lane & 15] = acc[mt].z;
    red[wave][mt * 16 + 4 * q + 3][lane & 15] = acc[mt].w;
  }
  __syncthreads();
  for (int i = tid; i < M * GD_TILE_N; i += 64 * NW) {
    const int m = i >> 4, c = i & 15;
    float s = red[0][m][c];
#pragma unroll
    for (int w2 = 1; w2 < NW; ++w2) s += red[w2][m][c];
    tileT[m][c] = s;
  }
  __syncthreads();
  switch (p.epi) {
    case EPI_ARGMAX: mfma_argmax(p, tileT, n0, 64 * NW); break;
    case EPI_PLAIN: mfma_epi<EPI_PLAIN>(p, tileT, n0, 64 * NW); break;
    case EPI_GELU: mfma_epi<EPI_GELU>(p, tileT, n0, 64 * NW); break;
    case EPI_SWIGLU: mfma_epi<EPI_SWIGLU>(p, tileT, n0, 64 * NW); break;
    case EPI_QKV: mfma_epi<EPI_QKV>(p, tileT, n0, 64 * NW); break;
    default: mfma_epi<EPI_QKV_ROPE>(p, tileT, n0, 64 * NW); break;
  }
}

// Greedy argmax over the per-workgroup partials of one row (one workgroup per row).
// Every thread loads all of its partials before comparing, so the reduction costs
// one memory round trip. nparts <= GD_WG * AM_FIN_PER.
#define AM_FIN_PER 16
__global__ __launch_bounds__(GD_WG) void k_argmax_finalize(const float* __restrict__ val, const int* __restrict__ idx,
                                                           int nparts, int M, int* out) {
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
  }
}
