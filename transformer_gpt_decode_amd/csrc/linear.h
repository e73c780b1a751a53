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

// Source of the activation rows.
#define PRO_COPY 0   // x rows as given
#define PRO_ATTN 3   // merge of split-context attention partials
#define PRO_EMBED 4  // token embedding (+ learned position) rows; block 0 also stores them to xres
// Row normalization applied after the source (LinParams::norm).
#define NORM_NONE 0
#define NORM_LN 1    // (x - mean) / sqrt(var + eps) * g + b, biased variance
#define NORM_RMS 2   // x / sqrt(mean(x^2) + eps) * g

#define EPI_PLAIN 0
#define EPI_GELU 1
#define EPI_SWIGLU 2
#define EPI_ARGMAX 3
#define EPI_QKV 4

#define GEMV_MAX_ROWS 4

struct LinParams {
  // ---- input rows
  int pro, norm;
  const float* x; int ldx;                  // COPY (and MFMA input)
  const float* ng; const float* nb; float eps;
  const float* apart; int Hq, nchunk, chunk; // ATTN: partials [M][Hq][nchunk][hd + 2]
  const void* wte; const void* wpe; int vocab, n_pos, emb_bf16;  // EMBED
  const int* row_tok; float* xres; int* err;
  const int* row_seq; const int* row_pos;
  // ---- weights
  const void* w; int M, N, K;
  // ---- epilogue
  int epi;
  const float* bias;
  const float* resid; int ldr;
  float* y; int ldy;
  float* am_val; int* am_idx;               // [gridDim.x][M]
  float* logits; int ldl;
  int qdim, kdim, hd;                       // QKV
  const float* rope_cs;                     // [n_pos][hd]: cos | sin of pair i (NULL: no RoPE)
  float* kc; float* vc; const int* table; int max_blocks, block_size, nblk;
};

// ------------------------------------------------------------ shared pieces

// Per-element epilogue for EPI_PLAIN / EPI_GELU.
__device__ __forceinline__ void epi_one(const LinParams& p, int m, int n, float v) {
  if (p.bias) v += p.bias[n];
  if (p.epi == EPI_GELU) v = gelu_clamped(v);
  if (p.resid) v = p.resid[(size_t)m * p.ldr + n] + v;
  p.y[(size_t)m * p.ldy + n] = v;
}

// QKV scatter of one output column (bias added). For the RoPE layout the caller passes
// the rotated value. q columns go to y; k and v columns into the cache.
__device__ __forceinline__ void qkv_store(const LinParams& p, int m, int n, float v) {
  if (n < p.qdim) {
    p.y[(size_t)m * p.ldy + n] = v;
    return;
  }
  const int pos = p.row_pos[m];
  if (pos < 0) return;
  const int bi = pos / p.block_size;
  const int blk = bi < p.max_blocks ? p.table[(size_t)p.row_seq[m] * p.max_blocks + bi] : -1;
  if ((unsigned)blk >= (unsigned)p.nblk) {
    atomicOr(p.err, GD_DERR_BLOCK);
    return;
  }
  const int slot = pos - bi * p.block_size;
  const int Hkv = p.kdim / p.hd;
  int kn = n - p.qdim;
  float* dst = p.kc;
  if (kn >= p.kdim) { kn -= p.kdim; dst = p.vc; }
  const int g = kn / p.hd, d = kn - g * p.hd;
  dst[(((size_t)blk * Hkv + g) * p.block_size + slot) * p.hd + d] = v;
}

// Epilogue of an adjacent column pair (n even): SwiGLU, or QKV (RoPE on q/k pairs).
__device__ __forceinline__ void epi_pair(const LinParams& p, int m, int n, float v0, float v1) {
  if (p.epi == EPI_SWIGLU) {
    p.y[(size_t)m * p.ldy + (n >> 1)] = silu(v0) * v1;
    return;
  }
  if (p.bias) { v0 += p.bias[n]; v1 += p.bias[n + 1]; }
  if (p.rope_cs && n < p.qdim + p.kdim) {
    const int pos = max(p.row_pos[m], 0);
    const int half = p.hd >> 1;
    const int i = (n % p.hd) >> 1;
    const float* cs = p.rope_cs + (size_t)min(pos, p.n_pos - 1) * p.hd;
    const float c = cs[i], s = cs[half + i];
    const float a = v0, b = v1;
    v0 = a * c - b * s;
    v1 = a * s + b * c;
  }
  qkv_store(p, m, n, v0);
  qkv_store(p, m, n + 1, v1);
}

__device__ __forceinline__ bool epi_is_pair(const LinParams& p) {
  return p.epi == EPI_SWIGLU || (p.epi == EPI_QKV && p.rope_cs);
}

// Stage M activation rows (K columns) into LDS xs[m * K + k].
__device__ void stage_rows(const LinParams& p, float* xs, float* s_stat) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int M = p.M, K = p.K;
  if (p.pro == PRO_ATTN) {
    // merge split-context partials: o = sum_c e^(m_c - max) o_c / sum_c e^(m_c - max) l_c
    const int hd = p.hd;
    const int nh = K / hd;
    float* wgt = s_stat;  // [M][nh][nchunk]
    for (int i = tid; i < M * nh; i += GD_WG) {
      const int m = i / nh, h = i - m * nh;
      const int nch = (p.row_pos[m] + p.chunk) / p.chunk;
      const float* pp = p.apart + ((size_t)m * p.Hq + h) * p.nchunk * (hd + 2);
      float mx = -INFINITY;
      for (int c = 0; c < nch; ++c) mx = fmaxf(mx, pp[(size_t)c * (hd + 2)]);
      float l = 0.f;
      for (int c = 0; c < nch; ++c) l = fmaf(pp[(size_t)c * (hd + 2) + 1], expf(pp[(size_t)c * (hd + 2)] - mx), l);
      const float inv = 1.0f / l;
      for (int c = 0; c < p.nchunk; ++c)
        wgt[(size_t)i * p.nchunk + c] = c < nch ? expf(pp[(size_t)c * (hd + 2)] - mx) * inv : 0.f;
    }
    __syncthreads();
    for (int i = tid; i < M * K; i += GD_WG) {
      const int m = i / K, k = i - m * K;
      const int h = k / hd, d = k - h * hd;
      const int nch = (p.row_pos[m] + p.chunk) / p.chunk;
      const float* pp = p.apart + ((size_t)m * p.Hq + h) * p.nchunk * (hd + 2) + 2 + d;
      const float* wg = wgt + ((size_t)m * nh + h) * p.nchunk;
      float o = 0.f;
      for (int c = 0; c < nch; ++c) o = fmaf(pp[(size_t)c * (hd + 2)], wg[c], o);
      xs[i] = o;
    }
    return;
  }
  if (p.pro == PRO_EMBED) {
    for (int i = tid; i < M * K; i += GD_WG) {
      const int m = i / K, k = i - m * K;
      int t = p.row_tok[m];
      if (t < 0 || t >= p.vocab) { if (k == 0) atomicOr(p.err, GD_DERR_TOKEN); t = 0; }
      int pos = p.row_pos[m];
      if (p.wpe && (pos < 0 || pos >= p.n_pos)) { if (k == 0) atomicOr(p.err, GD_DERR_POS); pos = 0; }
      float v;
      if (!p.emb_bf16) v = reinterpret_cast<const float*>(p.wte)[(size_t)t * K + k];
      else v = bf16_lo(reinterpret_cast<const uint16_t*>(p.wte)[(size_t)t * K + k]);
      if (p.wpe) {
        if (!p.emb_bf16) v += reinterpret_cast<const float*>(p.wpe)[(size_t)pos * K + k];
        else v += bf16_lo(reinterpret_cast<const uint16_t*>(p.wpe)[(size_t)pos * K + k]);
      }
      xs[i] = v;
      if (blockIdx.x == 0) p.xres[(size_t)m * K + k] = v;   // residual stream for the layer
    }
  } else {
    const int K4 = K >> 2;
    for (int i = tid; i < M * K4; i += GD_WG) {
      const int m = i / K4, k = (i - m * K4) << 2;
      *reinterpret_cast<f32x4*>(xs + m * K + k) = *reinterpret_cast<const f32x4*>(p.x + (size_t)m * p.ldx + k);
    }
  }
  if (p.norm == NORM_NONE) return;
  __syncthreads();
  // row statistics (two passes over LDS), one wave per row
  for (int m = wave; m < M; m += GD_WG / 64) {
    const float* xr = xs + m * K;
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
  for (int i = tid; i < M * K; i += GD_WG) {
    const int m = i / K, k = i - m * K;
    const float mu = s_stat[2 * m], r = s_stat[2 * m + 1];
    xs[i] = p.norm == NORM_RMS ? xs[i] * r * p.ng[k] : (xs[i] - mu) * r * p.ng[k] + p.nb[k];
  }
}

template <int WT>
struct WChunk;
template <>
struct WChunk<0> { typedef f32x4 T; static constexpr int CE = 4; };
template <>
struct WChunk<1> { typedef u32x4 T; static constexpr int CE = 8; };

// ------------------------------------------------------------------ GEMV

template <int WT, int NC, int RW>
__global__ __launch_bounds__(GD_WG) void k_gemv(LinParams p) {
  typedef typename WChunk<WT>::T VT;
  constexpr int CE = WChunk<WT>::CE;
  extern __shared__ __align__(16) float xs[];   // [M][K], then norm stats or attention merge weights
  float* s_stat = xs + ((p.M * p.K + 3) & ~3);
  __shared__ float s_am[GEMV_MAX_ROWS][4 * RW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int M = p.M, N = p.N, K = p.K;
  const int nw0 = (blockIdx.x * 4 + wave) * RW;              // first row of this wave

  // 1. weights first: they do not depend on anything
  VT w[RW][NC];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int n = nw0 + r;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int k = (lane + 64 * i) * CE;
      if (n < N && k < K)
        w[r][i] = __builtin_nontemporal_load(reinterpret_cast<const VT*>(
            reinterpret_cast<const char*>(p.w) + ((size_t)n * K + k) * (WT == 0 ? 4 : 2)));
      else
        w[r][i] = (VT){0, 0, 0, 0};
    }
  }
  // 2. activations into LDS
  stage_rows(p, xs, s_stat);
  __syncthreads();
  // 3. dot products
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
  // 4. epilogue
  if (p.epi == EPI_ARGMAX) {
    if (lane == 0) {
#pragma unroll
      for (int m = 0; m < GEMV_MAX_ROWS; ++m)
#pragma unroll
        for (int r = 0; r < RW; ++r)
          if (m < M) s_am[m][wave * RW + r] = acc[r][m];
    }
    if (p.logits && lane < M * RW) {
      // lane -> (m, r)
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
  if (epi_is_pair(p)) {
    // RW == 2 and nw0 is even: the wave holds both columns of the pair
    if (lane < M && nw0 + 1 < N) {
#pragma unroll
      for (int m = 0; m < GEMV_MAX_ROWS; ++m)
        if (lane == m) epi_pair(p, m, nw0, acc[0][m], acc[RW - 1][m]);
    }
    return;
  }
  if (lane < M * RW) {
#pragma unroll
    for (int m = 0; m < GEMV_MAX_ROWS; ++m)
#pragma unroll
      for (int r = 0; r < RW; ++r)
        if (lane == m * RW + r && nw0 + r < N) {
          if (p.epi == EPI_QKV) {
            float v = acc[r][m] + (p.bias ? p.bias[nw0 + r] : 0.f);
            qkv_store(p, m, nw0 + r, v);
          } else {
            epi_one(p, m, nw0 + r, acc[r][m]);
          }
        }
  }
}

// ------------------------------------------------------------------- MFMA

template <int WT, int MT, int NW>
__global__ __launch_bounds__(64 * NW) void k_mfma(LinParams p) {
  __shared__ float s_stat[GD_MAX_ROWS * 2];
  __shared__ float red[NW][GD_MAX_ROWS][GD_TILE_N + 1];
  __shared__ float tileT[GD_MAX_ROWS][GD_TILE_N + 1];
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
  if (p.epi == EPI_ARGMAX) {
    if (p.logits)
      for (int i = tid; i < M * GD_TILE_N; i += 64 * NW) {
        const int m = i >> 4, c = i & 15;
        if (n0 + c < N) p.logits[(size_t)m * p.ldl + n0 + c] = tileT[m][c];
      }
    if (tid < M) {
      float bv = tileT[tid][0];
      int bi = n0;
      for (int c = 1; c < GD_TILE_N && n0 + c < N; ++c)
        if (am_better(tileT[tid][c], n0 + c, bv, bi)) { bv = tileT[tid][c]; bi = n0 + c; }
      p.am_val[(size_t)blockIdx.x * M + tid] = bv;
      p.am_idx[(size_t)blockIdx.x * M + tid] = bi;
    }
    return;
  }
  if (epi_is_pair(p)) {
    for (int i = tid; i < M * (GD_TILE_N / 2); i += 64 * NW) {
      const int m = i >> 3, c = (i & 7) * 2;
      if (n0 + c + 1 < N) epi_pair(p, m, n0 + c, tileT[m][c], tileT[m][c + 1]);
    }
    return;
  }
  for (int i = tid; i < M * GD_TILE_N; i += 64 * NW) {
    const int m = i >> 4, c = i & 15;
    if (n0 + c < N) {
      if (p.epi == EPI_QKV) qkv_store(p, m, n0 + c, tileT[m][c] + (p.bias ? p.bias[n0 + c] : 0.f));
      else epi_one(p, m, n0 + c, tileT[m][c]);
    }
  }
}

// Greedy argmax over the per-workgroup partials of one row (one workgroup per row).
__global__ __launch_bounds__(GD_WG) void k_argmax_finalize(const float* __restrict__ val, const int* __restrict__ idx,
                                                           int nparts, int M, int* out) {
  __shared__ float sv[GD_WG / 64];
  __shared__ int si[GD_WG / 64];
  const int m = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float bv = 0.f;
  int bi = 0x7fffffff;
  bool have = false;
  for (int j = tid; j < nparts; j += GD_WG) {
    const float v = val[(size_t)j * M + m];
    const int i = idx[(size_t)j * M + m];
    if (!have || am_better(v, i, bv, bi)) { bv = v; bi = i; have = true; }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    const int oh = __shfl_xor((int)have, o, 64);
    if (oh && (!have || am_better(ov, oi, bv, bi))) { bv = ov; bi = oi; have = true; }
  }
  if (lane == 0) { sv[wave] = bv; si[wave] = have ? bi : 0x7fffffff; }
  __syncthreads();
  if (tid == 0) {
    float v0 = sv[0];
    int i0 = si[0];
    for (int w = 1; w < GD_WG / 64; ++w)
      if (si[w] != 0x7fffffff && (i0 == 0x7fffffff || am_better(sv[w], si[w], v0, i0))) { v0 = sv[w]; i0 = si[w]; }
    out[m] = i0;
  }
}
