// prefill.h -- the prompt pass for many rows at once: a pre-norm kernel, a tiled
// matrix-core GEMM with the decode epilogues, and tiled causal attention.
//
// A prompt of P tokens runs the same layer as a decode step, but on P rows at a time
// ("rvllm Metal backend", "The matmul pain story": prefill is where the tiled GEMM
// pays; "Numbers": prompt processing speed and time to first token). The linear
// layers are real matrix products there (M = P rows), so they run as 64 x 64 output
// tiles on the fp32 matrix cores, every weight tile read once per 64 rows. Attention
// over the prompt is causal: query tile i of 64 rows attends to key tiles 0..i (and
// every cached position before the prompt), with the K/V tiles staged in LDS and
// shared by the 64 queries, and an online softmax per query row.
#pragma once
#include "common.h"
#include "linear.h"
#include "attention.h"

#define PF_BM 64
#define PF_BN 64
#define PF_BK 32
#define PF_LDS (PF_BK + 4)   // LDS row stride of the GEMM tiles (16-byte aligned rows)
#define PF_NT 256

// Pre-norm of M rows into y (explicit form): LayerNorm (biased variance, eps inside the
// root, gain and shift) or RMSNorm (gain). One workgroup per row, two passes over the
// row held in registers.
template <int NORM>
__global__ __launch_bounds__(PF_NT) void k_rownorm(const float* __restrict__ x, int ldx, const float* __restrict__ g,
                                                   const float* __restrict__ b, float eps, int K, float* __restrict__ y,
                                                   int ldy) {
  __shared__ float s_red[PF_NT / 64];
  const int row = blockIdx.x, tid = threadIdx.x;
  const float* xr = x + (size_t)row * ldx;
  constexpr int MAXV = 16;   // K <= PF_NT * MAXV
  float v[MAXV];
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < MAXV; ++j) {
    const int k = tid + PF_NT * j;
    v[j] = k < K ? xr[k] : 0.f;
    s += v[j];
  }
  auto block_sum = [&](float a) {
    a = wave_sum(a);
    if ((tid & 63) == 0) s_red[tid >> 6] = a;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < PF_NT / 64; ++w) t += s_red[w];
    __syncthreads();
    return t;
  };
  float mu = 0.f;
  if (NORM == NORM_LN) mu = block_sum(s) / (float)K;
  float q = 0.f;
#pragma unroll
  for (int j = 0; j < MAXV; ++j) {
    const int k = tid + PF_NT * j;
    const float d = k < K ? v[j] - mu : 0.f;
    q = fmaf(d, d, q);
  }
  const float r = rsqrtf(block_sum(q) / (float)K + eps);
#pragma unroll
  for (int j = 0; j < MAXV; ++j) {
    const int k = tid + PF_NT * j;
    if (k < K) y[(size_t)row * ldy + k] = NORM == NORM_LN ? fmaf((v[j] - mu) * r, g[k], b[k]) : v[j] * r * g[k];
  }
}

// C = epilogue(A . W^T) for M rows: A = p.x [M][ldx] (float), W = p.w [N][K] row-major
// (float or bf16 bits), K a multiple of 32. Workgroup (tile n, tile m) computes a
// 64 x 64 output tile; each of its four waves a 32 x 32 quarter as 2 x 2
// v_mfma_f32_16x16x4f32 tiles. Per 32-wide K step the A and W tiles are staged in LDS
// (bf16 widened there) while the next step's tiles are already being loaded.
// Operands: lane l = 16 q + c takes A[row c][k0 + q] and W[col c][k0 + q] of a 4-wide
// K slice; the accumulator holds D[rows 4q .. 4q + 3][col c].
template <int WT, int EPI>
__global__ __launch_bounds__(PF_NT) void k_gemm_pf(LinParams p) {
  __shared__ __align__(16) float sA[PF_BM * PF_LDS];
  __shared__ __align__(16) float sW[PF_BN * PF_LDS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, c = lane & 15;
  const int n0 = blockIdx.x * PF_BN, m0 = blockIdx.y * PF_BM;
  const int M = p.M, N = p.N, K = p.K;
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;
  // this thread's share of a tile: row lr, columns 8 lc .. 8 lc + 7
  const int lr = tid >> 2, lc = tid & 3;
  const int am = min(m0 + lr, M - 1), wr = min(n0 + lr, N - 1);
  const float* a_src = p.x + (size_t)am * p.ldx + 8 * lc;
  f32x4 ra[2], rw[2];
  auto load = [&](int k0) {
    ra[0] = *reinterpret_cast<const f32x4*>(a_src + k0);
    ra[1] = *reinterpret_cast<const f32x4*>(a_src + k0 + 4);
    if constexpr (WT == 0) {
      const float* w = reinterpret_cast<const float*>(p.w) + (size_t)wr * K + k0 + 8 * lc;
      rw[0] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(w));
      rw[1] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(w) + 1);
    } else {
      const uint16_t* w = reinterpret_cast<const uint16_t*>(p.w) + (size_t)wr * K + k0 + 8 * lc;
      const u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(w));
      rw[0] = (f32x4){bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y)};
      rw[1] = (f32x4){bf16_lo(u.z), bf16_hi(u.z), bf16_lo(u.w), bf16_hi(u.w)};
    }
  };
  auto store = [&]() {
    *reinterpret_cast<f32x4*>(sA + lr * PF_LDS + 8 * lc) = ra[0];
    *reinterpret_cast<f32x4*>(sA + lr * PF_LDS + 8 * lc + 4) = ra[1];
    *reinterpret_cast<f32x4*>(sW + lr * PF_LDS + 8 * lc) = rw[0];
    *reinterpret_cast<f32x4*>(sW + lr * PF_LDS + 8 * lc + 4) = rw[1];
  };
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const int nk = K / PF_BK;
  load(0);
  store();
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) load((kt + 1) * PF_BK);   // in flight during this step's MFMAs
#pragma unroll
    for (int s = 0; s < PF_BK / 4; ++s) {
      float a[2], w[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = sA[(wm + 16 * i + c) * PF_LDS + 4 * s + q];
#pragma unroll
      for (int j = 0; j < 2; ++j) w[j] = sW[(wn + 16 * j + c) * PF_LDS + 4 * s + q];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], w[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
    if (kt + 1 < nk) {
      store();
      __syncthreads();
    }
  }
  // epilogue: this lane holds rows m0 + wm + 16 i + 4 q + v of column n0 + wn + 16 j + c
  constexpr bool PAIR = EpiTraits<EPI>::pair;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn + 16 * j + c;
      const float vv[4] = {acc[i][j].x, acc[i][j].y, acc[i][j].z, acc[i][j].w};
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + wm + 16 * i + 4 * q + v;
        const float v0 = vv[v];
        const float v1 = __shfl_xor(v0, 1);   // the odd neighbour's column (pairs)
        const bool own = m < M && (PAIR ? ((c & 1) == 0 && n + 1 < N) : n < N);
        if (own) {
          const EpiOps eo = epi_prefetch<EPI, false>(p, m, n);
          epi_store<EPI>(p, eo, m, n, v0, v1);
        }
      }
    }
}

// Causal attention of M prompt rows (positions p0 .. p0 + M - 1 of one sequence)
// against the cache, which already holds their K/V. Workgroup (query tile t, query
// head h): 64 query rows; key tiles of 64 positions staged in LDS (float, widened from
// a bf16 cache), scores of a 4 x 4 block per thread, the online softmax per row over
// the 16 threads that share it, then P V for a 4-row x 4-dim block per thread.
// Positions after a row's own are masked (never weighted). Output o [M][ldo] at the
// head's columns, normalized.
struct PfAttnParams {
  const float* q; int ldq;                // [M][ldq] post-RoPE queries
  const void* kc; const void* vc;         // this layer's pools [nblk][Hkv][B][HD]
  const int* table;                       // the sequence's block table (paged), or NULL
  long long kv0;                          // contiguous: element offset of the sequence's slot
  int block_size, nblk, Hq, Hkv, M, p0;
  float scale;
  float* out; int ldo;
};

template <int HD, bool PAGED, bool KV16>
__global__ __launch_bounds__(PF_NT) void k_attn_prefill(PfAttnParams p) {
  static_assert(HD == 64, "head_dim 64");
  constexpr int BQ = 64, BKV = 64, LS = HD + 4;   // LDS row stride (16-byte aligned)
  __shared__ __align__(16) float sQ[BQ * LS];
  __shared__ __align__(16) float sK[BKV * LS];
  __shared__ __align__(16) float sV[BKV * LS];
  __shared__ __align__(16) float sP[BQ * (BKV + 4)];
  const int tid = threadIdx.x;
  const int qt = blockIdx.x, h = blockIdx.y, kh = h / (p.Hq / p.Hkv);
  const int r0 = qt * BQ;                  // first row of the tile
  const int ti = tid >> 4, tj = tid & 15;  // this thread: rows 4 ti .., keys (or dims) 4 tj ..
  // the query tile (rows past M read as the last row; never stored)
  for (int e = tid; e < BQ * (HD / 4); e += PF_NT) {
    const int r = e / (HD / 4), d4 = e % (HD / 4);
    const int row = min(r0 + r, p.M - 1);
    *reinterpret_cast<f32x4*>(sQ + r * LS + 4 * d4) =
        *reinterpret_cast<const f32x4*>(p.q + (size_t)row * p.ldq + h * HD + 4 * d4);
  }
  float mrow[4], lrow[4], o[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    mrow[a] = -INFINITY;
    lrow[a] = 0.f;
#pragma unroll
    for (int d = 0; d < 4; ++d) o[a][d] = 0.f;
  }
  const int last_pos = p.p0 + min(r0 + BQ, p.M) - 1;   // the tile's last query position
  const int ntiles = last_pos / BKV + 1;
  for (int kt = 0; kt < ntiles; ++kt) {
    __syncthreads();   // the previous tile's K, V and P are no longer read
    for (int e = tid; e < BKV * (HD / 4); e += PF_NT) {
      const int r = e / (HD / 4), d4 = e % (HD / 4);
      const int pos = min(kt * BKV + r, last_pos);
      size_t off;
      if (PAGED) {
        const int bi = pos / p.block_size;
        int blk = p.table[bi];
        blk = (unsigned)blk < (unsigned)p.nblk ? blk : 0;
        off = (((size_t)blk * p.Hkv + kh) * p.block_size + (pos - bi * p.block_size)) * HD + 4 * d4;
      } else {
        off = (size_t)p.kv0 + ((size_t)kh * p.block_size + pos) * HD + 4 * d4;
      }
      *reinterpret_cast<f32x4*>(sK + r * LS + 4 * d4) = kv_load4<KV16, false>(p.kc, off);
      *reinterpret_cast<f32x4*>(sV + r * LS + 4 * d4) = kv_load4<KV16, false>(p.vc, off);
    }
    __syncthreads();
    // scores of rows 4 ti + a against keys 4 tj + b
    float s[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) s[a][b] = 0.f;
#pragma unroll 4
    for (int d = 0; d < HD; d += 4) {
      f32x4 qa[4], kb[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) qa[a] = *reinterpret_cast<const f32x4*>(sQ + (4 * ti + a) * LS + d);
#pragma unroll
      for (int b = 0; b < 4; ++b) kb[b] = *reinterpret_cast<const f32x4*>(sK + (4 * tj + b) * LS + d);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          float t = s[a][b];
          t = fmaf(qa[a].x, kb[b].x, t);
          t = fmaf(qa[a].y, kb[b].y, t);
          t = fmaf(qa[a].z, kb[b].z, t);
          t = fmaf(qa[a].w, kb[b].w, t);
          s[a][b] = t;
        }
    }
    // online softmax per row: its 64 keys sit on the 16 threads tj of row group ti
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int qpos = p.p0 + r0 + 4 * ti + a;
      float mx = -INFINITY;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int kpos = kt * BKV + 4 * tj + b;
        s[a][b] = kpos <= qpos ? s[a][b] * p.scale : -INFINITY;
        mx = fmaxf(mx, s[a][b]);
      }
      mx = group_max<16>(mx);
      const float nm = fmaxf(mrow[a], mx);   // finite: key 0 is always visible
      const float sc = attn_rescale(mrow[a], nm);
      float ls = 0.f;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float e = s[a][b] == -INFINITY ? 0.f : expf(s[a][b] - nm);
        sP[(4 * ti + a) * (BKV + 4) + 4 * tj + b] = e;
        ls += e;
      }
      lrow[a] = lrow[a] * sc + group_sum<16>(ls);
      mrow[a] = nm;
#pragma unroll
      for (int d = 0; d < 4; ++d) o[a][d] *= sc;
    }
    __syncthreads();
    // o[rows 4 ti + a][dims 4 tj + d] += P . V
#pragma unroll 4
    for (int j = 0; j < BKV; ++j) {
      const f32x4 vv = *reinterpret_cast<const f32x4*>(sV + j * LS + 4 * tj);
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const float pa = sP[(4 * ti + a) * (BKV + 4) + j];
        o[a][0] = fmaf(pa, vv.x, o[a][0]);
        o[a][1] = fmaf(pa, vv.y, o[a][1]);
        o[a][2] = fmaf(pa, vv.z, o[a][2]);
        o[a][3] = fmaf(pa, vv.w, o[a][3]);
      }
    }
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int row = r0 + 4 * ti + a;
    if (row < p.M) {
      const float inv = 1.0f / lrow[a];
      *reinterpret_cast<f32x4*>(p.out + (size_t)row * p.ldo + h * HD + 4 * tj) =
          (f32x4){o[a][0] * inv, o[a][1] * inv, o[a][2] * inv, o[a][3] * inv};
    }
  }
}
