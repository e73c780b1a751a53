// prefill.h -- the prompt pass for many rows at once: a pre-norm kernel, a tiled
// matrix-core GEMM with the decode epilogues (and the pre-norm inside), and tiled
// causal attention with its merge.
//
// A prompt of P tokens runs the same layer as a decode step, but on P rows at a time
// ("rvllm Metal backend", "The matmul pain story": prefill is where the tiled GEMM
// pays; "Numbers": prompt processing speed and time to first token). The linear
// layers are real matrix products there (M = P rows), so they run as 64 x 64 output
// tiles on the matrix cores (fp32, or bf16 in exact parts for bf16 weights), every
// weight tile read once per 64 rows. Attention over the prompt is causal: query tile i
// of 64 rows attends to key tiles 0..i (and every cached position before the prompt),
// with the K/V tiles staged in LDS and shared by the 64 queries, and an online softmax
// per query row.
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
// (float or bf16 bits), K a multiple of 32. Workgroup (tile n, tile m, split z)
// computes a 64 x 64 output tile over the z-th of gridDim.z shares of the 32-wide K
// steps; each of its four waves a 32 x 32 quarter as 2 x 2 v_mfma_f32_16x16x4f32 tiles.
// Operands: lane l = 16 q + c takes A[row c][k] and W[col c][k] of the same k; the
// accumulator holds D[rows 4q .. 4q + 3][col c].
//
// A step's MFMAs take about 1000 clocks per wave, well under a memory round trip, so
// the tiles of the next PF_PD steps are in flight in registers while a step computes:
// step s stores its tiles into LDS buffer s % 2 (bf16 widened there), one barrier, the
// MFMAs read them, and the registers take the loads of step s + PD. The steps are
// grouped by PD so that every register index is fixed at compile time; a group's steps
// past K load a clamped step and store zeros (no branch around any load).
// Split K (gridDim.z > 1) is for narrow outputs (few tiles for the CUs) of the plain
// epilogue whose output is the residual, updated in place (p.y == p.resid): each split
// adds its partial sums to it with float atomics, the bias coming from split 0, so the
// summation order of the S partials is not fixed.
//
// SPLIT: the products run on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16, 16 times
// the fp32 rate) without losing fp32 accuracy. An fp32 value is the exact sum of three
// bf16 parts (each the nearest bf16 to what the previous parts left: 8 + 8 + 8
// significant bits), and a product of two bf16 values is exact in fp32, so
//   a w = sum over the part pairs (i, j) of a_i w_j.
// bf16 weights are one part already: three MFMAs per product. fp32 weights are split as
// well and the six pairs with i + j <= 2 (parts numbered from 0) are kept; the three
// dropped terms are below 2^-24 of the product, the size of an fp32 rounding. The parts
// are formed once per workgroup when a tile is stored into LDS (one LDS plane each), and
// the sums accumulate in fp32 as before. Lane l = 16 q + c then holds eight consecutive
// k values of row c of each operand.
#define PF_PD 4   // K steps in flight
#define PF_LDB 40 // LDS row stride of the bf16 part planes (elements; 16-byte aligned rows)
template <int WT, bool SPLIT>
struct PfLds;
template <int WT>
struct PfLds<WT, false> {
  float a[2][PF_BM * PF_LDS];
  float w[2][PF_BN * PF_LDS];
};
template <int WT>
struct PfLds<WT, true> {
  uint16_t a[2][3][PF_BM * PF_LDB];                   // [buffer][part][row][k]
  uint16_t w[2][WT == 0 ? 3 : 1][PF_BN * PF_LDB];
};

// NRM: the pre-norm of the rows, applied inside the GEMM (QKV and MLP up, never split
// in K, so each workgroup sees whole rows over its K loop):
//  PFN_RMS:  RMSNorm: each staged value is multiplied by its column's gain (p.ng), the
//            row's sum of squares accumulates as the tiles pass, and the epilogue scales
//            by r = 1 / sqrt(mean(x^2) + eps);
//  PFN_FOLD: LayerNorm folded into fp32 weights (p.w = g W, p.fs its row sums, p.bias the
//            folded bias): the rows are staged shifted by their first element,
//            d = x - x_0, whose moments accumulate; the epilogue forms
//            r (acc - mean(d) s_n), as the decode kernels do.
#define PFN_NONE 0
#define PFN_RMS 1
#define PFN_FOLD 2

template <int WT, int EPI, bool SPLIT, int NRM = PFN_NONE>
__global__ __launch_bounds__(PF_NT) void k_gemm_pf(LinParams p) {
  static_assert(NRM != PFN_FOLD || WT == 0, "folded weights are fp32");
  __shared__ __align__(16) PfLds<WT, SPLIT> sm;
  __shared__ float s_r[PF_BM], s_mu[PF_BM];   // NRM: each tile row's r and mean(d)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, c = lane & 15;
  // Workgroups are placed round-robin over the 8 XCDs (each with its own L2) in launch
  // order; the launch index is renumbered so that an XCD gets a run of consecutive
  // logical tiles, ordered row tile fastest, then column tile, then K split: the tiles
  // of one XCD then share their W columns and K range, and each slice of A and W comes
  // from HBM about once instead of once per XCD. L = 8 k + x (x < 8) becomes x per + k
  // for the first 8 per indices (per = total / 8); the remainder keeps its index.
  const int GX = gridDim.x, GY = gridDim.y;
  const int lid = [&] {
    const int total = GX * GY * gridDim.z, L = blockIdx.x + GX * (blockIdx.y + GY * blockIdx.z), per = total >> 3;
    return L < 8 * per ? (L & 7) * per + (L >> 3) : L;
  }();
  const int ty = lid % GY, tx = (lid / GY) % GX;
  const int n0 = tx * PF_BN, m0 = ty * PF_BM;
  const int M = p.M, N = p.N, K = p.K;
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;
  // Tile loads shaped for the memory pipeline: each wave instruction reads whole tile
  // rows, eight 128-byte lines for fp32 (lane l: row 8 u + l / 8 of the wave's 16,
  // float4 l % 8) or sixteen 64-byte rows of bf16 W (row l / 4, eight values l % 4);
  // spread over 16 rows at 32 bytes each, the same bytes reach a CU far more slowly.
  const int ar = 16 * wave + (lane >> 3), ac = 4 * (lane & 7);   // fp32 unit u: row ar + 8 u
  const int br = 16 * wave + (lane >> 2), bc = 8 * (lane & 3);   // bf16 W unit
  const float* a_src[2];
  const void* w_src[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    a_src[u] = p.x + (size_t)min(m0 + ar + 8 * u, M - 1) * p.ldx + ac;
    if constexpr (WT == 0)
      w_src[u] = reinterpret_cast<const float*>(p.w) + (size_t)min(n0 + ar + 8 * u, N - 1) * K + ac;
    else
      w_src[u] = reinterpret_cast<const uint16_t*>(p.w) + (size_t)min(n0 + br, N - 1) * K + bc;
  }
  f32x4 ra[PF_PD][2], rw[PF_PD][2];   // fp32 tiles in flight (SPLIT bf16 W: raw bits in rb)
  u32x4 rb[PF_PD];
  f32x4 gv[PF_PD];                    // PFN_RMS: the gains of this thread's 4 columns
  float x0[2] = {0.f, 0.f};           // PFN_FOLD: each unit row's first element
  float st1[2] = {0.f, 0.f}, st2[2] = {0.f, 0.f};   // the unit rows' running sum and sum of squares
  if constexpr (NRM == PFN_FOLD) {
#pragma unroll
    for (int u = 0; u < 2; ++u) x0[u] = *(a_src[u] - ac);
  }
  const int nk = K / PF_BK, S = gridDim.z, z = lid / (GX * GY);
  // this split's groups of PD steps (the last group of the last split may reach past K)
  const int ng = (nk + PF_PD - 1) / PF_PD;
  const int g0 = z * ng / S, g1 = (z + 1) * ng / S;   // g0 < g1: S <= ng
  auto load = [&](int i, int st) {   // step st (clamped to the last one) into slot i
    const int k0 = min(st, nk - 1) * PF_BK;
#pragma unroll
    for (int u = 0; u < 2; ++u) ra[i][u] = *reinterpret_cast<const f32x4*>(a_src[u] + k0);
    if constexpr (NRM == PFN_RMS) gv[i] = *reinterpret_cast<const f32x4*>(p.ng + k0 + ac);
    if constexpr (WT == 0) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
        rw[i][u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(w_src[u]) + k0));
    } else {
      const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(w_src[0]) + k0));
      if constexpr (SPLIT) {
        rb[i] = v;
      } else {
        rw[i][0] = (f32x4){bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y)};
        rw[i][1] = (f32x4){bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
      }
    }
  };
  auto store = [&](int i, bool valid) {   // slot i into LDS buffer i % 2 (zeros past K)
    const int b = i & 1;
    if constexpr (NRM != PFN_NONE) {
      // the pre-norm's share of this step: statistics of the real columns, then the
      // values the MFMAs see (x g for RMSNorm, x - x_0 for the folded LayerNorm)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        f32x4& a = ra[i][u];
        if constexpr (NRM == PFN_FOLD) { a.x -= x0[u]; a.y -= x0[u]; a.z -= x0[u]; a.w -= x0[u]; }
        const float s1 = (a.x + a.y) + (a.z + a.w);
        const float s2 = fmaf(a.x, a.x, a.y * a.y) + fmaf(a.z, a.z, a.w * a.w);
        st1[u] += valid ? s1 : 0.f;
        st2[u] += valid ? s2 : 0.f;
        if constexpr (NRM == PFN_RMS) { a.x *= gv[i].x; a.y *= gv[i].y; a.z *= gv[i].z; a.w *= gv[i].w; }
      }
    }
    if constexpr (SPLIT) {
      const uint2 z2 = make_uint2(0u, 0u);
      auto put3 = [&](uint16_t (*planes)[PF_BM * PF_LDB], int row, const f32x4& v) {
        uint2 h, m, l;
        split3(v, h, m, l);
        *reinterpret_cast<uint2*>(planes[0] + row * PF_LDB + ac) = valid ? h : z2;
        *reinterpret_cast<uint2*>(planes[1] + row * PF_LDB + ac) = valid ? m : z2;
        *reinterpret_cast<uint2*>(planes[2] + row * PF_LDB + ac) = valid ? l : z2;
      };
#pragma unroll
      for (int u = 0; u < 2; ++u) put3(sm.a[b], ar + 8 * u, ra[i][u]);
      if constexpr (WT == 0) {
#pragma unroll
        for (int u = 0; u < 2; ++u) put3(sm.w[b], ar + 8 * u, rw[i][u]);
      } else {
        const u32x4 z4 = {0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(sm.w[b][0] + br * PF_LDB + bc) = valid ? rb[i] : z4;
      }
    } else {
      const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < 2; ++u)
        *reinterpret_cast<f32x4*>(sm.a[b] + (ar + 8 * u) * PF_LDS + ac) = valid ? ra[i][u] : z4;
      if constexpr (WT == 0) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
          *reinterpret_cast<f32x4*>(sm.w[b] + (ar + 8 * u) * PF_LDS + ac) = valid ? rw[i][u] : z4;
      } else {
        float* w = sm.w[b] + br * PF_LDS + bc;
        *reinterpret_cast<f32x4*>(w) = valid ? rw[i][0] : z4;
        *reinterpret_cast<f32x4*>(w + 4) = valid ? rw[i][1] : z4;
      }
    }
  };
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
  // A step's 32 K columns: MFMA t (0..7) contracts k = 8 q + t, so each lane reads its
  // eight operand values of a row with two 16-byte LDS loads, all before the MFMAs
  auto mfma = [&](int b) {
    if constexpr (SPLIT) {
      constexpr int NW = WT == 0 ? 3 : 1;
      u32x4 a[3][2], w[NW][2];
#pragma unroll
      for (int pa = 0; pa < 3; ++pa)
#pragma unroll
        for (int i = 0; i < 2; ++i)
          a[pa][i] = *reinterpret_cast<const u32x4*>(sm.a[b][pa] + (wm + 16 * i + c) * PF_LDB + 8 * q);
#pragma unroll
      for (int pw = 0; pw < NW; ++pw)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          w[pw][j] = *reinterpret_cast<const u32x4*>(sm.w[b][pw] + (wn + 16 * j + c) * PF_LDB + 8 * q);
      // the part pairs (pa, pw) with pa + pw <= 2, smallest terms first
#pragma unroll
      for (int s = 2; s >= 0; --s)
#pragma unroll
        for (int pa = 0; pa <= s; ++pa) {
          const int pw = s - pa;
          if (pw >= NW) continue;
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[pa][i]),
                                                                 __builtin_bit_cast(bf16x8_t, w[pw][j]), acc[i][j], 0, 0, 0);
        }
    } else {
      F8 a[2], w[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float* src = sm.a[b] + (wm + 16 * i + c) * PF_LDS + 8 * q;
        a[i].a = *reinterpret_cast<const f32x4*>(src);
        a[i].b = *reinterpret_cast<const f32x4*>(src + 4);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float* src = sm.w[b] + (wn + 16 * j + c) * PF_LDS + 8 * q;
        w[j].a = *reinterpret_cast<const f32x4*>(src);
        w[j].b = *reinterpret_cast<const f32x4*>(src + 4);
      }
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(f8_at(a[i], t), f8_at(w[j], t), acc[i][j], 0, 0, 0);
    }
  };
#pragma unroll
  for (int i = 0; i < PF_PD; ++i) load(i, g0 * PF_PD + i);
  // every group but the last issues the loads of the group after it
  for (int g = g0; g < g1 - 1; ++g) {
#pragma unroll
    for (int i = 0; i < PF_PD; ++i) {
      const int st = g * PF_PD + i;
      store(i, true);
      __syncthreads();   // buffer i % 2 written; its previous readers (step st - 2) are done
      load(i, st + PF_PD);
      mfma(i & 1);
    }
  }
#pragma unroll
  for (int i = 0; i < PF_PD; ++i) {
    store(i, (g1 - 1) * PF_PD + i < nk);
    __syncthreads();
    mfma(i & 1);
  }
  if constexpr (NRM != PFN_NONE) {
    // each row's statistics: the 8 lanes that staged it, then LDS for the epilogue
    const float invK = 1.0f / (float)K;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float s1 = group_sum<8>(st1[u]), s2 = group_sum<8>(st2[u]);
      const float mu = NRM == PFN_FOLD ? s1 * invK : 0.f;
      if ((lane & 7) == 0) {
        s_r[ar + 8 * u] = rsqrtf(fmaxf(s2 * invK - mu * mu, 0.f) + p.eps);
        s_mu[ar + 8 * u] = mu;
      }
    }
    __syncthreads();
  }
  // epilogue: this lane holds rows m0 + wm + 16 i + 4 q + v of column n0 + wn + 16 j + c
  constexpr bool PAIR = EpiTraits<EPI>::pair;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn + 16 * j + c;
      const float f0 = NRM == PFN_FOLD ? p.fs[min(n, N - 1)] : 0.f;   // folded row sum of this column
      const float vv[4] = {acc[i][j].x, acc[i][j].y, acc[i][j].z, acc[i][j].w};
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + wm + 16 * i + 4 * q + v;
        const int rl = wm + 16 * i + 4 * q + v;
        float v0 = vv[v];
        if (NRM == PFN_RMS) v0 *= s_r[rl];
        if (NRM == PFN_FOLD) v0 = s_r[rl] * (v0 - s_mu[rl] * f0);
        const float v1 = __shfl_xor(v0, 1);   // the odd neighbour's column (pairs)
        const bool own = m < M && (PAIR ? ((c & 1) == 0 && n + 1 < N) : n < N);
        if (EPI == EPI_PLAIN && S > 1) {
          if (own)
            __hip_atomic_fetch_add(p.y + (size_t)m * p.ldy + n, v0 + (z == 0 ? p.bias[n] : 0.f), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        } else if (own) {
          const EpiOps eo = epi_prefetch<EPI, false>(p, m, n);
          epi_store<EPI>(p, eo, m, n, v0, v1);
        }
      }
    }
}

// Causal attention of M prompt rows (positions p0 .. p0 + M - 1 of one sequence)
// against the cache, which already holds their K/V. Workgroup (query tile t, query
// head h, split s): 64 query rows against key tiles [s kt, (s + 1) kt) of the 64-position
// tiles the query tile reaches, on the fp32 matrix cores. Wave w owns queries
// 16 w .. 16 w + 15 of the tile and computes, per key tile, the transposed scores
// S^T = K Q^T (keys as rows) and then O^T += V^T P^T:
//  - v_mfma_f32_16x16x4f32 number s of a 16-key block contracts head dims 16 q + s, so
//    lane l = 16 q + c holds K[key c][16 q .. 16 q + 15] (LDS) and Q[query c][same dims]
//    (registers, loaded once);
//  - the score accumulator of key block b holds S^T[keys 16 b + 4 q + v][query c], which
//    is exactly the second product's operand P^T[k = q][n = c] for the key chunk
//    {16 b + 4 q + v}, so P never goes through LDS; the matching V^T values come from a
//    transposed copy of the V tile in LDS (4 consecutive keys per 16-byte read);
//  - every value a lane holds belongs to its query c, so the online softmax rescales the
//    output accumulators per lane; the running max is reduced over the four lanes of a
//    query each key tile, the running sum only at the end.
// Each key tile is staged in LDS (float, widened from a bf16 cache) while the next one
// is loaded into registers. Positions after a row's own are masked (never weighted).
// With one split (S = 1) the output o [M][ldo] is written normalized at the head's
// columns; with S > 1 every split writes its partial (running max, sum of weights,
// weighted V) per row and head, and k_attn_pf_merge combines them. Splitting the key
// range gives the launch enough workgroups for the CUs: one per (query tile, head) is
// 96 for a 512-row GPT-2 chunk.
#define PF_MAXS 8          // key-range splits at most
#define PF_PSTRIDE 68      // floats per partial: max, sum, 2 pad, 64 weighted-V values
struct PfAttnParams {
  const float* q; int ldq;                // [M][ldq] post-RoPE queries
  const void* kc; const void* vc;         // this layer's pools [nblk][Hkv][B][HD]
  const int* table;                       // the sequence's block table (paged), or NULL
  long long kv0;                          // contiguous: element offset of the sequence's slot
  int block_size, nblk, Hq, Hkv, M, p0;
  float scale;
  float* out; int ldo;
  int S, kt;                              // key-range splits (gridDim.z) and key tiles per split
  float* part;                            // S > 1: partials [M][Hq][S][PF_PSTRIDE]
};

__device__ __forceinline__ float f4_at(const f32x4& v, int u) {
  return u == 0 ? v.x : u == 1 ? v.y : u == 2 ? v.z : v.w;
}

template <int HD, bool PAGED, bool KV16>
__global__ __launch_bounds__(PF_NT) void k_attn_prefill(PfAttnParams p) {
  static_assert(HD == 64, "head_dim 64");
  constexpr int BQ = 64, BKV = 64, LS = HD + 4;   // LDS row strides (16-byte aligned rows)
  __shared__ __align__(16) float sK[BKV * LS];    // [key][dim]
  __shared__ __align__(16) float sVt[HD * LS];    // [dim][key]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q4 = lane >> 4, c = lane & 15;
  const int qt = blockIdx.x, h = blockIdx.y, kh = h / (p.Hq / p.Hkv), sp = blockIdx.z;
  const int r0 = qt * BQ;
  const int last_pos = p.p0 + min(r0 + BQ, p.M) - 1;   // the tile's last query position
  const int kt0 = sp * p.kt, kt1 = min(last_pos / BKV + 1, kt0 + p.kt);   // this split's key tiles
  const int row = r0 + 16 * wave + c;                  // this lane's query (rows >= M never stored)
  float* pp = p.part + (((size_t)row * p.Hq + h) * p.S + sp) * PF_PSTRIDE;
  if (kt0 >= kt1) {   // no key tile of this query tile falls in the split: an empty partial
    if (row < p.M) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) *reinterpret_cast<f32x4*>(pp + 4 + 16 * dt + 4 * q4) = (f32x4){0.f, 0.f, 0.f, 0.f};
      if (q4 == 0) { pp[0] = -INFINITY; pp[1] = 0.f; }
    }
    return;
  }
  const int qpos = p.p0 + row;
  // this lane's query values: dims 16 q4 .. 16 q4 + 15 of its row
  f32x4 qv[4];
  {
    const float* src = p.q + (size_t)min(row, p.M - 1) * p.ldq + h * HD + 16 * q4;
#pragma unroll
    for (int u = 0; u < 4; ++u) qv[u] = *reinterpret_cast<const f32x4*>(src + 4 * u);
  }
  // key tile loads: K unit e = tid + 256 u is (key e / 16, dims 4 (e % 16) ..), V unit
  // is (key e % 64, dims 4 (e / 64) ..), so that the transposed V stores of a wave fall
  // on 64 consecutive LDS words
  f32x4 kr[4], vr[4];
  auto kv_off = [&](int pos) -> size_t {
    if (PAGED) {
      const int bi = pos / p.block_size;
      int blk = p.table[bi];
      blk = (unsigned)blk < (unsigned)p.nblk ? blk : 0;
      return (((size_t)blk * p.Hkv + kh) * p.block_size + (pos - bi * p.block_size)) * HD;
    }
    return (size_t)p.kv0 + ((size_t)kh * p.block_size + pos) * HD;
  };
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = tid + PF_NT * u;
      const int pk = min(kt * BKV + (e >> 4), last_pos), pv = min(kt * BKV + (e & 63), last_pos);
      kr[u] = kv_load4<KV16, false>(p.kc, kv_off(pk) + 4 * (e & 15));
      vr[u] = kv_load4<KV16, false>(p.vc, kv_off(pv) + 4 * (e >> 6));
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = tid + PF_NT * u;
      *reinterpret_cast<f32x4*>(sK + (e >> 4) * LS + 4 * (e & 15)) = kr[u];
      float* vt = sVt + (4 * (e >> 6)) * LS + (e & 63);
      vt[0] = vr[u].x; vt[LS] = vr[u].y; vt[2 * LS] = vr[u].z; vt[3 * LS] = vr[u].w;
    }
  };
  f32x4 oacc[4];   // O^T[dims 16 dt + 4 q4 + v][query c]
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) oacc[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_lane = 0.f;
  load_tile(kt0);
  for (int kt = kt0; kt < kt1; ++kt) {
    __syncthreads();   // the previous tile is no longer read
    store_tile();
    __syncthreads();
    if (kt + 1 < kt1) load_tile(kt + 1);   // in flight during this tile's MFMAs
    // S^T for the four 16-key blocks
    f32x4 st[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      f32x4 kv[4];
      const float* src = sK + (16 * b + c) * LS + 16 * q4;
#pragma unroll
      for (int u = 0; u < 4; ++u) kv[u] = *reinterpret_cast<const f32x4*>(src + 4 * u);
      st[b] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 16; ++s)
        st[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(f4_at(kv[s >> 2], s & 3), f4_at(qv[s >> 2], s & 3), st[b], 0, 0, 0);
    }
    // scale and mask; the tile's max over the query's 64 keys (this lane's 16 and the
    // other three lanes of the query)
    float sv[4][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int kpos = kt * BKV + 16 * b + 4 * q4 + v;
        sv[b][v] = kpos <= qpos ? f4_at(st[b], v) * p.scale : -INFINITY;
        tmax = fmaxf(tmax, sv[b][v]);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    // -inf only while every key so far is after the query (never in split 0, which
    // holds key 0); then every weight below is 0 and the query stays empty
    const float nm = fmaxf(m_run, tmax);
    const float alpha = attn_rescale(m_run, nm);
    m_run = nm;
    l_lane *= alpha;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      oacc[dt].x *= alpha; oacc[dt].y *= alpha; oacc[dt].z *= alpha; oacc[dt].w *= alpha;
    }
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float e = sv[b][v] == -INFINITY ? 0.f : expf(sv[b][v] - nm);
        sv[b][v] = e;
        l_lane += e;
      }
    // O^T += V^T P^T over the 16 key chunks {16 b + 4 q + v}
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const f32x4 vt = *reinterpret_cast<const f32x4*>(sVt + (16 * dt + c) * LS + 16 * b + 4 * q4);
#pragma unroll
        for (int v = 0; v < 4; ++v)
          oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(f4_at(vt, v), sv[b][v], oacc[dt], 0, 0, 0);
      }
  }
  float l = l_lane + __shfl_xor(l_lane, 16);
  l += __shfl_xor(l, 32);
  if (row >= p.M) return;
  if (p.S == 1) {   // the whole key range: l > 0 (key 0 is visible to every row)
    const float inv = 1.0f / l;
    float* dst = p.out + (size_t)row * p.ldo + h * HD + 4 * q4;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      *reinterpret_cast<f32x4*>(dst + 16 * dt) =
          (f32x4){oacc[dt].x * inv, oacc[dt].y * inv, oacc[dt].z * inv, oacc[dt].w * inv};
  } else {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) *reinterpret_cast<f32x4*>(pp + 4 + 16 * dt + 4 * q4) = oacc[dt];
    if (q4 == 0) { pp[0] = m_run; pp[1] = l; }
  }
}

// Merge of the key-range partials of k_attn_prefill: row m, head h, dim d:
// o = sum_s e^(max_s - mx) o_s / sum_s e^(max_s - mx) l_s with mx the largest max_s
// (finite: split 0 holds key 0). One workgroup per row; thread e takes (h, d) =
// (e / 64, e % 64), its S partial values loaded together.
__global__ __launch_bounds__(PF_NT) void k_attn_pf_merge(const float* __restrict__ part, int Hq, int S,
                                                         float* __restrict__ out, int ldo) {
  const int row = blockIdx.x;
  for (int e = threadIdx.x; e < Hq * 64; e += PF_NT) {
    const int h = e >> 6, d = e & 63;
    const float* pp = part + ((size_t)row * Hq + h) * S * PF_PSTRIDE;
    float ms[PF_MAXS], ls[PF_MAXS], os[PF_MAXS];
#pragma unroll
    for (int s = 0; s < PF_MAXS; ++s) {
      const int t = min(s, S - 1);
      ms[s] = pp[t * PF_PSTRIDE];
      ls[s] = pp[t * PF_PSTRIDE + 1];
      os[s] = pp[t * PF_PSTRIDE + 4 + d];
    }
    float mx = -INFINITY;
#pragma unroll
    for (int s = 0; s < PF_MAXS; ++s) mx = fmaxf(mx, ms[s]);
    float l = 0.f, o = 0.f;
#pragma unroll
    for (int s = 0; s < PF_MAXS; ++s) {
      const float w = s < S ? attn_rescale(ms[s], mx) : 0.f;
      l = fmaf(ls[s], w, l);
      o = fmaf(os[s], w, o);
    }
    out[(size_t)row * ldo + e] = o / l;
  }
}
