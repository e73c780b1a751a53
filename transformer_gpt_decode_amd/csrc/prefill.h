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
#define PF_PD 4   // K steps in flight
template <int WT, int EPI>
__global__ __launch_bounds__(PF_NT) void k_gemm_pf(LinParams p) {
  __shared__ __align__(16) float sA[2][PF_BM * PF_LDS];
  __shared__ __align__(16) float sW[2][PF_BN * PF_LDS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, c = lane & 15;
  const int n0 = blockIdx.x * PF_BN, m0 = blockIdx.y * PF_BM;
  const int M = p.M, N = p.N, K = p.K;
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;
  // this thread's share of a tile: row lr, columns 8 lc .. 8 lc + 7
  const int lr = tid >> 2, lc = tid & 3;
  const int am = min(m0 + lr, M - 1), wr = min(n0 + lr, N - 1);
  const float* a_src = p.x + (size_t)am * p.ldx + 8 * lc;
  f32x4 ra[PF_PD][2], rw[PF_PD][2];
  const int nk = K / PF_BK, S = gridDim.z, z = blockIdx.z;
  // this split's groups of PD steps (the last group of the last split may reach past K)
  const int ng = (nk + PF_PD - 1) / PF_PD;
  const int g0 = z * ng / S, g1 = (z + 1) * ng / S;   // g0 < g1: S <= ng
  auto load = [&](int i, int st) {   // step st (clamped to the last one) into slot i
    const int k0 = min(st, nk - 1) * PF_BK;
    ra[i][0] = *reinterpret_cast<const f32x4*>(a_src + k0);
    ra[i][1] = *reinterpret_cast<const f32x4*>(a_src + k0 + 4);
    if constexpr (WT == 0) {
      const float* w = reinterpret_cast<const float*>(p.w) + (size_t)wr * K + k0 + 8 * lc;
      rw[i][0] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(w));
      rw[i][1] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(w) + 1);
    } else {
      const uint16_t* w = reinterpret_cast<const uint16_t*>(p.w) + (size_t)wr * K + k0 + 8 * lc;
      const u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(w));
      rw[i][0] = (f32x4){bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y)};
      rw[i][1] = (f32x4){bf16_lo(u.z), bf16_hi(u.z), bf16_lo(u.w), bf16_hi(u.w)};
    }
  };
  auto store = [&](int i, bool valid) {   // slot i into LDS buffer i % 2 (zeros past K)
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    float* a = sA[i & 1] + lr * PF_LDS + 8 * lc;
    float* w = sW[i & 1] + lr * PF_LDS + 8 * lc;
    *reinterpret_cast<f32x4*>(a) = valid ? ra[i][0] : z4;
    *reinterpret_cast<f32x4*>(a + 4) = valid ? ra[i][1] : z4;
    *reinterpret_cast<f32x4*>(w) = valid ? rw[i][0] : z4;
    *reinterpret_cast<f32x4*>(w + 4) = valid ? rw[i][1] : z4;
  };
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
  // A step's 32 K columns: MFMA t (0..7) contracts k = 8 q + t, so each lane reads its
  // eight operand values of a row with two 16-byte LDS loads, all before the MFMAs
  auto mfma = [&](int b) {
    F8 a[2], w[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float* src = sA[b] + (wm + 16 * i + c) * PF_LDS + 8 * q;
      a[i].a = *reinterpret_cast<const f32x4*>(src);
      a[i].b = *reinterpret_cast<const f32x4*>(src + 4);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float* src = sW[b] + (wn + 16 * j + c) * PF_LDS + 8 * q;
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
// tiles the query tile reaches; each key tile staged in LDS (float, widened from a bf16
// cache), scores of a 4 x 4 block per thread, the online softmax per row over the 16
// threads that share it, then P V for a 4-row x 4-dim block per thread. Positions after
// a row's own are masked (never weighted). With one split (S = 1) the output o [M][ldo]
// is written normalized at the head's columns; with S > 1 every split writes its
// partial (running max, sum of weights, weighted V) per row and head, and
// k_attn_pf_merge combines them. Splitting the key range gives the launch enough
// workgroups for the CUs: one per (query tile, head) is 96 for a 512-row GPT-2 chunk.
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

template <int HD, bool PAGED, bool KV16>
__global__ __launch_bounds__(PF_NT) void k_attn_prefill(PfAttnParams p) {
  static_assert(HD == 64, "head_dim 64");
  constexpr int BQ = 64, BKV = 64, LS = HD + 4;   // LDS row stride (16-byte aligned)
  __shared__ __align__(16) float sQ[BQ * LS];
  __shared__ __align__(16) float sK[BKV * LS];
  __shared__ __align__(16) float sV[BKV * LS];
  __shared__ __align__(16) float sP[BQ * (BKV + 4)];
  const int tid = threadIdx.x;
  const int qt = blockIdx.x, h = blockIdx.y, kh = h / (p.Hq / p.Hkv), sp = blockIdx.z;
  const int r0 = qt * BQ;                  // first row of the tile
  const int ti = tid >> 4, tj = tid & 15;  // this thread: rows 4 ti .., keys (or dims) 4 tj ..
  const int last_pos = p.p0 + min(r0 + BQ, p.M) - 1;   // the tile's last query position
  const int kt0 = sp * p.kt, kt1 = min(last_pos / BKV + 1, kt0 + p.kt);   // this split's key tiles
  // the partial of row 4 ti + a of the tile (S > 1)
  auto part_at = [&](int a) {
    return p.part + (((size_t)(r0 + 4 * ti + a) * p.Hq + h) * p.S + sp) * PF_PSTRIDE;
  };
  if (kt0 >= kt1) {   // no key tile of this query tile falls in the split: an empty partial
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      if (r0 + 4 * ti + a < p.M) {
        float* pp = part_at(a);
        *reinterpret_cast<f32x4*>(pp + 4 + 4 * tj) = (f32x4){0.f, 0.f, 0.f, 0.f};
        if (tj == 0) { pp[0] = -INFINITY; pp[1] = 0.f; }
      }
    }
    return;
  }
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
  for (int kt = kt0; kt < kt1; ++kt) {
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
      // -inf only while every key so far is after the row (never in split 0, which holds
      // key 0); then every weight below is 0 and the row stays empty
      const float nm = fmaxf(mrow[a], mx);
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
    if (row >= p.M) continue;
    if (p.S == 1) {   // the whole key range: l > 0 (key 0 is visible to every row)
      const float inv = 1.0f / lrow[a];
      *reinterpret_cast<f32x4*>(p.out + (size_t)row * p.ldo + h * HD + 4 * tj) =
          (f32x4){o[a][0] * inv, o[a][1] * inv, o[a][2] * inv, o[a][3] * inv};
    } else {
      float* pp = part_at(a);
      *reinterpret_cast<f32x4*>(pp + 4 + 4 * tj) = (f32x4){o[a][0], o[a][1], o[a][2], o[a][3]};
      if (tj == 0) { pp[0] = mrow[a]; pp[1] = lrow[a]; }
    }
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
