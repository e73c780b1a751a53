// mlp.h -- the GPT-2 MLP block of a few rows in one launch: pre-norm, FC + bias,
// clamped tanh-GELU, down-projection (+ bias), added to the residual.
//
// The block is y = x + W_proj gelu(W_fc LN(x) + b_fc) + b_proj ("bare-metal-llm",
// "What got built"; "batch_forge", the op/status table). As two GEMVs it costs two
// dependent launches; here workgroup (js, ns) takes the J hidden units of slice js
// (computing them needs the whole row) and adds their share of outputs n of slice ns,
// sum over j in js of W_proj[n][j] h_j, with float atomics. The 4 workgroups of a
// hidden slice compute the same hidden units (their W_fc rows come from HBM once and
// from the XCD's L2 after: the grid order puts them on one XCD), so that each output
// receives one atomic per hidden slice (64), a count that adds no measurable time on
// this GPU, where 256 per address add microseconds.
//
// Measured on this GPU it is slower than the two GEMVs (GPT-2 124M, one row: 7.4 us
// against 2 x 2.4 us plus a 1.7 us launch gap): each CU streams its slice's 147 KB of
// W_fc (4x the bytes per CU of the FC GEMV) through a load pipeline of about 64 bytes
// per clock. It stays an option (GD_OPT_FUSE_MLP), off by default.
//
// The launch reads the residual rows x and adds into a separate accumulator z (zero
// on entry): adding into x itself would race with other workgroups still reading x
// for the norm. The next launches fold z back (see the decode chain in runtime.hip).
//
// The pre-norm is folded (fp32 weights; as NRM_FOLDED in k_gemv): W'_fc = g o W_fc,
// b'_fc = b_fc + W_fc b, s_j = row sums of W'_fc; each wave shifts the row by its first
// element, d = x - x_0, and u_j = r (d . w'_j - a s_j) + b'_j with a = mean(d),
// r = 1 / sqrt(var + eps). W_proj is read from a copy packed per (js, ns): float4 c
// of output nl holds W_proj[ns NSL + nl][js J + 4c .. 4c + 3], so that lane nl of
// the first waves reads 16 contiguous bytes per chunk.
#pragma once
#include "common.h"

#define MLP_WG 512   // threads (8 waves)
#define MLP_NS 4     // output slices

struct MlpParams {
  const float* x; int ldx;        // residual rows [M][ldx] (the norm's input)
  int M, K;                       // rows (<= 4), model width
  float eps;
  const float* wfc;               // folded W_fc [ff][K]
  const float* bfc;               // folded bias [ff]
  const float* sfc;               // row sums of the folded W_fc [ff]
  const float* wpk;               // packed W_proj (see above)
  const float* bproj;             // [K]
  float* z; int ldz;              // accumulator rows [M][ldz], zero on entry
  int J, JS, NSL;                 // hidden units per slice, slices, outputs per output slice
};

// NC: 16-byte chunks of a row per lane (K <= 256 NC); RW: hidden units per wave
// (J <= 8 RW); CJ: float4 chunks of a hidden slice (J = 4 CJ).
template <int NC, int RW, int CJ>
__global__ __launch_bounds__(MLP_WG) void k_mlp(MlpParams p) {
  __shared__ __align__(16) float xs[4 * 256 * NC];   // rows [M][K]
  __shared__ __align__(16) float s_h[4][4 * CJ];      // hidden units of this slice [M][J]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int M = p.M, K = p.K, J = p.J;
  // grid order: the MLP_NS workgroups of a hidden slice are 8 apart (one XCD)
  const int id = blockIdx.x, xcd = id & 7, k8 = id >> 3;
  const int ns = k8 % MLP_NS, js = xcd + 8 * (k8 / MLP_NS);
  // every kernel argument at once (left to itself the compiler loads each late)
  asm volatile("" ::"s"(p.x), "s"(p.ldx), "s"(p.wfc), "s"(p.bfc), "s"(p.sfc), "s"(p.wpk), "s"(p.bproj), "s"(p.z),
               "s"(p.ldz), "s"(p.eps));

  // ---- loads, in the order they are needed: rows, hidden-unit operands, W_fc rows,
  // then phase-2 operands (vector loads complete in issue order)
  constexpr int XPT = (4 * 256 * NC / 4 + MLP_WG - 1) / MLP_WG;   // row chunks per thread (M <= 4)
  const int K4 = K >> 2;
  f32x4 xr[XPT];
#pragma unroll
  for (int i = 0; i < XPT; ++i) {
    const int c = min(tid + MLP_WG * i, M * K4 - 1);
    const int m = c / K4, k = (c - m * K4) << 2;
    xr[i] = *reinterpret_cast<const f32x4*>(p.x + (size_t)m * p.ldx + k);
  }
  const int j0 = js * J + wave * RW;                 // this wave's first hidden unit
  const int jl = min(j0 + min(lane, RW - 1), js * J + J - 1);
  const float bf = p.bfc[jl], sf = p.sfc[jl];        // lane r < RW: unit j0 + r
  f32x4 w[RW][NC];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int j = min(j0 + r, js * J + J - 1);
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int k = min((lane + 64 * i) * 4, K - 4);
      // plain loads: the other workgroups of the slice read the same rows from L2 (a
      // non-temporal hint would keep them out of it)
      w[r][i] = *reinterpret_cast<const f32x4*>(p.wfc + (size_t)j * K + k);
    }
  }
  const int nl = min(tid, p.NSL - 1), n = ns * p.NSL + nl;
  f32x4 wp[CJ];
  const f32x4* pk = reinterpret_cast<const f32x4*>(p.wpk) + ((size_t)(js * MLP_NS + ns) * CJ) * p.NSL + nl;
#pragma unroll
  for (int c = 0; c < CJ; ++c) wp[c] = __builtin_nontemporal_load(pk + (size_t)c * p.NSL);
  const float bp = p.bproj[n];
  __builtin_amdgcn_sched_barrier(0);   // every load above is issued before the first wait

  // ---- rows into LDS (clamped duplicates of the last chunk rewrite the same value)
#pragma unroll
  for (int i = 0; i < XPT; ++i) {
    const int c = min(tid + MLP_WG * i, M * K4 - 1);
    const int m = c / K4, k = (c - m * K4) << 2;
    *reinterpret_cast<f32x4*>(xs + m * K + k) = xr[i];
  }
  __syncthreads();

  // ---- phase 1: the wave's hidden units for every row
  const float invK = 1.0f / (float)K;
  float hv[RW][4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    if (m < M) {
      f32x4 d[NC];
      const float sh = xs[m * K];
      float st[2] = {0.f, 0.f};
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        const int k = (lane + 64 * i) * 4;
        d[i] = k < K ? *reinterpret_cast<const f32x4*>(xs + m * K + k) : (f32x4){sh, sh, sh, sh};
        d[i].x -= sh; d[i].y -= sh; d[i].z -= sh; d[i].w -= sh;   // zero past K
        st[0] += (d[i].x + d[i].y) + (d[i].z + d[i].w);
        st[1] += fmaf(d[i].x, d[i].x, d[i].y * d[i].y) + fmaf(d[i].z, d[i].z, d[i].w * d[i].w);
      }
      float acc[RW];
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < NC; ++i) {
          s = fmaf(w[r][i].x, d[i].x, s); s = fmaf(w[r][i].y, d[i].y, s);
          s = fmaf(w[r][i].z, d[i].z, s); s = fmaf(w[r][i].w, d[i].w, s);
        }
        acc[r] = s;
      }
      wave_sum_n<2>(st);
      wave_sum_n<RW>(acc);
      const float a = st[0] * invK;
      const float rs = rsqrtf(fmaxf(st[1] * invK - a * a, 0.f) + p.eps);
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        const float sr = __shfl(sf, r), br = __shfl(bf, r);
        hv[r][m] = gelu_clamped(fmaf(rs, acc[r] - a * sr, br));
      }
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < RW; ++r)
      if (wave * RW + r < J)
#pragma unroll
        for (int m = 0; m < 4; ++m)
          if (m < M) s_h[m][wave * RW + r] = hv[r][m];
  }
  __syncthreads();

  // ---- phase 2: this slice's share of outputs ns NSL .. + NSL, added to z
  if (tid < p.NSL) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if (m < M) {
        float y = 0.f;
#pragma unroll
        for (int c = 0; c < CJ; ++c) {
          const f32x4 hh = *reinterpret_cast<const f32x4*>(&s_h[m][4 * c]);
          y = fmaf(wp[c].x, hh.x, y); y = fmaf(wp[c].y, hh.y, y);
          y = fmaf(wp[c].z, hh.z, y); y = fmaf(wp[c].w, hh.w, y);
        }
        if (js == 0) y += bp;
        __hip_atomic_fetch_add(p.z + (size_t)m * p.ldz + n, y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}
