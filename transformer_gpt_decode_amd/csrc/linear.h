// linear.h -- y = epilogue(norm(x) . W^T) for 1..32 activation rows.
//
// A linear layer is y = x . W^T with W stored [out][in] ("rvllm Metal backend",
// "The matmul pain story"). Decode streams every weight once per step and does
// little arithmetic per byte, so the kernel is built around streaming W with
// 16-byte loads; X (at most 32 rows) is staged once per workgroup in LDS.
//
// Work unit: a tile of 16 output columns over a K range of `kc` elements. A
// workgroup (4 waves) takes `ntw` consecutive tiles of one K range; `ksplit`
// workgroups cover K and the last one to finish a tile sums the partial tiles in
// fixed order (deterministic split-K), then applies the epilogue.
//
// Two inner loops over the same tile:
//  VAR 0 (VALU GEMV, few rows): a 16-lane group per weight row, 8 weights per lane
//        per step, 16-lane reduction; each wave owns 4 rows of the tile.
//  VAR 1 (MFMA): v_mfma_f32_16x16x4f32. Lane l holds W[n0 + l%16][k + 8(l/16) .. +8]
//        and X[m0 + l%16][same k]; step t of 8 feeds element t of both, so the four
//        k-slots of one instruction are k + 8q + t (q = l/16) for A and B alike. The
//        4 waves split the K range by 32-element blocks and are summed in LDS.
//
// Prologue: optional LayerNorm / RMSNorm of the x rows (statistics over the whole
// row, two passes, per wave), applied while staging the K range into LDS.
// Epilogues: bias, tanh-GELU (clamped), residual add, SiLU-gated pairs, or logits
// with a fused greedy argmax (per-tile partials, last workgroup reduces).
#pragma once
#include "common.h"

#define LIN_ACT_NONE 0
#define LIN_ACT_GELU 1
#define LIN_ACT_SWIGLU 2
#define LIN_ACT_ARGMAX 3

struct LinearParams {
  const float* x; int ldx;
  const void* w;
  const float* bias;
  int norm; const float* ng; const float* nb; float eps;
  int act;
  const float* resid; int ldr;
  float* y; int ldy;
  int M, N, K;
  int kc, ksplit, ntw, ntiles, mpad;
  float* part;      // [ntiles][ksplit][M][16]
  int* ctr;         // [ntiles]
  float* am_val;    // [ntiles][M]
  int* am_idx;      // [ntiles][M]
  int* am_ctr;      // [1]
  int* am_out;      // [M]
  float* logits; int ldl;
};

template <int WT, int VAR, int MT>
__global__ __launch_bounds__(GD_WG) void k_linear(LinearParams p) {
  extern __shared__ __align__(16) float xs[];   // [mpad][kcp]
  __shared__ float st_mean[GD_MAX_ROWS], st_rstd[GD_MAX_ROWS];
  __shared__ float tileT[GD_MAX_ROWS][GD_TILE_N];
  __shared__ float red[4][GD_MAX_ROWS][GD_TILE_N];
  __shared__ int s_last;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int M = p.M, N = p.N, K = p.K;
  const int ks = blockIdx.x % p.ksplit;
  const int tg = blockIdx.x / p.ksplit;
  const int k0 = ks * p.kc;
  const int klen = min(K - k0, p.kc);
  const int kpad = (klen + 31) & ~31;
  const int kcp = p.kc + 4;
  const int mpad = p.mpad;

  // ---- norm statistics over the full rows
  if (p.norm) {
    for (int m = wave; m < M; m += 4) {
      const float* xr = p.x + (size_t)m * p.ldx;
      float mean = 0.f;
      if (p.norm == 1) {
        float s = 0.f;
        for (int k = lane; k < K; k += 64) s += xr[k];
        mean = wave_sum(s) / (float)K;
      }
      float v = 0.f;
      for (int k = lane; k < K; k += 64) { float t = xr[k] - mean; v = fmaf(t, t, v); }
      float var = wave_sum(v) / (float)K;
      if (lane == 0) { st_mean[m] = mean; st_rstd[m] = 1.0f / sqrtf(var + p.eps); }
    }
    __syncthreads();
  }
  // ---- stage x[:, k0 : k0+klen) (normalized) into LDS, zero padded to mpad x kpad
  {
    const int q4 = kpad >> 2;
    for (int idx = tid; idx < mpad * q4; idx += GD_WG) {
      int m = idx / q4, k = (idx - m * q4) << 2;
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (m < M && k < klen) {
        v = *reinterpret_cast<const f32x4*>(p.x + (size_t)m * p.ldx + k0 + k);
        if (p.norm == 1) {
          float mu = st_mean[m], r = st_rstd[m];
          f32x4 g = *reinterpret_cast<const f32x4*>(p.ng + k0 + k);
          f32x4 b = *reinterpret_cast<const f32x4*>(p.nb + k0 + k);
          v.x = (v.x - mu) * r * g.x + b.x; v.y = (v.y - mu) * r * g.y + b.y;
          v.z = (v.z - mu) * r * g.z + b.z; v.w = (v.w - mu) * r * g.w + b.w;
        } else if (p.norm == 2) {
          float r = st_rstd[m];
          f32x4 g = *reinterpret_cast<const f32x4*>(p.ng + k0 + k);
          v.x = v.x * r * g.x; v.y = v.y * r * g.y; v.z = v.z * r * g.z; v.w = v.w * r * g.w;
        }
      }
      *reinterpret_cast<f32x4*>(xs + m * kcp + k) = v;
    }
  }
  __syncthreads();

  const int t_begin = tg * p.ntw;
  const int t_end = min(p.ntiles, t_begin + p.ntw);
  for (int t = t_begin; t < t_end; ++t) {
    const int n0 = t * GD_TILE_N;
    if (VAR == 0) {
      // ---------------- VALU GEMV: wave owns rows n0 + 4*wave + (lane >> 4)
      const int r_in = wave * 4 + (lane >> 4);
      const int n = n0 + r_in;
      const int j = lane & 15;
      const size_t row_off = (size_t)n * K;
      const int nch = klen >> 3;
      for (int mg = 0; mg < mpad; mg += 4) {
        float acc0 = 0.f, acc1 = 0.f, acc2 = 0.f, acc3 = 0.f;
#pragma unroll 4
        for (int c = j; c < nch; c += 16) {
          float w[8];
          if (n < N) load_w8<WT>(p.w, row_off, k0 + c * 8, w);
          else { for (int i = 0; i < 8; ++i) w[i] = 0.f; }
          const float* x0 = xs + (mg + 0) * kcp + c * 8;
          f32x4 a0 = *reinterpret_cast<const f32x4*>(x0), b0 = *reinterpret_cast<const f32x4*>(x0 + 4);
          acc0 = fmaf(w[0], a0.x, acc0); acc0 = fmaf(w[1], a0.y, acc0); acc0 = fmaf(w[2], a0.z, acc0); acc0 = fmaf(w[3], a0.w, acc0);
          acc0 = fmaf(w[4], b0.x, acc0); acc0 = fmaf(w[5], b0.y, acc0); acc0 = fmaf(w[6], b0.z, acc0); acc0 = fmaf(w[7], b0.w, acc0);
          if (mg + 1 < M) {
            const float* x1 = x0 + kcp;
            f32x4 a1 = *reinterpret_cast<const f32x4*>(x1), b1 = *reinterpret_cast<const f32x4*>(x1 + 4);
            acc1 = fmaf(w[0], a1.x, acc1); acc1 = fmaf(w[1], a1.y, acc1); acc1 = fmaf(w[2], a1.z, acc1); acc1 = fmaf(w[3], a1.w, acc1);
            acc1 = fmaf(w[4], b1.x, acc1); acc1 = fmaf(w[5], b1.y, acc1); acc1 = fmaf(w[6], b1.z, acc1); acc1 = fmaf(w[7], b1.w, acc1);
          }
          if (mg + 2 < M) {
            const float* x2 = x0 + 2 * kcp;
            f32x4 a2 = *reinterpret_cast<const f32x4*>(x2), b2 = *reinterpret_cast<const f32x4*>(x2 + 4);
            acc2 = fmaf(w[0], a2.x, acc2); acc2 = fmaf(w[1], a2.y, acc2); acc2 = fmaf(w[2], a2.z, acc2); acc2 = fmaf(w[3], a2.w, acc2);
            acc2 = fmaf(w[4], b2.x, acc2); acc2 = fmaf(w[5], b2.y, acc2); acc2 = fmaf(w[6], b2.z, acc2); acc2 = fmaf(w[7], b2.w, acc2);
          }
          if (mg + 3 < M) {
            const float* x3 = x0 + 3 * kcp;
            f32x4 a3 = *reinterpret_cast<const f32x4*>(x3), b3 = *reinterpret_cast<const f32x4*>(x3 + 4);
            acc3 = fmaf(w[0], a3.x, acc3); acc3 = fmaf(w[1], a3.y, acc3); acc3 = fmaf(w[2], a3.z, acc3); acc3 = fmaf(w[3], a3.w, acc3);
            acc3 = fmaf(w[4], b3.x, acc3); acc3 = fmaf(w[5], b3.y, acc3); acc3 = fmaf(w[6], b3.z, acc3); acc3 = fmaf(w[7], b3.w, acc3);
          }
        }
        acc0 = group_sum<16>(acc0); acc1 = group_sum<16>(acc1);
        acc2 = group_sum<16>(acc2); acc3 = group_sum<16>(acc3);
        if (j == 0) {
          if (mg + 0 < M) tileT[mg + 0][r_in] = acc0;
          if (mg + 1 < M) tileT[mg + 1][r_in] = acc1;
          if (mg + 2 < M) tileT[mg + 2][r_in] = acc2;
          if (mg + 3 < M) tileT[mg + 3][r_in] = acc3;
        }
      }
      __syncthreads();
    } else {
      // ---------------- MFMA 16x16x4 f32: lane holds column n, k-slot q
      const int n = n0 + (lane & 15);
      const int q = lane >> 4;
      const int nb = kpad >> 5;
      f32x4 acc[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
      for (int b = wave; b < nb; b += 4) {
        const int kk = b * 32 + q * 8;
        float w[8];
        if (n < N && kk < klen) load_w8<WT>(p.w, (size_t)n * K, k0 + kk, w);
        else { for (int i = 0; i < 8; ++i) w[i] = 0.f; }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const float* xr = xs + (mt * 16 + (lane & 15)) * kcp + kk;
          f32x4 xa = *reinterpret_cast<const f32x4*>(xr), xb = *reinterpret_cast<const f32x4*>(xr + 4);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa.x, w[0], acc[mt], 0, 0, 0);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa.y, w[1], acc[mt], 0, 0, 0);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa.z, w[2], acc[mt], 0, 0, 0);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa.w, w[3], acc[mt], 0, 0, 0);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(xb.x, w[4], acc[mt], 0, 0, 0);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(xb.y, w[5], acc[mt], 0, 0, 0);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(xb.z, w[6], acc[mt], 0, 0, 0);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(xb.w, w[7], acc[mt], 0, 0, 0);
        }
      }
      // D[i][j]: lane holds j = lane % 16, rows i = 4q + v
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        red[wave][mt * 16 + 4 * q + 0][lane & 15] = acc[mt].x;
        red[wave][mt * 16 + 4 * q + 1][lane & 15] = acc[mt].y;
        red[wave][mt * 16 + 4 * q + 2][lane & 15] = acc[mt].z;
        red[wave][mt * 16 + 4 * q + 3][lane & 15] = acc[mt].w;
      }
      __syncthreads();
      for (int idx = tid; idx < M * GD_TILE_N; idx += GD_WG) {
        int m = idx >> 4, c = idx & 15;
        tileT[m][c] = ((red[0][m][c] + red[1][m][c]) + red[2][m][c]) + red[3][m][c];
      }
      __syncthreads();
    }

    // ---------------- split-K: last workgroup of the tile sums the partials in order
    if (p.ksplit > 1) {
      float* pt = p.part + (size_t)t * p.ksplit * M * GD_TILE_N;
      for (int idx = tid; idx < M * GD_TILE_N; idx += GD_WG)
        pt[(size_t)ks * M * GD_TILE_N + idx] = tileT[idx >> 4][idx & 15];
      fence_agent();
      __syncthreads();
      if (tid == 0) {
        int old = atomic_add_acq_rel(p.ctr + t, 1);
        s_last = (old == p.ksplit - 1);
        if (s_last) store_relaxed(p.ctr + t, 0);
      }
      __syncthreads();
      if (!s_last) continue;
      fence_agent();
      for (int idx = tid; idx < M * GD_TILE_N; idx += GD_WG) {
        float s = pt[idx];
        for (int k2 = 1; k2 < p.ksplit; ++k2) s += pt[(size_t)k2 * M * GD_TILE_N + idx];
        tileT[idx >> 4][idx & 15] = s;
      }
      __syncthreads();
    }

    // ---------------- epilogues
    if (p.act == LIN_ACT_SWIGLU) {
      // tile t holds gate columns 8t..8t+7 then the matching up columns
      for (int idx = tid; idx < M * 8; idx += GD_WG) {
        int m = idx >> 3, c = idx & 7;
        int jcol = t * 8 + c;
        if (n0 + 8 + c < N) p.y[(size_t)m * p.ldy + jcol] = silu(tileT[m][c]) * tileT[m][c + 8];
      }
    } else if (p.act == LIN_ACT_ARGMAX) {
      if (p.logits) {
        for (int idx = tid; idx < M * GD_TILE_N; idx += GD_WG) {
          int m = idx >> 4, c = idx & 15;
          if (n0 + c < N) p.logits[(size_t)m * p.ldl + n0 + c] = tileT[m][c];
        }
      }
      if (tid < M) {
        float bv = tileT[tid][0];
        int bi = n0;
        for (int c = 1; c < GD_TILE_N && n0 + c < N; ++c)
          if (am_better(tileT[tid][c], n0 + c, bv, bi)) { bv = tileT[tid][c]; bi = n0 + c; }
        p.am_val[(size_t)t * M + tid] = bv;
        p.am_idx[(size_t)t * M + tid] = bi;
      }
      fence_agent();
      __syncthreads();
      if (tid == 0) {
        int old = atomic_add_acq_rel(p.am_ctr, 1);
        s_last = (old == p.ntiles - 1);
        if (s_last) store_relaxed(p.am_ctr, 0);
      }
      __syncthreads();
      if (s_last) {
        fence_agent();
        for (int m = wave; m < M; m += 4) {
          float bv = __builtin_nanf("");
          int bi = 0x7fffffff;
          bool have = false;
          for (int tt = lane; tt < p.ntiles; tt += 64) {
            float v = p.am_val[(size_t)tt * M + m];
            int i = p.am_idx[(size_t)tt * M + m];
            if (!have || am_better(v, i, bv, bi)) { bv = v; bi = i; have = true; }
          }
#pragma unroll
          for (int o = 32; o > 0; o >>= 1) {
            float ov = __shfl_xor(bv, o, 64);
            int oi = __shfl_xor(bi, o, 64);
            int oh = __shfl_xor((int)have, o, 64);
            if (oh && (!have || am_better(ov, oi, bv, bi))) { bv = ov; bi = oi; have = true; }
          }
          if (lane == 0) p.am_out[m] = bi;
        }
      }
    } else {
      for (int idx = tid; idx < M * GD_TILE_N; idx += GD_WG) {
        int m = idx >> 4, c = idx & 15;
        int n = n0 + c;
        if (n < N) {
          float v = tileT[m][c];
          if (p.bias) v += p.bias[n];
          if (p.act == LIN_ACT_GELU) v = gelu_clamped(v);
          if (p.resid) v = p.resid[(size_t)m * p.ldr + n] + v;
          p.y[(size_t)m * p.ldy + n] = v;
        }
      }
    }
    __syncthreads();
  }
}
