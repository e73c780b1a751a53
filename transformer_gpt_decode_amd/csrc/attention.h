// attention.h -- causal attention of the new rows against the KV cache.
//
// Each row attends to every cached position of its sequence up to and including its
// own ("bare-metal-llm", "What got built": KV-cached causal attention; "rvllm Metal
// backend", "What the kernels do": scores Q K^T, mask, softmax, probs V). Positions
// past the row are never read, so no -inf mask is materialised. The cache is read
// straight from its blocks: position p of a sequence is block table[p / B], slot
// p mod B (the paged layout of the same post; a contiguous cache is one block per
// sequence slot). Query heads h use KV head h / (Hq / Hkv) (grouped-query attention).
//
// Decomposition (split context): one workgroup per (row, KV head, chunk of CH
// positions). Groups of HD/4 lanes take PPG positions each, with every K and V load
// of the group issued before any arithmetic (float4 per lane). Each group reduces
// its scores with a max-subtracted softmax; the groups are merged in LDS into one
// partial (max, sum, weighted V) per query head and chunk. The consumer merges the
// chunks (the O-projection prologue for few rows, or k_attn_merge).
#pragma once
#include "common.h"

struct AttnParams {
  const float* q; int ldq;          // [M][ldq]; query head h at h*HD (post-RoPE)
  const float* kc; const float* vc; // this layer's pools [nblk][Hkv][B][HD]
  const int* table; int max_blocks; // [slots][max_blocks]
  int block_size, nblk;
  int Hq, Hkv;
  const int* row_seq; const int* row_pos;
  int M, nchunk;
  float scale;
  float* part;                      // [M][Hq][nchunk][HD + 2]: max, sum, o[HD]
};

template <int HD, int G, int PPG>
__global__ __launch_bounds__(GD_WG) void k_attention(AttnParams p) {
  constexpr int LG = HD / 4;            // lanes per position group
  constexpr int NG = GD_WG / LG;        // position groups per workgroup
  constexpr int CH = NG * PPG;          // positions per workgroup
  __shared__ float s_m[NG][G], s_l[NG][G];
  __shared__ __align__(16) float s_o[NG][G][HD];

  const int c = blockIdx.x, kh = blockIdx.y, row = blockIdx.z;
  const int tid = threadIdx.x;
  const int grp = tid / LG, gl = tid % LG;
  const int seq = p.row_seq[row];
  const int T = p.row_pos[row] + 1;
  const int nch = (T + CH - 1) / CH;
  if (c >= nch) return;
  const int p0 = c * CH, p1 = min(T, p0 + CH);
  const int* tab = p.table + (size_t)seq * p.max_blocks;

  f32x4 kv[PPG], vv[PPG];
  bool ok[PPG];
#pragma unroll
  for (int j = 0; j < PPG; ++j) {
    const int pos = p0 + grp + NG * j;
    ok[j] = false;
    kv[j] = vv[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
    if (pos < p1) {
      const int bi = pos / p.block_size;
      const int blk = tab[bi];
      if ((unsigned)blk < (unsigned)p.nblk) {
        const size_t off = (((size_t)blk * p.Hkv + kh) * p.block_size + (pos - bi * p.block_size)) * HD + gl * 4;
        kv[j] = *reinterpret_cast<const f32x4*>(p.kc + off);
        vv[j] = *reinterpret_cast<const f32x4*>(p.vc + off);
        ok[j] = true;
      }
    }
  }
  f32x4 q[G];
#pragma unroll
  for (int g = 0; g < G; ++g)
    q[g] = *reinterpret_cast<const f32x4*>(p.q + (size_t)row * p.ldq + (kh * G + g) * HD + gl * 4);

#pragma unroll
  for (int g = 0; g < G; ++g) {
    float s[PPG];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < PPG; ++j) {
      float d = q[g].x * kv[j].x;
      d = fmaf(q[g].y, kv[j].y, d);
      d = fmaf(q[g].z, kv[j].z, d);
      d = fmaf(q[g].w, kv[j].w, d);
      s[j] = group_sum<LG>(d) * p.scale;
      if (ok[j]) mx = fmaxf(mx, s[j]);
    }
    float l = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < PPG; ++j) {
      if (ok[j]) {
        const float e = expf(s[j] - mx);
        l += e;
        o.x = fmaf(e, vv[j].x, o.x);
        o.y = fmaf(e, vv[j].y, o.y);
        o.z = fmaf(e, vv[j].z, o.z);
        o.w = fmaf(e, vv[j].w, o.w);
      }
    }
    if (gl == 0) { s_m[grp][g] = mx; s_l[grp][g] = l; }
    *reinterpret_cast<f32x4*>(&s_o[grp][g][gl * 4]) = o;
  }
  __syncthreads();
  // merge the NG groups into the chunk's partial: one thread per (query head g, dim d)
  if (tid < G * HD) {
    const int g = tid / HD, d = tid % HD;
    float m = -INFINITY;
    for (int i = 0; i < NG; ++i) m = fmaxf(m, s_m[i][g]);
    float l = 0.f, acc = 0.f;
    for (int i = 0; i < NG; ++i) {
      if (s_l[i][g] == 0.f) continue;   // group saw no position
      const float w = expf(s_m[i][g] - m);
      l = fmaf(s_l[i][g], w, l);
      acc = fmaf(s_o[i][g][d], w, acc);
    }
    float* pp = p.part + (((size_t)row * p.Hq + kh * G + g) * p.nchunk + c) * (HD + 2);
    pp[2 + d] = acc;
    if (d == 0) { pp[0] = m; pp[1] = l; }
  }
}

// Merge of the chunk partials into o[M][Hq*HD] (rows with more than 4 per call).
__global__ __launch_bounds__(GD_WG) void k_attn_merge(const float* __restrict__ part, int Hq, int hd, int nchunk,
                                                      int chunk, const int* __restrict__ row_pos, float* out,
                                                      int ldo) {
  const int m = blockIdx.x;
  const int nch = (row_pos[m] + chunk) / chunk;
  for (int i = threadIdx.x; i < Hq * hd; i += GD_WG) {
    const int h = i / hd, d = i - h * hd;
    const float* pp = part + ((size_t)m * Hq + h) * nchunk * (hd + 2);
    float mx = -INFINITY;
    for (int c = 0; c < nch; ++c) mx = fmaxf(mx, pp[(size_t)c * (hd + 2)]);
    float l = 0.f, o = 0.f;
    for (int c = 0; c < nch; ++c) {
      const float w = expf(pp[(size_t)c * (hd + 2)] - mx);
      l = fmaf(pp[(size_t)c * (hd + 2) + 1], w, l);
      o = fmaf(pp[(size_t)c * (hd + 2) + 2 + d], w, o);
    }
    out[(size_t)m * ldo + i] = o / l;
  }
}
