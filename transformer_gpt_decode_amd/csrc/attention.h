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
// Decomposition: one workgroup per (row, KV head, chunk of CH positions). Inside,
// groups of HD/4 lanes take one position each (float4 of K and of V per lane) and keep
// an online softmax (running max, sum, weighted V) for each of the G query heads
// sharing the KV head. Groups are merged in LDS. A row whose context spans several
// chunks writes per-chunk partials; the last chunk workgroup to finish (agent-scope
// counter) merges them in chunk order and resets the counter.
#pragma once
#include "common.h"

struct AttnParams {
  const float* q; int ldq;          // [M][ldq]; query head h at h*HD (post-RoPE)
  float* out; int ldo;              // [M][ldo]; head h at h*HD
  const float* kc; const float* vc; // this layer's pools [nblk][Hkv][B][HD]
  const int* table; int max_blocks; // [slots][max_blocks]
  int block_size, nblk;
  int Hq, Hkv;
  const int* row_seq; const int* row_pos;
  int M, nchunk, chunk;
  float scale;
  float* part;                      // [M][Hq][nchunk][HD + 2]
  int* ctr;                         // [M][Hkv]
};

template <int HD, int G>
__global__ __launch_bounds__(GD_WG) void k_attention(AttnParams p) {
  constexpr int LG = HD / 4;            // lanes per position group
  constexpr int NG = GD_WG / LG;        // position groups per workgroup
  __shared__ float s_m[NG][G], s_l[NG][G];
  __shared__ __align__(16) float s_o[NG][G][HD];
  __shared__ float s_fm[G], s_fl[G];
  __shared__ int s_last;

  const int c = blockIdx.x, kh = blockIdx.y, row = blockIdx.z;
  const int tid = threadIdx.x;
  const int grp = tid / LG, gl = tid % LG;
  const int seq = p.row_seq[row];
  const int T = p.row_pos[row] + 1;
  const int nch = (T + p.chunk - 1) / p.chunk;
  if (c >= nch) return;
  const int p0 = c * p.chunk, p1 = min(T, p0 + p.chunk);
  const int* tab = p.table + (size_t)seq * p.max_blocks;

  f32x4 q[G];
#pragma unroll
  for (int g = 0; g < G; ++g)
    q[g] = *reinterpret_cast<const f32x4*>(p.q + (size_t)row * p.ldq + (kh * G + g) * HD + gl * 4);

  float mx[G], ls[G];
  f32x4 o[G];
#pragma unroll
  for (int g = 0; g < G; ++g) { mx[g] = -INFINITY; ls[g] = 0.f; o[g] = (f32x4){0.f, 0.f, 0.f, 0.f}; }

  for (int pos = p0 + grp; pos < p1; pos += NG) {
    const int blk = tab[pos / p.block_size];
    if ((unsigned)blk >= (unsigned)p.nblk) continue;   // unset entry: flagged by the append kernel
    const int slot = pos - (pos / p.block_size) * p.block_size;
    const size_t off = (((size_t)blk * p.Hkv + kh) * p.block_size + slot) * HD + gl * 4;
    f32x4 k = *reinterpret_cast<const f32x4*>(p.kc + off);
    f32x4 v = *reinterpret_cast<const f32x4*>(p.vc + off);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float d = q[g].x * k.x;
      d = fmaf(q[g].y, k.y, d);
      d = fmaf(q[g].z, k.z, d);
      d = fmaf(q[g].w, k.w, d);
      float s = group_sum<LG>(d) * p.scale;
      float mn = fmaxf(mx[g], s);
      float corr = expf(mx[g] - mn);
      float e = expf(s - mn);
      ls[g] = ls[g] * corr + e;
      o[g].x = o[g].x * corr + e * v.x;
      o[g].y = o[g].y * corr + e * v.y;
      o[g].z = o[g].z * corr + e * v.z;
      o[g].w = o[g].w * corr + e * v.w;
      mx[g] = mn;
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (gl == 0) { s_m[grp][g] = mx[g]; s_l[grp][g] = ls[g]; }
    *reinterpret_cast<f32x4*>(&s_o[grp][g][gl * 4]) = o[g];
  }
  __syncthreads();
  // merge the NG groups: one thread per (query head g, dim d)
  float* pbase = p.part + ((size_t)row * p.Hq + kh * G) * p.nchunk * (HD + 2);
  if (tid < G * HD) {
    const int g = tid / HD, d = tid % HD;
    float m = -INFINITY;
    for (int i = 0; i < NG; ++i) m = fmaxf(m, s_m[i][g]);
    float l = 0.f, acc = 0.f;
    for (int i = 0; i < NG; ++i) {
      if (s_l[i][g] == 0.f) continue;   // group saw no position
      float w = expf(s_m[i][g] - m);
      l = fmaf(s_l[i][g], w, l);
      acc = fmaf(s_o[i][g][d], w, acc);
    }
    if (nch == 1) {
      p.out[(size_t)row * p.ldo + (kh * G + g) * HD + d] = acc / l;
    } else {
      float* pp = pbase + ((size_t)g * p.nchunk + c) * (HD + 2);
      pp[2 + d] = acc;
      if (d == 0) { pp[0] = m; pp[1] = l; }
    }
  }
  if (nch == 1) return;
  fence_agent();
  __syncthreads();
  if (tid == 0) {
    int* ctr = p.ctr + row * p.Hkv + kh;
    int old = atomic_add_acq_rel(ctr, 1);
    s_last = (old == nch - 1);
    if (s_last) store_relaxed(ctr, 0);
  }
  __syncthreads();
  if (!s_last) return;
  fence_agent();
  if (tid < G) {
    float m = -INFINITY;
    for (int cc = 0; cc < nch; ++cc) m = fmaxf(m, pbase[((size_t)tid * p.nchunk + cc) * (HD + 2)]);
    float l = 0.f;
    for (int cc = 0; cc < nch; ++cc) {
      const float* pp = pbase + ((size_t)tid * p.nchunk + cc) * (HD + 2);
      l = fmaf(pp[1], expf(pp[0] - m), l);
    }
    s_fm[tid] = m;
    s_fl[tid] = l;
  }
  __syncthreads();
  if (tid < G * HD) {
    const int g = tid / HD, d = tid % HD;
    const float m = s_fm[g];
    float acc = 0.f;
    for (int cc = 0; cc < nch; ++cc) {
      const float* pp = pbase + ((size_t)g * p.nchunk + cc) * (HD + 2);
      acc = fmaf(pp[2 + d], expf(pp[0] - m), acc);
    }
    p.out[(size_t)row * p.ldo + (kh * G + g) * HD + d] = acc / s_fl[g];
  }
}
