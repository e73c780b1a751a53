// attention.h -- causal attention of the new rows against the KV cache.
//
// Each row attends to every cached position of its sequence up to and including its
// own ("bare-metal-llm", "What got built": KV-cached causal attention; "rvllm Metal
// backend", "What the kernels do": scores Q K^T, mask, softmax, probs V). Positions
// past the row are never read, so no -inf mask is materialised. Position p of a
// sequence lives in cache block table[p / B], slot p mod B (the paged layout of the
// same post); a contiguous cache is one block per sequence slot, addressed directly
// from the row's slot offset. Query heads h use KV head h / (Hq / Hkv)
// (grouped-query attention).
//
// Decomposition (split context): one workgroup per (row, KV head, chunk). A row's
// T = pos + 1 positions are cut into GD_ATT_NCH chunks of ceil(T / GD_ATT_NCH)
// positions, so the number of partials per row is fixed and their consumer can load
// all of them without first reading the row's position. Inside a chunk, groups of
// HD/4 lanes take one position per step (float4 of K and V per lane, all loads of a
// step issued before the arithmetic) with an online max-subtracted softmax; the
// groups are merged in LDS into one partial (max, sum, weighted V) per query head.
// Empty chunks (T < GD_ATT_NCH) write max = -inf, sum = 0. For a few rows at short
// contexts, k_attn_o instead scans each row's whole context and applies the output
// projection in the same launch (see there).
#pragma once
#include "common.h"

struct AttnParams {
  const float* q; int ldq;            // [M][ldq]; query head h at h*HD (post-RoPE)
  const float* kc; const float* vc;   // this layer's pools [nblk][Hkv][B][HD]
  const int* table; int max_blocks;   // [slots][max_blocks] (paged)
  int block_size, nblk;
  int Hq, Hkv;
  const int* row_seq; const int* row_pos;
  const long long* row_kvoff;         // contiguous: the row's own slot offset
  int M;
  float scale;
  float* part;                        // [M][Hq][GD_ATT_NCH][HD + 2]: max, sum, o[HD]
};

// Online softmax of the G query heads of KV head kh of `row` over positions [p0, p1):
// groups of HD/4 lanes take one position per step (float4 of K and V per lane, all
// loads of a step issued before the arithmetic), each keeping a running max, sum and
// weighted V per query head; the groups are then merged in LDS. On return (after a
// barrier) thread tid < G * HD holds, for query head g = tid / HD and dimension
// d = tid % HD, the range's max, sum and weighted V (max -inf and zeros for an empty
// range).
template <int HD, int G, int PPG>
struct AttnScanLds {
  static constexpr int LG = HD / 4, NG = GD_WG / LG;
  float m[NG][G], l[NG][G];
  __align__(16) float o[NG][G][HD];
};

template <int HD, int G, int PPG, bool PAGED>
__device__ void attn_scan(const AttnParams& p, int row, int kh, int p0, int p1, AttnScanLds<HD, G, PPG>& sh,
                          float& m_out, float& l_out, float& o_out) {
  constexpr int LG = HD / 4;            // lanes per position group
  constexpr int NG = GD_WG / LG;        // position groups per workgroup
  constexpr int STEP = NG * PPG;        // positions per step
  const int tid = threadIdx.x;
  const int grp = tid / LG, gl = tid % LG;
  const int pos = p.row_pos[row];

  f32x4 q[G];
#pragma unroll
  for (int g = 0; g < G; ++g)
    q[g] = *reinterpret_cast<const f32x4*>(p.q + (size_t)row * p.ldq + (kh * G + g) * HD + gl * 4);
  const float* kbase = nullptr;
  const float* vbase = nullptr;
  const int* tab = nullptr;
  if (PAGED) {
    tab = p.table + (size_t)p.row_seq[row] * p.max_blocks;
  } else {
    const long long base = p.row_kvoff[row] - (long long)pos * HD + (long long)kh * p.block_size * HD;
    kbase = p.kc + base + gl * 4;
    vbase = p.vc + base + gl * 4;
  }

  float mx[G], l[G];
  f32x4 o[G];
#pragma unroll
  for (int g = 0; g < G; ++g) { mx[g] = -INFINITY; l[g] = 0.f; o[g] = (f32x4){0.f, 0.f, 0.f, 0.f}; }

  for (int s0 = p0; s0 < p1; s0 += STEP) {
    f32x4 kv[PPG], vv[PPG];
    bool ok[PPG];
#pragma unroll
    for (int j = 0; j < PPG; ++j) {
      const int ps = s0 + grp + NG * j;
      ok[j] = false;
      kv[j] = vv[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
      if (ps < p1) {
        if (PAGED) {
          const int bi = ps / p.block_size;
          const int blk = tab[bi];
          if ((unsigned)blk < (unsigned)p.nblk) {
            const size_t off = (((size_t)blk * p.Hkv + kh) * p.block_size + (ps - bi * p.block_size)) * HD + gl * 4;
            kv[j] = *reinterpret_cast<const f32x4*>(p.kc + off);
            vv[j] = *reinterpret_cast<const f32x4*>(p.vc + off);
            ok[j] = true;
          }
        } else {
          kv[j] = *reinterpret_cast<const f32x4*>(kbase + (size_t)ps * HD);
          vv[j] = *reinterpret_cast<const f32x4*>(vbase + (size_t)ps * HD);
          ok[j] = true;
        }
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float s[PPG];
      float smax = -INFINITY;
#pragma unroll
      for (int j = 0; j < PPG; ++j) {
        float d = q[g].x * kv[j].x;
        d = fmaf(q[g].y, kv[j].y, d);
        d = fmaf(q[g].z, kv[j].z, d);
        d = fmaf(q[g].w, kv[j].w, d);
        s[j] = group_sum<LG>(d) * p.scale;
        if (ok[j]) smax = fmaxf(smax, s[j]);
      }
      if (smax == -INFINITY) continue;   // this group saw no position in this step
      const float nm = fmaxf(mx[g], smax);
      const float sc = expf(mx[g] - nm);
      l[g] *= sc;
      o[g].x *= sc; o[g].y *= sc; o[g].z *= sc; o[g].w *= sc;
#pragma unroll
      for (int j = 0; j < PPG; ++j) {
        if (ok[j]) {
          const float e = expf(s[j] - nm);
          l[g] += e;
          o[g].x = fmaf(e, vv[j].x, o[g].x);
          o[g].y = fmaf(e, vv[j].y, o[g].y);
          o[g].z = fmaf(e, vv[j].z, o[g].z);
          o[g].w = fmaf(e, vv[j].w, o[g].w);
        }
      }
      mx[g] = nm;
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (gl == 0) { sh.m[grp][g] = mx[g]; sh.l[grp][g] = l[g]; }
    *reinterpret_cast<f32x4*>(&sh.o[grp][g][gl * 4]) = o[g];
  }
  __syncthreads();
  // merge the NG groups: one thread per (query head g, dim d)
  m_out = -INFINITY;
  l_out = o_out = 0.f;
  if (tid < G * HD) {
    const int g = tid / HD, d = tid % HD;
    float m = -INFINITY;
    for (int i = 0; i < NG; ++i) m = fmaxf(m, sh.m[i][g]);
    float ls = 0.f, acc = 0.f;
    if (m != -INFINITY) {
      for (int i = 0; i < NG; ++i) {
        if (sh.l[i][g] == 0.f) continue;   // group saw no position
        const float w = expf(sh.m[i][g] - m);
        ls = fmaf(sh.l[i][g], w, ls);
        acc = fmaf(sh.o[i][g][d], w, acc);
      }
    }
    m_out = m;
    l_out = ls;
    o_out = acc;
  }
}

template <int HD, int G, int PPG, bool PAGED>
__global__ __launch_bounds__(GD_WG) void k_attention(AttnParams p) {
  __shared__ AttnScanLds<HD, G, PPG> sh;
  const int c = blockIdx.x, kh = blockIdx.y, row = blockIdx.z;
  const int T = p.row_pos[row] + 1;
  const int L = (T + GD_ATT_NCH - 1) / GD_ATT_NCH;
  const int p0 = min(T, c * L), p1 = min(T, p0 + L);
  float m, l, o;
  attn_scan<HD, G, PPG, PAGED>(p, row, kh, p0, p1, sh, m, l, o);
  if (threadIdx.x < G * HD) {
    const int g = threadIdx.x / HD, d = threadIdx.x % HD;
    float* pp = p.part + (((size_t)row * p.Hq + kh * G + g) * GD_ATT_NCH + c) * (HD + 2);
    pp[2 + d] = o;
    if (d == 0) { pp[0] = m; pp[1] = l; }
  }
}

// Attention fused with the output projection, for a few rows at short contexts.
// Workgroup (slice s, KV head kh, row) scans the whole context of its G query heads
// (the attention is recomputed by every slice of the head: at short contexts its K/V
// come from cache), normalizes them, and adds their share of the projection,
// sum over g, d of o[g][d] W[n][(kh G + g) HD + d], to the residual rows n of its
// slice with float atomics (the bias from kh == 0). A slice is ROWS consecutive n; its
// weights (HD/4 lanes per row, float4 or four bf16 each) are loaded before the scan.
struct AttnOParams {
  const void* w;          // W_o [N][K] (K = Hq * HD), fp32 or bf16 bits
  const float* bias;      // never NULL
  float* y; int ldy;      // residual rows, updated in place
  int N, K;
};

template <int HD>
struct AttnORows { static constexpr int LG = HD / 4, PER_PASS = GD_WG / LG, PASSES = HD == 64 ? 3 : 1,
                   ROWS = PER_PASS * PASSES; };

template <int HD, int G, int PPG, bool PAGED, int WT>
__global__ __launch_bounds__(GD_WG) void k_attn_o(AttnParams p, AttnOParams po) {
  using RT = AttnORows<HD>;
  __shared__ AttnScanLds<HD, G, PPG> sh;
  __shared__ __align__(16) float s_o[G][HD];
  const int kh = blockIdx.y, row = blockIdx.z;
  const int tid = threadIdx.x, grp = tid / RT::LG, gl = tid % RT::LG;
  const int n0 = blockIdx.x * RT::ROWS;
  // the slice's weights first: they depend on nothing
  f32x4 wv[RT::PASSES][G];
#pragma unroll
  for (int ps = 0; ps < RT::PASSES; ++ps) {
    const int n = min(n0 + ps * RT::PER_PASS + grp, po.N - 1);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const size_t off = (size_t)n * po.K + (kh * G + g) * HD + gl * 4;
      if constexpr (WT == 0) {
        wv[ps][g] = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(po.w) + off);
      } else {
        const uint2 u = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(po.w) + off);
        wv[ps][g] = (f32x4){bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y)};
      }
    }
  }
  const int T = p.row_pos[row] + 1;
  float m, l, o;
  attn_scan<HD, G, PPG, PAGED>(p, row, kh, 0, T, sh, m, l, o);
  if (tid < G * HD) s_o[tid / HD][tid % HD] = l > 0.f ? o / l : 0.f;
  __syncthreads();
#pragma unroll
  for (int ps = 0; ps < RT::PASSES; ++ps) {
    const int n = n0 + ps * RT::PER_PASS + grp;
    float acc = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const f32x4 ov = *reinterpret_cast<const f32x4*>(&s_o[g][gl * 4]);
      acc = fmaf(wv[ps][g].x, ov.x, acc);
      acc = fmaf(wv[ps][g].y, ov.y, acc);
      acc = fmaf(wv[ps][g].z, ov.z, acc);
      acc = fmaf(wv[ps][g].w, ov.w, acc);
    }
    acc = group_sum<RT::LG>(acc);
    if (gl == 0 && n < po.N)
      __hip_atomic_fetch_add(po.y + (size_t)row * po.ldy + n, acc + (kh == 0 ? po.bias[n] : 0.f), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Merge of the chunk partials of M rows x Hq heads into dst[m * ldd + h * hd + d]:
// o = sum_c e^(max_c - max) o_c / sum_c e^(max_c - max) sum_c. Chunk 0 always holds at
// least one position, so the maximum is finite; empty chunks (max -inf, sum 0, o 0)
// get weight 0. attn_merge_issue loads each thread's partial outputs of its first EPT
// elements and the (max, sum) of its first (row, head, chunk) entry; a caller issues it
// before unrelated loads (vector loads complete in issue order) and runs
// attn_merge_finish later, so the merge costs one memory round trip. The chunk
// weights of each (row, head) are formed by 8 adjacent lanes and shared through LDS
// (s_w: M * Hq * GD_ATT_NCH floats). Called by the whole workgroup (nthr threads, a
// multiple of 64).
template <int EPT>
struct MergeRegs {
  float oc[EPT][GD_ATT_NCH];
  float mc, lc;
};

template <int EPT>
__device__ __forceinline__ void attn_merge_issue(const float* __restrict__ apart, int Hq, int hd, int M,
                                                 MergeRegs<EPT>& r, int nthr) {
  static_assert(GD_ATT_NCH == 8, "one chunk per lane of an 8-lane group");
  const int tid = threadIdx.x, K = Hq * hd, stride = hd + 2;
  const int total = M * K, npair = M * Hq * GD_ATT_NCH;
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int i = min(tid + nthr * j, total - 1);
    const int m = i / K, k = i - m * K;
    const int h = k / hd, d = k - h * hd;
    const float* pp = apart + ((size_t)m * Hq + h) * GD_ATT_NCH * stride + 2 + d;
#pragma unroll
    for (int c = 0; c < GD_ATT_NCH; ++c) r.oc[j][c] = pp[(size_t)c * stride];
  }
  const float* pp = apart + (size_t)min(tid, npair - 1) * stride;   // entry (m, h, c) = tid
  r.mc = pp[0];
  r.lc = pp[1];
}

template <int EPT>
__device__ void attn_merge_finish(const float* __restrict__ apart, int Hq, int hd, int M, const MergeRegs<EPT>& r,
                                  float* dst, int ldd, float* s_w, int nthr) {
  const int tid = threadIdx.x, K = Hq * hd, stride = hd + 2;
  const int total = M * K, npair = M * Hq * GD_ATT_NCH;
  for (int q0 = 0; q0 < npair; q0 += nthr) {   // npair is a multiple of 8: groups never straddle
    float mc = r.mc, lc = r.lc;
    if (q0 > 0) {
      const float* pp = apart + (size_t)min(q0 + tid, npair - 1) * stride;
      mc = pp[0];
      lc = pp[1];
    }
    const float mx = group_max<GD_ATT_NCH>(mc);
    const float e = expf(mc - mx);
    const float l = group_sum<GD_ATT_NCH>(lc * e);
    if (q0 + tid < npair) s_w[q0 + tid] = e / l;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int i = tid + nthr * j;
    if (i < total) {
      const int m = i / K, k = i - m * K;
      const float* w = s_w + ((size_t)m * Hq + k / hd) * GD_ATT_NCH;
      float o = 0.f;
#pragma unroll
      for (int c = 0; c < GD_ATT_NCH; ++c) o = fmaf(w[c], r.oc[j][c], o);
      dst[(size_t)m * ldd + k] = o;
    }
  }
  for (int i = tid + nthr * EPT; i < total; i += nthr) {   // elements beyond the register share
    const int m = i / K, k = i - m * K;
    const int h = k / hd, d = k - h * hd;
    const float* pp = apart + ((size_t)m * Hq + h) * GD_ATT_NCH * stride + 2 + d;
    const float* w = s_w + ((size_t)m * Hq + h) * GD_ATT_NCH;
    float o = 0.f;
#pragma unroll
    for (int c = 0; c < GD_ATT_NCH; ++c) o = fmaf(w[c], pp[(size_t)c * stride], o);
    dst[(size_t)m * ldd + k] = o;
  }
}

template <int EPT>
__device__ void attn_merge_rows(const float* __restrict__ apart, int Hq, int hd, int M, float* dst, int ldd,
                                float* s_w, int nthr) {
  MergeRegs<EPT> r;
  attn_merge_issue<EPT>(apart, Hq, hd, M, r, nthr);
  attn_merge_finish<EPT>(apart, Hq, hd, M, r, dst, ldd, s_w, nthr);
}

// Merge of the chunk partials into o[M][Hq*HD] (rows handled by the matrix-core
// kernel): one workgroup per row.
__global__ __launch_bounds__(GD_WG) void k_attn_merge(const float* __restrict__ part, int Hq, int hd, float* out,
                                                      int ldo) {
  __shared__ float s_w[GD_MAX_HEADS * GD_ATT_NCH];
  const int m = blockIdx.x;
  attn_merge_rows<4>(part + (size_t)m * Hq * GD_ATT_NCH * (hd + 2), Hq, hd, 1, out + (size_t)m * ldo, ldo, s_w,
                     GD_WG);
}
