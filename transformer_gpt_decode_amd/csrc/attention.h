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
// T = pos + 1 positions are cut into C chunks of ceil(T / C) positions (C = 1, GD_ATT_NCH or GD_ATT_NCH_LONG)
// (C = the grid's x extent), so the number of partials per row is fixed and their
// consumer can load all of them without first reading the row's position. Inside a
// chunk, groups of HD/4 lanes take one position per step (float4 of K and V per lane,
// all loads of a step issued before the arithmetic; with a contiguous cache the next
// step's loads are issued before the current step's arithmetic) with an online
// max-subtracted softmax; the groups are merged into one partial (max, sum, weighted V)
// per query head. Empty chunks (T < C) write max = -inf, sum = 0. With one chunk per
// row (enough rows and heads to fill the GPU) the kernel writes the normalized output
// itself and no merge follows. For a few rows at short contexts, k_attn_o instead scans
// each row's whole context and applies the output projection in the same launch (see
// there).
#pragma once
#include "common.h"

struct AttnParams {
  const float* q; int ldq;            // [M][ldq]; query head h at h*HD (post-RoPE)
  const void* kc; const void* vc;     // this layer's pools [nblk][Hkv][B][HD]: float, or bf16 bits
  const int* table; int max_blocks;   // [slots][max_blocks] (paged)
  int block_size, nblk;
  int Hq, Hkv;
  const int* row_seq; const int* row_pos;
  const long long* row_kvoff;         // contiguous: the row's own slot offset
  int M;
  float scale;
  float* part;                        // [M][Hq][C][gd_apart_stride(HD)]: max, sum, -, -, o[HD] (C chunks per row)
  float* out; int ldo;                // one chunk per row: the normalized output [M][ldo]
};

// Online softmax of the G query heads of KV head kh of `row` over positions [p0, p1):
// groups of HD/4 lanes take one position per step (float4 of K and V per lane, all
// loads of a step issued before the arithmetic), each keeping a running max, sum and
// weighted V per query head. The groups of a wave are then merged with cross-lane
// exchanges and the waves through LDS. On return (after a barrier) thread
// tid < G * HD holds, for query head g = tid / HD and dimension d = tid % HD, the
// range's max, sum and weighted V (max -inf and zeros for an empty range).
// A paged scan stages the block-table entries of its range in LDS, GD_ATT_TABN blocks
// (a segment of the range) at a time.
#define GD_ATT_TABN 256
template <int HD, int G, int PPG, int NT = GD_WG>
struct AttnScanLds {
  static constexpr int NW = NT / 64;
  float m[NW][G], l[NW][G];
  __align__(16) float o[NW][G][HD];
  int tab[GD_ATT_TABN];   // paged: cache blocks of the current segment
};

// This lane's query values (lanes gl of every position group: dims 4 gl .. 4 gl + 3
// of each query head of KV head kh).
template <int HD, int G>
__device__ __forceinline__ void attn_load_q(const AttnParams& p, int row, int kh, f32x4 (&q)[G]) {
  const int gl = threadIdx.x % (HD / 4);
#pragma unroll
  for (int g = 0; g < G; ++g)
    q[g] = *reinterpret_cast<const f32x4*>(p.q + (size_t)row * p.ldq + (kh * G + g) * HD + gl * 4);
}

// A row's metadata, read with scalar loads (row is uniform over the workgroup), so that
// waiting for them does not wait for vector loads issued earlier; the empty asm takes
// them all as operands, so they are issued together and waited for once.
struct AttnRow {
  int pos, seq;
  long long kvoff;
};

template <bool PAGED>
__device__ __forceinline__ AttnRow attn_row(const AttnParams& p, int row) {
  AttnRow r;
  r.pos = *(const __attribute__((address_space(4))) int*)(p.row_pos + row);
  r.seq = PAGED ? *(const __attribute__((address_space(4))) int*)(p.row_seq + row) : 0;
  r.kvoff = PAGED ? 0 : *(const __attribute__((address_space(4))) long long*)(p.row_kvoff + row);
  asm volatile("" ::"s"(r.pos), "s"(r.seq), "s"(r.kvoff));
  return r;
}

// The row of rank z among the launch's M (<= 64) rows in decreasing position order (ties
// to the lower index). Workgroups launched in rank order start the longest contexts
// first, so the shortest ones share CUs. Every wave ranks the rows itself from their
// positions (one load per lane); the result is uniform.
__device__ __forceinline__ int attn_row_by_rank(const AttnParams& p, int z) {
  const int lane = threadIdx.x & 63, M = p.M;
  const int pl = lane < M ? p.row_pos[lane] : -1;
  int rank = 0;
  for (int j = 0; j < M; ++j) {
    const int pj = __builtin_amdgcn_readlane(pl, j);
    rank += (pj > pl || (pj == pl && j < lane)) ? 1 : 0;
  }
  const unsigned long long b = __ballot(lane < M && rank == z);
  return __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(b));
}

// Weight of a partial with max m in a merge whose max is mm (0 when both are -inf).
__device__ __forceinline__ float attn_rescale(float m, float mm) { return mm == -INFINITY ? 0.f : expf(m - mm); }

// Four consecutive cache elements at element offset e, widened to float: a 16-byte
// load of a float cache or an 8-byte load of a bf16 cache (STREAM: non-temporal).
template <bool KV16, bool STREAM>
__device__ __forceinline__ f32x4 kv_load4(const void* base, size_t e) {
  if constexpr (KV16) {
    const uint2* p = reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(base) + e);
    uint2 u;
    if constexpr (STREAM) {
      u.x = __builtin_nontemporal_load(&p->x);
      u.y = __builtin_nontemporal_load(&p->y);
    } else {
      u = *p;
    }
    return (f32x4){bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y)};
  } else {
    const f32x4* p = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(base) + e);
    if constexpr (STREAM) return __builtin_nontemporal_load(p);
    return *p;
  }
}

// Loads are unconditional (a position past the range is clamped to its last position,
// an invalid cache block to block 0) and masked afterwards, so that the compiler keeps
// them where they are issued instead of sinking them into branches.
// Both caches run the same two-deep pipeline of steps. A paged range is scanned in
// segments of at most GD_ATT_TABN cache blocks whose block-table entries are first
// staged in LDS (one memory round trip per segment), so that a step's K/V addresses
// come from LDS and the next step's loads can be in flight while one is consumed.
// STREAM: each K/V element is read by one workgroup of the launch, so the contiguous
// loads carry the non-temporal hint (they then displace less of what other workgroups
// share in L2: the output projection's weights, the query rows).
template <int HD, int G, int PPG, bool PAGED, bool KV16, int NT = GD_WG, bool STREAM = false>
__device__ void attn_scan(const AttnParams& p, const AttnRow& rm, int kh, int p0, int p1, const f32x4 (&q)[G],
                          AttnScanLds<HD, G, PPG, NT>& sh, float& m_out, float& l_out, float& o_out) {
  constexpr int LG = HD / 4;            // lanes per position group
  constexpr int NG = NT / LG;           // position groups per workgroup
  constexpr int STEP = NG * PPG;        // positions per step
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x;
  const int grp = tid / LG, gl = tid % LG;
  const int pos = rm.pos;

  size_t cbase = 0;   // contiguous: element offset of position 0 of this head (+ this lane's 4)
  const int* tab = nullptr;
  int tb0 = 0;        // paged: first block of the current segment (sh.tab[0])
  if (PAGED) {
    tab = p.table + (size_t)rm.seq * p.max_blocks;
  } else {
    cbase = (size_t)(rm.kvoff - (long long)pos * HD + (long long)kh * p.block_size * HD) + gl * 4;
  }

  float mx[G], l[G];
  f32x4 o[G];
#pragma unroll
  for (int g = 0; g < G; ++g) { mx[g] = -INFINITY; l[g] = 0.f; o[g] = (f32x4){0.f, 0.f, 0.f, 0.f}; }

  f32x4 kv[PPG], vv[PPG], kv2[PPG], vv2[PPG];
  bool ok[PPG], ok2[PPG];
  auto issue = [&](int s0, int pe, f32x4 (&kv)[PPG], f32x4 (&vv)[PPG], bool (&ok)[PPG]) {
#pragma unroll
    for (int j = 0; j < PPG; ++j) {
      const int pr = s0 + grp + NG * j;
      const int ps = min(pr, pe - 1);
      ok[j] = pr < pe;
      size_t off;
      if (PAGED) {
        const int bi = ps / p.block_size;
        const int blk = sh.tab[bi - tb0];
        const bool valid = (unsigned)blk < (unsigned)p.nblk;
        ok[j] = ok[j] && valid;
        off = (((size_t)(valid ? blk : 0) * p.Hkv + kh) * p.block_size + (ps - bi * p.block_size)) * HD + gl * 4;
        kv[j] = kv_load4<KV16, false>(p.kc, off);
        vv[j] = kv_load4<KV16, false>(p.vc, off);
      } else {
        kv[j] = kv_load4<KV16, STREAM>(p.kc, cbase + (size_t)ps * HD);
        vv[j] = kv_load4<KV16, STREAM>(p.vc, cbase + (size_t)ps * HD);
      }
    }
    __builtin_amdgcn_sched_barrier(0);   // all of this step's loads go out before any arithmetic
  };
  auto consume = [&](const f32x4 (&kv)[PPG], const f32x4 (&vv)[PPG], const bool (&ok)[PPG]) {
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
        // computed for every position and masked after: a conditional here would let
        // the compiler sink the K load into the branch, behind later loads
        const float sj = group_sum<LG>(d) * p.scale;
        s[j] = ok[j] ? sj : -INFINITY;
        smax = fmaxf(smax, s[j]);
      }
      const float nm = fmaxf(mx[g], smax);   // -inf only if this group has seen no position yet
      const float sc = attn_rescale(mx[g], nm);
      l[g] *= sc;
      o[g].x *= sc; o[g].y *= sc; o[g].z *= sc; o[g].w *= sc;
#pragma unroll
      for (int j = 0; j < PPG; ++j) {
        const float ej = expf(s[j] - nm);
        const float e = ok[j] ? ej : 0.f;
        l[g] += e;
        o[g].x = fmaf(e, vv[j].x, o[g].x);
        o[g].y = fmaf(e, vv[j].y, o[g].y);
        o[g].z = fmaf(e, vv[j].z, o[g].z);
        o[g].w = fmaf(e, vv[j].w, o[g].w);
      }
      mx[g] = nm;
    }
  };
  // Two register sets: step i + 1 is in flight while step i is consumed (the wait
  // before a consume covers only the older set: loads complete in issue order). Every
  // path into the loop head has exactly the newer set in flight (an issue or exit
  // between the halves would make the compiler wait for every load there); the last
  // one or two steps are peeled off below the loop, so no load is issued past the range.
  auto scan_range = [&](int a, int b) {
    const int n = (b - a + STEP - 1) / STEP;
    issue(a, b, kv, vv, ok);
    int i = 0;
    for (; i + 2 < n; i += 2) {
      issue(a + (i + 1) * STEP, b, kv2, vv2, ok2);
      consume(kv, vv, ok);
      issue(a + (i + 2) * STEP, b, kv, vv, ok);
      consume(kv2, vv2, ok2);
    }
    if (i + 1 < n) {
      issue(a + (i + 1) * STEP, b, kv2, vv2, ok2);
      // passing the older set through empty asm makes this branch's arithmetic differ
      // from the other's, which the compiler would otherwise hoist above the issue
#pragma unroll
      for (int j = 0; j < PPG; ++j) asm volatile("" : "+v"(kv[j]), "+v"(vv[j]));
      consume(kv, vv, ok);
      consume(kv2, vv2, ok2);
    } else {
      consume(kv, vv, ok);
    }
  };
  if constexpr (PAGED) {
    // segments of at most GD_ATT_TABN blocks (p0, p1 and the block size are uniform, so
    // every thread takes the same path through the barriers)
    const int bs = p.block_size;
    for (int a = p0; a < p1;) {
      tb0 = a / bs;
      const int b = min(p1, (tb0 + GD_ATT_TABN) * bs);
      const int nbk = (b - 1) / bs - tb0 + 1;
      if (a != p0) __syncthreads();   // the previous segment's entries have been read
      for (int k = tid; k < nbk; k += NT) sh.tab[k] = tab[tb0 + k];
      __syncthreads();
      scan_range(a, b);
      a = b;
    }
  } else if (p0 < p1) {
    scan_range(p0, p1);
  }
  // merge the groups of each wave (lanes gl + LG r) by exchanges between lanes
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int off = LG; off < 64; off <<= 1) {
      const float m2 = __shfl_xor(mx[g], off), l2 = __shfl_xor(l[g], off);
      f32x4 o2;
      o2.x = __shfl_xor(o[g].x, off); o2.y = __shfl_xor(o[g].y, off);
      o2.z = __shfl_xor(o[g].z, off); o2.w = __shfl_xor(o[g].w, off);
      const float mm = fmaxf(mx[g], m2);
      const float s1 = attn_rescale(mx[g], mm), s2 = attn_rescale(m2, mm);
      l[g] = fmaf(l[g], s1, l2 * s2);
      o[g].x = fmaf(o[g].x, s1, o2.x * s2); o[g].y = fmaf(o[g].y, s1, o2.y * s2);
      o[g].z = fmaf(o[g].z, s1, o2.z * s2); o[g].w = fmaf(o[g].w, s1, o2.w * s2);
      mx[g] = mm;
    }
  }
  const int wave = tid >> 6, lane = tid & 63;
  if (lane < LG) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (lane == 0) { sh.m[wave][g] = mx[g]; sh.l[wave][g] = l[g]; }
      *reinterpret_cast<f32x4*>(&sh.o[wave][g][lane * 4]) = o[g];
    }
  }
  __syncthreads();
  // merge the waves: one thread per (query head g, dim d)
  m_out = -INFINITY;
  l_out = o_out = 0.f;
  if (tid < G * HD) {
    const int g = tid / HD, d = tid % HD;
    float mw[NW];
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) { mw[w] = sh.m[w][g]; mm = fmaxf(mm, mw[w]); }
    float ls = 0.f, acc = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float s = attn_rescale(mw[w], mm);
      ls = fmaf(sh.l[w][g], s, ls);
      acc = fmaf(sh.o[w][g][d], s, acc);
    }
    m_out = mm;
    l_out = ls;
    o_out = acc;
  }
}

// NT threads: 512 for one chunk per row, so that a long context scanned by one
// workgroup keeps twice the positions in flight.
template <int HD, int G, int PPG, bool PAGED, int NT, bool KV16>
__global__ __launch_bounds__(NT) void k_attention(AttnParams p) {
  __shared__ AttnScanLds<HD, G, PPG, NT> sh;
  const int c = blockIdx.x, kh = blockIdx.y, row = blockIdx.z;
  const AttnRow rm = attn_row<PAGED>(p, row);
  f32x4 q[G];
  attn_load_q<HD, G>(p, row, kh, q);
  const int T = rm.pos + 1, C = gridDim.x;
  const int L = (T + C - 1) / C;
  const int p0 = min(T, c * L), p1 = min(T, p0 + L);
  float m, l, o;
  attn_scan<HD, G, PPG, PAGED, KV16, NT, true>(p, rm, kh, p0, p1, q, sh, m, l, o);
  if (threadIdx.x < G * HD) {
    const int g = threadIdx.x / HD, d = threadIdx.x % HD;
    if (C == 1) {   // the whole context: l > 0 (the row's own position is in it)
      p.out[(size_t)row * p.ldo + (kh * G + g) * HD + d] = o / l;
    } else {
      float* pp = p.part + (((size_t)row * p.Hq + kh * G + g) * C + c) * gd_apart_stride(HD);
      pp[GD_APART_O + d] = o;
      if (d == 0) { pp[0] = m; pp[1] = l; }
    }
  }
}

// Attention fused with the output projection, for a few rows at short contexts.
// Workgroup (slice s, KV head kh, row) scans the whole context of its G query heads
// (the attention is recomputed by every slice of the head: at short contexts its K/V
// come from cache), normalizes them, and adds their share of the projection,
// sum over g, d of o[g][d] W[n][(kh G + g) HD + d], to the residual rows n of its
// slice with float atomics (the bias from kh == 0). A slice is ROWS consecutive n; its
// weights (HD/4 lanes per row, float4 or four bf16 each) and bias are loaded first.
// The atomics of all passes go out together at the end, after the last wait (vector
// memory operations of a wave complete in issue order: an atomic issued before a later
// wait would be waited for).
struct AttnOParams {
  const void* w;          // W_o [N][K] (K = Hq * HD): fp32, bf16 bits, or int8 codes
  const float* wsc;       // int8 codes: block scales [N][K / 32]
  const float* bias;      // never NULL
  float* y; int ldy;      // residual rows, updated in place
  int N, K;
};

template <int HD>
struct AttnORows { static constexpr int LG = HD / 4, PER_PASS = GD_WG / LG, PASSES = HD == 64 ? 3 : 1,
                   ROWS = PER_PASS * PASSES; };

template <int HD, int G, int PPG, bool PAGED, int WT, bool KV16>
__global__ __launch_bounds__(GD_WG) __attribute__((amdgpu_waves_per_eu(1, 2))) void k_attn_o(AttnParams p, AttnOParams po) {
  using RT = AttnORows<HD>;
  __shared__ AttnScanLds<HD, G, PPG> sh;
  __shared__ __align__(16) float s_o[G][HD];
  // Workgroups are placed round-robin over the 8 XCDs in launch order, and the slices
  // of one (KV head, row) read the same K/V: launch index L is renumbered so that
  // consecutive slices share an XCD and its L2 (the K/V then come from HBM about once
  // rather than once per XCD). L = 8 k + x with x < 8 becomes j = x per + k for the
  // first 8 per indices (per = total / 8); the remainder keeps its index.
  const int S = gridDim.x, total = S * gridDim.y * gridDim.z;
  const int L = blockIdx.x + S * (blockIdx.y + gridDim.y * blockIdx.z);
  const int per = total >> 3;
  const int j = L < 8 * per ? (L & 7) * per + (L >> 3) : L;
  const int slice = j % S, kh = (j / S) % gridDim.y, row = j / (S * gridDim.y);
  const int tid = threadIdx.x, grp = tid / RT::LG, gl = tid % RT::LG;
  const int n0 = slice * RT::ROWS;
  // Every kernel argument the launch reads, loaded at once: left to itself the compiler
  // loads each just before its first use, a chain of scalar round trips ahead of the
  // metadata, query and K/V loads.
  asm volatile("" ::"s"(p.q), "s"(p.kc), "s"(p.vc), "s"(p.row_pos), "s"(p.row_kvoff), "s"(p.row_seq), "s"(p.table),
               "s"(po.w), "s"(po.bias), "s"(po.y), "s"(p.ldq), "s"(p.max_blocks), "s"(p.block_size), "s"(p.nblk),
               "s"(p.Hkv), "s"(p.scale), "s"(po.ldy), "s"(po.N), "s"(po.K));
  // Then, in this order: the slice's weights and bias (vector loads that depend on
  // nothing), the row's metadata (scalar loads, waited for at once), the query and the
  // K/V loads. Vector loads complete in issue order, so the weights, needed last,
  // arrive first and the wait for the K/V covers them at no cost.
  f32x4 wv[RT::PASSES][G];
  float bv[RT::PASSES];
#pragma unroll
  for (int ps = 0; ps < RT::PASSES; ++ps) {
    const int n = min(n0 + ps * RT::PER_PASS + grp, po.N - 1);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const size_t off = (size_t)n * po.K + (kh * G + g) * HD + gl * 4;
      if constexpr (WT == 0) {
        wv[ps][g] = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(po.w) + off);
      } else if constexpr (WT == 1) {
        const uint2 u = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(po.w) + off);
        wv[ps][g] = (f32x4){bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y)};
      } else {
        const uint32_t u = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const int8_t*>(po.w) + off);
        wv[ps][g] = q8x4(u, po.wsc[off >> 5]);
      }
    }
    bv[ps] = po.bias[n];
  }
  const AttnRow rm = attn_row<PAGED>(p, row);
  f32x4 q[G];
  attn_load_q<HD, G>(p, row, kh, q);
  float m, l, o;
  attn_scan<HD, G, PPG, PAGED, KV16>(p, rm, kh, 0, rm.pos + 1, q, sh, m, l, o);
  if (tid < G * HD) s_o[tid / HD][tid % HD] = l > 0.f ? o / l : 0.f;
  __syncthreads();
  float acc[RT::PASSES];
#pragma unroll
  for (int ps = 0; ps < RT::PASSES; ++ps) {
    float a = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const f32x4 ov = *reinterpret_cast<const f32x4*>(&s_o[g][gl * 4]);
      a = fmaf(wv[ps][g].x, ov.x, a);
      a = fmaf(wv[ps][g].y, ov.y, a);
      a = fmaf(wv[ps][g].z, ov.z, a);
      a = fmaf(wv[ps][g].w, ov.w, a);
    }
    acc[ps] = group_sum<RT::LG>(a) + (kh == 0 ? bv[ps] : 0.f);
  }
  // every sum complete before the first atomic (the empty asm takes them as operands):
  // a wait placed after an atomic would wait for that atomic too
#pragma unroll
  for (int ps = 0; ps < RT::PASSES; ++ps) asm volatile("" ::"v"(acc[ps]));
#pragma unroll
  for (int ps = 0; ps < RT::PASSES; ++ps) {
    const int n = n0 + ps * RT::PER_PASS + grp;
    if (gl == 0 && n < po.N)
      __hip_atomic_fetch_add(po.y + (size_t)row * po.ldy + n, acc[ps], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Attention of one whole context per workgroup fused with the output projection, for
// many rows (rows x KV heads fill the GPU): workgroup (KV head kh, rank z) takes the row
// with the z-th longest context (attn_row_by_rank), scans that context (as k_attention
// with one chunk), normalizes o, and adds o . W_o[n][kh HD ..]
// for every output n (plus the bias from kh == 0) to the residual row with float
// atomics: Hkv contributions per address. Against the split-context kernel followed by
// a matrix-core projection launch it costs each workgroup its head's W_o columns
// (N x HD, from L2 after the first workgroup of the head) and one extra round trip,
// and saves the projection launch. One query head per KV head (G = 1); the projection
// reads its weights in groups of HD/4 lanes per output (float4 or four bf16 each), NP
// passes of NT / (HD/4) outputs, all issued at once after the scan; the sums go
// through LDS so that every atomic is issued after the last wait.
template <int HD, bool PAGED, int WT, int NT, int NP, bool KV16>
__global__ __launch_bounds__(NT) void k_attn_proj(AttnParams p, AttnOParams po) {
  // 4 positions per lane group and load round: 8 (fewer rounds for the longest rows)
  // measured 7 % slower at batch 32, the extra registers halving the resident workgroups
  constexpr int PPG = 4, LG = HD / 4, RPP = NT / LG;
  static_assert(HD == 64, "head_dim 64");
  static_assert(NP * RPP <= 2 * NT, "two outputs per thread at most");
  __shared__ AttnScanLds<HD, 1, PPG, NT> sh;
  __shared__ __align__(16) float s_o[HD];
  __shared__ float s_acc[NP * RPP];
  const int kh = blockIdx.y, tid = threadIdx.x;
  const int grp = tid / LG, gl = tid % LG;
  asm volatile("" ::"s"(p.q), "s"(p.kc), "s"(p.vc), "s"(p.row_pos), "s"(p.row_kvoff), "s"(p.row_seq), "s"(p.table),
               "s"(po.w), "s"(po.bias), "s"(po.y), "s"(p.ldq), "s"(p.max_blocks), "s"(p.block_size), "s"(p.nblk),
               "s"(p.Hkv), "s"(p.scale), "s"(po.ldy), "s"(po.N), "s"(po.K));
  // rows in decreasing context length: 7 % less time at batch 32 than launch order
  const int row = attn_row_by_rank(p, blockIdx.z);
  // the bias (added by kh == 0) of this thread's two outputs tid, tid + NT (N <= 2 NT)
  float bq[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) bq[j] = kh == 0 ? po.bias[min(tid + NT * j, po.N - 1)] : 0.f;
  const AttnRow rm = attn_row<PAGED>(p, row);
  f32x4 q[1];
  attn_load_q<HD, 1>(p, row, kh, q);
  float m, l, o;
  attn_scan<HD, 1, PPG, PAGED, KV16, NT, true>(p, rm, kh, 0, rm.pos + 1, q, sh, m, l, o);
  if (tid < HD) s_o[tid] = o / l;   // l > 0: the row's own position is in its context
  // this head's weight columns, every pass at once (clamped rows past N are never added)
  f32x4 wv[NP];
#pragma unroll
  for (int ps = 0; ps < NP; ++ps) {
    const int n = min(ps * RPP + grp, po.N - 1);
    const size_t off = (size_t)n * po.K + kh * HD + gl * 4;
    if constexpr (WT == 0) {
      wv[ps] = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(po.w) + off);
    } else {
      const uint2 u = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(po.w) + off);
      wv[ps] = (f32x4){bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y)};
    }
  }
  __syncthreads();
  const f32x4 ov = *reinterpret_cast<const f32x4*>(&s_o[gl * 4]);
#pragma unroll
  for (int ps = 0; ps < NP; ++ps) {
    float a = wv[ps].x * ov.x;
    a = fmaf(wv[ps].y, ov.y, a);
    a = fmaf(wv[ps].z, ov.z, a);
    a = fmaf(wv[ps].w, ov.w, a);
    a = group_sum<LG>(a);
    if (gl == 0) s_acc[ps * RPP + grp] = a;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = tid + NT * j;
    if (n < po.N)
      __hip_atomic_fetch_add(po.y + (size_t)row * po.ldy + n, s_acc[n] + bq[j], __ATOMIC_RELAXED,
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
  const int tid = threadIdx.x, K = Hq * hd, stride = gd_apart_stride(hd);
  const int total = M * K, npair = M * Hq * GD_ATT_NCH;
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int i = min(tid + nthr * j, total - 1);
    const int m = i / K, k = i - m * K;
    const int h = k / hd, d = k - h * hd;
    const float* pp = apart + ((size_t)m * Hq + h) * GD_ATT_NCH * stride + GD_APART_O + d;
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
  const int tid = threadIdx.x, K = Hq * hd, stride = gd_apart_stride(hd);
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
    const float* pp = apart + ((size_t)m * Hq + h) * GD_ATT_NCH * stride + GD_APART_O + d;
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

// Merge of C <= GD_ATT_NCH_LONG chunk partials (the long-context split) into
// o[M][Hq*HD]: one wave per (query head, row). Every load is issued at once (indices
// clamped to the last chunk, extra chunks weighted 0), so the merge costs one memory
// round trip: lane c takes chunk c's (max, sum), lane d the C values of dimension d;
// the chunk weights e^(max_c - max) are shared by lane exchanges. Empty chunks (max
// -inf) weigh 0; chunk 0 holds position 0, so max is finite.
__global__ __launch_bounds__(64) void k_attn_merge_n(const float* part, int Hq, int hd, int C, float* out, int ldo) {
  const int h = blockIdx.x, m = blockIdx.y, lane = threadIdx.x;
  const int stride = gd_apart_stride(hd), d = min(lane, hd - 1);
  const float* pp = part + ((size_t)m * Hq + h) * C * stride;
  const float2 ml = *reinterpret_cast<const float2*>(pp + (size_t)min(lane, C - 1) * stride);
  float ov[GD_ATT_NCH_LONG];
#pragma unroll
  for (int c = 0; c < GD_ATT_NCH_LONG; ++c) ov[c] = pp[(size_t)min(c, C - 1) * stride + GD_APART_O + d];
  // keeps the loads above where they are (the pointers are not restrict-qualified, so
  // the clobber binds them): left alone, the compiler moves the value loads below the
  // reductions, after a wait for the (max, sum) pairs (two round trips)
  asm volatile("" ::: "memory");
  const float mc = lane < C ? ml.x : -INFINITY;
  const float mx = wave_max(mc);
  const float w = attn_rescale(mc, mx);   // 0 for lanes >= C
  const float l = wave_sum((lane < C ? ml.y : 0.f) * w);
  float o = 0.f;
#pragma unroll
  for (int c = 0; c < GD_ATT_NCH_LONG; ++c) o = fmaf(__shfl(w, c), ov[c], o);
  if (lane < hd) out[(size_t)m * ldo + h * hd + lane] = o / l;
}

// Merge of the chunk partials into o[M][Hq*HD] (rows handled by the matrix-core
// kernel): one workgroup per row.
__global__ __launch_bounds__(GD_WG) void k_attn_merge(const float* __restrict__ part, int Hq, int hd, float* out,
                                                      int ldo) {
  __shared__ float s_w[GD_MAX_HEADS * GD_ATT_NCH];
  const int m = blockIdx.x;
  attn_merge_rows<4>(part + (size_t)m * Hq * GD_ATT_NCH * gd_apart_stride(hd), Hq, hd, 1, out + (size_t)m * ldo, ldo, s_w,
                     GD_WG);
}
