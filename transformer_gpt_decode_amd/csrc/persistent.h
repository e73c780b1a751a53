// persistent.h -- the whole decode step of one sequence in one launch (GPT-2 layout).
//
// A graph-replayed step pays a fixed cost at every kernel boundary (dispatch, first
// loads, completion), and a batch-1 step is a chain of dependent linear layers whose
// weights stream in a few microseconds each, so that cost dominates it. Here one
// workgroup per CU runs every phase of the step (per layer: QKV, attention, output
// projection, MLP up, MLP down; then the head and the greedy argmax).
//
// Hand-over between phases: every output of a phase is a 64-bit word (value bits |
// step tag) written with a relaxed device-scope atomic store and polled with relaxed
// device-scope atomic loads. A word is current when it carries this step's tag, so
// no fence, counter or reset is needed; the tag is a kernel argument that the host
// advances every step, and every (layer, phase) has a region of its own, so no word
// is rewritten within a step. Outputs read by every workgroup are stored in 8
// replicas and workgroup i reads replica i % 8 (workgroups are placed round-robin
// over the 8 XCDs), which spreads the polling over the memory channels.
//
// Inside a workgroup, wave 0 only stages inputs: it polls, computes the norm
// statistics, merges the attention partials and writes the phase's input to LDS.
// Waves 1..8 issue the weight loads of the next phase as soon as they finish the
// current one and then wait at the workgroup barrier; vector loads of one wave
// complete in issue order, so a wave that streams weights could not also poll
// without waiting for its weights first. The LDS input is double-buffered by phase
// parity, so one barrier per phase suffices.
//
// Every wait is bounded: a wave-0 poll that exceeds spin_ticks of the 100 MHz
// real-time counter marks the step aborted (GD_DERR_SYNC, and the abort tag that the
// other workgroups' polls also watch), and all waves leave at the next barrier.
// Co-residency of all workgroups is guaranteed by the launch: one workgroup per CU,
// with an LDS request that no two workgroups fit into.
#pragma once
#include "linear.h"

#define PK_WG 512                  // threads: wave 0 stages, waves 1..7 compute (2 waves per SIMD)
#define PK_CW 7                    // compute waves
#define PK_NREP 8                  // replicas of the exchange words read by every workgroup
#define PK_LDS_BYTES (96 * 1024)   // dynamic LDS request: more than half of a CU's 160 KB
#define PK_ACH 256                 // attention positions per chunk (one workgroup each)
#define PK_MAXNCH 4                // chunks per head: contexts up to 1024 positions
#define PK_DMAX 1024               // d_model limit
#define PK_INMAX 3328              // staged input floats per buffer (ff, attention partials)
#define PK_MAXWG 256               // workgroups (CUs) at most
#define GD_DERR_SYNC 8

// Pointers of layer l: layer 0's plus l times a constant stride (bytes for weights,
// floats for the K/V pools), so no table is read inside the kernel.
struct PKLayer {
  const float* n1g; const float* n1b;
  const void* wqkv; const float* bqkv;
  const void* wo; const float* bo;
  const float* n2g; const float* n2b;
  const void* wfc; const float* bfc;
  const void* wproj; const float* bproj;
  float* kc; float* vc;                    // K and V pools
};

struct PKParams {
  PKLayer L0;                              // layer 0
  long long w_stride, kv_stride;           // per layer: bytes of weights, floats of each pool
  int n_layer, d, H, ff, vocab, qkv;
  float eps, scale;
  const void* wte; const void* wpe; const float* nfg; const float* nfb;
  // KV cache addressing: position p of the sequence is block table[p / block_size]
  int paged, kv0, hd;                      // contiguous: element offset of position 0
  const int* table; int max_blocks, bs_shift, nblk, kv_hstride;
  // the step
  int seq, pos, nch;                       // attended positions pos + 1 in nch chunks
  unsigned tag;
  long long spin_ticks;                    // bound of every wait (100 MHz ticks)
  const int* tok; int* next; float* logits; int* len; int* err;
  // exchange words (offsets in words)
  uint64_t* xb;
  unsigned* abort_tag;
  long long xl;                            // words per layer
  long long x_att, x_xo, x_h, x_xd;        // regions in a layer (QKV at 0, one replica)
  long long rs_att, rs_d, rs_h;            // replica strides of the replicated regions
  long long x_arg;                         // argmax partials (2 words per workgroup)
};

// Global-memory views of pointers read from memory: without them the compiler emits
// flat accesses, which also count against the LDS wait counter (and every barrier here
// waits for LDS operations only).
#define PK_GLOBAL __attribute__((address_space(1)))
template <class T>
__device__ __forceinline__ const PK_GLOBAL T* gp(const T* a) { return (const PK_GLOBAL T*)a; }
template <class T>
__device__ __forceinline__ PK_GLOBAL T* gpw(T* a) { return (PK_GLOBAL T*)a; }
template <class T>
__device__ __forceinline__ T* pk_adv(T* a, long long bytes) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(const_cast<void*>((const void*)a)) + bytes);
}
__device__ __forceinline__ PKLayer pk_layer(const PKParams& p, int l) {
  const long long wb = (long long)l * p.w_stride, kb = (long long)l * p.kv_stride * 4;
  PKLayer r;
  r.n1g = pk_adv(p.L0.n1g, wb); r.n1b = pk_adv(p.L0.n1b, wb);
  r.wqkv = pk_adv(p.L0.wqkv, wb); r.bqkv = pk_adv(p.L0.bqkv, wb);
  r.wo = pk_adv(p.L0.wo, wb); r.bo = pk_adv(p.L0.bo, wb);
  r.n2g = pk_adv(p.L0.n2g, wb); r.n2b = pk_adv(p.L0.n2b, wb);
  r.wfc = pk_adv(p.L0.wfc, wb); r.bfc = pk_adv(p.L0.bfc, wb);
  r.wproj = pk_adv(p.L0.wproj, wb); r.bproj = pk_adv(p.L0.bproj, wb);
  r.kc = pk_adv(p.L0.kc, kb); r.vc = pk_adv(p.L0.vc, kb);
  return r;
}
__device__ __forceinline__ void pk_err(const int* err, int bits) {
  __hip_atomic_fetch_or(gpw(const_cast<int*>(err)), bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t pk_word(float v, unsigned tag) {
  return ((uint64_t)tag << 32) | (uint64_t)__float_as_uint(v);
}
__device__ __forceinline__ void pk_store(uint64_t* a, uint64_t w) {
  __hip_atomic_store(gpw(a), w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t pk_load(const uint64_t* a) {
  return __hip_atomic_load(gpw(const_cast<uint64_t*>(a)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroup barrier that waits only for LDS operations (s_barrier alone does not
// order LDS; the memory clobber keeps the compiler from moving LDS accesses across).
__device__ __forceinline__ void pk_bar() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Element offset of the K/V slot of (seq, position) in a layer pool, or -1. A
// contiguous cache holds the sequence's positions at consecutive slots from kv0; a
// paged one (block size 1 << bs_shift) holds position ps in block
// table[ps >> bs_shift], slot ps & (block size - 1).
__device__ __forceinline__ int pk_slot(const PKParams& p, int ps) {
  if (!p.paged) return p.kv0 + ps * p.hd;
  const int bi = ps >> p.bs_shift;
  const int blk = bi < p.max_blocks ? *gp(p.table + p.seq * p.max_blocks + bi) : -1;
  if ((unsigned)blk >= (unsigned)p.nblk) return -1;
  return ((blk * p.H << p.bs_shift) + (ps & ((1 << p.bs_shift) - 1))) * p.hd;
}

// Wave 0: waits until the n (even, <= 4096) words at src (16-byte aligned) carry the
// step tag and writes their values to dst (LDS). Polling re-reads little: first one
// 16-byte pair per lane, spread over the vector, until all 64 pairs are current (the
// abort tag is read in the same round); then the vector is copied into the LDS buffer
// wbuf with direct global-to-LDS loads (device-coherent cache policy, no registers in
// flight), 128 words per instruction, and only blocks that still hold a stale word
// are copied again. Returns false on timeout or when another workgroup aborted the step.
#define PK_CPOL_SC1 16   // cache policy of the device-scope atomic load (bypasses the XCD's L2)
typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ bool pk_fail(const PKParams& p, long long t0, unsigned ab, int* s_abort) {
  if (ab != p.tag && (long long)__builtin_amdgcn_s_memrealtime() - t0 <= p.spin_ticks) return false;
  if ((threadIdx.x & 63) == 0) {
    __hip_atomic_store(gpw(p.abort_tag), p.tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    pk_err(p.err, GD_DERR_SYNC);
    *s_abort = 1;
  }
  return true;
}

__device__ __forceinline__ bool pk_get(const uint64_t* src, int n, float* dst, uint64_t* wbuf, const PKParams& p,
                                       long long t0, int* s_abort) {
  const int lane = threadIdx.x & 63;
  // 1. samples (longer vectors only: there they cut the polling traffic)
  if (n > 512) {
  const int sp = 2 * (int)((unsigned)lane * (unsigned)(n >> 1) / 64u);
  for (;;) {
    const uint64_t a = pk_load(src + sp), b = pk_load(src + sp + 1);
    const unsigned ab = __hip_atomic_load(gpw(p.abort_tag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool ok = (unsigned)(a >> 32) == p.tag && (unsigned)(b >> 32) == p.tag;
    if (__builtin_amdgcn_ballot_w64(!ok) == 0) break;
    if (pk_fail(p, t0, ab, s_abort)) return false;
  }
  }
  // 2. the whole vector, block by block
  const int nb = (n + 127) >> 7;
  unsigned pending = nb >= 32 ? 0xffffffffu : (1u << nb) - 1u;
  for (;;) {
    for (unsigned m = pending; m; m &= m - 1) {
      const int b0 = __builtin_ctz(m) << 7;
      const int i = min(b0 + 2 * lane, n - 2);   // lanes past the end repeat the last pair
      __builtin_amdgcn_global_load_lds(src + i, (lds_ptr_t)(wbuf + b0), 16, 0, PK_CPOL_SC1);
    }
    const unsigned ab = __hip_atomic_load(gpw(p.abort_tag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);   // the copies have landed in LDS
    asm volatile("" ::: "memory");
    for (unsigned m = pending; m; m &= m - 1) {
      const int bi = __builtin_ctz(m), b0 = bi << 7;
      const bool ok = (unsigned)(wbuf[b0 + 2 * lane] >> 32) == p.tag && (unsigned)(wbuf[b0 + 2 * lane + 1] >> 32) == p.tag;
      if (__builtin_amdgcn_ballot_w64(!ok) == 0) pending &= ~(1u << bi);
    }
    if (!pending) break;
    if (pk_fail(p, t0, ab, s_abort)) return false;
  }
  for (int k = lane; k < n; k += 64) dst[k] = __uint_as_float((uint32_t)wbuf[k]);
  return true;
}

// Wave 0: LayerNorm of the D values in x (LDS) into y (LDS); g and b are this lane's
// gain/shift values (elements lane + 64 j), loaded before the poll.
template <int D>
__device__ __forceinline__ void pk_layernorm(const float* x, float* y, float eps, const float* g, const float* b) {
  constexpr int J = (D + 63) / 64;
  const int lane = threadIdx.x & 63;
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int i = lane + 64 * j;
    if (D % 64 == 0 || i < D) s += x[i];
  }
  const float mu = wave_sum(s) / (float)D;
  float v = 0.f;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int i = lane + 64 * j;
    if (D % 64 == 0 || i < D) { const float t = x[i] - mu; v = fmaf(t, t, v); }
  }
  const float rs = 1.0f / sqrtf(wave_sum(v) / (float)D + eps);
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int i = lane + 64 * j;
    if (D % 64 == 0 || i < D) y[i] = (x[i] - mu) * rs * g[j] + b[j];
  }
}

// Wave 0: this lane's gain and shift values of a norm over D.
template <int D>
__device__ __forceinline__ void pk_norm_params(const float* gsrc, const float* bsrc, float* g, float* b) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < (D + 63) / 64; ++j) {
    const int i = min(lane + 64 * j, D - 1);
    g[j] = *gp(gsrc + i);
    b[j] = *gp(bsrc + i);
  }
}

// Compute waves: the weight rows of one phase. Wave cw owns rows r0 + cw + PK_CW i
// (i < R) of [r0, r1); lane l holds 16-byte chunks l + 64 c (c < NC) of each row, and
// the bias of each row. Loads are unconditional (clamped) so that their count is
// fixed; rows past r1 are never used.
template <int WT, int K, int R>
struct PKRowsK {
  static constexpr int CE = WChunk<WT>::CE, NC = (K + 64 * CE - 1) / (64 * CE);
  typename WChunk<WT>::T w[R][NC];
  float b[R];
};

template <int WT, int K, int R>
__device__ __forceinline__ void pk_issue(PKRowsK<WT, K, R>& rr, const void* W, const float* bias, int N, int r0,
                                         int cw, int lane) {
  typedef typename WChunk<WT>::T VT;
  constexpr int CE = WChunk<WT>::CE, NC = PKRowsK<WT, K, R>::NC;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int n = min(r0 + cw + PK_CW * i, N - 1);
    // 32-bit byte offset from a uniform base (a matrix is < 4 GB); chunk c adds 1 KB
    // (fp32) or 1 KB (bf16) to the row's lane offset
    const char* row = reinterpret_cast<const char*>(W) + (uint32_t)n * (uint32_t)(K * (WT == 0 ? 4 : 2));
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int k = (K % (64 * CE) == 0) ? (lane + 64 * c) * CE : min((lane + 64 * c) * CE, K - CE);
      rr.w[i][c] = __builtin_nontemporal_load(gp(reinterpret_cast<const VT*>(row + (uint32_t)k * (WT == 0 ? 4u : 2u))));
    }
    rr.b[i] = bias ? *gp(bias + n) : 0.f;   // (uniform: no bias for the head rows)
  }
}

// Per-lane partial dot product of row i of rr with the LDS vector x (length K).
template <int WT, int K, int R>
__device__ __forceinline__ float pk_dot(const PKRowsK<WT, K, R>& rr, int i, const float* x, int lane) {
  constexpr int CE = WChunk<WT>::CE, NC = PKRowsK<WT, K, R>::NC;
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int k = (lane + 64 * c) * CE;
    if (K % (64 * CE) == 0 || k < K) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(x + k);
      if constexpr (WT == 0) {
        s = fmaf(rr.w[i][c].x, a.x, s); s = fmaf(rr.w[i][c].y, a.y, s);
        s = fmaf(rr.w[i][c].z, a.z, s); s = fmaf(rr.w[i][c].w, a.w, s);
      } else {
        const f32x4 a2 = *reinterpret_cast<const f32x4*>(x + k + 4);
        s = fmaf(bf16_lo(rr.w[i][c].x), a.x, s); s = fmaf(bf16_hi(rr.w[i][c].x), a.y, s);
        s = fmaf(bf16_lo(rr.w[i][c].y), a.z, s); s = fmaf(bf16_hi(rr.w[i][c].y), a.w, s);
        s = fmaf(bf16_lo(rr.w[i][c].z), a2.x, s); s = fmaf(bf16_hi(rr.w[i][c].z), a2.y, s);
        s = fmaf(bf16_lo(rr.w[i][c].w), a2.z, s); s = fmaf(bf16_hi(rr.w[i][c].w), a2.w, s);
      }
    }
  }
  return s;
}

// Rows [r0, r1) of a phase with N outputs for workgroup wg of nwg.
__device__ __forceinline__ void pk_range(int N, int wg, int nwg, int& r0, int& r1) {
  r0 = (int)((unsigned)N * (unsigned)wg / (unsigned)nwg);   // N * nwg < 2^32
  r1 = (int)((unsigned)N * (unsigned)(wg + 1) / (unsigned)nwg);
}

// Barrier of the compute waves only (wave 0 may be polling): an LDS counter that
// grows by PK_CW per use; `use` counts this wave's uses.
__device__ __forceinline__ void pk_cbar(int* ctr, int& use, int lane, long long t0, long long limit, int* err) {
  ++use;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  if (lane == 0) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < PK_CW * use) {
    if ((long long)__builtin_amdgcn_s_memrealtime() - t0 > limit) {
      if (lane == 0) pk_err(err, GD_DERR_SYNC);
      break;
    }
  }
  asm volatile("" ::: "memory");
}

// One attention chunk of head h (compute waves; t = thread index among them): positions
// [p0, p1) of the sequence, the current position's k and v taken from LDS (its cache
// slot is being written in this same step). Writes the chunk's (max, sum, weighted V)
// to the exchange.
template <int HD, int H>
__device__ __forceinline__ void pk_attention(const PKParams& p, int l, int h, int c, const float* qkv_in, float* s_att,
                                             int* s_cbar, int& cuse, long long t0) {
  constexpr int LG = HD / 4;                    // lanes per position
  constexpr int NGRP = PK_CW * 64 / LG;         // position groups
  constexpr int PPG = (PK_ACH + NGRP - 1) / NGRP;
  const int t = threadIdx.x - 64, lane = threadIdx.x & 63;
  const int grp = t / LG, gl = t % LG;
  const int T = p.pos + 1;
  const int p0 = c * PK_ACH, p1 = min(T, p0 + PK_ACH);
  const PKLayer L = pk_layer(p, l);
  const f32x4 q = *reinterpret_cast<const f32x4*>(qkv_in + gl * 4);
  const f32x4 kcur = *reinterpret_cast<const f32x4*>(qkv_in + HD + gl * 4);
  const f32x4 vcur = *reinterpret_cast<const f32x4*>(qkv_in + 2 * HD + gl * 4);
  const char* kb = reinterpret_cast<const char*>(L.kc);
  const char* vb = reinterpret_cast<const char*>(L.vc);
  // every load is issued (position 0's slot stands in for positions outside the chunk,
  // the current one and unmapped blocks), and the values are chosen afterwards:
  // a load under a per-lane branch would be waited for at the branch's join
  const int off0 = max(pk_slot(p, 0), 0);
  f32x4 kv[PPG], vv[PPG];
  bool ok[PPG], cur[PPG];
  int blk[PPG];   // paged: each position's block, all table entries loaded before any wait
  const int bmask = (1 << p.bs_shift) - 1;
  // rounds of NGRP positions that the chunk needs (uniform: the loads of rounds past it
  // are skipped by a scalar branch, and their slots keep the current k and v, masked out)
  const int rounds = (p1 - p0 + NGRP - 1) / NGRP;
  if (p.paged) {
#pragma unroll
    for (int j = 0; j < PPG; ++j) {
      if (j < rounds) {
        const int ps = min(p0 + grp + NGRP * j, p.pos);
        blk[j] = *gp(p.table + p.seq * p.max_blocks + (ps >> p.bs_shift));
      }
    }
  }
#pragma unroll
  for (int j = 0; j < PPG; ++j) {
    const int ps = p0 + grp + NGRP * j;
    kv[j] = kcur;
    vv[j] = vcur;
    ok[j] = false;
    cur[j] = false;
    if (j >= rounds) continue;
    int off;
    if (p.paged) off = (unsigned)blk[j] < (unsigned)p.nblk ? ((blk[j] * p.H << p.bs_shift) + (ps & bmask)) * HD : -1;
    else off = p.kv0 + ps * HD;
    off = ps < p1 && ps != p.pos ? off : -1;
    ok[j] = ps < p1 && (ps == p.pos || off >= 0);
    cur[j] = ps == p.pos;
    const uint32_t o = (uint32_t)((off >= 0 ? off : off0) + h * p.kv_hstride + gl * 4) * 4u;   // bytes (a pool is < 2 GB)
    kv[j] = *gp(reinterpret_cast<const f32x4*>(kb + o));
    vv[j] = *gp(reinterpret_cast<const f32x4*>(vb + o));
  }
#pragma unroll
  for (int j = 0; j < PPG; ++j) {
    kv[j] = cur[j] ? kcur : kv[j];
    vv[j] = cur[j] ? vcur : vv[j];
  }
  float sc[PPG];
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < PPG; ++j) {
    float dd = q.x * kv[j].x;
    dd = fmaf(q.y, kv[j].y, dd);
    dd = fmaf(q.z, kv[j].z, dd);
    dd = fmaf(q.w, kv[j].w, dd);
    sc[j] = group_sum<LG>(dd) * p.scale;
    if (ok[j]) mx = fmaxf(mx, sc[j]);
  }
  float lsum = 0.f;
  f32x4 o = (f32x4){0.f, 0.f, 0.f, 0.f};
  if (mx != -INFINITY) {
#pragma unroll
    for (int j = 0; j < PPG; ++j) {
      if (ok[j]) {
        const float e = expf(sc[j] - mx);
        lsum += e;
        o.x = fmaf(e, vv[j].x, o.x);
        o.y = fmaf(e, vv[j].y, o.y);
        o.z = fmaf(e, vv[j].z, o.z);
        o.w = fmaf(e, vv[j].w, o.w);
      }
    }
  }
  // merge of the position groups: the chunk's maximum over the waves (LDS), then each
  // group's share rescaled to it, summed over the groups of a wave with lane swaps and
  // over the waves through LDS. s_att: maxima [PK_CW] | sums [PK_CW] | (at float 16,
  // 16-byte aligned) vectors [PK_CW][HD]
  const int cw = t >> 6;
  const float wm = wave_max(mx);   // -inf for a wave whose groups saw no position
  if (lane == 0) s_att[cw] = wm;
  pk_cbar(s_cbar, cuse, lane, t0, p.spin_ticks, p.err);
  float M = s_att[0];
#pragma unroll
  for (int w = 1; w < PK_CW; ++w) M = fmaxf(M, s_att[w]);
  const float f = mx == -INFINITY ? 0.f : expf(mx - M);
  float ls = lsum * f;
  f32x4 ov = (f32x4){o.x * f, o.y * f, o.z * f, o.w * f};
#pragma unroll
  for (int sh = LG; sh < 64; sh <<= 1) {   // lanes gl, gl + LG, ... hold the same dims
    ls += __shfl_xor(ls, sh, 64);
    ov.x += __shfl_xor(ov.x, sh, 64);
    ov.y += __shfl_xor(ov.y, sh, 64);
    ov.z += __shfl_xor(ov.z, sh, 64);
    ov.w += __shfl_xor(ov.w, sh, 64);
  }
  float* s_ws = s_att + PK_CW;
  float* s_wo = s_att + 16;
  static_assert(2 * PK_CW <= 16, "merge layout");
  if (lane == 0) s_ws[cw] = ls;
  if (lane < LG) *reinterpret_cast<f32x4*>(s_wo + cw * HD + gl * 4) = ov;
  pk_cbar(s_cbar, cuse, lane, t0, p.spin_ticks, p.err);
  if (t < HD) {
    float acc = 0.f, lt = 0.f;
#pragma unroll
    for (int w = 0; w < PK_CW; ++w) { acc += s_wo[w * HD + t]; lt += s_ws[w]; }
    uint64_t* dst = p.xb + (size_t)l * p.xl + p.x_att + (size_t)(c * H + h) * (HD + 2);
#pragma unroll
    for (int r = 0; r < PK_NREP; ++r) {
      pk_store(dst + (size_t)r * p.rs_att + 2 + t, pk_word(acc, p.tag));
      if (t == 0) {
        pk_store(dst + (size_t)r * p.rs_att, pk_word(M, p.tag));
        pk_store(dst + (size_t)r * p.rs_att + 1, pk_word(lt, p.tag));
      }
    }
  }
  pk_cbar(s_cbar, cuse, lane, t0, p.spin_ticks, p.err);   // s_att is free again
}

// Wave 0: the inputs of every phase (it runs the same sequence of barriers as the
// compute waves, see k_decode1).
template <int WT, int D, int FF, int HD>
__device__ __forceinline__ void pk_stage(const PKParams& p, float* s_x, float* s_in, float* s_raw, uint64_t* wbuf,
                                         int* s_abort, int unit, long long t0) {
  constexpr int H = D / HD, J = (D + 63) / 64;
  const int lane = threadIdx.x & 63;
  const int wg = blockIdx.x, nwg = gridDim.x, rep = wg % PK_NREP;
  const int ah = unit >= 0 ? unit % H : 0;
  int ph = 0;
  auto in_buf = [&](int k) { return s_in + (k & 1) * PK_INMAX; };
  for (int l = 0; l < p.n_layer; ++l) {
    const PKLayer L = pk_layer(p, l);
    const uint64_t* X = p.xb + (size_t)l * p.xl;
    // A: residual (embedding or the previous layer's output), pre-norm
    {
      float g[J], b[J];
      pk_norm_params<D>(L.n1g, L.n1b, g, b);
      bool ok = true;
      if (l == 0) {
        int tk = *gp(p.tok);
        if (tk < 0 || tk >= p.vocab) { if (lane == 0 && wg == 0) pk_err(p.err, GD_DERR_TOKEN); tk = 0; }
#pragma unroll
        for (int j = 0; j < J; ++j) {
          const int i = lane + 64 * j;
          if (D % 64 == 0 || i < D) {
            float v, u;
            if (WT == 0) {
              v = *gp(reinterpret_cast<const float*>(p.wte) + (size_t)tk * D + i);
              u = *gp(reinterpret_cast<const float*>(p.wpe) + (size_t)p.pos * D + i);
            } else {
              v = bf16_lo(*gp(reinterpret_cast<const uint16_t*>(p.wte) + (size_t)tk * D + i));
              u = bf16_lo(*gp(reinterpret_cast<const uint16_t*>(p.wpe) + (size_t)p.pos * D + i));
            }
            s_x[i] = v + u;
          }
        }
      } else {
        ok = pk_get(p.xb + (size_t)(l - 1) * p.xl + p.x_xd + (size_t)rep * p.rs_d, D, s_x, wbuf, p, t0, s_abort);
      }
      if (ok) pk_layernorm<D>(s_x, in_buf(ph), p.eps, g, b);
    }
    pk_bar();
    if (*s_abort) return;
    ++ph;
    // B: q, k, v of this workgroup's attention head: 3 HD consecutive words (one replica)
    if (unit >= 0) pk_get(X + (size_t)ah * 3 * HD, 3 * HD, in_buf(ph), wbuf, p, t0, s_abort);
    pk_bar();
    if (*s_abort) return;
    ++ph;
    // C: attention partials of every head, merged into the projection's input
    if (pk_get(X + p.x_att + (size_t)rep * p.rs_att, H * p.nch * (HD + 2), s_raw, wbuf, p, t0, s_abort)) {
      float* o = in_buf(ph);
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int i = lane + 64 * j;
        if (D % 64 == 0 || i < D) {
          const int hh = i / HD, jj = i % HD;
          float m = -INFINITY;
          for (int c = 0; c < p.nch; ++c) m = fmaxf(m, s_raw[(c * H + hh) * (HD + 2)]);
          float ls = 0.f, acc = 0.f;
          for (int c = 0; c < p.nch; ++c) {
            const float* pc = s_raw + (c * H + hh) * (HD + 2);
            if (pc[1] == 0.f) continue;   // chunk without positions
            const float wgt = expf(pc[0] - m);
            ls = fmaf(pc[1], wgt, ls);
            acc = fmaf(pc[2 + jj], wgt, acc);
          }
          o[i] = ls > 0.f ? acc / ls : 0.f;
        }
      }
    }
    pk_bar();
    if (*s_abort) return;
    ++ph;
    // D: residual after the output projection, pre-norm
    {
      float g[J], b[J];
      pk_norm_params<D>(L.n2g, L.n2b, g, b);
      if (pk_get(X + p.x_xo + (size_t)rep * p.rs_d, D, s_x, wbuf, p, t0, s_abort))
        pk_layernorm<D>(s_x, in_buf(ph), p.eps, g, b);
    }
    pk_bar();
    if (*s_abort) return;
    ++ph;
    // E: MLP hidden activations
    pk_get(X + p.x_h + (size_t)rep * p.rs_h, FF, in_buf(ph), wbuf, p, t0, s_abort);
    pk_bar();
    if (*s_abort) return;
    ++ph;
  }
  // head input: final norm of the last residual
  {
    float g[J], b[J];
    pk_norm_params<D>(p.nfg, p.nfb, g, b);
    if (pk_get(p.xb + (size_t)(p.n_layer - 1) * p.xl + p.x_xd + (size_t)rep * p.rs_d, D, s_x, wbuf, p, t0, s_abort))
      pk_layernorm<D>(s_x, in_buf(ph), p.eps, g, b);
  }
  pk_bar();
  if (*s_abort) return;
  pk_bar();   // the compute waves' argmax partials are in LDS
  if (wg != 0) return;
  // greedy argmax over the workgroup partials (workgroup 0)
  int res = 0;
  if (pk_get(p.xb + p.x_arg, 2 * nwg, s_raw, wbuf, p, t0, s_abort)) {
    float bv = 0.f;
    int bi = 0x7fffffff;
    for (int i = lane; i < nwg; i += 64) {
      const float v = s_raw[2 * i];
      const int ix = __float_as_int(s_raw[2 * i + 1]);
      if (ix != 0x7fffffff && (bi == 0x7fffffff || am_better(v, ix, bv, bi))) { bv = v; bi = ix; }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (oi != 0x7fffffff && (bi == 0x7fffffff || am_better(ov, oi, bv, bi))) { bv = ov; bi = oi; }
    }
    res = bi == 0x7fffffff ? 0 : bi;
  }
  if (lane == 0) {
    *gpw(p.next) = res;
    *gpw(p.len + p.seq) = p.pos + 1;
  }
}

// Waves 1..8: weights and arithmetic of every phase.
template <int WT, int D, int FF, int HD>
__device__ __forceinline__ void pk_compute(const PKParams& p, float* s_x, float* s_in, float* s_att, float* s_am,
                                           int* s_abort, int* s_cbar, int unit, long long t0) {
  constexpr int H = D / HD, QKV = 3 * D;
  const int tid = threadIdx.x, lane = tid & 63;
  const int cw = __builtin_amdgcn_readfirstlane((tid >> 6) - 1);   // wave-uniform
  const int wg = blockIdx.x, nwg = gridDim.x;
  const int ah = unit >= 0 ? unit % H : 0, ac = unit >= 0 ? unit / H : 0;
  int ph = 0, cuse = 0;
  auto in_buf = [&](int k) { return s_in + (k & 1) * PK_INMAX; };
  const int kvoff = pk_slot(p, p.pos);   // the current position's K/V slot
  if (kvoff < 0 && wg == 0 && tid == 64) pk_err(p.err, GD_DERR_BLOCK);
  int q0, q1, f0, f1, e0, e1;
  pk_range(QKV, wg, nwg, q0, q1);
  pk_range(FF, wg, nwg, f0, f1);
  pk_range(D, wg, nwg, e0, e1);
  PKRowsK<WT, D, 2> rq;    // QKV and MLP-up rows
  PKRowsK<WT, D, 1> ro;    // output-projection rows
  PKRowsK<WT, FF, 1> rd;   // MLP-down rows
  pk_issue(rq, pk_layer(p, 0).wqkv, pk_layer(p, 0).bqkv, QKV, q0, cw, lane);
  for (int l = 0; l < p.n_layer; ++l) {
    const PKLayer L = pk_layer(p, l);
    uint64_t* X = p.xb + (size_t)l * p.xl;
    // A: QKV + bias; q, k, v to the exchange (head-major), k and v into the cache slot
    pk_bar();
    if (*s_abort) return;
    {
      const float* xin = in_buf(ph);
      float v[2] = {pk_dot(rq, 0, xin, lane), pk_dot(rq, 1, xin, lane)};
      wave_sum_n<2>(v);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int n = q0 + cw + PK_CW * i;
        if (n < q1) {
          const float y = v[i] + rq.b[i];
          const int part = n / D, hh = (n % D) / HD, j = n % HD;
          if (lane == 0) pk_store(X + hh * 3 * HD + part * HD + j, pk_word(y, p.tag));
          if (lane == 1 && part > 0 && kvoff >= 0)
            *gpw((part == 1 ? L.kc : L.vc) + (uint32_t)(kvoff + hh * p.kv_hstride + j)) = y;
        }
      }
    }
    ++ph;
    // B: attention (its K/V loads would wait behind earlier-issued weight loads)
    pk_bar();
    if (*s_abort) return;
    if (unit >= 0) pk_attention<HD, H>(p, l, ah, ac, in_buf(ph), s_att, s_cbar, cuse, t0);
    pk_issue(ro, L.wo, L.bo, D, e0, cw, lane);   // output projection: weights ahead
    ++ph;
    // C: output projection + bias + residual
    pk_bar();
    if (*s_abort) return;
    {
      const float v = wave_sum(pk_dot(ro, 0, in_buf(ph), lane));
      const int n = e0 + cw;
      if (n < e1 && lane < PK_NREP)
        pk_store(X + p.x_xo + (size_t)lane * p.rs_d + n, pk_word(s_x[n] + v + ro.b[0], p.tag));
    }
    pk_issue(rq, L.wfc, L.bfc, FF, f0, cw, lane);   // MLP up: weights ahead
    ++ph;
    // D: MLP up + bias + clamped tanh-GELU
    pk_bar();
    if (*s_abort) return;
    {
      const float* xin = in_buf(ph);
      float v[2] = {pk_dot(rq, 0, xin, lane), pk_dot(rq, 1, xin, lane)};
      wave_sum_n<2>(v);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int n = f0 + cw + PK_CW * i;
        if (n < f1 && lane < PK_NREP)
          pk_store(X + p.x_h + (size_t)lane * p.rs_h + n, pk_word(gelu_clamped(v[i] + rq.b[i]), p.tag));
      }
    }
    pk_issue(rd, L.wproj, L.bproj, D, e0, cw, lane);   // MLP down: weights ahead
    ++ph;
    // E: MLP down + bias + residual
    pk_bar();
    if (*s_abort) return;
    {
      const float v = wave_sum(pk_dot(rd, 0, in_buf(ph), lane));
      const int n = e0 + cw;
      if (n < e1 && lane < PK_NREP)
        pk_store(X + p.x_xd + (size_t)lane * p.rs_d + n, pk_word(s_x[n] + v + rd.b[0], p.tag));
    }
    if (l + 1 < p.n_layer) pk_issue(rq, pk_layer(p, l + 1).wqkv, pk_layer(p, l + 1).bqkv, QKV, q0, cw, lane);
    ++ph;
  }
  // head: tied-embedding logits of this workgroup's vocabulary rows, running argmax
  pk_bar();
  if (*s_abort) return;
  {
    const float* xin = in_buf(ph);
    int h0, h1;
    pk_range(p.vocab, wg, nwg, h0, h1);
    float bv = 0.f;
    int bi = 0x7fffffff;
    for (int j0 = 0; h0 + cw + PK_CW * j0 < h1; j0 += 4) {
      PKRowsK<WT, D, 4> rh;
      pk_issue(rh, p.wte, (const float*)nullptr, h1, h0 + PK_CW * j0, cw, lane);
      float v[4] = {pk_dot(rh, 0, xin, lane), pk_dot(rh, 1, xin, lane), pk_dot(rh, 2, xin, lane),
                    pk_dot(rh, 3, xin, lane)};
      wave_sum_n<4>(v);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = h0 + cw + PK_CW * (j0 + i);
        if (n < h1) {
          if (p.logits && lane == 0) *gpw(p.logits + n) = v[i];
          if (bi == 0x7fffffff || am_better(v[i], n, bv, bi)) { bv = v[i]; bi = n; }
        }
      }
    }
    if (lane == 0) { s_am[2 * cw] = bv; s_am[2 * cw + 1] = __int_as_float(bi); }
  }
  pk_bar();
  if (cw == 0 && lane == 0) {   // this workgroup's partial
    float bv = s_am[0];
    int bi = __float_as_int(s_am[1]);
    for (int w2 = 1; w2 < PK_CW; ++w2) {
      const float v = s_am[2 * w2];
      const int i = __float_as_int(s_am[2 * w2 + 1]);
      if (i != 0x7fffffff && (bi == 0x7fffffff || am_better(v, i, bv, bi))) { bv = v; bi = i; }
    }
    pk_store(p.xb + p.x_arg + 2 * wg, pk_word(bv, p.tag));
    pk_store(p.xb + p.x_arg + 2 * wg + 1, pk_word(__int_as_float(bi), p.tag));
  }
}

// One decode step of one sequence; D, FF, HD: d_model, d_ff, head_dim.
template <int WT, int D, int FF, int HD>
__global__ __launch_bounds__(PK_WG) void k_decode1(PKParams p) {
  static_assert(D <= PK_DMAX && FF <= PK_INMAX && (D / HD) * PK_MAXNCH * (HD + 2) <= PK_INMAX, "staging sizes");
  extern __shared__ __align__(16) float lds[];
  float* s_x = lds;                                // residual [D]
  float* s_in = lds + PK_DMAX;                     // staged inputs [2][PK_INMAX], by phase parity
  float* s_raw = s_in + 2 * PK_INMAX;              // raw attention / argmax partials
  float* s_att = s_raw + PK_INMAX;                 // attention position-group partials
  float* s_am = s_att + 2304;                      // per-wave argmax (value, index bits)
  uint64_t* wbuf = reinterpret_cast<uint64_t*>(s_am + 2 * PK_CW + 2);   // wave 0's poll buffer [PK_INMAX]
  __shared__ int s_abort, s_cbar;
  const long long t0 = (long long)__builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) { s_abort = 0; s_cbar = 0; }
  __syncthreads();
  // this workgroup's attention unit (head, chunk) for the step, if any
  const int units = (D / HD) * p.nch, nwg = gridDim.x, wg = blockIdx.x;
  const int ustride = max(1, nwg / units);
  const int unit = (wg % ustride == 0 && wg / ustride < units) ? wg / ustride : -1;
  if (threadIdx.x < 64) pk_stage<WT, D, FF, HD>(p, s_x, s_in, s_raw, wbuf, &s_abort, unit, t0);
  else pk_compute<WT, D, FF, HD>(p, s_x, s_in, s_att, s_am, &s_abort, &s_cbar, unit, t0);
}
