// misc.h -- step plumbing, embedding, standalone argmax.
#pragma once
#include "common.h"

// Per-row metadata and input embedding shared by decode and prefill.
struct RowParams {
  const int* table; int max_blocks, block_size, nblk, Hkv, hd;  // KV cache addressing
  const void* wte; const void* wpe; int vocab, n_pos, d, emb_bf16;
  int emb_q8; const float* wte_sc; const float* wpe_sc;          // 8-bit tables: codes and block scales
  float* x;                                                      // [rows][d]
  int* row_seq; int* row_pos; int* row_tok; long long* row_kvoff;
  const float* rope; float* row_cs;   // RoPE table [n_pos][hd] (cos | sin) and each row's copy
  int* err;
};

// Element offset of (sequence, position)'s K/V slot inside one layer pool, or -1
// (position p lives in block table[p / B], slot p mod B: "rvllm Metal backend",
// "What the kernels do", paged KV cache).
__device__ __forceinline__ long long kv_slot_offset(const RowParams& r, int seq, int pos) {
  if (pos < 0) return -1;
  const int bi = pos / r.block_size;
  const int blk = bi < r.max_blocks ? r.table[(size_t)seq * r.max_blocks + bi] : -1;
  if ((unsigned)blk >= (unsigned)r.nblk) return -1;
  return ((long long)blk * r.Hkv * r.block_size + (pos - bi * r.block_size)) * r.hd;
}

// Row b's embedding x_b = wte[t] (+ wpe[p]) ("bare-metal-llm", "Picking the model" and
// "What got built": token and learned position embeddings) and its cache slot.
// Called by the whole workgroup with the row's sequence, position and token.
__device__ void row_setup(const RowParams& r, int b, int seq, int pos, int tok) {
  if (tok < 0 || tok >= r.vocab) { if (threadIdx.x == 0) atomicOr(r.err, GD_DERR_TOKEN); tok = 0; }
  int ppos = pos;
  if (r.wpe && (ppos < 0 || ppos >= r.n_pos)) { if (threadIdx.x == 0) atomicOr(r.err, GD_DERR_POS); ppos = 0; }
  if (threadIdx.x == 0) {
    const long long off = kv_slot_offset(r, seq, pos);
    if (off < 0) atomicOr(r.err, GD_DERR_BLOCK);
    r.row_kvoff[b] = off;
  }
  for (int i = threadIdx.x; i < r.d; i += GD_WG) {
    float v;
    const size_t et = (size_t)tok * r.d + i, ep = (size_t)ppos * r.d + i;
    if (r.emb_q8) v = (float)reinterpret_cast<const int8_t*>(r.wte)[et] * r.wte_sc[et >> 5];
    else if (!r.emb_bf16) v = reinterpret_cast<const float*>(r.wte)[et];
    else v = bf16_lo(reinterpret_cast<const uint16_t*>(r.wte)[et]);
    if (r.wpe) {
      if (r.emb_q8) v += (float)reinterpret_cast<const int8_t*>(r.wpe)[ep] * r.wpe_sc[ep >> 5];
      else if (!r.emb_bf16) v += reinterpret_cast<const float*>(r.wpe)[ep];
      else v += bf16_lo(reinterpret_cast<const uint16_t*>(r.wpe)[ep]);
    }
    r.x[(size_t)b * r.d + i] = v;
  }
  if (r.rope) {
    const int rp = min(max(pos, 0), r.n_pos - 1);
    for (int i = threadIdx.x; i < r.hd; i += GD_WG) r.row_cs[(size_t)b * r.hd + i] = r.rope[(size_t)rp * r.hd + i];
  }
}

// Decode step set-up, on the device so the step replays as one graph: row b runs
// slot seq_ids[b] at its current length, which is then advanced. One workgroup per row.
// Steps whose first QKV launch is a GEMV (at most 4 rows) do the same inside that
// launch instead (PRO_EMBED in linear.h), and their argmax finalize advances the
// lengths.
__global__ __launch_bounds__(GD_WG) void k_setup_decode(RowParams r, const int* __restrict__ seq_ids,
                                                        const int* __restrict__ tokens, int* len,
                                                        const int* __restrict__ cap) {
  __shared__ int s_pos, s_tok, s_seq;
  const int b = blockIdx.x;
  if (threadIdx.x == 0) {
    const int s = seq_ids[b];
    int pos = len[s];
    if (pos >= cap[s]) { atomicOr(r.err, GD_DERR_POS); pos = cap[s] - 1; }
    const int tok = tokens[b];
    r.row_seq[b] = s;
    r.row_pos[b] = pos;
    r.row_tok[b] = tok;
    len[s] = pos + 1;
    s_pos = pos; s_tok = tok; s_seq = s;
  }
  __syncthreads();
  row_setup(r, b, s_seq, s_pos, s_tok);
}

// Prefill set-up of rows whose (sequence, position, token) the host has uploaded.
__global__ __launch_bounds__(GD_WG) void k_setup_rows(RowParams r) {
  const int b = blockIdx.x;
  row_setup(r, b, r.row_seq[b], r.row_pos[b], r.row_tok[b]);
}

// Standalone greedy argmax over rows of logits: per (row, chunk of 4096) partials,
// the last workgroup to finish reduces them in index order.
__global__ __launch_bounds__(GD_WG) void k_argmax_rows(const float* __restrict__ logits, int rows, int vocab,
                                                       int nchunk, float* pv, int* pi, int* ctr, int* out) {
  __shared__ float sv[GD_WG / 64];
  __shared__ int si[GD_WG / 64];
  __shared__ int s_last;
  const int c = blockIdx.x, row = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* r = logits + (size_t)row * vocab;
  const int b = c * 4096, e = min(vocab, b + 4096);
  float bv = __builtin_nanf("");
  int bi = 0x7fffffff;
  bool have = false;
  for (int i = b + tid; i < e; i += GD_WG) {
    float v = r[i];
    if (!have || am_better(v, i, bv, bi)) { bv = v; bi = i; have = true; }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float ov = __shfl_xor(bv, o, 64);
    int oi = __shfl_xor(bi, o, 64);
    int oh = __shfl_xor((int)have, o, 64);
    if (oh && (!have || am_better(ov, oi, bv, bi))) { bv = ov; bi = oi; have = true; }
  }
  if (lane == 0) { sv[wave] = bv; si[wave] = have ? bi : 0x7fffffff; }
  __syncthreads();
  if (tid == 0) {
    float v0 = sv[0];
    int i0 = si[0];
    for (int w = 1; w < GD_WG / 64; ++w)
      if (si[w] != 0x7fffffff && (i0 == 0x7fffffff || am_better(sv[w], si[w], v0, i0))) { v0 = sv[w]; i0 = si[w]; }
    pv[(size_t)row * nchunk + c] = v0;
    pi[(size_t)row * nchunk + c] = i0;
  }
  fence_agent();
  __syncthreads();
  if (tid == 0) {
    int old = atomic_add_acq_rel(ctr + row, 1);
    s_last = (old == nchunk - 1);
    if (s_last) store_relaxed(ctr + row, 0);
  }
  __syncthreads();
  if (!s_last || tid != 0) return;
  fence_agent();
  float v0 = pv[(size_t)row * nchunk];
  int i0 = pi[(size_t)row * nchunk];
  for (int k = 1; k < nchunk; ++k) {
    float v = pv[(size_t)row * nchunk + k];
    int i = pi[(size_t)row * nchunk + k];
    if (am_better(v, i, v0, i0)) { v0 = v; i0 = i; }
  }
  out[row] = i0;
}

// Returns after `ticks` of the 100 MHz real-time counter (bounded by its own clock).
// A profiled decode step is enqueued behind it whole, so its launches then run back to
// back with no host enqueue gaps inside the per-launch event pairs.
__global__ void k_gate(long long ticks) {
  const long long t0 = (long long)__builtin_amdgcn_s_memrealtime();
  while ((long long)__builtin_amdgcn_s_memrealtime() - t0 < ticks) __builtin_amdgcn_s_sleep(64);
}

// ------------------------------------------------------------------ sampling
//
// Temperature / top-k sampling of each head row ("batch_forge" README, status table:
// greedy, temperature and top-k sampling; its demo samples at temperature 0.7). Rule:
// the top_k largest logits (ties to the lower index), weights exp((l - l_max) / T), and
// the first candidate in that order whose cumulative weight exceeds u times the total;
// a NaN among the logits gives the first NaN's index. u drives the draw of the token
// after position p of sequence slot s: the top 24 bits of the first word of
// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC 2011) with counter (p, s, 0, 0) and key
// (seed, 0), times 2^-24.
#define GD_SAMPLE_NT 1024
#define GD_SAMPLE_VPT 64         // logits per thread: vocab <= GD_SAMPLE_NT * GD_SAMPLE_VPT
#define GD_SAMPLE_MAX_K 256

struct SampleParams {
  const float* logits; int ldl;    // [rows][ldl]
  int V, top_k;
  float inv_temp;
  unsigned long long seed;
  const int* row_seq; const int* row_pos;
  int* out;                        // [rows]
};

// Ten rounds of two 64 x 64 -> 128-bit products of counter words with the round
// multipliers; the high halves are xored with the other counter words and the key,
// which advances by the Weyl increments after every round. Returns output word 0.
__device__ __forceinline__ unsigned long long philox4x64_w0(unsigned long long c0, unsigned long long c1,
                                                            unsigned long long c2, unsigned long long c3,
                                                            unsigned long long k0, unsigned long long k1) {
  const unsigned long long M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const unsigned long long W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const unsigned long long hi0 = __umul64hi(M0, c0), lo0 = M0 * c0;
    const unsigned long long hi1 = __umul64hi(M1, c2), lo1 = M1 * c2;
    c0 = hi1 ^ c1 ^ k0;
    c1 = lo1;
    c2 = hi0 ^ c3 ^ k1;
    c3 = lo0;
    k0 += W0;
    k1 += W1;
  }
  return c0;
}

// Order-preserving key of a non-NaN float (larger float, larger key; -0 as +0); 0 is
// below every key and pads the rows.
__device__ __forceinline__ uint32_t sample_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) == 0) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float sample_val(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Exclusive prefix sums over the workgroup (thread order) of a and b, and their totals.
__device__ __forceinline__ void block_scan2(int a, int b, int& ea, int& eb, int& ta, int& tb, int* s_w) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, NW = GD_SAMPLE_NT / 64;
  int ia = a, ib = b;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int xa = __shfl_up(ia, o, 64), xb = __shfl_up(ib, o, 64);
    if (lane >= o) { ia += xa; ib += xb; }
  }
  if (lane == 63) { s_w[wave] = ia; s_w[NW + wave] = ib; }
  __syncthreads();
  int pa = 0, pb = 0;
  ta = tb = 0;
  for (int w = 0; w < NW; ++w) {
    if (w < wave) { pa += s_w[w]; pb += s_w[NW + w]; }
    ta += s_w[w];
    tb += s_w[NW + w];
  }
  ea = pa + ia - a;
  eb = pb + ib - b;
  __syncthreads();
}

__global__ __launch_bounds__(GD_SAMPLE_NT) void k_sample(SampleParams p) {
  __shared__ unsigned s_hist[256];
  __shared__ int s_w[2 * GD_SAMPLE_NT / 64];
  __shared__ int s_nan, s_digit, s_kk;
  __shared__ uint32_t s_ck[GD_SAMPLE_MAX_K];
  __shared__ int s_ci[GD_SAMPLE_MAX_K];
  __shared__ float s_sv[GD_SAMPLE_MAX_K];
  __shared__ int s_si[GD_SAMPLE_MAX_K];
  const int row = blockIdx.x, tid = threadIdx.x, V = p.V, k = p.top_k;
  const float* L = p.logits + (size_t)row * p.ldl;
  const int i0 = tid * GD_SAMPLE_VPT;   // blocked: thread t holds indices [i0, i0 + VPT)
  if (tid == 0) { s_nan = 0x7fffffff; s_digit = 0; s_kk = 1; }
  __syncthreads();
  uint32_t key[GD_SAMPLE_VPT];
  int nan_i = 0x7fffffff;
  if (i0 + GD_SAMPLE_VPT <= V) {
    // a whole span: loads at immediate offsets from one base address
    const float* b = L + i0;
#pragma unroll
    for (int j = 0; j < GD_SAMPLE_VPT; ++j) {
      const float f = b[j];
      key[j] = f == f ? sample_key(f) : 0u;
      if (f != f) nan_i = min(nan_i, i0 + j);
    }
  } else {
#pragma unroll
    for (int j = 0; j < GD_SAMPLE_VPT; ++j) {
      const int i = i0 + j;
      const float f = i < V ? L[i] : 0.f;
      key[j] = (i < V && f == f) ? sample_key(f) : 0u;
      if (i < V && f != f) nan_i = min(nan_i, i);
    }
  }
  if (nan_i != 0x7fffffff) atomicMin(&s_nan, nan_i);
  // radix select of the k-th largest key, 8 bits at a time from the top
  uint32_t prefix = 0, mask = 0;
  int kk = k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) s_hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < GD_SAMPLE_VPT; ++j)
      if ((key[j] & mask) == prefix && key[j] != 0u) atomicAdd(&s_hist[(key[j] >> shift) & 255u], 1u);
    __syncthreads();
    if (tid < 64) {
      // lane l holds bins 255 - 4l .. 252 - 4l (descending); suffix counts by lane scan
      int c[4], sum = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) { c[j] = (int)s_hist[255 - 4 * tid - j]; sum += c[j]; }
      int inc = sum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int x = __shfl_up(inc, o, 64);
        if (tid >= o) inc += x;
      }
      int before = inc - sum;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (before < kk && kk <= before + c[j]) { s_digit = 255 - 4 * tid - j; s_kk = kk - before; }
        before += c[j];
      }
    }
    __syncthreads();
    prefix |= (uint32_t)s_digit << shift;
    mask |= 255u << shift;
    kk = s_kk;
    __syncthreads();
  }
  // the candidates: every key above the k-th largest, then the kk lowest-index keys equal to it
  int n_gt = 0, n_eq = 0;
#pragma unroll
  for (int j = 0; j < GD_SAMPLE_VPT; ++j) {
    n_gt += key[j] > prefix;
    n_eq += key[j] == prefix;
  }
  int e_gt, e_eq, t_gt, t_eq;
  block_scan2(n_gt, n_eq, e_gt, e_eq, t_gt, t_eq, s_w);
#pragma unroll
  for (int j = 0; j < GD_SAMPLE_VPT; ++j) {
    // (bounds kept even when NaNs leave fewer than k keys: the NaN rule decides then)
    if (key[j] > prefix) {
      if (e_gt < GD_SAMPLE_MAX_K) { s_ck[e_gt] = key[j]; s_ci[e_gt] = i0 + j; }
      ++e_gt;
    } else if (key[j] == prefix) {
      if (e_eq < kk && t_gt + e_eq < GD_SAMPLE_MAX_K) { s_ck[t_gt + e_eq] = key[j]; s_ci[t_gt + e_eq] = i0 + j; }
      ++e_eq;
    }
  }
  __syncthreads();
  // rank order: larger logit first, ties to the lower index
  if (tid < k) {
    const uint32_t mk = s_ck[tid];
    const int mi = s_ci[tid];
    int r = 0;
    for (int j = 0; j < k; ++j) r += (s_ck[j] > mk) || (s_ck[j] == mk && s_ci[j] < mi);
    r = min(r, k - 1);
    s_sv[r] = sample_val(mk);
    s_si[r] = mi;
  }
  __syncthreads();
  if (tid != 0) return;
  if (s_nan != 0x7fffffff) { p.out[row] = s_nan; return; }
  const unsigned long long w0 = philox4x64_w0((unsigned long long)p.row_pos[row], (unsigned long long)p.row_seq[row],
                                              0ull, 0ull, p.seed, 0ull);
  const float u = (float)(w0 >> 40) * (1.0f / 16777216.0f);
  const float top = s_sv[0];
  float total = 0.f;
  for (int r = 0; r < k; ++r) total += expf((s_sv[r] - top) * p.inv_temp);
  const float target = u * total;
  float cum = 0.f;
  int pick = s_si[k - 1];
  for (int r = 0; r < k; ++r) {
    cum += expf((s_sv[r] - top) * p.inv_temp);
    if (target < cum) { pick = s_si[r]; break; }
  }
  p.out[row] = pick;
}
