// misc.h -- step plumbing, embedding, standalone argmax.
#pragma once
#include "common.h"

// Per-row metadata and input embedding shared by decode and prefill.
struct RowParams {
  const int* table; int max_blocks, block_size, nblk, Hkv, hd;  // KV cache addressing
  const void* wte; const void* wpe; int vocab, n_pos, d, emb_bf16;
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
    if (!r.emb_bf16) v = reinterpret_cast<const float*>(r.wte)[(size_t)tok * r.d + i];
    else v = bf16_lo(reinterpret_cast<const uint16_t*>(r.wte)[(size_t)tok * r.d + i]);
    if (r.wpe) {
      if (!r.emb_bf16) v += reinterpret_cast<const float*>(r.wpe)[(size_t)ppos * r.d + i];
      else v += bf16_lo(reinterpret_cast<const uint16_t*>(r.wpe)[(size_t)ppos * r.d + i]);
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
