// misc.h -- step plumbing, embedding, standalone argmax.
#pragma once
#include "common.h"

// Decode step set-up, on the device so the step can be replayed as one graph:
// row b runs slot seq_ids[b] at its current length, which is then advanced.
__global__ void k_setup_decode(int B, const int* __restrict__ seq_ids, const int* __restrict__ tokens,
                               int* len, const int* __restrict__ cap, int* row_seq, int* row_pos,
                               int* row_tok, int* err) {
  int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  int s = seq_ids[b];
  int pos = len[s];
  if (pos >= cap[s]) { atomicOr(err, GD_DERR_POS); pos = cap[s] - 1; }
  row_seq[b] = s;
  row_pos[b] = pos;
  row_tok[b] = tokens[b];
  len[s] = pos + 1;
}

// x = wte[t] (+ wpe[p]) -- token embedding and learned positions ("bare-metal-llm",
// "Picking the model" and "What got built": embedding lookup).
template <int WT>
__global__ __launch_bounds__(GD_WG) void k_embed(const void* __restrict__ wte, const void* __restrict__ wpe,
                                                 int vocab, int n_pos, int d, const int* __restrict__ row_tok,
                                                 const int* __restrict__ row_pos, float* x, int ldx, int* err) {
  const int m = blockIdx.x;
  int t = row_tok[m];
  if (t < 0 || t >= vocab) { if (threadIdx.x == 0) atomicOr(err, GD_DERR_TOKEN); t = 0; }
  int pos = row_pos[m];
  if (wpe && (pos < 0 || pos >= n_pos)) { if (threadIdx.x == 0) atomicOr(err, GD_DERR_POS); pos = 0; }
  for (int i = threadIdx.x; i < d; i += GD_WG) {
    float v;
    if (WT == 0) v = reinterpret_cast<const float*>(wte)[(size_t)t * d + i];
    else v = bf16_lo(reinterpret_cast<const uint16_t*>(wte)[(size_t)t * d + i]);
    if (wpe) {
      if (WT == 0) v += reinterpret_cast<const float*>(wpe)[(size_t)pos * d + i];
      else v += bf16_lo(reinterpret_cast<const uint16_t*>(wpe)[(size_t)pos * d + i]);
    }
    x[(size_t)m * ldx + i] = v;
  }
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
