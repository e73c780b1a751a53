// common.h -- device helpers shared by the decode kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define GD_WG 256          // threads per workgroup for every kernel here (4 waves)
#define GD_MAX_ROWS 32     // rows (sequences or prompt positions) per forward call
#define GD_TILE_N 16       // output columns per linear tile
#define GD_ATT_NCH 8       // context chunks (attention workgroups) per row and KV head
#define GD_ATT_NCH_LONG 32 // chunks for long contexts with few rows (merged by a launch of their own)
#define GD_MAX_HEADS 32    // query heads per layer
// Split-context attention partials, per (row, query head, chunk): the running max, the
// sum of weights, two unused words (so that the values start 16-byte aligned) and the
// hd unnormalized weighted sums of V.
#define GD_APART_O 4
__host__ __device__ constexpr int gd_apart_stride(int hd) { return hd + GD_APART_O; }

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Device error flag bits (mirrors gd_device_errors).
#define GD_DERR_TOKEN 1
#define GD_DERR_POS 2
#define GD_DERR_BLOCK 4

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// Signed byte j (0..3) of a word, as float (8-bit block weights).
__device__ __forceinline__ float q8_at(uint32_t w, int j) { return (float)((int32_t)(w << (24 - 8 * j)) >> 24); }
// Four int8 codes of a word times the block scale.
__device__ __forceinline__ f32x4 q8x4(uint32_t w, float s) {
  return (f32x4){q8_at(w, 0) * s, q8_at(w, 1) * s, q8_at(w, 2) * s, q8_at(w, 3) * s};
}
// float -> bfloat16 bits, rounded to nearest with ties to even (NaN kept a NaN).
__device__ __forceinline__ uint16_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// Eight consecutive weights starting at element k of row `row` (16-byte aligned).
template <int WT>
__device__ __forceinline__ void load_w8(const void* __restrict__ W, size_t row_off, int k, float w[8]) {
  if (WT == 0) {
    const f32x4* p = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(W) + row_off + k);
    f32x4 a = __builtin_nontemporal_load(p);
    f32x4 b = __builtin_nontemporal_load(p + 1);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  } else {
    const u32x4* p = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(W) + row_off + k);
    u32x4 u = __builtin_nontemporal_load(p);
    w[0] = bf16_lo(u.x); w[1] = bf16_hi(u.x);
    w[2] = bf16_lo(u.y); w[3] = bf16_hi(u.y);
    w[4] = bf16_lo(u.z); w[5] = bf16_hi(u.z);
    w[6] = bf16_lo(u.w); w[7] = bf16_hi(u.w);
  }
}

// Cross-lane reductions with DPP (data-parallel primitives: the lane permutation is
// part of the VALU instruction, no LDS traffic). Steps: quad_perm (1,0,3,2) and
// (2,3,0,1) sum pairs then quads, row_half_mirror adds the other quad of each group of
// 8, row_mirror the other half of each row of 16; the four rows of the wave are
// combined through readlane. Every lane of a group gets the group's result.
#define DPP_QUAD_1032 0xB1
#define DPP_QUAD_2301 0x4E
#define DPP_ROW_MIRROR 0x140
#define DPP_ROW_HALF_MIRROR 0x141

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of G lanes (G = 4, 8, 16 or 64); every lane gets the sum.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(G == 4 || G == 8 || G == 16 || G == 64, "group size");
  v += dpp_f<DPP_QUAD_1032>(v);
  v += dpp_f<DPP_QUAD_2301>(v);
  if (G >= 8) v += dpp_f<DPP_ROW_HALF_MIRROR>(v);
  if (G >= 16) v += dpp_f<DPP_ROW_MIRROR>(v);
  if (G == 64) {
    const int b = __float_as_int(v);
    v = (__int_as_float(__builtin_amdgcn_readlane(b, 0)) + __int_as_float(__builtin_amdgcn_readlane(b, 16))) +
        (__int_as_float(__builtin_amdgcn_readlane(b, 32)) + __int_as_float(__builtin_amdgcn_readlane(b, 48)));
  }
  return v;
}

// Maximum over aligned groups of G lanes (G = 8, 16 or 64).
template <int G>
__device__ __forceinline__ float group_max(float v) {
  static_assert(G == 8 || G == 16 || G == 64, "group size");
  v = fmaxf(v, dpp_f<DPP_QUAD_1032>(v));
  v = fmaxf(v, dpp_f<DPP_QUAD_2301>(v));
  v = fmaxf(v, dpp_f<DPP_ROW_HALF_MIRROR>(v));
  if (G >= 16) v = fmaxf(v, dpp_f<DPP_ROW_MIRROR>(v));
  if (G == 64) {
    const int b = __float_as_int(v);
    v = fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 0)), __int_as_float(__builtin_amdgcn_readlane(b, 16))),
              fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 32)), __int_as_float(__builtin_amdgcn_readlane(b, 48))));
  }
  return v;
}

__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }

// Wave sums of NV values at once: each DPP step is applied to all of them, so the
// reductions overlap instead of running one after another.
template <int NV>
__device__ __forceinline__ void wave_sum_n(float (&v)[NV]) {
#pragma unroll
  for (int k = 0; k < NV; ++k) v[k] += dpp_f<DPP_QUAD_1032>(v[k]);
#pragma unroll
  for (int k = 0; k < NV; ++k) v[k] += dpp_f<DPP_QUAD_2301>(v[k]);
#pragma unroll
  for (int k = 0; k < NV; ++k) v[k] += dpp_f<DPP_ROW_HALF_MIRROR>(v[k]);
#pragma unroll
  for (int k = 0; k < NV; ++k) v[k] += dpp_f<DPP_ROW_MIRROR>(v[k]);
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int b = __float_as_int(v[k]);
    v[k] = (__int_as_float(__builtin_amdgcn_readlane(b, 0)) + __int_as_float(__builtin_amdgcn_readlane(b, 16))) +
           (__int_as_float(__builtin_amdgcn_readlane(b, 32)) + __int_as_float(__builtin_amdgcn_readlane(b, 48)));
  }
}

__device__ __forceinline__ float wave_max(float v) { return group_max<64>(v); }

// Agent-scope (whole device) atomics and fences for the last-arriver reductions.
__device__ __forceinline__ int atomic_add_acq_rel(int* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_relaxed(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void fence_agent() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "agent"); }

// tanh-GELU with the tanh argument clamped to [-15, 15] (tanh is +-1 in float there),
// so that no evaluation path of tanh can overflow to Inf/Inf ("bare-metal-llm",
// "The bug worth telling"; "batch_forge", the GELU clamp paragraph).
__device__ __forceinline__ float gelu_clamped(float u) {
  float a = 0.7978845608028654f * (u + 0.044715f * u * u * u);
  a = fminf(fmaxf(a, -15.0f), 15.0f);
  return 0.5f * u * (1.0f + tanhf(a));
}

// silu(z) = z / (1 + e^-z) ("rvllm Metal backend", "What the kernels do").
__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// Greedy argmax combine: NaN beats every number, the first NaN wins, ties go to the
// lower index. Returns true if (vb, ib) should replace (va, ia).
__device__ __forceinline__ bool am_better(float vb, int ib, float va, int ia) {
  bool nb = vb != vb, na = va != va;
  if (na && nb) return ib < ia;
  if (na) return false;
  if (nb) return true;
  if (vb > va) return true;
  if (vb < va) return false;
  return ib < ia;
}
