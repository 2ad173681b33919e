// Device-side helpers shared by the routing and GEMM kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(4))) int i32x4_t;
typedef __attribute__((ext_vector_type(2))) int i32x2_t;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// ----------------------------------------------------------------------------- sort keys
// Order-preserving map of an fp32 logit to u32: larger logit -> larger key.
// -0.0 is folded onto +0.0 so that the two tie.  Every finite or infinite
// input maps to a key >= 0x007FFFFF, so key 0 marks an empty slot.
__device__ __forceinline__ uint32_t logit_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_logit(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}
// Selection key: logit key in the high word, inverted expert index in the low
// word, so that the maximum is the larger logit and, on equal logits, the
// lower expert index.
__device__ __forceinline__ uint64_t pick_key(uint32_t key, int expert) {
  return ((uint64_t)key << 32) | (uint32_t)(~(uint32_t)expert);
}
__device__ __forceinline__ int pick_expert(uint64_t p) { return (int)(~(uint32_t)p); }
__device__ __forceinline__ uint32_t pick_logit_key(uint64_t p) { return (uint32_t)(p >> 32); }

// ----------------------------------------------------------------------------- wave shuffles
__device__ __forceinline__ uint32_t shfl_xor_u32(uint32_t v, int m) {
  return (uint32_t)__shfl_xor((int)v, m, kWave);
}
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = shfl_xor_u32((uint32_t)v, m), hi = shfl_xor_u32((uint32_t)(v >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  uint32_t lo = (uint32_t)__shfl((int)(uint32_t)v, src, kWave);
  uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(v >> 32), src, kWave);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}
__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}
__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    uint64_t p = shfl_xor_u64(v, m);
    v = p > v ? p : v;
  }
  return v;
}
// Inclusive prefix sum over the wave (Hillis-Steele with shuffles).
__device__ __forceinline__ int wave_incl_scan_i32(int v) {
  int lane = lane_id();
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int p = __shfl_up(v, d, kWave);
    if (lane >= d) v += p;
  }
  return v;
}

// Bitonic sort of one value per lane across the wave, descending by lane.
template <class T>
__device__ __forceinline__ T bitonic64_desc(T v) {
  const int lane = lane_id();
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      T p;
      if constexpr (sizeof(T) == 8) p = shfl_xor_u64(v, stride);
      else p = shfl_xor_u32(v, stride);
      const bool keep_max = ((lane & size) == 0) == ((lane & stride) == 0);
      v = keep_max ? (v > p ? v : p) : (v < p ? v : p);
    }
  }
  return v;
}

// Bitonic sort of 128 u64 values, v0 at position lane and v1 at lane+64, descending.
__device__ __forceinline__ void bitonic128_desc(uint64_t& v0, uint64_t& v1) {
  const int lane = lane_id();
#pragma unroll
  for (int size = 2; size <= 128; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride == 64) {
        // positions lane and lane+64 of one register pair; size == 128 here
        uint64_t hi = v0 > v1 ? v0 : v1, lo = v0 > v1 ? v1 : v0;
        v0 = hi;
        v1 = lo;
      } else {
        uint64_t p0 = shfl_xor_u64(v0, stride), p1 = shfl_xor_u64(v1, stride);
        const bool lower = (lane & stride) == 0;
        const bool km0 = ((lane & size) == 0) == lower;
        const bool km1 = (((lane + 64) & size) == 0) == lower;
        v0 = km0 ? (v0 > p0 ? v0 : p0) : (v0 < p0 ? v0 : p0);
        v1 = km1 ? (v1 > p1 ? v1 : p1) : (v1 < p1 ? v1 : p1);
      }
    }
  }
}

// Orders this wave's earlier LDS writes before its later LDS reads.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ----------------------------------------------------------------------------- number formats
// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Two fp32 -> two e4m3fn codes (low byte = a), hardware RNE conversion; the
// inputs are clamped to +-448 first because the conversion itself does not
// saturate.
__device__ __forceinline__ uint32_t pack_fp8x2(float a, float b) {
  a = fminf(fmaxf(a, -448.0f), 448.0f);
  b = fminf(fmaxf(b, -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + __expf(-g)) * u;
}

}  // namespace moe
