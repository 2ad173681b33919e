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

// ----------------------------------------------------------------------------- wave exchanges
// Value of lane (lane ^ M), in VALU instructions only (no LDS round trip): DPP quad
// permutes for 1 and 2, DPP row rotates for 4 and 8, and gfx950's permlane16/32 swaps for
// 16 and 32.  Lane mappings were checked on the hardware.
template <int M>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
  const int x = (int)v;
  if constexpr (M == 1) {
    return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
  } else if constexpr (M == 2) {
    return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
  } else if constexpr (M == 4) {
    const int lo = __builtin_amdgcn_mov_dpp(x, 0x124, 0xF, 0xF, false);   // row_ror:4  (i <- i-4)
    const int hi = __builtin_amdgcn_mov_dpp(x, 0x12C, 0xF, 0xF, false);   // row_ror:12 (i <- i+4)
    return (uint32_t)((__lane_id() & 4) ? lo : hi);
  } else if constexpr (M == 8) {
    return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, false);  // row_ror:8
  } else if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (__lane_id() & 16) ? r[0] : r[1];
  } else {
    static_assert(M == 32, "xor distance must be a power of two below 64");
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (__lane_id() & 32) ? r[0] : r[1];
  }
}
// Run-time distance (folded to one case once the caller's loop is unrolled).
__device__ __forceinline__ uint32_t xor_lane_u32(uint32_t v, int m) {
  switch (m) {
    case 1: return xor_lane<1>(v);
    case 2: return xor_lane<2>(v);
    case 4: return xor_lane<4>(v);
    case 8: return xor_lane<8>(v);
    case 16: return xor_lane<16>(v);
    default: return xor_lane<32>(v);
  }
}
__device__ __forceinline__ uint64_t xor_lane_u64(uint64_t v, int m) {
  const uint32_t lo = xor_lane_u32((uint32_t)v, m), hi = xor_lane_u32((uint32_t)(v >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint32_t shfl_xor_u32(uint32_t v, int m) { return xor_lane_u32(v, m); }
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) { return xor_lane_u64(v, m); }
// Broadcast of lane `src` (wave-uniform) through a scalar register.
__device__ __forceinline__ uint32_t readlane_u32(uint32_t v, int src) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, src);
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int src) {
  return ((uint64_t)readlane_u32((uint32_t)(v >> 32), src) << 32) | readlane_u32((uint32_t)v, src);
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __uint_as_float(xor_lane_u32(__float_as_uint(v), m));
  return v;
}
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const uint64_t b = xor_lane_u64(__double_as_longlong(v), m);
    v += __longlong_as_double((long long)b);
  }
  return v;
}
__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += (int)xor_lane_u32((uint32_t)v, m);
  return v;
}
__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __uint_as_float(xor_lane_u32(__float_as_uint(v), m)));
  return v;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const uint64_t p = xor_lane_u64(v, m);
    v = p > v ? p : v;
  }
  return v;
}
// Inclusive prefix sum over the wave (Hillis-Steele with shuffles; off the per-token path).
__device__ __forceinline__ int wave_incl_scan_i32(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int p = __shfl_up(v, d, kWave);
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

// Descending bitonic sort across the wave of values replicated within aligned groups of L
// lanes (L a power of two, wave-uniform).  Stages whose partner lane lies inside the same
// group would compare equal values and are skipped, so G = 64/L groups cost
// log2(G)(log2(G)+1)/2 exchanges; the j-th largest group value ends at lane j*L.
__device__ __forceinline__ uint32_t bitonic64_desc_grouped(uint32_t v, int L) {
  const int lane = lane_id();
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride < L) continue;
      const uint32_t p = shfl_xor_u32(v, stride);
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
        const uint64_t hi = v0 > v1 ? v0 : v1, lo = v0 > v1 ? v1 : v0;
        v0 = hi;
        v1 = lo;
      } else {
        const uint64_t p0 = shfl_xor_u64(v0, stride), p1 = shfl_xor_u64(v1, stride);
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
