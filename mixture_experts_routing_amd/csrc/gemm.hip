// Two-stage expert GEMM on MFMA (gfx950): stage 1 gate-up + SiLU-mul, stage 2 down
// projection + routed weight + scatter.
//
// [P2] "[MoE] Port moe_gemm_2stage (stage1+stage2) to the new fx.* pipeline -- fp8
// (gfx942 + gfx950)" (ROCm/FlyDSL #947): B-first MFMA (the weight is the first
// operand, the gathered activation rows the second), rows gathered through the
// sorted ids with sentinel rows contributing zero, silu(gate)*up producing bf16,
// per-token x per-channel fp8 dequant in the stage-2 epilogue, routed weight,
// atomic or reduce epilogue, padding lanes issuing no atomics.
//
// Decode kernels (gemm1_kernel, gemm2_kernel; one 256-thread workgroup = 4 waves):
//  * block = one BLOCK_M-row block of the sorted list (one expert) x one tile of
//    output channels.  Blocks past num_valid exit at once.
//  * each wave owns two 16-row groups of weight rows (stage 1: 16 gate rows and the
//    matching 16 up rows; stage 2: 32 consecutive model_dim rows) and streams
//    them straight from HBM into registers; K may be split over the block's waves.
//    The gathered activation rows are read per wave from L2.
//  * MFMA: bf16 16x16x32 (two per 128-byte chunk) or fp8 e4m3 16x16x128 (one per
//    chunk).  Lane (i, g) = (lane % 16, lane / 16) carries bytes [16g, 16g+16) and
//    [64+16g, 64+16g+16) of row i of the chunk for both operands; the MFMA sums over K,
//    so this common permutation of K leaves the result unchanged.
//  * accumulator lane layout: lane (j, g) holds output rows 4g..4g+3 (channels)
//    of column j (the j-th gathered row), so a lane owns 4 consecutive channels
//    of one slot.
// The prefill kernel (gemm_prefill_kernel, further down) tiles many rows per expert.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

struct alignas(16) u32x4 {
  uint32_t x, y, z, w;
};

__device__ __forceinline__ i32x4_t ld16(const uint8_t* p) {
  return *reinterpret_cast<const i32x4_t*>(p);
}
// The same for bytes read exactly once per call (decode weight rows): non-temporal, so the
// caches keep the rows that are reused (gathered activations, sorted lists).
__device__ __forceinline__ i32x4_t ld16_stream(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const i32x4_t*>(p));
}

// Output modes of stage 2 (moe_mode): fp32 atomic accumulation, fp32 slot rows, packed
// bf16 atomic accumulation straight into the bf16 output, or bf16 slot rows.
enum { OM_ATOMIC = 0, OM_REDUCE = 1, OM_ATOMIC_BF16 = 2, OM_REDUCE_BF16 = 3 };

// out[0..1] += (lo, hi): both values rounded to bf16 (nearest even), then one packed bf16
// atomic add (the sum is rounded to bf16 again); out must be 4-byte aligned.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void atomic_add_bf16x2(uint16_t* out, float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  __builtin_amdgcn_global_atomic_fadd_v2bf16((__attribute__((address_space(1))) bf16x2_t*)out, v);
}

// Block -> (row block, channel tile).  Workgroups are handed to the 8 XCDs round
// robin by id, so id L runs on XCD L % 8.  Each XCD is given one contiguous range
// of the (tile-major, row-block-minor) order: the row blocks of one expert that
// share a weight tile then run on the same XCD and share its L2.
__device__ __forceinline__ bool block_tile(int mbs, int nts, int& mb, int& nt) {
  const int n = mbs * nts;
  const int per = (n + 7) >> 3;
  const int L = (int)blockIdx.x;
  const int v = (L & 7) * per + (L >> 3);
  if (v >= n) return false;
  nt = v / mbs;
  mb = v - nt * mbs;
  return true;
}
// The same with the (row-block-major, tile-minor) order: all weight tiles of a row block, and
// the row blocks of one expert, run next to each other on one XCD, which then fetches the
// gathered rows once for all weight tiles and each weight tile once for the expert's blocks.
__device__ __forceinline__ bool block_tile_rows(int mbs, int nts, int& mb, int& nt) {
  const int n = mbs * nts;
  const int per = (n + 7) >> 3;
  const int L = (int)blockIdx.x;
  const int v = (L & 7) * per + (L >> 3);
  if (v >= n) return false;
  mb = v / nts;
  nt = v - mb * nts;
  return true;
}
static inline unsigned xcd_grid(int64_t mbs, int64_t nts) {
  return (unsigned)(((mbs * nts + 7) / 8) * 8);
}

// 16 bytes per lane from global memory straight into LDS at lds + 16 * lane (lds is the
// wave-uniform LDS byte address, in M0).  Written as assembly so that the compiler, which
// does not see these loads, keeps its own waits on the register loads around them (loads
// it does not count only make its counts conservative) and inserts no blanket wait before
// LDS reads; the code that uses the staged bytes waits for them explicitly.
// The same with a wave-uniform 64-bit base and a 32-bit per-lane offset.
__device__ __forceinline__ void dma16_to_lds_s(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base),
               "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}
// The same, non-temporal: for bytes no other tile reads again soon (prefill weight chunks).
__device__ __forceinline__ void dma16_to_lds_s_nt(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(off), "s"(base),
               "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}
// 4 bytes per lane (lane l's at lds + 4 l), the same way; base must be wave-uniform.
__device__ __forceinline__ void dma4_to_lds_s(const void* base, uint32_t off, uint32_t lds) {
  const uint64_t b = reinterpret_cast<uintptr_t>(base);
  const uint64_t ub = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(b >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(reinterpret_cast<const void*>(ub)),
               "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}
__device__ __forceinline__ void dma16_to_lds(const void* g, uint32_t lds) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m0v) : "memory");
}

template <bool FP8>
__device__ __forceinline__ void mfma_chunk(f32x4_t& acc, const i32x4_t (&a)[2], const i32x4_t (&b)[2]) {
  if constexpr (FP8) {
    i32x8_t av = {a[0][0], a[0][1], a[0][2], a[0][3], a[1][0], a[1][1], a[1][2], a[1][3]};
    i32x8_t bv = {b[0][0], b[0][1], b[0][2], b[0][3], b[1][0], b[1][1], b[1][2], b[1][3]};
    // A/B format 0 = fp8 e4m3; block scales 127 = 2^0
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 0, 0, 0, 127, 0, 127);
  } else {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[0]),
                                                 __builtin_bit_cast(bf16x8_t, b[0]), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[1]),
                                                 __builtin_bit_cast(bf16x8_t, b[1]), acc, 0, 0, 0);
  }
}

// Element types of the GEMM operands (moe_dtype).
enum { DT_BF16 = 0, DT_FP8 = 1, DT_FP4 = 2 };

// MXFP4 chunk (128 bytes = 256 E2M1 elements per row): two 16x16x128 MFMAs in format 4
// (FP4 E2M1).  Lane (i, g) holds bytes [16g, 16g+16) of row i for the first and
// [64+16g, 64+16g+16) for the second: 32 elements each, exactly one MX block, whose E8M0
// scale the lane supplies (sa*, sb* in the low byte).  The MFMA reads four registers per
// operand in this format; the upper four are left undefined.
__device__ __forceinline__ void mfma_fp4(f32x4_t& acc, const i32x4_t (&a)[2], const i32x4_t (&b)[2],
                                         int sa0, int sa1, int sb0, int sb1) {
  const i32x8_t a0 = __builtin_shufflevector(a[0], a[0], 0, 1, 2, 3, -1, -1, -1, -1);
  const i32x8_t b0 = __builtin_shufflevector(b[0], b[0], 0, 1, 2, 3, -1, -1, -1, -1);
  const i32x8_t a1 = __builtin_shufflevector(a[1], a[1], 0, 1, 2, 3, -1, -1, -1, -1);
  const i32x8_t b1 = __builtin_shufflevector(b[1], b[1], 0, 1, 2, 3, -1, -1, -1, -1);
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a0, b0, acc, 4, 4, 0, sa0, 0, sb0);
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a1, b1, acc, 4, 4, 0, sa1, 0, sb1);
}

// Streams the byte range [kb0, kb1) of K (rows are kbytes long; kb0, kb1 multiples of
// 128) for NG weight-row groups against NT gathered activation tiles.  wrow[ng]: this
// lane's weight row; xrow[tt]: this lane's activation row (nullptr = padding row,
// contributes zero).  Within a 128-byte chunk, lane group g takes bytes [16g, 16g+16)
// and [64+16g, 64+16g+16), so each load instruction covers 64 contiguous bytes per row.
// The last chunk of an fp8 (fp4) row may be half: 64 bytes; its second half reads as zero.
// FP4: wsc / xsc point at the rows' E8M0 scales (8 per chunk); lane group g takes the
// scales of blocks g and 4 + g of each chunk (a padding row takes 2^0), with one 8-byte load
// per row and chunk when the scale rows are 8-byte aligned (K % 256 == 0), else two 4-byte
// loads.
// Weight rows: wrow[ng] already holds this lane's part of the address.  Natural layout
// (PRE false): chunk kb of the lane's row at wrow + kb, its second half 64 bytes on.
// Fragment-order layout (PRE true): the 16-row group's chunk kb at wrow + 16 kb, second half
// 1024 bytes on (see preshuffle_kernel); mxfp4 scales in fragment order too
// (preshuffle_scales_kernel).
template <int DT, int NG, int NT, int U, bool PRE>
__device__ __forceinline__ void mainloop(const uint8_t* const (&wrow)[NG],
                                         const uint8_t* const (&xrow)[NT],
                                         const uint8_t* const (&wsc)[NG],
                                         const uint8_t* const (&xsc)[NT], int kb0, int kb1,
                                         int kbytes, f32x4_t (&acc)[NG][NT]) {
  constexpr bool FP4 = DT == DT_FP4;
  constexpr int wshift = PRE ? 4 : 0, whalf = PRE ? 1024 : 64;
  // fragment order: each weight load covers 1 KB of whole lines, read once per call, so it
  // is non-temporal; the natural layout reads each line in two halves by two loads, and the
  // line must stay cached between them
  auto wld = [](const uint8_t* q) { return PRE ? ld16_stream(q) : ld16(q); };
  const int g = lane_id() >> 4, g16 = g * 16;
  const i32x4_t zero = {0, 0, 0, 0};
  const bool pair8 = (kbytes & 127) == 0;  // scale rows of kbytes / 16 bytes, a multiple of 8
  // activation tiles with at least one real row (wave-uniform): a tile of padding rows
  // issues no loads at all (at decode sizes most tiles of a 64-row block are padding)
  bool live[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) live[tt] = __ballot(xrow[tt] != nullptr) != 0;
  // scale bytes of chunk kb for blocks (g, 4 + g); a half chunk has no second block
  // the two scale words of chunk kb (a padding row: 2^0 everywhere)
  auto scales = [&](const uint8_t* r, int kb, bool in1) -> uint2 {
    if (!r) return make_uint2(0x7F7F7F7Fu, 0x7F7F7F7Fu);
    if (in1 && pair8) return *reinterpret_cast<const uint2*>(r + kb / 16);
    const uint32_t lo = *reinterpret_cast<const uint32_t*>(r + kb / 16);
    return make_uint2(lo, in1 ? *reinterpret_cast<const uint32_t*>(r + kb / 16 + 4) : 0x7F7F7F7Fu);
  };
  auto byte_g = [&](uint32_t w) { return (int)((w >> (8 * g)) & 0xFFu); };
  // weight scales: in fragment order (PRE; wsc points at the lane's 8 bytes of the group's
  // first chunk, whole chunks only) chunk kb's line is kb bytes on; else the natural rows
  auto wscales = [&](const uint8_t* r, int kbb, bool in1) -> uint2 {
    if constexpr (PRE) return *reinterpret_cast<const uint2*>(r + kbb);
    return scales(r, kbb, in1);
  };
  int kb = kb0;
  const int kend_full = kb1 < (kbytes & ~127) ? kb1 : (kbytes & ~127);
  for (; kb + 128 * U <= kend_full; kb += 128 * U) {
    i32x4_t wa[U][NG][2], xb[U][NT][2];
    uint2 wsa[U][NG], xsa[U][NT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int off = kb + 128 * u + g16;
      const int woff = (kb + 128 * u) << wshift;
#pragma unroll
      for (int ng = 0; ng < NG; ++ng) {
        wa[u][ng][0] = wld(wrow[ng] + woff);
        wa[u][ng][1] = wld(wrow[ng] + woff + whalf);
        if constexpr (FP4) wsa[u][ng] = wscales(wsc[ng], kb + 128 * u, true);
      }
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        xb[u][tt][0] = xb[u][tt][1] = zero;
        if constexpr (FP4) xsa[u][tt] = make_uint2(0x7F7F7F7Fu, 0x7F7F7F7Fu);
        if (live[tt]) {
          xb[u][tt][0] = xrow[tt] ? ld16(xrow[tt] + off) : zero;
          xb[u][tt][1] = xrow[tt] ? ld16(xrow[tt] + off + 64) : zero;
          if constexpr (FP4) xsa[u][tt] = scales(xsc[tt], kb + 128 * u, true);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int ng = 0; ng < NG; ++ng)
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
          if constexpr (FP4)
            mfma_fp4(acc[ng][tt], wa[u][ng], xb[u][tt], byte_g(wsa[u][ng].x), byte_g(wsa[u][ng].y),
                     byte_g(xsa[u][tt].x), byte_g(xsa[u][tt].y));
          else
            mfma_chunk<DT == DT_FP8>(acc[ng][tt], wa[u][ng], xb[u][tt]);
        }
  }
  for (; kb < kb1 && kb < kbytes; kb += 128) {
    const int off = kb + g16;
    const int woff = kb << wshift;
    const bool in1 = kb + 64 < kbytes;
    i32x4_t wa[NG][2], xb[NT][2];
    uint2 wsa[NG], xsa[NT];
#pragma unroll
    for (int ng = 0; ng < NG; ++ng) {
      wa[ng][0] = wld(wrow[ng] + woff);
      wa[ng][1] = in1 ? wld(wrow[ng] + woff + whalf) : zero;
      if constexpr (FP4) wsa[ng] = wscales(wsc[ng], kb, in1);
    }
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      xb[tt][0] = xb[tt][1] = zero;
      if constexpr (FP4) xsa[tt] = make_uint2(0x7F7F7F7Fu, 0x7F7F7F7Fu);
      if (live[tt]) {
        xb[tt][0] = xrow[tt] ? ld16(xrow[tt] + off) : zero;
        xb[tt][1] = (in1 && xrow[tt]) ? ld16(xrow[tt] + off + 64) : zero;
        if constexpr (FP4) xsa[tt] = scales(xsc[tt], kb, in1);
      }
    }
#pragma unroll
    for (int ng = 0; ng < NG; ++ng)
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        if constexpr (FP4)
          mfma_fp4(acc[ng][tt], wa[ng], xb[tt], byte_g(wsa[ng].x), byte_g(wsa[ng].y), byte_g(xsa[tt].x),
                   byte_g(xsa[tt].y));
        else
          mfma_chunk<DT == DT_FP8>(acc[ng][tt], wa[ng], xb[tt]);
      }
  }
}

// K split over KS waves of a block: wave kp takes chunks [kp*n/KS, (kp+1)*n/KS).
__device__ __forceinline__ void k_range(int kbytes, int kp, int ks, int& kb0, int& kb1) {
  const int nch = (kbytes + 127) >> 7;
  kb0 = (kp * nch / ks) * 128;
  kb1 = ((kp + 1) * nch / ks) * 128;
}

// Sums the partial accumulators of the KS waves that share a row group into the
// wave with kp == 0 (LDS, one barrier).  Returns false on the other waves.
template <int KS, int RG, int NG, int NT>
__device__ __forceinline__ bool reduce_k_split(f32x4_t (&acc)[NG][NT], int rg, int kp,
                                               f32x4_t* red) {
  if constexpr (KS == 1) {
    return true;
  } else {
    const int lane = lane_id();
    if (kp > 0) {
#pragma unroll
      for (int a = 0; a < NG; ++a)
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
          red[((((kp - 1) * RG + rg) * NG + a) * NT + tt) * 64 + lane] = acc[a][tt];
    }
    __syncthreads();
    if (kp > 0) return false;
#pragma unroll
    for (int q = 1; q < KS; ++q)
#pragma unroll
      for (int a = 0; a < NG; ++a)
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) acc[a][tt] += red[((((q - 1) * RG + rg) * NG + a) * NT + tt) * 64 + lane];
    return true;
  }
}

// ----------------------------------------------------------------------------- stage 1
// Block = 4 waves = RG = 4/KS row groups x KS parts of K.  A row group is 16 gate
// channels and the matching 16 up channels.  grid: I/(16*RG) channel tiles x cap/BM
// row blocks (see block_tile).  Output: bf16 rows a[s, I] (for fp8 the pre-requant
// rows).  If zero_y is set, the blocks first clear that fp32 buffer (stage 2's
// accumulator), which saves a launch.
template <int BM, int DT, int U, int KS>
__global__ void __launch_bounds__(256) gemm1_kernel(
    const uint8_t* __restrict__ x, const void* __restrict__ x_scale_v,
    const uint8_t* __restrict__ w1, const void* __restrict__ w1_scale_v,
    const int32_t* __restrict__ sorted_ids, const int32_t* __restrict__ expert_ids,
    const int32_t* __restrict__ num_valid, int T, int E, int k, int D, int I, int mbs,
    uint16_t* __restrict__ a_out, float4* __restrict__ zero_y, int64_t zero_n4, int pre) {
  constexpr int NT = BM / 16;
  constexpr int RG = 4 / KS;
  constexpr bool FP8 = DT == DT_FP8, FP4 = DT == DT_FP4;
  const float* x_scale = static_cast<const float*>(x_scale_v);
  const float* w1_scale = static_cast<const float*>(w1_scale_v);
  __shared__ f32x4_t red[KS > 1 ? (KS - 1) * RG * 2 * NT * 64 : 1];
  if (zero_y)
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < zero_n4; i += (int64_t)gridDim.x * 256)
      zero_y[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  int mb, nt;
  if (!block_tile(mbs, I / (16 * RG), mb, nt)) return;
  if (mb * BM >= *num_valid) return;
  const int e = expert_ids[mb];
  if ((unsigned)e >= (unsigned)E) return;  // defensive: ids come from the routing step
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int rg = wave / KS, kp = wave % KS;
  const int i16 = lane & 15, g = lane >> 4;
  const int n_w = nt * 16 * RG + rg * 16;  // first gate channel of this row group
  const int n_slots = T * k;
  const int rowb = DT == DT_BF16 ? D * 2 : DT == DT_FP8 ? D : D / 2;
  const int rows_s = D / 32;  // FP4: E8M0 scales per row
  // weight rows n_w.. (gate) and I + n_w.. (up) of expert e: 16-row groups
  const size_t lane_w = pre ? (size_t)lane * 16 : (size_t)i16 * rowb + 16 * g;
  const uint8_t* wrow[2] = {w1 + ((size_t)e * 2 * I + n_w) * rowb + lane_w,
                            w1 + ((size_t)e * 2 * I + I + n_w) * rowb + lane_w};
  const uint8_t* wsc[2] = {nullptr, nullptr};
  if constexpr (FP4) {
    const uint8_t* ws8 = static_cast<const uint8_t*>(w1_scale_v);
    // fragment order: group base (rows n_w, I + n_w are multiples of 16) + this row's 8 bytes
    wsc[0] = pre ? ws8 + ((size_t)e * 2 * I + n_w) * rows_s + i16 * 8 : ws8 + ((size_t)e * 2 * I + n_w + i16) * rows_s;
    wsc[1] = pre ? ws8 + ((size_t)e * 2 * I + I + n_w) * rows_s + i16 * 8
                 : ws8 + ((size_t)e * 2 * I + I + n_w + i16) * rows_s;
  }
  const uint8_t* xrow[NT];
  const uint8_t* xsc[NT];
  int slot[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const int s = sorted_ids[mb * BM + tt * 16 + i16];
    slot[tt] = s;
    const bool real = (unsigned)s < (unsigned)n_slots;
    xrow[tt] = real ? x + (size_t)(s / k) * rowb : nullptr;
    xsc[tt] = FP4 && real ? static_cast<const uint8_t*>(x_scale_v) + (size_t)(s / k) * rows_s : nullptr;
  }
  f32x4_t acc[2][NT];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) acc[a][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  int kb0, kb1;
  k_range(rowb, kp, KS, kb0, kb1);
  if (pre) mainloop<DT, 2, NT, U, true>(wrow, xrow, wsc, xsc, kb0, kb1, rowb, acc);
  else mainloop<DT, 2, NT, U, false>(wrow, xrow, wsc, xsc, kb0, kb1, rowb, acc);
  if (!reduce_k_split<KS, RG, 2, NT>(acc, rg, kp, red)) return;

  const int n0 = n_w + 4 * g;  // this lane's 4 channels
  float sg[4] = {1.f, 1.f, 1.f, 1.f}, su[4] = {1.f, 1.f, 1.f, 1.f};
  if constexpr (FP8) {
    const float* ws = w1_scale + (size_t)e * 2 * I;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sg[r] = ws[n0 + r];
      su[r] = ws[I + n0 + r];
    }
  }
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const int s = slot[tt];
    if ((unsigned)s >= (unsigned)n_slots) continue;
    float xs = 1.f;
    if constexpr (FP8) xs = x_scale[s / k];
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float gg = acc[0][tt][r] * (sg[r] * xs);
      const float uu = acc[1][tt][r] * (su[r] * xs);
      v[r] = silu_mul(gg, uu);
    }
    uint2 pk;
    pk.x = pack_bf16x2(v[0], v[1]);
    pk.y = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<uint2*>(a_out + (size_t)s * I + n0) = pk;
  }
}

// fp8: per slot row, scale = amax/448 (1 for a zero row), codes = e4m3(a/scale).
// One wave per row; rows of at most 512 NQ values are read once into registers (8 values per
// lane and 512-value group), so the conversion does not read the row again after the
// amax reduction; longer rows (NQ = 0) read it twice.
template <int NQ>
__global__ void __launch_bounds__(256) requant_rows_kernel(const uint16_t* __restrict__ a_bf16,
                                                           int rows, int I,
                                                           uint8_t* __restrict__ a_codes,
                                                           float* __restrict__ a_scale) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = lane_id();
  const uint16_t* src = a_bf16 + (size_t)row * I;
  auto convert = [&](const u32x4& v, int c, float scale) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t out[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t lo = pack_fp8x2(bf16_bits_to_f32(w[2 * q] & 0xFFFFu) / scale,
                                     bf16_bits_to_f32(w[2 * q] >> 16) / scale);
      const uint32_t hi = pack_fp8x2(bf16_bits_to_f32(w[2 * q + 1] & 0xFFFFu) / scale,
                                     bf16_bits_to_f32(w[2 * q + 1] >> 16) / scale);
      out[q] = lo | (hi << 16);
    }
    *reinterpret_cast<uint2*>(a_codes + (size_t)row * I + c) = make_uint2(out[0], out[1]);
  };
  auto vmax = [](float m, const u32x4& v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q)
      m = fmaxf(m, fmaxf(fabsf(bf16_bits_to_f32(w[q] & 0xFFFFu)), fabsf(bf16_bits_to_f32(w[q] >> 16))));
    return m;
  };
  float amax = 0.f;
  if constexpr (NQ > 0) {
    u32x4 v[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int c = lane * 8 + 512 * q;
      v[q] = c < I ? *reinterpret_cast<const u32x4*>(src + c) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) amax = vmax(amax, v[q]);
    amax = wave_max_f32(amax);
    const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
#pragma unroll
    for (int q = 0; q < NQ; ++q)
      if (lane * 8 + 512 * q < I) convert(v[q], lane * 8 + 512 * q, scale);
    if (lane == 0) a_scale[row] = scale;
  } else {
    for (int c = lane * 8; c < I; c += 512) amax = vmax(amax, *reinterpret_cast<const u32x4*>(src + c));
    amax = wave_max_f32(amax);
    const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
    for (int c = lane * 8; c < I; c += 512) convert(*reinterpret_cast<const u32x4*>(src + c), c, scale);
    if (lane == 0) a_scale[row] = scale;
  }
}

// MXFP4: each block of 32 consecutive bf16 values of a slot row becomes one E8M0 scale
// 2^(floor(log2 amax) - 2) (an all-zero block takes 2^0) and 32 E2M1 codes of value/scale,
// rounded to nearest even on the E2M1 grid (0, 0.5, 1, 1.5, 2, 3, 4, 6) and saturated at 6;
// element 2j in the low nibble.  value/scale is exact (a power-of-two scaling), so only the
// final rounding decides, on exact values.  One thread per block.
__device__ __forceinline__ uint32_t e2m1_code(float v, int shift) {
  const float y = fabsf(ldexpf(v, shift));
  const uint32_t m = y <= 0.25f ? 0u : y < 0.75f ? 1u : y <= 1.25f ? 2u : y < 1.75f ? 3u
                   : y <= 2.5f  ? 4u : y < 3.5f  ? 5u : y <= 5.0f  ? 6u : 7u;
  return m | (__float_as_uint(v) >> 31 << 3);
}
__global__ void __launch_bounds__(256) requant_mx_kernel(const uint16_t* __restrict__ a_bf16,
                                                         int64_t nblocks,
                                                         uint8_t* __restrict__ a_codes,
                                                         uint8_t* __restrict__ a_scale) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  const u32x4* src = reinterpret_cast<const u32x4*>(a_bf16 + b * 32);
  uint32_t w[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x4 v = src[q];
    w[4 * q] = v.x;
    w[4 * q + 1] = v.y;
    w[4 * q + 2] = v.z;
    w[4 * q + 3] = v.w;
  }
  float amax = 0.f;
#pragma unroll
  for (int q = 0; q < 16; ++q)
    amax = fmaxf(amax, fmaxf(fabsf(bf16_bits_to_f32(w[q] & 0xFFFFu)), fabsf(bf16_bits_to_f32(w[q] >> 16))));
  int ex = 0;
  frexpf(amax, &ex);  // amax = m 2^ex, m in [0.5, 1): floor(log2 amax) = ex - 1
  const int e = amax > 0.f ? min(254, max(0, ex - 1 - 2 + 127)) : 127;
  const int shift = 127 - e;  // value / 2^(e - 127)
  uint32_t out[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t o = 0;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const uint32_t p = w[4 * q + h];
      o |= (e2m1_code(bf16_bits_to_f32(p & 0xFFFFu), shift) | (e2m1_code(bf16_bits_to_f32(p >> 16), shift) << 4)) << (8 * h);
    }
    out[q] = o;
  }
  *reinterpret_cast<uint4*>(a_codes + b * 16) = make_uint4(out[0], out[1], out[2], out[3]);
  a_scale[b] = (uint8_t)e;
}

// ----------------------------------------------------------------------------- stage 2
// Block = 4 waves = RG = 4/KS row groups x KS parts of K; a row group is 16*NG
// model_dim rows (NG = 2, or 4 for short rows without a K split: see gemm2_ks).
// grid: ceil(D/(16*NG*RG)) channel tiles x cap/BM row blocks.
template <int BM, int DT, int U, int OM, int KS, int NG>
__global__ void __launch_bounds__(256) gemm2_kernel(
    const uint8_t* __restrict__ a, const void* __restrict__ a_scale_v,
    const uint8_t* __restrict__ w2, const void* __restrict__ w2_scale_v,
    const float* __restrict__ topk_w, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ expert_ids, const int32_t* __restrict__ num_valid, int T, int E,
    int k, int D, int I, int mbs, void* __restrict__ y, int pre) {
  constexpr int NT = BM / 16;
  constexpr int RG = 4 / KS;
  constexpr bool FP8 = DT == DT_FP8, FP4 = DT == DT_FP4;
  const float* a_scale = static_cast<const float*>(a_scale_v);
  const float* w2_scale = static_cast<const float*>(w2_scale_v);
  __shared__ f32x4_t red[KS > 1 ? (KS - 1) * RG * NG * NT * 64 : 1];
  int mb, nt;
  if (!block_tile(mbs, (D + 16 * NG * RG - 1) / (16 * NG * RG), mb, nt)) return;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int rg = wave / KS, kp = wave % KS;
  const int d_w = nt * 16 * NG * RG + rg * 16 * NG;
  // a partial last tile only happens with KS == 1 (the host keeps D % (32*RG) == 0
  // otherwise, with NG == 2), so leaving here never skips a barrier; D % 64 == 0 keeps a
  // wave's 16*NG rows inside D once d_w < D
  if (KS == 1 && d_w >= D) return;
  // The valid count, the block's expert and its slot ids are independent loads (mb < mbs keeps
  // them in bounds): issued together, before the branch that uses them, so that a wave waits
  // one memory latency for all three before its weight stream starts.
  const int i16 = lane & 15, g = lane >> 4;
  int slot[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) slot[tt] = sorted_ids[mb * BM + tt * 16 + i16];
  const int nv = *num_valid;
  const int e = expert_ids[mb];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) asm volatile("" ::"v"(slot[tt]));  // keeps the loads above the branch
  // blocks past the valid count, and (defensive: ids come from the routing step) bad ids
  if (mb * BM >= nv || (unsigned)e >= (unsigned)E) return;
  const int n_slots = T * k;
  const int rowb = DT == DT_BF16 ? I * 2 : DT == DT_FP8 ? I : I / 2;
  const int rows_s = I / 32;  // FP4: E8M0 scales per row
  const size_t lane_w = pre ? (size_t)lane * 16 : (size_t)i16 * rowb + 16 * g;
  const uint8_t* wrow[NG];
  const uint8_t* wsc[NG];
#pragma unroll
  for (int q = 0; q < NG; ++q) {
    wrow[q] = w2 + ((size_t)e * D + d_w + 16 * q) * rowb + lane_w;
    wsc[q] = nullptr;
    if constexpr (FP4)
      wsc[q] = static_cast<const uint8_t*>(w2_scale_v) +
               (pre ? ((size_t)e * D + d_w + 16 * q) * rows_s + i16 * 8 : ((size_t)e * D + d_w + 16 * q + i16) * rows_s);
  }
  const uint8_t* xrow[NT];
  const uint8_t* xsc[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const int s = slot[tt];
    const bool real = (unsigned)s < (unsigned)n_slots;
    xrow[tt] = real ? a + (size_t)s * rowb : nullptr;
    xsc[tt] = FP4 && real ? static_cast<const uint8_t*>(a_scale_v) + (size_t)s * rows_s : nullptr;
  }
  // the epilogue's factors (routed weight, fp8: times the slot's row scale), loaded while the
  // weights stream
  float fac[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const int s = slot[tt];
    fac[tt] = 0.f;
    if ((unsigned)s < (unsigned)n_slots) fac[tt] = FP8 ? topk_w[s] * a_scale[s] : topk_w[s];
  }
  f32x4_t acc[NG][NT];
#pragma unroll
  for (int q = 0; q < NG; ++q)
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) acc[q][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  int kb0, kb1;
  k_range(rowb, kp, KS, kb0, kb1);
  // A block whose real rows all sit in its first 16 (decode sizes with 64-row blocks, where an
  // expert holds a few slots; the sort puts an expert's slots ahead of its padding) runs that
  // row group alone, two chunks per batch of loads (short rows, no K split): mxfp4 rows of 256
  // bytes in one memory round trip per wave instead of two, and no MFMAs on the padding row
  // groups, whose accumulators stay zero and which the epilogue skips.  (Four chunks per batch
  // would take the kernel past 256 registers, to one wave per SIMD.)
  bool small = false;
  if constexpr (NT > 1 && KS == 1) small = (rowb == 256 || rowb == 512) && __ballot(xrow[1] != nullptr) == 0;
  if (small) {
    if constexpr (NT > 1 && KS == 1) {
      f32x4_t a1[NG][1];
#pragma unroll
      for (int q = 0; q < NG; ++q) a1[q][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const uint8_t* const x1[1] = {xrow[0]};
      const uint8_t* const s1[1] = {xsc[0]};
      if (pre) mainloop<DT, NG, 1, 2, true>(wrow, x1, wsc, s1, kb0, kb1, rowb, a1);
      else mainloop<DT, NG, 1, 2, false>(wrow, x1, wsc, s1, kb0, kb1, rowb, a1);
#pragma unroll
      for (int q = 0; q < NG; ++q) acc[q][0] = a1[q][0];
    }
  } else if (pre) {
    mainloop<DT, NG, NT, U, true>(wrow, xrow, wsc, xsc, kb0, kb1, rowb, acc);
  } else {
    mainloop<DT, NG, NT, U, false>(wrow, xrow, wsc, xsc, kb0, kb1, rowb, acc);
  }
  if (!reduce_k_split<KS, RG, NG, NT>(acc, rg, kp, red)) return;

  float ws[NG][4];
#pragma unroll
  for (int q = 0; q < NG; ++q)
#pragma unroll
    for (int r = 0; r < 4; ++r) ws[q][r] = 1.f;
  if constexpr (FP8) {
#pragma unroll
    for (int q = 0; q < NG; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) ws[q][r] = w2_scale[(size_t)e * D + d_w + 16 * q + 4 * g + r];
  }
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const int s = slot[tt];
    if ((unsigned)s >= (unsigned)n_slots) continue;  // padding rows issue no store and no atomic
    const float sc = fac[tt];
#pragma unroll
    for (int q = 0; q < NG; ++q) {
      const int d0 = d_w + 16 * q + 4 * g;
      float c[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) c[r] = acc[q][tt][r] * (FP8 ? sc * ws[q][r] : sc);
      if constexpr (OM == OM_REDUCE) {
        *reinterpret_cast<float4*>(static_cast<float*>(y) + (size_t)s * D + d0) = make_float4(c[0], c[1], c[2], c[3]);
      } else if constexpr (OM == OM_REDUCE_BF16) {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + (size_t)s * D + d0) =
            make_uint2(pack_bf16x2(c[0], c[1]), pack_bf16x2(c[2], c[3]));
      } else if constexpr (OM == OM_ATOMIC) {
        float* dst = static_cast<float*>(y) + (size_t)(s / k) * D + d0;
#pragma unroll
        for (int r = 0; r < 4; ++r) atomicAdd(dst + r, c[r]);
      } else {
        uint16_t* dst = static_cast<uint16_t*>(y) + (size_t)(s / k) * D + d0;
        atomic_add_bf16x2(dst, c[0], c[1]);
        atomic_add_bf16x2(dst + 2, c[2], c[3]);
      }
    }
  }
}

// ----------------------------------------------------------------------------- prefill tiles
// Many gathered rows per expert (prefill): a weight tile serves up to four 64-row blocks of
// one expert, and both operands go through LDS.
//  * loads: a 16-byte load whose 64 lanes cover 16 rows x 64 B (the MFMA operand layout)
//    streams about a third as fast from L2 as one covering 8 rows x 128 B with 8
//    consecutive lanes per row.  Both operands are therefore brought in full 128-byte rows
//    by direct-to-LDS loads and read back in MFMA layout; logical segment s of row r sits at
//    segment s ^ ((r / 2) % 8), which keeps both the loads and the reads conflict-free;
//  * stage 1 (gate-up): weight rows are the first MFMA operand, so a lane ends up with 4
//    consecutive channels of one slot (gate and up pair in the same lane);
//  * stage 2 (down): the operands are swapped, so a lane holds one model_dim channel of
//    4 slots and 16 lanes cover 16 consecutive channels of one slot: each atomic
//    instruction adds into 64 contiguous bytes per row; the slot rows of the reduce modes
//    are regrouped through LDS and stored 256 (fp32) or 128 (bf16) contiguous bytes per row.
enum { PF_G1 = 0, PF_G2_ATOMIC = 1, PF_G2_REDUCE = 2, PF_G2_ATOMIC_BF16 = 3, PF_G2_REDUCE_BF16 = 4 };
constexpr int kPfRows = 64;                          // rows of one sorted block
constexpr int kPfMaxBlocks = 4;                      // sorted blocks per tile
constexpr int kPfMaxRows = kPfRows * kPfMaxBlocks;   // 256
// LDS of one CU, less the slot ids and the per-row epilogue factors
constexpr int kPfRingBytes = 160 * 1024 - kPfMaxRows * 8;

struct PfArgs {
  const uint8_t* act;
  const void* act_scale;  // fp8: fp32 per row; mxfp4: E8M0 bytes [rows, K/32]
  const uint8_t* w;
  const void* w_scale;    // fp8: fp32 per row; mxfp4: E8M0 bytes [E, rows, K/32]
  const float* topk_w;
  int T, k, N, K, e;
  int nt0, nt1;  // the run of channel tiles [nt0, nt1) this workgroup computes
  void* out;
  int pre;  // weights in fragment order (preshuffle_kernel)
  int wnt;  // the tile covers all of its expert's blocks: no other tile reads its weight chunks
};

// One tile of NB sorted blocks (64 NB slot rows) x 256 weight rows, 8 waves, for each channel
// tile of a run [nt0, nt1).  The chunks of the run's channel tiles form one stream through the
// LDS ring: the first chunks of the next channel tile are in flight while the current one's
// epilogue runs, and the slot ids, factors and slot-row offsets are set up once per run.
// Wave w computes weight rows 64 (w % 4) .. + 63 against the slot-row groups tt with
// tt % 2 == w / 4.  Both operands are staged by direct-to-LDS loads, one 128-byte K chunk
// at a time, double buffered.  A load instruction fills 1 KB = 8 rows x 128 B; lane l takes
// row l/8 and physical segment l%8, which holds logical segment (l%8) ^ ((row/2) % 8): every
// 8 consecutive lanes read one full 128-byte line, and the 16 rows that an MFMA operand
// reads (one 16-byte segment each) land in 16 different bank groups.  The per-lane parts of
// the load addresses are fixed; each chunk only advances the wave-uniform bases.
// mxfp4: a chunk is 256 E2M1 elements (two MFMAs per fragment pair), and its E8M0 scales (8
// bytes per row) follow the rows in each buffer as [row][8]: the slot rows', then the weight
// rows'.  They come by 4-byte direct-to-LDS loads, 32 rows x 8 B per instruction, exactly two
// per wave and chunk (a wave with fewer rows left repeats its first, writing the same bytes),
// so they are waited for with the chunk's rows.
// s_fac[row]: the row's epilogue factor, read from LDS so that the epilogue issues no
// dependent global loads (gate-up: the token's fp8 scale; down: the routed weight, times the
// slot's fp8 scale; 0 for padding rows).
template <int DT, int MODE, int NB>
__device__ __forceinline__ void prefill_tile(const PfArgs& p, const int* __restrict__ s_slot,
                                             const float* __restrict__ s_fac,
                                             uint8_t* __restrict__ ring) {
  constexpr bool G1 = MODE == PF_G1;
  constexpr bool RED = MODE == PF_G2_REDUCE || MODE == PF_G2_REDUCE_BF16;  // slot rows through LDS
  constexpr bool FP8 = DT == DT_FP8, FP4 = DT == DT_FP4;
  constexpr int MH = 2 * NB;  // slot-row groups per wave
  // LDS ring: NBUF buffers of (slot rows | weight rows | mxfp4 scales) for one 128-byte chunk
  // each; short tiles fit three buffers and load two chunks ahead
  constexpr int TOKB = kPfRows * NB * 128, DATB = TOKB + 256 * 128;
  constexpr int BUF = DATB + (FP4 ? (kPfRows * NB + 256) * 8 : 0);
  constexpr int NBUF = 3 * BUF <= kPfRingBytes ? 3 : 2;
  constexpr int NDMA = NB + 4 + (FP4 ? 2 : 0);  // load instructions per wave and chunk
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int wr = wave & 3, th = wave >> 2;
  const int i16 = lane & 15, g = lane >> 4;
  const int n_slots = p.T * p.k;
  const int rowb = DT == DT_BF16 ? p.K * 2 : DT == DT_FP8 ? p.K : p.K / 2;
  const int N = p.N;
  const int pseg = lane & 7, rsub = lane >> 3;
  // ((8 j + rsub) / 2) % 8 = (4 (j % 2) + rsub / 2) % 8; every instruction of this wave has
  // j % 2 == wave % 2
  const int ls = pseg ^ ((4 * (wave & 1) + (rsub >> 1)) & 7);

  // slot rows: instruction jj = wave + 8 v covers tile rows 8 jj .. 8 jj + 7
  uint32_t toff[NB];
#pragma unroll
  for (int v = 0; v < NB; ++v) {
    const int s = s_slot[8 * (wave + 8 * v) + rsub];
    const bool ok = (unsigned)s < (unsigned)n_slots;  // padding slots read row 0 (dropped)
    toff[v] = (uint32_t)((ok ? (G1 ? s / p.k : s) : 0) * rowb);
  }
  // weight rows: instruction jw = wave + 8 u covers block rows 8 jw .. 8 jw + 7, i.e. group
  // q = (br / 16) % 4 of wave group br / 64.  Rows past N read row 0 (results not stored).
  const uint8_t* wexp = G1 ? p.w + (size_t)p.e * 2 * N * rowb : p.w + (size_t)p.e * N * rowb;
  // Fragment-order weights: instruction jw = wave + 8 u copies half jw % 2 (1 KB, already in
  // MFMA lane order) of the chunk of block row group jw / 2 (rows 16 (jw / 2) .. + 15).
  uint32_t woff[4];
  auto set_woff = [&](int nt) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int jw = wave + 8 * u;
      const int br = p.pre ? 16 * (jw >> 1) : 8 * jw + rsub;
      const int wg = br >> 6, q = (br >> 4) & 3, i = br & 15;
      int row, ch;
      if constexpr (G1) {
        ch = nt * 128 + 32 * wg + 16 * (q & 1) + i;
        row = (q >= 2 ? N : 0) + ch;
      } else {
        ch = nt * 256 + br;
        row = ch;
      }
      woff[u] = (uint32_t)((ch < N ? row : 0) * rowb);
      if (p.pre) woff[u] += (uint32_t)(1024 * (jw & 1) + 16 * lane);
    }
  };
  const int nch = (rowb + 127) >> 7;
  const uint32_t ring_lds = (uint32_t)(uintptr_t)ring;
  // mxfp4 scale loads: instruction j < 2 NB covers slot rows 32 j .. + 31, the others weight
  // rows 32 (j - 2 NB) .. + 31; lane l takes row l / 2, bytes 4 (l % 2) .. + 3 of the chunk's 8
  const int srow = p.K / 32;  // scale bytes per row
  uint32_t soff[2] = {0u, 0u}, sdst[2] = {0u, 0u};
  const uint8_t* wscale = nullptr;
  auto set_soff = [&](int nt) {
    if constexpr (FP4) {
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        int j = wave + 8 * x;
        if (j >= 2 * NB + 8) j = wave;  // repeat the wave's first load
        const int r = lane >> 1;
        if (j < 2 * NB) {
          const int s = s_slot[32 * j + r];
          const bool ok = (unsigned)s < (unsigned)n_slots;
          soff[x] = (uint32_t)((ok ? (G1 ? s / p.k : s) : 0) * srow) + 4u * (lane & 1);
          sdst[x] = (uint32_t)(DATB + 256 * j);
        } else {
          const int br = 32 * (j - 2 * NB) + r, wg = br >> 6, q = (br >> 4) & 3, i = br & 15;
          const int ch = G1 ? nt * 128 + 32 * wg + 16 * (q & 1) + i : nt * 256 + br;
          const int row = G1 && q >= 2 ? N + ch : ch;
          const int rr = ch < N ? row : 0;
          // fragment order: [16-row group][chunk][row in group][8 bytes]; chunk c is 128 bytes on
          soff[x] = (uint32_t)(p.pre ? (rr >> 4) * (srow >> 3) * 128 + (rr & 15) * 8 : rr * srow) + 4u * (lane & 1);
          sdst[x] = (uint32_t)(DATB + kPfRows * NB * 8 + 256 * (j - 2 * NB));
        }
      }
    }
  };
  if constexpr (FP4) wscale = static_cast<const uint8_t*>(p.w_scale) + (size_t)p.e * (G1 ? 2 * N : N) * srow;
  // chunk c of the next channel tile to load into buffer b.  In a half last chunk (fp8,
  // K % 128 == 64) the lanes of the missing half read the present half again; their weight
  // operand bytes are zeroed.
  auto issue = [&](int c, int b) {
    const uint32_t bo = ring_lds + (uint32_t)(b * BUF);
    const uint32_t lo = (c * 128 + 64 >= rowb && ls >= 4) ? 16u * (ls & 3) : 16u * ls;
    const uint8_t* tb = p.act + (size_t)c * 128;
    const uint8_t* wb = wexp + (size_t)c * (p.pre ? 2048 : 128);
    const uint32_t wlo = p.pre ? 0u : lo;
#pragma unroll
    for (int v = 0; v < NB; ++v) dma16_to_lds_s(tb, toff[v] + lo, bo + (wave + 8 * v) * 1024);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (p.wnt) dma16_to_lds_s_nt(wb, woff[u] + wlo, bo + TOKB + (wave + 8 * u) * 1024);
      else dma16_to_lds_s(wb, woff[u] + wlo, bo + TOKB + (wave + 8 * u) * 1024);
    }
    if constexpr (FP4) {
      const uint8_t* sa = static_cast<const uint8_t*>(p.act_scale) + (size_t)c * 8;
      const uint8_t* sw = wscale + (size_t)c * (p.pre ? 128 : 8);
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const bool tokrow = sdst[x] < (uint32_t)(DATB + kPfRows * NB * 8);
        dma4_to_lds_s(tokrow ? sa : sw, soff[x], bo + sdst[x]);
      }
    }
  };

  const int fsw = (i16 >> 1) & 7;  // read-side swizzle of row i16 of any 16-row group
  // weight fragment (q, h) of this lane, relative to the buffer's weight rows: natural rows
  // swizzled as the slot rows, or fragment order (group 4 wr + q, half h, 16 bytes per lane)
  int wofs[4][2];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      wofs[q][h] = p.pre ? ((4 * wr + q) * 2 + h) * 1024 + 16 * lane
                         : (64 * wr + 16 * q + i16) * 128 + 16 * ((4 * h + g) ^ fsw);
  // the chunk stream: chunk ic of channel tile int_ is the next to load, into buffer ib
  const int gtot = (p.nt1 - p.nt0) * nch;
  int ic = 0, int_ = p.nt0, ib = 0;
  auto issue_next = [&]() {
    issue(ic, ib);
    ib = ib + 1 == NBUF ? 0 : ib + 1;
    if (++ic == nch) {
      ic = 0;
      if (++int_ < p.nt1) {
        set_woff(int_);
        set_soff(int_);
      }
    }
  };
  set_woff(p.nt0);
  set_soff(p.nt0);
  issue_next();
  if (NBUF == 3 && gtot > 1) issue_next();
  if (NBUF == 3 && gtot > 1) asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(NDMA) : "memory");
  else asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  int cb = 0;  // buffer of the chunk being computed
  for (int nt = p.nt0; nt < p.nt1; ++nt) {
    f32x4_t acc[4][MH];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int m = 0; m < MH; ++m) acc[q][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    uint8_t* tb = ring;
    for (int c = 0; c < nch; ++c) {
      // the buffer of chunk gc + NBUF - 1 was last read in chunk gc - 1, before the last barrier
      const int gc = (nt - p.nt0) * nch + c;
      const bool more = gc + NBUF - 1 < gtot;
      if (more) issue_next();
      tb = ring + cb * BUF;
      const uint8_t* wbuf = tb + TOKB;
      // mxfp4: this lane's scale bytes (blocks g and 4 + g of the chunk) of its weight rows
      int wsc0[4] = {127, 127, 127, 127}, wsc1[4] = {127, 127, 127, 127};
      if constexpr (FP4) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint2 v = *reinterpret_cast<const uint2*>(tb + DATB + kPfRows * NB * 8 + (64 * wr + 16 * q + i16) * 8);
          wsc0[q] = (int)((v.x >> (8 * g)) & 0xFFu);
          wsc1[q] = (int)((v.y >> (8 * g)) & 0xFFu);
        }
      }
      i32x4_t wf[4][2];
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          wf[q][h] = *reinterpret_cast<const i32x4_t*>(&wbuf[wofs[q][h]]);
      if (c * 128 + 64 >= rowb) {  // half last chunk
        const i32x4_t zero = {0, 0, 0, 0};
#pragma unroll
        for (int q = 0; q < 4; ++q) wf[q][1] = zero;
      }
      // slot-row fragments: a ring of 4, read 3 groups ahead of the MFMAs that use them
      i32x4_t tf[4][2];
      int tsc0[4], tsc1[4];
      auto rd = [&](int m) {
        const int tt = 2 * m + th;
#pragma unroll
        for (int h = 0; h < 2; ++h)
          tf[m & 3][h] = *reinterpret_cast<const i32x4_t*>(&tb[(tt * 16 + i16) * 128 + 16 * ((4 * h + g) ^ fsw)]);
        if constexpr (FP4) {
          const uint2 v = *reinterpret_cast<const uint2*>(tb + DATB + (tt * 16 + i16) * 8);
          tsc0[m & 3] = (int)((v.x >> (8 * g)) & 0xFFu);
          tsc1[m & 3] = (int)((v.y >> (8 * g)) & 0xFFu);
        }
      };
#pragma unroll
      for (int m = 0; m < 3 && m < MH; ++m) rd(m);
#pragma unroll
      for (int m = 0; m < MH; ++m) {
        if (m + 3 < MH) rd(m + 3);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if constexpr (FP4) {
            if constexpr (G1) mfma_fp4(acc[q][m], wf[q], tf[m & 3], wsc0[q], wsc1[q], tsc0[m & 3], tsc1[m & 3]);
            else mfma_fp4(acc[q][m], tf[m & 3], wf[q], tsc0[m & 3], tsc1[m & 3], wsc0[q], wsc1[q]);
          } else {
            if constexpr (G1) mfma_chunk<FP8>(acc[q][m], wf[q], tf[m & 3]);
            else mfma_chunk<FP8>(acc[q][m], tf[m & 3], wf[q]);
          }
        }
      }
      cb = cb + 1 == NBUF ? 0 : cb + 1;
      // chunk gc + 1 has landed (only the loads issued in this chunk may still be in flight)
      // and every wave is done with this chunk's buffer; after a tile's last chunk the
      // epilogue first runs while the next tile's first chunks load
      if (c + 1 == nch) break;
      if (NBUF == 3 && more) asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(NDMA) : "memory");
      else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    // the reduce epilogue stages slot rows through the last chunk's buffer, once every wave
    // has read its fragments
    if (RED) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    uint8_t* const stage = tb;
    const int row0 = G1 ? nt * 128 + wr * 32 : nt * 256 + wr * 64;
    if (row0 < N) {
      if constexpr (G1) {
        // acc[q][m][r]: channel row0 + 16*(q&1) + 4g + r (q<2 gate, q>=2 up), slot column i16
        // of group tt = 2 m + th
        const int I = N;
        uint16_t* a_out = reinterpret_cast<uint16_t*>(p.out);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int n0 = row0 + 16 * h + 4 * g;
          float sg[4] = {1.f, 1.f, 1.f, 1.f}, su[4] = {1.f, 1.f, 1.f, 1.f};
          if constexpr (FP8) {
            const float* ws = static_cast<const float*>(p.w_scale) + (size_t)p.e * 2 * I;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              sg[r] = ws[n0 + r];
              su[r] = ws[I + n0 + r];
            }
          }
#pragma unroll
          for (int m = 0; m < MH; ++m) {
            const int s = s_slot[(2 * m + th) * 16 + i16];
            if ((unsigned)s >= (unsigned)n_slots) continue;
            float xs = 1.f;
            if constexpr (FP8) xs = s_fac[(2 * m + th) * 16 + i16];
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
              v[r] = silu_mul(acc[h][m][r] * (sg[r] * xs), acc[2 + h][m][r] * (su[r] * xs));
            uint2 pk;
            pk.x = pack_bf16x2(v[0], v[1]);
            pk.y = pack_bf16x2(v[2], v[3]);
            *reinterpret_cast<uint2*>(a_out + (size_t)s * I + n0) = pk;
          }
        }
      } else {
        // acc[q][m][r]: slot row (2 m + th)*16 + 4g + r, model_dim channel row0 + 16q + i16
        const int D = N;
        float ws[4] = {1.f, 1.f, 1.f, 1.f};
        if constexpr (FP8) {
#pragma unroll
          for (int q = 0; q < 4; ++q) ws[q] = static_cast<const float*>(p.w_scale)[(size_t)p.e * D + row0 + 16 * q + i16];
        }
        if constexpr (MODE == PF_G2_ATOMIC_BF16) {
          // channel pairs (2c, 2c+1) sit in lanes i16 = 2c and 2c+1: the even lane adds the pairs
          // of slot rows r = 0, 1, the odd lane those of r = 2, 3, after one exchange of two
          // values between the two lanes
          uint16_t* out = reinterpret_cast<uint16_t*>(p.out);
          const bool odd = (i16 & 1) != 0;
#pragma unroll
          for (int m = 0; m < MH; ++m) {
            int sr[4];
            float sc[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              sr[r] = s_slot[(2 * m + th) * 16 + 4 * g + r];
              sc[r] = s_fac[(2 * m + th) * 16 + 4 * g + r];
            }
            const int s_a = odd ? sr[2] : sr[0], s_b = odd ? sr[3] : sr[1];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              float cv[4];
#pragma unroll
              for (int r = 0; r < 4; ++r) cv[r] = acc[q][m][r] * (FP8 ? sc[r] * ws[q] : sc[r]);
              const float ra = __uint_as_float(xor_lane<1>(__float_as_uint(odd ? cv[0] : cv[2])));
              const float rb = __uint_as_float(xor_lane<1>(__float_as_uint(odd ? cv[1] : cv[3])));
              const int dch = row0 + 16 * q + (i16 & ~1);
              if ((unsigned)s_a < (unsigned)n_slots)  // padding rows issue nothing
                atomic_add_bf16x2(out + (size_t)(s_a / p.k) * D + dch, odd ? ra : cv[0], odd ? cv[2] : ra);
              if ((unsigned)s_b < (unsigned)n_slots)
                atomic_add_bf16x2(out + (size_t)(s_b / p.k) * D + dch, odd ? rb : cv[1], odd ? cv[3] : rb);
            }
          }
        } else if constexpr (RED) {
          // slot rows through LDS (a ring buffer no wave reads any more): each wave
          // writes its 16 rows x 64 channels of group m in fp32, then each store instruction
          // covers whole 256-byte (fp32) or 128-byte (bf16) row pieces: fp32, lane l of store v
          // takes channels 4 (l % 16) .. + 3 of row 4 v + l / 16; bf16, channels 8 (l % 8) .. + 7
          // of row 8 v + l / 8.  Rows are padded to 68 floats: the 16 lanes i16 of each of the
          // four rows g land in different banks.
          float* stg = reinterpret_cast<float*>(stage + wave * (16 * 68 * 4));
#pragma unroll
          for (int m = 0; m < MH; ++m) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float sc = s_fac[(2 * m + th) * 16 + 4 * g + r];
#pragma unroll
              for (int q = 0; q < 4; ++q) stg[(4 * g + r) * 68 + 16 * q + i16] = acc[q][m][r] * (FP8 ? sc * ws[q] : sc);
            }
            wave_lds_sync();
            if constexpr (MODE == PF_G2_REDUCE) {
              float* y = reinterpret_cast<float*>(p.out);
              const int j4 = lane & 15, rho0 = lane >> 4;
#pragma unroll
              for (int v = 0; v < 4; ++v) {
                const int rho = 4 * v + rho0;
                const int s = s_slot[(2 * m + th) * 16 + rho];
                const f32x4_t val = *reinterpret_cast<const f32x4_t*>(&stg[rho * 68 + 4 * j4]);
                if ((unsigned)s < (unsigned)n_slots)  // padding rows issue nothing
                  __builtin_nontemporal_store(val, reinterpret_cast<f32x4_t*>(y + (size_t)s * D + row0 + 4 * j4));
              }
            } else {
              uint16_t* y = reinterpret_cast<uint16_t*>(p.out);
              const int j8 = lane & 7, rho0 = lane >> 3;
#pragma unroll
              for (int v = 0; v < 2; ++v) {
                const int rho = 8 * v + rho0;
                const int s = s_slot[(2 * m + th) * 16 + rho];
                const f32x4_t lo = *reinterpret_cast<const f32x4_t*>(&stg[rho * 68 + 8 * j8]);
                const f32x4_t hi = *reinterpret_cast<const f32x4_t*>(&stg[rho * 68 + 8 * j8 + 4]);
                const i32x4_t val = {(int)pack_bf16x2(lo[0], lo[1]), (int)pack_bf16x2(lo[2], lo[3]),
                                     (int)pack_bf16x2(hi[0], hi[1]), (int)pack_bf16x2(hi[2], hi[3])};
                if ((unsigned)s < (unsigned)n_slots)  // padding rows issue nothing
                  __builtin_nontemporal_store(val, reinterpret_cast<i32x4_t*>(y + (size_t)s * D + row0 + 8 * j8));
              }
            }
            wave_lds_sync();  // the staging rows are rewritten for the next group
          }
        } else {
          float* y = reinterpret_cast<float*>(p.out);
#pragma unroll
          for (int m = 0; m < MH; ++m) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int s = s_slot[(2 * m + th) * 16 + 4 * g + r];
              if ((unsigned)s >= (unsigned)n_slots) continue;  // padding rows issue nothing
              const float sc = s_fac[(2 * m + th) * 16 + 4 * g + r];
              float* dst = y + (size_t)(s / p.k) * D + row0 + i16;
#pragma unroll
              for (int q = 0; q < 4; ++q) atomicAdd(dst + 16 * q, acc[q][m][r] * (FP8 ? sc * ws[q] : sc));
            }
          }
        }
      }
    }
    // only the reduce mode runs several channel tiles per workgroup (the host launches the
    // others with one): their kernels keep a single pass, whose chunk loop the compiler does
    // not see follow an epilogue with memory operations it counts as pending
    if (!RED || nt + 1 == p.nt1) return;
    // the next chunk has landed, the epilogue's loads and stores are done and no wave reads
    // the staging.  A builtin wait, which the compiler sees: after an opaque one it would
    // assume the epilogue's memory operations still pending and wait for every load in flight
    // before each chunk's fragment reads.
    __builtin_amdgcn_s_waitcnt(0x70);  // vmcnt(0) expcnt(7) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
  }
}

// Block = 8 waves; tile = up to kPfMaxBlocks consecutive sorted blocks of one expert, counted
// from the expert's first block (the workgroups of the tile's other blocks exit at once) x a run
// of ntr consecutive tiles of 256 weight rows (gemm1: 128 gate and the matching 128 up
// channels; gemm2: 256 model_dim rows).
template <int DT, int MODE>
__global__ void __launch_bounds__(512, 1) gemm_prefill_kernel(
    const uint8_t* __restrict__ act, const void* __restrict__ act_scale,
    const uint8_t* __restrict__ w, const void* __restrict__ w_scale,
    const float* __restrict__ topk_w, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ expert_ids, const int32_t* __restrict__ num_valid, int T, int E,
    int k, int N, int K, int mbs, int ntr, void* __restrict__ out, float4* __restrict__ zero_y,
    int64_t zero_n4, int pre) {
  constexpr bool G1 = MODE == PF_G1;
  __shared__ __align__(16) uint8_t ring[kPfRingBytes];
  __shared__ int s_slot[kPfMaxRows];
  __shared__ float s_fac[kPfMaxRows];
  if (zero_y)
    for (int64_t i = (int64_t)blockIdx.x * 512 + threadIdx.x; i < zero_n4; i += (int64_t)gridDim.x * 512)
      zero_y[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  const int tile_n = G1 ? 128 : 256;
  const int nts = (N + tile_n - 1) / tile_n;
  int mb, ntg;
  if (!block_tile_rows(mbs, (nts + ntr - 1) / ntr, mb, ntg)) return;
  const int nvb = *num_valid / kPfRows;  // sorted blocks holding slots
  if (mb >= nvb) return;
  const int e = expert_ids[mb];
  if ((unsigned)e >= (unsigned)E) return;  // defensive: ids come from the routing step
  // blocks of expert e right before mb (expert_ids is non-decreasing), 64 per step, every
  // wave on its own
  int before = 0;
  for (int base = mb - 1;; base -= 64) {
    const int idx = base - lane_id();
    const bool same = idx >= 0 && expert_ids[idx] == e;
    const uint64_t run = ~__ballot(same);
    const int n = run == 0 ? 64 : __builtin_ctzll(run);
    before += n;
    if (n < 64) break;
  }
  if (before % kPfMaxBlocks != 0) return;
  int nb = 1;
  while (nb < kPfMaxBlocks && mb + nb < nvb && expert_ids[mb + nb] == e) ++nb;
  for (int i = threadIdx.x; i < kPfRows * nb; i += 512) {
    const int s = sorted_ids[mb * kPfRows + i];
    float f = 0.f;
    if ((unsigned)s < (unsigned)(T * k)) {
      if constexpr (G1) {
        f = DT == DT_FP8 ? static_cast<const float*>(act_scale)[s / k] : 1.f;
      } else {
        f = topk_w[s];
        if constexpr (DT == DT_FP8) f *= static_cast<const float*>(act_scale)[s];
      }
    }
    s_slot[i] = s;
    s_fac[i] = f;
  }
  __syncthreads();  // s_slot, s_fac
  // a tile holding all of the expert's blocks is the only reader of its weight chunks, which
  // then go through non-temporal loads and leave the L2 to the gathered rows (Kimi fp8
  // T=4096: gate-up 614 -> 603 us, down 946 -> 874 us); where two tiles share them, the second
  // one's hits would be lost (T=16384 gate-up: 1320 -> 1454 us)
  const int solo = before == 0 && (mb + nb >= nvb || expert_ids[mb + nb] != e);
  const int nt0 = ntg * ntr, nt1 = nt0 + ntr < nts ? nt0 + ntr : nts;
  const PfArgs p{act, act_scale, w, w_scale, topk_w, T, k, N, K, e, nt0, nt1, out, pre, solo};
  switch (nb) {
    case 1: prefill_tile<DT, MODE, 1>(p, s_slot, s_fac, ring); break;
    case 2: prefill_tile<DT, MODE, 2>(p, s_slot, s_fac, ring); break;
    case 3: prefill_tile<DT, MODE, 3>(p, s_slot, s_fac, ring); break;
    default: prefill_tile<DT, MODE, 4>(p, s_slot, s_fac, ring); break;
  }
}

// The tiled kernel pays off once the experts carry several 64-row blocks on average.  Its
// direct-to-LDS loads take 32-bit byte offsets: the rows it gathers (x for the gate-up, the
// intermediate a for the down projection) and one expert's weights must each span less than
// 2 GB (larger shapes run the decode kernels, which address in 64 bits).
// mxfp4 needs K % 256 == 0 on both GEMMs (whole 8-byte scale groups per chunk).
// Channel tiles per prefill workgroup.  In the reduce mode the epilogue of each tile (its
// slot-row stores) then overlaps the loads of the next one's first chunks, which pays where K
// is short and the stores are a large share of a tile: runs of up to 8 equal lengths for at
// most 8 chunks of K (Kimi-K2.5 fp8 down projection, 4 chunks, 28 channel tiles: 1546 ->
// 1285 us at T=16384 with runs of 7; runs of 4 1465 us, of 10 1534 us, of 14 1653 us), one
// tile otherwise (GPT-OSS, 45 chunks: 538 us alone, 587 us in runs of 2); bf16 slot rows take
// the same runs.  The other modes compute one channel tile per workgroup.
static int prefill_ntr(bool reduce, int nts, int nch) {
  if (!reduce || nch > 8) return 1;
  for (int r = nts < 8 ? nts : 8; r > 1; --r)
    if (nts % r == 0) return r;
  return nts < 4 ? nts : 4;
}

static bool use_prefill(int stage, int dt, int B, int64_t T, int k, int E, int64_t D, int64_t I) {
  const int64_t kMax = (int64_t)1 << 31;
  if (dt == DT_FP4 && (D % 256 || I % 256)) return false;
  if (B != kPfRows || T * k < 32LL * E) return false;
  // the byte offsets of the gathered rows (token rows of x for the gate-up, slot rows of a
  // for the down projection) and of one expert's weight rows
  const int64_t rD = dt == DT_BF16 ? 2 * D : dt == DT_FP8 ? D : D / 2;
  const int64_t rI = dt == DT_BF16 ? 2 * I : dt == DT_FP8 ? I : I / 2;
  return stage == 1 ? T * rD < kMax && 2 * I * rD < kMax : T * k * rI < kMax && D * rI < kMax;
}

// ----------------------------------------------------------------------------- combine
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
// The combine kernels read each accumulator or slot row once and write each output once:
// both go through non-temporal accesses, so they do not displace cached data.
__global__ void __launch_bounds__(256) finalize_atomic_kernel(const float* __restrict__ y, int64_t n4,
                                                              uint16_t* __restrict__ out) {
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(y) + i);
    const u32x2_t o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    __builtin_nontemporal_store(o, reinterpret_cast<u32x2_t*>(out) + i);
  }
}

__global__ void __launch_bounds__(256) finalize_reduce_kernel(const float* __restrict__ y, int T,
                                                              int k, int D,
                                                              uint16_t* __restrict__ out) {
  const int d4 = D / 4;
  const int64_t n4 = (int64_t)T * d4;
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    const int64_t t = i / d4;
    const int c = (int)(i - t * d4);
    // slots j = 0, 1, ... added in order; the loads of 8 slots are issued before their adds
    const f32x4_t* row = reinterpret_cast<const f32x4_t*>(y + (size_t)t * k * D) + c;
    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < k; j0 += 8) {
      f32x4_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (j0 + u < k) v[u] = __builtin_nontemporal_load(row + (size_t)(j0 + u) * (D / 4));
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (j0 + u < k) {
          s[0] += v[u][0];
          s[1] += v[u][1];
          s[2] += v[u][2];
          s[3] += v[u][3];
        }
    }
    const u32x2_t o = {pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3])};
    __builtin_nontemporal_store(o, reinterpret_cast<u32x2_t*>(out) + i);
  }
}

// bf16 slot rows: 8 channels per thread (16-byte loads and stores), each value widened to
// fp32 exactly and added in slot order, as in the fp32 version.
__global__ void __launch_bounds__(256) finalize_reduce_bf16_kernel(const uint16_t* __restrict__ y,
                                                                   int T, int k, int D,
                                                                   uint16_t* __restrict__ out) {
  const int d8 = D / 8;
  const int64_t n8 = (int64_t)T * d8;
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    const int64_t t = i / d8;
    const int c = (int)(i - t * d8);
    const i32x4_t* row = reinterpret_cast<const i32x4_t*>(y + (size_t)t * k * D) + c;
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < k; j0 += 8) {
      i32x4_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (j0 + u < k) v[u] = __builtin_nontemporal_load(row + (size_t)(j0 + u) * (D / 8));
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (j0 + u < k) {
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const uint32_t w = (uint32_t)v[u][h];
            s[2 * h] += __uint_as_float(w << 16);
            s[2 * h + 1] += __uint_as_float(w & 0xFFFF0000u);
          }
        }
    }
    const i32x4_t o = {(int)pack_bf16x2(s[0], s[1]), (int)pack_bf16x2(s[2], s[3]),
                       (int)pack_bf16x2(s[4], s[5]), (int)pack_bf16x2(s[6], s[7])};
    __builtin_nontemporal_store(o, reinterpret_cast<i32x4_t*>(out) + i);
  }
}

__global__ void __launch_bounds__(256) zero_f32_kernel(float4* __restrict__ p, int64_t n4) {
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// ----------------------------------------------------------------------------- host side
// ----------------------------------------------------------------------------- weight layout
// Fragment order: for each group of 16 consecutive rows (rows R*16 .. R*16+15 of rowb bytes)
// and each 128-byte K chunk c, 2 KB = [half h][lane l = i + 16 g][16 bytes] holding bytes
// [c*128 + 64 h + 16 g, + 16) of row 16 R + i -- the 16 bytes lane l loads for its h-th
// operand register of the chunk.  One 16-byte piece per thread; the stores are contiguous.
__global__ void __launch_bounds__(256) preshuffle_kernel(const uint8_t* __restrict__ w, int64_t n16,
                                                         int rowb, uint8_t* __restrict__ out) {
  const int nch = rowb >> 7;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < n16; t += (int64_t)gridDim.x * 256) {
    const int l = (int)(t & 63), h = (int)((t >> 6) & 1);
    const int64_t cr = t >> 7;  // chunk index within the whole matrix: R * nch + c
    const int64_t R = cr / nch;
    const int c = (int)(cr - R * nch);
    const int64_t row = R * 16 + (l & 15);
    const u32x4 v = *reinterpret_cast<const u32x4*>(w + row * rowb + c * 128 + 64 * h + 16 * (l >> 4));
    *reinterpret_cast<u32x4*>(out + t * 16) = v;
  }
}

// E8M0 block scales of mxfp4 weights in fragment order: for each group of 16 consecutive rows
// (nsb = K/32 scale bytes per row) and each 256-element chunk c, 128 bytes = [row i][8 bytes]
// holding scale bytes [8 c, 8 c + 8) of row 16 R + i: the 8 bytes each lane of a decode wave
// loads for its row of the chunk, all 16 rows in one line.  One 8-byte piece per thread.
__global__ void __launch_bounds__(256) preshuffle_scales_kernel(const uint8_t* __restrict__ s, int64_t n8,
                                                                int nsb, uint8_t* __restrict__ out) {
  const int nch = nsb >> 3;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < n8; t += (int64_t)gridDim.x * 256) {
    const int i = (int)(t & 15);
    const int64_t cr = t >> 4;  // R * nch + c
    const int64_t R = cr / nch;
    const int c = (int)(cr - R * nch);
    const uint2 v = *reinterpret_cast<const uint2*>(s + (R * 16 + i) * nsb + c * 8);
    *reinterpret_cast<uint2*>(out + t * 8) = v;
  }
}

static int grid_1d(int64_t n, int cap_blocks = 4096) {
  int64_t b = (n + 255) / 256;
  if (b < 1) b = 1;
  return (int)(b < cap_blocks ? b : cap_blocks);
}

hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t st) {
  const int64_t n4 = n / 4;  // callers pass multiples of 4 (D % 64 == 0)
  if (n4 == 0) return hipSuccess;
  zero_f32_kernel<<<grid_1d(n4), 256, 0, st>>>(reinterpret_cast<float4*>(p), n4);
  return hipGetLastError();
}

hipError_t launch_preshuffle_scales(const void* s, int64_t rows, int nsb, void* out, hipStream_t st) {
  const int64_t n8 = rows * (nsb / 8);
  if (n8 == 0) return hipSuccess;
  preshuffle_scales_kernel<<<grid_1d(n8), 256, 0, st>>>(static_cast<const uint8_t*>(s), n8, nsb,
                                                        static_cast<uint8_t*>(out));
  return hipGetLastError();
}

hipError_t launch_preshuffle(const void* w, int64_t rows, int rowb, void* out, hipStream_t st) {
  const int64_t n16 = rows * (rowb / 16);
  if (n16 == 0) return hipSuccess;
  preshuffle_kernel<<<grid_1d(n16), 256, 0, st>>>(static_cast<const uint8_t*>(w), n16, rowb,
                                                 static_cast<uint8_t*>(out));
  return hipGetLastError();
}

hipError_t launch_finalize(int mode, const void* y, int T, int k, int D, uint16_t* out,
                           hipStream_t st) {
  const int64_t n4 = (int64_t)T * D / 4;
  if (n4 == 0 || mode == OM_ATOMIC_BF16) return hipSuccess;  // bf16 atomics wrote out itself
  const float* yf = static_cast<const float*>(y);
  if (mode == OM_ATOMIC)
    finalize_atomic_kernel<<<grid_1d(n4), 256, 0, st>>>(yf, n4, out);
  else if (mode == OM_REDUCE)
    finalize_reduce_kernel<<<grid_1d(n4), 256, 0, st>>>(yf, T, k, D, out);
  else
    finalize_reduce_bf16_kernel<<<grid_1d(n4 / 2), 256, 0, st>>>(static_cast<const uint16_t*>(y), T, k, D, out);
  return hipGetLastError();
}

// K-split choice: enough waves for ~12 rounds of the 256 CUs x 16 wave slots, since
// every tile of a call does the same work and the last round runs part-empty, but no wave's
// share of a row below 1 KB: shorter shares spend more of each wave on its start-up than on
// streaming (mxfp4 gate-up at the Kimi-K2.5 shape, 3.5 KB rows: 258 us split four ways, 245
// two ways, 242 unsplit; the GPT-OSS gate-up, 5.6 KB rows, is 3% faster four ways than two).
static int pick_ks(int64_t waves_ks1, int rowb, int64_t target = 256LL * 16 * 12) {
  int ks = waves_ks1 >= target ? 1 : waves_ks1 * 2 >= target ? 2 : 4;
  while (ks > 1 && rowb / ks < 1024) ks >>= 1;
  return ks;
}
static int row_bytes_of(int dt, int K) { return dt == DT_BF16 ? 2 * K : dt == DT_FP8 ? K : K / 2; }

template <int BM, int DT, int KS>
static void gemm1_go(const void* x, const void* x_scale, const void* w1, const void* w1_scale,
                     const int32_t* sorted_ids, const int32_t* expert_ids,
                     const int32_t* num_valid, int mbs, int T, int E, int k, int D, int I,
                     uint16_t* a_bf16, float* zero_y, int64_t zero_n, int pre, hipStream_t st) {
  // chunks per batch of loads: bf16 with 16-row blocks takes six (two waves per SIMD, 12 KB
  // of weights in flight per wave; 0.7% faster than four at three waves per SIMD on the
  // DeepSeek-R1 gate-up at T=4 and T=16)
  constexpr int U = BM == 64 ? 2 : DT == DT_BF16 ? 6 : 4;
  constexpr int RG = 4 / KS;
  const dim3 grid(xcd_grid(mbs, I / (16 * RG)));
  gemm1_kernel<BM, DT, U, KS><<<grid, 256, 0, st>>>(
      (const uint8_t*)x, x_scale, (const uint8_t*)w1, w1_scale, sorted_ids, expert_ids, num_valid,
      T, E, k, D, I, mbs, a_bf16, reinterpret_cast<float4*>(zero_y), zero_n / 4, pre);
}

template <int BM, int DT>
static void gemm1_ks(int ks, const void* x, const void* x_scale, const void* w1,
                     const void* w1_scale, const int32_t* sorted_ids, const int32_t* expert_ids,
                     const int32_t* num_valid, int mbs, int T, int E, int k, int D, int I,
                     uint16_t* a_bf16, float* zero_y, int64_t zero_n, int pre, hipStream_t st) {
  if (ks == 4)
    gemm1_go<BM, DT, 4>(x, x_scale, w1, w1_scale, sorted_ids, expert_ids, num_valid, mbs, T, E, k, D, I, a_bf16, zero_y, zero_n, pre, st);
  else if (ks == 2)
    gemm1_go<BM, DT, 2>(x, x_scale, w1, w1_scale, sorted_ids, expert_ids, num_valid, mbs, T, E, k, D, I, a_bf16, zero_y, zero_n, pre, st);
  else
    gemm1_go<BM, DT, 1>(x, x_scale, w1, w1_scale, sorted_ids, expert_ids, num_valid, mbs, T, E, k, D, I, a_bf16, zero_y, zero_n, pre, st);
}

// The quantised types write bf16 rows to the workspace, then requantise them into a.
static hipError_t requant(int dt, const uint16_t* a_bf16, int T, int k, int I, void* a, void* a_scale,
                          hipStream_t st) {
  const int rows = T * k;
  if (dt == DT_FP8) {
    const unsigned g = (unsigned)((rows + 3) / 4);
    uint8_t* codes = reinterpret_cast<uint8_t*>(a);
    float* sc = static_cast<float*>(a_scale);
    if (I <= 512) requant_rows_kernel<1><<<g, 256, 0, st>>>(a_bf16, rows, I, codes, sc);
    else if (I <= 1024) requant_rows_kernel<2><<<g, 256, 0, st>>>(a_bf16, rows, I, codes, sc);
    else if (I <= 2048) requant_rows_kernel<4><<<g, 256, 0, st>>>(a_bf16, rows, I, codes, sc);
    else requant_rows_kernel<0><<<g, 256, 0, st>>>(a_bf16, rows, I, codes, sc);
  } else {
    const int64_t nblocks = (int64_t)rows * (I / 32);
    requant_mx_kernel<<<(unsigned)((nblocks + 255) / 256), 256, 0, st>>>(
        a_bf16, nblocks, reinterpret_cast<uint8_t*>(a), static_cast<uint8_t*>(a_scale));
  }
  return hipGetLastError();
}

hipError_t launch_gemm1(int dt, int pre, const void* x, const void* x_scale, const void* w1,
                        const void* w1_scale, const int32_t* sorted_ids,
                        const int32_t* expert_ids, const int32_t* num_valid, int64_t cap, int T,
                        int E, int k, int D, int I, int B, void* a, void* a_scale, void* ws,
                        float* zero_y, int64_t zero_n, hipStream_t st) {
  if (T == 0) return hipSuccess;
  uint16_t* a_bf16 = dt != DT_BF16 ? reinterpret_cast<uint16_t*>(ws) : reinterpret_cast<uint16_t*>(a);
  const int mbs = (int)(cap / B);
  if (use_prefill(1, dt, B, T, k, E, D, I)) {
    const int ntr = prefill_ntr(PF_G1, (I + 127) / 128, 0);
    const dim3 grid(xcd_grid(mbs, ((I + 127) / 128 + ntr - 1) / ntr));
#define MOE_PF1(DTV)                                                                                   \
  gemm_prefill_kernel<DTV, PF_G1><<<grid, 512, 0, st>>>((const uint8_t*)x, x_scale, (const uint8_t*)w1, \
                                                       w1_scale, nullptr, sorted_ids, expert_ids,       \
                                                       num_valid, T, E, k, I, D, mbs, ntr, a_bf16,      \
                                                       reinterpret_cast<float4*>(zero_y), zero_n / 4, pre)
    if (dt == DT_FP8)
      MOE_PF1(DT_FP8);
    else if (dt == DT_FP4)
      MOE_PF1(DT_FP4);
    else
      MOE_PF1(DT_BF16);
#undef MOE_PF1
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || dt == DT_BF16) return err;
    return requant(dt, a_bf16, T, k, I, a, a_scale, st);
  }
  const int64_t n_act = (int64_t)T * k < E ? (int64_t)T * k : E;
  const int ks = pick_ks(n_act * (I / 16), row_bytes_of(dt, D));  // a block covers 16*(4/ks) channels; I % 64 == 0
#define MOE_G1_DT(BMV, DTV) \
  gemm1_ks<BMV, DTV>(ks, x, x_scale, w1, w1_scale, sorted_ids, expert_ids, num_valid, mbs, T, E, k, D, I, a_bf16, zero_y, zero_n, pre, st)
#define MOE_G1(BMV)                          \
  if (dt == DT_FP8) MOE_G1_DT(BMV, DT_FP8);   \
  else if (dt == DT_FP4) MOE_G1_DT(BMV, DT_FP4); \
  else MOE_G1_DT(BMV, DT_BF16);
  if (B == 16) {
    MOE_G1(16)
  } else if (B == 32) {
    MOE_G1(32)
  } else {
    MOE_G1(64)
  }
#undef MOE_G1
#undef MOE_G1_DT
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || dt == DT_BF16) return err;
  return requant(dt, a_bf16, T, k, I, a, a_scale, st);
}

template <int BM, int DT, int OM, int KS, int NG = 2, int UU = 0>
static void gemm2_go(int mbs, const void* a, const void* a_scale, const void* w2,
                     const void* w2_scale, const float* topk_w, const int32_t* sorted_ids,
                     const int32_t* expert_ids, const int32_t* num_valid, int T, int E, int k,
                     int D, int I, void* y, int pre, hipStream_t st) {
  constexpr int U = UU ? UU : BM == 64 ? 2 : 4;
  constexpr int RG = 4 / KS;
  const dim3 grid(xcd_grid(mbs, (D + 16 * NG * RG - 1) / (16 * NG * RG)));
  gemm2_kernel<BM, DT, U, OM, KS, NG><<<grid, 256, 0, st>>>(
      (const uint8_t*)a, a_scale, (const uint8_t*)w2, w2_scale, topk_w, sorted_ids, expert_ids,
      num_valid, T, E, k, D, I, mbs, y, pre);
}

template <int BM, int DT, int OM>
static void gemm2_ks(int ks, int mbs, const void* a, const void* a_scale, const void* w2,
                     const void* w2_scale, const float* topk_w, const int32_t* sorted_ids,
                     const int32_t* expert_ids, const int32_t* num_valid, int T, int E, int k,
                     int D, int I, void* y, int pre, hipStream_t st) {
  if (ks == 4)
    gemm2_go<BM, DT, OM, 4>(mbs, a, a_scale, w2, w2_scale, topk_w, sorted_ids, expert_ids, num_valid, T, E, k, D, I, y, pre, st);
  else if (ks == 2)
    gemm2_go<BM, DT, OM, 2>(mbs, a, a_scale, w2, w2_scale, topk_w, sorted_ids, expert_ids, num_valid, T, E, k, D, I, y, pre, st);
  else if (BM == 64 && DT != DT_FP4 && (DT == DT_BF16 ? 2 * I : I) <= 1024)
    // rows of at most 1 KB without a K split (Kimi-K2.5's fp8 share: 512 bytes) leave each
    // wave only a few chunks to stream: four 16-row groups per wave put twice the bytes in
    // flight per wave (two waves per SIMD instead of three; gemm2 at Kimi fp8 T=64: 221 -> 191
    // us).  mxfp4 with two chunks per iteration would drop to one wave per SIMD; with one
    // chunk per iteration (rows of at most 512 bytes: Kimi's mxfp4 share has 256) it keeps two
    // (gemm2 at Kimi mxfp4 T=64: 165 -> 138 us in fragment order).
    gemm2_go<BM, DT, OM, 1, 4>(mbs, a, a_scale, w2, w2_scale, topk_w, sorted_ids, expert_ids, num_valid, T, E, k, D, I, y, pre, st);
  else if (BM == 64 && DT == DT_FP4 && I / 2 <= 512)
    gemm2_go<BM, DT, OM, 1, 4, 1>(mbs, a, a_scale, w2, w2_scale, topk_w, sorted_ids, expert_ids, num_valid, T, E, k, D, I, y, pre, st);
  else
    gemm2_go<BM, DT, OM, 1>(mbs, a, a_scale, w2, w2_scale, topk_w, sorted_ids, expert_ids, num_valid, T, E, k, D, I, y, pre, st);
}

hipError_t launch_gemm2(int dt, int pre, const void* a, const void* a_scale, const void* w2,
                        const void* w2_scale, const float* topk_w, const int32_t* sorted_ids,
                        const int32_t* expert_ids, const int32_t* num_valid, int64_t cap, int T,
                        int E, int k, int D, int I, int B, int mode, void* y, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const int mbs = (int)(cap / B);
  if (use_prefill(2, dt, B, T, k, E, D, I)) {
    const int ntr = prefill_ntr(mode == OM_REDUCE || mode == OM_REDUCE_BF16, (D + 255) / 256,
                                (row_bytes_of(dt, I) + 127) / 128);
    const dim3 grid(xcd_grid(mbs, ((D + 255) / 256 + ntr - 1) / ntr));
#define MOE_PF2(DTV, MD)                                                                                \
  gemm_prefill_kernel<DTV, MD><<<grid, 512, 0, st>>>((const uint8_t*)a, a_scale, (const uint8_t*)w2,    \
                                                    w2_scale, topk_w, sorted_ids, expert_ids, num_valid, \
                                                    T, E, k, D, I, mbs, ntr, y, nullptr, 0, pre)
#define MOE_PF2_MODES(F8)                                   \
  if (mode == OM_REDUCE) MOE_PF2(F8, PF_G2_REDUCE);                   \
  else if (mode == OM_REDUCE_BF16) MOE_PF2(F8, PF_G2_REDUCE_BF16);    \
  else if (mode == OM_ATOMIC) MOE_PF2(F8, PF_G2_ATOMIC);              \
  else MOE_PF2(F8, PF_G2_ATOMIC_BF16);
    if (dt == DT_FP8) {
      MOE_PF2_MODES(DT_FP8)
    } else if (dt == DT_FP4) {
      MOE_PF2_MODES(DT_FP4)
    } else {
      MOE_PF2_MODES(DT_BF16)
    }
#undef MOE_PF2_MODES
#undef MOE_PF2
    return hipGetLastError();
  }
  const int64_t n_act = (int64_t)T * k < E ? (int64_t)T * k : E;
  // ks >= 2 needs D % 64 == 0, which always holds.  The down projection takes a higher wave
  // target than the gate-up: at DeepSeek-R1's shape and T=16 (28672 waves without a split)
  // four K parts instead of two ran 2% faster
  const int ks = pick_ks(n_act * (D / 32), row_bytes_of(dt, I), 256LL * 16 * 16);
#define MOE_G2_OM(BMV, DTV, OMV) \
  gemm2_ks<BMV, DTV, OMV>(ks, mbs, a, a_scale, w2, w2_scale, topk_w, sorted_ids, expert_ids, num_valid, T, E, k, D, I, y, pre, st)
#define MOE_G2_DT(BMV, DTV)                                  \
  if (mode == OM_REDUCE) MOE_G2_OM(BMV, DTV, OM_REDUCE);                \
  else if (mode == OM_REDUCE_BF16) MOE_G2_OM(BMV, DTV, OM_REDUCE_BF16); \
  else if (mode == OM_ATOMIC) MOE_G2_OM(BMV, DTV, OM_ATOMIC);           \
  else MOE_G2_OM(BMV, DTV, OM_ATOMIC_BF16);
#define MOE_G2(BMV)                             \
  if (dt == DT_FP8) {                           \
    MOE_G2_DT(BMV, DT_FP8)                      \
  } else if (dt == DT_FP4) {                    \
    MOE_G2_DT(BMV, DT_FP4)                      \
  } else {                                      \
    MOE_G2_DT(BMV, DT_BF16)                     \
  }
  if (B == 16) {
    MOE_G2(16)
  } else if (B == 32) {
    MOE_G2(32)
  } else {
    MOE_G2(64)
  }
#undef MOE_G2
#undef MOE_G2_DT
#undef MOE_G2_OM
  return hipGetLastError();
}

}  // namespace moe
