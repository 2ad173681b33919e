// Router: top-k gating (softmax | sigmoid) fused with the block-padded expert sort.
//
// [P1] "Fuse TopKGatingSoftmax and MoE Sorting kernels" (ROCm/FlyDSL #582): the
// top-k gating softmax and the MoE sorting step run as one launch for decode-sized
// token counts.  [P3] "Optimize fused router forward/backward kernels"
// (NVIDIA/TransformerEngine #3012), "Changes / Forward kernels": score function,
// then top-k selection, with a cheaper path for small k; "Hardening": group-limited
// routing (topk a multiple of group_topk).
//
// Design (gfx950, wave64):
//  * one wavefront per token; the selection (plain or group-limited) is in route_select.h.
//  * sort: experts are ranked per token in descending order, slots s = t*k + j.
//    A token never picks an expert twice, so a slot's rank inside its expert's
//    list is the number of earlier tokens that picked the same expert.  Waves
//    own contiguous token ranges; each wave counts its picks into its own LDS
//    byte histogram, a per-expert prefix over waves gives each wave's base,
//    and each wave then places its slots walking its tokens in order.
//  * T <= 16, E <= 1024 and T*k <= 4096: everything in one 1024-thread workgroup.
//  * T <= 128, E <= 2560: select (one token per wave; also the sentinel fill of the sort
//    outputs) -> one-workgroup sort (two launches).
//  * Otherwise: select -> per-chunk counts -> per-expert prefix over chunks with a
//    padded scan per 64 experts -> per-chunk scatter, which also combines the group
//    offsets and writes the block experts (four launches, 64-token chunks); where each
//    chunk's workgroup can read all E x nch counts (one byte each, at most 128 KB) the prefix
//    and the padded scan run inside the scatter kernel instead (three launches), and with at
//    most 32768 ids in all each chunk's workgroup counts them all itself (two launches).
#include "moe_device.h"
#include "moe_internal.h"
#include "route_select.h"

namespace moe {

// Sentinel fill of sorted_ids [cap) and -1 fill of expert_ids [cap/B): share `part` of
// `nparts`, written with nthreads threads (int4 stores; cap is a multiple of B >= 16).
// Real slots and block experts are written over it later.
__device__ __forceinline__ void prefill_share(int32_t* __restrict__ sorted_ids, int cap,
                                              int32_t* __restrict__ expert_ids, int B, int sentinel,
                                              int part, int nparts, int tid, int nthreads) {
  const int n4 = cap / 4, per = (n4 + nparts - 1) / nparts;
  const int a = part * per, b = min(n4, a + per);
  const int4 s4 = make_int4(sentinel, sentinel, sentinel, sentinel);
  for (int i = a + tid; i < b; i += nthreads) reinterpret_cast<int4*>(sorted_ids)[i] = s4;
  const int nb = cap / B, pe = (nb + nparts - 1) / nparts;
  const int ea = part * pe, eb = min(nb, ea + pe);
  for (int i = ea + tid; i < eb; i += nthreads) expert_ids[i] = -1;
}

// Block experts of expert e: o = its padded offset, c = its count (> 0).
__device__ __forceinline__ void write_block_experts(int e, int o, int c, int B,
                                                    int32_t* __restrict__ expert_ids) {
  const int p = (c + B - 1) / B * B;
  for (int b = o / B; b < (o + p) / B; ++b) expert_ids[b] = e;
}

// Shared by the single-workgroup sorts (16 waves), once wave w has counted its tokens'
// picks into hist[w][e] (bytes): in place, hist[w][e] becomes the exclusive prefix over
// waves; cnt[e] = the expert's count; off[e] = its padded exclusive offset.  Returns the
// padded total (num_valid); ends with a barrier.
__device__ int block_prefix_scan(uint8_t* s_hist, int32_t* s_cnt, int32_t* s_off,
                                 int32_t* s_wsum, int E, int B) {
  const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6;
  const int E4 = (E + 3) & ~3;
  const int per = (E + 1023) / 1024;
  const int e0 = tid * per;
  int local = 0;
  for (int q = 0; q < per; ++q) {
    const int e = e0 + q;
    if (e < E) {
      int c = 0;
      for (int ww = 0; ww < 16; ++ww) {
        const int h = s_hist[ww * E4 + e];
        s_hist[ww * E4 + e] = (uint8_t)c;
        c += h;
      }
      s_cnt[e] = c;
      local += (c + B - 1) / B * B;
    }
  }
  const int incl = wave_incl_scan_i32(local);
  if (lane == 63) s_wsum[w] = incl;
  __syncthreads();
  if (w == 0) {
    const int x = lane < 16 ? s_wsum[lane] : 0;
    const int xi = wave_incl_scan_i32(x);
    if (lane < 16) s_wsum[lane] = xi - x;
    if (lane == 15) s_wsum[16] = xi;
  }
  __syncthreads();
  int run = s_wsum[w] + incl - local;
  const int nv = s_wsum[16];
  for (int q = 0; q < per; ++q) {
    const int e = e0 + q;
    if (e < E) {
      s_off[e] = run;
      run += (s_cnt[e] + B - 1) / B * B;
    }
  }
  __syncthreads();
  return nv;
}

// ----------------------------------------------------------------------------- single workgroup
// Dynamic LDS: cand [16][128] u64 | hist [16][E4] u8 | cnt [E4] i32 | off [E4] i32 |
//              wsum [20] i32 | ids [T*k] i32 | (GROUPED) keys [16][E4] u32
template <int NV, bool GROUPED>
__global__ void __launch_bounds__(1024) route_oneshot_kernel(
    const float* __restrict__ logits, int T, int E, int k, int score, int renorm, GroupSel gs,
    int B, float* __restrict__ topk_w, int32_t* __restrict__ topk_ids,
    int32_t* __restrict__ sorted_ids, int cap, int32_t* __restrict__ expert_ids,
    int32_t* __restrict__ num_valid) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint64_t* s_cand = reinterpret_cast<uint64_t*>(smem);
  uint8_t* s_hist = smem + 16 * kMaxCand * sizeof(uint64_t);
  const int E4 = (E + 3) & ~3;
  int32_t* s_cnt = reinterpret_cast<int32_t*>(s_hist + 16 * E4);
  int32_t* s_off = s_cnt + E4;
  int32_t* s_wsum = s_off + E4;
  int32_t* s_ids = s_wsum + 20;

  const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6;
  if constexpr (GROUPED)  // 16-byte aligned for the spread scan's 16-byte reads
    gs.keys = reinterpret_cast<uint32_t*>((reinterpret_cast<uintptr_t>(s_ids + T * k) + 15) & ~(uintptr_t)15) +
              w * E4;
  const int sentinel = T * k;
  prefill_share(sorted_ids, cap, expert_ids, B, sentinel, 0, 1, tid, 1024);
  for (int i = tid; i < 16 * E4 / 4; i += 1024) reinterpret_cast<uint32_t*>(s_hist)[i] = 0u;
  __syncthreads();

  // waves own contiguous token ranges (at most 4 tokens each)
  const int tw = (T + 15) / 16;
  const int t0 = w * tw, t1 = min(T, t0 + tw);
  uint8_t* my_hist = s_hist + w * E4;
  for (int t = t0; t < t1; ++t) {
    select_token<NV, GROUPED, true>(logits + (size_t)t * E, E, k, score, renorm, gs,
                                    s_cand + w * kMaxCand, topk_w + (size_t)t * k,
                                    topk_ids + (size_t)t * k, [&](int r, int e) {
                                      s_ids[t * k + r] = e;
                                      if ((unsigned)e < (unsigned)E) my_hist[e] += 1;
                                    });
    wave_lds_sync();
  }
  // the barrier's workgroup-scope release/acquire orders the fill stores before the slot
  // stores written over them below (all of the workgroup's waves share one CU and its L2; a
  // device-scope fence would also write back and invalidate the L2)
  __syncthreads();

  const int nv = block_prefix_scan(s_hist, s_cnt, s_off, s_wsum, E, B);

  // scatter: each wave walks its tokens in order (a token's k experts are distinct)
  for (int t = t0; t < t1; ++t) {
    for (int j = lane; j < k; j += 64) {
      const int e = s_ids[t * k + j];
      if ((unsigned)e >= (unsigned)E) continue;
      const int r = my_hist[e];
      my_hist[e] = (uint8_t)(r + 1);
      sorted_ids[s_off[e] + r] = t * k + j;
    }
    wave_lds_sync();
  }
  for (int e = tid; e < E; e += 1024)
    if (s_cnt[e] > 0) write_block_experts(e, s_off[e], s_cnt[e], B, expert_ids);
  if (tid == 0) *num_valid = nv;
}

// ----------------------------------------------------------------------------- multi workgroup
// One token per wave; each workgroup also writes one share of the sentinel / -1 fill of
// sorted_ids and expert_ids.  Dynamic LDS (GROUPED): keys [4][E4] u32.
template <int NV, bool GROUPED>
__device__ __forceinline__ void select_block(const float* __restrict__ logits, int T, int E, int k,
                                             int score, int renorm, GroupSel gs, int B, int cap,
                                             float* __restrict__ topk_w,
                                             int32_t* __restrict__ topk_ids,
                                             int32_t* __restrict__ sorted_ids,
                                             int32_t* __restrict__ expert_ids) {
  __shared__ uint64_t s_cand[4][kMaxCand];
  extern __shared__ __align__(16) unsigned char s_dyn[];
  const int w = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + w;
  prefill_share(sorted_ids, cap, expert_ids, B, T * k, blockIdx.x, gridDim.x, threadIdx.x, 256);
  if (t >= T) return;
  if constexpr (GROUPED) gs.keys = reinterpret_cast<uint32_t*>(s_dyn) + w * ((E + 3) & ~3);
  select_token<NV, GROUPED, true>(logits + (size_t)t * E, E, k, score, renorm, gs, s_cand[w],
                                  topk_w + (size_t)t * k, topk_ids + (size_t)t * k,
                                  [](int, int) {});
}

template <int NV, bool GROUPED>
__global__ void __launch_bounds__(256) route_select_kernel(const float* __restrict__ logits,
                                                           int T, int E, int k, int score,
                                                           int renorm, GroupSel gs, int B,
                                                           int cap, float* __restrict__ topk_w,
                                                           int32_t* __restrict__ topk_ids,
                                                           int32_t* __restrict__ sorted_ids,
                                                           int32_t* __restrict__ expert_ids) {
  select_block<NV, GROUPED>(logits, T, E, k, score, renorm, gs, B, cap, topk_w, topk_ids,
                            sorted_ids, expert_ids);
}

// The plain selection for 65 <= E <= 1536 (2 <= NV <= 24) and the group-limited one for
// E <= 256 (NV <= 4) fit 64 registers: 8 waves per SIMD, one token each, so a T = 8192 call is
// resident at once (at 72 registers, 7 waves per SIMD, an eighth of its tokens waited for a
// second round).  Larger rows and NV = 1 (plain) would spill there and keep the kernel above.
template <int NV, bool GROUPED>
constexpr bool select_occ() {
  return GROUPED ? NV <= 4 : NV >= 2 && NV <= 24;
}
template <int NV, bool GROUPED>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(8)))
route_select_occ_kernel(const float* __restrict__ logits, int T, int E, int k, int score,
                        int renorm, GroupSel gs, int B, int cap, float* __restrict__ topk_w,
                        int32_t* __restrict__ topk_ids, int32_t* __restrict__ sorted_ids,
                        int32_t* __restrict__ expert_ids) {
  select_block<NV, GROUPED>(logits, T, E, k, score, renorm, gs, B, cap, topk_w, topk_ids,
                            sorted_ids, expert_ids);
}

// Single-workgroup sort after the select kernel (T <= kSort1MaxT, E <= kSort1MaxE): 16
// waves own contiguous token ranges of at most 8 tokens, whose ids are loaded once into
// registers (one per token and lane for k <= 64); byte histograms per wave, the shared
// prefix and padded scan, then ordered placement and block experts.  Padding and tail hold
// the select kernel's fill.
// Dynamic LDS: hist [16][E4] u8 | cnt [E4] i32 | off [E4] i32 | wsum [20] i32
__global__ void __launch_bounds__(1024) route_sort1_kernel(const int32_t* __restrict__ topk_ids,
                                                           int T, int E, int k, int B,
                                                           int32_t* __restrict__ sorted_ids,
                                                           int32_t* __restrict__ expert_ids,
                                                           int32_t* __restrict__ num_valid) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int E4 = (E + 3) & ~3;
  uint8_t* s_hist = smem;
  int32_t* s_cnt = reinterpret_cast<int32_t*>(s_hist + 16 * E4);
  int32_t* s_off = s_cnt + E4;
  int32_t* s_wsum = s_off + E4;
  const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6;
  for (int i = tid; i < 16 * E4 / 4; i += 1024) reinterpret_cast<uint32_t*>(s_hist)[i] = 0u;
  constexpr int TW = kSort1MaxT / 16;
  const int tw = (T + 15) / 16;
  const int t0 = w * tw, t1 = min(T, t0 + tw);
  int ids[TW];
#pragma unroll
  for (int q = 0; q < TW; ++q)
    ids[q] = (t0 + q < t1 && lane < k) ? topk_ids[(size_t)(t0 + q) * k + lane] : -1;
  __syncthreads();
  uint8_t* my_hist = s_hist + w * E4;
#pragma unroll
  for (int q = 0; q < TW; ++q) {
    const int t = t0 + q;
    if (t >= t1) break;
    for (int j = lane; j < k; j += 64) {
      const int e = j < 64 ? ids[q] : topk_ids[(size_t)t * k + j];
      if ((unsigned)e < (unsigned)E) my_hist[e] += 1;
    }
    wave_lds_sync();
  }
  __syncthreads();
  const int nv = block_prefix_scan(s_hist, s_cnt, s_off, s_wsum, E, B);
#pragma unroll
  for (int q = 0; q < TW; ++q) {
    const int t = t0 + q;
    if (t >= t1) break;
    for (int j = lane; j < k; j += 64) {
      const int e = j < 64 ? ids[q] : topk_ids[(size_t)t * k + j];
      if ((unsigned)e >= (unsigned)E) continue;
      const int r = my_hist[e];
      my_hist[e] = (uint8_t)(r + 1);
      sorted_ids[s_off[e] + r] = t * k + j;
    }
    wave_lds_sync();
  }
  for (int e = tid; e < E; e += 1024)
    if (s_cnt[e] > 0) write_block_experts(e, s_off[e], s_cnt[e], B, expert_ids);
  if (tid == 0) *num_valid = nv;
}

// Multi-workgroup sort.  cnt is expert-major: cnt[e * nch + chunk] = picks of expert e
// among the chunk's tokens.
__global__ void __launch_bounds__(1024) route_count_kernel(const int32_t* __restrict__ topk_ids,
                                                           int T, int E, int k, int nch,
                                                           int32_t* __restrict__ cnt) {
  extern __shared__ __align__(16) unsigned char smem[];
  int32_t* h = reinterpret_cast<int32_t*>(smem);
  const int tid = threadIdx.x, chunk = blockIdx.x;
  for (int e = tid; e < E; e += 1024) h[e] = 0;
  __syncthreads();
  const int t0 = chunk * kChunkTokens, t1 = min(T, t0 + kChunkTokens);
  const int s0 = t0 * k, s1 = t1 * k;
  for (int s = s0 + tid; s < s1; s += 1024) {
    const int e = topk_ids[s];
    if ((unsigned)e < (unsigned)E) atomicAdd(&h[e], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += 1024) cnt[(size_t)e * nch + chunk] = h[e];
}

// 64 experts per workgroup, 4 per wave: each expert's exclusive prefix over the chunks (in
// place; 64 chunks per coalesced load and wave scan), its total, and the padded exclusive
// scan over the workgroup's 64 experts; gsum[group] = the group's padded total.
__global__ void __launch_bounds__(1024) route_colscan_kernel(int32_t* __restrict__ cnt, int nch,
                                                             int E, int B,
                                                             int32_t* __restrict__ tot,
                                                             int32_t* __restrict__ loff,
                                                             int32_t* __restrict__ gsum) {
  __shared__ int s_c[64];
  const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6;
  const int eb = blockIdx.x * 64 + w * 4;
  int c[4] = {0, 0, 0, 0};
  for (int ch = 0; ch < nch; ch += 64) {
    const int i = ch + lane;
    int v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = (eb + q < E && i < nch) ? cnt[(size_t)(eb + q) * nch + i] : 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int incl = wave_incl_scan_i32(v[q]);
      if (eb + q < E && i < nch) cnt[(size_t)(eb + q) * nch + i] = c[q] + incl - v[q];
      c[q] += (int)readlane_u32((uint32_t)incl, 63);
    }
  }
  if (lane < 4) s_c[w * 4 + lane] = lane == 0 ? c[0] : lane == 1 ? c[1] : lane == 2 ? c[2] : c[3];
  __syncthreads();
  if (w == 0) {
    const int e = blockIdx.x * 64 + lane;
    const int cc = s_c[lane];
    const int p = (cc + B - 1) / B * B;
    const int incl = wave_incl_scan_i32(p);
    if (e < E) {
      tot[e] = cc;
      loff[e] = incl - p;
    }
    if (lane == 63) gsum[blockIdx.x] = incl;
  }
}

// Per chunk: 16 waves x 4 tokens; byte histograms per wave, then ordered placement.  The
// ids of a wave's tokens and their experts' bases are loaded once, before the histogram
// (k <= 64: one register per token and lane).  The workgroups also write the block experts
// of experts chunk, chunk + nch, ...; padding and tail hold the select kernel's fill.
__global__ void __launch_bounds__(1024) route_scatter_kernel(
    const int32_t* __restrict__ topk_ids, int T, int E, int k, int B, int nch,
    const int32_t* __restrict__ cnt, const int32_t* __restrict__ tot,
    const int32_t* __restrict__ loff, const int32_t* __restrict__ gsum,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ expert_ids,
    int32_t* __restrict__ num_valid) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int s_goff[129];  // E <= 8160: at most 128 groups of 64 experts, then the total
  const int E4 = (E + 3) & ~3;
  uint8_t* s_hist = smem;
  const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6, chunk = blockIdx.x;
  const int ngroups = (E + 63) / 64;
  for (int i = tid; i < 16 * E4 / 4; i += 1024) reinterpret_cast<uint32_t*>(s_hist)[i] = 0u;
  if (w == 0) {
    const int g0 = 2 * lane, g1 = 2 * lane + 1;
    const int x0 = g0 < ngroups ? gsum[g0] : 0, x1 = g1 < ngroups ? gsum[g1] : 0;
    const int xi = wave_incl_scan_i32(x0 + x1);
    if (g0 < ngroups) s_goff[g0] = xi - x0 - x1;
    if (g1 < ngroups) s_goff[g1] = xi - x1;
    if (lane == 63) s_goff[128] = xi;
  }
  constexpr int TPW = kChunkTokens / 16;
  const int t0 = chunk * kChunkTokens + w * TPW, t1 = min(T, t0 + TPW);
  int ids[TPW], base[TPW];
#pragma unroll
  for (int q = 0; q < TPW; ++q)
    ids[q] = (t0 + q < t1 && lane < k) ? topk_ids[(size_t)(t0 + q) * k + lane] : -1;
#pragma unroll
  for (int q = 0; q < TPW; ++q)
    base[q] = (unsigned)ids[q] < (unsigned)E ? loff[ids[q]] + cnt[(size_t)ids[q] * nch + chunk] : 0;
  __syncthreads();
  uint8_t* my_hist = s_hist + w * E4;
#pragma unroll
  for (int q = 0; q < TPW; ++q) {
    const int t = t0 + q;
    if (t >= t1) break;
    for (int j = lane; j < k; j += 64) {
      const int e = j < 64 ? ids[q] : topk_ids[(size_t)t * k + j];
      if ((unsigned)e < (unsigned)E) my_hist[e] += 1;
    }
    wave_lds_sync();
  }
  __syncthreads();
  for (int e = tid; e < E; e += 1024) {
    int c = 0;
    for (int ww = 0; ww < 16; ++ww) {
      const int h = s_hist[ww * E4 + e];
      s_hist[ww * E4 + e] = (uint8_t)c;
      c += h;
    }
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < TPW; ++q) {
    const int t = t0 + q;
    if (t >= t1) break;
    for (int j = lane; j < k; j += 64) {
      const int e = j < 64 ? ids[q] : topk_ids[(size_t)t * k + j];
      if ((unsigned)e >= (unsigned)E) continue;
      const int bj = j < 64 ? base[q] : loff[e] + cnt[(size_t)e * nch + chunk];
      const int r = my_hist[e];
      my_hist[e] = (uint8_t)(r + 1);
      sorted_ids[s_goff[e >> 6] + bj + r] = t * k + j;
    }
    wave_lds_sync();
  }
  // 64-bit stride: nch * 1024 passes INT_MAX from T = 2^27 tokens on (E <= 15 allows such T)
  for (int64_t e = chunk + (int64_t)nch * tid; e < E; e += (int64_t)nch * 1024) {
    const int c = tot[e];
    if (c > 0) write_block_experts((int)e, s_goff[e >> 6] + loff[e], c, B, expert_ids);
  }
  const int nv = s_goff[128];
  if (chunk == 0 && tid == 0) *num_valid = nv;
}

// ----------------------------------------------------------------------------- fused prefix
// Where every chunk may read all per-chunk counts (route_fused_scan), the prefix over chunks
// and the padded scan run inside the scatter kernel: three launches instead of four.  Counts
// are bytes (a chunk of 64 tokens picks an expert at most 64 times), expert-major with rows of
// nchp = nch rounded up to 16 bytes: cnt8[e * nchp + chunk]; the row tails are never written
// and never summed.
__global__ void __launch_bounds__(1024) route_count8_kernel(const int32_t* __restrict__ topk_ids,
                                                            int T, int E, int k, int nch,
                                                            uint8_t* __restrict__ cnt8) {
  extern __shared__ __align__(16) unsigned char smem[];
  int32_t* h = reinterpret_cast<int32_t*>(smem);
  const int tid = threadIdx.x, chunk = blockIdx.x;
  const int nchp = (nch + 15) & ~15;
  for (int e = tid; e < E; e += 1024) h[e] = 0;
  __syncthreads();
  const int t0 = chunk * kChunkTokens, t1 = min(T, t0 + kChunkTokens);
  for (int s = t0 * k + tid; s < t1 * k; s += 1024) {
    const int e = topk_ids[s];
    if ((unsigned)e < (unsigned)E) atomicAdd(&h[e], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += 1024) cnt8[(size_t)e * nchp + chunk] = (uint8_t)h[e];
}

// Bytes of a dword at chunk positions c0 .. c0 + 3 below `lim`: a byte mask.
__device__ __forceinline__ uint32_t bytes_below(int lim, int c0) {
  const int n = lim - c0;
  return n <= 0 ? 0u : n >= 4 ? 0xFFFFFFFFu : (1u << (8 * n)) - 1u;
}

// Per chunk, as route_scatter_kernel, but each workgroup first sums every expert's row of
// chunk counts (its total, and the part before this chunk: v_sad_u8 adds four bytes at once)
// and scans the padded totals itself.  The ids of its tokens are loaded before the counts, so
// both are in flight together.
// Dynamic LDS: hist [16][E4] u8 | tot [E4] i32 | pre [E4] i32 | off [E4] i32 | wsum [20] i32
// ids loaded per thread and batch when counting all of them (graph replay at 512/4, T = 8192:
// 8 per batch 16.4 us, 16 16.3 us, 32 16.6 us)
constexpr int kCountAllIdsPerThread = 16;
// COUNT_ALL (few ids in all, T < 65536): there are no chunk counts; each workgroup counts all
// T*k ids itself, into one LDS word per expert (its total in the low half, the part before this
// chunk in the high half), which saves the count launch.
template <bool COUNT_ALL>
__global__ void __launch_bounds__(1024) route_scan_scatter_kernel(
    const int32_t* __restrict__ topk_ids, int T, int E, int k, int B, int nch,
    const uint8_t* __restrict__ cnt8, int32_t* __restrict__ sorted_ids,
    int32_t* __restrict__ expert_ids, int32_t* __restrict__ num_valid) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int E4 = (E + 3) & ~3;
  const int nchp = (nch + 15) & ~15;
  uint8_t* s_hist = smem;
  int32_t* s_tot = reinterpret_cast<int32_t*>(smem + 16 * E4);
  int32_t* s_pre = s_tot + E4;
  int32_t* s_off = s_pre + E4;
  int32_t* s_wsum = s_off + E4;
  const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6, chunk = blockIdx.x;
  constexpr int TPW = kChunkTokens / 16;
  const int t0 = chunk * kChunkTokens + w * TPW, t1 = min(T, t0 + TPW);
  int ids[TPW];
#pragma unroll
  for (int q = 0; q < TPW; ++q)
    ids[q] = (t0 + q < t1 && lane < k) ? topk_ids[(size_t)(t0 + q) * k + lane] : -1;
  for (int i = tid; i < 16 * E4 / 4; i += 1024) reinterpret_cast<uint32_t*>(s_hist)[i] = 0u;
  if constexpr (COUNT_ALL) {
    uint32_t* h = reinterpret_cast<uint32_t*>(s_tot);
    for (int e = tid; e < E4; e += 1024) h[e] = 0u;
    __syncthreads();
    // slot s = t*k + j lies before this chunk iff s < lim
    const int n = T * k, lim = chunk * kChunkTokens * k;
    for (int s0 = tid; s0 < n; s0 += kCountAllIdsPerThread * 1024) {
      int ev[kCountAllIdsPerThread];
#pragma unroll
      for (int u = 0; u < kCountAllIdsPerThread; ++u)
        ev[u] = s0 + u * 1024 < n ? topk_ids[s0 + u * 1024] : -1;
#pragma unroll
      for (int u = 0; u < kCountAllIdsPerThread; ++u)
        if ((unsigned)ev[u] < (unsigned)E) atomicAdd(&h[ev[u]], s0 + u * 1024 < lim ? 0x10001u : 1u);
    }
    __syncthreads();
    for (int e = tid; e < E; e += 1024) {
      const uint32_t v = h[e];
      s_pre[e] = (int)(v >> 16);
      s_tot[e] = (int)(v & 0xFFFFu);
    }
  } else {
    // L lanes share an expert's row of R 16-byte pieces (L = R rounded up to a power of two,
    // at most 64): a wave load covers whole consecutive rows, four passes of loads are in
    // flight together, and a butterfly over the L lanes adds the pieces' sums.
    const int R = nchp / 16;
    int L = 1;
    while (L < R && L < 64) L <<= 1;
    const int lgL = __builtin_ctz(L);
    const int sub = lane & (L - 1);
    const int pass = 16 * (64 >> lgL);  // rows per workgroup and pass
    const uint4* cnt16 = reinterpret_cast<const uint4*>(cnt8);
    const uint4 zero4 = make_uint4(0u, 0u, 0u, 0u);
    for (int base = w * (64 >> lgL); base < E; base += 4 * pass) {  // wave-uniform
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = base + u * pass + (lane >> lgL);
        v[u] = (e < E && sub < R) ? cnt16[(size_t)e * R + sub] : zero4;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = base + u * pass + (lane >> lgL);
        uint32_t tot = 0, pre = 0;
        for (int q = sub; q < R; q += 64) {  // several pieces per lane only when R > 64
          const uint4 x = q == sub ? v[u] : e < E ? cnt16[(size_t)e * R + q] : zero4;
          const uint32_t d[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const int c0 = 16 * q + 4 * h;
            tot = __builtin_amdgcn_sad_u8(d[h] & bytes_below(nch, c0), 0u, tot);
            pre = __builtin_amdgcn_sad_u8(d[h] & bytes_below(chunk, c0), 0u, pre);
          }
        }
        if (L > 1) tot += xor_lane<1>(tot), pre += xor_lane<1>(pre);
        if (L > 2) tot += xor_lane<2>(tot), pre += xor_lane<2>(pre);
        if (L > 4) tot += xor_lane<4>(tot), pre += xor_lane<4>(pre);
        if (L > 8) tot += xor_lane<8>(tot), pre += xor_lane<8>(pre);
        if (L > 16) tot += xor_lane<16>(tot), pre += xor_lane<16>(pre);
        if (L > 32) tot += xor_lane<32>(tot), pre += xor_lane<32>(pre);
        if (sub == 0 && e < E) {
          s_tot[e] = (int)tot;
          s_pre[e] = (int)pre;
        }
      }
    }
  }
  __syncthreads();
  // padded exclusive offsets of the experts, in expert order (each thread a contiguous range)
  const int per = (E + 1023) / 1024;
  const int e0 = tid * per;
  int local = 0;
  for (int q = 0; q < per; ++q)
    if (e0 + q < E) local += (s_tot[e0 + q] + B - 1) / B * B;
  const int incl = wave_incl_scan_i32(local);
  if (lane == 63) s_wsum[w] = incl;
  __syncthreads();
  if (w == 0) {
    const int x = lane < 16 ? s_wsum[lane] : 0;
    const int xi = wave_incl_scan_i32(x);
    if (lane < 16) s_wsum[lane] = xi - x;
    if (lane == 15) s_wsum[16] = xi;
  }
  __syncthreads();
  {
    int run = s_wsum[w] + incl - local;
    for (int q = 0; q < per; ++q) {
      const int e = e0 + q;
      if (e < E) {
        s_off[e] = run;
        run += (s_tot[e] + B - 1) / B * B;
      }
    }
  }
  uint8_t* my_hist = s_hist + w * E4;
#pragma unroll
  for (int q = 0; q < TPW; ++q) {
    const int t = t0 + q;
    if (t >= t1) break;
    for (int j = lane; j < k; j += 64) {
      const int e = j < 64 ? ids[q] : topk_ids[(size_t)t * k + j];
      if ((unsigned)e < (unsigned)E) my_hist[e] += 1;
    }
    wave_lds_sync();
  }
  __syncthreads();  // s_off; the histograms
  for (int e = tid; e < E; e += 1024) {
    int c = 0;
    for (int ww = 0; ww < 16; ++ww) {
      const int h = s_hist[ww * E4 + e];
      s_hist[ww * E4 + e] = (uint8_t)c;
      c += h;
    }
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < TPW; ++q) {
    const int t = t0 + q;
    if (t >= t1) break;
    for (int j = lane; j < k; j += 64) {
      const int e = j < 64 ? ids[q] : topk_ids[(size_t)t * k + j];
      if ((unsigned)e >= (unsigned)E) continue;
      const int r = my_hist[e];
      my_hist[e] = (uint8_t)(r + 1);
      sorted_ids[s_off[e] + s_pre[e] + r] = t * k + j;
    }
    wave_lds_sync();
  }
  for (int64_t e = chunk + (int64_t)nch * tid; e < E; e += (int64_t)nch * 1024) {
    const int c = s_tot[e];
    if (c > 0) write_block_experts((int)e, s_off[e], c, B, expert_ids);
  }
  if (chunk == 0 && tid == 0) *num_valid = s_wsum[16];
}

__global__ void write_zero_i32(int32_t* p) { *p = 0; }

// ----------------------------------------------------------------------------- host side
int64_t sorted_capacity(int64_t T, int64_t E, int64_t k, int64_t B) {
  const int64_t n = T * k;
  const int64_t worst = n + (E < n ? E : n) * (B - 1);
  return (worst + B - 1) / B * B;
}

bool route_is_oneshot(int T, int E, int k) {
  return T <= kOneShotMaxT && E <= kOneShotMaxE && T * k <= kOneShotMaxSlots;
}

bool route_is_twostage(int T, int E, int k) {
  return !route_is_oneshot(T, E, k) && T <= kSort1MaxT && E <= kSort1MaxE;
}

static int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

// The fused prefix: every chunk's workgroup reads all E rows of count bytes, and its LDS holds
// 28 bytes per expert.  Up to 128 KB per workgroup it beats the separate prefix launch (graph
// replay: T = 8192, E = 512, k = 4: 23.1 -> 18.9 us; E = 1024: 27.2 -> 25.9 us; the Kimi-K2.5
// share at T = 16384, 98.5 KB: 32.6 -> 27.7 us).  Beyond, neither wins throughout: fused is
// faster for E = 2304, k = 36 at T = 4096 and 8192 (147 and 295 KB: 34.0 -> 31.5, 44.6 -> 43.0
// us) and E = 1024 at T = 16384 (256 KB: 37.6 -> 35.1 us), slower for E = 4096 at T = 4096 (256
// KB: 35.6 -> 36.6), E = 3000 at T = 8192 (384 KB: 42.7 -> 45.1), E = 2304 at T = 12000 (442
// KB: 52.1 -> 56.8) and the Kimi share at T = 33288 (203 KB: 55.6 -> 84.2 us).
static bool route_fused_scan(int E, int nch) {
  return E <= 4096 && (int64_t)E * ((nch + 15) / 16 * 16) <= 128 * 1024;
}

// Few ids in all: every chunk's workgroup counts all T*k of them (route_scan_scatter_kernel
// <true>), two launches in all; the packed counts need T < 65536.  Graph replay against the
// three-launch fused prefix: T*k = 32768 at E = 512, k = 4, T = 8192: 17.7 -> 16.4 us;
// E = 128, k = 4, T = 4096: 14.1 -> 11.8 us; E = 1024, k = 4, T = 8192: 22.3 -> 19.2 us.  Past
// that it loses: 54000 ids (E = 385, k = 9) 17.9 -> 18.0 us, 65536 (E = 512, k = 8) 18.9 -> 20.7.
constexpr int64_t kCountAllMaxIds = 32768;
static bool route_count_all(int T, int E, int k) {
  return E <= 4096 && T < 65536 && (int64_t)T * k <= kCountAllMaxIds;
}

// The larger of the two layouts: int32 counts, totals, offsets and group sums (four launches)
// or byte counts in rows of nch rounded up to 16 (fused prefix).
int64_t route_workspace_bytes(int T, int E, int k) {
  if (T == 0 || route_is_oneshot(T, E, k) || route_is_twostage(T, E, k)) return 0;
  const int64_t nchunks = (T + kChunkTokens - 1) / kChunkTokens;
  const int64_t unfused = align256(nchunks * E * 4) + align256((int64_t)E * 4) * 2 + align256(128 * 4);
  const int64_t fused = align256((int64_t)E * ((nchunks + 15) / 16 * 16));
  return fused > unfused ? fused : unfused;
}

template <int NV, bool GROUPED>
static hipError_t launch_route_nv(const float* logits, int T, int E, int k, int score, int renorm,
                                  const GroupSel& gs, int B, float* topk_w, int32_t* topk_ids,
                                  int32_t* sorted_ids, int64_t cap, int32_t* expert_ids,
                                  int32_t* num_valid, void* ws, hipStream_t st) {
  if constexpr (GROUPED && NV > kGroupMaxE / 64) {
    return hipErrorInvalidValue;
  } else {
    const int E4 = (E + 3) & ~3;
    if (route_is_oneshot(T, E, k)) {
      if constexpr (NV <= kOneShotMaxE / 64) {
        // at most 16 KB + 24 KB + 80 B + 16 KB (E <= 1024, T*k <= 4096), plus 64 KB of keys
        // for group-limited selection
        const size_t lds = 16 * kMaxCand * sizeof(uint64_t) + 16 * (size_t)E4 + 2 * 4 * (size_t)E4 +
                           20 * 4 + 4 * (size_t)T * k + (GROUPED ? 16 + 16 * 4 * (size_t)E4 : 0);
        if (lds > 64 * 1024) {
          const hipError_t err =
              hipFuncSetAttribute((const void*)route_oneshot_kernel<NV, GROUPED>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
          if (err != hipSuccess) return err;
        }
        route_oneshot_kernel<NV, GROUPED><<<1, 1024, lds, st>>>(
            logits, T, E, k, score, renorm, gs, B, topk_w, topk_ids, sorted_ids, (int)cap,
            expert_ids, num_valid);
        return hipGetLastError();
      }
    }
    // keys of 4 waves for group-limited selection (<= 64 KB for E <= 4096) beside the 4 KB
    // of static candidate buffers
    const size_t sel_lds = GROUPED ? 4 * 4 * (size_t)E4 : 0;
    if (GROUPED && sel_lds + 4 * kMaxCand * sizeof(uint64_t) > 64 * 1024) {
      const hipError_t err =
          hipFuncSetAttribute((const void*)route_select_kernel<NV, GROUPED>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)sel_lds);
      if (err != hipSuccess) return err;
    }
    auto launch_select = [&]() {
      if constexpr (select_occ<NV, GROUPED>())
        route_select_occ_kernel<NV, GROUPED><<<(T + 3) / 4, 256, sel_lds, st>>>(
            logits, T, E, k, score, renorm, gs, B, (int)cap, topk_w, topk_ids, sorted_ids,
            expert_ids);
      else
        route_select_kernel<NV, GROUPED><<<(T + 3) / 4, 256, sel_lds, st>>>(
            logits, T, E, k, score, renorm, gs, B, (int)cap, topk_w, topk_ids, sorted_ids,
            expert_ids);
    };
    if (route_is_twostage(T, E, k)) {
      launch_select();
      const size_t lds = 24 * (size_t)E4 + 20 * 4;  // <= 61.5 KB for E <= 2560
      route_sort1_kernel<<<1, 1024, lds, st>>>(topk_ids, T, E, k, B, sorted_ids, expert_ids,
                                               num_valid);
      return hipGetLastError();
    }
    const int nch = (T + kChunkTokens - 1) / kChunkTokens;
    char* wsb = reinterpret_cast<char*>(ws);
    const bool count_all = route_count_all(T, E, k);
    if (count_all || route_fused_scan(E, nch)) {
      uint8_t* cnt8 = reinterpret_cast<uint8_t*>(wsb);
      launch_select();
      if (!count_all)
        route_count8_kernel<<<nch, 1024, (size_t)E4 * 4, st>>>(topk_ids, T, E, k, nch, cnt8);
      const size_t lds = 28 * (size_t)E4 + 20 * 4;  // <= 112 KB for E <= 4096
      const void* fn = count_all ? (const void*)route_scan_scatter_kernel<true>
                                 : (const void*)route_scan_scatter_kernel<false>;
      if (lds > 64 * 1024) {
        const hipError_t err =
            hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (err != hipSuccess) return err;
      }
      if (count_all)
        route_scan_scatter_kernel<true><<<nch, 1024, lds, st>>>(topk_ids, T, E, k, B, nch, cnt8,
                                                                sorted_ids, expert_ids, num_valid);
      else
        route_scan_scatter_kernel<false><<<nch, 1024, lds, st>>>(topk_ids, T, E, k, B, nch, cnt8,
                                                                 sorted_ids, expert_ids, num_valid);
      return hipGetLastError();
    }
    int32_t* cnt = reinterpret_cast<int32_t*>(wsb);
    int32_t* tot = reinterpret_cast<int32_t*>(wsb + align256((int64_t)nch * E * 4));
    int32_t* loff =
        reinterpret_cast<int32_t*>(reinterpret_cast<char*>(tot) + align256((int64_t)E * 4));
    int32_t* gsum =
        reinterpret_cast<int32_t*>(reinterpret_cast<char*>(loff) + align256((int64_t)E * 4));
    launch_select();
    route_count_kernel<<<nch, 1024, (size_t)E4 * 4, st>>>(topk_ids, T, E, k, nch, cnt);
    route_colscan_kernel<<<(E + 63) / 64, 1024, 0, st>>>(cnt, nch, E, B, tot, loff, gsum);
    const size_t lds = 16 * (size_t)E4;
    if (lds > 64 * 1024) {
      // byte histograms of 16 waves for E > 4096 need more than the default 64 KB of LDS
      const hipError_t err = hipFuncSetAttribute((const void*)route_scatter_kernel,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 (int)lds);
      if (err != hipSuccess) return err;
    }
    route_scatter_kernel<<<nch, 1024, lds, st>>>(topk_ids, T, E, k, B, nch, cnt, tot, loff,
                                                 gsum, sorted_ids, expert_ids, num_valid);
    return hipGetLastError();
  }
}

bool route_is_grouped(int E, int n_group, int topk_group) {
  return n_group > 1 && topk_group < n_group && E % n_group == 0;
}

hipError_t launch_route(const float* logits, int T, int E, int k, int score, int renorm,
                        int n_group, int topk_group, int B, float* topk_w, int32_t* topk_ids,
                        int32_t* sorted_ids, int64_t cap, int32_t* expert_ids,
                        int32_t* num_valid, void* ws, hipStream_t st) {
  if (T == 0) {
    write_zero_i32<<<1, 1, 0, st>>>(num_valid);
    return hipGetLastError();
  }
  const bool grouped = route_is_grouped(E, n_group, topk_group);
  GroupSel gs;
  if (grouped) {
    if (n_group > kGroupMaxGroups || E > kGroupMaxE || k % topk_group != 0 ||
        k > topk_group * (E / n_group))
      return hipErrorInvalidValue;
    gs.n = n_group;
    gs.keep = topk_group;
    gs.size = E / n_group;
    gs.m = k / topk_group;
    // spread scan: n a power of two, each group an equal number of keys on each of its lanes
    const int L = 64 / n_group;
    if ((n_group & (n_group - 1)) == 0 && gs.size % L == 0 && gs.m <= 4) {
      gs.lanes = L;
      gs.per = gs.size / L;
    }
  }
  const int nv = (E + 63) / 64;
#define MOE_ROUTE_NV(N)                                                                          \
  if (nv <= N)                                                                                   \
    return grouped ? launch_route_nv<N, true>(logits, T, E, k, score, renorm, gs, B, topk_w,     \
                                              topk_ids, sorted_ids, cap, expert_ids, num_valid,  \
                                              ws, st)                                            \
                   : launch_route_nv<N, false>(logits, T, E, k, score, renorm, gs, B, topk_w,    \
                                               topk_ids, sorted_ids, cap, expert_ids, num_valid, \
                                               ws, st);
  MOE_ROUTE_NV(1)
  MOE_ROUTE_NV(2)
  MOE_ROUTE_NV(4)
  MOE_ROUTE_NV(8)
  MOE_ROUTE_NV(12)
  MOE_ROUTE_NV(16)
  MOE_ROUTE_NV(24)
  MOE_ROUTE_NV(36)
  MOE_ROUTE_NV(48)
  MOE_ROUTE_NV(64)
  MOE_ROUTE_NV(96)
  MOE_ROUTE_NV(128)
#undef MOE_ROUTE_NV
  return hipErrorInvalidValue;
}

}  // namespace moe
