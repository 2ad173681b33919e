// Router: top-k gating (softmax | sigmoid) fused with the block-padded expert sort.
//
// [P1] "Fuse TopKGatingSoftmax and MoE Sorting kernels" (ROCm/FlyDSL #582): the
// top-k gating softmax and the MoE sorting step run as one launch for decode-sized
// token counts.  [P3] "Optimize fused router forward/backward kernels"
// (NVIDIA/TransformerEngine #3012), "Changes / Forward kernels": score function,
// then top-k selection, with a cheaper path for small k.
//
// Design (gfx950, wave64):
//  * one wavefront per token.  Lane l holds the logits of experts l, l+64, ...
//    as order-preserving u32 keys.
//  * selection: the k-th largest of the 64 per-lane maxima is a threshold that
//    at least k keys reach; the keys at or above it (typically a few dozen) are
//    compacted into LDS (a ballot per register gives each lane its slot) and
//    bitonic-sorted across the wave as (key, ~expert) pairs.  All cross-lane steps
//    are DPP/permlane exchanges.  If more than 128 keys reach the threshold (heavy
//    ties) or k > 64, a slower exact path extracts the maximum k times.
//  * sort: experts are ranked per token in descending order, slots s = t*k + j.
//    A token never picks an expert twice, so a slot's rank inside its expert's
//    list is the number of earlier tokens that picked the same expert.  Waves
//    own contiguous token ranges; each wave counts its picks into its own LDS
//    byte histogram, a per-expert prefix over waves gives each wave's base,
//    and each wave then places its slots walking its tokens in order.
//  * T <= 64, E <= 1024 and T*k <= 4096: everything in one 1024-thread workgroup.
//    Otherwise: select -> per-chunk counts -> per-expert prefix over chunks -> padded
//    scan over experts -> per-chunk scatter (five launches, 64-token chunks).
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kMaxCand = 128;

// Weight arithmetic runs in fp64 and is rounded to fp32 once: exp of an fp32
// logit difference loses |l - m| * 2^-24 relative accuracy in fp32, which for
// wide logit ranges exceeds the 1e-6 contract.
__device__ __forceinline__ double score_of(double l, double m, bool softmax) {
  return softmax ? exp(l - m) : 1.0 / (1.0 + exp(-l));
}

// Softmax denominator over all E logits of the token (only for softmax without
// renormalisation): sum exp(l - max).
template <int NV>
__device__ double full_softmax_denominator(const uint32_t (&keys)[NV], int E, double m) {
  const int lane = lane_id();
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < NV; ++i)
    if (lane + 64 * i < E) s += exp((double)key_logit(keys[i]) - m);
  return wave_sum_f64(s);
}

// Selects the top-k experts of one token (row of E logits) with the calling wave.
// Writes topk weights/ids for ranks 0..k-1 and calls on_pick(rank, expert) on the
// lane that owns each rank (rank = p*64 + lane), in increasing rank order per lane.
template <int NV, class OnPick>
__device__ void select_token(const float* __restrict__ row, int E, int k, int score, int renorm,
                             uint64_t* __restrict__ cand, float* __restrict__ w_out,
                             int32_t* __restrict__ id_out, OnPick on_pick) {
  const int lane = lane_id();
  uint32_t keys[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + 64 * i;
    keys[i] = e < E ? logit_key(__builtin_nontemporal_load(row + e)) : 0u;
  }
  const bool softmax = score == 0;

  // fast path: threshold from the lane maxima, compaction, one bitonic sort
  if (k <= 64) {
    uint32_t lm = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) lm = keys[i] > lm ? keys[i] : lm;
    const uint32_t tau = readlane_u32(bitonic64_desc(lm), k - 1);
    // compaction of the keys >= tau: a ballot per register gives each lane its slot
    int c = 0;  // wave-uniform
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const bool p = keys[i] >= tau;
      const uint64_t mask = __ballot(p);
      const int pos = c + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
      if (p && pos < kMaxCand) cand[pos] = pick_key(keys[i], lane + 64 * i);
      c += __popcll(mask);
    }
    if (c <= kMaxCand) {
      wave_lds_sync();
      uint64_t v0 = lane < c ? cand[lane] : 0ull;
      uint64_t v1 = lane + 64 < c ? cand[lane + 64] : 0ull;
      wave_lds_sync();
      if (c <= 64) {
        v0 = bitonic64_desc(v0);
      } else {
        bitonic128_desc(v0, v1);
      }
      // rank = lane; ranks < k <= 64 all sit in v0
      const double m = (double)key_logit(pick_logit_key(readlane_u64(v0, 0)));
      const bool mine = lane < k;
      const double sc = mine ? score_of((double)key_logit(pick_logit_key(v0)), m, softmax) : 0.0;
      double denom = 1.0;
      if (renorm) denom = wave_sum_f64(sc);
      else if (softmax) denom = full_softmax_denominator<NV>(keys, E, m);
      if (mine) {
        const int e = pick_expert(v0);
        w_out[lane] = (float)(sc / denom);
        id_out[lane] = e;
        on_pick(lane, e);
      }
      return;
    }
    wave_lds_sync();  // the candidate buffer is reused by the next token
  }

  // exact slow path: extract the maximum k times, 64 ranks per pass.  The picked
  // logit is parked in w_out and turned into the weight once the denominator is known.
  double denom_all = 1.0;
  double m = 0.0;
  double part = 0.0;
  bool have_m = false;
  for (int p = 0; p * 64 < k; ++p) {
    uint64_t mine = 0;
    const int nr = min(64, k - p * 64);
    for (int jj = 0; jj < nr; ++jj) {
      uint64_t best = 0;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const uint64_t pk = keys[i] ? pick_key(keys[i], lane + 64 * i) : 0ull;
        best = pk > best ? pk : best;
      }
      best = wave_max_u64(best);
      const int e = pick_expert(best);
      if (!have_m) {
        m = (double)key_logit(pick_logit_key(best));
        have_m = true;
        if (softmax && !renorm) denom_all = full_softmax_denominator<NV>(keys, E, m);
      }
#pragma unroll
      for (int i = 0; i < NV; ++i)
        if (lane + 64 * i == e) keys[i] = 0u;
      if (lane == jj) mine = best;
    }
    if (lane < nr) {
      const int r = p * 64 + lane;
      const float l = key_logit(pick_logit_key(mine));
      part += score_of((double)l, m, softmax);
      const int e = pick_expert(mine);
      w_out[r] = l;
      id_out[r] = e;
      on_pick(r, e);
    }
  }
  double denom = 1.0;
  if (renorm) denom = wave_sum_f64(part);
  else if (softmax) denom = denom_all;
  for (int r = lane; r < k; r += 64)  // same lane parked w_out[r]
    w_out[r] = (float)(score_of((double)w_out[r], m, softmax) / denom);
}

// ----------------------------------------------------------------------------- single workgroup
// Dynamic LDS: cand [16][128] u64 | hist [16][E4] u8 | cnt [E4] i32 | off [E4] i32 |
//              wsum [20] i32 | ids [T*k] i32
template <int NV>
__global__ void __launch_bounds__(1024) route_oneshot_kernel(
    const float* __restrict__ logits, int T, int E, int k, int score, int renorm, int B,
    float* __restrict__ topk_w, int32_t* __restrict__ topk_ids, int32_t* __restrict__ sorted_ids,
    int cap, int32_t* __restrict__ expert_ids, int32_t* __restrict__ num_valid) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint64_t* s_cand = reinterpret_cast<uint64_t*>(smem);
  uint8_t* s_hist = smem + 16 * kMaxCand * sizeof(uint64_t);
  const int E4 = (E + 3) & ~3;
  int32_t* s_cnt = reinterpret_cast<int32_t*>(s_hist + 16 * E4);
  int32_t* s_off = s_cnt + E4;
  int32_t* s_wsum = s_off + E4;
  int32_t* s_ids = s_wsum + 20;

  const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6;
  for (int i = tid; i < 16 * E4 / 4; i += 1024) reinterpret_cast<uint32_t*>(s_hist)[i] = 0u;
  __syncthreads();

  // waves own contiguous token ranges (at most 4 tokens each)
  const int tw = (T + 15) / 16;
  const int t0 = w * tw, t1 = min(T, t0 + tw);
  uint8_t* my_hist = s_hist + w * E4;
  for (int t = t0; t < t1; ++t) {
    select_token<NV>(logits + (size_t)t * E, E, k, score, renorm, s_cand + w * kMaxCand,
                     topk_w + (size_t)t * k, topk_ids + (size_t)t * k, [&](int r, int e) {
                       s_ids[t * k + r] = e;
                       if ((unsigned)e < (unsigned)E) my_hist[e] += 1;
                     });
    wave_lds_sync();
  }
  __syncthreads();

  // per-expert: exclusive prefix over waves (in place), count, padded count
  const int per = (E + 1023) / 1024;  // <= 1 expert per thread for E <= 1024
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
  // block exclusive scan of the padded counts
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

  // scatter: each wave walks its tokens in order (a token's k experts are distinct)
  const int sentinel = T * k;
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
  // padding rows, block experts, tail
  for (int e = tid; e < E; e += 1024) {
    const int c = s_cnt[e];
    if (c == 0) continue;
    const int o = s_off[e], p = (c + B - 1) / B * B;
    for (int q = c; q < p; ++q) sorted_ids[o + q] = sentinel;
    for (int b = o / B; b < (o + p) / B; ++b) expert_ids[b] = e;
  }
  for (int i = nv + tid; i < cap; i += 1024) sorted_ids[i] = sentinel;
  for (int b = nv / B + tid; b < cap / B; b += 1024) expert_ids[b] = -1;
  if (tid == 0) *num_valid = nv;
}

// ----------------------------------------------------------------------------- multi workgroup
template <int NV>
__global__ void __launch_bounds__(256) route_select_kernel(const float* __restrict__ logits,
                                                           int T, int E, int k, int score,
                                                           int renorm, float* __restrict__ topk_w,
                                                           int32_t* __restrict__ topk_ids) {
  __shared__ uint64_t s_cand[4][kMaxCand];
  const int w = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + w;
  if (t >= T) return;
  select_token<NV>(logits + (size_t)t * E, E, k, score, renorm, s_cand[w],
                   topk_w + (size_t)t * k, topk_ids + (size_t)t * k, [](int, int) {});
}

// cnt[chunk][e] = picks of expert e among the chunk's tokens
__global__ void __launch_bounds__(1024) route_count_kernel(const int32_t* __restrict__ topk_ids,
                                                           int T, int E, int k,
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
  for (int e = tid; e < E; e += 1024) cnt[(size_t)chunk * E + e] = h[e];
}

// exclusive prefix over chunks per expert (in place), and the total per expert
__global__ void __launch_bounds__(256) route_colscan_kernel(int32_t* __restrict__ cnt,
                                                            int nchunks, int E,
                                                            int32_t* __restrict__ tot) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= E) return;
  int c = 0;
  for (int ch = 0; ch < nchunks; ++ch) {
    const int v = cnt[(size_t)ch * E + e];
    cnt[(size_t)ch * E + e] = c;
    c += v;
  }
  tot[e] = c;
}

// padded exclusive scan over experts; expert_ids, padding, tail, num_valid
__global__ void __launch_bounds__(1024) route_scan_kernel(const int32_t* __restrict__ tot, int E,
                                                          int B, int sentinel, int cap,
                                                          int32_t* __restrict__ off,
                                                          int32_t* __restrict__ sorted_ids,
                                                          int32_t* __restrict__ expert_ids,
                                                          int32_t* __restrict__ num_valid) {
  __shared__ int s_wsum[17];
  __shared__ int s_nv;
  const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6;
  const int per = (E + 1023) / 1024;
  const int e0 = tid * per;
  int local = 0;
  for (int q = 0; q < per; ++q)
    if (e0 + q < E) local += (tot[e0 + q] + B - 1) / B * B;
  const int incl = wave_incl_scan_i32(local);
  if (lane == 63) s_wsum[w] = incl;
  __syncthreads();
  if (w == 0) {
    const int x = lane < 16 ? s_wsum[lane] : 0;
    const int xi = wave_incl_scan_i32(x);
    if (lane < 16) s_wsum[lane] = xi - x;
    if (lane == 15) s_nv = xi;
  }
  __syncthreads();
  int run = s_wsum[w] + incl - local;
  for (int q = 0; q < per; ++q) {
    const int e = e0 + q;
    if (e < E) {
      const int c = tot[e], p = (c + B - 1) / B * B;
      off[e] = run;
      for (int r = c; r < p; ++r) sorted_ids[run + r] = sentinel;
      for (int b = run / B; b < (run + p) / B; ++b) expert_ids[b] = e;
      run += p;
    }
  }
  const int nv = s_nv;
  for (int i = nv + tid; i < cap; i += 1024) sorted_ids[i] = sentinel;
  for (int b = nv / B + tid; b < cap / B; b += 1024) expert_ids[b] = -1;
  if (tid == 0) *num_valid = nv;
}

// per chunk: 16 waves x 4 tokens; byte histograms per wave, then ordered placement.  The
// ids of a wave's tokens are loaded once (k <= 64: one register per token and lane).
__global__ void __launch_bounds__(1024) route_scatter_kernel(const int32_t* __restrict__ topk_ids,
                                                             int T, int E, int k,
                                                             const int32_t* __restrict__ cnt,
                                                             const int32_t* __restrict__ off,
                                                             int32_t* __restrict__ sorted_ids) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int E4 = (E + 3) & ~3;
  uint8_t* s_hist = smem;
  const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6, chunk = blockIdx.x;
  for (int i = tid; i < 16 * E4 / 4; i += 1024) reinterpret_cast<uint32_t*>(s_hist)[i] = 0u;
  constexpr int TPW = kChunkTokens / 16;
  const int t0 = chunk * kChunkTokens + w * TPW, t1 = min(T, t0 + TPW);
  int ids[TPW];
#pragma unroll
  for (int q = 0; q < TPW; ++q)
    ids[q] = (t0 + q < t1 && lane < k) ? topk_ids[(size_t)(t0 + q) * k + lane] : -1;
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
  const int32_t* base = cnt + (size_t)chunk * E;
#pragma unroll
  for (int q = 0; q < TPW; ++q) {
    const int t = t0 + q;
    if (t >= t1) break;
    for (int j = lane; j < k; j += 64) {
      const int e = j < 64 ? ids[q] : topk_ids[(size_t)t * k + j];
      if ((unsigned)e >= (unsigned)E) continue;
      const int r = my_hist[e];
      my_hist[e] = (uint8_t)(r + 1);
      sorted_ids[off[e] + base[e] + r] = t * k + j;
    }
    wave_lds_sync();
  }
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

static int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

int64_t route_workspace_bytes(int T, int E, int k) {
  (void)k;
  if (T == 0 || route_is_oneshot(T, E, k)) return 0;
  const int64_t nchunks = (T + kChunkTokens - 1) / kChunkTokens;
  return align256(nchunks * E * 4) + align256((int64_t)E * 4) * 2;
}

template <int NV>
static hipError_t launch_route_nv(const float* logits, int T, int E, int k, int score, int renorm,
                                  int B, float* topk_w, int32_t* topk_ids, int32_t* sorted_ids,
                                  int64_t cap, int32_t* expert_ids, int32_t* num_valid, void* ws,
                                  hipStream_t st) {
  const int E4 = (E + 3) & ~3;
  if (route_is_oneshot(T, E, k)) {
    if constexpr (NV <= kOneShotMaxE / 64) {
      // at most 16 KB + 24 KB + 80 B + 16 KB (E <= 1024, T*k <= 4096): below the 64 KB default
      const size_t lds = 16 * kMaxCand * sizeof(uint64_t) + 16 * (size_t)E4 + 2 * 4 * (size_t)E4 + 20 * 4 +
                         4 * (size_t)T * k;
      route_oneshot_kernel<NV><<<1, 1024, lds, st>>>(logits, T, E, k, score, renorm, B, topk_w,
                                                     topk_ids, sorted_ids, (int)cap, expert_ids,
                                                     num_valid);
      return hipGetLastError();
    }
  }
  const int nchunks = (T + kChunkTokens - 1) / kChunkTokens;
  int32_t* cnt = reinterpret_cast<int32_t*>(ws);
  int32_t* tot = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) + align256((int64_t)nchunks * E * 4));
  int32_t* off = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(tot) + align256((int64_t)E * 4));
  route_select_kernel<NV><<<(T + 3) / 4, 256, 0, st>>>(logits, T, E, k, score, renorm, topk_w, topk_ids);
  route_count_kernel<<<nchunks, 1024, (size_t)E4 * 4, st>>>(topk_ids, T, E, k, cnt);
  route_colscan_kernel<<<(E + 255) / 256, 256, 0, st>>>(cnt, nchunks, E, tot);
  route_scan_kernel<<<1, 1024, 0, st>>>(tot, E, B, T * k, (int)cap, off, sorted_ids, expert_ids, num_valid);
  const size_t lds = 16 * (size_t)E4;
  if (lds > 64 * 1024) {
    // byte histograms of 16 waves for E > 4096 need more than the default 64 KB of LDS
    const hipError_t err = hipFuncSetAttribute((const void*)route_scatter_kernel,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
  }
  route_scatter_kernel<<<nchunks, 1024, lds, st>>>(topk_ids, T, E, k, cnt, off, sorted_ids);
  return hipGetLastError();
}

hipError_t launch_route(const float* logits, int T, int E, int k, int score, int renorm, int B,
                        float* topk_w, int32_t* topk_ids, int32_t* sorted_ids, int64_t cap,
                        int32_t* expert_ids, int32_t* num_valid, void* ws, hipStream_t st) {
  if (T == 0) {
    write_zero_i32<<<1, 1, 0, st>>>(num_valid);
    return hipGetLastError();
  }
  const int nv = (E + 63) / 64;
#define MOE_ROUTE_NV(N)                                                                        \
  if (nv <= N)                                                                                 \
    return launch_route_nv<N>(logits, T, E, k, score, renorm, B, topk_w, topk_ids, sorted_ids, \
                              cap, expert_ids, num_valid, ws, st);
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
