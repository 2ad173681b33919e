// Scores for the load-balancing auxiliary loss, forward and backward.
//
// [P3] "[Common] Optimize fused router forward/backward kernels" (NVIDIA/TransformerEngine
// #3012), the summary, the benchmark tables ("aux_loss fprop / bprop", E/k = 512/22 and
// 2304/36, fp32, T = 8192) and the file table: a router kernel that computes the scores
// the auxiliary loss is built from, with its backward.  Per token, over all E experts:
//  * scores: softmax of the logits, or the sigmoids divided by their sum (a distribution
//    over the experts either way);
//  * routing map: 1 at the token's top-k experts (largest logits, ties to the lower
//    index), else 0;
//  * backward (the map passes no gradient), g the gradient of the scores:
//      softmax:             dl_c = p_c (g_c - sum_e p_e g_e)
//      normalised sigmoid:  dl_c = s_c (1 - s_c) / S * (g_c - sum_e q_e g_e),  S = sum_e s_e
//
// One wave per token, the row in registers (lane l holds experts l, l+64, ...): coalesced
// 256-byte loads and stores.  exp of a logit difference is taken at the exact difference
// (two-sum of the fp32 operands) with a first-order correction for its low part, and sums
// accumulate in fp64, so the scores keep a few ulp of relative accuracy for any logit range.
// The routing map is assembled as a byte row in LDS by the shared top-k selection and
// written out as dwords (bytes when E is not a multiple of 4).
#include "moe_device.h"
#include "moe_internal.h"
#include "route_select.h"

namespace moe {

// exp(a - b) for fp32 a >= b - 88 or so: d = a - b split exactly into hi + lo (Knuth's
// two-sum), exp(hi) * (1 + lo).
__device__ __forceinline__ float exp_diff(float a, float b) {
  const float hi = a - b;
  const float bb = hi - a;
  const float lo = (a - (hi - bb)) + (-b - bb);
  return expf(hi) * (1.0f + lo);
}

// 1 / (1 + exp(-l)) with the hardware reciprocal (1 ulp); an underflowing result flushes to 0
__device__ __forceinline__ float sigmoid_f(float l) {
  return __builtin_amdgcn_rcpf(1.0f + expf(-l));
}

// y = the unnormalised scores of the row (exp(l - max) or the sigmoid; 0 in empty slots)
// and inv_sum = 1 / sum y, so that y * inv_sum is the token's distribution.
template <int NV>
__device__ __forceinline__ void row_scores(float (&x)[NV], float (&y)[NV], int E, bool softmax,
                                           double& inv_sum) {
  const int lane = lane_id();
  double acc = 0.0;
  if (softmax) {
    float lm = x[0];
#pragma unroll
    for (int i = 1; i < NV; ++i) lm = fmaxf(lm, x[i]);
    const float m = wave_max_f32(lm);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      y[i] = lane + 64 * i < E ? exp_diff(x[i], m) : 0.0f;
      acc += (double)y[i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      y[i] = lane + 64 * i < E ? sigmoid_f(x[i]) : 0.0f;
      acc += (double)y[i];
    }
  }
  inv_sum = 1.0 / wave_sum_f64(acc);
}

// Dynamic LDS: map bytes [4][E4].
template <int NV>
__device__ __forceinline__ void aux_scores_block(const float* __restrict__ logits, int T, int E,
                                                 int k, int score, float* __restrict__ scores,
                                                 uint8_t* __restrict__ rmap) {
  __shared__ uint64_t s_cand[4][kMaxCand];
  extern __shared__ __align__(16) unsigned char s_map[];
  const int w = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + w;
  if (t >= T) return;
  const int lane = lane_id();
  const int E4 = (E + 3) & ~3;
  const bool softmax = score == 0;
  const float* row = logits + (size_t)t * E;
  uint8_t* mrow = s_map + w * E4;

  float x[NV], y[NV];
  load_row<NV>(row, E, x);
  double inv;
  row_scores<NV>(x, y, E, softmax, inv);
  const float rinv = (float)inv;
  float* out = scores + (size_t)t * E;
#pragma unroll
  for (int i = 0; i < NV; ++i)
    if (lane + 64 * i < E) __builtin_nontemporal_store(y[i] * rinv, out + lane + 64 * i);

  for (int e4 = lane; e4 < E4 / 4; e4 += 64) reinterpret_cast<uint32_t*>(mrow)[e4] = 0u;
  wave_lds_sync();
  GroupSel none;
  if (k <= 64) {
    select_from_row<NV, false, false>(x, row, E, k, score, 1, none, s_cand[w], nullptr, nullptr,
                                      [&](int, int e) { mrow[e] = 1; });
  } else {
    select_token_exact<NV, false, false>(row, E, k, softmax, 1, ~0ull, 1, 0.0, nullptr, nullptr,
                                         [&](int, int e) { mrow[e] = 1; });
  }
  wave_lds_sync();
  uint8_t* mo = rmap + (size_t)t * E;
  if ((E & 3) == 0) {
    for (int e4 = lane; e4 < E / 4; e4 += 64)
      __builtin_nontemporal_store(reinterpret_cast<const uint32_t*>(mrow)[e4],
                                  reinterpret_cast<uint32_t*>(mo) + e4);
  } else {
    for (int e = lane; e < E; e += 64) mo[e] = mrow[e];
  }
}

template <int NV>
__global__ void __launch_bounds__(256) aux_scores_backward_kernel(
    const float* __restrict__ logits, const float* __restrict__ grad_scores, int T, int E,
    int score, float* __restrict__ grad_logits) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = lane_id();
  float x[NV], y[NV], g[NV];
  load_row<NV>(logits + (size_t)t * E, E, x);
  const float* gr = grad_scores + (size_t)t * E;
#pragma unroll
  for (int i = 0; i < NV; ++i)
    g[i] = lane + 64 * i < E ? __builtin_nontemporal_load(gr + lane + 64 * i) : 0.0f;
  float* out = grad_logits + (size_t)t * E;
  if (score == 0) {
    double inv;
    row_scores<NV>(x, y, E, true, inv);  // y = exp(l - max)
    double dot = 0.0;
#pragma unroll
    for (int i = 0; i < NV; ++i) dot += (double)y[i] * (double)g[i];
    const float d = (float)(wave_sum_f64(dot) * inv);  // sum_e p_e g_e
    const float rinv = (float)inv;
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (lane + 64 * i < E) __builtin_nontemporal_store(y[i] * rinv * (g[i] - d), out + lane + 64 * i);
  } else {
    // u = exp(-l): s = 1 / (1 + u) and s (1 - s) = u s^2, both accurate for every l (no
    // cancellation in 1 - s); u = inf (l below about -88) has s = 0 and s (1 - s) = 0
    double ssum = 0.0, dot = 0.0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      if (lane + 64 * i < E) {
        const float u = expf(-x[i]);
        const float sv = __builtin_amdgcn_rcpf(1.0f + u);
        y[i] = u < __builtin_inff() ? u * sv * sv : 0.0f;
        ssum += (double)sv;
        dot += (double)sv * (double)g[i];
      }
    }
    const double inv = 1.0 / wave_sum_f64(ssum);
    const float d = (float)(wave_sum_f64(dot) * inv);  // sum_e q_e g_e
    const float rinv = (float)inv;
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (lane + 64 * i < E) __builtin_nontemporal_store(y[i] * rinv * (g[i] - d), out + lane + 64 * i);
  }
}

template <int NV>
__global__ void __launch_bounds__(256) aux_scores_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int score,
                                                         float* __restrict__ scores,
                                                         uint8_t* __restrict__ rmap) {
  aux_scores_block<NV>(logits, T, E, k, score, scores, rmap);
}
// As for the router's select kernel: for 65 <= E <= 1024 the forward fits 64 registers, 8
// waves per SIMD (a T = 8192 call resident at once; 37 registers at E = 512, 65 without the
// bound); elsewhere it would spill.
template <int NV>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(8)))
aux_scores_occ_kernel(const float* __restrict__ logits, int T, int E, int k, int score,
                      float* __restrict__ scores, uint8_t* __restrict__ rmap) {
  aux_scores_block<NV>(logits, T, E, k, score, scores, rmap);
}

template <int NV>
static hipError_t launch_aux_nv(const float* logits, int T, int E, int k, int score,
                                float* scores, uint8_t* rmap, hipStream_t st) {
  const size_t lds = 4 * (size_t)((E + 3) & ~3);
  if constexpr (NV >= 2 && NV <= 16)
    aux_scores_occ_kernel<NV><<<(T + 3) / 4, 256, lds, st>>>(logits, T, E, k, score, scores, rmap);
  else
    aux_scores_kernel<NV><<<(T + 3) / 4, 256, lds, st>>>(logits, T, E, k, score, scores, rmap);
  return hipGetLastError();
}

template <int NV>
static hipError_t launch_aux_bwd_nv(const float* logits, const float* grad, int T, int E,
                                    int score, float* out, hipStream_t st) {
  aux_scores_backward_kernel<NV><<<(T + 3) / 4, 256, 0, st>>>(logits, grad, T, E, score, out);
  return hipGetLastError();
}

hipError_t launch_aux_scores(const float* logits, int T, int E, int k, int score, float* scores,
                             uint8_t* routing_map, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const int nv = (E + 63) / 64;
#define MOE_AUX_NV(N) \
  if (nv <= N) return launch_aux_nv<N>(logits, T, E, k, score, scores, routing_map, st);
  MOE_AUX_NV(1)
  MOE_AUX_NV(2)
  MOE_AUX_NV(4)
  MOE_AUX_NV(8)
  MOE_AUX_NV(12)
  MOE_AUX_NV(16)
  MOE_AUX_NV(24)
  MOE_AUX_NV(36)
  MOE_AUX_NV(48)
  MOE_AUX_NV(64)
#undef MOE_AUX_NV
  return hipErrorInvalidValue;
}

hipError_t launch_aux_scores_backward(const float* logits, const float* grad_scores, int T, int E,
                                      int score, float* grad_logits, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const int nv = (E + 63) / 64;
#define MOE_AUX_NV(N) \
  if (nv <= N) return launch_aux_bwd_nv<N>(logits, grad_scores, T, E, score, grad_logits, st);
  MOE_AUX_NV(1)
  MOE_AUX_NV(2)
  MOE_AUX_NV(4)
  MOE_AUX_NV(8)
  MOE_AUX_NV(12)
  MOE_AUX_NV(16)
  MOE_AUX_NV(24)
  MOE_AUX_NV(36)
  MOE_AUX_NV(48)
  MOE_AUX_NV(64)
#undef MOE_AUX_NV
  return hipErrorInvalidValue;
}

}  // namespace moe
