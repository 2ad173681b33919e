// Router backward: gradient of the routed weights with respect to the logits.
//
// [P3] "[Common] Optimize fused router forward/backward kernels" (NVIDIA/TransformerEngine
// #3012), "Changes / Backward kernels": the fused router has a backward pass (a sum per
// token, then a per-element gradient).  It is the derivative of the forward's weights at
// the selection the forward made; the selection itself is piecewise constant.  With g the
// gradient of the k weights of a token and S its picks:
//  * softmax, renormalised:  dl_j = w_j (g_j - sum_i w_i g_i)                      (j in S)
//  * sigmoid, renormalised:  dl_j = s_j (1 - s_j) (g_j - sum_i w_i g_i) / sum_i s_i  (j in S)
//  * softmax over all E:     dl_e = p_e (G_e - sum_j w_j g_j), G_e = g_j at pick j, else 0
//  * sigmoid:                dl_j = s_j (1 - s_j) g_j                               (j in S)
// and 0 for every other expert.  w are the forward's weights; s_j = sigmoid(l_j).
//
// One wave per token: the picks sit one per lane (64 per pass), their sums are wave
// reductions, and the row of E gradients is written in two passes -- the value every
// expert outside S gets (0, or -p_e * dot for the full softmax), coalesced, then, after
// those stores have completed, the k entries of S.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

__global__ void __launch_bounds__(256) route_backward_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ topk_ids,
    const float* __restrict__ topk_w, const float* __restrict__ grad_w, int T, int E, int k,
    int score, int renorm, float* __restrict__ grad) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = lane_id();
  const bool softmax = score == 0;
  const float* row = logits + (size_t)t * E;
  float* out = grad + (size_t)t * E;
  const int32_t* ids = topk_ids + (size_t)t * k;
  const float* w = topk_w + (size_t)t * k;
  const float* g = grad_w + (size_t)t * k;

  // pass 1: sums over the picks (dot = sum w g; sigmoid renorm: also sum s); the first 64
  // picks' expert, weight, gradient and sigmoid stay in registers for pass 3
  float dot = 0.f, ssum = 0.f;
  int e0 = -1;
  float w0 = 0.f, g0 = 0.f, s0 = 0.f;
  for (int j0 = 0; j0 < k; j0 += 64) {
    const int j = j0 + lane;
    if (j < k) {
      const int e = ids[j];
      const float wj = w[j], gj = g[j];
      dot += wj * gj;
      float sj = 0.f;
      if (!softmax) sj = 1.f / (1.f + __expf(-row[e]));
      ssum += sj;
      if (j0 == 0) {
        e0 = e;
        w0 = wj;
        g0 = gj;
        s0 = sj;
      }
    }
  }
  dot = wave_sum_f32(dot);
  if (!softmax && renorm) ssum = wave_sum_f32(ssum);

  // pass 2: every expert's value outside the picks
  if (softmax && !renorm) {
    float m = -__builtin_inff();
    for (int e = lane; e < E; e += 64) m = fmaxf(m, row[e]);
    m = wave_max_f32(m);
    float z = 0.f;
    for (int e = lane; e < E; e += 64) z += __expf(row[e] - m);
    z = wave_sum_f32(z);
    const float c = -dot / z;
    for (int e = lane; e < E; e += 64) out[e] = __expf(row[e] - m) * c;
  } else {
    for (int e = lane; e < E; e += 64) out[e] = 0.f;
  }
  // the row's stores have completed before the picks' entries are written over them
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // pass 3: the picks
  for (int j0 = 0; j0 < k; j0 += 64) {
    const int j = j0 + lane;
    if (j >= k) continue;
    const int e = j0 == 0 ? e0 : ids[j];
    if ((unsigned)e >= (unsigned)E) continue;  // defensive: ids come from the forward
    const float wj = j0 == 0 ? w0 : w[j], gj = j0 == 0 ? g0 : g[j];
    float d;
    if (softmax) {
      d = wj * (gj - dot);  // renorm, or the full softmax with p_e = w_j
    } else {
      const float s = j0 == 0 ? s0 : 1.f / (1.f + __expf(-row[e]));
      d = renorm ? s * (1.f - s) * (gj - dot) / ssum : s * (1.f - s) * gj;
    }
    out[e] = d;
  }
}

hipError_t launch_route_backward(const float* logits, const int32_t* topk_ids, const float* topk_w,
                                 const float* grad_w, int T, int E, int k, int score, int renorm,
                                 float* grad_logits, hipStream_t st) {
  if (T == 0) return hipSuccess;
  route_backward_kernel<<<(T + 3) / 4, 256, 0, st>>>(logits, topk_ids, topk_w, grad_w, T, E, k, score,
                                                     renorm, grad_logits);
  return hipGetLastError();
}

}  // namespace moe
