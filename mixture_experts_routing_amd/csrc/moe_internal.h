// Internal launcher interface between the C ABI (abi.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Routing: largest T and E handled by the single-workgroup path.
constexpr int kOneShotMaxT = 16;
constexpr int kOneShotMaxE = 1024;
constexpr int kOneShotMaxSlots = 4096;
// Multi-workgroup routing: tokens per sort chunk (16 waves x 4 tokens).
constexpr int kChunkTokens = 64;
// Two-launch routing (select, then a one-workgroup sort): at most 8 tokens per wave; the
// byte histograms hold per-expert ranks up to T (< 256); with two int arrays per expert
// they take at most 61.5 KB of LDS.
constexpr int kSort1MaxT = 128;
constexpr int kSort1MaxE = 2560;
// per-expert ranks inside a one-workgroup sort or a 64-token chunk live in LDS bytes
static_assert(kOneShotMaxT <= 255 && kSort1MaxT <= 255 && kChunkTokens <= 255, "byte ranks");

int64_t sorted_capacity(int64_t T, int64_t E, int64_t k, int64_t B);
bool route_is_oneshot(int T, int E, int k);
bool route_is_twostage(int T, int E, int k);
int64_t route_workspace_bytes(int T, int E, int k);

// Group-limited selection runs when n_group > 1 and topk_group < n_group (n_group = 1 is the
// plain top-k); requires n_group <= 64, E <= 4096, E % n_group == 0, k % topk_group == 0.
bool route_is_grouped(int E, int n_group, int topk_group);
hipError_t launch_route(const float* logits, int T, int E, int k, int score, int renorm,
                        int n_group, int topk_group, int B, float* topk_w, int32_t* topk_ids,
                        int32_t* sorted_ids, int64_t cap, int32_t* expert_ids,
                        int32_t* num_valid, void* ws, hipStream_t st);

// Auxiliary-loss scores (E <= 4096): scores [T, E] fp32 and routing map [T, E] bytes; and
// the gradient of the scores with respect to the logits.
hipError_t launch_aux_scores(const float* logits, int T, int E, int k, int score, float* scores,
                             uint8_t* routing_map, hipStream_t st);
hipError_t launch_aux_scores_backward(const float* logits, const float* grad_scores, int T, int E,
                                      int score, float* grad_logits, hipStream_t st);

// pre: weights in fragment order (launch_preshuffle), which needs rows of whole 128-byte
// chunks and 16-row groups; mxfp4 weight scales in fragment order too
// (launch_preshuffle_scales).
hipError_t launch_gemm1(int dt, int pre, const void* x, const void* x_scale, const void* w1,
                        const void* w1_scale, const int32_t* sorted_ids,
                        const int32_t* expert_ids, const int32_t* num_valid, int64_t cap, int T,
                        int E, int k, int D, int I, int B, void* a, void* a_scale, void* ws,
                        float* zero_y, int64_t zero_n, hipStream_t st);

hipError_t launch_gemm2(int dt, int pre, const void* a, const void* a_scale, const void* w2,
                        const void* w2_scale, const float* topk_w, const int32_t* sorted_ids,
                        const int32_t* expert_ids, const int32_t* num_valid, int64_t cap, int T,
                        int E, int k, int D, int I, int B, int mode, void* y, hipStream_t st);

hipError_t launch_route_backward(const float* logits, const int32_t* topk_ids, const float* topk_w,
                                 const float* grad_w, int T, int E, int k, int score, int renorm,
                                 float* grad_logits, hipStream_t st);

hipError_t launch_finalize(int mode, const void* y, int T, int k, int D, uint16_t* out,
                           hipStream_t st);

hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t st);

// Weight rows (rows a multiple of 16, rowb a multiple of 128 bytes) into fragment order.
hipError_t launch_preshuffle(const void* w, int64_t rows, int rowb, void* out, hipStream_t st);
// mxfp4 E8M0 scale rows (rows a multiple of 16, nsb scale bytes per row, a multiple of 8) into
// fragment order.
hipError_t launch_preshuffle_scales(const void* s, int64_t rows, int nsb, void* out, hipStream_t st);

// moe_forward_noalloc: size of the static per-device workspace and its device address on the
// current device (taken once per device with hipGetSymbolAddress).
constexpr int64_t kNoAllocScratchBytes = 32LL << 20;
hipError_t noalloc_scratch(void** ptr);

}  // namespace moe
