// C ABI of the MoE-layer hot path: argument validation, workspace layout and
// launch order.  Every check runs before the first HIP call; nothing here
// allocates, frees or synchronises.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "../../include/moe.h"
#include "moe_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool ok_ptr(const void* p) { return p != nullptr && aligned16(p); }
int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

// [P3] "Hardening": topk in [1, E], tokens*experts within a signed 32-bit int.
int check_route_dims(int T, int E, int topk, int block_m) {
  if (T < 0 || E < 1) return MOE_EINVAL;
  if (topk < 1 || topk > E) return MOE_EINVAL;
  if (E > MOE_MAX_EXPERTS) return MOE_EUNSUPPORTED;
  if (block_m != 16 && block_m != 32 && block_m != 64) return MOE_EUNSUPPORTED;
  if ((int64_t)T * E > INT_MAX) return MOE_ERANGE;
  if (moe::sorted_capacity(T, E, topk, block_m) > INT_MAX) return MOE_ERANGE;
  return MOE_OK;
}

bool quantised(int dtype) { return dtype == MOE_FP8_E4M3 || dtype == MOE_MXFP4; }

// Bytes of a weight row of K elements.
int64_t row_bytes(int dtype, int64_t K) {
  return dtype == MOE_BF16 ? 2 * K : dtype == MOE_FP8_E4M3 ? K : K / 2;
}
// Splits the MOE_PRESHUFFLED flag off dtype.
int base_dtype(int dtype, int* pre) {
  if (pre) *pre = (dtype & MOE_PRESHUFFLED) != 0;
  return dtype & ~MOE_PRESHUFFLED;
}

int check_layer_dims(int dtype, int T, int E, int topk, int D, int I, int block_m) {
  if (dtype != MOE_BF16 && dtype != MOE_FP8_E4M3 && dtype != MOE_MXFP4) return MOE_EINVAL;
  int st = check_route_dims(T, E, topk, block_m);
  if (st) return st;
  if (D < 64 || I < 64 || D % 64 || I % 64) return MOE_EUNSUPPORTED;
  // mxfp4: whole 16x16x128 MFMAs along K (two per 128-byte chunk)
  if (dtype == MOE_MXFP4 && (D % 128 || I % 128)) return MOE_EUNSUPPORTED;
  const int64_t eb = dtype == MOE_BF16 ? 2 : 1;
  // row offsets inside the kernels are 32-bit per slot row; element counts are 64-bit
  if ((int64_t)T * topk * I > INT_MAX || (int64_t)T * topk * D > INT_MAX) return MOE_ERANGE;
  (void)eb;
  return MOE_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ELAUNCH; }

bool ok_mode(int mode) {
  return mode == MOE_OUT_ATOMIC || mode == MOE_OUT_REDUCE || mode == MOE_OUT_ATOMIC_BF16 ||
         mode == MOE_OUT_REDUCE_BF16;
}

struct Layout {
  int64_t off[MOE_WS_NFIELDS];
  int64_t total;
};

Layout forward_layout(int dtype, int mode, int T, int E, int topk, int D, int I, int block_m) {
  Layout L;
  const int64_t n = (int64_t)T * topk;
  const int64_t cap = moe::sorted_capacity(T, E, topk, block_m);
  int64_t p = 0;
  auto take = [&](int f, int64_t bytes) {
    L.off[f] = p;
    p += align256(bytes > 0 ? bytes : 1);
  };
  take(0, n * 4);
  take(1, n * 4);
  take(2, cap * 4);
  take(3, cap / block_m * 4);
  take(4, 4);
  const int64_t rws = moe::route_workspace_bytes(T, E, topk);
  if (rws > 0) take(5, rws);
  else L.off[5] = -1;
  take(6, dtype == MOE_BF16 ? n * I * 2 : dtype == MOE_FP8_E4M3 ? n * I : n * I / 2);
  if (dtype == MOE_FP8_E4M3) {
    take(7, n * 4);
    take(8, n * I * 2);
  } else if (dtype == MOE_MXFP4) {
    take(7, n * I / 32);
    take(8, n * I * 2);
  } else {
    L.off[7] = -1;
    L.off[8] = -1;
  }
  if (mode == MOE_OUT_ATOMIC_BF16) L.off[9] = -1;
  else take(9, (mode == MOE_OUT_ATOMIC ? (int64_t)T : n) * D * (mode == MOE_OUT_REDUCE_BF16 ? 2 : 4));
  L.total = p;
  return L;
}

}  // namespace

extern "C" {

const char* moe_strerror(int status) {
  switch (status) {
    case MOE_OK: return "success";
    case MOE_EINVAL: return "invalid argument (enum, pointer, alignment, topk or T)";
    case MOE_ERANGE: return "size out of range (tokens*experts or a derived size exceeds int32)";
    case MOE_ENOSPC: return "sorted capacity or workspace too small";
    case MOE_EUNSUPPORTED: return "unsupported shape (E > 8160, block_m, or D/I not multiples of 64)";
    case MOE_ELAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

int64_t moe_sorted_capacity(int T, int E, int topk, int block_m) {
  const int st = check_route_dims(T, E, topk, block_m);
  if (st) return st;
  return moe::sorted_capacity(T, E, topk, block_m);
}

int64_t moe_route_workspace_bytes(int T, int E, int topk, int block_m) {
  const int st = check_route_dims(T, E, topk, block_m);
  if (st) return st;
  return moe::route_workspace_bytes(T, E, topk);
}

int64_t moe_gemm1_workspace_bytes(int dtype, int T, int topk, int I) {
  dtype = base_dtype(dtype, nullptr);
  if (dtype != MOE_BF16 && dtype != MOE_FP8_E4M3 && dtype != MOE_MXFP4) return MOE_EINVAL;
  if (T < 0 || topk < 1 || I < 64 || I % 64) return MOE_EINVAL;
  if (dtype == MOE_BF16) return 0;
  return (int64_t)T * topk * I * 2;  // the bf16 rows before the requant
}

int64_t moe_forward_workspace_layout(int dtype, int mode, int T, int E, int topk, int D, int I,
                                     int block_m, int64_t* offsets) {
  dtype = base_dtype(dtype, nullptr);
  if (!ok_mode(mode)) return MOE_EINVAL;
  const int st = check_layer_dims(dtype, T, E, topk, D, I, block_m);
  if (st) return st;
  const Layout L = forward_layout(dtype, mode, T, E, topk, D, I, block_m);
  if (offsets)
    for (int f = 0; f < MOE_WS_NFIELDS; ++f) offsets[f] = L.off[f];
  return L.total;
}

size_t moe_forward_workspace_bytes(int dtype, int mode, int T, int E, int topk, int D, int I,
                                   int block_m) {
  const int64_t total = moe_forward_workspace_layout(dtype, mode, T, E, topk, D, I, block_m, nullptr);
  return total < 0 ? 0 : (size_t)total;
}

// [P3] "Hardening": topk a multiple of group_topk.  A selection over the kept groups needs
// at least topk experts in them.
static int check_groups(int E, int topk, int n_group, int topk_group) {
  if (n_group < 1 || E % n_group) return MOE_EINVAL;
  if (topk_group < 1 || topk_group > n_group) return MOE_EINVAL;
  if (topk % topk_group) return MOE_EINVAL;
  if ((int64_t)topk > (int64_t)topk_group * (E / n_group)) return MOE_EINVAL;
  if (moe::route_is_grouped(E, n_group, topk_group) && (n_group > 64 || E > 4096))
    return MOE_EUNSUPPORTED;
  return MOE_OK;
}

static int route_impl(const float* logits, int T, int E, int topk, int n_group, int topk_group,
                      int score, int renorm, int block_m, float* topk_weights, int32_t* topk_ids,
                      int32_t* sorted_token_ids, int64_t sorted_cap, int32_t* expert_ids,
                      int32_t* num_valid, void* workspace, size_t ws_bytes, void* stream) {
  int st = check_route_dims(T, E, topk, block_m);
  if (st) return st;
  st = check_groups(E, topk, n_group, topk_group);
  if (st) return st;
  if (score != MOE_SCORE_SOFTMAX && score != MOE_SCORE_SIGMOID) return MOE_EINVAL;
  if (renorm != 0 && renorm != 1) return MOE_EINVAL;
  if (!ok_ptr(num_valid)) return MOE_EINVAL;
  if (T > 0) {
    if (!ok_ptr(logits) || !ok_ptr(topk_weights) || !ok_ptr(topk_ids) || !ok_ptr(sorted_token_ids) ||
        !ok_ptr(expert_ids))
      return MOE_EINVAL;
  }
  if (sorted_cap < moe::sorted_capacity(T, E, topk, block_m)) return MOE_ENOSPC;
  const int64_t need = moe::route_workspace_bytes(T, E, topk);
  if ((int64_t)ws_bytes < need) return MOE_ENOSPC;
  if (need > 0 && !ok_ptr(workspace)) return MOE_EINVAL;
  const int64_t cap = moe::sorted_capacity(T, E, topk, block_m);
  return launch_status(moe::launch_route(logits, T, E, topk, score, renorm, n_group, topk_group,
                                         block_m, topk_weights, topk_ids, sorted_token_ids, cap,
                                         expert_ids, num_valid, workspace, (hipStream_t)stream));
}

int moe_topk_softmax_sort(const float* logits, int T, int E, int topk, int score, int renorm,
                          int block_m, float* topk_weights, int32_t* topk_ids,
                          int32_t* sorted_token_ids, int64_t sorted_cap, int32_t* expert_ids,
                          int32_t* num_valid, void* workspace, size_t ws_bytes, void* stream) {
  return route_impl(logits, T, E, topk, 1, 1, score, renorm, block_m, topk_weights, topk_ids,
                    sorted_token_ids, sorted_cap, expert_ids, num_valid, workspace, ws_bytes,
                    stream);
}

int moe_topk_softmax_sort_grouped(const float* logits, int T, int E, int topk, int n_group,
                                  int topk_group, int score, int renorm, int block_m,
                                  float* topk_weights, int32_t* topk_ids,
                                  int32_t* sorted_token_ids, int64_t sorted_cap,
                                  int32_t* expert_ids, int32_t* num_valid, void* workspace,
                                  size_t ws_bytes, void* stream) {
  return route_impl(logits, T, E, topk, n_group, topk_group, score, renorm, block_m,
                    topk_weights, topk_ids, sorted_token_ids, sorted_cap, expert_ids, num_valid,
                    workspace, ws_bytes, stream);
}

static int check_aux_dims(int T, int E, int topk) {
  if (T < 0 || E < 1) return MOE_EINVAL;
  if (topk < 1 || topk > E) return MOE_EINVAL;
  if (E > 4096) return MOE_EUNSUPPORTED;
  if ((int64_t)T * E > INT_MAX) return MOE_ERANGE;
  return MOE_OK;
}

int moe_aux_loss_scores(const float* logits, int T, int E, int topk, int score, float* scores,
                        uint8_t* routing_map, void* stream) {
  const int st = check_aux_dims(T, E, topk);
  if (st) return st;
  if (score != MOE_SCORE_SOFTMAX && score != MOE_SCORE_SIGMOID) return MOE_EINVAL;
  if (T > 0 && (!ok_ptr(logits) || !ok_ptr(scores) || !ok_ptr(routing_map))) return MOE_EINVAL;
  return launch_status(
      moe::launch_aux_scores(logits, T, E, topk, score, scores, routing_map, (hipStream_t)stream));
}

int moe_aux_loss_scores_backward(const float* logits, const float* grad_scores, int T, int E,
                                 int score, float* grad_logits, void* stream) {
  const int st = check_aux_dims(T, E, 1);
  if (st) return st;
  if (score != MOE_SCORE_SOFTMAX && score != MOE_SCORE_SIGMOID) return MOE_EINVAL;
  if (T > 0 && (!ok_ptr(logits) || !ok_ptr(grad_scores) || !ok_ptr(grad_logits)))
    return MOE_EINVAL;
  return launch_status(moe::launch_aux_scores_backward(logits, grad_scores, T, E, score,
                                                       grad_logits, (hipStream_t)stream));
}

static int check_gemm_common(int dtype, int T, int E, int topk, int D, int I, int block_m,
                             int64_t sorted_cap, const int32_t* sorted_token_ids,
                             const int32_t* expert_ids, const int32_t* num_valid) {
  const int st = check_layer_dims(dtype, T, E, topk, D, I, block_m);
  if (st) return st;
  if (sorted_cap < moe::sorted_capacity(T, E, topk, block_m)) return MOE_ENOSPC;
  if (T > 0 && (!ok_ptr(sorted_token_ids) || !ok_ptr(expert_ids) || !ok_ptr(num_valid)))
    return MOE_EINVAL;
  return MOE_OK;
}

int moe_topk_softmax_backward(const float* logits, const int32_t* topk_ids,
                              const float* topk_weights, const float* grad_topk_weights, int T,
                              int E, int topk, int score, int renorm, float* grad_logits,
                              void* stream) {
  if (T < 0 || E < 1 || topk < 1 || topk > E) return MOE_EINVAL;
  if (E > MOE_MAX_EXPERTS) return MOE_EUNSUPPORTED;
  if ((int64_t)T * E > INT_MAX) return MOE_ERANGE;
  if (score != MOE_SCORE_SOFTMAX && score != MOE_SCORE_SIGMOID) return MOE_EINVAL;
  if (renorm != 0 && renorm != 1) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!ok_ptr(logits) || !ok_ptr(topk_ids) || !ok_ptr(topk_weights) || !ok_ptr(grad_topk_weights) ||
      !ok_ptr(grad_logits))
    return MOE_EINVAL;
  return launch_status(moe::launch_route_backward(logits, topk_ids, topk_weights, grad_topk_weights, T, E,
                                                  topk, score, renorm, grad_logits, (hipStream_t)stream));
}

int moe_gemm1_gateup(int dtype, const void* x, const void* x_scale, const void* w1,
                     const void* w1_scale, const int32_t* sorted_token_ids,
                     const int32_t* expert_ids, const int32_t* num_valid, int64_t sorted_cap,
                     int T, int E, int topk, int D, int I, int block_m, void* a, void* a_scale,
                     void* workspace, size_t ws_bytes, void* stream) {
  int pre;
  dtype = base_dtype(dtype, &pre);
  int st = check_gemm_common(dtype, T, E, topk, D, I, block_m, sorted_cap, sorted_token_ids,
                             expert_ids, num_valid);
  if (st) return st;
  if (pre && row_bytes(dtype, D) % 128) return MOE_EUNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!ok_ptr(x) || !ok_ptr(w1) || !ok_ptr(a)) return MOE_EINVAL;
  if (quantised(dtype)) {
    if (!ok_ptr(x_scale) || !ok_ptr(w1_scale) || !ok_ptr(a_scale)) return MOE_EINVAL;
    if ((int64_t)ws_bytes < moe_gemm1_workspace_bytes(dtype, T, topk, I)) return MOE_ENOSPC;
    if (!ok_ptr(workspace)) return MOE_EINVAL;
  }
  const int64_t cap = moe::sorted_capacity(T, E, topk, block_m);
  return launch_status(moe::launch_gemm1(dtype, pre, x, x_scale, w1, w1_scale, sorted_token_ids,
                                         expert_ids, num_valid, cap, T, E, topk, D, I, block_m, a,
                                         a_scale, workspace, nullptr, 0, (hipStream_t)stream));
}

int moe_gemm2_down(int dtype, const void* a, const void* a_scale, const void* w2,
                   const void* w2_scale, const float* topk_weights,
                   const int32_t* sorted_token_ids, const int32_t* expert_ids,
                   const int32_t* num_valid, int64_t sorted_cap, int T, int E, int topk, int D,
                   int I, int block_m, int mode, void* y, void* stream) {
  int pre;
  dtype = base_dtype(dtype, &pre);
  if (!ok_mode(mode)) return MOE_EINVAL;
  int st = check_gemm_common(dtype, T, E, topk, D, I, block_m, sorted_cap, sorted_token_ids,
                             expert_ids, num_valid);
  if (st) return st;
  if (pre && row_bytes(dtype, I) % 128) return MOE_EUNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!ok_ptr(a) || !ok_ptr(w2) || !ok_ptr(topk_weights) || !ok_ptr(y)) return MOE_EINVAL;
  if (quantised(dtype) && (!ok_ptr(a_scale) || !ok_ptr(w2_scale))) return MOE_EINVAL;
  const int64_t cap = moe::sorted_capacity(T, E, topk, block_m);
  return launch_status(moe::launch_gemm2(dtype, pre, a, a_scale, w2, w2_scale, topk_weights,
                                         sorted_token_ids, expert_ids, num_valid, cap, T, E, topk,
                                         D, I, block_m, mode, y, (hipStream_t)stream));
}

int moe_finalize(int mode, const void* y, int T, int topk, int D, uint16_t* out, void* stream) {
  if (!ok_mode(mode)) return MOE_EINVAL;
  if (T < 0 || topk < 1 || D < 64 || D % 64) return T < 0 || topk < 1 ? MOE_EINVAL : MOE_EUNSUPPORTED;
  if ((int64_t)T * topk * D > INT_MAX) return MOE_ERANGE;
  if (T == 0 || mode == MOE_OUT_ATOMIC_BF16) return MOE_OK;  // bf16 atomics: stage 2 wrote out
  if (!ok_ptr(y) || !ok_ptr(out)) return MOE_EINVAL;
  return launch_status(moe::launch_finalize(mode, y, T, topk, D, out, (hipStream_t)stream));
}

}  // extern "C"

// moe_forward's checks and launches; `workspace(total, &ws)` supplies the workspace once every
// argument check has passed and returns MOE_OK or an error code.
template <class GetWorkspace>
static int forward_impl(int dtype, int score, int renorm, int mode, const float* logits, const void* x,
                        const void* x_scale, const void* w1, const void* w1_scale, const void* w2,
                        const void* w2_scale, int T, int E, int topk, int D, int I, int block_m,
                        GetWorkspace workspace, uint16_t* out, void* stream) {
  int pre;
  dtype = base_dtype(dtype, &pre);
  if (!ok_mode(mode)) return MOE_EINVAL;
  if (score != MOE_SCORE_SOFTMAX && score != MOE_SCORE_SIGMOID) return MOE_EINVAL;
  if (renorm != 0 && renorm != 1) return MOE_EINVAL;
  int st = check_layer_dims(dtype, T, E, topk, D, I, block_m);
  if (st) return st;
  if (pre && (row_bytes(dtype, D) % 128 || row_bytes(dtype, I) % 128)) return MOE_EUNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!ok_ptr(logits) || !ok_ptr(x) || !ok_ptr(w1) || !ok_ptr(w2) || !ok_ptr(out)) return MOE_EINVAL;
  if (quantised(dtype) && (!ok_ptr(x_scale) || !ok_ptr(w1_scale) || !ok_ptr(w2_scale))) return MOE_EINVAL;
  const Layout L = forward_layout(dtype, mode, T, E, topk, D, I, block_m);
  char* ws = nullptr;
  st = workspace(L.total, &ws);
  if (st) return st;

  auto at = [&](int f) -> void* { return L.off[f] < 0 ? nullptr : ws + L.off[f]; };
  float* topk_w = static_cast<float*>(at(0));
  int32_t* topk_ids = static_cast<int32_t*>(at(1));
  int32_t* sorted = static_cast<int32_t*>(at(2));
  int32_t* eids = static_cast<int32_t*>(at(3));
  int32_t* nvalid = static_cast<int32_t*>(at(4));
  void* rws = at(5);
  void* a = at(6);
  void* a_scale = at(7);
  void* g1ws = at(8);
  void* y = at(9);
  // ATOMIC clears the fp32 accumulator, ATOMIC_BF16 the bf16 output (T*D/2 floats' worth)
  float* zero = mode == MOE_OUT_ATOMIC ? static_cast<float*>(y)
              : mode == MOE_OUT_ATOMIC_BF16 ? reinterpret_cast<float*>(out) : nullptr;
  const int64_t zero_n = mode == MOE_OUT_ATOMIC ? (int64_t)T * D : mode == MOE_OUT_ATOMIC_BF16 ? (int64_t)T * D / 2 : 0;
  void* y2 = mode == MOE_OUT_ATOMIC_BF16 ? static_cast<void*>(out) : y;
  const int64_t cap = moe::sorted_capacity(T, E, topk, block_m);
  hipStream_t s = (hipStream_t)stream;

  // the atomic accumulator is cleared by the gate-up kernel's blocks on their way in
  hipError_t e = moe::launch_route(logits, T, E, topk, score, renorm, 1, 1, block_m, topk_w, topk_ids,
                                   sorted, cap, eids, nvalid, rws, s);
  if (e == hipSuccess)
    e = moe::launch_gemm1(dtype, pre, x, x_scale, w1, w1_scale, sorted, eids, nvalid, cap, T, E, topk,
                          D, I, block_m, a, a_scale, g1ws, zero, zero_n, s);
  if (e == hipSuccess)
    e = moe::launch_gemm2(dtype, pre, a, a_scale, w2, w2_scale, topk_w, sorted, eids, nvalid, cap, T,
                          E, topk, D, I, block_m, mode, y2, s);
  if (e == hipSuccess) e = moe::launch_finalize(mode, y, T, topk, D, out, s);
  return launch_status(e);
}

extern "C" {

int moe_forward(int dtype, int score, int renorm, int mode, const float* logits, const void* x,
                const void* x_scale, const void* w1, const void* w1_scale, const void* w2,
                const void* w2_scale, int T, int E, int topk, int D, int I, int block_m,
                void* workspace, size_t ws_bytes, uint16_t* out, void* stream) {
  auto caller_ws = [&](int64_t total, char** ws) -> int {
    if (!ok_ptr(workspace)) return MOE_EINVAL;
    if ((int64_t)ws_bytes < total) return MOE_ENOSPC;
    *ws = static_cast<char*>(workspace);
    return MOE_OK;
  };
  return forward_impl(dtype, score, renorm, mode, logits, x, x_scale, w1, w1_scale, w2, w2_scale, T, E,
                      topk, D, I, block_m, caller_ws, out, stream);
}

int moe_forward_noalloc(int dtype, int score, int renorm, int mode, const float* logits,
                        const void* x, const void* x_scale, const void* w1, const void* w1_scale,
                        const void* w2, const void* w2_scale, int T, int E, int topk, int D, int I,
                        int block_m, uint16_t* out, void* stream) {
  auto static_ws = [&](int64_t total, char** ws) -> int {
    if (total > moe::kNoAllocScratchBytes) return MOE_ENOSPC;
    void* p = nullptr;
    if (moe::noalloc_scratch(&p) != hipSuccess) return MOE_ELAUNCH;
    *ws = static_cast<char*>(p);
    return MOE_OK;
  };
  return forward_impl(dtype, score, renorm, mode, logits, x, x_scale, w1, w1_scale, w2, w2_scale, T, E,
                      topk, D, I, block_m, static_ws, out, stream);
}

int64_t moe_forward_noalloc_max_bytes(void) { return moe::kNoAllocScratchBytes; }

int moe_preshuffle_weights(int dtype, const void* w, int64_t rows, int K, void* w_out,
                           void* stream) {
  if (dtype != MOE_BF16 && dtype != MOE_FP8_E4M3 && dtype != MOE_MXFP4) return MOE_EINVAL;
  if (rows < 0 || K < 1) return MOE_EINVAL;
  if (rows % 16 || row_bytes(dtype, K) % 128 || (dtype == MOE_MXFP4 && K % 2)) return MOE_EUNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!ok_ptr(w) || !ok_ptr(w_out) || w == w_out) return MOE_EINVAL;
  const int64_t rb = row_bytes(dtype, K);
  if (rb > INT_MAX) return MOE_ERANGE;
  return launch_status(moe::launch_preshuffle(w, rows, (int)rb, w_out, (hipStream_t)stream));
}

int moe_preshuffle_scales(const uint8_t* s, int64_t rows, int K, uint8_t* s_out, void* stream) {
  if (rows < 0 || K < 1) return MOE_EINVAL;
  if (rows % 16 || K % 256) return MOE_EUNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!ok_ptr(s) || !ok_ptr(s_out) || s == s_out) return MOE_EINVAL;
  return launch_status(moe::launch_preshuffle_scales(s, rows, K / 32, s_out, (hipStream_t)stream));
}

}  // extern "C"
