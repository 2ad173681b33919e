/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE-layer forward hot path.
 *
 * The layer: router top-k gating (softmax or sigmoid) fused with a stable,
 * block-padded expert sort, then a two-stage expert GEMM -- gate-up with
 * silu(gate)*up, then a down projection scaled by the routed weight and
 * combined into out[token, model_dim].
 *
 * Sources (web pages; cited by title and section):
 *  [P1] "[Feat] Fuse TopKGatingSoftmax and MoE Sorting kernels" (ROCm/FlyDSL #582)
 *  [P2] "[MoE] Port moe_gemm_2stage (stage1+stage2) to the new fx.* pipeline --
 *       fp8 (gfx942 + gfx950)" (ROCm/FlyDSL #947)
 *  [P3] "[Common] Optimize fused router forward/backward kernels"
 *       (NVIDIA/TransformerEngine #3012)
 *  [P4] "[RadeonFlow] flydsl mxfp4 a4w4 MoE: bring gemm1/gemm2 to parity with
 *       the HIP backend" (ROCm/aiter #3828)
 *
 * Conventions for every entry point
 *  - Tensor arguments are DEVICE pointers to dense row-major storage that the
 *    caller allocates and owns.  The library never allocates, frees or
 *    synchronises: it validates arguments on the host, enqueues kernels on
 *    `stream` (a hipStream_t passed as void*; NULL = the null stream) and
 *    returns.  Raw base pointers and integer sizes only ([P4] "Changes / ABI":
 *    bare device addresses as kernel arguments).
 *  - Return value: MOE_OK (0) or a negative moe_status.  On any error other
 *    than MOE_ELAUNCH nothing has been enqueued.  All argument checks run
 *    before the first HIP call.  No C++ exception crosses the ABI.  Faults
 *    inside kernels surface at the caller's next synchronisation.
 *  - Alignment: tensors of 2-byte or wider elements and every fp8 tensor
 *    must be 16-byte aligned; otherwise MOE_EINVAL.
 *  - Calls on different streams may run concurrently if their output and
 *    workspace buffers are disjoint; the library keeps no global state (apart
 *    from moe_forward_noalloc's static workspace, see there).
 *  - Size limits of the layer calls: T*k*D and T*k*I below 2^31 (per-slot-row
 *    offsets are 32-bit), else MOE_ERANGE; at the Kimi-K2.5 share (k=9, D=7168)
 *    that is T <= 33288.  The LDS-tiled prefill GEMMs run when block_m = 64,
 *    T*k >= 32*E and the rows they gather and one expert's weights each span
 *    less than 2 GB: T rows of D elements and 2*I rows of D for the gate-up,
 *    T*k rows of I elements and D rows of I for the down projection, in bytes
 *    of the dtype (mxfp4 also needs D and I multiples of 256).  Past those
 *    limits the decode kernels (64-bit addressing) compute the same result,
 *    several times slower at prefill sizes; at the Kimi-K2.5 share every T
 *    the layer calls accept stays on the prefill GEMMs.
 *
 * Notation: T tokens, E experts, k = topk, D = model_dim, I = inter_dim,
 * B = block_m.  Slot s = t*k + j is token t's j-th ranked expert.  The
 * sentinel slot value is T*k.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum moe_status {
  MOE_OK = 0,
  MOE_EINVAL = -1,        /* bad enum, null or misaligned pointer, topk not in [1,E], T < 0 */
  MOE_ERANGE = -2,        /* T*E (or a derived size) does not fit a signed 32-bit int ([P3] "Hardening") */
  MOE_ENOSPC = -3,        /* sorted_cap or ws_bytes smaller than required */
  MOE_EUNSUPPORTED = -4,  /* E > 8160, block_m not in {16,32,64}, D or I not a positive multiple of 64
                             (of 128 for MOE_MXFP4) */
  MOE_ELAUNCH = -5        /* a kernel launch failed (hipGetLastError) */
};

enum moe_score { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 };
enum moe_dtype { MOE_BF16 = 0, MOE_FP8_E4M3 = 1, MOE_MXFP4 = 2 };
enum moe_mode { MOE_OUT_ATOMIC = 0, MOE_OUT_REDUCE = 1, MOE_OUT_ATOMIC_BF16 = 2, MOE_OUT_REDUCE_BF16 = 3 };

/* OR-ed into the dtype of moe_gemm1_gateup, moe_gemm2_down and moe_forward (and accepted,
 * and ignored, by the workspace-size functions): w1 and w2 are in fragment order, as written
 * by moe_preshuffle_weights, and for mxfp4 so are w1_scale and w2_scale, as written by
 * moe_preshuffle_scales (fp8 per-row scales keep their layout).  Needs rows of whole
 * 128-byte K chunks (fp8: D and I multiples of 128; mxfp4: of 256), else MOE_EUNSUPPORTED.
 * Results are bit-identical to the natural layout's. */
#define MOE_PRESHUFFLED 0x100

/* Largest E accepted ([P3] "Hardening": the radix top-k path's 8160-expert bound). */
#define MOE_MAX_EXPERTS 8160

/* ---------------------------------------------------------------- host helpers
 * Pure host functions: no device work, callable without a GPU. */

/* Length of sorted_token_ids that always suffices:
 * roundup_B(T*k + min(E, T*k)*(B-1)).  Returns a negative moe_status for
 * invalid arguments. */
int64_t moe_sorted_capacity(int T, int E, int topk, int block_m);

/* Workspace bytes moe_topk_softmax_sort needs (0 when T is small enough for
 * the single-workgroup path).  Negative moe_status on invalid arguments. */
int64_t moe_route_workspace_bytes(int T, int E, int topk, int block_m);

/* Workspace bytes moe_gemm1_gateup needs: 0 for bf16; for fp8 and mxfp4 the bf16
 * intermediate rows [T*k, I] that are requantised. */
int64_t moe_gemm1_workspace_bytes(int dtype, int T, int topk, int I);

/* moe_forward's workspace: the routing outputs, the intermediate and the fp32
 * accumulator, each at a 256-byte aligned offset.  Fields (byte offsets written
 * to offsets[0..MOE_WS_NFIELDS-1]; a field a configuration does not use has
 * offset -1):
 *   0 topk_weights fp32 [T,k]      1 topk_ids int32 [T,k]
 *   2 sorted_token_ids int32 [cap] 3 expert_ids int32 [cap/B]
 *   4 num_valid int32 [1]          5 routing scratch
 *   6 a: bf16 [T*k,I], e4m3 [T*k,I] or packed mxfp4 [T*k,I/2]
 *   7 a_scale: fp32 [T*k] (fp8), E8M0 uint8 [T*k,I/32] (mxfp4)
 *   8 gemm1 scratch (fp8, mxfp4: bf16 [T*k,I])
 *   9 y: ATOMIC fp32 [T,D] accumulator, REDUCE fp32 [T*k,D] slot rows,
 *        REDUCE_BF16 bf16 [T*k,D] slot rows
 *        (ATOMIC_BF16: unused, -1; the stage-2 atomics add into out itself)
 * Returns the total size in bytes, or a negative moe_status. */
#define MOE_WS_NFIELDS 10
int64_t moe_forward_workspace_layout(int dtype, int mode, int T, int E, int topk, int D, int I,
                                     int block_m, int64_t* offsets);

/* Total workspace bytes of moe_forward (the value moe_forward_workspace_layout returns), or 0
 * when the arguments are invalid (a valid layout is never empty: every field takes at least
 * 256 bytes); moe_forward_workspace_layout gives the status code of an invalid call. */
size_t moe_forward_workspace_bytes(int dtype, int mode, int T, int E, int topk, int D, int I,
                                   int block_m);

/* Static description of a status code. */
const char* moe_strerror(int status);

/* ---------------------------------------------------------------- routing
 * [P1] "Motivation", "Relevant Files", "Additional Details": top-k gating
 * softmax fused with the MoE sorting step; [P3] "Changes / Forward kernels"
 * and the flowchart: score function (softmax or sigmoid), then top-k.
 *
 * Per token t: the k experts with the largest fp32 logits, best first, ties
 * to the lower expert index (selection on the logits equals selection on the
 * strictly increasing score).  -0.0 and +0.0 are equal.  NaN logits are
 * outside the contract.
 * Weights (fp32): softmax renormalised over the k picks
 * (= softmax of the picked logits), or sigmoid(logit) divided by the sum over
 * the picks; with renorm = 0 the score itself (softmax over all E, or the
 * sigmoid) at the picks.
 * Sort: c_e = #slots routed to e; each non-empty expert's slots, ascending,
 * padded with the sentinel T*k up to a multiple of B, concatenated by expert
 * index; experts with no slot get no block.  num_valid = total padded length.
 *
 *   logits           fp32  [T, E]               in
 *   topk_weights     fp32  [T, k]               out
 *   topk_ids         int32 [T, k]               out, rank order
 *   sorted_token_ids int32 [sorted_cap]         out, slots; sentinel T*k in the padding and
 *                                               in [num_valid, sorted_cap)
 *   expert_ids       int32 [sorted_cap / B]     out, expert of each B-row block; -1 past num_valid
 *   num_valid        int32 [1]                  out
 *   workspace        moe_route_workspace_bytes(...) bytes (may be NULL when that is 0)
 * T = 0 is valid: only num_valid (= 0) is written.
 * Deterministic: repeated calls give bit-identical outputs. */
int moe_topk_softmax_sort(const float* logits, int T, int E, int topk, int score, int renorm,
                          int block_m, float* topk_weights, int32_t* topk_ids,
                          int32_t* sorted_token_ids, int64_t sorted_cap, int32_t* expert_ids,
                          int32_t* num_valid, void* workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- group-limited routing
 * [P3] "Hardening" (topk must be a multiple of group_topk) and the review's group scores of
 * the forward kernels: top-k limited to the best groups of experts.  The E experts form
 * n_group groups of E/n_group consecutive experts.  A group's score is the sum of its
 * m = topk/topk_group largest expert scores (softmax over all E, or the sigmoid; fp64,
 * best first); the topk_group groups with the largest scores are kept (ties to the lower
 * group index) and the top-k of the logits is taken among their experts, as in
 * moe_topk_softmax_sort.  Weights, sort and outputs are those of moe_topk_softmax_sort
 * (with renorm = 0 and softmax the weight is still the softmax over all E).  Group
 * decisions depend on fp64 sums; two groups whose scores agree to rounding may be ranked
 * either way.
 *   n_group     >= 1, divides E; 1 (or topk_group = n_group) is the plain top-k
 *   topk_group  in [1, n_group]; topk % topk_group == 0 and topk <= topk_group * E/n_group,
 *               else MOE_EINVAL
 * Group-limited selection needs n_group <= 64 and E <= 4096 (MOE_EUNSUPPORTED otherwise).
 * Workspace and capacity as for moe_topk_softmax_sort. */
int moe_topk_softmax_sort_grouped(const float* logits, int T, int E, int topk, int n_group,
                                  int topk_group, int score, int renorm, int block_m,
                                  float* topk_weights, int32_t* topk_ids,
                                  int32_t* sorted_token_ids, int64_t sorted_cap,
                                  int32_t* expert_ids, int32_t* num_valid, void* workspace,
                                  size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- routing backward
 * [P3] "Changes / Backward kernels" and the summary's "Backward (E=2304, K=36)": the fused
 * router's backward.  The gradient of the weights moe_topk_softmax_sort returned, with
 * respect to the logits, at the selection it made (nothing flows through the selection,
 * which is piecewise constant).  Per token, with g = grad_topk_weights, w = topk_weights,
 * S its picks, s = sigmoid(logit):
 *   softmax, renorm=1:  dl[e_j] = w_j (g_j - sum_i w_i g_i)
 *   sigmoid, renorm=1:  dl[e_j] = s_j (1 - s_j) (g_j - sum_i w_i g_i) / sum_i s_i
 *   softmax, renorm=0:  dl[e]   = p_e (G_e - sum_j w_j g_j), p = softmax over all E,
 *                                 G_e = g_j if e = e_j, else 0   (every expert)
 *   sigmoid, renorm=0:  dl[e_j] = s_j (1 - s_j) g_j
 * and dl = 0 for every other expert.  fp32 arithmetic.
 *
 *   logits             fp32  [T, E]   the forward's input
 *   topk_ids           int32 [T, k]   and topk_weights fp32 [T, k]: the forward's outputs
 *   grad_topk_weights  fp32  [T, k]
 *   grad_logits        fp32  [T, E]   out, every element written
 * Validation as for moe_topk_softmax_sort (no block_m, no sort outputs). */
int moe_topk_softmax_backward(const float* logits, const int32_t* topk_ids,
                              const float* topk_weights, const float* grad_topk_weights, int T,
                              int E, int topk, int score, int renorm, float* grad_logits,
                              void* stream);

/* ---------------------------------------------------------------- auxiliary-loss scores
 * [P3] the summary, the "aux_loss fprop / bprop" benchmark rows and the file table: the
 * router kernel that computes the scores of the load-balancing auxiliary loss, forward and
 * backward.  Per token, over all E experts:
 *   scores       fp32  [T, E]  out: softmax of the logits, or the sigmoids divided by
 *                              their sum (score = MOE_SCORE_SIGMOID); each row sums to 1
 *   routing_map  uint8 [T, E]  out: 1 at the token's topk experts (largest logits, ties
 *                              to the lower index, as moe_topk_softmax_sort), else 0
 *   logits       fp32  [T, E]  in
 * Accuracy: relative error of a few fp32 ulp per score for any logit range.
 * Validation: topk in [1, E], E <= 4096 (else MOE_EUNSUPPORTED), T*E within int32, pointers
 * non-null and 16-byte aligned when T > 0.  T = 0 writes nothing. */
int moe_aux_loss_scores(const float* logits, int T, int E, int topk, int score, float* scores,
                        uint8_t* routing_map, void* stream);

/* Gradient of moe_aux_loss_scores' scores with respect to the logits (the routing map is
 * piecewise constant and passes none).  g = grad_scores, p the softmax, s the sigmoids,
 * S = sum_e s_e, q = s / S:
 *   softmax:  dl_c = p_c (g_c - sum_e p_e g_e)
 *   sigmoid:  dl_c = s_c (1 - s_c) / S * (g_c - sum_e q_e g_e)
 *   logits, grad_scores  fp32 [T, E] in;  grad_logits  fp32 [T, E] out, every element.
 * fp32 arithmetic with fp64 sums.  Validation as for moe_aux_loss_scores. */
int moe_aux_loss_scores_backward(const float* logits, const float* grad_scores, int T, int E,
                                 int score, float* grad_logits, void* stream);

/* ---------------------------------------------------------------- weight preshuffle
 * [P2] the gate-up helper commit ("make_gateup_weight_view": a preshuffle of the weights into
 * the order the MFMA consumes them) and the stage-2 decode profile (the gap is memory-latency
 * bound, led by the weight loads).  A one-time layout change of a weight tensor: for each
 * group of 16 consecutive rows and each 128-byte chunk of K, 2 KB holding, for half h (0, 1)
 * and lane l = i + 16 g (i < 16, g < 4), the 16 bytes [128 c + 64 h + 16 g, + 16) of row
 * 16 R + i.  Each 1 KB is then what one wave's 16-byte load brings in for one operand
 * register, contiguous in memory.  Scales are not touched: fp8 per-row scales keep their
 * layout, mxfp4 E8M0 blocks go through moe_preshuffle_scales.
 *   w      [rows, K] in the dtype's storage (bf16: 2K bytes per row, fp8: K, mxfp4: K/2);
 *          an expert tensor [E, N, K] is rows = E*N
 *   w_out  the same size; must not overlap w
 * rows must be a multiple of 16 and a row a whole number of 128-byte chunks
 * (MOE_EUNSUPPORTED otherwise); dtype without flags. */
int moe_preshuffle_weights(int dtype, const void* w, int64_t rows, int K, void* w_out,
                           void* stream);

/* The E8M0 block scales of an mxfp4 weight tensor into fragment order, the companion of
 * moe_preshuffle_weights for MOE_PRESHUFFLED mxfp4 calls ([P4] "Summary": a4w4 with one
 * E8M0 scale per 32 elements along K; the same one-time layout change as for the weights).
 * For each group of 16 consecutive rows and each 256-element chunk c of K (one 128-byte chunk
 * of E2M1 codes), 128 bytes holding, for row i < 16, the 8 scale bytes [8 c, 8 c + 8) of row
 * 16 R + i: the scales a wave reads for one chunk of 16 weight rows are one line.
 *   s      uint8 [rows, K/32] (an expert tensor [E, N, K/32] is rows = E*N)
 *   s_out  the same size; must not overlap s
 * rows must be a multiple of 16 and K of 256 (MOE_EUNSUPPORTED otherwise); null or
 * mis-aligned pointers, rows < 0 or K < 1 give MOE_EINVAL. */
int moe_preshuffle_scales(const uint8_t* s, int64_t rows, int K, uint8_t* s_out, void* stream);

/* ---------------------------------------------------------------- stage 1
 * [P2] gate-up helper and stage-1 commits ("silu(gate)*up with optional fp8
 * weight/act dequant -> bf16"; B-first MFMA with the weight as the first
 * operand; sorted-row gather).
 *
 * For every B-row block b < num_valid/B with e = expert_ids[b] and every row
 * holding a real slot s (token t = s / k):
 *   g[n] = sum_d W1[e, n, d] * x[t, d],  u[n] = sum_d W1[e, I+n, d] * x[t, d]   (n < I)
 *   a[s, n] = bf16_rne(silu(g[n]) * u[n]),  silu(z) = z / (1 + exp(-z))
 * Rows [0,I) of each expert's W1 are the gate, rows [I,2I) the up projection.
 * fp8 (e4m3fn): x[t,:] carries scale x_scale[t], W1[e,n,:] scale w1_scale[e,n];
 * the bf16 row a[s,:] is then requantised: a_scale[s] = amax_n|a[s,n]| / 448
 * (1.0 for an all-zero row), codes = e4m3_rne(a / a_scale[s]) clamped to +-448.
 *
 * mxfp4 ([P4] "Summary": 4-bit activations and weights, "a4w4"; the format is the OCP
 * Microscaling one): x, W1 (and W2, a) hold E2M1 codes two per byte, element 2j in the
 * low nibble, with one E8M0 scale 2^(s-127) per block of 32 consecutive elements along K;
 * the bf16 row a[s,:] is requantised block by block: scale 2^(floor(log2 amax) - 2) (2^0
 * for an all-zero block), codes = E2M1 round-to-nearest-even of a/scale, saturating at 6.
 *
 *   x         bf16 [T, D] | e4m3 [T, D] | mxfp4 uint8 [T, D/2]
 *   x_scale   fp32 [T] (fp8) | E8M0 uint8 [T, D/32] (mxfp4) | NULL (bf16)
 *   w1        bf16 [E, 2I, D] | e4m3 | mxfp4 uint8 [E, 2I, D/2]
 *   w1_scale  fp32 [E, 2I] (fp8) | E8M0 uint8 [E, 2I, D/32] (mxfp4)
 *   sorted_token_ids, expert_ids, num_valid: as written by moe_topk_softmax_sort
 *   a         bf16 [T*k, I] | e4m3 [T*k, I] | mxfp4 uint8 [T*k, I/2]   out (every slot row)
 *   a_scale   fp32 [T*k] (fp8) | E8M0 uint8 [T*k, I/32] (mxfp4)         out
 *   workspace moe_gemm1_workspace_bytes(...) bytes (fp8, mxfp4), else may be NULL */
int moe_gemm1_gateup(int dtype, const void* x, const void* x_scale, const void* w1,
                     const void* w1_scale, const int32_t* sorted_token_ids,
                     const int32_t* expert_ids, const int32_t* num_valid, int64_t sorted_cap,
                     int T, int E, int topk, int D, int I, int block_m, void* a, void* a_scale,
                     void* workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- stage 2
 * [P2] stage-2 commit: down projection with per-token(row) x per-channel
 * (model_dim) fp8 dequant, the routed weight, and two epilogue modes:
 * atomic accumulation into out[token, model_dim], or a plain store of
 * out[token*topk + slot, model_dim] for a separate reduction, in fp32 or in the
 * output's 16-bit type.  Padding rows issue no store and no atomic.
 *
 * For every real slot s = t*k + j in a block of expert e:
 *   c_s[d] = topk_weights[s] * sum_n W2[e, d, n] * a[s, n]
 *            (fp8: * a_scale[s] * w2_scale[e, d])
 *   ATOMIC:      y[t, d] += c_s[d]   (y fp32 [T, D]; the caller zeroes it first)
 *   REDUCE:      y[s, d]  = c_s[d]   (y fp32 [T*k, D])
 *   REDUCE_BF16: y[s, d]  = bf16_rne(c_s[d])   (y bf16 [T*k, D]: half the bytes of REDUCE
 *                to write here and to read in moe_finalize; each contribution moves by at
 *                most 2^-8 * |c_s[d]|, half a bf16 step)
 *   ATOMIC_BF16: y[t, d] += c_s[d]   (y bf16 [T, D], zeroed by the caller; [P2] "atomic
 *                scatter into out": each c_s[d] is rounded to bf16 and added to the
 *                pair (d, d+1) with one packed bf16 atomic add, which rounds the running
 *                sum to bf16 again.  Half the atomic operations of ATOMIC; the result
 *                depends on the order of the k adds, and beyond ATOMIC's rounding it may
 *                differ from the exact sum by up to about (k+1) * 2^-8 * sum_j |c_{t*k+j}[d]|:
 *                k + 1 roundings to bf16, each of at most half a bf16 step, 2^-8 of a value
 *                no larger in magnitude than that sum.)
 *
 *   mxfp4: the block scales of a and W2 enter the products; no per-row factors.
 *
 *   a, a_scale        as written by moe_gemm1_gateup
 *   w2                bf16 [E, D, I] | e4m3 [E, D, I] | mxfp4 uint8 [E, D, I/2]
 *   w2_scale          fp32 [E, D] (fp8) | E8M0 uint8 [E, D, I/32] (mxfp4)
 *   topk_weights      fp32 [T, k] */
int moe_gemm2_down(int dtype, const void* a, const void* a_scale, const void* w2,
                   const void* w2_scale, const float* topk_weights,
                   const int32_t* sorted_token_ids, const int32_t* expert_ids,
                   const int32_t* num_valid, int64_t sorted_cap, int T, int E, int topk, int D,
                   int I, int block_m, int mode, void* y, void* stream);

/* ---------------------------------------------------------------- combine
 * [P2] stage-2 commit and summary: the reduce mode's separate reduction kernel.
 * ATOMIC: out[t, d] = bf16_rne(y[t, d]), y fp32 [T, D].
 * REDUCE: out[t, d] = bf16_rne(sum_j y[t*k + j, d]) summed in fp32, j ascending.
 * REDUCE_BF16: the same over the bf16 slot rows (each widened to fp32 exactly).
 * ATOMIC_BF16: nothing to do (stage 2 wrote the bf16 result); y and out are not used.
 *   y   as written by moe_gemm2_down in the same mode (fp32, or bf16 for REDUCE_BF16)
 *   out bf16 [T, D] */
int moe_finalize(int mode, const void* y, int T, int topk, int D, uint16_t* out, void* stream);

/* ---------------------------------------------------------------- whole layer
 * moe_topk_softmax_sort -> (ATOMIC: zero the accumulator; ATOMIC_BF16: zero out)
 * -> moe_gemm1_gateup -> moe_gemm2_down -> moe_finalize, all on `stream`, with every
 * intermediate in `workspace` at the offsets moe_forward_workspace_layout reports (so
 * they can be read back).  out bf16 [T, D]. */
int moe_forward(int dtype, int score, int renorm, int mode, const float* logits, const void* x,
                const void* x_scale, const void* w1, const void* w1_scale, const void* w2,
                const void* w2_scale, int T, int E, int topk, int D, int I, int block_m,
                void* workspace, size_t ws_bytes, uint16_t* out, void* stream);

/* ---------------------------------------------------------------- no-allocation variant
 * For callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  moe_forward with the same arguments
 * minus the workspace: the workspace lives in a static device array of
 * moe_forward_noalloc_max_bytes() bytes (32 MiB) that every device the library runs on holds
 * from module load until the process ends; the call allocates nothing.  The intermediates
 * sit at the offsets moe_forward_workspace_layout reports, inside that array.
 * Errors: those of moe_forward, and MOE_ENOSPC when moe_forward_workspace_bytes(...) exceeds
 * the array (then nothing is enqueued; the DeepSeek-R1, GPT-OSS and Kimi-K2.5 decode shapes
 * need at most about 3 MB); MOE_ELAUNCH if the array's device address cannot be obtained.
 * Every call on one device uses that device's array: calls that overlap on one device (other
 * streams, other threads) race and must be ordered by the caller.  The array keeps the last
 * call's contents; every call rewrites what it reads. */
int moe_forward_noalloc(int dtype, int score, int renorm, int mode, const float* logits,
                        const void* x, const void* x_scale, const void* w1, const void* w1_scale,
                        const void* w2, const void* w2_scale, int T, int E, int topk, int D, int I,
                        int block_m, uint16_t* out, void* stream);

/* Size in bytes of moe_forward_noalloc's static workspace. */
int64_t moe_forward_noalloc_max_bytes(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
