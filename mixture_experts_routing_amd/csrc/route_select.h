// Per-token top-k selection with one wavefront, shared by the router (route.hip) and the
// auxiliary-loss scores (route_aux.hip).
//
// [P1] "Fuse TopKGatingSoftmax and MoE Sorting kernels" (ROCm/FlyDSL #582): top-k gating
// per token.  [P3] "Optimize fused router forward/backward kernels"
// (NVIDIA/TransformerEngine #3012), "Changes / Forward kernels": the score function, then
// the top-k; "Hardening": topk must be a multiple of group_topk (group-limited routing).
//
// Lane l holds the logits of experts l, l+64, ... as order-preserving u32 keys.  The lanes
// form G lane groups (G the power of two >= 2k, at most 64); the k-th largest of the G
// lane-group maxima is a threshold that at least k keys reach.  The keys at or above it
// (typically a few to a few dozen) are compacted into LDS (a ballot per register gives each
// lane its slot), and each candidate's rank is the number of larger (key, ~expert) pairs
// among them.  If more than 128 keys reach the threshold (heavy ties) or k > 64, a slower
// exact path extracts the maximum k times.
//
// Group-limited selection (GROUPED): the E experts form n groups of E/n consecutive
// experts; a group's score is the sum of its m = k/topk_group best expert scores (softmax
// numerators exp(l - max) or sigmoids, fp64, best first).  The topk_group best groups stay
// (ties to the lower group index) and the logits of the other groups are masked out before
// the selection above.  The token's keys are staged in LDS.  With n a power of two, m <= 4
// and E/n a multiple of 64/n, each group is spread over 64/n lanes: a lane keeps the top 4
// of its contiguous slice of keys and the lists are merged across the group's lanes by a
// butterfly; otherwise lane j scans group j alone.
#pragma once

#include "moe_device.h"

namespace moe {

constexpr int kMaxCand = 128;
// Group-limited selection: at most 64 groups (one lane each) and E <= 4096 (keys in LDS).
constexpr int kGroupMaxGroups = 64;
constexpr int kGroupMaxE = 4096;

// Wave-uniform description of the group-limited selection; keys is this wave's LDS buffer
// of E u32 keys.
struct GroupSel {
  int n = 1;      // groups
  int keep = 1;   // groups kept (topk_group)
  int size = 1;   // experts per group
  int m = 1;      // best experts summed per group (k / keep)
  int lanes = 0;  // lanes per group in the spread scan (64 / n), 0 = one lane per group
  int per = 0;    // keys per lane in the spread scan (size / lanes)
  uint32_t* keys = nullptr;
};

// Inserts key x into the descending list t (0 = empty slot).
__device__ __forceinline__ void top4_insert(uint32_t (&t)[4], uint32_t x) {
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const uint32_t hi = max(t[i], x);
    x = min(t[i], x);
    t[i] = hi;
  }
  t[3] = max(t[3], x);
}

// t := the 4 largest of t and the list of lane ^ M (both descending).  The elementwise
// maximum of one list and the other reversed holds them as a bitonic sequence, which two
// compare stages sort.
template <int M>
__device__ __forceinline__ void top4_merge(uint32_t (&t)[4]) {
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = xor_lane<M>(t[i]);
  const uint32_t p0 = max(t[0], o[3]), p1 = max(t[1], o[2]), p2 = max(t[2], o[1]),
                 p3 = max(t[3], o[0]);
  const uint32_t a0 = max(p0, p2), a2 = min(p0, p2), a1 = max(p1, p3), a3 = min(p1, p3);
  t[0] = max(a0, a1);
  t[1] = min(a0, a1);
  t[2] = max(a2, a3);
  t[3] = min(a2, a3);
}

// Weight arithmetic runs in fp64 and is rounded to fp32 once: exp of an fp32
// logit difference loses |l - m| * 2^-24 relative accuracy in fp32, which for
// wide logit ranges exceeds the 1e-6 contract.
__device__ __forceinline__ double score_of(double l, double m, bool softmax) {
  return softmax ? exp(l - m) : 1.0 / (1.0 + exp(-l));
}

// Softmax denominator over all E logits of the token (only for softmax without
// renormalisation): sum exp(l - max).  Empty slots hold NaN.
template <int NV>
__device__ double full_softmax_denominator(const float (&x)[NV], double m) {
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < NV; ++i)
    if (x[i] == x[i]) s += exp((double)x[i] - m);
  return wave_sum_f64(s);
}

// Group of expert e for groups of `size` experts (inv = 1/size in fp32): the fp32 quotient
// is within one of the true one for e, size < 2^13, and one correction step fixes it.
__device__ __forceinline__ int group_of(int e, int size, float inv) {
  int q = (int)((float)e * inv);
  const int r = e - q * size;
  q += (int)(r >= size) - (int)(r < 0);
  return q;
}

// Bit j set for each kept group j.  m_all is the token's largest logit (the softmax shift).
template <int NV>
__device__ uint64_t group_keep_mask(const float (&x)[NV], int E, bool softmax, double m_all,
                                    const GroupSel& gs) {
  const int lane = lane_id();
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + 64 * i;
    if (e < E) gs.keys[e] = logit_key(x[i]);
  }
  wave_lds_sync();
  uint64_t keep = 0;
  if (gs.lanes > 0) {
    // spread scan: lanes [g*L, (g+1)*L) hold group g, each a contiguous slice of `per` keys
    const int L = gs.lanes, c = gs.per;
    const int g = lane >> __builtin_ctz(L), sub = lane & (L - 1);
    const uint32_t* p = gs.keys + g * gs.size + sub * c;
    uint32_t t[4] = {0u, 0u, 0u, 0u};
    if ((c & 3) == 0) {
      for (int q = 0; q < c; q += 4) {
        const uint4 v = *reinterpret_cast<const uint4*>(p + q);
        top4_insert(t, v.x);
        top4_insert(t, v.y);
        top4_insert(t, v.z);
        top4_insert(t, v.w);
      }
    } else {
      for (int q = 0; q < c; ++q) top4_insert(t, p[q]);
    }
    wave_lds_sync();  // the key buffer is reused by the next token
    if (L > 1) top4_merge<1>(t);
    if (L > 2) top4_merge<2>(t);
    if (L > 4) top4_merge<4>(t);
    if (L > 8) top4_merge<8>(t);
    if (L > 16) top4_merge<16>(t);
    if (L > 32) top4_merge<32>(t);
    double sc = 0.0;
    for (int r = 0; r < gs.m; ++r) sc += score_of((double)key_logit(t[r]), m_all, softmax);
    int rank = 0;
    const uint64_t sb = __builtin_bit_cast(uint64_t, sc);
    for (int j = 0; j < gs.n; ++j) {
      const double o = __builtin_bit_cast(double, readlane_u64(sb, j * L));
      rank += (o > sc) || (o == sc && j < g);
    }
    const uint64_t lead = __ballot(sub == 0 && rank < gs.keep);
    for (int j = 0; j < gs.n; ++j) keep |= ((lead >> (j * L)) & 1ull) << j;
    return keep;
  }
  double sc = -1.0;  // group scores are >= 0; lanes past the groups never rank ahead
  if (lane < gs.n) {
    const int b = lane * gs.size;
    uint64_t prev = ~0ull;
    sc = 0.0;
    for (int r = 0; r < gs.m; ++r) {
      uint64_t best = 0;
#pragma unroll 4
      for (int q = 0; q < gs.size; ++q) {
        const uint64_t pk = pick_key(gs.keys[b + q], b + q);
        best = (pk < prev && pk > best) ? pk : best;
      }
      prev = best;
      sc += score_of((double)key_logit(pick_logit_key(best)), m_all, softmax);
    }
  }
  wave_lds_sync();  // the key buffer is reused by the next token
  int rank = 0;
  const uint64_t sb = __builtin_bit_cast(uint64_t, sc);
  for (int j = 0; j < gs.n; ++j) {
    const double o = __builtin_bit_cast(double, readlane_u64(sb, j));
    rank += (o > sc) || (o == sc && j < lane);
  }
  return __ballot(lane < gs.n && rank < gs.keep);
}

// Exact selection for heavy ties (more than 128 keys at the threshold) and k > 64: the
// maximum (key, ~expert) pair strictly below the previous pick, k times, 64 ranks per
// pass.  Reads the row again from memory and keeps no per-register state, so that it does
// not raise the register budget of the common path.  The picked logit is parked in w_out
// and turned into the weight once the denominator is known.  With GROUPED only experts of
// the groups in `keep` are eligible and m_all (the row's largest logit) is the softmax
// shift of the full-softmax weights.
template <int NV, bool GROUPED, bool OUT, class OnPick>
__device__ void select_token_exact(const float* __restrict__ row, int E, int k, bool softmax,
                                   int renorm, uint64_t keep, int gsize, double m_all,
                                   float* __restrict__ w_out, int32_t* __restrict__ id_out,
                                   OnPick on_pick) {
  const int lane = lane_id();
  const float ginv = 1.0f / (float)gsize;
  double m = 0.0, denom_all = 1.0, part = 0.0;
  uint64_t prev = ~0ull;
  for (int p = 0; p * 64 < k; ++p) {
    uint64_t mine = 0;
    const int nr = min(64, k - p * 64);
    for (int jj = 0; jj < nr; ++jj) {
      uint64_t best = 0;
#pragma unroll 4
      for (int i = 0; i < NV; ++i) {
        const int e = lane + 64 * i;
        bool ok = e < E;
        if constexpr (GROUPED) ok = ok && ((keep >> group_of(e, gsize, ginv)) & 1ull);
        if (ok) {
          const uint64_t pk = pick_key(logit_key(row[e]), e);
          if (pk < prev && pk > best) best = pk;
        }
      }
      best = wave_max_u64(best);
      if (OUT && p == 0 && jj == 0) {
        m = (double)key_logit(pick_logit_key(best));
        if (softmax && !renorm) {
          if constexpr (GROUPED) m = m_all;
          double s = 0.0;
#pragma unroll 4
          for (int i = 0; i < NV; ++i) {
            const int e = lane + 64 * i;
            if (e < E) s += exp((double)row[e] - m);
          }
          denom_all = wave_sum_f64(s);
        }
      }
      prev = best;
      if (lane == jj) mine = best;
    }
    if (lane < nr) {
      const int r = p * 64 + lane;
      const int e = pick_expert(mine);
      if constexpr (OUT) {
        const float l = key_logit(pick_logit_key(mine));
        part += score_of((double)l, m, softmax);
        w_out[r] = l;
        id_out[r] = e;
      }
      on_pick(r, e);
    }
  }
  if constexpr (OUT) {
    double denom = 1.0;
    if (renorm) denom = wave_sum_f64(part);
    else if (softmax) denom = denom_all;
    for (int r = lane; r < k; r += 64)  // same lane parked w_out[r]
      w_out[r] = (float)(score_of((double)w_out[r], m, softmax) / denom);
  }
}

// The largest key of the wave and the k-th largest of its 64/L lane-group maxima (groups of L
// consecutive lanes), for a group width fixed at compile time: a butterfly takes each group's
// maximum, and a descending bitonic network over the groups (each maximum repeated over its
// group's lanes, so only distances of at least L take part) sorts them.
template <int L>
__device__ __forceinline__ void group_threshold(uint32_t lk, int k, uint32_t& top, uint32_t& tk) {
  const int lane = lane_id();
#pragma unroll
  for (int mm = 1; mm < L; mm <<= 1) {
    const uint32_t o = xor_lane_u32(lk, mm);
    lk = o > lk ? o : lk;
  }
#pragma unroll
  for (int size = 2 * L; size <= 64; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride >= L; stride >>= 1) {
      const uint32_t p = xor_lane_u32(lk, stride);
      const bool keep_max = ((lane & size) == 0) == ((lane & stride) == 0);
      lk = keep_max ? (lk > p ? lk : p) : (lk < p ? lk : p);
    }
  }
  top = readlane_u32(lk, 0);
  tk = readlane_u32(lk, (k - 1) * L);
}

// Loads a token's row: lane l gets experts l, l+64, ...; empty slots hold NaN, which no
// comparison selects.
template <int NV>
__device__ __forceinline__ void load_row(const float* __restrict__ row, int E, float (&x)[NV]) {
  const int lane = lane_id();
  const float* rl = row + lane;
  if (E == 64 * NV) {  // every register full (wave-uniform): unpredicated loads
#pragma unroll
    for (int i = 0; i < NV; ++i) x[i] = __builtin_nontemporal_load(rl + 64 * i);
  } else {
#pragma unroll
    for (int i = 0; i < NV; ++i)
      x[i] = lane + 64 * i < E ? __builtin_nontemporal_load(rl + 64 * i) : __builtin_nanf("");
  }
}

// Selects the top-k experts of one token from its row x (as load_row leaves it; with
// GROUPED the logits outside the kept groups are replaced by NaN in place).  With OUT,
// writes topk weights/ids for ranks 0..k-1; always calls on_pick(rank, expert) once per
// rank, on the lane that owns it.  row is re-read only by the exact path.
template <int NV, bool GROUPED, bool OUT, class OnPick>
__device__ void select_from_row(float (&x)[NV], const float* __restrict__ row, int E, int k,
                                int score, int renorm, const GroupSel& gs,
                                uint64_t* __restrict__ cand, float* __restrict__ w_out,
                                int32_t* __restrict__ id_out, OnPick on_pick) {
  const int lane = lane_id();
  const bool softmax = score == 0;
  uint64_t keep = ~0ull;
  double m_all = 0.0, den_all = 1.0;
  if constexpr (GROUPED) {
    float lm = x[0];
#pragma unroll
    for (int i = 1; i < NV; ++i) lm = fmaxf(lm, x[i]);
    m_all = (double)wave_max_f32(lm);
    if (OUT && softmax && !renorm) den_all = full_softmax_denominator<NV>(x, m_all);
    keep = group_keep_mask<NV>(x, E, softmax, m_all, gs);
    const float ginv = 1.0f / (float)gs.size;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !((keep >> group_of(e, gs.size, ginv)) & 1ull)) x[i] = __builtin_nanf("");
    }
  }
  if (k <= 64) {
    float lm = x[0];
#pragma unroll
    for (int i = 1; i < NV; ++i) lm = fmaxf(lm, x[i]);
    // threshold: k-th largest of the G lane-group maxima (as order-preserving keys, 0 = empty)
    const uint32_t lk = lm == lm ? logit_key(lm) : 0u;
    int G = 2;
    while (G < 2 * k && G < 64) G <<= 1;
    uint32_t top, tk;  // the largest eligible key, the threshold key
    switch (64 / G) {  // wave-uniform: one straight-line network per group width
      case 32: group_threshold<32>(lk, k, top, tk); break;
      case 16: group_threshold<16>(lk, k, top, tk); break;
      case 8: group_threshold<8>(lk, k, top, tk); break;
      case 4: group_threshold<4>(lk, k, top, tk); break;
      case 2: group_threshold<2>(lk, k, top, tk); break;
      default: group_threshold<1>(lk, k, top, tk); break;
    }
    const float tau = tk == 0u ? -__builtin_inff() : key_logit(tk);
    // compaction of the logits >= tau: a ballot per register gives each lane its slot
    int c = 0;  // wave-uniform
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const bool p = x[i] >= tau;
      const uint64_t mask = __ballot(p);
      if (mask) {
        const int pos = c + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                           __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
        if (p && pos < kMaxCand) cand[pos] = pick_key(logit_key(x[i]), lane + 64 * i);
        c += __popcll(mask);
      }
    }
    if (c <= kMaxCand) {
      wave_lds_sync();
      const uint64_t v0 = lane < c ? cand[lane] : 0ull;
      const uint64_t v1 = lane + 64 < c ? cand[lane + 64] : 0ull;
      // rank = number of larger candidates (broadcast reads); pick keys are distinct
      int r0 = 0, r1 = 0;
      if (c <= 64) {
        for (int i = 0; i < c; ++i) r0 += cand[i] > v0;
      } else {
        for (int i = 0; i < c; ++i) {
          const uint64_t o = cand[i];
          r0 += o > v0;
          r1 += o > v1;
        }
      }
      wave_lds_sync();  // the candidate buffer is reused by the next token
      const bool in0 = lane < c && r0 < k, in1 = lane + 64 < c && r1 < k;
      if constexpr (OUT) {
        // full softmax of a group-limited selection: shift and denominator of the whole row
        const double m = (GROUPED && softmax && !renorm) ? m_all : (double)key_logit(top);
        const double sc0 = in0 ? score_of((double)key_logit(pick_logit_key(v0)), m, softmax) : 0.0;
        const double sc1 = in1 ? score_of((double)key_logit(pick_logit_key(v1)), m, softmax) : 0.0;
        double denom = 1.0;
        if (renorm) denom = wave_sum_f64(sc0 + sc1);
        else if (softmax) denom = GROUPED ? den_all : full_softmax_denominator<NV>(x, m);
        if (in0) {
          w_out[r0] = (float)(sc0 / denom);
          id_out[r0] = pick_expert(v0);
        }
        if (in1) {
          w_out[r1] = (float)(sc1 / denom);
          id_out[r1] = pick_expert(v1);
        }
      }
      if (in0) on_pick(r0, pick_expert(v0));
      if (in1) on_pick(r1, pick_expert(v1));
      return;
    }
    wave_lds_sync();
  }
  select_token_exact<NV, GROUPED, OUT>(row, E, k, softmax, renorm, keep, gs.size, m_all, w_out,
                                       id_out, on_pick);
}

// Loads the token's row and selects (see select_from_row).  Without GROUPED and with
// k > 64 the row goes straight to the exact path, which reads it itself.
template <int NV, bool GROUPED, bool OUT, class OnPick>
__device__ void select_token(const float* __restrict__ row, int E, int k, int score, int renorm,
                             const GroupSel& gs, uint64_t* __restrict__ cand,
                             float* __restrict__ w_out, int32_t* __restrict__ id_out,
                             OnPick on_pick) {
  if (!GROUPED && k > 64) {
    select_token_exact<NV, false, OUT>(row, E, k, score == 0, renorm, ~0ull, 1, 0.0, w_out,
                                       id_out, on_pick);
    return;
  }
  float x[NV];
  load_row<NV>(row, E, x);
  select_from_row<NV, GROUPED, OUT>(x, row, E, k, score, renorm, gs, cand, w_out, id_out,
                                    on_pick);
}

}  // namespace moe
