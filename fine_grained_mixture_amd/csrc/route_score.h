// Per-token scoring of the routers for many experts (topk_kernel, and the
// fused router-and-top-k kernel): one wave per token, lane l holding the keys
// of experts l, l + 64, ... (EPL of them, -inf past E).
//
// The top k + 1 by key (larger key first, equal keys to the lower expert id:
// the router top-k of the Quartz model card Architecture table), the gates
// (softmax probabilities, renormalised over the selected experts or not; or
// the selected sigmoid scores over their sum, the Sutra-1.3B "48 + 1 experts"
// card), each expert's routing probability added to psum (the P of the
// research page's balancing statistic), the selected experts counted in the
// block's LDS histogram, and the margin between the k-th and (k+1)-th keys.
// Lane l's best two (key, expert) pairs are cached; each of the k + 1 rounds
// takes the wave-wide maximum key; a single lane holding it wins (a ballot),
// several lanes holding it fall back to the lowest expert id among them. The
// winner moves its second pair up; a lane that wins twice re-scans its
// experts ranked after the last one it gave away.
#pragma once

#include <float.h>
#include <limits.h>
#include <math.h>

#include "moe_device.h"

namespace moe {
namespace {

__device__ __forceinline__ int wave_min_i32(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = min(v, __shfl_xor(v, m, 64));
  return v;
}

// Best two of the lane's experts ranked after (lk, lm) in the selection
// order: key < lk, or key == lk with a larger index m (a larger expert id).
template <int EPL>
__device__ __forceinline__ void lane_top2(const float (&key)[EPL], float lk, int lm, float& k1,
                                          int& m1, float& k2, int& m2) {
  k1 = -INFINITY;
  k2 = -INFINITY;
  m1 = 0;
  m2 = 0;
#pragma unroll
  for (int m = 0; m < EPL; ++m) {
    const bool elig = key[m] < lk || (key[m] == lk && m > lm);
    const float v = elig ? key[m] : -INFINITY;
    const bool c1 = v > k1, c2 = v > k2;
    k2 = c1 ? k1 : (c2 ? v : k2);
    m2 = c1 ? m1 : (c2 ? m : m2);
    k1 = c1 ? v : k1;
    m1 = c1 ? m : m1;
  }
}

// key: the selection keys (softmax: the logits; sigmoid: sigmoid(l) + bias);
// sc: the sigmoid scores (SIG only). key is overwritten. Lanes j < k return
// the j-th selected expert and its gate in my_id, my_gate; mg is the margin.
template <int EPL, int R, bool SIG>
__device__ __forceinline__ void score_token(float (&key)[EPL], float (&sc)[EPL], int E, int k,
                                            int rounds, int renorm, float (&psum)[EPL],
                                            int* s_cnt, int& my_id_out, float& my_gate_out,
                                            float& mg_out) {
  const int lane = lane_id();
  float k1, k2;
  int m1, m2;
  lane_top2<EPL>(key, INFINITY, -1, k1, m1, k2, m2);
  int cached = 2;          // pairs of the lane still exact
  float lk = INFINITY;     // the lane's last pair given away
  int lm = -1;

  // k + 1 rounds of the wave-wide maximum
  int sel_id[R];
  float sel_key[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    sel_id[r] = 0;
    sel_key[r] = 0.f;
    if (r < rounds) {
      const float mx = wave_max(k1);
      const uint64_t tied = __ballot(k1 == mx);
      int wl;
      if (__popcll(tied) == 1) {
        wl = __ffsll((unsigned long long)tied) - 1;
      } else {   // equal keys in several lanes: the lowest expert id
        const int cand = k1 == mx ? lane + 64 * m1 : INT_MAX;
        wl = __builtin_amdgcn_readfirstlane(wave_min_i32(cand)) & 63;
      }
      const int wm = __builtin_amdgcn_readlane(m1, wl);
      sel_id[r] = wl + 64 * wm;
      sel_key[r] = mx;
      if (lane == wl) {
        lk = k1;
        lm = m1;
        k1 = k2;
        m1 = m2;
        k2 = -INFINITY;
        --cached;
      }
      if (r + 1 < rounds && __ballot(cached == 0) != 0) {
        float n1, n2;
        int j1, j2;
        lane_top2<EPL>(key, lk, lm, n1, j1, n2, j2);
        if (cached == 0) {
          k1 = n1;
          m1 = j1;
          k2 = n2;
          m2 = j2;
          cached = 2;
        }
      }
    }
  }

  // gates and routing probabilities
  float my_gate = 0.f;
  int my_id = 0;
  if (!SIG) {
    const float mxl = sel_key[0];
    float se = 0.f;
#pragma unroll
    for (int m = 0; m < EPL; ++m) {   // the key is the logit, -inf past E
      key[m] = __expf(key[m] - mxl);
      se += key[m];
    }
    se = wave_sum(se);
    const float inv = 1.0f / se;
#pragma unroll
    for (int m = 0; m < EPL; ++m) psum[m] += key[m] * inv;
    float ssel = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float g = r < k ? __expf(sel_key[r] - mxl) : 0.f;
      ssel += g;
      if (lane == r) {
        my_id = sel_id[r];
        my_gate = g;
      }
    }
    my_gate /= renorm ? ssel : se;
  } else {
    float ss = 0.f;
#pragma unroll
    for (int m = 0; m < EPL; ++m) {
      if (lane + 64 * m >= E) sc[m] = 0.f;
      ss += sc[m];
    }
    ss = wave_sum(ss);
    const float inv = 1.0f / ss;
#pragma unroll
    for (int m = 0; m < EPL; ++m) psum[m] += sc[m] * inv;
    // sigmoid score of each winner, from the lane holding it (the key also
    // carries the selection bias, which must not reach the gates)
    float ssel = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (r < k) {
        const int id = sel_id[r];
        float mine = 0.f;
#pragma unroll
        for (int m = 0; m < EPL; ++m) mine = id == lane + 64 * m ? sc[m] : mine;
        const float g = __shfl(mine, id & 63, 64);
        ssel += g;
        if (lane == r) {
          my_id = id;
          my_gate = g;
        }
      }
    }
    my_gate /= ssel;
  }
  if (lane < k) atomicAdd(&s_cnt[my_id], 1);   // integer counts: order-independent
  float mg = INFINITY;
#pragma unroll
  for (int r = 1; r < R; ++r)
    if (r == k && k < E) mg = sel_key[r - 1] - sel_key[r];
  my_id_out = my_id;
  my_gate_out = my_gate;
  mg_out = mg;
}

}  // namespace
}  // namespace moe
