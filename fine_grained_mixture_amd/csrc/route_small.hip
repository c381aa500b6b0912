// Fused router for the fine-grained layers with few routed experts (E <= 64:
// 24 on the Quartz model card, 32 on the Moonfrost MoE card, 48 on the
// Sutra-1.3B card), bf16 inputs.
//
// One workgroup per 16 tokens:
//   1. logits[16, E] = x[16, d] W_r[d, E] + logit_bias with
//      v_mfma_f32_16x16x32_bf16: the token rows are the A operand loaded
//      straight from memory (8 consecutive k per lane); W_r is staged through
//      LDS in 256-row chunks, transposed so each lane reads 8 consecutive k of
//      one expert; the four waves take the k32 steps round-robin and their
//      partial sums are added in a fixed order;
//   2. one lane per token walks its E scores and keeps the best k+1 in a
//      register list (strictly larger keys move ahead, so equal keys keep the
//      lower expert id first), then computes gates and the routing
//      probabilities -- no cross-lane traffic;
//   3. the block's per-expert slot counts and probability sums, summed over the
//      16 tokens in order.

#include <float.h>
#include <math.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kTB = kRouteBlockSmall;   // tokens per workgroup
constexpr int kKC = 256;                // rows of W_r per LDS chunk
constexpr int kLdsW = kKC + 8;          // padded LDS row (elements)

template <int EP, int KMAX>
__global__ void __launch_bounds__(256) route_small_kernel(RouteSmallArgs a) {
  constexpr int NS = EP / 16;
  __shared__ __attribute__((aligned(16))) bf16_t Ws[EP * kLdsW];
  __shared__ float s_part[4][kTB][EP + 1];
  __shared__ float s_log[kTB][EP + 1];
  __shared__ float s_p[kTB][EP + 1];
  __shared__ int s_ids[kTB][KMAX];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, d = a.d, k = a.k;
  const int64_t t0 = (int64_t)blockIdx.x * kTB;
  const bf16_t* x = static_cast<const bf16_t*>(a.x);
  const bf16_t* W = static_cast<const bf16_t*>(a.w_router);

  // padded expert rows stay zero
  for (int i = tid; i < (EP - E) * kLdsW; i += 256) Ws[E * kLdsW + i] = 0;

  floatx4 acc[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int64_t arow = min(t0 + (lane & 15), a.T - 1);
  const bf16_t* xr = x + arow * d + 8 * (lane >> 4);

  for (int kc0 = 0; kc0 < d; kc0 += kKC) {
    const int kcn = min(kKC, d - kc0);
    __syncthreads();
    const int nel = kcn * E;
    const bf16_t* wsrc = W + (int64_t)kc0 * E;
    for (int i = tid; i < nel; i += 256) {
      const int kk = i / E;
      const int e = i - kk * E;
      Ws[e * kLdsW + kk] = wsrc[i];
    }
    __syncthreads();
    for (int ks = wave; ks < kcn / 32; ks += 4) {
      const bf16x8 av = *reinterpret_cast<const bf16x8*>(xr + kc0 + ks * 32);
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const bf16x8 bv = *reinterpret_cast<const bf16x8*>(
            &Ws[(16 * j + (lane & 15)) * kLdsW + ks * 32 + 8 * (lane >> 4)]);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[j], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < NS; ++j)
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) s_part[wave][4 * (lane >> 4) + e4][16 * j + (lane & 15)] = acc[j][e4];
  __syncthreads();
  for (int i = tid; i < kTB * EP; i += 256) {
    const int r = i / EP, c = i - (i / EP) * EP;
    float v = s_part[0][r][c] + s_part[1][r][c] + s_part[2][r][c] + s_part[3][r][c];
    if (c < E && a.logit_bias) v += a.logit_bias[c];
    s_log[r][c] = v;
  }
  __syncthreads();

  if (wave == 0 && lane < kTB) {
    const int64_t t = t0 + lane;
    const bool valid = t < a.T;
    float kv[KMAX];
    int ki[KMAX];
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
      kv[i] = -INFINITY;
      ki[i] = 0;
    }
    const bool sig = a.score == MOE_SIGMOID;
    for (int e = 0; e < E; ++e) {
      const float l = s_log[lane][e];
      float ck = sig ? 1.0f / (1.0f + __expf(-l)) + (a.select_bias ? a.select_bias[e] : 0.f) : l;
      int ci = e;
#pragma unroll
      for (int i = 0; i < KMAX; ++i) {
        const bool gt = ck > kv[i];
        const float tk = kv[i];
        const int ti = ki[i];
        kv[i] = gt ? ck : tk;
        ki[i] = gt ? ci : ti;
        ck = gt ? tk : ck;
        ci = gt ? ti : ci;
      }
    }
    float gates[KMAX];
    if (!sig) {
      const float m = kv[0];
      float se = 0.f;
      for (int e = 0; e < E; ++e) {
        const float p = __expf(s_log[lane][e] - m);
        s_p[lane][e] = p;
        se += p;
      }
      const float inv = 1.0f / se;
      for (int e = 0; e < E; ++e) s_p[lane][e] = valid ? s_p[lane][e] * inv : 0.f;
      float ssel = 0.f;
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (j < k) ssel += __expf(kv[j] - m);
      const float den = a.renorm ? ssel : se;
#pragma unroll
      for (int j = 0; j < KMAX; ++j) gates[j] = j < k ? __expf(kv[j] - m) / den : 0.f;
    } else {
      float ss = 0.f;
      for (int e = 0; e < E; ++e) {
        const float s = 1.0f / (1.0f + __expf(-s_log[lane][e]));
        s_p[lane][e] = s;
        ss += s;
      }
      const float inv = 1.0f / ss;
      for (int e = 0; e < E; ++e) s_p[lane][e] = valid ? s_p[lane][e] * inv : 0.f;
      float ssel = 0.f;
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        gates[j] = j < k ? 1.0f / (1.0f + __expf(-s_log[lane][ki[j]])) : 0.f;
        ssel += gates[j];
      }
#pragma unroll
      for (int j = 0; j < KMAX; ++j) gates[j] /= ssel;
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j < k) {
        s_ids[lane][j] = valid ? ki[j] : -1;
        if (valid) {
          a.topk_idx[t * k + j] = ki[j];
          a.topk_gate[t * k + j] = gates[j];
        }
      }
    }
    if (valid && a.topk_margin) {
      float mg = INFINITY;
#pragma unroll
      for (int j = 1; j < KMAX; ++j)
        if (j == k && k < E) mg = kv[j - 1] - kv[j];
      a.topk_margin[t] = mg;
    }
  }
  __syncthreads();

  for (int e = tid; e < E; e += 256) {
    int c = 0;
    float ps = 0.f;
    for (int t = 0; t < kTB; ++t) {
      ps += s_p[t][e];
      for (int j = 0; j < k; ++j) c += s_ids[t][j] == e;
    }
    a.blk_counts[(int64_t)blockIdx.x * E + e] = c;
    a.blk_psum[(int64_t)blockIdx.x * E + e] = ps;
  }
}

}  // namespace

hipError_t launch_route_small(const RouteSmallArgs& a, hipStream_t s) {
  const int64_t nblk = (a.T + kTB - 1) / kTB;
  if (nblk == 0) return hipSuccess;
  if (a.E > kRouteSmallMaxE || a.k + 1 > 16) return hipErrorInvalidValue;
  const int ep = (a.E + 15) / 16 * 16;
  const int k1 = a.k + 1;
#define MOE_RS(EPV, KM) \
  hipLaunchKernelGGL((route_small_kernel<EPV, KM>), dim3((unsigned)nblk), dim3(256), 0, s, a)
#define MOE_RS_K(EPV)                \
  do {                               \
    if (k1 <= 4) MOE_RS(EPV, 4);     \
    else if (k1 <= 8) MOE_RS(EPV, 8); \
    else MOE_RS(EPV, 16);            \
  } while (0)
  switch (ep) {
    case 16: MOE_RS_K(16); break;
    case 32: MOE_RS_K(32); break;
    case 48: MOE_RS_K(48); break;
    default: MOE_RS_K(64); break;
  }
#undef MOE_RS_K
#undef MOE_RS
  return hipGetLastError();
}

}  // namespace moe
