// Fused router for the fine-grained layers with few routed experts (E <= 64:
// 24 on the Quartz model card, 32 on the Moonfrost MoE card, 48 on the
// Sutra-1.3B card), bf16 inputs.
//
// One workgroup per 16 tokens:
//   1. logits[16, E] = x[16, d] W_r[d, E] + logit_bias with
//      v_mfma_f32_16x16x32_bf16: the token rows are the A operand loaded
//      straight from memory (8 consecutive k per lane); W_r is copied into LDS
//      in 256-row chunks in its own [k][e] layout and the B operand is read
//      with ds_read_b64_tr_b16 (lane group of 16: source lane s addresses row
//      k0 + s/4, experts e0 + 4 (s%4); output lane j gets 4 consecutive k of
//      expert e0 + j); the four waves take the k32 steps round-robin and
//      their partial sums are added in a fixed order;
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

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef short shortx8 __attribute__((ext_vector_type(8)));

template <int EP, int KMAX, bool VEC>
__global__ void __launch_bounds__(256) route_small_kernel(RouteSmallArgs a) {
  constexpr int NS = EP / 16;
  __shared__ __attribute__((aligned(16))) bf16_t Ws[kKC * EP];   // [k][e], row EP
  __shared__ float s_part[4][kTB][EP + 1];
  __shared__ float s_log[kTB][EP + 1];
  __shared__ float s_p[kTB][EP + 1];
  __shared__ int s_cnt[EP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, d = a.d, k = a.k;
  const int64_t t0 = (int64_t)blockIdx.x * kTB;
  const bf16_t* x = static_cast<const bf16_t*>(a.x);
  const bf16_t* W = static_cast<const bf16_t*>(a.w_router);

  if (tid < EP) s_cnt[tid] = 0;
  // padded expert columns: their logits are never read, but keep them finite
  if (EP > E)
    for (int i = tid; i < kKC * (EP - E); i += 256) Ws[(i / (EP - E)) * EP + E + i % (EP - E)] = 0;

  floatx4 acc[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int64_t arow = min(t0 + (lane & 15), a.T - 1);
  const bf16_t* xr = x + arow * d + 8 * (lane >> 4);

  for (int kc0 = 0; kc0 < d; kc0 += kKC) {
    const int kcn = min(kKC, d - kc0);
    // this wave's token-row fragments of the chunk (k32 steps wave, wave + 4),
    // requested before the weight staging so their latency overlaps it
    bf16x8 av[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int ks = wave + 4 * q;
      if (ks < kcn / 32) av[q] = *reinterpret_cast<const bf16x8*>(xr + kc0 + ks * 32);
    }
    __syncthreads();
    const bf16_t* wsrc = W + (int64_t)kc0 * E;
    if (VEC) {
      // E % 8 == 0: 16-byte pieces, E / 8 per row
      const int cpr = E >> 3;
      for (int i = tid; i < kcn * cpr; i += 256) {
        const int kk = i / cpr, c = i - kk * cpr;
        *reinterpret_cast<u32x4*>(&Ws[kk * EP + 8 * c]) =
            *reinterpret_cast<const u32x4*>(wsrc + (int64_t)kk * E + 8 * c);
      }
    } else {
      for (int i = tid; i < kcn * E; i += 256) {
        const int kk = i / E, e = i - kk * E;
        Ws[kk * EP + e] = wsrc[i];
      }
    }
    __syncthreads();
    const int g16 = lane >> 4, s16 = lane & 15;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int ks = wave + 4 * q;
      if (ks >= kcn / 32) break;
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        // B operand: 8 consecutive k (32 ks + 8 g16 ..) of expert 16 j + s16
        const bf16_t* p0 = &Ws[(ks * 32 + 8 * g16 + (s16 >> 2)) * EP + 16 * j + 4 * (s16 & 3)];
        const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) shortx4*)p0);
        const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) shortx4*)(p0 + 4 * EP));
        const shortx8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[q], __builtin_bit_cast(bf16x8, v),
                                                         acc[j], 0, 0, 0);
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
      if (j < k && valid) {
        a.topk_idx[t * k + j] = ki[j];
        a.topk_gate[t * k + j] = gates[j];
        atomicAdd(&s_cnt[ki[j]], 1);   // integer counts: order-independent
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
    float ps = 0.f;
#pragma unroll
    for (int t = 0; t < kTB; ++t) ps += s_p[t][e];
    a.blk_counts[(int64_t)blockIdx.x * E + e] = s_cnt[e];
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
#define MOE_RS(EPV, KM)                                                                      \
  do {                                                                                       \
    if (a.E % 8 == 0)                                                                        \
      hipLaunchKernelGGL((route_small_kernel<EPV, KM, true>), dim3((unsigned)nblk), dim3(256), 0, \
                         s, a);                                                              \
    else                                                                                     \
      hipLaunchKernelGGL((route_small_kernel<EPV, KM, false>), dim3((unsigned)nblk), dim3(256), \
                         0, s, a);                                                           \
  } while (0)
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
