// Gate-weighted combine of the MoE layer on gfx950.
//
// y[t] = shared[t] + sum over token t's kept slots j (ascending j) of
// gate[t, j] * y_routed[row_of_slot[t, j]]: the shared experts always run with
// weight one and the routed ones are weighted by their gates (Moonfrost MoE
// card: a token passes through its top-3 routed experts plus the shared one).
// Summation is in float32 in that fixed order, so the output is bitwise
// reproducible.
//
// One wave per token, grid-stride over tokens. Lane j < k holds the token's
// slot j (row, gate), broadcast with readlane. A dropped slot loads row 0
// (never used) rather than branching around its load, so all of a token's row
// loads of a column pass are issued before the first FMA waits for them; its
// FMAs are skipped. The next token's slot pairs are requested while the
// current token is combined. Columns go in passes of Q 16-byte pieces per lane
// (256 Q floats per pass).

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kWaves = 4;

template <bool LOWP_BF16, int KMAX, int Q>
__global__ void __launch_bounds__(256) combine_kernel(CombineArgs a) {
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int d4 = a.d >> 2;
  const int k = a.k;
  const int64_t nw = (int64_t)gridDim.x * kWaves;
  const floatx4* yr = reinterpret_cast<const floatx4*>(a.y_routed);

  int nxt_row = -1;
  float nxt_gate = 0.f;
  auto load_slots = [&](int64_t t) {
    nxt_row = -1;
    nxt_gate = 0.f;
    if (t < a.T && lane < k) {
      nxt_row = a.row_of_slot[t * k + lane];
      nxt_gate = a.topk_gate[t * k + lane];
    }
  };
  int64_t t = (int64_t)blockIdx.x * kWaves + wave;
  load_slots(t);
  for (; t < a.T; t += nw) {
    // this token's slots (a dropped slot has row -1)
    const int my_row = nxt_row;
    const float my_gate = nxt_gate;
    load_slots(t + nw);
    int row[KMAX];
    bool kept[KMAX];
    float gate[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      const int r = __builtin_amdgcn_readlane(my_row, j);
      kept[j] = j < k && r >= 0;
      row[j] = max(r, 0);
      gate[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_gate), j));
    }
    const floatx4* ys = a.y_shared ? reinterpret_cast<const floatx4*>(a.y_shared + t * a.d) : nullptr;
    floatx4* yo = reinterpret_cast<floatx4*>(a.y + t * a.d);
    for (int c0 = 0; c0 < d4; c0 += 64 * Q) {
      floatx4 acc[Q], v[KMAX][Q];
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const int c = min(c0 + lane + 64 * q, d4 - 1);
        acc[q] = ys ? ys[c] : floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
          if (j < k) v[j][q] = yr[(int64_t)row[j] * d4 + c];
      }
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (kept[j]) {
#pragma unroll
          for (int q = 0; q < Q; ++q) {
            acc[q][0] = fmaf(gate[j], v[j][q][0], acc[q][0]);
            acc[q][1] = fmaf(gate[j], v[j][q][1], acc[q][1]);
            acc[q][2] = fmaf(gate[j], v[j][q][2], acc[q][2]);
            acc[q][3] = fmaf(gate[j], v[j][q][3], acc[q][3]);
          }
        }
      }
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const int c = c0 + lane + 64 * q;
        if (c >= d4) continue;
        yo[c] = acc[q];
        if (a.y_lowp) {
          if (LOWP_BF16) {
            u32x2 p;
            p[0] = (uint32_t)f32_to_bf16(acc[q][0]) | ((uint32_t)f32_to_bf16(acc[q][1]) << 16);
            p[1] = (uint32_t)f32_to_bf16(acc[q][2]) | ((uint32_t)f32_to_bf16(acc[q][3]) << 16);
            reinterpret_cast<u32x2*>(static_cast<bf16_t*>(a.y_lowp) + t * a.d)[c] = p;
          } else {
            reinterpret_cast<floatx4*>(static_cast<float*>(a.y_lowp) + t * a.d)[c] = acc[q];
          }
        }
      }
    }
  }
}

template <bool LOWP_BF16, int KMAX>
hipError_t launch_q(const CombineArgs& a, unsigned grid, hipStream_t s) {
  // 16-byte pieces per lane and pass: enough for d <= 256 Q, at most 4 (2 when
  // up to 16 rows are held)
  const int d4 = a.d >> 2;
  if constexpr (KMAX > 8) {
    if (d4 <= 64)
      hipLaunchKernelGGL((combine_kernel<LOWP_BF16, KMAX, 1>), dim3(grid), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((combine_kernel<LOWP_BF16, KMAX, 2>), dim3(grid), dim3(256), 0, s, a);
  } else {
    if (d4 <= 64)
      hipLaunchKernelGGL((combine_kernel<LOWP_BF16, KMAX, 1>), dim3(grid), dim3(256), 0, s, a);
    else if (d4 <= 128)
      hipLaunchKernelGGL((combine_kernel<LOWP_BF16, KMAX, 2>), dim3(grid), dim3(256), 0, s, a);
    else if (d4 <= 192)
      hipLaunchKernelGGL((combine_kernel<LOWP_BF16, KMAX, 3>), dim3(grid), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((combine_kernel<LOWP_BF16, KMAX, 4>), dim3(grid), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

template <bool LOWP_BF16>
hipError_t launch_k(const CombineArgs& a, unsigned grid, hipStream_t s) {
  if (a.k <= 2) return launch_q<LOWP_BF16, 2>(a, grid, s);
  if (a.k <= 4) return launch_q<LOWP_BF16, 4>(a, grid, s);
  if (a.k <= 8) return launch_q<LOWP_BF16, 8>(a, grid, s);
  return launch_q<LOWP_BF16, 16>(a, grid, s);
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.k < 1 || a.k > 16 || a.d % 4) return hipErrorInvalidValue;
  // one wave per token, up to 8 workgroups of 4 waves per CU over 256 CUs
  const int64_t waves = a.T < 8192 ? a.T : 8192;
  const unsigned grid = (unsigned)((waves + kWaves - 1) / kWaves);
  return a.dtype == MOE_BF16 ? launch_k<true>(a, grid, s) : launch_k<false>(a, grid, s);
}

}  // namespace moe
