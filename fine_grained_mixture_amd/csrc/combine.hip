// Gate-weighted combine of the MoE layer on gfx950.
//
// y[t] = shared[t] + sum over token t's kept slots j (ascending j) of
// gate[t, j] * y_routed[row_of_slot[t, j]]: the shared experts always run with
// weight one and the routed ones are weighted by their gates (Moonfrost MoE
// card: a token passes through its top-3 routed experts plus the shared one).
// Summation is in float32 in that fixed order, so the output is bitwise
// reproducible. One workgroup per token row, 16-byte lane accesses.

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kMaxK = 16;

template <bool LOWP_BF16>
__global__ void __launch_bounds__(256) combine_kernel(CombineArgs a) {
  const int d4 = a.d >> 2;
  const int k = a.k;
  for (int64_t t = blockIdx.x; t < a.T; t += gridDim.x) {
    int rows[kMaxK];
    float gates[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      rows[j] = -1;
      gates[j] = 0.f;
      if (j < k) {
        rows[j] = a.row_of_slot[t * k + j];
        gates[j] = a.topk_gate[t * k + j];
      }
    }
    for (int c = threadIdx.x; c < d4; c += blockDim.x) {
      floatx4 acc = a.y_shared
                        ? reinterpret_cast<const floatx4*>(a.y_shared + t * a.d)[c]
                        : floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < kMaxK; ++j) {
        if (j < k && rows[j] >= 0) {
          const floatx4 v = reinterpret_cast<const floatx4*>(a.y_routed + (int64_t)rows[j] * a.d)[c];
          acc[0] = fmaf(gates[j], v[0], acc[0]);
          acc[1] = fmaf(gates[j], v[1], acc[1]);
          acc[2] = fmaf(gates[j], v[2], acc[2]);
          acc[3] = fmaf(gates[j], v[3], acc[3]);
        }
      }
      reinterpret_cast<floatx4*>(a.y + t * a.d)[c] = acc;
      if (a.y_lowp) {
        if (LOWP_BF16) {
          u32x2 p;
          p[0] = (uint32_t)f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16);
          p[1] = (uint32_t)f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16);
          reinterpret_cast<u32x2*>(static_cast<bf16_t*>(a.y_lowp) + t * a.d)[c] = p;
        } else {
          reinterpret_cast<floatx4*>(static_cast<float*>(a.y_lowp) + t * a.d)[c] = acc;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int64_t grid = a.T < 65536 ? a.T : 65536;
  if (a.dtype == MOE_BF16)
    hipLaunchKernelGGL(combine_kernel<true>, dim3((unsigned)grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
