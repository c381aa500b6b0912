// Elementwise and per-expert steps of the backward of rank-r experts (each
// matrix W[in, out] = U[in, r] diag(s) V[out, r]^T, dormouse "TSCT low-rank
// experts" card). The products between them run on the backward GEMM
// (gemm_bwd.hip); these kernels scale by s, round to bf16 where a product
// takes the result as an operand, and reduce the s gradients.
//
//   scale_round: out[row, c] = bf16(in[row, c] * s[e(row), c % r]) for the
//     dispatched rows, e(row) the expert whose rows [offsets[e],
//     offsets[e+1]) hold row; up to two (in, s, out) jobs per launch.
//   swiglu_h:    h[row, f] = bf16(SiLU(a) * b) from the recomputed a, b.
//   ds_sum:      ds[e, i] = sum over the expert's rows, in row order, of
//     p[row, i] * q[row, i]; up to three jobs per launch, one workgroup per
//     (expert, job); nothing is accumulated with atomics.

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

// The expert whose row range holds `row` (offsets ascending, E + 1 entries).
__device__ __forceinline__ int expert_of_row(const int32_t* offsets, int E, int row) {
  int lo = 0, hi = E;   // offsets[lo] <= row < offsets[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= row) lo = mid;
    else hi = mid;
  }
  return lo;
}

__global__ void __launch_bounds__(256) scale_round_kernel(LowRankScaleJobs J) {
  const int64_t R = *J.rows;
  const int r = J.r;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // one element
  const int job = blockIdx.y;
  if (job >= J.n) return;
  const LowRankScaleJob& jb = J.job[job];
  const int64_t row = i / r;
  const int c = (int)(i - row * r);
  if (row >= R) return;
  const int e = expert_of_row(J.offsets, J.E, (int)row);
  const float s = bf16_to_f32(jb.s[(int64_t)e * r + c]);
  jb.out[row * jb.ldo + c] = f32_to_bf16(jb.in[row * jb.ldi + c] * s);
}

__global__ void __launch_bounds__(256) swiglu_h_kernel(const float* ab, bf16_t* h,
                                                       const int32_t* rows, int F) {
  const int64_t R = *rows;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = i / F;
  const int f = (int)(i - row * F);
  if (row >= R) return;
  const float a = ab[row * 2 * F + f], b = ab[row * 2 * F + F + f];
  h[row * F + f] = f32_to_bf16(silu_f32(a) * b);
}

// One workgroup per (expert, job): 256 threads = 4 row groups x 64 columns;
// row group w sums rows w, w + 4, ... of the expert in order, then the four
// partials are added in group order.
__global__ void __launch_bounds__(256) ds_sum_kernel(LowRankDsJobs J) {
  __shared__ float part[4][64];
  const int e = blockIdx.x, job = blockIdx.y;
  if (job >= J.n) return;
  const LowRankDsJob& jb = J.job[job];
  const int c = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = J.r;
  const int r0 = J.offsets[e], r1 = J.offsets[e + 1];
  float acc = 0.f;
  if (c < r)
    for (int row = r0 + w; row < r1; row += 4)
      acc += jb.p[(int64_t)row * jb.ldp + c] * jb.q[(int64_t)row * jb.ldq + c];
  part[w][c] = acc;
  __syncthreads();
  if (w == 0 && c < r)
    jb.ds[(int64_t)e * r + c] = ((part[0][c] + part[1][c]) + part[2][c]) + part[3][c];
}

}  // namespace

hipError_t launch_scale_round(const LowRankScaleJobs& J, int64_t R_max, hipStream_t s) {
  if (J.n < 1 || J.n > 2 || J.r < 1 || J.r > 64) return hipErrorInvalidValue;
  const int64_t n = R_max * J.r;
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256), (unsigned)J.n);
  hipLaunchKernelGGL(scale_round_kernel, grid, dim3(256), 0, s, J);
  return hipGetLastError();
}

hipError_t launch_swiglu_h(const float* ab, bf16_t* h, const int32_t* rows, int64_t R_max, int F,
                           hipStream_t s) {
  const int64_t n = R_max * F;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(swiglu_h_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, ab, h,
                     rows, F);
  return hipGetLastError();
}

hipError_t launch_ds_sum(const LowRankDsJobs& J, hipStream_t s) {
  if (J.n < 1 || J.n > 3 || J.r < 1 || J.r > 64 || J.E < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(ds_sum_kernel, dim3((unsigned)J.E, (unsigned)J.n), dim3(256), 0, s, J);
  return hipGetLastError();
}

}  // namespace moe
