// Elementwise and per-expert steps of the backward of rank-r experts (each
// matrix W[in, out] = U[in, r] diag(s) V[out, r]^T, dormouse "TSCT low-rank
// experts" card). The products between them run on the backward GEMM
// (gemm_bwd.hip), whose epilogue also writes the s-scaled bf16 copies; these
// kernels form h and reduce the s gradients.
//
//   swiglu_h:    h[row, f] = bf16(SiLU(a) * b) from the recomputed a, b.
//   ds_sum:      ds[e, i] = sum over the expert's rows, in row order, of
//     p[row, i] * q[row, i]; up to three jobs per launch, one workgroup per
//     (expert, job); nothing is accumulated with atomics.

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

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
