// Grouped expert GEMM for few rows per group (decode-sized batches), bf16
// operands, fp32 accumulation. With a handful of rows per expert the work is
// reading the weights once, so the layout serves bandwidth rather than MFMA:
//
//   one workgroup per (group, 64-column chunk), so each weight row is read
//   as whole 128-byte lines; its threads split the chunk into 8 column
//   groups of 8 consecutive columns (one 16-byte load per weight row) and the
//   K dimension into interleaved groups of 8-row chunks (32 groups with 256
//   threads, 64 with 512), taken two chunks at a time so that every load of
//   both is in flight before the first FMA; the weight slice B[K, 64] (and
//   B1's for the fused SwiGLU) streams through once per pass of up to ROWS
//   rows; each thread keeps ROWS x 8 partial sums (x2 for gate and up) in
//   registers, and the K-group partials are added through LDS in K-group
//   order, so the result does not depend on scheduling.
//
// Epilogues as in the large-tile kernel: fp32 rows (+ column bias), or
// bf16 h = SiLU(gate) * up.

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kCols = 64;      // output columns per workgroup (whole 128-byte lines)
constexpr int kCG = kCols / 8; // column groups of 8 columns
constexpr int kRows = 4;       // rows per pass (ROWS = 1 for single-row groups)

__device__ __forceinline__ void unpack8(const u32x4 v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(v[i] << 16);
    f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
  }
}

// THREADS / 8 K groups (256 threads: 32; 512: 64, for one or two rows per
// group, where the loads in flight per workgroup are what bounds the kernel:
// the down projection at Quartz T = 1 takes 9.8 against 12.0 us). ROWS rows
// per pass: 1 or 2 keep the fused gate/up's registers within 512 threads.
template <int EPI, bool DUAL, int THREADS, int ROWS>
__global__ void __launch_bounds__(THREADS) skinny_kernel(GemmLaunch L, int nch0, int nch1) {
  constexpr int NB = DUAL ? 2 : 1;
  constexpr int kKG = THREADS / kCG;   // K groups
  constexpr int kRows = ROWS;
  __shared__ float s_part[NB][kKG][kRows][kCols];

  int bid = blockIdx.x, prob = 0;
  if (bid >= L.p[0].G * nch0) {
    prob = 1;
    bid -= L.p[0].G * nch0;
  }
  const GemmProblem& P = L.p[prob];
  const int nch = prob ? nch1 : nch0;
  const int g = bid / nch, ch = bid - g * nch;
  int r0 = 0, r1 = P.M;
  if (P.row_off) {
    r0 = P.row_off[g];
    r1 = P.row_off[g + 1];
  }
  if (r0 >= r1) return;

  const int tid = threadIdx.x;
  const int cg = tid % kCG, kg = tid / kCG;
  const int n0 = ch * kCols;
  const int K = P.K, N = P.N;
  const bf16_t* A = static_cast<const bf16_t*>(P.A);
  const bf16_t* B0 = static_cast<const bf16_t*>(P.B0) + g * P.b_group_stride + n0 + 8 * cg;
  const bf16_t* B1 = DUAL ? static_cast<const bf16_t*>(P.B1) + g * P.b_group_stride + n0 + 8 * cg
                          : nullptr;
  const int nkc = K / 8;   // chunks of 8 K rows; K group kg takes chunks kg, kg + kKG, ...

  for (int p0 = r0; p0 < r1; p0 += kRows) {
    const int nr = min(kRows, r1 - p0);
    const bf16_t* arow[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int row = p0 + min(r, nr - 1);
      arow[r] = A + (int64_t)(P.a_rows ? P.a_rows[row] : row) * P.lda;
    }
    float acc[NB][kRows][8];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r = 0; r < kRows; ++r)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[b][r][c] = 0.f;

    // two chunks per iteration: all of their loads are issued before the FMAs
    for (int kc = kg; kc < nkc; kc += 2 * kKG) {
      const bool two = kc + kKG < nkc;
      u32x4 wv[2][NB][8], av[2][kRows];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k0 = 8 * (two ? kc + h * kKG : kc);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          wv[h][0][kk] = *reinterpret_cast<const u32x4*>(B0 + (int64_t)(k0 + kk) * P.ldb);
          if (DUAL)
            wv[h][NB - 1][kk] = *reinterpret_cast<const u32x4*>(B1 + (int64_t)(k0 + kk) * P.ldb);
        }
#pragma unroll
        for (int r = 0; r < kRows; ++r) av[h][r] = *reinterpret_cast<const u32x4*>(arow[r] + k0);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (h == 0 || two) {
#pragma unroll
          for (int kk = 0; kk < 8; ++kk) {
            float w[NB][8];
#pragma unroll
            for (int b = 0; b < NB; ++b) unpack8(wv[h][b][kk], w[b]);
#pragma unroll
            for (int r = 0; r < kRows; ++r) {
              if (r < nr) {   // wave-uniform: rows past the group's end do no work
                const uint32_t ab = av[h][r][kk >> 1];
                const float a = __uint_as_float((kk & 1) ? (ab & 0xffff0000u) : (ab << 16));
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                  for (int c = 0; c < 8; ++c) acc[b][r][c] = fmaf(a, w[b][c], acc[b][r][c]);
              }
            }
          }
        }
      }
    }
    __syncthreads();   // previous pass's partials are read
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r = 0; r < kRows; ++r)
#pragma unroll
        for (int c = 0; c < 8; c += 4)
          *reinterpret_cast<floatx4*>(&s_part[b][kg][r][8 * cg + c]) =
              floatx4{acc[b][r][c], acc[b][r][c + 1], acc[b][r][c + 2], acc[b][r][c + 3]};
    __syncthreads();

    // thread -> (row, column); K groups added in order (threads past the
    // kRows rows idle)
    const int col = tid % kCols, r = tid / kCols;
    if (r < nr) {
      float v0 = 0.f, v1 = 0.f;
#pragma unroll 8
      for (int q = 0; q < kKG; ++q) {
        v0 += s_part[0][q][r][col];
        if (DUAL) v1 += s_part[NB - 1][q][r][col];
      }
      const int row = p0 + r;
      const int64_t ccol = (int64_t)g * P.c_group_col + n0 + col;
      if (EPI == kEpiStoreF32) {
        if (P.col_bias) v0 += P.col_bias[n0 + col];
        static_cast<float*>(P.C)[(int64_t)row * P.ldc + ccol] = v0;
      } else {
        static_cast<bf16_t*>(P.C)[(int64_t)row * P.ldc + ccol] = f32_to_bf16(silu_f32(v0) * v1);
        if (P.ab) {
          float* abp = P.ab + (int64_t)row * P.ab_ld + (int64_t)g * P.ab_group_col + n0 + col;
          abp[0] = v0;
          abp[N] = v1;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_skinny(const GemmLaunch& L, int epilogue, hipStream_t s, bool wide,
                              int rows) {
  int nch[2] = {0, 0}, blocks = 0;
  for (int i = 0; i < L.n_problems; ++i) {
    const GemmProblem& P = L.p[i];
    if (P.N % kCols || P.K % 8) return hipErrorInvalidValue;
    nch[i] = P.N / kCols;
    blocks += P.G * nch[i];
  }
  if (blocks == 0) return hipSuccess;
  // 64 K groups pay off where K holds more than one 8-row chunk per group
  for (int i = 0; i < L.n_problems; ++i) wide = wide && L.p[i].K > 8 * 64;
  if (epilogue == kEpiSwiGLU && wide && rows <= 1)
    hipLaunchKernelGGL((skinny_kernel<kEpiSwiGLU, true, 512, 1>), dim3(blocks), dim3(512), 0, s,
                       L, nch[0], nch[1]);
  else if (epilogue == kEpiSwiGLU && wide && rows == 2)
    hipLaunchKernelGGL((skinny_kernel<kEpiSwiGLU, true, 512, 2>), dim3(blocks), dim3(512), 0, s,
                       L, nch[0], nch[1]);
  else if (epilogue == kEpiSwiGLU)
    hipLaunchKernelGGL((skinny_kernel<kEpiSwiGLU, true, 256, kRows>), dim3(blocks), dim3(256), 0,
                       s, L, nch[0], nch[1]);
  else if (wide)
    hipLaunchKernelGGL((skinny_kernel<kEpiStoreF32, false, 512, kRows>), dim3(blocks), dim3(512),
                       0, s, L, nch[0], nch[1]);
  else
    hipLaunchKernelGGL((skinny_kernel<kEpiStoreF32, false, 256, kRows>), dim3(blocks), dim3(256),
                       0, s, L, nch[0], nch[1]);
  return hipGetLastError();
}

}  // namespace moe
