// Products of the layer backward for float32 layers (MOE_F32: activations,
// weights and every product operand in float32, no rounding points): the same
// work items as gemm_bwd_kernel (BwdGemm descriptors: 256 x 128 output tiles of
// row plans, ragged or chunked k ranges, k segments over two weights, column
// splits over two outputs) on the fp32 FMA units.
//
// A work item's 256 rows run as four 64-row sub-tiles in turn, stopping at
// the item's last row (an expert's few rows then cost one sub-tile): 256
// threads, each owning 4 rows x 8 columns of the sub-tile; K-steps of 16
// staged through LDS as [k][row] and [k][col], so that a thread's 4 + 8
// operands of one k are contiguous reads. Every output is summed over k in
// ascending order by one thread: the result does not depend on scheduling.
// Lanes whose k or row lies outside the work item read zero.

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kBM = kGemmBigBM;   // 256
constexpr int kBN = 128;
constexpr int kBK = 16;
constexpr int kSub = 64;                      // rows per sub-tile
constexpr int kThreads = 256;

__device__ __forceinline__ float sigmoid_prec(float z) { return 1.0f / (1.0f + expf(-z)); }

template <bool A_KC, bool B_KC, int EPI>
__global__ void __launch_bounds__(kThreads) gemm_bwd_f32_kernel(BwdLaunch L) {
  __shared__ float As[kBK][kSub + 4];
  __shared__ float Bs[kBK][kBN + 4];

  const int bid = blockIdx.x;
  int pi = 0;
#pragma unroll
  for (int i = 1; i < kBwdMaxProblems; ++i)
    if (i < L.n && bid >= L.start[i]) pi = i;
  const BwdGemm& P = L.p[pi];
  const int local = bid - L.start[pi];

  int s, c = 0, r0, r_end, kb, ke;
  const int nt = local % P.n_tiles_n;
  const int mt = local / P.n_tiles_n;
  const int n0 = nt * kBN;
  if (P.plan) {
    if (mt >= P.plan[0]) return;
    s = P.plan[1 + 2 * mt];
    r0 = P.plan[2 + 2 * mt];
    r_end = min(P.m_off[s + 1], r0 + kBM);
    kb = 0;
    ke = P.K;
  } else {
    const int mtile = mt % P.n_tiles_m, rest = mt / P.n_tiles_m;
    c = rest % P.n_chunks;
    s = rest / P.n_chunks;
    if (s >= P.G) return;
    r0 = mtile * kBM;
    r_end = min(P.M, r0 + kBM);
    if (P.k_off) {
      kb = P.k_off[s];
      ke = P.k_off[s + 1];
    } else {
      kb = c * P.k_chunk;
      ke = min(P.K, kb + P.k_chunk);
    }
  }
  if (r0 >= r_end) return;
  const int N = P.N;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const float* A = static_cast<const float*>(P.A) + s * P.a_group;

  for (int rs = r0; rs < r_end; rs += kSub) {   // the 64-row sub-tiles
    float acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;

    // k-contiguous A: this thread's row of the sub-tile (gathered when a_gather)
    int64_t arow = -1;
    if (A_KC) {
      const int r = rs + (tid >> 2);
      if (r < r_end) arow = P.a_gather ? P.a_gather[r] : r;
    }
    for (int k0 = kb; k0 < ke; k0 += kBK) {
      if (A_KC) {
        // thread -> sub-tile row tid / 4, 4 consecutive k
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int kk = (tid & 3) * 4 + q, k = k0 + kk;
          As[kk][tid >> 2] = (arow >= 0 && k < ke) ? A[arow * P.lda + k] : 0.f;
        }
      } else {
        // A stored [k][m]: thread -> k-row tid / 16, 4 consecutive m
        const int kk = tid >> 4, k = k0 + kk;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int mm = (tid & 15) * 4 + q, m = rs + mm;
          As[kk][mm] = (k < ke && m < r_end) ? A[(int64_t)k * P.lda + m] : 0.f;
        }
      }
      if (B_KC) {
        // B stored [n][k] (in segments of k_seg over B0, B1): thread -> column
        // tid / 2, k half tid % 2
        const int nn = tid >> 1, n = n0 + nn;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int kk = (tid & 1) * 8 + q, k = k0 + kk;
          float v = 0.f;
          if (k < ke && n < N) {
            const int seg = P.k_seg ? k / P.k_seg : 0;
            const float* base = static_cast<const float*>((seg & 1) ? P.B1 : P.B0) +
                                s * P.b_group + (int64_t)(seg >> 1) * P.b_seg;
            v = base[(int64_t)n * P.ldb + (k - seg * P.k_seg)];
          }
          Bs[kk][nn] = v;
        }
      } else {
        // B stored [k][n]: thread -> k-row tid / 16, 8 consecutive n
        const int kk = tid >> 4, k = k0 + kk;
        const float* B = static_cast<const float*>(P.B0) + s * P.b_group;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int nn = (tid & 15) * 8 + q, n = n0 + nn;
          Bs[kk][nn] = (k < ke && n < N) ? B[(int64_t)k * P.ldb + n] : 0.f;
        }
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < kBK; ++kk) {
        float a[4], b[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
        for (int j = 0; j < 8; ++j) b[j] = Bs[kk][tx * 8 + j];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
      }
      __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = rs + ty * 4 + i;
      if (row >= r_end) continue;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int col = n0 + tx * 8 + j;
        if (col >= N) continue;
        if (EPI == kBwdStoreF32) {
          float* cb = (col < P.c_split ? P.C0 + col : P.C1 + (col - P.c_split)) +
                      s * P.c_group + (int64_t)c * P.c_chunk;
          cb[(int64_t)row * P.ldc] = acc[i][j];
        } else {
          // dh in acc; the gate and up products a, b of the same element
          const float* ab = P.ab + s * P.ab_group + (int64_t)row * P.ab_ld + col;
          const float a = ab[0], b = ab[P.half];
          const float sg = sigmoid_prec(a);
          const float v = acc[i][j];
          float* o = P.C0 + s * P.c_group + (int64_t)row * P.ldc + col;
          o[0] = v * b * (sg * (1.0f + a * (1.0f - sg)));
          o[P.half] = v * (a * sg);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_bwd_f32(BwdLaunch& L, bool a_kc, bool b_kc, int epi, hipStream_t s) {
  if (L.n < 1 || L.n > kBwdMaxProblems) return hipErrorInvalidValue;
  int64_t total = 0;
  for (int i = 0; i < L.n; ++i) {
    const BwdGemm& P = L.p[i];
    if (P.N < 1 || (!P.plan && (P.n_tiles_m < 1 || P.n_chunks < 1)) || P.C2)
      return hipErrorInvalidValue;
    if (b_kc && P.k_seg < 0) return hipErrorInvalidValue;
    L.start[i] = (int32_t)total;
    total += bwd_tiles(P);
  }
  L.start[L.n] = (int32_t)total;
  if (total == 0) return hipSuccess;
  if (total >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)total), block(kThreads);
  if (epi == kBwdSwiGLU) {
    if (!a_kc || !b_kc) return hipErrorInvalidValue;
    for (int i = 0; i < L.n; ++i)
      if (!L.p[i].ab || L.p[i].half < L.p[i].N) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_bwd_f32_kernel<true, true, kBwdSwiGLU>), grid, block, 0, s, L);
  } else if (a_kc && b_kc) {
    hipLaunchKernelGGL((gemm_bwd_f32_kernel<true, true, kBwdStoreF32>), grid, block, 0, s, L);
  } else if (!a_kc && !b_kc) {
    hipLaunchKernelGGL((gemm_bwd_f32_kernel<false, false, kBwdStoreF32>), grid, block, 0, s, L);
  } else if (a_kc && !b_kc) {
    hipLaunchKernelGGL((gemm_bwd_f32_kernel<true, false, kBwdStoreF32>), grid, block, 0, s, L);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
