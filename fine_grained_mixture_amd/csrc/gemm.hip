// Grouped GEMMs of the MoE layer on gfx950.
//
// The expert FFNs of the fine-grained MoE layer are many moderate GEMMs, one
// per expert, over the rows routed to it (stacked (E, hidden, ffn) expert
// tensors with the tokens grouped per expert: Moonfrost site, stacking card).
// One launch covers every group, and optionally a second problem (the shared
// experts), so the whole expert stage is two launches with no host sync.
//
// bf16 path: 128 x 128 output tiles (or 128 x (64 gate + 64 up) for the fused
// SwiGLU), 256 threads as 2 x 2 waves, K-step 64 staged through LDS with a
// register-staged double buffer, v_mfma_f32_16x16x32_bf16 with fp32
// accumulation. B arrives [K, N] with N contiguous; the MFMA B operand needs 8
// consecutive k per lane, so B is transposed on its way into LDS: each thread
// loads 2 adjacent columns from 8 consecutive rows (dword loads, coalesced
// along N) and writes two 16-byte k-runs.
//
// fp32 path: a plain LDS-tiled VALU GEMM with the same problem description.

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

struct TileRef {
  int problem, g, r0, r_end, n0;
};

// Map a workgroup index onto (problem, group, row range, first column).
__device__ __forceinline__ bool resolve_tile(const GemmLaunch& L, int bid, int bm, int bn,
                                             TileRef& t) {
  int prob = 0, local = bid;
  if (bid >= L.tiles0) {
    if (L.n_problems < 2) return false;
    prob = 1;
    local = bid - L.tiles0;
  }
  const GemmProblem& P = L.p[prob];
  const int mt = local / P.n_tiles_n;
  const int nt = local - mt * P.n_tiles_n;
  if (P.row_off) {
    const int count = P.plan[0];
    if (mt >= count) return false;
    t.g = P.plan[1 + 2 * mt];
    t.r0 = P.plan[2 + 2 * mt];
    t.r_end = min(P.row_off[t.g + 1], t.r0 + bm);
  } else {
    const int mtg = (P.M + bm - 1) / bm;
    if (mt >= mtg * P.G) return false;
    t.g = mt / mtg;
    t.r0 = (mt - t.g * mtg) * bm;
    t.r_end = min(P.M, t.r0 + bm);
  }
  t.problem = prob;
  t.n0 = nt * bn;
  return t.r0 < t.r_end;
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel
// ---------------------------------------------------------------------------
constexpr int kBM = kGemmBM;      // 128
constexpr int kBK = 64;
constexpr int kLdsK = kBK + 8;    // padded LDS row: 144 bytes, conflict-free 16-byte reads

template <int EPI, bool DUAL, bool BGUARD>
__global__ void __launch_bounds__(kThreads)
gemm_bf16_kernel(GemmLaunch L) {
  constexpr int BN = DUAL ? 64 : 128;   // columns per B matrix in one tile
  __shared__ __attribute__((aligned(16))) bf16_t As[2][kBM * kLdsK];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][128 * kLdsK];

  TileRef tile;
  if (!resolve_tile(L, blockIdx.x, kBM, BN, tile)) return;
  const GemmProblem& P = L.p[tile.problem];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int N = P.N;
  const int K = P.K;
  const int64_t ldb = P.ldb;

  // ---- A loader: 8 threads per 128-byte row chunk, rows rb + 32 i
  const bf16_t* A = static_cast<const bf16_t*>(P.A);
  const int a_c = tid & 7;
  const int a_rb = tid >> 3;
  const bf16_t* a_src[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int r = min(tile.r0 + a_rb + 32 * i, tile.r_end - 1);
    int64_t arow = P.a_rows ? P.a_rows[r] : r;
    a_src[i] = A + arow * P.lda + 8 * a_c;
  }

  // ---- B loader: unit = (column pair p, k-group q)
  const bf16_t* B0 = static_cast<const bf16_t*>(P.B0) + tile.g * P.b_group_stride;
  const bf16_t* B1 = DUAL ? static_cast<const bf16_t*>(P.B1) + tile.g * P.b_group_stride : nullptr;
  int b_p[2], b_q[2], b_row[2];
  const bf16_t* b_src[2];
#pragma unroll
  for (int v = 0; v < 2; ++v) {
    if (DUAL) {
      b_p[v] = tid & 31;
      b_q[v] = tid >> 5;
      b_src[v] = v == 0 ? B0 : B1;
      b_row[v] = v * 64 + 2 * b_p[v];
    } else {
      const int u = tid + v * kThreads;
      b_p[v] = u & 63;
      b_q[v] = u >> 6;
      b_src[v] = B0;
      b_row[v] = 2 * b_p[v];
    }
  }

  u32x4 a_reg[4];
  uint32_t b_reg[2][8];

  auto load_tiles = [&](int kt) {
    const int k0 = kt * kBK;
#pragma unroll
    for (int i = 0; i < 4; ++i) a_reg[i] = *reinterpret_cast<const u32x4*>(a_src[i] + k0);
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int col = tile.n0 + 2 * b_p[v];
      const bf16_t* src = b_src[v] + (int64_t)(k0 + 8 * b_q[v]) * ldb + col;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bf16_t* p = src + i * ldb;
        if (!BGUARD) {
          b_reg[v][i] = *reinterpret_cast<const uint32_t*>(p);
        } else {
          uint32_t lo = col < N ? p[0] : 0u;
          uint32_t hi = col + 1 < N ? p[1] : 0u;
          b_reg[v][i] = lo | (hi << 16);
        }
      }
    }
  };

  auto store_tiles = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4*>(&As[buf][(a_rb + 32 * i) * kLdsK + 8 * a_c]) = a_reg[i];
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      u32x4 lo, hi;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t x0 = b_reg[v][2 * m], x1 = b_reg[v][2 * m + 1];
        lo[m] = (x0 & 0xffffu) | (x1 << 16);
        hi[m] = (x0 >> 16) | (x1 & 0xffff0000u);
      }
      *reinterpret_cast<u32x4*>(&Bs[buf][b_row[v] * kLdsK + 8 * b_q[v]]) = lo;
      *reinterpret_cast<u32x4*>(&Bs[buf][(b_row[v] + 1) * kLdsK + 8 * b_q[v]]) = hi;
    }
  };

  // ---- wave tile
  const int wm = wave >> 1, wn = wave & 1;
  constexpr int NJ = DUAL ? 2 : 4;
  floatx4 acc[4][NJ];
  floatx4 acc2[4][DUAL ? 2 : 1];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < (DUAL ? 2 : 1); ++j) acc2[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  const int lrow = lane & 15;
  const int lk = 8 * (lane >> 4);

  auto compute = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < kBK / 32; ++kk) {
      const int koff = kk * 32 + lk;
      bf16x8 a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(&As[buf][(64 * wm + 16 * i + lrow) * kLdsK + koff]);
      if (!DUAL) {
        bf16x8 b[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          b[j] = *reinterpret_cast<const bf16x8*>(&Bs[buf][(64 * wn + 16 * j + lrow) * kLdsK + koff]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
      } else {
        bf16x8 bg[2], bu[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          bg[j] = *reinterpret_cast<const bf16x8*>(&Bs[buf][(32 * wn + 16 * j + lrow) * kLdsK + koff]);
          bu[j] = *reinterpret_cast<const bf16x8*>(&Bs[buf][(64 + 32 * wn + 16 * j + lrow) * kLdsK + koff]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bg[j], acc[i][j], 0, 0, 0);
            acc2[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bu[j], acc2[i][j], 0, 0, 0);
          }
      }
    }
  };

  const int nk = K / kBK;
  load_tiles(0);
  store_tiles(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_tiles(kt + 1);
    compute(cur);
    if (kt + 1 < nk) store_tiles(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds column (lane & 15), rows 4 * (lane >> 4) + e
  const int64_t ccol0 = tile.g * P.c_group_col;
  if (EPI == kEpiStoreF32) {
    float* C = static_cast<float*>(P.C);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int col = tile.n0 + 64 * wn + 16 * j + lrow;
      if (BGUARD && col >= N) continue;
      const float bias = P.col_bias ? P.col_bias[col] : 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = tile.r0 + 64 * wm + 16 * i + 4 * (lane >> 4) + e;
          if (row < tile.r_end) C[(int64_t)row * P.ldc + ccol0 + col] = acc[i][j][e] + bias;
        }
    }
  } else {
    bf16_t* C = static_cast<bf16_t*>(P.C);
#pragma unroll
    for (int j = 0; j < (DUAL ? 2 : 1); ++j) {
      const int col = tile.n0 + 32 * wn + 16 * j + lrow;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = tile.r0 + 64 * wm + 16 * i + 4 * (lane >> 4) + e;
          if (row < tile.r_end) {
            const float h = silu_f32(acc[i][j][e]) * acc2[i][j][e];
            C[(int64_t)row * P.ldc + ccol0 + col] = f32_to_bf16(h);
          }
        }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 VALU kernel: 64 x 64 tiles (x2 for the dual SwiGLU), K-step 16
// ---------------------------------------------------------------------------
constexpr int kFBM = kGemmBM_F32;  // 64
constexpr int kFBN = 64;
constexpr int kFBK = 16;

template <int EPI, bool DUAL>
__global__ void __launch_bounds__(kThreads)
gemm_f32_kernel(GemmLaunch L) {
  __shared__ float As[kFBK][kFBM + 1];
  __shared__ float Bs[DUAL ? 2 : 1][kFBK][kFBN + 1];

  TileRef tile;
  if (!resolve_tile(L, blockIdx.x, kFBM, kFBN, tile)) return;
  const GemmProblem& P = L.p[tile.problem];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const float* A = static_cast<const float*>(P.A);
  const float* B[2] = {static_cast<const float*>(P.B0) + tile.g * P.b_group_stride,
                       DUAL ? static_cast<const float*>(P.B1) + tile.g * P.b_group_stride : nullptr};
  float acc[DUAL ? 2 : 1][4][4] = {};

  for (int k0 = 0; k0 < P.K; k0 += kFBK) {
    // A tile: 64 rows x 16 k, 4 elements per thread
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + i * kThreads;
      const int r = idx >> 4, kk = idx & 15;
      const int row = min(tile.r0 + r, tile.r_end - 1);
      const int64_t arow = P.a_rows ? P.a_rows[row] : row;
      As[kk][r] = A[arow * P.lda + k0 + kk];
    }
#pragma unroll
    for (int v = 0; v < (DUAL ? 2 : 1); ++v)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int idx = tid + i * kThreads;
        const int kk = idx >> 6, c = idx & 63;
        const int col = tile.n0 + c;
        Bs[v][kk][c] = col < P.N ? B[v][(int64_t)(k0 + kk) * P.ldb + col] : 0.f;
      }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kFBK; ++kk) {
      float a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty + 16 * i];
#pragma unroll
      for (int v = 0; v < (DUAL ? 2 : 1); ++v)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float b = Bs[v][kk][tx + 16 * j];
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[v][i][j] = fmaf(a[i], b, acc[v][i][j]);
        }
    }
    __syncthreads();
  }

  const int64_t ccol0 = tile.g * P.c_group_col;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = tile.r0 + ty + 16 * i;
    if (row >= tile.r_end) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = tile.n0 + tx + 16 * j;
      if (col >= P.N) continue;
      float* C = static_cast<float*>(P.C);
      if (EPI == kEpiStoreF32) {
        C[(int64_t)row * P.ldc + ccol0 + col] = acc[0][i][j] + (P.col_bias ? P.col_bias[col] : 0.f);
      } else {
        const float g = acc[0][i][j];
        const float u = acc[DUAL ? 1 : 0][i][j];
        C[(int64_t)row * P.ldc + ccol0 + col] = g / (1.0f + __expf(-g)) * u;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Tile list of a grouped problem: for each group, ceil(rows / bm) M-tiles.
// ---------------------------------------------------------------------------
__device__ int block_exclusive_scan(int v, int* smem, int& total) {
  const int lane = lane_id(), wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int incl = wave_incl_scan_i32(v);
  if (lane == 63) smem[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const int wi = wave_incl_scan_i32(lane < nw ? smem[lane] : 0);
    if (lane < nw) smem[lane] = wi;
  }
  __syncthreads();
  const int base = wave > 0 ? smem[wave - 1] : 0;
  total = smem[nw - 1];
  __syncthreads();
  return base + incl - v;
}

__global__ void __launch_bounds__(1024) plan_kernel(const int32_t* offsets, int G, int bm,
                                                    int32_t* plan) {
  __shared__ int smem[16];
  const int per = (G + blockDim.x - 1) / blockDim.x;
  const int g0 = threadIdx.x * per;
  int local = 0;
  for (int g = g0; g < min(G, g0 + per); ++g) local += (offsets[g + 1] - offsets[g] + bm - 1) / bm;
  int total;
  int pos = block_exclusive_scan(local, smem, total);
  for (int g = g0; g < min(G, g0 + per); ++g) {
    const int r0 = offsets[g], r1 = offsets[g + 1];
    for (int r = r0; r < r1; r += bm) {
      plan[1 + 2 * pos] = g;
      plan[2 + 2 * pos] = r;
      ++pos;
    }
  }
  if (threadIdx.x == 0) plan[0] = total;
}

int grid_of(const GemmLaunch& L) {
  int n = L.tiles0;
  if (L.n_problems > 1) n += L.p[1].max_m_tiles * L.p[1].n_tiles_n;
  return n;
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmLaunch& L, int epilogue, hipStream_t s) {
  const int grid = grid_of(L);
  if (grid <= 0) return hipSuccess;
  bool guard = false;
  for (int i = 0; i < L.n_problems; ++i) {
    const int bn = epilogue == kEpiSwiGLU ? 64 : 128;
    if (L.p[i].N % bn != 0 || (L.p[i].ldb & 1)) guard = true;
  }
  if (epilogue == kEpiSwiGLU) {
    if (guard) return hipErrorInvalidValue;   // host validation guarantees N % 64 == 0
    hipLaunchKernelGGL((gemm_bf16_kernel<kEpiSwiGLU, true, false>), dim3(grid), dim3(kThreads), 0,
                       s, L);
  } else if (guard) {
    hipLaunchKernelGGL((gemm_bf16_kernel<kEpiStoreF32, false, true>), dim3(grid), dim3(kThreads), 0,
                       s, L);
  } else {
    hipLaunchKernelGGL((gemm_bf16_kernel<kEpiStoreF32, false, false>), dim3(grid), dim3(kThreads),
                       0, s, L);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_f32(const GemmLaunch& L, int epilogue, hipStream_t s) {
  const int grid = grid_of(L);
  if (grid <= 0) return hipSuccess;
  if (epilogue == kEpiSwiGLU)
    hipLaunchKernelGGL((gemm_f32_kernel<kEpiSwiGLU, true>), dim3(grid), dim3(kThreads), 0, s, L);
  else
    hipLaunchKernelGGL((gemm_f32_kernel<kEpiStoreF32, false>), dim3(grid), dim3(kThreads), 0, s, L);
  return hipGetLastError();
}

hipError_t launch_plan(const int32_t* offsets, int32_t G, int32_t bm, int32_t* plan,
                       hipStream_t s) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, s, offsets, G, bm, plan);
  return hipGetLastError();
}

}  // namespace moe
