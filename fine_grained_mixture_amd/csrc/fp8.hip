// fp8 (OCP E4M3) expert products on gfx950.
//
// Storage (the storage ladder's fp8 rung, dormouse "TSCT low-rank experts"
// card): every value of a vector is a code of the E4M3 grid times one power of
// two, per row for activations and per output column for weights, the
// smallest power that brings the vector's largest magnitude to at most 448.
// Scaling by a power of two is exact, so the only rounding is the hardware's
// round-to-nearest-even onto the grid (v_cvt_pk_fp8_f32).
//
// quant_rows_kernel: one wave per row, the row held in registers; its maximum
//   magnitude by a wave reduction, then 8 codes per 16-byte piece.
// quant_cols_kernel: weights [K, N] -> codes [N, K] (k-contiguous, the order
//   the MFMA operand is read in) and one scale per column.
// gemm_fp8_kernel: both operands k-contiguous codes. 256 x 128 output tiles
//   (SwiGLU: 256 rows x 64 gate + 64 up columns), K-step 64 codes (64 bytes
//   per row, the bf16 kernel's byte geometry), three-stage direct-to-LDS ring,
//   2 x 2 waves of 128 x 64 on v_mfma_scale_f32_32x32x64_f8f6f4 with unit
//   scales. Lane l of the MFMA supplies row (or column) l % 32 at 32
//   consecutive codes k = 32 (l / 32) .. + 31, two ds_read_b128 from the
//   XOR-swizzled tile; A and B use the same byte order, which is all the
//   product needs. The epilogue multiplies by the row and column scales.

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kBM = kGemmBigBM;   // 256
constexpr int kBNT = 128;         // B rows (output columns) per tile
constexpr int kBK = 64;           // codes (bytes) per K-step
constexpr int kStages = 3;
constexpr int kThreads = 256;
constexpr int kAStageBytes = kBM * kBK;    // 16 KiB
constexpr int kBStageBytes = kBNT * kBK;   // 8 KiB
constexpr int kStageBytes = kAStageBytes + kBStageBytes;
constexpr int kE8M0One = 127;   // MFMA block scale 2^0

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// Direct-to-LDS 16-byte load (lane L writes LDS base + 16 L). Written as asm
// so that the compiler inserts no waits for it: the ring's vmcnt waits are
// explicit. m0 is a reserved register, so its clobber is not honoured; the
// compiler uses m0 nowhere else in these kernels, which a CPU test checks.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "s"(lds)
               : "memory", "m0");
}

// tile [rows][64 bytes]: 4 chunks of 16 codes, chunk ^ ((row >> 2) & 3)
__device__ __forceinline__ int kc_off(int row, int chunk) {
  return row * 64 + 16 * (chunk ^ ((row >> 2) & 3));
}

__device__ __forceinline__ v8i frag32(const unsigned char* t, int row, int half) {
  const u32x4 lo = *reinterpret_cast<const u32x4*>(t + kc_off(row, 2 * half));
  const u32x4 hi = *reinterpret_cast<const u32x4*>(t + kc_off(row, 2 * half + 1));
  v8i v;
  v[0] = (int)lo[0];
  v[1] = (int)lo[1];
  v[2] = (int)lo[2];
  v[3] = (int)lo[3];
  v[4] = (int)hi[0];
  v[5] = (int)hi[1];
  v[6] = (int)hi[2];
  v[7] = (int)hi[3];
  return v;
}

// Power-of-two scale exponent: the smallest s with amax 2^-s <= 448.
__device__ __forceinline__ int fp8_scale_exp(float amax) {
  if (!(amax > 0.f)) return 0;
  int ex;
  const float fr = frexpf(amax, &ex);   // amax = fr 2^ex, fr in [0.5, 1)
  return fr <= 0.875f ? ex - 9 : ex - 8;
}

// Four values (already scaled into [-448, 448]) to four codes, byte i = value i.
__device__ __forceinline__ uint32_t pack4_fp8(float a, float b, float c, float d) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, 0, false) & 0xffffu;
  return lo | (hi << 16);
}

struct TileRef {
  int problem, g, r0, r_end, n0;
};

__device__ __forceinline__ bool resolve(const GemmLaunch& L, int bid, int bn, TileRef& t) {
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
    if (mt >= P.plan[0]) return false;
    t.g = P.plan[1 + 2 * mt];
    t.r0 = P.plan[2 + 2 * mt];
    t.r_end = min(P.row_off[t.g + 1], t.r0 + kBM);
  } else {
    const int mtg = (P.M + kBM - 1) / kBM;
    if (mt >= mtg * P.G) return false;
    t.g = mt / mtg;
    t.r0 = (mt - t.g * mtg) * kBM;
    t.r_end = min(P.M, t.r0 + kBM);
  }
  t.problem = prob;
  t.n0 = nt * bn;
  return t.r0 < t.r_end;
}

template <int EPI, bool DUAL>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_fp8_kernel(GemmLaunch L) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kStages * kStageBytes];
  __shared__ float s_rs[kBM];   // the tile's row scales
  constexpr int BN = DUAL ? 64 : 128;

  const int nwg = gridDim.x;
  int bid = blockIdx.x;
  {
    // runs of C consecutive tiles per XCD (shared A rows in its L2), the runs
    // dealt round-robin over the 8 XCDs
    const int C = L.p[0].n_tiles_n * 2;
    const int full = nwg / (8 * C) * (8 * C);
    if (bid < full) {
      const int x = bid & 7, i = bid >> 3;
      bid = ((i / C) * 8 + x) * C + (i % C);
    }
  }
  TileRef tile;
  if (!resolve(L, bid, BN, tile)) return;
  const GemmProblem& P = L.p[tile.problem];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = P.N, K = P.K;

  for (int r = tid; r < kBM; r += kThreads) {
    const int row = min(tile.r0 + r, tile.r_end - 1);
    s_rs[r] = P.a_scale[P.a_rows ? P.a_rows[row] : row];
  }

  // A: wave w, load j covers rows 16 (4 w + j) .. +15: lane -> row + L / 4,
  // chunk (L % 4) ^ (L / 16)
  const int cc = (lane & 3) ^ (lane >> 4);
  const uint8_t* A = static_cast<const uint8_t*>(P.A);
  const uint8_t* a_src[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = min(tile.r0 + 16 * (4 * wave + j) + (lane >> 2), tile.r_end - 1);
    const int64_t arow = P.a_rows ? P.a_rows[r] : r;
    a_src[j] = A + arow * P.lda + 16 * cc;
  }
  // B: wave w, load j covers B-tile rows 16 (2 w + j) .. +15 (dual: rows
  // 0..63 gate columns, 64..127 up columns)
  const uint8_t* b_src[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int br = 16 * (2 * wave + j) + (lane >> 2);
    const uint8_t* base;
    int n;
    if (DUAL) {
      base = static_cast<const uint8_t*>(br < 64 ? P.B0 : P.B1);
      n = tile.n0 + (br & 63);
    } else {
      base = static_cast<const uint8_t*>(P.B0);
      n = tile.n0 + br;
    }
    n = min(n, N - 1);
    b_src[j] = base + tile.g * P.b_group_stride + (int64_t)n * P.ldb + 16 * cc;
  }

  const uint32_t smem_base =
      (uint32_t)(uintptr_t)((__attribute__((address_space(3))) unsigned char*)smem);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  auto issue = [&](int kt) {
    const uint32_t As = smem_base + (kt % kStages) * kStageBytes;
    const uint32_t Bs = As + kAStageBytes;
    const int k0 = kt * kBK;
#pragma unroll
    for (int j = 0; j < 4; ++j) dma16(a_src[j] + k0, As + (4 * wave_u + j) * 1024);
#pragma unroll
    for (int j = 0; j < 2; ++j) dma16(b_src[j] + k0, Bs + (2 * wave_u + j) * 1024);
  };

  const int wm = wave >> 1, wn = wave & 1;
  floatx16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
  const int l32 = lane & 31, lhi = lane >> 5;
  int brow[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) brow[j] = (DUAL ? 64 * j + 32 * wn : 64 * wn + 32 * j) + l32;

  const int nk = K / kBK;
  auto step = [&](int st, int kt_next) {
    const unsigned char* As = smem + st * kStageBytes;
    const unsigned char* Bs = As + kAStageBytes;
    const uint32_t Asn = smem_base + (kt_next % kStages) * kStageBytes;
    const uint32_t Bsn = Asn + kAStageBytes;
    const int k0n = kt_next * kBK;
    const bool do_issue = kt_next < nk;
    v8i a[4], b[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = frag32(As, 128 * wm + 32 * i + l32, lhi);
#pragma unroll
    for (int j = 0; j < 2; ++j) b[j] = frag32(Bs, brow[j], lhi);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int i = q >> 1, j = q & 1;
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          a[i], b[j], acc[i][j], 0, 0, 0, kE8M0One, 0, kE8M0One);
      if (do_issue && q < 6) {
        __builtin_amdgcn_sched_barrier(0);
        if (q < 4) dma16(a_src[q] + k0n, Asn + (4 * wave_u + q) * 1024);
        else dma16(b_src[q - 4] + k0n, Bsn + (2 * wave_u + q - 4) * 1024);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  constexpr int kWaitVm6 = 6 | (7 << 4) | (15 << 8);
  constexpr int kWaitVm0 = (7 << 4) | (15 << 8);
  issue(0);
  if (nk > 1) issue(1);
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) __builtin_amdgcn_s_waitcnt(kWaitVm6);
    else __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    step(kt % kStages, kt + 2);
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- epilogue through a private 18 KiB LDS slice per wave
  __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4));
  __builtin_amdgcn_s_barrier();
  unsigned char* stage = smem + wave * (kStages * kStageBytes / 4);
  const int64_t ccol0 = tile.g * P.c_group_col;
  const int row_base = tile.r0 + 128 * wm;
  const int rl_base = 128 * wm;
  if (EPI == kEpiStoreF32) {
    float* C = static_cast<float*>(P.C);
    float* st = reinterpret_cast<float*>(stage);
    // the tile's rows of C as a raw buffer; the cache policy of its stores is
    // an immediate, so each policy is a store of its own
    const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
        C + (int64_t)tile.r0 * P.ldc + ccol0, 0, 0x7fffffff, kBufferRsrcWord3);
    const int col = tile.n0 + 64 * wn + 4 * (lane & 15);
    floatx4 cs = {0.f, 0.f, 0.f, 0.f};
    if (col < N) cs = *reinterpret_cast<const floatx4*>(P.b_scale0 + tile.g * P.b_scale_group + col);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q)
          st[(8 * (q >> 2) + 4 * lhi + (q & 3)) * 72 + 32 * j + l32] = acc[i][j][q];
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        const int r = 4 * rr + (lane >> 4);
        const int row = row_base + 32 * i + r;
        const float rs = s_rs[rl_base + 32 * i + r];
        floatx4 v = *reinterpret_cast<const floatx4*>(&st[r * 72 + 4 * (lane & 15)]);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = v[e] * rs * cs[e];
        if (row < tile.r_end && col < N) {
          // byte offset from the tile's first row: below 2^31 while 256 ldc < 2^29
          const int off = (int)(((int64_t)(row - tile.r0) * P.ldc + col) * 4);
          if (P.c_stream)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), crs, off, 0, kCpolNT);
          else
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), crs, off, 0, 0);
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
  } else {
    bf16_t* C = static_cast<bf16_t*>(P.C);
    bf16_t* st = reinterpret_cast<bf16_t*>(stage);
    const int gcol = tile.n0 + 32 * wn + l32;   // this lane's gate / up column
    const float sg = P.b_scale0[tile.g * P.b_scale_group + gcol];
    const float su = P.b_scale1[tile.g * P.b_scale_group + gcol];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int r = 32 * i + 8 * (q >> 2) + 4 * lhi + (q & 3);
        const float rs = s_rs[rl_base + r];
        const float a = acc[i][0][q] * rs * sg;
        const float b = acc[i][1][q] * rs * su;
        st[r * 40 + l32] = f32_to_bf16(silu_f32(a) * b);
      }
    __builtin_amdgcn_wave_barrier();
    const int col = tile.n0 + 32 * wn + 8 * (lane & 3);
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const int r = 16 * rr + (lane >> 2);
      const int row = row_base + r;
      const u32x4 v = *reinterpret_cast<const u32x4*>(&st[r * 40 + 8 * (lane & 3)]);
      if (row < tile.r_end && col < N)
        *reinterpret_cast<u32x4*>(C + (int64_t)row * P.ldc + ccol0 + col) = v;
    }
  }
}

// One row per wave; the row's 16-byte pieces stay in registers (NP per lane)
// between the maximum and the conversion.
template <int NP>
__global__ void __launch_bounds__(256) quant_rows_kernel(const uint16_t* src, int64_t ld,
                                                         int64_t rows, int K,
                                                         const int32_t* n_valid, uint8_t* q,
                                                         float* scale) {
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int64_t nrows = rows;
  if (n_valid) nrows = min(rows, (int64_t)*n_valid);
  const int np = K / 8;
  for (int64_t r = (int64_t)blockIdx.x * 4 + wave; r < nrows; r += (int64_t)gridDim.x * 4) {
    const u32x4* s4 = reinterpret_cast<const u32x4*>(src + r * ld);
    u32x4 v[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int p = lane + 64 * i;
      v[i] = s4[min(p, np - 1)];
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      if (lane + 64 * i < np) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          amax = fmaxf(amax, fabsf(__uint_as_float(v[i][e] << 16)));
          amax = fmaxf(amax, fabsf(__uint_as_float(v[i][e] & 0xffff0000u)));
        }
      }
    }
    amax = wave_max(amax);
    const int sc = fp8_scale_exp(amax);
    u32x2* out = reinterpret_cast<u32x2*>(q + r * K);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int p = lane + 64 * i;
      if (p < np) {
        float f[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f[2 * e] = ldexpf(__uint_as_float(v[i][e] << 16), -sc);
          f[2 * e + 1] = ldexpf(__uint_as_float(v[i][e] & 0xffff0000u), -sc);
        }
        u32x2 w;
        w[0] = pack4_fp8(f[0], f[1], f[2], f[3]);
        w[1] = pack4_fp8(f[4], f[5], f[6], f[7]);
        out[p] = w;
      }
    }
    if (lane == 0) scale[r] = ldexpf(1.0f, sc);
  }
}

// One workgroup per (group, 64 columns).
__global__ void __launch_bounds__(256) quant_cols_kernel(const uint16_t* w, int K, int N,
                                                         uint8_t* q, float* scale) {
  __shared__ float s_am[4][64];
  __shared__ int s_sc[64];
  const int nch = N / 64;
  const int g = blockIdx.x / nch, n0 = (blockIdx.x - g * nch) * 64;
  const int t = threadIdx.x, c = t & 63, kg = t >> 6;
  const uint16_t* W = w + (int64_t)g * K * N;
  float amax = 0.f;
  for (int k = kg; k < K; k += 4) amax = fmaxf(amax, fabsf(bf16_to_f32(W[(int64_t)k * N + n0 + c])));
  s_am[kg][c] = amax;
  __syncthreads();
  if (t < 64) {
    const float a = fmaxf(fmaxf(s_am[0][t], s_am[1][t]), fmaxf(s_am[2][t], s_am[3][t]));
    const int sc = fp8_scale_exp(a);
    s_sc[t] = sc;
    scale[(int64_t)g * N + n0 + t] = ldexpf(1.0f, sc);
  }
  __syncthreads();
  uint8_t* Q = q + (int64_t)g * N * K;
  const int nq = K / 4;
  for (int item = t; item < 64 * nq; item += 256) {
    const int col = item & 63, kq = item >> 6;
    const int sc = s_sc[col];
    float f[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      f[i] = ldexpf(bf16_to_f32(W[(int64_t)(4 * kq + i) * N + n0 + col]), -sc);
    *reinterpret_cast<uint32_t*>(Q + (int64_t)(n0 + col) * K + 4 * kq) = pack4_fp8(f[0], f[1], f[2], f[3]);
  }
}

int grid_of(const GemmLaunch& L) {
  int n = L.tiles0;
  if (L.n_problems > 1) n += L.p[1].max_m_tiles * L.p[1].n_tiles_n;
  return n;
}

}  // namespace

hipError_t launch_gemm_fp8(const GemmLaunch& L, int epilogue, hipStream_t s) {
  for (int i = 0; i < L.n_problems; ++i) {
    const GemmProblem& P = L.p[i];
    // the fp32 epilogue addresses a tile's rows of C with 32-bit byte offsets
    if (epilogue == kEpiStoreF32 && P.ldc >= ((int64_t)1 << 21)) return hipErrorInvalidValue;
    if (P.K % kBK || P.N % 64 || P.lda % 16 || P.ldb % 16 || !P.a_scale || !P.b_scale0)
      return hipErrorInvalidValue;
    if (epilogue == kEpiSwiGLU && !P.b_scale1) return hipErrorInvalidValue;
  }
  const int grid = grid_of(L);
  if (grid <= 0) return hipSuccess;
  if (epilogue == kEpiSwiGLU)
    hipLaunchKernelGGL((gemm_fp8_kernel<kEpiSwiGLU, true>), dim3(grid), dim3(kThreads), 0, s, L);
  else
    hipLaunchKernelGGL((gemm_fp8_kernel<kEpiStoreF32, false>), dim3(grid), dim3(kThreads), 0, s, L);
  return hipGetLastError();
}

hipError_t launch_quant_rows(const uint16_t* src, int64_t ld, int64_t rows, int32_t K,
                             const int32_t* n_valid, uint8_t* q, float* scale, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  // rows of up to 64 * 8 * 8 = 4096 values, kept in registers
  if (K % 8 || ld % 8 || K <= 0 || K > 4096) return hipErrorInvalidValue;
  const int64_t waves = rows < (1 << 20) ? rows : (1 << 20);
  const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
  const int np = K / 8;
  if (np <= 64)
    hipLaunchKernelGGL((quant_rows_kernel<1>), grid, block, 0, s, src, ld, rows, K, n_valid, q, scale);
  else if (np <= 128)
    hipLaunchKernelGGL((quant_rows_kernel<2>), grid, block, 0, s, src, ld, rows, K, n_valid, q, scale);
  else if (np <= 256)
    hipLaunchKernelGGL((quant_rows_kernel<4>), grid, block, 0, s, src, ld, rows, K, n_valid, q, scale);
  else
    hipLaunchKernelGGL((quant_rows_kernel<8>), grid, block, 0, s, src, ld, rows, K, n_valid, q, scale);
  return hipGetLastError();
}

hipError_t launch_quant_cols(const uint16_t* w, int64_t G, int32_t K, int32_t N, uint8_t* q,
                             float* scale, hipStream_t s) {
  if (G == 0) return hipSuccess;
  if (K % 4 || N % 64 || K <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quant_cols_kernel, dim3((unsigned)(G * (N / 64))), dim3(256), 0, s, w, K, N,
                     q, scale);
  return hipGetLastError();
}

}  // namespace moe
