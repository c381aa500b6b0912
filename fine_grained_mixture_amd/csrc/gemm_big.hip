// Grouped GEMM for the expert FFNs on gfx950 (bf16 in, fp32 accumulate).
//
// Workgroup tile 256 x 128 (for the fused SwiGLU: 256 rows x 64 gate + 64 up
// columns of the same output range), K-step 32, 256 threads = 2 x 2 waves,
// each wave 128 x 64 with v_mfma_f32_32x32x16_bf16 (8 accumulator blocks of
// 32 x 32, 128 registers). 72 KiB of LDS and <= 256 registers per lane let
// two workgroups share a CU, so one computes while the other waits at its
// barrier or on memory.
//
// Operands: A rows are k-contiguous (token rows, optionally gathered through
// a_rows), stored in LDS [row][k]; B = W[K, N] is n-contiguous, stored in LDS
// [k][n] exactly as in memory, and read with ds_read_b64_tr_b16, which hands
// each lane 4 consecutive k of one column: within a 16-lane group, output lane
// j receives element i from the address of source lane 4i + j/4, element j%4,
// so source lane s points at row k0 + s/4, columns n0 + 4 (s%4). Two such reads
// give the 8 consecutive k of the MFMA B operand with no register transpose.
// Both LDS tiles are XOR-swizzled in 16-byte chunks to spread banks.
//
// Global -> LDS uses direct-to-LDS loads (global_load_lds_dwordx4: lane L of a
// wave writes its 16 bytes at LDS base + 16 L), so no registers stage the
// tiles; the swizzle is applied by choosing which global chunk each lane
// fetches. A three-stage ring keeps two K-steps in flight: each wave waits for
// its own loads of the step (vmcnt), one workgroup barrier per step publishes
// it and releases the stage the next loads overwrite. The loads of a step are
// interleaved with the MFMAs of the step two behind it.
//
// The epilogue stages each wave's results through a private LDS slice and
// writes whole 16-byte pieces of rows (fp32 rows, or bf16 h = SiLU(gate) * up).

#include <type_traits>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kBM = kGemmBigBM;   // 256
constexpr int kBNT = 128;         // output columns per tile (dual: 64 + 64)
constexpr int kBK = 32;
constexpr int kStages = 3;
constexpr int kThreads = 256;
constexpr int kAStage = kBM * kBK;     // elements
constexpr int kBStage = kBK * kBNT;
constexpr int kStageBytes = (kAStage + kBStage) * 2;   // 24 KiB

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

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

__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "s"(lds)
               : "memory", "m0");
}

// A tile [256][32] bf16: 64-byte rows of 4 chunks, chunk ^ ((row >> 2) & 3)
__device__ __forceinline__ int a_off(int row, int chunk) {
  return row * 64 + 16 * (chunk ^ ((row >> 2) & 3));
}
// B tile [32][128] bf16: 256-byte rows of 16 chunks, chunk ^ (2 (k & 3))
__device__ __forceinline__ int b_off(int k, int chunk) {
  return k * 256 + 16 * (chunk ^ ((k & 3) << 1));
}

template <int EPI, bool DUAL>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_big_kernel(GemmLaunch L) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kStages * kStageBytes];
  constexpr int BN = DUAL ? 64 : 128;   // problem columns per tile

  const int nwg = gridDim.x;
  int bid = blockIdx.x;
  {
    // Workgroups are dealt to the 8 XCDs round-robin. Give each XCD runs of
    // C consecutive tiles (four M-tiles' worth of N-tiles: the N-tiles of an
    // M-tile share its A rows, and the M-tiles of an expert, about four at
    // the Quartz shape, share its weights in that XCD's L2), with the runs
    // themselves dealt round-robin so that long tiles (the shared experts'
    // down projection has twice the K) spread over several XCDs (four at the
    // Quartz shape: 128 such tiles make four runs). Runs of two M-tiles
    // measured 1-2% slower, runs of eight slower still, and one contiguous
    // range per XCD cut at equal K-weighted work no faster.
    const int C = L.p[0].n_tiles_n * 4;
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
  const int64_t ldb = P.ldb;

  // A: wave w, load j (0..3) covers rows 64 w + 16 j .. +15; lane L -> row
  // 16 j + L / 4 of that block, slot L % 4 = chunk (L % 4) ^ (L / 16)
  const bf16_t* A = static_cast<const bf16_t*>(P.A);
  const bf16_t* a_src[4];
  {
    const int c = (lane & 3) ^ (lane >> 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = min(tile.r0 + 64 * wave + 16 * j + (lane >> 2), tile.r_end - 1);
      const int64_t arow = P.a_rows ? P.a_rows[r] : r;
      a_src[j] = A + arow * P.lda + 8 * c;
    }
  }
  // B: wave w, load j (0..1) covers k-rows 8 w + 4 j .. +3; lane L -> k-row
  // 8 w + 4 j + L / 16, slot L % 16 = chunk (L % 16) ^ (2 (L / 16))
  const bf16_t* b_src;
  {
    const int c = (lane & 15) ^ ((lane >> 4) << 1);
    const bf16_t* Bbase;
    int col;
    if (DUAL) {
      Bbase = static_cast<const bf16_t*>(c < 8 ? P.B0 : P.B1);
      col = tile.n0 + 8 * (c & 7);
    } else {
      Bbase = static_cast<const bf16_t*>(P.B0);
      col = tile.n0 + 8 * c;
    }
    col = min(col, N - 8);
    b_src = Bbase + tile.g * P.b_group_stride + (int64_t)(8 * wave + (lane >> 4)) * ldb + col;
  }

  const uint32_t smem_base =
      (uint32_t)(uintptr_t)((__attribute__((address_space(3))) unsigned char*)smem);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  auto issue = [&](int kt) {
    const uint32_t As = smem_base + (kt % kStages) * kStageBytes;
    const uint32_t Bs = As + kAStage * 2;
    const int k0 = kt * kBK;
#pragma unroll
    for (int j = 0; j < 4; ++j) dma16(a_src[j] + k0, As + (4 * wave_u + j) * 1024);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      dma16(b_src + (int64_t)(k0 + 4 * j) * ldb, Bs + (2 * wave_u + j) * 1024);
  };

  // wave tile: rows 128 wm .. +127; columns single 64 wn .. +63,
  // dual gate 32 wn .. +31 and up 64 + 32 wn .. +31
  const int wm = wave >> 1, wn = wave & 1;
  floatx16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  const int l32 = lane & 31, lhi = lane >> 5;
  const int g16 = lane >> 4, s16 = lane & 15;
  const int bk_lane = 8 * (g16 >> 1) + (s16 >> 2);
  const int bn_lane = 16 * (g16 & 1) + 4 * (s16 & 3);
  int bcol[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) bcol[j] = (DUAL ? 64 * j + 32 * wn : 64 * wn + 32 * j) + bn_lane;

  typedef short shortx8 __attribute__((ext_vector_type(8)));
  const int nk = K / kBK;
  // One K-step: the fragments of both k16 halves are requested first; the six
  // direct-to-LDS loads of step kt_next go out one after each of the first six
  // MFMAs. A load whose issue stalls (the CU's load path is shared by eight
  // waves) then waits behind MFMAs already in flight instead of in front of
  // them.
  // NI: how many of the wave's four 32-row blocks hold rows of the tile (the
  // last tile of an expert is partial); the others skip their fragment reads
  // and MFMAs, which frees the SIMD for the co-resident workgroup's wave. The
  // loads and barriers are the same for every wave.
  auto step = [&](int st, int kt_next, auto ni) {
    constexpr int NI = decltype(ni)::value;
    const unsigned char* As = smem + st * kStageBytes;
    const unsigned char* Bs = As + kAStage * 2;
    const uint32_t Asn = smem_base + (kt_next % kStages) * kStageBytes;
    const uint32_t Bsn = Asn + kAStage * 2;
    const int k0n = kt_next * kBK;
    const bool do_issue = kt_next < nk;
    bf16x8 a[2][4], b[2][2];
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
#pragma unroll
      for (int i = 0; i < NI; ++i)
        a[ks][i] = *reinterpret_cast<const bf16x8*>(As + a_off(128 * wm + 32 * i + l32, 2 * ks + lhi));
      if (NI > 0) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int k = 16 * ks + bk_lane;
          const int n = bcol[j];
          const int o0 = b_off(k, n >> 3) + 2 * (n & 7);
          const int o1 = b_off(k + 4, n >> 3) + 2 * (n & 7);
          const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) shortx4*)(Bs + o0));
          const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) shortx4*)(Bs + o1));
          const shortx8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          b[ks][j] = __builtin_bit_cast(bf16x8, v);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int ks = q >> 3, i = (q >> 1) & 3, j = q & 1;
      if (i < NI)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks][i], b[ks][j], acc[i][j], 0, 0, 0);
      if (do_issue && q < 6) {
        __builtin_amdgcn_sched_barrier(0);
        if (q < 4) dma16(a_src[q] + k0n, Asn + (4 * wave_u + q) * 1024);
        else dma16(b_src + (int64_t)(k0n + 4 * (q - 4)) * ldb, Bsn + (2 * wave_u + q - 4) * 1024);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  constexpr int kWaitVm6 = 6 | (7 << 4) | (15 << 8);
  constexpr int kWaitVm0 = (7 << 4) | (15 << 8);
  auto main_loop = [&](auto ni) {
    issue(0);
    if (nk > 1) issue(1);
    for (int kt = 0; kt < nk; ++kt) {
      if (kt + 1 < nk) __builtin_amdgcn_s_waitcnt(kWaitVm6);   // step kt landed
      else __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();   // stage kt published; stage (kt - 1) % 3 released
      __builtin_amdgcn_sched_barrier(0);
      step(kt % kStages, kt + 2, ni);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  {
    const int rows_here = tile.r_end - tile.r0 - 128 * wm;
    const int nib = __builtin_amdgcn_readfirstlane(min(4, max(0, (rows_here + 31) / 32)));
    switch (nib) {
      case 4: main_loop(std::integral_constant<int, 4>()); break;
      case 3: main_loop(std::integral_constant<int, 3>()); break;
      case 2: main_loop(std::integral_constant<int, 2>()); break;
      case 1: main_loop(std::integral_constant<int, 1>()); break;
      default: main_loop(std::integral_constant<int, 0>()); break;
    }
  }

  // ---- epilogue through a private 18 KiB LDS slice per wave
  __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4));
  __builtin_amdgcn_s_barrier();
  unsigned char* stage = smem + wave * (kStages * kStageBytes / 4);
  const int64_t ccol0 = tile.g * P.c_group_col;
  const int row_base = tile.r0 + 128 * wm;
  if (EPI == kEpiStoreF32) {
    float* C = static_cast<float*>(P.C);
    float* st = reinterpret_cast<float*>(stage);
    // the tile's rows of C as a raw buffer (stores past its range are dropped)
    const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
        C + (int64_t)tile.r0 * P.ldc + ccol0, 0, 0x7fffffff, kBufferRsrcWord3);
    const int col0 = tile.n0 + 64 * wn;
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
        const int col = col0 + 4 * (lane & 15);
        floatx4 v = *reinterpret_cast<const floatx4*>(&st[r * 72 + 4 * (lane & 15)]);
        if (P.col_bias) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] += col + e < N ? P.col_bias[col + e] : 0.f;
        }
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
    if (P.ab) {
      // the gate and up sums themselves, for the backward: each of the two is
      // staged as the wave's 128 rows x 32 columns (row pitch 36 floats), then
      // written as 16-byte pieces, 8 per row, with streaming stores: nothing
      // reads them before the backward (Quartz forward keeping them 0.285 ->
      // 0.25-0.26 ms, forward + backward about 1% faster)
      float* sf = reinterpret_cast<float*>(stage);
      float* abp = P.ab + tile.g * P.ab_group_col + tile.n0 + 32 * wn + 4 * (lane & 7);
#pragma unroll
      for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int q = 0; q < 16; ++q)
            sf[(32 * i + 8 * (q >> 2) + 4 * lhi + (q & 3)) * 36 + l32] = acc[i][half][q];
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int it = 0; it < 16; ++it) {
          const int r = 8 * it + (lane >> 3);
          const int row = row_base + r;
          const floatx4 v = *reinterpret_cast<const floatx4*>(&sf[r * 36 + 4 * (lane & 7)]);
          if (row < tile.r_end)
            __builtin_nontemporal_store(v, reinterpret_cast<floatx4*>(abp + (int64_t)row * P.ab_ld + half * N));
        }
        __builtin_amdgcn_wave_barrier();
      }
    }
    bf16_t* C = static_cast<bf16_t*>(P.C);
    bf16_t* st = reinterpret_cast<bf16_t*>(stage);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const float h = silu_f32(acc[i][0][q]) * acc[i][1][q];
        st[(32 * i + 8 * (q >> 2) + 4 * lhi + (q & 3)) * 40 + l32] = f32_to_bf16(h);
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

int grid_of(const GemmLaunch& L) {
  int n = L.tiles0;
  if (L.n_problems > 1) n += L.p[1].max_m_tiles * L.p[1].n_tiles_n;
  return n;
}

}  // namespace

hipError_t launch_gemm_big(const GemmLaunch& L, int epilogue, hipStream_t s) {
  const int grid = grid_of(L);
  if (grid <= 0) return hipSuccess;
  // the fp32 epilogue addresses a tile's rows of C with 32-bit byte offsets
  for (int i = 0; i < L.n_problems; ++i)
    if (epilogue == kEpiStoreF32 && L.p[i].ldc >= ((int64_t)1 << 21)) return hipErrorInvalidValue;
  if (epilogue == kEpiSwiGLU)
    hipLaunchKernelGGL((gemm_big_kernel<kEpiSwiGLU, true>), dim3(grid), dim3(kThreads), 0, s, L);
  else
    hipLaunchKernelGGL((gemm_big_kernel<kEpiStoreF32, false>), dim3(grid), dim3(kThreads), 0, s, L);
  return hipGetLastError();
}

}  // namespace moe
