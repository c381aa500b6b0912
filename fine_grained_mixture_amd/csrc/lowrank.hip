// Fused low-rank SwiGLU experts on gfx950 (bf16, rank 64).
//
// Each expert matrix is W = U diag(s) V^T of rank r (dormouse site, "TSCT
// low-rank experts" card: rank 64, which is what lets a 1.07B-parameter bank
// fit a 16 GB card). For the rows routed to expert e:
//   zg = rho((A U_gate) * s_gate),  zu = rho((A U_up) * s_up)        [rows, r]
//   h  = rho(SiLU(zg V_gate^T) * (zu V_up^T))                       [rows, F]
//   zd = rho((h U_down) * s_down)                                    [rows, r]
//   y  = zd V_down^T                                                 [rows, d]
// with rho = round to bf16 and every product accumulated in fp32 by
// v_mfma_f32_16x16x32_bf16.
//
// fp8 factors (the storage ladder's fp8 rung): the codes are widened to bf16
// exactly on their way to the MFMA, U's power-of-two column scales are folded
// into s and V's are applied to the product's output columns, so the products
// and rounding points are the bf16 ones; U codes arrive transposed ([r, in],
// k-contiguous), which needs no transposing loader.
//
// One workgroup per (expert, chunk of up to 64 rows), from the device tile
// list. The rank-r intermediates and h never leave the CU: zg|zu and zd live in
// LDS, and h is produced 64 columns at a time and immediately folded into the
// zd accumulators, so HBM traffic is the expert weights (streamed once per
// chunk), the token rows and the fp32 output rows. U matrices arrive [in, r]
// (r contiguous) and are transposed on their way into LDS; V matrices arrive
// [out, r], which is already the k-contiguous order the MFMA B operand needs,
// so they are read straight from memory.

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kR = 64;          // rank of the tiles; a smaller rank (16, 32, 48) runs
                                // with the factor entries past it read as zero
constexpr int kBM = kLowRankBM; // 64 rows per workgroup
constexpr int kLd = 72;         // padded LDS row for 64-wide k tiles
constexpr int kLdZ = 136;       // padded LDS row for the [rows, 2r] zg|zu tile

// The factors are read with streaming (non-temporal) loads: each expert's are
// read by its one or two row chunks only, so they should not push the token
// rows (read by k experts each) out of the caches (Dormouse shape: 172 -> 163
// us for the kernel, -1.3% per layer call).
__device__ __forceinline__ void load_b_pair(const bf16_t* src, int64_t ldb, uint32_t* reg) {
#pragma unroll
  for (int i = 0; i < 8; ++i) reg[i] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(src + i * ldb));
}

// Two adjacent columns x 8 consecutive k (as loaded by load_b_pair) written as
// two k-contiguous 16-byte runs: rows `row` and `row + 1` of a [n][k] tile.
__device__ __forceinline__ void store_b_pair(bf16_t* lds, int row, int kq, const uint32_t* reg) {
  u32x4 lo, hi;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint32_t x0 = reg[2 * m], x1 = reg[2 * m + 1];
    lo[m] = (x0 & 0xffffu) | (x1 << 16);
    hi[m] = (x0 >> 16) | (x1 & 0xffff0000u);
  }
  *reinterpret_cast<u32x4*>(&lds[row * kLd + 8 * kq]) = lo;
  *reinterpret_cast<u32x4*>(&lds[(row + 1) * kLd + 8 * kq]) = hi;
}

// Four E4M3 codes (byte i = value i) to four bf16 values, exactly: an E4M3
// value has at most four significant bits.
__device__ __forceinline__ u32x2 cvt4_fp8_bf16(uint32_t w) {
  typedef float floatx2 __attribute__((ext_vector_type(2)));
  const floatx2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const floatx2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  u32x2 r;
  r[0] = (__float_as_uint(lo[0]) >> 16) | (__float_as_uint(lo[1]) & 0xffff0000u);
  r[1] = (__float_as_uint(hi[0]) >> 16) | (__float_as_uint(hi[1]) & 0xffff0000u);
  return r;
}
__device__ __forceinline__ bf16x8 cvt8_fp8_bf16(u32x2 w) {
  const u32x2 a = cvt4_fp8_bf16(w[0]), b = cvt4_fp8_bf16(w[1]);
  const u32x4 v = {a[0], a[1], b[0], b[1]};
  return __builtin_bit_cast(bf16x8, v);
}
// 16 codes to 16 bf16 values written as two 16-byte pieces.
__device__ __forceinline__ void store16_fp8_bf16(bf16_t* dst, u32x4 w) {
  const u32x2 a = cvt4_fp8_bf16(w[0]), b = cvt4_fp8_bf16(w[1]);
  const u32x2 c = cvt4_fp8_bf16(w[2]), d = cvt4_fp8_bf16(w[3]);
  *reinterpret_cast<u32x4*>(dst) = u32x4{a[0], a[1], b[0], b[1]};
  *reinterpret_cast<u32x4*>(dst + 8) = u32x4{c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ floatx4 mfma(const bf16x8& a, const bf16x8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <bool Q8, bool FULL>
__global__ void __launch_bounds__(256) lowrank_kernel(LowRankArgs a) {
  // zg | zu lives through stages 1-3; the other tiles share one region, as
  // no two of the groups are live together: stage 1 (A chunk, U_gate|U_up
  // chunk), stages 2-3 (h chunk, U_down chunk), stage 4 (zd). 44 KiB in all,
  // so three workgroups fit on a CU.
  __shared__ __attribute__((aligned(16))) bf16_t Zs[kBM * kLdZ];                 // zg | zu
  __shared__ __attribute__((aligned(16))) bf16_t Sh[kBM * kLd + 2 * kR * kLd];   // shared region
  bf16_t* const As = Sh;                 // [kBM][kLd]    stage 1
  bf16_t* const Bs = Sh + kBM * kLd;     // [2 kR][kLd]   stage 1, [n][k]
  bf16_t* const Hs = Sh;                 // [kBM][kLd]    stages 2-3
  bf16_t* const Bd = Sh + kBM * kLd;     // [kR][kLd]     stages 2-3, [n][k]
  bf16_t* const Zd = Sh;                 // [kBM][kLd]    stage 4

  const int tile = blockIdx.x;
  if (tile >= a.plan[0]) return;
  const int e = a.plan[1 + 2 * tile];
  const int r0 = a.plan[2 + 2 * tile];
  const int r_end = min(a.offsets[e + 1], r0 + kBM);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lk = 8 * (lane >> 4);
  const int d = a.d, F = a.F;
  // factor row length; columns rk .. kR - 1 of every tile are zero (FULL: the
  // rank is kR and every mask folds away)
  const int rk = FULL ? kR : a.rank;

  const bf16_t* A = static_cast<const bf16_t*>(a.A);
  const bf16_t* Ug = static_cast<const bf16_t*>(a.u_gate) + (int64_t)e * d * rk;
  const bf16_t* Uu = static_cast<const bf16_t*>(a.u_up) + (int64_t)e * d * rk;
  const bf16_t* Vg = static_cast<const bf16_t*>(a.v_gate) + (int64_t)e * F * rk;
  const bf16_t* Vu = static_cast<const bf16_t*>(a.v_up) + (int64_t)e * F * rk;
  const bf16_t* Ud = static_cast<const bf16_t*>(a.u_down) + (int64_t)e * F * rk;
  const bf16_t* Vd = static_cast<const bf16_t*>(a.v_down) + (int64_t)e * d * rk;
  // fp8 factors: U codes [r][in] (k-contiguous rows), V codes [out][r]
  const uint8_t* Ug8 = static_cast<const uint8_t*>(a.u_gate) + (int64_t)e * rk * d;
  const uint8_t* Uu8 = static_cast<const uint8_t*>(a.u_up) + (int64_t)e * rk * d;
  const uint8_t* Ud8 = static_cast<const uint8_t*>(a.u_down) + (int64_t)e * rk * F;
  const uint8_t* Vg8 = static_cast<const uint8_t*>(a.v_gate) + (int64_t)e * F * rk;
  const uint8_t* Vu8 = static_cast<const uint8_t*>(a.v_up) + (int64_t)e * F * rk;
  const uint8_t* Vd8 = static_cast<const uint8_t*>(a.v_down) + (int64_t)e * d * rk;
  const bf16_t* sg = static_cast<const bf16_t*>(a.s_gate) + (int64_t)e * rk;
  const bf16_t* su = static_cast<const bf16_t*>(a.s_up) + (int64_t)e * rk;
  const bf16_t* sd = static_cast<const bf16_t*>(a.s_down) + (int64_t)e * rk;

  // A rows of this chunk (clamped: rows past r_end are computed, never stored)
  const int a_c = tid & 7, a_rb = tid >> 3;
  const bf16_t* a_src[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = min(r0 + a_rb + 32 * i, r_end - 1);
    const int64_t arow = a.a_rows ? a.a_rows[r] : r;
    a_src[i] = A + arow * a.lda + 8 * a_c;
  }
  // B transposing loader: unit (column pair p, k-group q)
  const int bp = tid & 31, bq = tid >> 5;

  // ---- stage 1: zg | zu = A [U_gate | U_up]; wave w owns columns 32w..32w+31
  floatx4 acc1[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc1[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  // the next K-step's A rows and U columns are requested before this step's
  // MFMAs, so their latency overlaps the arithmetic
  u32x4 ar[2];
  uint32_t br[2][8];
  // fp8: B-tile row n = t / 2 (gate rows 0..63, up 64..127), 32 codes at
  // k0 + 32 (t % 2)
  u32x4 bq8[2];
  const int u8_row = (tid >> 1) & (kR - 1);   // U row (rank index) of this thread
  const bool u8_ok = u8_row < rk;
  const uint8_t* u8_src = ((tid >> 1) < kR ? Ug8 : Uu8) + (int64_t)(u8_ok ? u8_row : 0) * d +
                          32 * (tid & 1);
  const bool b_ok = 2 * bp < rk;   // this thread's column pair of U is within the rank
  auto load1 = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) ar[i] = *reinterpret_cast<const u32x4*>(a_src[i] + k0);
    if (Q8) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        bq8[i] = u8_ok ? *reinterpret_cast<const u32x4*>(u8_src + k0 + 16 * i) : u32x4{0, 0, 0, 0};
    } else if (b_ok) {
      load_b_pair(Ug + (int64_t)(k0 + 8 * bq) * rk + 2 * bp, rk, br[0]);
      load_b_pair(Uu + (int64_t)(k0 + 8 * bq) * rk + 2 * bp, rk, br[1]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) br[0][i] = br[1][i] = 0u;
    }
  };
  load1(0);
  for (int k0 = 0; k0 < d; k0 += 64) {
    __syncthreads();   // the previous step's tiles are consumed
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<u32x4*>(&As[(a_rb + 32 * i) * kLd + 8 * a_c]) = ar[i];
    if (Q8) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        store16_fp8_bf16(&Bs[(tid >> 1) * kLd + 32 * (tid & 1) + 16 * i], bq8[i]);
    } else {
      store_b_pair(Bs, 2 * bp, bq, br[0]);
      store_b_pair(Bs, kR + 2 * bp, bq, br[1]);
    }
    __syncthreads();
    if (k0 + 64 < d) load1(k0 + 64);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 av[4], bv[2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        av[i] = *reinterpret_cast<const bf16x8*>(&As[(16 * i + lr) * kLd + 32 * kk + lk]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bv[j] = *reinterpret_cast<const bf16x8*>(&Bs[(32 * wave + 16 * j + lr) * kLd + 32 * kk + lk]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc1[i][j] = mfma(av[i], bv[j], acc1[i][j]);
    }
  }
  // scale by s and round: column c < r is gate, c >= r is up
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int col = 32 * wave + 16 * j + lr;
    const int rc = col & (kR - 1);   // rank index of this column
    float sc = rc >= rk ? 0.f : (col < kR ? bf16_to_f32(sg[rc]) : bf16_to_f32(su[rc]));
    if (Q8 && rc < rk)   // U's column scale folded into s (a power of two: exact)
      sc *= col < kR ? a.u_gate_scale[(int64_t)e * rk + rc] : a.u_up_scale[(int64_t)e * rk + rc];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        Zs[(16 * i + 4 * (lane >> 4) + q) * kLdZ + col] = f32_to_bf16(acc1[i][j][q] * sc);
  }
  __syncthreads();

  // ---- stages 2-3: per 64 columns of F, h chunk then zd += h U_down
  floatx4 accd[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) accd[i] = floatx4{0.f, 0.f, 0.f, 0.f};
  // per 64 columns of F: U_down rows (transposing load) and the V_gate / V_up
  // fragments, requested one chunk ahead
  uint32_t bd[8];
  u32x4 bd8;              // fp8: U_down codes, row t / 4, 16 codes at f0 + 16 (t % 4)
  bf16x8 bgv[2], buv[2];
  float vgs = 1.f, vus = 1.f;   // fp8: V rows' scales of this lane's column
  auto load2 = [&](int f0) {
    const int n = f0 + 16 * wave + lr;
    if (Q8) {
      bd8 = (tid >> 2) < rk
                ? *reinterpret_cast<const u32x4*>(Ud8 + (int64_t)(tid >> 2) * F + f0 + 16 * (tid & 3))
                : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bool ok = 32 * kk + lk < rk;
        bgv[kk] = ok ? cvt8_fp8_bf16(*reinterpret_cast<const u32x2*>(Vg8 + (int64_t)n * rk + 32 * kk + lk))
                     : bf16x8{};
        buv[kk] = ok ? cvt8_fp8_bf16(*reinterpret_cast<const u32x2*>(Vu8 + (int64_t)n * rk + 32 * kk + lk))
                     : bf16x8{};
      }
      vgs = a.v_gate_scale[(int64_t)e * F + n];
      vus = a.v_up_scale[(int64_t)e * F + n];
    } else {
      if (b_ok) {
        load_b_pair(Ud + (int64_t)(f0 + 8 * bq) * rk + 2 * bp, rk, bd);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) bd[i] = 0u;
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bool ok = 32 * kk + lk < rk;
        bgv[kk] = ok ? __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(Vg + (int64_t)n * rk + 32 * kk + lk)) : bf16x8{};
        buv[kk] = ok ? __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(Vu + (int64_t)n * rk + 32 * kk + lk)) : bf16x8{};
      }
    }
  };
  load2(0);
  for (int f0 = 0; f0 < F; f0 += 64) {
    floatx4 accg[4], accu[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) accg[i] = accu[i] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8 ag = *reinterpret_cast<const bf16x8*>(&Zs[(16 * i + lr) * kLdZ + 32 * kk + lk]);
        const bf16x8 au = *reinterpret_cast<const bf16x8*>(&Zs[(16 * i + lr) * kLdZ + kR + 32 * kk + lk]);
        accg[i] = mfma(ag, bgv[kk], accg[i]);
        accu[i] = mfma(au, buv[kk], accu[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        Hs[(16 * i + 4 * (lane >> 4) + q) * kLd + 16 * wave + lr] =
            f32_to_bf16(silu_f32(accg[i][q] * vgs) * (accu[i][q] * vus));
    if (Q8) store16_fp8_bf16(&Bd[(tid >> 2) * kLd + 16 * (tid & 3)], bd8);
    else store_b_pair(Bd, 2 * bp, bq, bd);
    __syncthreads();
    if (f0 + 64 < F) load2(f0 + 64);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const bf16x8 bv = *reinterpret_cast<const bf16x8*>(&Bd[(16 * wave + lr) * kLd + 32 * kk + lk]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(&Hs[(16 * i + lr) * kLd + 32 * kk + lk]);
        accd[i] = mfma(av, bv, accd[i]);
      }
    }
    __syncthreads();
  }
  {
    const int col = 16 * wave + lr;
    float sc = col < rk ? bf16_to_f32(sd[col]) : 0.f;
    if (Q8 && col < rk) sc *= a.u_down_scale[(int64_t)e * rk + col];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        Zd[(16 * i + 4 * (lane >> 4) + q) * kLd + col] = f32_to_bf16(accd[i][q] * sc);
  }
  __syncthreads();

  // ---- stage 4: y = zd V_down^T, 64 output columns per pass
  float* Y = a.y;
  // V_down fragments requested one 64-column pass ahead
  bf16x8 bvd[2];
  float vds = 1.f;
  auto load4 = [&](int n0) {
    const int n = n0 + 16 * wave + lr;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const bool ok = 32 * kk + lk < rk;
      if (!ok)
        bvd[kk] = bf16x8{};
      else if (Q8)
        bvd[kk] = cvt8_fp8_bf16(*reinterpret_cast<const u32x2*>(Vd8 + (int64_t)n * rk + 32 * kk + lk));
      else
        bvd[kk] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(Vd + (int64_t)n * rk + 32 * kk + lk));
    }
    if (Q8) vds = a.v_down_scale[(int64_t)e * d + n];
  };
  load4(0);
  for (int n0 = 0; n0 < d; n0 += 64) {
    floatx4 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
    const bf16x8 b0 = bvd[0], b1 = bvd[1];
    const float ys = vds;
    if (n0 + 64 < d) load4(n0 + 64);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const bf16x8 bv = kk ? b1 : b0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(&Zd[(16 * i + lr) * kLd + 32 * kk + lk]);
        acc[i] = mfma(av, bv, acc[i]);
      }
    }
    const int n = n0 + 16 * wave + lr;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = r0 + 16 * i + 4 * (lane >> 4) + q;
        if (row < r_end) Y[(int64_t)row * d + n] = Q8 ? acc[i][q] * ys : acc[i][q];
      }
  }
}

}  // namespace

hipError_t launch_lowrank(const LowRankArgs& a, hipStream_t s) {
  if (a.max_tiles <= 0) return hipSuccess;
  if (a.rank < 16 || a.rank > kR || a.rank % 16) return hipErrorInvalidValue;
  const dim3 grid((unsigned)a.max_tiles), block(256);
  if (a.fp8 && a.rank == kR)
    hipLaunchKernelGGL((lowrank_kernel<true, true>), grid, block, 0, s, a);
  else if (a.fp8)
    hipLaunchKernelGGL((lowrank_kernel<true, false>), grid, block, 0, s, a);
  else if (a.rank == kR)
    hipLaunchKernelGGL((lowrank_kernel<false, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((lowrank_kernel<false, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
