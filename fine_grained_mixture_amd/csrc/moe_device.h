// Device-side helpers for the MoE kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;  // raw bf16 bits in memory

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// float32 -> bf16, round to nearest even (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ float load_elem(const float* p) { return *p; }
__device__ __forceinline__ float load_elem(const bf16_t* p) { return bf16_to_f32(*p); }

__device__ __forceinline__ void store_elem(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_elem(bf16_t* p, float v) { *p = f32_to_bf16(v); }

// SiLU(z) = z * sigmoid(z), with the hardware reciprocal (v_rcp_f32).
__device__ __forceinline__ float silu_f32(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// Monotone map of a float onto uint32 (larger float -> larger integer); -0
// maps as +0, so that the two zeros compare equal, as floats do.
__device__ __forceinline__ uint32_t float_orderable(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float orderable_float(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
  return __uint_as_float(u);
}

// (key, id) packed into one integer: a larger packed value means a larger key,
// and among equal keys the lower expert id.
__device__ __forceinline__ uint64_t pack_key_id(float key, int id) {
  return (static_cast<uint64_t>(float_orderable(key)) << 32) |
         static_cast<uint64_t>(0xffffffffu - static_cast<uint32_t>(id));
}
__device__ __forceinline__ int packed_id(uint64_t p) {
  return static_cast<int>(0xffffffffu - static_cast<uint32_t>(p & 0xffffffffu));
}
__device__ __forceinline__ float packed_key(uint64_t p) {
  return orderable_float(static_cast<uint32_t>(p >> 32));
}

// Intra-row (16-lane) exchanges on the DPP path: after the quad_perm steps a
// quad holds one value, row_half_mirror pairs quad q with quad 1 - q of each
// 8, row_mirror pairs the two 8-lane halves of each row.
constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = dpp_u32<CTRL>(static_cast<uint32_t>(v));
  const uint32_t hi = dpp_u32<CTRL>(static_cast<uint32_t>(v >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Sums and maxima: every lane ends with the same value, combined in a fixed
// order, so the result does not depend on scheduling.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<kDppQuadXor1>(v);
  v += dpp_f32<kDppQuadXor2>(v);
  v += dpp_f32<kDppRowHalfMirror>(v);
  v += dpp_f32<kDppRowMirror>(v);
  v += __shfl_xor(v, 16, kWave);
  v += __shfl_xor(v, 32, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_f32<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_f32<kDppRowHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kDppRowMirror>(v));
  v = fmaxf(v, __shfl_xor(v, 16, kWave));
  v = fmaxf(v, __shfl_xor(v, 32, kWave));
  return v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Inclusive prefix sums over the 64 lanes of a wave in lane order, on the DPP
// path (no LDS round trips): row_shr:1, 2, 4, 8 scan each row of 16 lanes,
// then row_bcast:15 adds row 0's total to row 1 and row 2's to row 3
// (row_mask 0xA), and row_bcast:31 adds lane 31's running total to rows 2 and
// 3 (row_mask 0xC). Lanes whose DPP source does not exist, and rows the mask
// leaves out, add 0. The additions run in one fixed order.
constexpr int kDppRowShr1 = 0x111;
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_or0_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_or0_f64(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, ROW_MASK,
                                                            0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL,
                                                            ROW_MASK, 0xF, false);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ int wave_incl_scan_i32(int v) {
  v += dpp_or0_i32<kDppRowShr1, 0xF>(v);
  v += dpp_or0_i32<kDppRowShr2, 0xF>(v);
  v += dpp_or0_i32<kDppRowShr4, 0xF>(v);
  v += dpp_or0_i32<kDppRowShr8, 0xF>(v);
  v += dpp_or0_i32<kDppRowBcast15, 0xA>(v);
  v += dpp_or0_i32<kDppRowBcast31, 0xC>(v);
  return v;
}
__device__ __forceinline__ double wave_incl_scan_f64(double v) {
  v += dpp_or0_f64<kDppRowShr1, 0xF>(v);
  v += dpp_or0_f64<kDppRowShr2, 0xF>(v);
  v += dpp_or0_f64<kDppRowShr4, 0xF>(v);
  v += dpp_or0_f64<kDppRowShr8, 0xF>(v);
  v += dpp_or0_f64<kDppRowBcast15, 0xA>(v);
  v += dpp_or0_f64<kDppRowBcast31, 0xC>(v);
  return v;
}
// lane 63's value in every lane (a scalar read)
__device__ __forceinline__ int lane63_i32(int v) { return __builtin_amdgcn_readlane(v, 63); }
__device__ __forceinline__ double lane63_f64(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), 63);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Bits of a wave ballot below this lane.
__device__ __forceinline__ uint64_t lanemask_lt() {
  int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

}  // namespace moe
