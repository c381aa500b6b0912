// Element-wise and per-token parts of the layer backward on gfx950.
//
// combine_bwd_kernel: the gradient of the gate-weighted combine. For token t
//   and kept slot j (row = row_of_slot[t, j]) the routed expert output was
//   weighted by gate[t, j], so its upstream rows are gate * dy[t] (rounded to
//   bf16, the operand of the expert products) and the gate's gradient is the
//   dot product of dy[t] with that expert's output row. One wave per token,
//   16-byte pieces of dy per lane, the k dot products reduced across the wave
//   in a fixed order. The token's row is also copied to its slots' rows of
//   x_perm, the row order of the weight-gradient products.
// router_bwd_kernel: the gradient of the router logits. The top-k choice and
//   the slot counts are held fixed; the gates depend on the logits through the
//   softmax (renormalised over the selected experts or not) or through the
//   sigmoid scores divided by their selected sum, and the aux statistic
//   depends on them through the per-expert mean routing probability P.
// dx_gather_kernel: the input gradient of a token, summed in a fixed order
//   from its router part, its shared-expert part and its kept slots' rows.
// reduce_chunks_kernel: fixed-order sums of split-K partial products.

#include <type_traits>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kWaves = 4;

__device__ __forceinline__ u32x2 pack_bf16x4(float a, float b, float c, float d) {
  u32x2 p;
  p[0] = (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
  p[1] = (uint32_t)f32_to_bf16(c) | ((uint32_t)f32_to_bf16(d) << 16);
  return p;
}

template <int KMAX, bool F32>
__global__ void __launch_bounds__(256) combine_bwd_kernel(CombineBwdArgs a) {
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int d4 = a.d >> 2;
  const int k = a.k;
  const int64_t nw = (int64_t)gridDim.x * kWaves;
  const floatx4* yr = reinterpret_cast<const floatx4*>(a.y_routed);
  for (int64_t t = (int64_t)blockIdx.x * kWaves + wave; t < a.T; t += nw) {
    int my_row = -1;
    float my_gate = 0.f;
    if (lane < k) {
      my_row = a.row_of_slot[t * k + lane];
      my_gate = a.topk_gate[t * k + lane];
    }
    int row[KMAX];
    bool kept[KMAX];
    float gate[KMAX], part[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      const int r = __builtin_amdgcn_readlane(my_row, j);
      kept[j] = j < k && r >= 0;
      row[j] = max(r, 0);
      gate[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_gate), j));
      part[j] = 0.f;
    }
    const floatx4* dyt = reinterpret_cast<const floatx4*>(a.dy + t * a.d);
    // activation-type rows: 4 values are 8 bytes (bf16) or 16 (float32)
    typedef typename std::conditional<F32, floatx4, u32x2>::type act4;
    const act4* xt = static_cast<const act4*>(a.x) + t * d4;
    act4* xp = static_cast<act4*>(a.x_perm);
    act4* dyr = static_cast<act4*>(a.dy_routed);
    for (int c = lane; c < d4; c += 64) {
      const floatx4 g = dyt[c];
      act4 xv{};
      if (xp) xv = xt[c];
      floatx4 v[KMAX];
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (kept[j]) v[j] = yr[(int64_t)row[j] * d4 + c];
      if (xp) {
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
          if (kept[j]) xp[(int64_t)row[j] * d4 + c] = xv;
      }
      if (!F32 && a.dy_shared)
        reinterpret_cast<u32x2*>(a.dy_shared + t * a.d)[c] = pack_bf16x4(g[0], g[1], g[2], g[3]);
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (kept[j]) {
          part[j] = fmaf(g[0], v[j][0], part[j]);
          part[j] = fmaf(g[1], v[j][1], part[j]);
          part[j] = fmaf(g[2], v[j][2], part[j]);
          part[j] = fmaf(g[3], v[j][3], part[j]);
          const floatx4 gy = {gate[j] * g[0], gate[j] * g[1], gate[j] * g[2], gate[j] * g[3]};
          if constexpr (F32) dyr[(int64_t)row[j] * d4 + c] = gy;
          else dyr[(int64_t)row[j] * d4 + c] = pack_bf16x4(gy[0], gy[1], gy[2], gy[3]);
        }
      }
    }
    float mine = 0.f;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j < k) {
        const float sj = wave_sum(part[j]);
        if (lane == j) mine = kept[j] ? sj : 0.f;
      }
    }
    if (lane < k) a.dgate[t * k + lane] = mine;
  }
}

__device__ __forceinline__ void store_dl(void* dl, int64_t i, float v, bool f32) {
  if (f32) static_cast<float*>(dl)[i] = v;
  else static_cast<uint16_t*>(dl)[i] = f32_to_bf16(v);
}

// One wave per token; lane e (+ 64 c) holds expert e's logit.
__global__ void __launch_bounds__(256) router_bwd_kernel(RouterBwdArgs a) {
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int E = a.E, k = a.k;
  const int64_t nw = (int64_t)gridDim.x * kWaves;
  const float inv_tk = 1.0f / ((float)a.T * (float)k);
  for (int64_t t = (int64_t)blockIdx.x * kWaves + wave; t < a.T; t += nw) {
    const float* lt = a.logits + t * E;
    // slot data on lanes j < k
    int sel = -1;
    float g = 0.f, dg = 0.f, lsel = 0.f;
    if (lane < k) {
      sel = a.topk_idx[t * k + lane];
      g = a.topk_gate[t * k + lane];
      dg = a.dgate[t * k + lane];
      lsel = lt[sel];
    }
    // full-distribution statistics
    float mx = -__builtin_huge_valf();
    for (int e = lane; e < E; e += 64) mx = fmaxf(mx, lt[e]);
    mx = wave_max(mx);
    float z = 0.f, fz = 0.f;   // softmax: sum exp, sum f exp; sigmoid: sum s, sum f s
    for (int e = lane; e < E; e += 64) {
      const float l = lt[e];
      const float w = a.score == MOE_SIGMOID ? __builtin_amdgcn_rcpf(1.0f + __expf(-l))
                                             : __expf(l - mx);
      const float f = (float)a.counts[e] * inv_tk;
      z += w;
      fz = fmaf(f, w, fz);
    }
    z = wave_sum(z);
    fz = wave_sum(fz);
    const float fbar = fz / z;   // sum_e f_e prob_e
    // per-slot terms
    float vsel = 0.f;   // added at e = sel_j
    float dense = 0.f;  // softmax without renormalisation: -sum_j p_sel_j dg_j
    if (a.score == MOE_SIGMOID) {
      const float st = lane < k ? __builtin_amdgcn_rcpf(1.0f + __expf(-lsel)) : 0.f;
      const float ssel = wave_sum(st);
      const float gdg = wave_sum(lane < k ? g * dg : 0.f);
      vsel = lane < k ? (dg - gdg) / ssel * st * (1.0f - st) : 0.f;
    } else if (a.renorm) {
      const float gdg = wave_sum(lane < k ? g * dg : 0.f);
      vsel = lane < k ? g * (dg - gdg) : 0.f;
    } else {
      const float p = lane < k ? __expf(lsel - mx) / z : 0.f;
      dense = -wave_sum(p * dg);
      vsel = p * dg;
    }
    for (int e = lane; e < E; e += 64) {
      const float l = lt[e];
      float dl = 0.f;
      if (a.score == MOE_SIGMOID) {
        const float st = __builtin_amdgcn_rcpf(1.0f + __expf(-l));
        if (a.aux_scale != 0.f) {
          const float f = (float)a.counts[e] * inv_tk;
          dl = a.aux_scale * (f - fbar) / z * st * (1.0f - st);
        }
      } else {
        const float p = __expf(l - mx) / z;
        dl = p * dense;
        if (a.aux_scale != 0.f) {
          const float f = (float)a.counts[e] * inv_tk;
          dl = fmaf(a.aux_scale * p, f - fbar, dl);
        }
      }
      for (int j = 0; j < k; ++j) {
        const int sj = __builtin_amdgcn_readlane(sel, j);
        const float vj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(vsel), j));
        if (sj == e) dl += vj;
      }
      store_dl(a.dl, t * E + e, dl, a.f32_out);
    }
  }
}

// The same with each lane holding experts 4 (lane + 64 i) .. + 3, i < NV
// (E % 4 == 0, E <= 256 NV): the token's logits are read once, as 16-byte
// pieces, and stay in registers for the three passes; dl leaves as 8-byte
// pieces.
template <int NV>
__global__ void __launch_bounds__(256) router_bwd_vec_kernel(RouterBwdArgs a) {
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int E = a.E, k = a.k, E4 = a.E >> 2;
  const int64_t nw = (int64_t)gridDim.x * kWaves;
  const float inv_tk = 1.0f / ((float)a.T * (float)k);
  const bool sig = a.score == MOE_SIGMOID;
  floatx4 f[NV];   // the experts' slot fractions, the same for every token
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int idx = lane + 64 * i;
    f[i] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (idx < E4) {
#pragma unroll
      for (int q = 0; q < 4; ++q) f[i][q] = (float)a.counts[4 * idx + q] * inv_tk;
    }
  }
  for (int64_t t = (int64_t)blockIdx.x * kWaves + wave; t < a.T; t += nw) {
    const float* lt = a.logits + t * E;
    const floatx4* lt4 = reinterpret_cast<const floatx4*>(lt);
    floatx4 l[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = lane + 64 * i;
      l[i] = idx < E4 ? lt4[idx] : floatx4{0.f, 0.f, 0.f, 0.f};
    }
    int sel = -1;
    float g = 0.f, dg = 0.f, lsel = 0.f;
    if (lane < k) {
      sel = a.topk_idx[t * k + lane];
      g = a.topk_gate[t * k + lane];
      dg = a.dgate[t * k + lane];
      lsel = lt[sel];
    }
    float mx = -__builtin_huge_valf();
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (lane + 64 * i < E4) mx = fmaxf(fmaxf(fmaxf(mx, l[i][0]), fmaxf(l[i][1], l[i][2])), l[i][3]);
    mx = wave_max(mx);
    float z = 0.f, fz = 0.f;
    floatx4 w[NV];   // softmax: exp(l - max); sigmoid: the scores
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      w[i] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (lane + 64 * i < E4) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float v = sig ? __builtin_amdgcn_rcpf(1.0f + __expf(-l[i][q]))
                              : __expf(l[i][q] - mx);
          w[i][q] = v;
          z += v;
          fz = fmaf(f[i][q], v, fz);
        }
      }
    }
    z = wave_sum(z);
    fz = wave_sum(fz);
    const float fbar = fz / z;
    float vsel = 0.f, dense = 0.f;
    if (sig) {
      const float st = lane < k ? __builtin_amdgcn_rcpf(1.0f + __expf(-lsel)) : 0.f;
      const float ssel = wave_sum(st);
      const float gdg = wave_sum(lane < k ? g * dg : 0.f);
      vsel = lane < k ? (dg - gdg) / ssel * st * (1.0f - st) : 0.f;
    } else if (a.renorm) {
      const float gdg = wave_sum(lane < k ? g * dg : 0.f);
      vsel = lane < k ? g * (dg - gdg) : 0.f;
    } else {
      const float p = lane < k ? __expf(lsel - mx) / z : 0.f;
      dense = -wave_sum(p * dg);
      vsel = p * dg;
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = lane + 64 * i;
      if (idx >= E4) continue;
      float dl[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float v = 0.f;
        if (sig) {
          if (a.aux_scale != 0.f) {
            const float st = w[i][q];
            v = a.aux_scale * (f[i][q] - fbar) / z * st * (1.0f - st);
          }
        } else {
          const float p = w[i][q] / z;
          v = p * dense;
          if (a.aux_scale != 0.f) v = fmaf(a.aux_scale * p, f[i][q] - fbar, v);
        }
        dl[q] = v;
      }
      for (int j = 0; j < k; ++j) {
        const int sj = __builtin_amdgcn_readlane(sel, j);
        const float vj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(vsel), j));
        if ((sj >> 2) == idx) dl[sj & 3] += vj;
      }
      if (a.f32_out)
        reinterpret_cast<floatx4*>(static_cast<float*>(a.dl) + t * E)[idx] =
            floatx4{dl[0], dl[1], dl[2], dl[3]};
      else
        reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.dl) + t * E)[idx] =
            pack_bf16x4(dl[0], dl[1], dl[2], dl[3]);
    }
  }
}

template <int KMAX>
__global__ void __launch_bounds__(256) dx_gather_kernel(DxGatherArgs a) {
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int d4 = a.d >> 2;
  const int k = a.k;
  const int64_t nw = (int64_t)gridDim.x * kWaves;
  const floatx4* xr = reinterpret_cast<const floatx4*>(a.dx_rows);
  for (int64_t t = (int64_t)blockIdx.x * kWaves + wave; t < a.T; t += nw) {
    const int my_row = lane < k ? a.row_of_slot[t * k + lane] : -1;
    int row[KMAX];
    bool kept[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      const int r = __builtin_amdgcn_readlane(my_row, j);
      kept[j] = j < k && r >= 0;
      row[j] = max(r, 0);
    }
    floatx4* dxt = reinterpret_cast<floatx4*>(a.dx + t * a.d);
    const floatx4* dst = a.dx_shared ? reinterpret_cast<const floatx4*>(a.dx_shared + t * a.d)
                                     : nullptr;
    for (int c = lane; c < d4; c += 64) {
      floatx4 acc = dxt[c];
      floatx4 v[KMAX];
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (kept[j]) v[j] = xr[(int64_t)row[j] * d4 + c];
      if (dst) acc += dst[c];
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (kept[j]) acc += v[j];
      dxt[c] = acc;
    }
  }
}

__global__ void __launch_bounds__(256) reduce_chunks_kernel(const float* part, float* out,
                                                            int64_t groups, int64_t chunks,
                                                            int64_t n) {
  const int64_t n4 = n >> 2;
  const int64_t total = groups * n4;
  const floatx4* p = reinterpret_cast<const floatx4*>(part);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int64_t g = i / n4, e = i - g * n4;
    floatx4 acc = p[(g * chunks) * n4 + e];
    for (int64_t c = 1; c < chunks; ++c) acc += p[(g * chunks + c) * n4 + e];
    reinterpret_cast<floatx4*>(out)[i] = acc;
  }
}

unsigned wave_grid(int64_t T) {
  const int64_t waves = T < 8192 ? T : 8192;
  return (unsigned)((waves + kWaves - 1) / kWaves);
}

}  // namespace

hipError_t launch_combine_bwd(const CombineBwdArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.k < 1 || a.k > 16 || a.d % 4) return hipErrorInvalidValue;
  const unsigned grid = wave_grid(a.T);
#define MOE_CB(F32)                                                                       \
  do {                                                                                    \
    if (a.k <= 2) hipLaunchKernelGGL((combine_bwd_kernel<2, F32>), dim3(grid), dim3(256), 0, s, a); \
    else if (a.k <= 4) hipLaunchKernelGGL((combine_bwd_kernel<4, F32>), dim3(grid), dim3(256), 0, s, a); \
    else if (a.k <= 8) hipLaunchKernelGGL((combine_bwd_kernel<8, F32>), dim3(grid), dim3(256), 0, s, a); \
    else hipLaunchKernelGGL((combine_bwd_kernel<16, F32>), dim3(grid), dim3(256), 0, s, a); \
  } while (0)
  if (a.f32) MOE_CB(true);
  else MOE_CB(false);
#undef MOE_CB
  return hipGetLastError();
}

hipError_t launch_router_bwd(const RouterBwdArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.k < 1 || a.k > 64 || a.E < a.k) return hipErrorInvalidValue;
  // many experts: the register-resident variant (3x faster at E = 1024; at
  // E = 24 the plain one is faster)
  const bool vec = a.E >= 256 && a.E % 4 == 0 && a.E <= 4096 &&
                   reinterpret_cast<uintptr_t>(a.logits) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(a.dl) % 16 == 0;
  const dim3 grid(wave_grid(a.T)), block(256);
  if (!vec) hipLaunchKernelGGL(router_bwd_kernel, grid, block, 0, s, a);
  else if (a.E <= 512) hipLaunchKernelGGL(router_bwd_vec_kernel<2>, grid, block, 0, s, a);
  else if (a.E <= 1024) hipLaunchKernelGGL(router_bwd_vec_kernel<4>, grid, block, 0, s, a);
  else if (a.E <= 2048) hipLaunchKernelGGL(router_bwd_vec_kernel<8>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(router_bwd_vec_kernel<16>, grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dx_gather(const DxGatherArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.k < 1 || a.k > 16 || a.d % 4) return hipErrorInvalidValue;
  const unsigned grid = wave_grid(a.T);
  if (a.k <= 2) hipLaunchKernelGGL((dx_gather_kernel<2>), dim3(grid), dim3(256), 0, s, a);
  else if (a.k <= 4) hipLaunchKernelGGL((dx_gather_kernel<4>), dim3(grid), dim3(256), 0, s, a);
  else if (a.k <= 8) hipLaunchKernelGGL((dx_gather_kernel<8>), dim3(grid), dim3(256), 0, s, a);
  else hipLaunchKernelGGL((dx_gather_kernel<16>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_reduce_chunks(const float* part, float* out, int64_t groups, int64_t chunks,
                                int64_t n, hipStream_t s) {
  if (groups == 0 || n == 0) return hipSuccess;
  if (n % 4 || chunks < 1) return hipErrorInvalidValue;
  const int64_t total = groups * (n >> 2);
  const int64_t blocks = (total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096;
  hipLaunchKernelGGL(reduce_chunks_kernel, dim3((unsigned)blocks), dim3(256), 0, s, part, out,
                     groups, chunks, n);
  return hipGetLastError();
}

}  // namespace moe
