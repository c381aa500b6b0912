// Fused router for the fine-grained layers with few routed experts (E <= 64:
// 24 on the Quartz model card, 32 on the Moonfrost MoE card, 48 on the
// Sutra-1.3B card), bf16 inputs.
//
// One workgroup per 16 tokens, four waves:
//   1. logits[16, 16 NS] = x[16, d] W_r with v_mfma_f32_16x16x32_bf16, the
//      K dimension split into four contiguous ranges, one per wave. Each wave
//      copies the W_r rows of its range into its own LDS slice (direct-to-LDS
//      loads of the contiguous block when E % 4 == 0, row pitch E; else
//      element-wise into a padded [k][16 NS] layout), so no wave waits for
//      another before its MFMAs. The token rows are the A operand read from
//      memory, a wave's fragments requested together; the B operand comes
//      from LDS through ds_read_b64_tr_b16 (within a 16-lane group, output
//      lane j receives element i from the address of source lane 4i + j/4,
//      so source lane s points at row k0 + s/4, columns n0 + 4 (s%4)).
//   2. The four partial sums meet in LDS and are added in wave order, plus
//      logit_bias. Wave w then scores tokens 4w .. 4w+3, one per 16-lane DPP
//      row, lane l holding experts 16 j + l%16.
//   3. Top-(k+1) by k+1 rounds of a row-wide maximum of (key, id) packed so
//      that equal keys resolve to the lower expert id, the winner's entry
//      removed after each round; gates and routing probabilities with sums
//      over the row in a fixed order.
//   4. The workgroup's per-expert slot counts and probability sums, summed
//      over its rows and waves in a fixed order.
#include <float.h>
#include <math.h>

#include "moe_device.h"
#include "moe_internal.h"


namespace moe {
namespace {

constexpr int kWaves = 4;
constexpr int kTB = kRouteBlockSmall;    // tokens per workgroup
static_assert(kTB == 16, "one MFMA row block per workgroup");
constexpr int kWsPerNs = 8 * 1024;        // LDS per wave slice of W_r rows, per 16 experts
constexpr int kWsPad = 256;               // reads of padding columns past a slice's last row
constexpr int XB = 16;                    // k steps of token-row fragments in flight

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef short shortx8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ uint64_t row_max_u64(uint64_t v) {
  v = max_u64(v, dpp_u64<kDppQuadXor1>(v));
  v = max_u64(v, dpp_u64<kDppQuadXor2>(v));
  v = max_u64(v, dpp_u64<kDppRowHalfMirror>(v));
  v = max_u64(v, dpp_u64<kDppRowMirror>(v));
  return v;
}
__device__ __forceinline__ float row_sum(float v) {
  v += dpp_f32<kDppQuadXor1>(v);
  v += dpp_f32<kDppQuadXor2>(v);
  v += dpp_f32<kDppRowHalfMirror>(v);
  v += dpp_f32<kDppRowMirror>(v);
  return v;
}
__device__ __forceinline__ float sigmoid_f32(float z) { return 1.0f / (1.0f + __expf(-z)); }

template <int NS, int KMAX, bool DMA>
__global__ void __launch_bounds__(256) route_small_kernel(RouteSmallArgs a) {
  constexpr int EP = 16 * NS;
  constexpr int ws_slice = kWsPerNs * NS;
  __shared__ __attribute__((aligned(16))) unsigned char s_w[kWaves][ws_slice + kWsPad];
  __shared__ float s_part[kWaves * kTB * (EP + 1)];   // [wave][token][expert] partial logits
  __shared__ float s_ps[kWaves][EP];
  __shared__ int s_ct[kWaves][EP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, d = a.d, k = a.k;
  const int pitch = DMA ? E : EP;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * kTB;
  const bf16_t* x = static_cast<const bf16_t*>(a.x);
  const bf16_t* W = static_cast<const bf16_t*>(a.w_router);
  const bf16_t* xr = x + min(t0 + l16, a.T - 1) * d + 8 * g;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  unsigned char* Ws = s_w[wave_u];
  const uint32_t ws_base =
      (uint32_t)(uintptr_t)((__attribute__((address_space(3))) unsigned char*)Ws);

  // this wave's k steps: [s_lo, s_hi) of d / 32
  const int ns = d / 32;
  const int s_lo = wave * ns / kWaves, s_hi = (wave + 1) * ns / kWaves;
  const int KC = ws_slice / (64 * pitch);   // k steps per LDS chunk (>= 8)

  floatx4 acc[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
  bf16x8 xf[XB];

  for (int c0 = s_lo; c0 < s_hi; c0 += KC) {
    const int cn = min(KC, s_hi - c0);
    // stage rows [32 c0, 32 (c0 + cn)) of W_r in this wave's slice
    if (DMA) {
      const unsigned char* src = reinterpret_cast<const unsigned char*>(W + (int64_t)32 * c0 * E);
      const int nbytes = 32 * cn * E * 2;
      for (int off = 0; off < nbytes; off += 1024)
        if (off + 16 * lane < nbytes) dma16(src + off + 16 * lane, ws_base + off);
    } else {
      bf16_t* wl = reinterpret_cast<bf16_t*>(Ws);
      for (int i = lane; i < 32 * cn * E; i += 64) {
        const int kk = i / E, e = i - kk * E;
        wl[kk * EP + e] = W[(int64_t)(32 * c0 + kk) * E + e];
      }
    }
    for (int b0 = 0; b0 < cn; b0 += XB) {
      const int bn = min(XB, cn - b0);
#pragma unroll
      for (int u = 0; u < XB; ++u)
        xf[u] = *reinterpret_cast<const bf16x8*>(xr + 32 * (c0 + b0 + min(u, bn - 1)));
      __builtin_amdgcn_s_waitcnt(0);   // W slice and fragments landed (this wave only)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < XB; ++u) {
        if (u >= bn) break;
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          const int kk = 32 * (b0 + u) + 8 * g + (l16 >> 2);
          const int col = 16 * j + 4 * (l16 & 3);
          const unsigned char* p0 = Ws + 2 * (kk * pitch + col);
          const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) shortx4*)p0);
          const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) shortx4*)(p0 + 8 * pitch));
          const shortx8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[u], __builtin_bit_cast(bf16x8, v),
                                                           acc[j], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // partial logits of this wave: token row 4 g + i, expert 16 j + l16
#pragma unroll
  for (int j = 0; j < NS; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) s_part[(wave * kTB + 4 * g + i) * (EP + 1) + 16 * j + l16] = acc[j][i];
  __syncthreads();

  // ---- wave w scores tokens 4 w + g (one per 16-lane row); lane holds experts 16 j + l16
  const int tk = 4 * wave + g;
  const int64_t t = t0 + tk;
  const bool tval = t < a.T;
  const bool sig = a.score == MOE_SIGMOID;
  float key[NS], lg[NS];
  int eid[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    eid[j] = 16 * j + l16;
    const bool ve = eid[j] < E;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) v += s_part[(w * kTB + tk) * (EP + 1) + eid[j]];
    if (ve && a.logit_bias) v += a.logit_bias[eid[j]];
    lg[j] = v;
    const float sb = ve && sig && a.select_bias ? a.select_bias[eid[j]] : 0.f;
    key[j] = !ve ? -INFINITY : (sig ? sigmoid_f32(v) + sb : v);
  }
  const int rounds = min(k + 1, E);
  uint64_t sel[KMAX];
#pragma unroll
  for (int r = 0; r < KMAX; ++r) sel[r] = 0;
#pragma unroll
  for (int r = 0; r < KMAX; ++r) {
    if (r >= rounds) break;
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < NS; ++j) best = max_u64(best, pack_key_id(key[j], eid[j]));
    best = row_max_u64(best);
    sel[r] = best;
    const int id = packed_id(best);
#pragma unroll
    for (int j = 0; j < NS; ++j)
      if (eid[j] == id) key[j] = -INFINITY;
  }

  float gate[KMAX], prob[NS];
  float tot = 0.f;
  if (!sig) {
    const float m = packed_key(sel[0]);
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      prob[j] = eid[j] < E ? __expf(lg[j] - m) : 0.f;
      tot += prob[j];
    }
    tot = row_sum(tot);
    float ssel = 0.f;
#pragma unroll
    for (int r = 0; r < KMAX; ++r) {
      gate[r] = r < k ? __expf(packed_key(sel[r]) - m) : 0.f;
      ssel += gate[r];
    }
    const float den = a.renorm ? ssel : tot;
#pragma unroll
    for (int r = 0; r < KMAX; ++r) gate[r] /= den;
  } else {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      prob[j] = eid[j] < E ? sigmoid_f32(lg[j]) : 0.f;
      tot += prob[j];
    }
    tot = row_sum(tot);
    float ssel = 0.f;
#pragma unroll
    for (int r = 0; r < KMAX; ++r) {
      float s = 0.f;
      if (r < k) {
        const int id = packed_id(sel[r]);
#pragma unroll
        for (int j = 0; j < NS; ++j) s += eid[j] == id ? prob[j] : 0.f;
        s = row_sum(s);
      }
      gate[r] = s;
      ssel += s;
    }
#pragma unroll
    for (int r = 0; r < KMAX; ++r) gate[r] /= ssel;
  }
  const float inv = 1.0f / tot;
#pragma unroll
  for (int j = 0; j < NS; ++j) prob[j] = tval ? prob[j] * inv : 0.f;

  if (tval) {
#pragma unroll
    for (int r = 0; r < KMAX; ++r) {
      if (r < k && l16 == r) {
        a.topk_idx[t * k + r] = packed_id(sel[r]);
        a.topk_gate[t * k + r] = gate[r];
      }
    }
    if (a.topk_margin && l16 == 15) {
      float mg = INFINITY;
#pragma unroll
      for (int r = 1; r < KMAX; ++r)
        if (r == k && k < E) mg = packed_key(sel[r - 1]) - packed_key(sel[r]);
      a.topk_margin[t] = mg;
    }
  }
  // block statistics: the wave's 4 tokens (rows), then the waves in order
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    int cnt = 0;
    if (tval) {
#pragma unroll
      for (int r = 0; r < KMAX; ++r)
        if (r < k && packed_id(sel[r]) == eid[j]) ++cnt;
    }
    float ps = prob[j];
    cnt += __shfl_xor(cnt, 16, 64);
    cnt += __shfl_xor(cnt, 32, 64);
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    if (g == 0) {
      s_ct[wave][eid[j]] = cnt;
      s_ps[wave][eid[j]] = ps;
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) {
    int c = 0;
    float p = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      c += s_ct[w][e];
      p += s_ps[w][e];
    }
    a.blk_counts[(int64_t)blockIdx.x * E + e] = c;
    a.blk_psum[(int64_t)blockIdx.x * E + e] = p;
  }
}

}  // namespace

hipError_t launch_route_small(const RouteSmallArgs& a, hipStream_t s) {
  const int64_t nblk = (a.T + kTB - 1) / kTB;
  if (nblk == 0) return hipSuccess;
  if (a.E > kRouteSmallMaxE || a.k + 1 > 16 || a.d % 32) return hipErrorInvalidValue;
  const int ns = (a.E + 15) / 16;
  const int k1 = a.k + 1;
  const bool dma = a.E % 4 == 0;
#define MOE_RS(NSV, KM)                                                                      \
  do {                                                                                       \
    if (dma)                                                                                 \
      hipLaunchKernelGGL((route_small_kernel<NSV, KM, true>), dim3((unsigned)nblk), dim3(256), \
                         0, s, a);                                                           \
    else                                                                                     \
      hipLaunchKernelGGL((route_small_kernel<NSV, KM, false>), dim3((unsigned)nblk), dim3(256), \
                         0, s, a);                                                           \
  } while (0)
#define MOE_RS_K(NSV)                 \
  do {                                \
    if (k1 <= 4) MOE_RS(NSV, 4);      \
    else if (k1 <= 8) MOE_RS(NSV, 8); \
    else MOE_RS(NSV, 16);             \
  } while (0)
  switch (ns) {
    case 1: MOE_RS_K(1); break;
    case 2: MOE_RS_K(2); break;
    case 3: MOE_RS_K(3); break;
    default: MOE_RS_K(4); break;
  }
#undef MOE_RS_K
#undef MOE_RS
  return hipGetLastError();
}

}  // namespace moe
