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
//   3. Top-(k+1) of the (key, id) pairs, packed so that equal keys resolve to
//      the lower expert id: with one group per workgroup, each pair's place
//      among the token's pairs, counted at once; with several, k+1 rounds of
//      a row-wide maximum, the winner's entry removed after each round. Gates
//      and routing probabilities with sums over the row in a fixed order.
//   4. The workgroup's per-expert slot counts and probability sums, summed
//      over its rows and waves in a fixed order.
#include <float.h>
#include <math.h>

#include "moe_device.h"
#include "moe_internal.h"
#include "route_tail.h"

#include <algorithm>


namespace moe {
namespace {

constexpr int kWaves = 4;
constexpr int kTB = kRouteBlockSmall;    // tokens per group
static_assert(kTB == 16, "one MFMA row block per group");
constexpr int kWsPad = 256;               // reads of padding columns past a slice's last row
constexpr int XB = 16;                    // k steps of token-row fragments in flight

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef short shortx8 __attribute__((ext_vector_type(8)));

// Direct-to-LDS 16-byte load (lane L writes LDS base + 16 L), as asm so that
// the compiler adds no waits for it. m0 is a reserved register, so its clobber
// is not honoured; the compiler uses m0 nowhere else here (a CPU test checks).
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

// LDS of the kernel: four W_r slices (one per wave), the partial logits and
// the per-wave block statistics, filling the 160 KiB of a CU.
template <int NS>
constexpr int part_bytes() { return kWaves * kTB * (16 * NS + 1) * 4; }
template <int NS>
constexpr int stat_bytes() { return 2 * kWaves * 16 * NS * 4; }
template <int NS>
constexpr int slice_bytes() {
  return ((160 * 1024 - part_bytes<NS>() - stat_bytes<NS>()) / kWaves - kWsPad) & ~1023;
}

// RES: every wave's K range fits its LDS slice and the fragment registers, so
// W_r is staged once and each group only loads token rows.
template <int NS, int KMAX, bool DMA, bool RES>
__global__ void __launch_bounds__(256) route_small_kernel(RouteSmallArgs a, int groups,
                                                          ScanArgs sa, RankArgs ra) {
  constexpr int EP = 16 * NS;
  constexpr int ws_slice = slice_bytes<NS>();
  __shared__ __attribute__((aligned(16))) unsigned char s_w[kWaves][ws_slice + kWsPad];
  // [wave][token][expert] partial logits; after a group's logits are summed,
  // each wave's slice holds its top-k exchange (4 tokens' pairs and picks)
  __shared__ __attribute__((aligned(16))) float s_part[kWaves * kTB * (EP + 1)];
  static_assert(4 * (EP + KMAX) * 8 <= kTB * (EP + 1) * 4, "top-k exchange fits a slice");
  __shared__ float s_ps[kWaves][EP];
  __shared__ int s_ct[kWaves][EP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, d = a.d, k = a.k;
  const int pitch = DMA ? E : EP;
  const int l16 = lane & 15, g = lane >> 4;
  const bf16_t* x = static_cast<const bf16_t*>(a.x);
  const bf16_t* W = static_cast<const bf16_t*>(a.w_router);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  unsigned char* Ws = s_w[wave_u];
  const uint32_t ws_base =
      (uint32_t)(uintptr_t)((__attribute__((address_space(3))) unsigned char*)Ws);
  const bool sig = a.score == MOE_SIGMOID;

  // this wave's k steps: [s_lo, s_hi) of d / 32; KC of them fit in its slice
  const int ns = d / 32;
  const int s_lo = wave * ns / kWaves, s_hi = (wave + 1) * ns / kWaves;
  const int KC = ws_slice / (64 * pitch);

  // copies W_r rows [32 c0, 32 (c0 + cn)) into this wave's slice
  auto stage = [&](int c0, int cn) {
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
  };
  bf16x8 xf[XB];
  // token-row fragments of steps [c0 + b0, c0 + b0 + bn), all requested at once
  auto load_x = [&](const bf16_t* xr, int c0b0, int bn) {
#pragma unroll
    for (int u = 0; u < XB; ++u)
      if (u < bn) xf[u] = *reinterpret_cast<const bf16x8*>(xr + 32 * (c0b0 + u));
  };
  // MFMAs of bn steps whose B rows start at row kl0 of the slice (a guarded
  // body rather than an early exit, so that xf stays in registers)
  auto mfma = [&](floatx4* acc, int kl0, int bn) {
#pragma unroll
    for (int u = 0; u < XB; ++u) {
      if (u < bn) {
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          const int kk = kl0 + 32 * u + 8 * g + (l16 >> 2);
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
    }
  };

  const int64_t blk_t0 = (int64_t)blockIdx.x * groups * kTB;
  auto x_row = [&](int64_t t0) { return x + min(t0 + l16, a.T - 1) * d + 8 * g; };
  if (RES) {
    // the whole K range of the wave stays in LDS for every group
    load_x(x_row(blk_t0), s_lo, s_hi - s_lo);
    stage(s_lo, s_hi - s_lo);
  }
  // block statistics of this lane's expert slots, accumulated over the groups
  int st_cnt[NS];
  float st_ps[NS];
  int eid[NS];
  float lbias[NS], sbias[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    st_cnt[j] = 0;
    st_ps[j] = 0.f;
    eid[j] = 16 * j + l16;
    const bool ve = eid[j] < E;
    lbias[j] = ve && a.logit_bias ? a.logit_bias[eid[j]] : 0.f;
    sbias[j] = ve && sig && a.select_bias ? a.select_bias[eid[j]] : 0.f;
  }
  // A group's outputs are stored after the next group's fragments have
  // landed: stores count in vmcnt, so storing before that wait would make it
  // wait for them too. Lane l16 holds selection l16 (< k) of its row's token.
  int64_t out_t = -1;
  int out_idx = 0;
  float out_gate = 0.f, out_margin = 0.f;
  float out_lg[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) out_lg[j] = 0.f;
  auto store_out = [&]() {
    if (out_t >= 0) {
      if (l16 < k) {
        a.topk_idx[out_t * k + l16] = out_idx;
        a.topk_gate[out_t * k + l16] = out_gate;
      }
      if (a.topk_margin && l16 == 15) a.topk_margin[out_t] = out_margin;
      if (a.logits) {
#pragma unroll
        for (int j = 0; j < NS; ++j)
          if (eid[j] < E) a.logits[out_t * E + eid[j]] = out_lg[j];
      }
    }
  };

  for (int grp = 0; grp < groups; ++grp) {
    const int64_t t0 = blk_t0 + (int64_t)grp * kTB;
    if (t0 >= a.T) break;
    const bf16_t* xr = x_row(t0);
    floatx4 acc[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (RES) {
      __builtin_amdgcn_s_waitcnt(0);   // slice (first group) and fragments landed
      __builtin_amdgcn_sched_barrier(0);
      store_out();
      mfma(acc, 0, s_hi - s_lo);
      __builtin_amdgcn_sched_barrier(0);
    } else {
      store_out();
      for (int c0 = s_lo; c0 < s_hi; c0 += KC) {
        const int cn = min(KC, s_hi - c0);
        stage(c0, cn);
        for (int b0 = 0; b0 < cn; b0 += XB) {
          const int bn = min(XB, cn - b0);
          load_x(xr, c0 + b0, bn);
          __builtin_amdgcn_s_waitcnt(0);   // slice chunk and fragments landed
          __builtin_amdgcn_sched_barrier(0);
          mfma(acc, 32 * b0, bn);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    // partial logits of this wave: token row 4 g + i, expert 16 j + l16
#pragma unroll
    for (int j = 0; j < NS; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        s_part[(wave * kTB + 4 * g + i) * (EP + 1) + 16 * j + l16] = acc[j][i];
    // next group's fragments travel while this group is scored (rows are
    // clamped to the last token, so a load past the batch's end is a harmless
    // re-read; the launch's last group loads nothing, and the branch is
    // uniform, so the loads still go out back to back)
    if (RES && grp + 1 < groups) {
      __builtin_amdgcn_sched_barrier(0);
      load_x(x_row(t0 + kTB), s_lo, s_hi - s_lo);
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();

    // ---- wave w scores tokens 4 w + g (one per 16-lane row); lane holds experts 16 j + l16
    const int tk = 4 * wave + g;
    const int64_t t = t0 + tk;
    const bool tval = t < a.T;
    float key[NS], lg[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const bool ve = eid[j] < E;
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) v += s_part[(w * kTB + tk) * (EP + 1) + eid[j]];
      v += lbias[j];
      lg[j] = v;
      key[j] = !ve ? -INFINITY : (sig ? sigmoid_f32(v) + sbias[j] : v);
    }
    __syncthreads();   // s_part is free for the next group

    // Top-(k+1). One group per workgroup (the chain of one group is the
    // launch's latency): each (key, id) pair's place among the token's
    // pairs, all counted at once. The row's pairs go through this wave's own
    // slice of s_part (no other wave touches it until this wave's next
    // partials); LDS operations of one wave run in order. Unused slots hold 0,
    // below every pair. Several groups (throughput): k + 1 rounds of a
    // row-wide maximum, the winner removed after each; fewer instructions.
    // Either way sel[r] is the r-th largest pair for r < rounds, else 0.
    const int rounds = min(k + 1, E);
    uint64_t sel[KMAX];
    if (groups == 1) {
      uint64_t pk[NS];
#pragma unroll
      for (int j = 0; j < NS; ++j) pk[j] = eid[j] < E ? pack_key_id(key[j], eid[j]) : 0;
      uint64_t* s_pk = reinterpret_cast<uint64_t*>(s_part + wave * kTB * (EP + 1)) + g * EP;
      uint64_t* s_sel = reinterpret_cast<uint64_t*>(s_part + wave * kTB * (EP + 1)) + 4 * EP +
                        g * KMAX;
#pragma unroll
      for (int j = 0; j < NS; ++j) s_pk[16 * j + l16] = pk[j];
      __builtin_amdgcn_wave_barrier();
      int place[NS];
#pragma unroll
      for (int j = 0; j < NS; ++j) place[j] = 0;
#pragma unroll
      for (int q = 0; q < EP; q += 2) {
        const uint64_t v0 = s_pk[q], v1 = s_pk[q + 1];
#pragma unroll
        for (int j = 0; j < NS; ++j) place[j] += (v0 > pk[j]) + (v1 > pk[j]);
      }
#pragma unroll
      for (int r = 0; r < KMAX; ++r) s_sel[r] = 0;
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int j = 0; j < NS; ++j)
        if (eid[j] < E && place[j] < rounds) s_sel[place[j]] = pk[j];
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int r = 0; r < KMAX; ++r) sel[r] = s_sel[r];
    } else {
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
      // sigmoid score of each selected expert, taken from the lane holding it
      float ssel = 0.f;
#pragma unroll
      for (int r = 0; r < KMAX; ++r) {
        float sc = 0.f;
        if (r < k) {
          const int id = packed_id(sel[r]);
#pragma unroll
          for (int j = 0; j < NS; ++j) sc += eid[j] == id ? prob[j] : 0.f;
          sc = row_sum(sc);   // one non-zero term
        }
        gate[r] = sc;
        ssel += sc;
      }
#pragma unroll
      for (int r = 0; r < KMAX; ++r) gate[r] /= ssel;
    }
    const float inv = 1.0f / tot;

    out_t = tval ? t : -1;
#pragma unroll
    for (int j = 0; j < NS; ++j) out_lg[j] = lg[j];
#pragma unroll
    for (int r = 0; r < KMAX; ++r) {
      if (l16 == r) {
        out_idx = packed_id(sel[r]);
        out_gate = gate[r];
      }
    }
    out_margin = INFINITY;
#pragma unroll
    for (int r = 1; r < KMAX; ++r)
      if (r == k && k < E) out_margin = packed_key(sel[r - 1]) - packed_key(sel[r]);
    if (tval) {
#pragma unroll
      for (int j = 0; j < NS; ++j) {
#pragma unroll
        for (int r = 0; r < KMAX; ++r)
          if (r < k && packed_id(sel[r]) == eid[j]) ++st_cnt[j];
        st_ps[j] += prob[j] * inv;
      }
    }
  }

  store_out();

  // ---- block statistics: the wave's rows in a fixed pairing order, then the
  // waves in order
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    int cnt = st_cnt[j];
    float ps = st_ps[j];
    cnt += __shfl_xor(cnt, 16, 64);
    cnt += __shfl_xor(cnt, 32, 64);
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    if (g == 0) {
      s_ct[wave][16 * j + l16] = cnt;
      s_ps[wave][16 * j + l16] = ps;
    }
  }
  __syncthreads();
  // E <= 64: thread e (a lane of wave 0) holds expert e's totals
  int c = 0;
  float p = 0.f;
  if (tid < E) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      c += s_ct[w][tid];
      p += s_ps[w][tid];
    }
    a.blk_counts[(int64_t)blockIdx.x * E + tid] = c;
    a.blk_psum[(int64_t)blockIdx.x * E + tid] = p;
  }

  // One routing block for the whole batch (the layer call, T <= 16 G): this
  // workgroup holds everything the scan and the rank need, so wave 0 writes
  // the per-expert outputs and ranks the block here instead of in a second
  // launch. The block's expert ids were stored before the barrier above.
  if (sa.E > 0 && wave == 0) {
    __shared__ int s_cnt0[64], s_off0[64];
    const int excl = scan_outputs(sa, c, p);
    s_cnt0[lane] = 0;   // no earlier blocks
    s_off0[lane] = excl;
    __builtin_amdgcn_wave_barrier();
    BlockIds B;
    load_block_ids(ra, 0, B);
    rank_block(ra, 0, B, s_cnt0, s_off0);
  }
}

}  // namespace

hipError_t launch_route_small(const RouteSmallArgs& a, int groups, hipStream_t s,
                              const ScanArgs* tail_scan, const RankArgs* tail_rank) {
  const int64_t nblk = (a.T + (int64_t)kTB * groups - 1) / ((int64_t)kTB * groups);
  if (nblk == 0) return hipSuccess;
  // scan and rank in this launch: one block of the same tokens, slot ids in
  // the rank's registers
  ScanArgs sa{};
  RankArgs ra{};
  if (tail_scan && tail_rank) {
    if (nblk != 1 || tail_scan->nblk != 1 || tail_rank->nblk != 1 ||
        (int64_t)tail_rank->tb * tail_rank->k > 64 * kMaxChunks || tail_rank->T != a.T)
      return hipErrorInvalidValue;
    sa = *tail_scan;
    ra = *tail_rank;
  }
  if (a.E > kRouteSmallMaxE || a.k + 1 > 16 || a.d % 32 || groups < 1) return hipErrorInvalidValue;
  const int ns = (a.E + 15) / 16;
  const int k1 = a.k + 1;
  const bool dma = a.E % 4 == 0;
  // the largest K range of a wave against its slice and the fragment registers
  const int pitch = dma ? a.E : 16 * ns;
  const int steps_w = (a.d / 32 + kWaves - 1) / kWaves;
  int slice = 0;
  switch (ns) {
    case 1: slice = slice_bytes<1>(); break;
    case 2: slice = slice_bytes<2>(); break;
    case 3: slice = slice_bytes<3>(); break;
    default: slice = slice_bytes<4>(); break;
  }
  const bool res = steps_w <= XB && steps_w * 64 * pitch <= slice;
#define MOE_RS3(NSV, KM, DM)                                                              \
  do {                                                                                    \
    if (res)                                                                              \
      hipLaunchKernelGGL((route_small_kernel<NSV, KM, DM, true>), dim3((unsigned)nblk),   \
                         dim3(256), 0, s, a, groups, sa, ra);                                     \
    else                                                                                  \
      hipLaunchKernelGGL((route_small_kernel<NSV, KM, DM, false>), dim3((unsigned)nblk),  \
                         dim3(256), 0, s, a, groups, sa, ra);                                     \
  } while (0)
#define MOE_RS(NSV, KM)                   \
  do {                                    \
    if (dma) MOE_RS3(NSV, KM, true);      \
    else MOE_RS3(NSV, KM, false);         \
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
#undef MOE_RS3
  return hipGetLastError();
}

}  // namespace moe
