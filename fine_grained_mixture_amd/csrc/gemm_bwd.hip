// Products of the layer backward on gfx950 (bf16 operands, fp32 accumulate).
//
// The backward multiplies the same stacked expert tensors as the forward but
// with other operands transposed: the input gradient needs dY W^T (the weight
// read along its contiguous dimension), the weight gradients need X^T dY (both
// operands read across their rows, summed over a ragged range of dispatched
// rows). On the MFMA both cases reduce to how an operand tile is read:
//
//   k-contiguous operand (rows of 32 k, 64 bytes): stored in LDS [row][k] and
//     read with ds_read_b128, 8 consecutive k of one row per lane;
//   k-strided operand (k-rows of the tile's width): stored in LDS [k][col]
//     exactly as in memory and read with ds_read_b64_tr_b16, which hands each
//     lane 4 consecutive k of one column; two such reads give the 8 k of the
//     MFMA operand.
//
// The v_mfma_f32_32x32x16_bf16 operands are symmetric (lane l supplies
// row/column l % 32 at k = 8 (l / 32) .. + 7 for both A and B), so one tile
// reader per storage order serves either operand.
//
// gemm_bwd_kernel: 256 x 128 output tiles, K-step 32, three-stage ring of
// direct-to-LDS loads (global_load_lds_dwordx4), 2 x 2 waves of 128 x 64 as in
// the forward expert kernel. Lanes whose k lies past the work item's range
// load from a zeroed 16-byte page, so ragged k ranges (the weight gradients'
// per-expert row counts) accumulate exact zeros in the tail.
//
// swiglu_bwd_kernel: 128 rows x 64 expert columns; per K-step it stages the
// token rows, the upstream-gradient rows, and the gate, up and down weight
// slices, and accumulates a = x Wg, b = x Wu and dh = dy Wd^T side by side,
// so the epilogue forms da and db without writing dh or the recomputed gate
// and up values to memory.

#include <type_traits>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kBM = kGemmBigBM;   // 256
constexpr int kBN = 128;
constexpr int kBK = 32;
constexpr int kStages = 3;
constexpr int kThreads = 256;
constexpr int kAStageBytes = kBM * kBK * 2;   // 16 KiB
constexpr int kBStageBytes = kBK * kBN * 2;   // 8 KiB
constexpr int kStageBytes = kAStageBytes + kBStageBytes;

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef short shortx8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// Source of the lanes whose k lies outside the work item's range.
__device__ __attribute__((aligned(16))) uint32_t g_zero16[4];

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

// k-contiguous tile [rows][32]: 64-byte rows of 4 chunks, chunk ^ ((row >> 2) & 3)
__device__ __forceinline__ int kc_off(int row, int chunk) {
  return row * 64 + 16 * (chunk ^ ((row >> 2) & 3));
}
// k-strided tile [32][COLS]: rows of COLS / 8 chunks, chunk ^ (2 (k & 3))
template <int COLS>
__device__ __forceinline__ int ks_off(int k, int chunk) {
  return k * (COLS * 2) + 16 * (chunk ^ ((k & 3) << 1));
}

__device__ __forceinline__ bf16x8 frag_kc(const unsigned char* t, int row, int chunk) {
  return *reinterpret_cast<const bf16x8*>(t + kc_off(row, chunk));
}
// Lane roles of the transposed read: within a 16-lane group, source lane s
// points at k-row k + s / 4, columns n + 4 (s % 4); output lane j receives
// column n + j at 4 consecutive k.
template <int COLS>
__device__ __forceinline__ bf16x8 frag_ks(const unsigned char* t, int k, int n) {
  const int o0 = ks_off<COLS>(k, n >> 3) + 2 * (n & 7);
  const int o1 = ks_off<COLS>(k + 4, n >> 3) + 2 * (n & 7);
  const shortx4 lo =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) shortx4*)(t + o0));
  const shortx4 hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) shortx4*)(t + o1));
  const shortx8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

template <bool A_KC, bool B_KC, int EPI>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_bwd_kernel(BwdLaunch L) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kStages * kStageBytes];

  int bid = blockIdx.x;
  {
    // runs of C consecutive work items per XCD (they share operand rows in
    // that XCD's L2), the runs dealt round-robin over the 8 XCDs
    const int C = L.p[0].n_tiles_n * 2;
    const int nwg = gridDim.x;
    const int full = nwg / (8 * C) * (8 * C);
    if (bid < full) {
      const int x = bid & 7, i = bid >> 3;
      bid = ((i / C) * 8 + x) * C + (i % C);
    }
  }
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
  const int nk = ke > kb ? (ke - kb + kBK - 1) / kBK : 0;
  const int N = P.N;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const bf16_t* zero = reinterpret_cast<const bf16_t*>(g_zero16);

  // ---- per-lane sources of the direct-to-LDS loads
  // A: 4 loads per wave and step. k-contiguous: load j covers rows
  // 16 (4 w + j) .. +15, lane -> row + L / 4, chunk (L % 4) ^ (L / 16).
  // k-strided [32][256]: load j covers k-rows 2 (4 w + j) + {0, 1}, lane ->
  // k-row + L / 32, chunk (L % 32) ^ (2 (k-row & 3)).
  const bf16_t* A = static_cast<const bf16_t*>(P.A) + s * P.a_group;
  const bf16_t* a_src[4];
  int a_k[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (A_KC) {
      const int cc = (lane & 3) ^ (lane >> 4);
      const int r = min(r0 + 16 * (4 * wave + j) + (lane >> 2), r_end - 1);
      const int64_t arow = P.a_gather ? P.a_gather[r] : r;
      a_src[j] = A + arow * P.lda + 8 * cc;
      a_k[j] = 8 * cc;
    } else {
      const int kl = 2 * (4 * wave + j) + (lane >> 5);
      const int cc = (lane & 31) ^ ((kl & 3) << 1);
      const int m = min(r0 + 8 * cc, r_end - 8);
      a_src[j] = A + (int64_t)kl * P.lda + m;
      a_k[j] = kl;
    }
  }
  // B: 2 loads per wave and step. k-strided [32][128]: load j covers k-rows
  // 8 w + 4 j .. +3, lane -> k-row + L / 16, chunk (L % 16) ^ (2 (L / 16)).
  // k-contiguous [128][32]: load j covers rows 16 (2 w + j) .. +15 as for A.
  const bf16_t* b_src[2];   // k-strided: pointer at k-row kl
  int64_t b_off[2];         // k-contiguous: element offset from the segment base
  int b_k[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if (B_KC) {
      const int cc = (lane & 3) ^ (lane >> 4);
      const int n = min(n0 + 16 * (2 * wave + j) + (lane >> 2), N - 1);
      b_src[j] = nullptr;
      b_off[j] = (int64_t)n * P.ldb + 8 * cc;
      b_k[j] = 8 * cc;
    } else {
      b_off[j] = 0;
      const int kl = 8 * wave + 4 * j + (lane >> 4);
      const int cc = (lane & 15) ^ ((lane >> 4) << 1);
      const int n = min(n0 + 8 * cc, N - 8);
      b_src[j] = static_cast<const bf16_t*>(P.B0) + s * P.b_group + (int64_t)kl * P.ldb + n;
      b_k[j] = kl;
    }
  }
  // k-contiguous B: base of the segment holding k0 (K-steps never straddle
  // segments: k_seg is a multiple of 32)
  auto b_seg_base = [&](int k0) -> const bf16_t* {
    const int q = P.k_seg ? k0 / P.k_seg : 0;
    const bf16_t* base = static_cast<const bf16_t*>((q & 1) ? P.B1 : P.B0);
    return base + s * P.b_group + (int64_t)(q >> 1) * P.b_seg - (int64_t)q * P.k_seg;
  };
  auto a_ptr = [&](int j, int k0) -> const bf16_t* {
    if (k0 + a_k[j] >= ke) return zero;
    return A_KC ? a_src[j] + k0 : a_src[j] + (int64_t)k0 * P.lda;
  };
  auto b_ptr = [&](int j, int k0, const bf16_t* seg) -> const bf16_t* {
    if (k0 + b_k[j] >= ke) return zero;
    if (B_KC) return seg + b_off[j] + k0;
    return b_src[j] + (int64_t)k0 * P.ldb;
  };

  const uint32_t smem_base =
      (uint32_t)(uintptr_t)((__attribute__((address_space(3))) unsigned char*)smem);
  auto issue = [&](int kt) {
    const uint32_t As = smem_base + (kt % kStages) * kStageBytes;
    const uint32_t Bs = As + kAStageBytes;
    const int k0 = kb + kt * kBK;
    const bf16_t* seg = B_KC ? b_seg_base(k0) : nullptr;
#pragma unroll
    for (int j = 0; j < 4; ++j) dma16(a_ptr(j, k0), As + (4 * wave_u + j) * 1024);
#pragma unroll
    for (int j = 0; j < 2; ++j) dma16(b_ptr(j, k0, seg), Bs + (2 * wave_u + j) * 1024);
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
  const int g16 = lane >> 4, s16 = lane & 15;
  const int bk_lane = 8 * (g16 >> 1) + (s16 >> 2);
  const int bn_lane = 16 * (g16 & 1) + 4 * (s16 & 3);

  // NI, NJ: how many of the wave's four 32-row and two 32-column blocks hold
  // output of the work item (an expert's last rows, or columns past N); the
  // others skip their fragment reads and MFMAs, which frees the SIMD for the
  // co-resident workgroup's wave. The loads and barriers are the same for
  // every wave.
  auto step = [&](int st, int kt_next, auto ni, auto nj) {
    constexpr int NI = decltype(ni)::value, NJ = decltype(nj)::value;
    const unsigned char* As = smem + st * kStageBytes;
    const unsigned char* Bs = As + kAStageBytes;
    const uint32_t Asn = smem_base + (kt_next % kStages) * kStageBytes;
    const uint32_t Bsn = Asn + kAStageBytes;
    const int k0n = kb + kt_next * kBK;
    const bool do_issue = kt_next < nk;
    const bf16_t* segn = (B_KC && do_issue) ? b_seg_base(k0n) : nullptr;
    bf16x8 a[2][4], b[2][2];
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      if (NJ > 0) {
#pragma unroll
        for (int i = 0; i < NI; ++i)
          a[ks][i] = A_KC ? frag_kc(As, 128 * wm + 32 * i + l32, 2 * ks + lhi)
                          : frag_ks<kBM>(As, 16 * ks + bk_lane, 128 * wm + 32 * i + bn_lane);
      }
      if (NI > 0) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          b[ks][j] = B_KC ? frag_kc(Bs, 64 * wn + 32 * j + l32, 2 * ks + lhi)
                          : frag_ks<kBN>(Bs, 16 * ks + bk_lane, 64 * wn + 32 * j + bn_lane);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int ks = q >> 3, i = (q >> 1) & 3, j = q & 1;
      if (i < NI && j < NJ)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks][i], b[ks][j], acc[i][j], 0, 0, 0);
      if (do_issue && q < 6) {
        __builtin_amdgcn_sched_barrier(0);
        if (q < 4) dma16(a_ptr(q, k0n), Asn + (4 * wave_u + q) * 1024);
        else dma16(b_ptr(q - 4, k0n, segn), Bsn + (2 * wave_u + q - 4) * 1024);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  constexpr int kWaitVm6 = 6 | (7 << 4) | (15 << 8);
  constexpr int kWaitVm0 = (7 << 4) | (15 << 8);
  auto main_loop = [&](auto ni, auto nj) {
    if (nk > 0) issue(0);
    if (nk > 1) issue(1);
    for (int kt = 0; kt < nk; ++kt) {
      if (kt + 1 < nk) __builtin_amdgcn_s_waitcnt(kWaitVm6);   // step kt landed
      else __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();   // stage kt published; stage (kt - 1) % 3 released
      __builtin_amdgcn_sched_barrier(0);
      step(kt % kStages, kt + 2, ni, nj);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  if constexpr (EPI == kBwdSwiGLU || !A_KC) {
    // every block runs: the SwiGLU epilogue's operand prefetch leaves no
    // registers for the skipping variants (they spill), and the weight
    // gradients' tiles are whole in M (the k range is what is ragged there),
    // where the extra variants cost 7% at the Quartz shape
    main_loop(std::integral_constant<int, 4>(), std::integral_constant<int, 2>());
  } else {
    using std::integral_constant;
    const int rows_here = r_end - r0 - 128 * wm;
    const int cols_here = N - n0 - 64 * wn;
    const int nib = __builtin_amdgcn_readfirstlane(min(4, max(0, (rows_here + 31) / 32)));
    const int njb = __builtin_amdgcn_readfirstlane(min(2, max(0, (cols_here + 31) / 32)));
    if (nib == 0 || njb == 0) {
      main_loop(integral_constant<int, 0>(), integral_constant<int, 0>());
    } else if (njb == 2) {
      switch (nib) {
        case 4: main_loop(integral_constant<int, 4>(), integral_constant<int, 2>()); break;
        case 3: main_loop(integral_constant<int, 3>(), integral_constant<int, 2>()); break;
        case 2: main_loop(integral_constant<int, 2>(), integral_constant<int, 2>()); break;
        default: main_loop(integral_constant<int, 1>(), integral_constant<int, 2>()); break;
      }
    } else {
      switch (nib) {
        case 4: main_loop(integral_constant<int, 4>(), integral_constant<int, 1>()); break;
        case 3: main_loop(integral_constant<int, 3>(), integral_constant<int, 1>()); break;
        case 2: main_loop(integral_constant<int, 2>(), integral_constant<int, 1>()); break;
        default: main_loop(integral_constant<int, 1>(), integral_constant<int, 1>()); break;
      }
    }
  }

  // ---- epilogue through a private 18 KiB LDS slice per wave: each 32-row
  // block of the wave's results is staged, then written as 16-byte pieces of
  // rows (lane -> row 4 rr + L / 16 of the block, columns col .. col + 3)
  __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4));
  __builtin_amdgcn_s_barrier();
  float* st = reinterpret_cast<float*>(smem + wave * (kStages * kStageBytes / 4));
  const int row_base = r0 + 128 * wm;
  const int col = n0 + 64 * wn + 4 * (lane & 15);
  auto stage_block = [&](int i) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q)
        st[(8 * (q >> 2) + 4 * lhi + (q & 3)) * 72 + 32 * j + l32] = acc[i][j][q];
  };
  if (EPI == kBwdStoreF32) {
    float* cbase = nullptr;
    if (col < N) {
      cbase = (col < P.c_split ? P.C0 + col : P.C1 + (col - P.c_split)) + s * P.c_group +
              (int64_t)c * P.c_chunk;
    }
    // the scaled bf16 copy: this lane's four column scales
    uint16_t* c2base = P.C2 && col < N ? P.C2 + col : nullptr;
    float sc[4] = {0.f, 0.f, 0.f, 0.f};
    if (c2base) {
#pragma unroll
      for (int e = 0; e < 4; ++e) sc[e] = bf16_to_f32(P.c2_scale[s * P.c2_scale_group + col + e]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      stage_block(i);
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        const int r = 4 * rr + (lane >> 4);
        const int row = row_base + 32 * i + r;
        const floatx4 v = *reinterpret_cast<const floatx4*>(&st[r * 72 + 4 * (lane & 15)]);
        if (row < r_end && cbase) *reinterpret_cast<floatx4*>(cbase + (int64_t)row * P.ldc) = v;
        if (row < r_end && c2base) {
          u32x2 q;
          q[0] = (uint32_t)f32_to_bf16(v[0] * sc[0]) | ((uint32_t)f32_to_bf16(v[1] * sc[1]) << 16);
          q[1] = (uint32_t)f32_to_bf16(v[2] * sc[2]) | ((uint32_t)f32_to_bf16(v[3] * sc[3]) << 16);
          *reinterpret_cast<u32x2*>(c2base + (int64_t)row * P.ldc2) = q;
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
  } else {
    // dh in acc; a and b of the same elements come from the forward. The
    // loads of block i + 1 are issued before block i is processed, so their
    // latency overlaps its arithmetic and stores (addresses are clamped into
    // the valid rows and columns; out-of-range results are not stored). They
    // are streaming loads: each value is read once, and the tiles' dY and
    // W_down rows keep the caches (Quartz dh 128 -> 123 us).
    const float* abase = P.ab + s * P.ab_group + min(col, N - 4);
    floatx4 ca[8], cb[8], na[8], nb[8];
    auto load_ab = [&](int i, floatx4* va, floatx4* vb) {
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        const int row = min(row_base + 32 * i + 4 * rr + (lane >> 4), r_end - 1);
        const float* p = abase + (int64_t)row * P.ab_ld;
        va[rr] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(p));
        vb[rr] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(p + P.half));
      }
    };
    load_ab(0, ca, cb);
    bf16_t* obase = static_cast<bf16_t*>(static_cast<void*>(P.C0)) + s * P.c_group + col;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      stage_block(i);
      if (i + 1 < 4) load_ab(i + 1, na, nb);
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        const int r = 4 * rr + (lane >> 4);
        const int row = row_base + 32 * i + r;
        const floatx4 v = *reinterpret_cast<const floatx4*>(&st[r * 72 + 4 * (lane & 15)]);
        if (row < r_end && col < N) {
          float da[4], db[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float a = ca[rr][e], b = cb[rr][e];
            const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-a));
            da[e] = v[e] * b * (sg * (1.0f + a * (1.0f - sg)));
            db[e] = v[e] * (a * sg);
          }
          u32x2 pa, pb;
          pa[0] = (uint32_t)f32_to_bf16(da[0]) | ((uint32_t)f32_to_bf16(da[1]) << 16);
          pa[1] = (uint32_t)f32_to_bf16(da[2]) | ((uint32_t)f32_to_bf16(da[3]) << 16);
          pb[0] = (uint32_t)f32_to_bf16(db[0]) | ((uint32_t)f32_to_bf16(db[1]) << 16);
          pb[1] = (uint32_t)f32_to_bf16(db[2]) | ((uint32_t)f32_to_bf16(db[3]) << 16);
          bf16_t* o = obase + (int64_t)row * P.ldc;
          *reinterpret_cast<u32x2*>(o) = pa;
          *reinterpret_cast<u32x2*>(o + P.half) = pb;
        }
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        ca[rr] = na[rr];
        cb[rr] = nb[rr];
      }
    }
  }
}

// ---------------------------------------------------------------------------
constexpr int kSB = kSwigluBwdBM;   // 128 rows
constexpr int kSN = 64;             // expert columns
constexpr int kSXBytes = kSB * kBK * 2;        // 8 KiB (x rows, and dy rows)
constexpr int kSWBytes = kBK * kSN * 2;        // 4 KiB (each weight slice)
constexpr int kSStageBytes = 2 * kSXBytes + 3 * kSWBytes;   // 28 KiB

__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
swiglu_bwd_kernel(SwigluBwdLaunch L) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * kSStageBytes];

  int local = blockIdx.x, pi = 0;
  if (local >= L.tiles0) {
    if (L.n < 2) return;
    pi = 1;
    local -= L.tiles0;
  }
  const SwigluBwdProblem& P = L.p[pi];
  const int nt = local % P.n_tiles_n, mt = local / P.n_tiles_n;
  int s, r0, r_end;
  if (P.plan) {
    // the plan's tiles are kGemmBigBM rows: work item mt takes half mt & 1
    const int pt = mt >> 1;
    if (pt >= P.plan[0]) return;
    s = P.plan[1 + 2 * pt];
    const int p0 = P.plan[2 + 2 * pt];
    r0 = p0 + kSB * (mt & 1);
    r_end = min(P.m_off[s + 1], p0 + kGemmBigBM);
  } else {
    const int mtg = (P.M + kSB - 1) / kSB;
    s = mt / mtg;
    if (s >= P.G) return;
    r0 = (mt - s * mtg) * kSB;
    r_end = min(P.M, r0 + kSB);
  }
  if (r0 >= r_end) return;
  const int n0 = nt * kSN;
  const int d = P.d, F = P.F;
  const int nk = d / kBK;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);

  // x and dy rows: 2 loads per wave and step each, rows 16 (2 w + j) + L / 4
  const bf16_t* x_src[2];
  const bf16_t* y_src[2];
  {
    const int cc = (lane & 3) ^ (lane >> 4);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = min(r0 + 16 * (2 * wave + j) + (lane >> 2), r_end - 1);
      const int64_t xr = P.x_rows ? P.x_rows[r] : r;
      x_src[j] = static_cast<const bf16_t*>(P.X) + xr * P.ldx + 8 * cc;
      y_src[j] = static_cast<const bf16_t*>(P.DY) + (int64_t)r * P.ldy + 8 * cc;
    }
  }
  // gate and up slices [32][64]: one load per wave, k-rows 8 w + L / 8,
  // chunk (L % 8) ^ (2 (k-row & 3)); down slice [64][32] (k-contiguous): rows
  // 16 w + L / 4
  const bf16_t *g_src, *u_src, *d_src;
  {
    const int kl = 8 * wave + (lane >> 3);
    const int cc = (lane & 7) ^ ((kl & 3) << 1);
    const int64_t off = s * P.w_group + (int64_t)kl * F + n0 + 8 * cc;
    g_src = static_cast<const bf16_t*>(P.Wg) + off;
    u_src = static_cast<const bf16_t*>(P.Wu) + off;
    const int cd = (lane & 3) ^ (lane >> 4);
    const int f = n0 + 16 * wave + (lane >> 2);
    d_src = static_cast<const bf16_t*>(P.Wd) + s * P.w_group + (int64_t)f * d + 8 * cd;
  }
  const uint32_t smem_base =
      (uint32_t)(uintptr_t)((__attribute__((address_space(3))) unsigned char*)smem);
  auto issue = [&](int kt) {
    const uint32_t S0 = smem_base + (kt & 1) * kSStageBytes;
    const int k0 = kt * kBK;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      dma16(x_src[j] + k0, S0 + (2 * wave_u + j) * 1024);
      dma16(y_src[j] + k0, S0 + kSXBytes + (2 * wave_u + j) * 1024);
    }
    dma16(g_src + (int64_t)k0 * F, S0 + 2 * kSXBytes + wave_u * 1024);
    dma16(u_src + (int64_t)k0 * F, S0 + 2 * kSXBytes + kSWBytes + wave_u * 1024);
    dma16(d_src + k0, S0 + 2 * kSXBytes + 2 * kSWBytes + wave_u * 1024);
  };

  // wave tile: rows 64 wm .. +63, columns 32 wn .. +31 of a, b and dh
  const int wm = wave >> 1, wn = wave & 1;
  floatx16 acc_a[2], acc_b[2], acc_h[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc_a[i][q] = acc_b[i][q] = acc_h[i][q] = 0.f;

  const int l32 = lane & 31, lhi = lane >> 5;
  const int g16 = lane >> 4, s16 = lane & 15;
  const int bk_lane = 8 * (g16 >> 1) + (s16 >> 2);
  const int bn_lane = 16 * (g16 & 1) + 4 * (s16 & 3);

  issue(0);
  for (int kt = 0; kt < nk; ++kt) {
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));   // this wave's loads of step kt
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();   // step kt published; the other stage released
    __builtin_amdgcn_sched_barrier(0);
    if (kt + 1 < nk) issue(kt + 1);
    const unsigned char* S0 = smem + (kt & 1) * kSStageBytes;
    const unsigned char* Xs = S0;
    const unsigned char* Ys = S0 + kSXBytes;
    const unsigned char* Gs = S0 + 2 * kSXBytes;
    const unsigned char* Us = Gs + kSWBytes;
    const unsigned char* Ds = Us + kSWBytes;
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      bf16x8 xa[2], ya[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        xa[i] = frag_kc(Xs, 64 * wm + 32 * i + l32, 2 * ks + lhi);
        ya[i] = frag_kc(Ys, 64 * wm + 32 * i + l32, 2 * ks + lhi);
      }
      const bf16x8 bg = frag_ks<kSN>(Gs, 16 * ks + bk_lane, 32 * wn + bn_lane);
      const bf16x8 bu = frag_ks<kSN>(Us, 16 * ks + bk_lane, 32 * wn + bn_lane);
      const bf16x8 bd = frag_kc(Ds, 32 * wn + l32, 2 * ks + lhi);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        acc_a[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa[i], bg, acc_a[i], 0, 0, 0);
        acc_b[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa[i], bu, acc_b[i], 0, 0, 0);
        acc_h[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ya[i], bd, acc_h[i], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: lane holds column l32 of each 32 x 32 block
  bf16_t* out = static_cast<bf16_t*>(P.DAB) + s * P.ab_group;
  const int col = n0 + 32 * wn + l32;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int row = r0 + 64 * wm + 32 * i + 8 * (q >> 2) + 4 * lhi + (q & 3);
      const float a = acc_a[i][q], b = acc_b[i][q], dh = acc_h[i][q];
      const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-a));
      const float silu = a * sg;
      const float dsilu = sg * (1.0f + a * (1.0f - sg));
      if (row < r_end) {
        bf16_t* o = out + (int64_t)row * P.ldab + col;
        o[0] = f32_to_bf16(dh * b * dsilu);
        o[F] = f32_to_bf16(dh * silu);
      }
    }
}

}  // namespace

int64_t bwd_tiles(const BwdGemm& P) {
  if (P.plan) return (int64_t)P.max_m_tiles * P.n_tiles_n;
  return (int64_t)P.G * P.n_chunks * P.n_tiles_m * P.n_tiles_n;
}

hipError_t launch_gemm_bwd(BwdLaunch& L, bool a_kc, bool b_kc, int epi, hipStream_t s) {
  if (L.n < 1 || L.n > kBwdMaxProblems) return hipErrorInvalidValue;
  int64_t total = 0;
  for (int i = 0; i < L.n; ++i) {
    const BwdGemm& P = L.p[i];
    // shapes the tile loaders assume
    // k-strided operands: their columns (M or N) in 16-byte pieces;
    // k-contiguous ones: K in 16-byte pieces
    if (P.N < 8 || P.N % 8) return hipErrorInvalidValue;
    if (!a_kc && (P.a_gather || P.M < 8 || P.M % 8)) return hipErrorInvalidValue;
    if ((a_kc || b_kc) && P.K % 8) return hipErrorInvalidValue;
    if (b_kc && P.k_seg % kBK) return hipErrorInvalidValue;
    if (!P.plan && (P.n_tiles_m < 1 || P.n_chunks < 1)) return hipErrorInvalidValue;
    // the scaled copy: one fp32 result per element (no column split, no
    // K chunks), and its scale vector
    if (P.C2 && (epi != kBwdStoreF32 || !P.c2_scale || P.c_split < P.N || P.n_chunks != 1 ||
                 P.N % 4))
      return hipErrorInvalidValue;
    L.start[i] = (int32_t)total;
    total += bwd_tiles(P);
  }
  L.start[L.n] = (int32_t)total;
  if (total == 0) return hipSuccess;
  if (total >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)total), block(kThreads);
  // the layouts the layer backward uses: dgrad and dh (k-contiguous both),
  // wgrad (k-strided both), and rows times a row-major weight
  if (epi == kBwdSwiGLU) {
    if (!a_kc || !b_kc) return hipErrorInvalidValue;
    for (int i = 0; i < L.n; ++i)
      if (!L.p[i].ab || L.p[i].N % 4 || L.p[i].half < L.p[i].N) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_bwd_kernel<true, true, kBwdSwiGLU>), grid, block, 0, s, L);
  } else if (a_kc && b_kc) {
    hipLaunchKernelGGL((gemm_bwd_kernel<true, true, kBwdStoreF32>), grid, block, 0, s, L);
  } else if (!a_kc && !b_kc) {
    hipLaunchKernelGGL((gemm_bwd_kernel<false, false, kBwdStoreF32>), grid, block, 0, s, L);
  } else if (a_kc && !b_kc) {
    // rows times a row-major weight (the rank-r experts' U x and V products)
    hipLaunchKernelGGL((gemm_bwd_kernel<true, false, kBwdStoreF32>), grid, block, 0, s, L);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const SwigluBwdLaunch& L, hipStream_t s) {
  if (L.n < 1 || L.n > 2) return hipErrorInvalidValue;
  int64_t total = 0;
  for (int i = 0; i < L.n; ++i) {
    const SwigluBwdProblem& P = L.p[i];
    if (P.d % kBK || P.F % kSN || P.d < kBK) return hipErrorInvalidValue;
    const int64_t t = P.plan ? (int64_t)2 * P.max_m_tiles * P.n_tiles_n
                             : (int64_t)P.G * ((P.M + kSB - 1) / kSB) * P.n_tiles_n;
    if (i == 0 && t != L.tiles0) return hipErrorInvalidValue;
    total += t;
  }
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(swiglu_bwd_kernel, dim3((unsigned)total), dim3(kThreads), 0, s, L);
  return hipGetLastError();
}

}  // namespace moe
