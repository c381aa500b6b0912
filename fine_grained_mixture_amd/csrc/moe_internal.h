// Internal declarations shared by the host library and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// Tokens per routing block: the top-k kernels histogram, and the rank kernel
// ranks, blocks of this many consecutive tokens (one workgroup / one wave
// each). The fused small-E router uses 16-token blocks, the generic one 64.
constexpr int kRouteBlockSmall = 16;
constexpr int kRouteBlock = 64;
// Largest expert count the fused small-E router handles.
constexpr int kRouteSmallMaxE = 64;
// Rows per M-tile of the grouped GEMMs.
constexpr int kGemmBM = 128;
// Rows per tile of the large-tile expert GEMM (256 x 128 output tiles).
constexpr int kGemmBigBM = 256;
constexpr int kGemmBM_F32 = 64;
// Rows per workgroup of the fused low-rank expert kernel.
constexpr int kLowRankBM = 64;

// One problem of a grouped GEMM launch: C[r, :] (op)= A[arow(r), :] x B_g for
// every row r of every group g.
//   rows of group g: [row_off[g], row_off[g+1]) if row_off, else [0, M)
//   arow(r) = a_rows ? a_rows[r] : r       (a_rows gathers token rows)
//   B_g = B0 (+ B1 for dual) + g * b_group_stride, [K, N] row-major (N contiguous)
//   C row r, columns [g * c_group_col, ... + N) with leading dimension ldc
struct GemmProblem {
  const void* A;
  const int32_t* a_rows;
  int64_t lda;
  const void* B0;
  const void* B1;
  int64_t b_group_stride;
  int64_t ldb;
  void* C;
  int64_t ldc;
  int64_t c_group_col;
  const float* col_bias;     // [N] or null, added in the fp32 epilogue
  const int32_t* row_off;    // [G+1] device, or null for uniform groups
  const int32_t* plan;       // device tile list for row_off groups: plan[0] = count,
                             // then (group, first row) pairs
  int32_t M, N, K, G;
  int32_t n_tiles_n;         // N-tiles per M-tile
  int32_t max_m_tiles;       // upper bound of M-tiles (grid sizing)
};

enum GemmEpilogue : int {
  kEpiStoreF32 = 0,   // C (float) = acc (+ col_bias)
  kEpiSwiGLU = 1,     // dual: C (dtype) = round(SiLU(acc_gate) * acc_up)
};

// Batches of at most this many tokens run the expert GEMMs with the skinny
// kernel (few rows per expert: weight-bandwidth bound).
constexpr int kSkinnyMaxT = 4;

// Up to two problems share one launch: tiles of p[0] come first, then p[1].
struct GemmLaunch {
  GemmProblem p[2];
  int32_t n_problems;
  int32_t tiles0;            // tiles of p[0] (uniform groups: static count)
};

hipError_t launch_gemm_bf16(const GemmLaunch& L, int epilogue, hipStream_t s);
hipError_t launch_gemm_f32(const GemmLaunch& L, int epilogue, hipStream_t s);
// 256 x 128 tiles (dual: 256 x (64 + 64)); N multiple of 8, K of 32.
hipError_t launch_gemm_big(const GemmLaunch& L, int epilogue, hipStream_t s);
// Tile list of a row_off problem from offsets[0..G] (one workgroup).
// Few rows per group (bf16): one workgroup per (group, 64 columns), weights
// streamed once per pass of 4 rows; row_off groups or uniform groups of M rows.
hipError_t launch_gemm_skinny(const GemmLaunch& L, int epilogue, hipStream_t s);
hipError_t launch_plan(const int32_t* offsets, int32_t G, int32_t bm, int32_t* plan,
                       hipStream_t s);

// Routing.
struct TopkArgs {
  const float* logits;       // [T, E] fp32, logit_bias already added
  const float* select_bias;  // [E] or null (sigmoid rule)
  int32_t* topk_idx;         // [T, k]
  float* topk_gate;          // [T, k]
  float* topk_margin;        // [T] or null
  int32_t* blk_counts;       // [nblk, E]
  float* blk_psum;           // [nblk, E]
  int64_t T;
  int32_t E, k, score, renorm;
  int32_t tb;                // tokens per block (multiple of 4)
};
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);

// Fused router for E <= kRouteSmallMaxE, bf16: logits by MFMA, top-k, gates,
// block histogram and probability sums, kRouteBlockSmall tokens per block.
struct RouteSmallArgs {
  const void* x;             // [T, d] bf16
  const void* w_router;      // [d, E] bf16
  const float* logit_bias;   // [E] or null
  const float* select_bias;  // [E] or null
  int32_t* topk_idx;
  float* topk_gate;
  float* topk_margin;        // or null
  int32_t* blk_counts;       // [nblk, E]
  float* blk_psum;           // [nblk, E]
  int64_t T;
  int32_t d, E, k, score, renorm;
};
// Groups of kRouteBlockSmall tokens each workgroup of the fused router
// handles for T tokens; its routing blocks are kRouteBlockSmall * groups
// tokens long.
int route_small_groups(int64_t T, int k);
hipError_t launch_route_small(const RouteSmallArgs& a, int groups, hipStream_t s);

struct ScanArgs {
  const int32_t* blk_counts;  // [nblk, E]
  const float* blk_psum;      // [nblk, E]
  int32_t* blk_base;          // [nblk, E] out: slots of expert e in earlier blocks
  int32_t* counts;            // [E]
  int32_t* kept;              // [E]
  int32_t* offsets;           // [E+1]
  int32_t* n_dropped;         // [1]
  float* aux;                 // [2]
  float* f;                   // [E] or null
  float* P;                   // [E] or null
  float* psum_tot;            // [E] scratch: per-expert probability sums (E > 64)
  int32_t* plan;              // routed tile list (rows per tile plan_bm) or null
  int32_t plan_bm;
  int32_t nblk, E, k, capacity;
  int64_t T;
  float aux_coef;
};
hipError_t launch_scan(const ScanArgs& a, hipStream_t s);

// select_bias[e] += gamma * sign(Tk - E counts[e]) for e < E.
hipError_t launch_bias_update(const int32_t* counts, float* bias, int E, int64_t Tk, float gamma,
                              hipStream_t s);

struct RankArgs {
  const int32_t* topk_idx;   // [T, k]
  const int32_t* blk_base;   // [nblk, E]
  const int32_t* offsets;    // [E+1]
  int32_t* row_of_slot;      // [T, k]
  int32_t* sorted_token;     // [R_max]
  uint8_t* dropped;          // [T, k] or null
  int64_t T;
  int32_t E, k, capacity, nblk;
  int32_t tb;                // tokens per block, as for the top-k tables
};
hipError_t launch_rank(const RankArgs& a, hipStream_t s);

// x_perm[r] = x[sorted_token[r]] for r < offsets[E]; row_bytes multiple of 16.
hipError_t launch_gather(const void* x, const int32_t* sorted_token, const int32_t* offsets,
                         int32_t E, int64_t r_max, int64_t row_bytes, void* x_perm,
                         hipStream_t s);

struct CombineArgs {
  const float* y_routed;     // [R_max, d]
  const float* y_shared;     // [T, d] or null
  const int32_t* row_of_slot;
  const float* topk_gate;
  float* y;                  // [T, d]
  void* y_lowp;              // [T, d] or null
  int64_t T;
  int32_t d, k, dtype;
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);

// Fused low-rank (rank 64) SwiGLU experts, bf16. Rows of expert e are
// [offsets[e], offsets[e+1]); A row of dispatched row r is a_rows[r] (or r).
struct LowRankArgs {
  const void* A;             // [*, d] bf16 token rows
  const int32_t* a_rows;     // [R_max] or null
  int64_t lda;
  const void *u_gate, *s_gate, *v_gate, *u_up, *s_up, *v_up, *u_down, *s_down, *v_down;
  const int32_t* offsets;    // [E+1]
  const int32_t* plan;       // tile list with kLowRankBM rows per tile
  float* y;                  // [R_max, d]
  int32_t d, F, E, max_tiles;
};
hipError_t launch_lowrank(const LowRankArgs& a, hipStream_t s);

}  // namespace moe
