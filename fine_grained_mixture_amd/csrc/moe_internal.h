// Internal declarations shared by the host library and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// Tokens per routing block: the top-k kernels histogram, and the rank kernel
// ranks, blocks of this many consecutive tokens (one workgroup / one wave
// each). The fused small-E router uses 16-token blocks, the generic one 32.
constexpr int kRouteBlockSmall = 16;
constexpr int kRouteBlock = 32;
// Largest expert count the fused small-E router handles.
constexpr int kRouteSmallMaxE = 64;
// Rows per M-tile of the grouped GEMMs.
constexpr int kGemmBM = 128;
// Rows per tile of the large-tile expert GEMM (256 x 128 output tiles).
constexpr int kGemmBigBM = 256;
// MI355X's Infinity Cache (the memory-side cache in front of HBM), bytes
constexpr int64_t kInfinityCacheBytes = (int64_t)256 << 20;
// Raw buffer descriptor word 3 (32-bit data format), and the cache-policy bit
// of a non-temporal (streaming) buffer store.
constexpr int kBufferRsrcWord3 = 0x00020000;
constexpr int kCpolNT = 2;
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
  const float* a_scale;      // fp8 products: per A row (indexed like A's rows after
                             // the a_rows gather), and per B column of group g at
  const float* b_scale0;     // b_scale + g * b_scale_group (b_scale1: the dual's up)
  const float* b_scale1;
  int64_t b_scale_group;
  float* ab;                 // SwiGLU epilogue, or null: the gate and up sums,
                             // gate at ab[row * ab_ld + g * ab_group_col + n],
                             // up N columns further
  int64_t ab_ld, ab_group_col;
  const int32_t* row_off;    // [G+1] device, or null for uniform groups
  const int32_t* plan;       // device tile list for row_off groups: plan[0] = count,
                             // then (group, first row) pairs
  int32_t M, N, K, G;
  int32_t n_tiles_n;         // N-tiles per M-tile
  int32_t max_m_tiles;       // upper bound of M-tiles (grid sizing)
  int32_t c_stream;          // fp32 epilogue of the bf16 tile kernel: store C with
                             // non-temporal (streaming) stores
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
// fp8 (E4M3) products: A rows and B = W^T rows both k-contiguous codes
// (B0/B1 + g * b_group_stride + n * ldb + k), 256 x 128 tiles (dual: 256 x
// (64 + 64)); the epilogue multiplies by a_scale[row] * b_scale[col]. K
// multiple of 64.
hipError_t launch_gemm_fp8(const GemmLaunch& L, int epilogue, hipStream_t s);
// Quantise rows to E4M3: for row r < min(rows, *n_valid) (n_valid may be
// null), s = the smallest power of two with amax(row) / s <= 448, codes
// q[r * K + k] = RNE(src[r * ld + k] / s) and scale[r] = s. K multiple of 8,
// at most 4096.
hipError_t launch_quant_rows(const uint16_t* src, int64_t ld, int64_t rows, int32_t K,
                             const int32_t* n_valid, uint8_t* q, float* scale, hipStream_t s);
// Quantise the columns of W[g] ([K, N] bf16, g < G) to E4M3 codes stored
// k-contiguous: q[g][n][k], scale[g][n]. K and N multiples of 8.
hipError_t launch_quant_cols(const uint16_t* w, int64_t G, int32_t K, int32_t N, uint8_t* q,
                             float* scale, hipStream_t s);
// Tile list of a row_off problem from offsets[0..G] (one workgroup).
// Few rows per group (bf16): one workgroup per (group, 64 columns), weights
// streamed once per pass of 4 rows; row_off groups or uniform groups of M rows.
// wide: 512 threads (64 K groups), for one or two rows per group, taken
// where every problem's K exceeds 512: the fp32-store epilogue, and the fused
// SwiGLU with passes of `rows` rows (1 or 2, the most a group holds).
hipError_t launch_gemm_skinny(const GemmLaunch& L, int epilogue, hipStream_t s, bool wide = false,
                              int rows = kSkinnyMaxT);
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
  int32_t wave_rows;         // set by launch_topk: waves keep their probability
                             // sums in LDS rows (0: they add them in turn)
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
  float* logits;             // [T, E] or null: the logits, logit_bias included
  int64_t T;
  int32_t d, E, k, score, renorm;
};
// Groups of kRouteBlockSmall tokens each workgroup of the fused router
// handles for T tokens; its routing blocks are kRouteBlockSmall * groups
// tokens long.
int route_small_groups(int64_t T, int k);
struct ScanArgs;
struct RankArgs;
// With tail_scan and tail_rank (the launch makes a single routing block), the
// launch also writes the scan's outputs and ranks the block.
hipError_t launch_route_small(const RouteSmallArgs& a, int groups, hipStream_t s,
                              const ScanArgs* tail_scan = nullptr,
                              const RankArgs* tail_rank = nullptr);

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
// scan and rank in one launch: E <= 64, nblk <= 256, the same blocks for both.
hipError_t launch_scan_rank(const ScanArgs& a, const RankArgs& r, hipStream_t s);

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

// Fused low-rank SwiGLU experts (rank 16, 32, 48 or 64 in rank-64 tiles), bf16
// products. Rows of expert e are
// [offsets[e], offsets[e+1]); A row of dispatched row r is a_rows[r] (or r).
// fp8 factors (fp8 != 0): U codes stored transposed [E, r, in], V codes
// [E, out, r] as in bf16, each with power-of-two scales: u_*_scale [E, r],
// v_gate/up_scale [E, F], v_down_scale [E, d]; s stays bf16.
struct LowRankArgs {
  const void* A;             // [*, d] bf16 token rows
  const int32_t* a_rows;     // [R_max] or null
  int64_t lda;
  const void *u_gate, *s_gate, *v_gate, *u_up, *s_up, *v_up, *u_down, *s_down, *v_down;
  const float *u_gate_scale, *u_up_scale, *u_down_scale;
  const float *v_gate_scale, *v_up_scale, *v_down_scale;
  int32_t fp8;
  const int32_t* offsets;    // [E+1]
  const int32_t* plan;       // tile list with kLowRankBM rows per tile
  float* y;                  // [R_max, d]
  int32_t d, F, E, max_tiles;
  int32_t rank;              // 16, 32, 48 or 64
};
hipError_t launch_lowrank(const LowRankArgs& a, hipStream_t s);


// ---- backward --------------------------------------------------------------

// One product of the backward: C[m, n] = sum over the work item's k range of
// A(m, k) B(k, n), bf16 operands, fp32 result. Tiles are kGemmBigBM x 128.
//   A(m, k), k-contiguous:  A[(a_gather ? a_gather[m] : m) * lda + k]
//            k-strided:     A[k * lda + m]
//            (group s adds s * a_group elements)
//   B(k, n), k-strided:     B0[k * ldb + n]  (+ s * b_group)
//            k-contiguous:  K is cut in segments of k_seg (one segment when
//                           k_seg == 0); segment q reads (q odd ? B1 : B0)
//                           + s * b_group + (q / 2) * b_seg at
//                           [n * ldb + k - q * k_seg]
//   Work items:
//     plan != null: M-ragged groups, rows of group s are [m_off[s], m_off[s+1])
//       in the plan's kGemmBigBM-row tiles; k in [0, K)
//     otherwise: groups s < G of rows [0, M); k in [k_off[s], k_off[s+1]) when
//       k_off, else chunk c < n_chunks covers [c k_chunk, min(K, (c+1) k_chunk))
//   Output: column n < c_split goes to C0, n >= c_split to C1 at n - c_split;
//     element offset s * c_group + c * c_chunk + row * ldc. An empty k range
//     writes zeros.
enum BwdEpilogue : int {
  kBwdStoreF32 = 0,   // C (float) as above
  kBwdSwiGLU = 1,     // the product is dh: with a = ab[row, n], b = ab[row, half + n]
                      // (ab + s * ab_group, leading dimension ab_ld), writes bf16
                      // C0[row, n] = dh b SiLU'(a) and C0[row, half + n] = dh SiLU(a)
};
struct BwdGemm {
  const void* A;
  const int32_t* a_gather;   // k-contiguous A only
  int64_t lda, a_group;
  const void* B0;
  const void* B1;
  int64_t ldb, b_group, b_seg;
  int32_t k_seg;
  float* C0;
  float* C1;
  int64_t ldc, c_group, c_chunk;
  int32_t c_split;
  const int32_t* m_off;
  const int32_t* plan;
  const int32_t* k_off;
  int32_t k_chunk, n_chunks;
  int32_t M, N, K, G;
  int32_t n_tiles_m, n_tiles_n, max_m_tiles;
  const float* ab;           // kBwdSwiGLU only
  int64_t ab_ld, ab_group;
  int32_t half;
  // kBwdStoreF32, optional: also C2[row, col] = bf16(C[row, col] *
  // c2_scale[s * c2_scale_group + col]) (a per-group column scale)
  uint16_t* C2;
  int64_t ldc2;
  const uint16_t* c2_scale;
  int64_t c2_scale_group;
};
constexpr int kBwdMaxProblems = 5;
// Problems of one launch share the operand layouts; tiles of p[i] are
// [start[i], start[i + 1]).
struct BwdLaunch {
  BwdGemm p[kBwdMaxProblems];
  int32_t start[kBwdMaxProblems + 1];
  int32_t n;
};
// Work items (workgroups) of one problem.
int64_t bwd_tiles(const BwdGemm& P);
hipError_t launch_gemm_bwd(BwdLaunch& L, bool a_kcontig, bool b_kcontig, int epilogue,
                           hipStream_t s);
// The same work items with float32 operands and outputs (the SwiGLU epilogue
// writes float32 da, db); no scaled copy (C2).
hipError_t launch_gemm_bwd_f32(BwdLaunch& L, bool a_kcontig, bool b_kcontig, int epilogue,
                               hipStream_t s);

// SwiGLU backward of one expert group, fused with the recomputation of its
// gate and up products: for rows r of group s and columns f < F
//   a = X[xrow(r)] Wg_s[:, f],  b = X[xrow(r)] Wu_s[:, f],  dh = DY[r] Wd_s[f, :]^T
//   DAB[r, f] = bf16(dh b SiLU'(a)),  DAB[r, F + f] = bf16(dh SiLU(a))
// (+ s * ab_group). Rows: the two kSwigluBwdBM-row halves of each tile of a
// kGemmBigBM-row plan over m_off, or rows [0, M) of each group s < G.
constexpr int kSwigluBwdBM = 128;
struct SwigluBwdProblem {
  const void* X;
  const int32_t* x_rows;
  int64_t ldx;
  const void* DY;
  int64_t ldy;
  const void* Wg;
  const void* Wu;
  const void* Wd;
  int64_t w_group;
  void* DAB;
  int64_t ldab, ab_group;
  const int32_t* m_off;
  const int32_t* plan;
  int32_t M, d, F, G, n_tiles_n, max_m_tiles;
};
struct SwigluBwdLaunch {
  SwigluBwdProblem p[2];
  int32_t n, tiles0;
};
hipError_t launch_swiglu_bwd(const SwigluBwdLaunch& L, hipStream_t s);

// Upstream rows of the expert products and the gate gradients, one token per
// wave: for kept slots j of token t (row = row_of_slot[t, j])
//   dy_routed[row] = bf16(gate[t, j] dy[t]),  dgate[t, j] = <dy[t], y_routed[row]>
// (dgate 0 for dropped slots), dy_shared[t] = bf16(dy[t]) when non-null, and
// the token rows of the expert products x_perm[row] = x[t] when non-null.
struct CombineBwdArgs {
  const float* dy;
  const void* x;             // [T, d] in the activation type
  void* x_perm;              // [R_max, d] in the activation type, or null
  const float* y_routed;
  const int32_t* row_of_slot;
  const float* topk_gate;
  void* dy_routed;           // [R_max, d]: bf16, or float32 when f32
  uint16_t* dy_shared;       // bf16 layers only, or null
  float* dgate;
  int64_t T;
  int32_t d, k;
  int32_t f32;               // float32 layer: no rounding of the routed rows
};
hipError_t launch_combine_bwd(const CombineBwdArgs& a, hipStream_t s);

// Gradient of the router logits, one token per wave, rounded to bf16 (or kept
// in float32 for float32 layers).
struct RouterBwdArgs {
  const float* logits;       // [T, E], logit_bias included
  const int32_t* topk_idx;   // [T, k]
  const float* topk_gate;    // [T, k]
  const float* dgate;        // [T, k]
  const int32_t* counts;     // [E] pre-drop slot counts
  void* dl;                  // [T, E] out: bf16, or float32 when f32_out
  int64_t T;
  int32_t E, k, score, renorm;
  float aux_scale;           // d(loss)/d(aux) * aux_coef * E / T
  int32_t f32_out;
};
hipError_t launch_router_bwd(const RouterBwdArgs& a, hipStream_t s);

// dx[t] = (dx[t] + dx_shared[t]) + sum over kept slots j, ascending, of
// dx_rows[row_of_slot[t, j]]; dx_shared may be null.
struct DxGatherArgs {
  const float* dx_rows;
  const float* dx_shared;
  const int32_t* row_of_slot;
  float* dx;
  int64_t T;
  int32_t d, k;
};
hipError_t launch_dx_gather(const DxGatherArgs& a, hipStream_t s);

// out[g * n + i] = sum over c < chunks, ascending, of part[(g * chunks + c) * n + i]
// for g < groups, i < n (n multiple of 4).
hipError_t launch_reduce_chunks(const float* part, float* out, int64_t groups, int64_t chunks,
                                int64_t n, hipStream_t s);

// Backward of rank-r experts: the steps between its products.
// h[row, f] = bf16(SiLU(ab[row, f]) * ab[row, F + f]) for rows < *rows.
hipError_t launch_swiglu_h(const float* ab, uint16_t* h, const int32_t* rows, int64_t R_max,
                           int F, hipStream_t s);
// ds[e, i] = sum over the rows of expert e, in order, of p[row, i] q[row, i].
struct LowRankDsJob {
  const float* p;
  int64_t ldp;
  const float* q;
  int64_t ldq;
  float* ds;                 // [E, r]
};
struct LowRankDsJobs {
  LowRankDsJob job[3];
  int32_t n;
  const int32_t* offsets;
  int32_t E, r;
};
hipError_t launch_ds_sum(const LowRankDsJobs& J, hipStream_t s);

// Records a failed HIP call's text for moe_last_error(); returns MOE_EHIP.
int report_hip_error(hipError_t e);
// The whole layer forward on a given workspace (api.cpp), and its argument
// validation alone, which touches no device.
int layer_forward_on(const moe_config* c, int64_t T, const void* x, const moe_weights* w,
                     moe_outputs* o, void* ws, size_t ws_bytes, void* stream);
int layer_forward_check(const moe_config* c, int64_t T, const void* x, const moe_weights* w,
                        const moe_outputs* o, size_t* ws_bytes_out);

}  // namespace moe
