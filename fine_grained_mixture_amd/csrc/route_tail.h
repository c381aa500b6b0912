// Device functions shared by the routing kernels: the per-expert outputs of
// the scan (one wave) and the ranking of one routing block (one wave).
#pragma once

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// One wave, lane e = expert e (E <= 64), given expert e's pre-drop slot count
// c: capacity, counts, kept, offsets, drops and the tile list of the routed
// grouped GEMM. Returns expert e's first row.
__device__ inline int scan_outputs_rows(const ScanArgs& a, int c) {
  const int E = a.E;
  const int e = lane_id();
  const bool ve = e < E;
  const int kp = ve ? (a.capacity > 0 ? min(c, a.capacity) : c) : 0;
  const int incl = wave_incl_scan_i32(kp);
  const int excl = incl - kp;
  const int total_kept = lane63_i32(incl);
  const int drop = lane63_i32(wave_incl_scan_i32(ve ? c - kp : 0));
  if (ve) {
    a.counts[e] = c;
    a.kept[e] = kp;
    a.offsets[e] = excl;
  }
  if (e == 0) {
    a.offsets[E] = total_kept;
    a.n_dropped[0] = drop;
  }

  // tile list of the routed grouped GEMM, (expert, first row) in expert order
  if (a.plan) {
    const int nt = (kp + a.plan_bm - 1) / a.plan_bm;
    const int ti = wave_incl_scan_i32(nt);
    const int total = lane63_i32(ti);
    int tp = ti - nt;
    for (int r = 0; r < kp; r += a.plan_bm, ++tp) {
      a.plan[1 + 2 * tp] = e;
      a.plan[2 + 2 * tp] = excl + r;
    }
    if (e == 0) a.plan[0] = total;
  }
  return excl;
}

// One wave, lane e = expert e: the aux statistic from expert e's pre-drop
// slot count c and probability sum P: f_e = c / (T k), P_e = P / T.
__device__ inline void scan_outputs_aux(const ScanArgs& a, int c, float P) {
  const int E = a.E;
  const int e = lane_id();
  const bool ve = e < E;
  const double fe = ve && a.T > 0 ? (double)c / ((double)a.T * a.k) : 0.0;
  const double Pe = ve && a.T > 0 ? (double)P / (double)a.T : 0.0;
  if (ve && a.f) a.f[e] = (float)fe;
  if (ve && a.P) a.P[e] = (float)Pe;
  const double prod = lane63_f64(wave_incl_scan_f64(fe * Pe));
  if (e == 0) {
    const double raw = (double)E * prod;
    a.aux[0] = (float)raw;
    a.aux[1] = (float)(a.aux_coef * raw);
  }
}

// Both of the above. Returns expert e's first row.
__device__ inline int scan_outputs(const ScanArgs& a, int c, float P) {
  scan_outputs_aux(a, c, P);
  return scan_outputs_rows(a, c);
}

constexpr int kMaxChunks = 15;   // tb * k / 64 slots of a block, tb * k <= 960

struct BlockIds {
  int ids[kMaxChunks];
};

// Every expert id of block b, requested at once.
__device__ __forceinline__ void load_block_ids(const RankArgs& a, int b, BlockIds& B) {
  const int lane = lane_id();
  const int64_t s_begin = (int64_t)b * a.tb * a.k;
  const int64_t s_end = min(a.T, (int64_t)(b + 1) * a.tb) * a.k;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    const int64_t s = s_begin + 64 * c + lane;
    B.ids[c] = s < s_end ? a.topk_idx[s] : -1;
  }
}

// Ranks block b. cnt[e] (this wave's own LDS row) starts as the slots of
// expert e in earlier blocks and is advanced; offs[e] is the expert's first
// row.
__device__ __forceinline__ void rank_block(const RankArgs& a, int b, const BlockIds& B, int* cnt,
                                           const int* offs) {
  const int E = a.E, k = a.k;
  const int lane = lane_id();
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const int64_t s_begin = (int64_t)b * a.tb * k;
  const int64_t s_end = min(a.T, (int64_t)(b + 1) * a.tb) * k;
  const uint64_t lt = lanemask_lt();
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    const int64_t s = s_begin + 64 * c + lane;
    if (s_begin + 64 * c >= s_end) break;
    const bool valid = s < s_end;
    const int e = valid ? B.ids[c] : 0;
    uint64_t match = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool on = (e >> bit) & 1;
      const uint64_t bb = __ballot(valid && on);
      match &= on ? bb : ~bb;
    }
    const int rank = __popcll(match & lt);
    const int total = __popcll(match);
    int pos = 0;
    if (valid) pos = cnt[e] + rank;
    __builtin_amdgcn_wave_barrier();
    if (valid && rank == 0) cnt[e] = pos + total;
    __builtin_amdgcn_wave_barrier();
    if (valid) {
      const bool keep = a.capacity == 0 || pos < a.capacity;
      const int row = keep ? offs[e] + pos : -1;
      a.row_of_slot[s] = row;
      if (keep) a.sorted_token[row] = (int32_t)(s / k);
      if (a.dropped) a.dropped[s] = keep ? 0 : 1;
    }
  }
}

}  // namespace moe
