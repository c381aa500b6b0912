// Routing and dispatch kernels of the MoE layer on gfx950.
//
//   topk   : scores, top-k selection, gates, per-block expert histogram and
//            per-block sums of the routing probabilities (router top-k of the
//            Quartz model card Architecture table; sigmoid scoring with a
//            balancing bias on the Sutra-1.3B "48 + 1 experts" card)
//   scan   : per-expert totals, capacity, exclusive prefix sums (dropless or
//            capacity routing: dormouse "dropless MoE" card, Moonfrost stacking
//            card), aux statistic (0.01-weighted balancing loss, research page
//            Architecture), and the grouped-GEMM tile list
//   rank   : each slot's position in its expert's token-ordered queue, drops,
//            row_of_slot and sorted_token
//   gather : x_perm[row] = x[sorted_token[row]]
//
// Nothing here uses floating-point atomics: every sum is taken in a fixed
// order, so routing outputs and the aux statistic are bitwise reproducible.

#include <float.h>

#include "moe_device.h"
#include "moe_internal.h"
#include "route_score.h"
#include "route_tail.h"

namespace moe {
namespace {

// ---------------------------------------------------------------------------
// top-k (many experts): one wave per token, the waves of a workgroup sharing
// one tb-token block, tb / nwaves consecutive tokens per wave. Lane l owns
// experts l, l + 64, ... and caches its best two (key, expert) pairs, in the
// selection order (larger key first, then the lower expert). Each of the
// k + 1 rounds takes the wave-wide maximum key; a single lane holding it wins
// (found with a ballot), several lanes holding it (equal keys) fall back to
// the lowest expert id among them. The winner moves its second pair up. A
// lane that wins twice has no cached pair left: before the next round it
// re-scans its experts ranked after the last one it gave away. Everything
// per token is branch-free apart from wave-uniform control flow: experts past
// E carry key -inf. The next token's logit row is loaded while the current
// one is reduced, and a token's outputs are stored after that load is issued
// (stores count in vmcnt, so earlier stores would hold up the wait for it).
// ---------------------------------------------------------------------------
// Threads per workgroup: as many waves as the per-lane registers allow
// (EPL logits, keys, scores and sums).
template <int EPL, int R>
constexpr int topk_threads() {
  return EPL <= 4 ? 1024 : (EPL <= 16 ? 512 : 256);
}

template <int EPL, int R, bool SIG>
__global__ void __launch_bounds__((topk_threads<EPL, R>())) topk_kernel(TopkArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  int* s_cnt = reinterpret_cast<int*>(smem_raw);                 // [E]
  float* s_ps = reinterpret_cast<float*>(smem_raw) + a.E;        // [E] or [waves][E]

  const int E = a.E, k = a.k;
  const int lane = lane_id();
  // wave-uniform, so token indices and row descriptors live in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int blk = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    s_cnt[e] = 0;
    s_ps[e] = 0.f;
  }
  __syncthreads();

  float psum[EPL], sbias[EPL];
#pragma unroll
  for (int m = 0; m < EPL; ++m) {
    psum[m] = 0.f;
    const int e = lane + 64 * m;
    sbias[m] = SIG && a.select_bias && e < E ? a.select_bias[e] : 0.f;
  }

  const int rounds = min(k + 1, E);
  const int nwaves = blockDim.x >> 6;
  const int per_wave = a.tb / nwaves;
  const int64_t t_begin = (int64_t)blk * a.tb + wave * per_wave;
  const int64_t t_end = min(a.T, t_begin + per_wave);

  // a token's logit row through a buffer descriptor of exactly E floats:
  // lanes past E read 0 from the hardware's range check, with one address
  // register and immediate offsets for the whole row
  float nxt[EPL];
  auto load_row = [&](int64_t t) {
    // t is the same in every lane: say so, so that the descriptor is built
    // in scalar registers (a per-lane one would need a waterfall loop)
    // (readfirstlane returns a signed int: both halves go through uint32_t,
    // so that the low word is never sign-extended into the high one)
    const uint64_t base = reinterpret_cast<uint64_t>(a.logits + t * E);
    const uint32_t hi = static_cast<uint32_t>(
        __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(base >> 32))));
    const uint32_t lo = static_cast<uint32_t>(
        __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(base))));
    const uint64_t ubase = (static_cast<uint64_t>(hi) << 32) | lo;
    const __amdgpu_buffer_rsrc_t row = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void*>(ubase), (short)0, E * 4, 0x00020000);
#pragma unroll
    for (int m = 0; m < EPL; ++m)
      nxt[m] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(row, (lane + 64 * m) * 4, 0, 0));
  };
  if (t_begin < t_end) load_row(t_begin);
  int64_t out_t = -1;
  int out_id = 0;
  float out_gate = 0.f, out_margin = 0.f;
  auto store_out = [&]() {
    if (out_t >= 0) {
      if (lane < k) {
        a.topk_idx[out_t * k + lane] = out_id;
        a.topk_gate[out_t * k + lane] = out_gate;
      }
      if (lane == 0 && a.topk_margin) a.topk_margin[out_t] = out_margin;
    }
  };

  for (int64_t t = t_begin; t < t_end; ++t) {
    // scores of this lane's experts (SIG: sigmoid(l), else the logit) and
    // their selection keys
    float sc[EPL], key[EPL];
#pragma unroll
    for (int m = 0; m < EPL; ++m) {
      const bool ok = lane + 64 * m < E;
      const float l = nxt[m];
      if (SIG) sc[m] = 1.0f / (1.0f + __expf(-l));
      key[m] = ok ? (SIG ? sc[m] + sbias[m] : l) : -INFINITY;
    }
    store_out();
    load_row(min(t + 1, t_end - 1));

    int my_id;
    float my_gate, mg;
    score_token<EPL, R, SIG>(key, sc, E, k, rounds, a.renorm, psum, s_cnt, my_id, my_gate, mg);
    out_t = t;
    out_id = my_id;
    out_gate = my_gate;
    out_margin = mg;
  }
  store_out();

  // per-block probability sums, the waves' partials added in wave order: each
  // wave's partials in an LDS row of its own, then each thread sums its
  // experts' rows (one barrier); without room for the rows, the waves add
  // into one row in turn (a barrier each). Both give the same sums.
  if (a.wave_rows) {
#pragma unroll
    for (int m = 0; m < EPL; ++m) {
      const int e = lane + 64 * m;
      if (e < E) s_ps[wave * E + e] = psum[m];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
      float p = 0.f;
      for (int w = 0; w < nwaves; ++w) p += s_ps[w * E + e];
      a.blk_counts[(int64_t)blk * E + e] = s_cnt[e];
      a.blk_psum[(int64_t)blk * E + e] = p;
    }
    return;
  }
  for (int w = 0; w < nwaves; ++w) {
    if (wave == w) {
#pragma unroll
      for (int m = 0; m < EPL; ++m) {
        const int e = lane + 64 * m;
        if (e < E) s_ps[e] += psum[m];
      }
    }
    __syncthreads();
  }
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    a.blk_counts[(int64_t)blk * E + e] = s_cnt[e];
    a.blk_psum[(int64_t)blk * E + e] = s_ps[e];
  }
}

// ---------------------------------------------------------------------------
// scan: one workgroup of 1024 threads.
// ---------------------------------------------------------------------------
__device__ int block_scan_excl(int v, int* smem, int& total) {
  const int lane = lane_id(), wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int incl = wave_incl_scan_i32(v);
  if (lane == 63) smem[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const int wi = wave_incl_scan_i32(lane < nw ? smem[lane] : 0);
    if (lane < nw) smem[lane] = wi;
  }
  __syncthreads();
  const int base = wave > 0 ? smem[wave - 1] : 0;
  total = smem[nw - 1];
  __syncthreads();
  return base + incl - v;
}

// Sum over the workgroup in a fixed order (a wave's prefix sum, then waves in
// order).
__device__ double block_sum_fixed(double v, double* smem) {
  const int lane = lane_id(), wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = lane63_f64(wave_incl_scan_f64(v));
  if (lane == 0) smem[wave] = v;
  __syncthreads();
  double tot = 0.0;
  for (int w = 0; w < nw; ++w) tot += smem[w];
  __syncthreads();
  return tot;
}

// Column pass of the scan for experts [c0, c0 + CW): per-expert totals of the
// block tables and each block's exclusive prefix (slots of the expert in
// earlier blocks, i.e. earlier tokens). 1024 threads: the blocks are split
// over 1024 / CW row groups, each summing its consecutive blocks.
template <int kColReg>
__device__ void scan_columns(const ScanArgs& a, int c0, int CW, int* s_part, float* s_fpart,
                             int* cnt_out, float* psum_out) {
  const int E = a.E, nblk = a.nblk;
  const int tid = threadIdx.x;
  const int RG = 1024 / CW;
  const int rg = tid / CW, cl = tid - rg * CW;
  const int per = (nblk + RG - 1) / RG;
  const int b0 = min(nblk, rg * per), b1 = min(nblk, b0 + per);
  const int e = c0 + cl;
  // a range of up to kColReg blocks is read once, all loads in flight, and
  // kept in registers for the prefix pass below
  const bool in_reg = b1 - b0 <= kColReg;
  int creg[kColReg];
  int cs = 0;
  float ps = 0.f;
  if (e < E && in_reg) {
#pragma unroll
    for (int i = 0; i < kColReg; ++i)
      creg[i] = b0 + i < b1 ? a.blk_counts[(int64_t)(b0 + i) * E + e] : 0;
#pragma unroll
    for (int i = 0; i < kColReg; ++i) {
      cs += creg[i];
      if (b0 + i < b1) ps += a.blk_psum[(int64_t)(b0 + i) * E + e];
    }
  } else if (e < E) {
#pragma unroll 8
    for (int b = b0; b < b1; ++b) {
      cs += a.blk_counts[(int64_t)b * E + e];
      ps += a.blk_psum[(int64_t)b * E + e];
    }
  }
  s_part[tid] = cs;
  s_fpart[tid] = ps;
  __syncthreads();
  if (rg == 0 && e < E) {
    int run = 0;
    float pr = 0.f;
    for (int g = 0; g < RG; ++g) {
      const int c = s_part[g * CW + cl];
      s_part[g * CW + cl] = run;
      run += c;
      pr += s_fpart[g * CW + cl];
    }
    cnt_out[e] = run;
    psum_out[e] = pr;
  }
  __syncthreads();
  if (e < E) {
    int run = s_part[tid];
    if (in_reg) {
#pragma unroll
      for (int i = 0; i < kColReg; ++i) {
        if (b0 + i < b1) a.blk_base[(int64_t)(b0 + i) * E + e] = run;
        run += creg[i];
      }
    } else {
#pragma unroll 8
      for (int b = b0; b < b1; ++b) {
        a.blk_base[(int64_t)b * E + e] = run;
        run += a.blk_counts[(int64_t)b * E + e];
      }
    }
  }
  __syncthreads();
}

__device__ __forceinline__ int scan_cw(int E) { return E <= 16 ? 16 : (E <= 32 ? 32 : 64); }

// Many experts: one workgroup per 16 experts (64 row groups of the blocks, so
// that many CUs share the latency-bound reads), totals to global memory.
constexpr int kScanColsW = 16;
__global__ void __launch_bounds__(1024) scan_cols_kernel(ScanArgs a) {
  __shared__ int s_part[1024];
  __shared__ float s_fpart[1024];
  scan_columns<16>(a, blockIdx.x * kScanColsW, kScanColsW, s_part, s_fpart, a.counts,
                   a.psum_tot);
}

// FUSED: the column pass runs here (few experts); otherwise the totals come
// from scan_cols_kernel.
template <bool FUSED>
__global__ void __launch_bounds__(1024) scan_kernel(ScanArgs a) {
  __shared__ int s_part[1024];
  __shared__ float s_fpart[1024];
  __shared__ int s_i[16];
  __shared__ double s_d[16];
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  int* s_cnt = reinterpret_cast<int*>(smem_raw);                  // [E]
  float* s_P = reinterpret_cast<float*>(smem_raw) + a.E;          // [E]

  const int E = a.E;
  const int tid = threadIdx.x;
  // 1) per-expert totals and the block prefix
  if (FUSED) {
    const int CW = scan_cw(E);
    for (int c0 = 0; c0 < E; c0 += CW) scan_columns<8>(a, c0, CW, s_part, s_fpart, s_cnt, s_P);
  } else {
    for (int e = tid; e < E; e += blockDim.x) {
      s_cnt[e] = a.counts[e];
      s_P[e] = a.psum_tot[e];
    }
    __syncthreads();
  }

  // 2) capacity, prefix sum of kept counts, drops
  const int epT = (E + blockDim.x - 1) / blockDim.x;
  const int e0 = tid * epT;
  int local_kept = 0, local_drop = 0;
  for (int e = e0; e < min(E, e0 + epT); ++e) {
    const int c = s_cnt[e];
    const int kp = a.capacity > 0 ? min(c, a.capacity) : c;
    local_kept += kp;
    local_drop += c - kp;
  }
  int total_kept;
  const int row_start = block_scan_excl(local_kept, s_i, total_kept);
  int total_drop;
  (void)block_scan_excl(local_drop, s_i, total_drop);
  int pos = row_start;
  for (int e = e0; e < min(E, e0 + epT); ++e) {
    const int c = s_cnt[e];
    const int kp = a.capacity > 0 ? min(c, a.capacity) : c;
    a.counts[e] = c;
    a.kept[e] = kp;
    a.offsets[e] = pos;
    pos += kp;
  }
  if (tid == 0) {
    a.offsets[E] = total_kept;
    a.n_dropped[0] = total_drop;
  }

  // 3) aux statistic: f_i = counts_i / (T k), P_i = psum_i / T
  const double Tk = (double)a.T * a.k;
  double part = 0.0;
  for (int e = e0; e < min(E, e0 + epT); ++e) {
    const double fe = a.T > 0 ? (double)s_cnt[e] / Tk : 0.0;
    const double Pe = a.T > 0 ? (double)s_P[e] / (double)a.T : 0.0;
    part += fe * Pe;
    if (a.f) a.f[e] = (float)fe;
    if (a.P) a.P[e] = (float)Pe;
  }
  const double tot = block_sum_fixed(part, s_d);
  if (tid == 0) {
    const double raw = (double)E * tot;
    a.aux[0] = (float)raw;
    a.aux[1] = (float)(a.aux_coef * raw);
  }

  // 4) tile list of the routed grouped GEMM: ceil(kept / plan_bm) M-tiles per
  //    expert, (expert, first row) in expert order
  if (a.plan) {
    int local = 0;
    for (int e = e0; e < min(E, e0 + epT); ++e) {
      const int c = s_cnt[e];
      const int kp = a.capacity > 0 ? min(c, a.capacity) : c;
      local += (kp + a.plan_bm - 1) / a.plan_bm;
    }
    int total;
    int tp = block_scan_excl(local, s_i, total);
    int row = row_start;
    for (int e = e0; e < min(E, e0 + epT); ++e) {
      const int c = s_cnt[e];
      const int kp = a.capacity > 0 ? min(c, a.capacity) : c;
      for (int r = 0; r < kp; r += a.plan_bm) {
        a.plan[1 + 2 * tp] = e;
        a.plan[2 + 2 * tp] = row + r;
        ++tp;
      }
      row += kp;
    }
    if (tid == 0) a.plan[0] = total;
  }
}

// Few experts (E <= 64): the blocks are split into 16 contiguous parts, one
// wave each, lane e summing expert e over its part; after one workgroup
// barrier every wave writes the block prefix of its part and wave 0 alone
// derives the per-expert outputs with wave-wide scans, so the kernel is two
// rounds of global loads and no further synchronisation.
constexpr int kScanParts = 16;
constexpr int kScanReg = 16;   // a part of at most this many blocks stays in registers

__global__ void __launch_bounds__(1024) scan_small_kernel(ScanArgs a) {
  __shared__ int s_c[kScanParts][64];
  __shared__ float s_p[kScanParts][64];
  const int E = a.E, nblk = a.nblk;
  const int e = lane_id(), part = threadIdx.x >> 6;
  const bool ve = e < E;
  const int b0 = (int)((int64_t)part * nblk / kScanParts);
  const int b1 = (int)((int64_t)(part + 1) * nblk / kScanParts);
  const bool in_reg = b1 - b0 <= kScanReg;

  // 1) this part's totals, blocks in order
  int creg[kScanReg];
  int cs = 0;
  float ps = 0.f;
  if (ve && in_reg) {
    float preg[kScanReg];
#pragma unroll
    for (int i = 0; i < kScanReg; ++i) {
      const bool in = b0 + i < b1;
      creg[i] = in ? a.blk_counts[(int64_t)(b0 + i) * E + e] : 0;
      preg[i] = in ? a.blk_psum[(int64_t)(b0 + i) * E + e] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < kScanReg; ++i) {
      cs += creg[i];
      ps += preg[i];
    }
  } else if (ve) {
#pragma unroll 8
    for (int b = b0; b < b1; ++b) {
      cs += a.blk_counts[(int64_t)b * E + e];
      ps += a.blk_psum[(int64_t)b * E + e];
    }
  }
  s_c[part][e] = cs;
  s_p[part][e] = ps;
  __syncthreads();

  // 2) block prefix: slots of expert e in the blocks before each block
  if (ve) {
    int base = 0;
    for (int q = 0; q < part; ++q) base += s_c[q][e];
    if (in_reg) {
#pragma unroll
      for (int i = 0; i < kScanReg; ++i) {
        if (b0 + i < b1) a.blk_base[(int64_t)(b0 + i) * E + e] = base;
        base += creg[i];
      }
    } else {
      for (int b = b0; b < b1; ++b) {
        a.blk_base[(int64_t)b * E + e] = base;
        base += a.blk_counts[(int64_t)b * E + e];
      }
    }
  }
  if (part != 0) return;

  // 3) wave 0: totals and probability sums, then the per-expert outputs
  int c = 0;
  float P = 0.f;
  if (ve) {
    for (int q = 0; q < kScanParts; ++q) {
      c += s_c[q][e];
      P += s_p[q][e];
    }
  }
  scan_outputs(a, c, P);
}

// ---------------------------------------------------------------------------
// rank: one wave per block of tb tokens. Slots are visited in token order (t,
// then j) 64 at a time; lanes holding the same expert are found with ballots
// over the id bits, and each lane's position is the expert's running count
// plus the number of lower lanes with that expert.
// ---------------------------------------------------------------------------
// Four blocks per workgroup; each wave copies its block's base counts and the
// expert offsets into its own LDS rows.
__global__ void __launch_bounds__(256) rank_kernel(RankArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  const int E = a.E;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  int* cnt = reinterpret_cast<int*>(smem_raw) + wave * 2 * E;
  int* offs = cnt + E;
  const int b = blockIdx.x * 4 + wave;
  if (b >= a.nblk) return;
  BlockIds B;
  load_block_ids(a, b, B);
  for (int e = lane; e < E; e += 64) {
    cnt[e] = a.blk_base[(int64_t)b * E + e];
    offs[e] = a.offsets[e];
  }
  __builtin_amdgcn_wave_barrier();
  rank_block(a, b, B, cnt, offs);
}

// Blocks of at most 64 slots (one chunk) and many experts: no running count
// crosses chunks, so each lane reads just its own expert's base and first row
// instead of the wave copying both tables of E entries.
__global__ void __launch_bounds__(256) rank_one_chunk_kernel(RankArgs a) {
  const int E = a.E, k = a.k;
  const int lane = lane_id();
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (b >= a.nblk) return;
  const int64_t s_begin = (int64_t)b * a.tb * k;
  const int64_t s_end = min(a.T, (int64_t)(b + 1) * a.tb) * k;
  const int64_t s = s_begin + lane;
  const bool valid = s < s_end;
  const int e = valid ? a.topk_idx[s] : 0;
  const int base = valid ? a.blk_base[(int64_t)b * E + e] : 0;
  const int off = valid ? a.offsets[e] : 0;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  uint64_t match = __ballot(valid);
  for (int bit = 0; bit < nbits; ++bit) {
    const bool on = (e >> bit) & 1;
    const uint64_t bb = __ballot(valid && on);
    match &= on ? bb : ~bb;
  }
  if (valid) {
    const int pos = base + __popcll(match & lanemask_lt());
    const bool keep = a.capacity == 0 || pos < a.capacity;
    const int row = keep ? off + pos : -1;
    a.row_of_slot[s] = row;
    if (keep) a.sorted_token[row] = (int32_t)(s / k);
    if (a.dropped) a.dropped[s] = keep ? 0 : 1;
  }
}

// ---------------------------------------------------------------------------
// scan and rank in one launch, for the layer call with few experts (E <= 64)
// and few blocks (nblk <= kScanParts * kScanReg): every workgroup derives the
// per-expert totals and its blocks' prefixes from the block tables itself,
// 16 waves summing one part of the blocks each as scan_small_kernel does
// (nblk * E * 4 bytes read from L2 per workgroup, less than the cost of a
// second launch and its wait); workgroup 0 also writes the per-expert
// outputs and the tile list; then wave w of workgroup g ranks block 16 g + w
// from the bases and offsets kept in LDS. One more workgroup, the launch's
// last, sums the routing probabilities and writes the aux statistic.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(1024) scan_rank_small_kernel(ScanArgs a, RankArgs r) {
  __shared__ int s_c[kScanParts][64];
  __shared__ float s_p[kScanParts][64];
  __shared__ int s_base[kScanParts][64];   // the bases of blocks g0 .. g0 + 15
  __shared__ int s_off[64];
  const int E = a.E, nblk = a.nblk;
  const int e = lane_id(), part = threadIdx.x >> 6;
  const bool ve = e < E;
  const bool lead = blockIdx.x == 0;
  // the launch's last workgroup only sums the probabilities and writes the
  // aux statistic, off the ranking workgroups' path
  const bool aux = blockIdx.x == gridDim.x - 1;
  const int g0 = kScanParts * blockIdx.x;
  const int rb = g0 + part;   // the block this wave ranks
  BlockIds B;
  if (rb < nblk) load_block_ids(r, rb, B);

  // 1) this part's totals, blocks in order (at most kScanReg of them)
  const int b0 = (int)((int64_t)part * nblk / kScanParts);
  const int b1 = (int)((int64_t)(part + 1) * nblk / kScanParts);
  int creg[kScanReg];
#pragma unroll
  for (int i = 0; i < kScanReg; ++i)
    creg[i] = ve && b0 + i < b1 ? a.blk_counts[(int64_t)(b0 + i) * E + e] : 0;
  float ps = 0.f;
  if (aux) {
    float preg[kScanReg];
#pragma unroll
    for (int i = 0; i < kScanReg; ++i)
      preg[i] = ve && b0 + i < b1 ? a.blk_psum[(int64_t)(b0 + i) * E + e] : 0.f;
#pragma unroll
    for (int i = 0; i < kScanReg; ++i) ps += preg[i];
  }
  int cs = 0;
#pragma unroll
  for (int i = 0; i < kScanReg; ++i) cs += creg[i];
  s_c[part][e] = cs;
  s_p[part][e] = ps;
  __syncthreads();
  if (aux) {
    if (part == 0) {
      int c = 0;
      float P = 0.f;
      if (ve) {
        for (int q = 0; q < kScanParts; ++q) {
          c += s_c[q][e];
          P += s_p[q][e];
        }
      }
      scan_outputs_aux(a, c, P);
    }
    return;
  }

  // 2) the bases of this workgroup's blocks, written by the wave holding each
  //    block's part, and the experts' first rows
  int base = 0;
  for (int q = 0; q < part; ++q) base += s_c[q][e];
#pragma unroll
  for (int i = 0; i < kScanReg; ++i) {
    const int b = b0 + i;
    if (b < b1 && b >= g0 && b < g0 + kScanParts) s_base[b - g0][e] = base;
    base += creg[i];
  }
  if (part == 0) {
    int c = 0;
    if (ve)
      for (int q = 0; q < kScanParts; ++q) c += s_c[q][e];
    // 3) workgroup 0 writes the per-expert outputs; every workgroup keeps
    //    the first rows
    int excl;
    if (lead) {
      excl = scan_outputs_rows(a, c);
    } else {
      const int kp = ve ? (a.capacity > 0 ? min(c, a.capacity) : c) : 0;
      excl = wave_incl_scan_i32(kp) - kp;
    }
    s_off[e] = excl;
  }
  __syncthreads();

  // 4) rank this wave's block
  if (rb < nblk) rank_block(r, rb, B, s_base[part], s_off);
}

// ---------------------------------------------------------------------------
// bias update (loss-free balancing): select_bias[e] += gamma * sign(T k - E
// counts[e]), the integer comparison of expert e's pre-drop slot count with
// the mean, one float32 addition per expert.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) bias_update_kernel(const int32_t* counts, float* bias,
                                                          int E, int64_t Tk, float gamma) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= E) return;
  const int64_t diff = Tk - (int64_t)E * counts[e];
  const float step = diff > 0 ? gamma : (diff < 0 ? -gamma : 0.f);
  bias[e] = bias[e] + step;
}

// ---------------------------------------------------------------------------
// gather: RPW rows per wave, C 16-byte pieces per lane and row. The wave's
// tokens come in one load, then every piece of its RPW rows is requested
// before the first store (RPW C pieces in flight per lane); rows longer than
// 64 C pieces take several such blocks.
// ---------------------------------------------------------------------------
template <int RPW, int C>
__global__ void __launch_bounds__(256) gather_kernel(const unsigned char* x,
                                                     const int32_t* sorted_token,
                                                     const int32_t* offsets, int E,
                                                     int64_t row_bytes, unsigned char* out) {
  const int64_t rows = offsets[E];
  const int lane = lane_id();
  const int nchunk = (int)(row_bytes >> 4);
  const int64_t step = (int64_t)gridDim.x * 4 * RPW;
  for (int64_t r0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW; r0 < rows;
       r0 += step) {
    int tk = 0;
    if (lane < RPW && r0 + lane < rows) tk = sorted_token[r0 + lane];
    for (int cb = 0; cb < nchunk; cb += 64 * C) {
      u32x4 v[RPW][C];
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        const int64_t t = __builtin_amdgcn_readlane(tk, i);
        const u32x4* src = reinterpret_cast<const u32x4*>(x + t * row_bytes);
#pragma unroll
        for (int j = 0; j < C; ++j) {
          const int c = cb + lane + 64 * j;
          if (r0 + i < rows && c < nchunk) v[i][j] = src[c];
        }
      }
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        u32x4* dst = reinterpret_cast<u32x4*>(out + (r0 + i) * row_bytes);
#pragma unroll
        for (int j = 0; j < C; ++j) {
          const int c = cb + lane + 64 * j;
          if (r0 + i < rows && c < nchunk) dst[c] = v[i][j];
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  const int nblk = (int)((a.T + a.tb - 1) / a.tb);
  if (nblk == 0) return hipSuccess;
  const int epl = (a.E + 63) / 64;
  const int k1 = a.k + 1;
  // LDS: counts [E] and the waves' probability-sum rows [waves][E] when they
  // fit in 48 KiB, else one shared row
  auto args = [&](int threads, size_t& shm) {
    TopkArgs b = a;
    const int nw = threads / 64;
    const size_t rows = (size_t)a.E * 4 * (1 + nw);
    b.wave_rows = rows <= 48 * 1024 ? nw : 0;
    shm = b.wave_rows ? rows : (size_t)a.E * 8;
    return b;
  };
#define MOE_TOPK(EPLV, KM)                                                                   \
  do {                                                                                       \
    size_t shm = 0;                                                                          \
    const TopkArgs b = args(topk_threads<EPLV, KM>(), shm);                                  \
    if (a.score == MOE_SIGMOID)                                                              \
      hipLaunchKernelGGL((topk_kernel<EPLV, KM, true>), dim3(nblk),                          \
                         dim3(topk_threads<EPLV, KM>()), shm, s, b);                         \
    else                                                                                     \
      hipLaunchKernelGGL((topk_kernel<EPLV, KM, false>), dim3(nblk),                         \
                         dim3(topk_threads<EPLV, KM>()), shm, s, b);                         \
  } while (0)
#define MOE_TOPK_K(EPLV)                \
  do {                                  \
    if (k1 <= 4) MOE_TOPK(EPLV, 4);     \
    else if (k1 <= 8) MOE_TOPK(EPLV, 8); \
    else MOE_TOPK(EPLV, 16);            \
  } while (0)
  if (epl <= 1) MOE_TOPK_K(1);
  else if (epl <= 2) MOE_TOPK_K(2);
  else if (epl <= 4) MOE_TOPK_K(4);
  else if (epl <= 8) MOE_TOPK_K(8);
  else if (epl <= 16) MOE_TOPK_K(16);
  else if (epl <= 32) MOE_TOPK_K(32);
  else MOE_TOPK_K(64);
#undef MOE_TOPK_K
#undef MOE_TOPK
  return hipGetLastError();
}

hipError_t launch_scan(const ScanArgs& a, hipStream_t s) {
  if (a.E <= 64) {
    hipLaunchKernelGGL(scan_small_kernel, dim3(1), dim3(1024), 0, s, a);
  } else if (!a.psum_tot) {
    hipLaunchKernelGGL(scan_kernel<true>, dim3(1), dim3(1024), (size_t)a.E * 8, s, a);
  } else {
    hipLaunchKernelGGL(scan_cols_kernel, dim3((a.E + kScanColsW - 1) / kScanColsW), dim3(1024),
                       0, s, a);
    hipLaunchKernelGGL(scan_kernel<false>, dim3(1), dim3(1024), (size_t)a.E * 8, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_scan_rank(const ScanArgs& a, const RankArgs& r, hipStream_t s) {
  if (a.nblk == 0) return hipSuccess;
  if (a.E > 64 || a.nblk > kScanParts * kScanReg || (int64_t)r.tb * r.k > 64 * kMaxChunks ||
      r.nblk != a.nblk)
    return hipErrorInvalidValue;
  // the ranking workgroups, then one for the aux statistic
  hipLaunchKernelGGL(scan_rank_small_kernel, dim3((a.nblk + kScanParts - 1) / kScanParts + 1),
                     dim3(1024), 0, s, a, r);
  return hipGetLastError();
}

hipError_t launch_rank(const RankArgs& a, hipStream_t s) {
  if (a.nblk == 0) return hipSuccess;
  if ((int64_t)a.tb * a.k > 64 * kMaxChunks) return hipErrorInvalidValue;   // ids in registers
  if ((int64_t)a.tb * a.k <= 64 && a.E > 64)
    hipLaunchKernelGGL(rank_one_chunk_kernel, dim3((a.nblk + 3) / 4), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(rank_kernel, dim3((a.nblk + 3) / 4), dim3(256), (size_t)a.E * 32, s, a);
  return hipGetLastError();
}

hipError_t launch_bias_update(const int32_t* counts, float* bias, int E, int64_t Tk, float gamma,
                              hipStream_t s) {
  if (E <= 0) return hipSuccess;
  hipLaunchKernelGGL(bias_update_kernel, dim3((E + 255) / 256), dim3(256), 0, s, counts, bias, E,
                     Tk, gamma);
  return hipGetLastError();
}

hipError_t launch_gather(const void* x, const int32_t* sorted_token, const int32_t* offsets,
                         int32_t E, int64_t r_max, int64_t row_bytes, void* x_perm,
                         hipStream_t s) {
  if (r_max == 0) return hipSuccess;
  if (row_bytes % 16) return hipErrorInvalidValue;
  const int64_t nchunk = row_bytes / 16;
  const unsigned char* xs = static_cast<const unsigned char*>(x);
  unsigned char* xp = static_cast<unsigned char*>(x_perm);
  // workgroups of four waves, RPW rows each, at most 16384 workgroups; eight
  // 16-byte pieces in flight per lane (RPW C = 8) measured best from d = 768
  // to 1536 (Quartz shape, cold: 15 us against 17.4 for one row per wave)
  auto grid = [&](int rpw) {
    const int64_t g = (r_max + 4 * rpw - 1) / (4 * rpw);
    return dim3((unsigned)(g < 16384 ? g : 16384));
  };
#define MOE_GATHER(RPWV, CV)                                                                 \
  hipLaunchKernelGGL((gather_kernel<RPWV, CV>), grid(RPWV), dim3(256), 0, s, xs, sorted_token, \
                     offsets, E, row_bytes, xp)
  if (nchunk <= 64) MOE_GATHER(8, 1);
  else if (nchunk <= 128) MOE_GATHER(4, 2);
  else if (nchunk <= 256) MOE_GATHER(2, 4);
  else MOE_GATHER(1, 8);
#undef MOE_GATHER
  return hipGetLastError();
}

}  // namespace moe
