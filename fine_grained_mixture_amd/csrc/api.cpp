// C ABI of the MoE layer: argument validation, workspace layout and the
// sequence of kernel launches. This file launches through the kernel files'
// launch_* helpers and performs no device-to-host transfer of any kind: every
// data-dependent size (expert row counts, tile lists) stays on the device.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <string>

#include "../../include/moe.h"
#include "moe_internal.h"

namespace moe {
namespace {

thread_local std::string g_last_error;
thread_local const char* g_stage_names[64];
thread_local int g_n_stages = 0;

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// A legal layer: d and F multiples of 8, 1 <= k <= E <= 4096. Layers that are
// legal but outside what the kernels cover are told apart by supported_config.
bool valid_config(const moe_config* c) {
  if (!c) return false;
  if (c->hidden <= 0 || c->hidden % 8) return false;
  if (c->ffn <= 0 || c->ffn % 8) return false;
  if (c->top_k < 1) return false;
  if (c->n_routed < c->top_k || c->n_routed > 4096) return false;
  if (c->n_shared < 0 || c->n_shared > 64) return false;
  if (c->rank < 0) return false;
  if (c->score != MOE_SOFTMAX && c->score != MOE_SIGMOID) return false;
  if (c->score == MOE_SIGMOID && c->renorm_topk != 1) return false;
  if (c->renorm_topk != 0 && c->renorm_topk != 1) return false;
  if (c->capacity < 0) return false;
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16 && c->dtype != MOE_FP8) return false;
  return true;
}

// What the library's kernels cover beyond valid_config: low-rank experts up to
// the fused kernel's rank-64 tiles, fp8 rows that fit the quantiser's registers.
bool supported_config(const moe_config* c) {
  // the products' tiles: d and F whole 64-column chunks; the top-k keeps at
  // most 15 selections per token in registers
  if (c->hidden % 64 || c->ffn % 64 || c->top_k > 15) return false;
  // the bf16 tile kernel's fp32 epilogue addresses a tile's 256 output rows
  // of pitch d with 32-bit byte offsets
  if (c->dtype != MOE_F32 && c->hidden >= (1 << 21)) return false;
  // low-rank experts: bf16 with rank 16, 32, 48 or 64; fp8 factors with rank 64
  if (c->rank != 0 && (c->rank > 64 || c->rank % 16 || c->dtype == MOE_F32 ||
                       (c->dtype == MOE_FP8 && c->rank != 64)))
    return false;
  // fp8: the rows entering the dense products (x over d, h over F, the shared
  // h over S F) are quantised whole in registers, up to 4096 values
  if (c->dtype == MOE_FP8 && (c->hidden > 4096 || (int64_t)c->n_shared * c->ffn > 4096 ||
                              c->ffn > 4096))
    return false;
  return true;
}

// x, W_r and the activations are bf16 for MOE_BF16 and MOE_FP8.
bool act_bf16(const moe_config* c) { return c->dtype != MOE_F32; }
bool fp8(const moe_config* c) { return c->dtype == MOE_FP8; }

size_t elem_size(const moe_config* c) { return act_bf16(c) ? 2 : 4; }

int plan_bm(const moe_config* c) {
  if (c->dtype == MOE_F32) return kGemmBM_F32;
  return c->rank > 0 ? kLowRankBM : kGemmBigBM;
}

}  // namespace

// Token groups of 16 per workgroup of the fused router: about one workgroup
// per CU, and a block of 16 G tokens keeps its k-slot ids within the rank
// kernel's registers (16 G k <= 64 * 15).
int route_small_groups(int64_t T, int k) {
  static int n_cu = 0;
  if (n_cu == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      n_cu = n;
    else
      n_cu = 256;
  }
  const int64_t n16 = (T + kRouteBlockSmall - 1) / kRouteBlockSmall;
  int64_t G = (n16 + n_cu - 1) / n_cu;
  G = std::min<int64_t>(G, 60 / k);
  return (int)std::max<int64_t>(G, 1);
}

namespace {

// bf16 layers with few experts use the fused router (16-token blocks).
bool fused_router(const moe_config* c) {
  return act_bf16(c) && c->n_routed <= kRouteSmallMaxE;
}
int route_tb(const moe_config* c, int64_t T) {
  return fused_router(c) ? kRouteBlockSmall * route_small_groups(T, c->top_k) : kRouteBlock;
}

struct Layout {
  int64_t T = 0, R = 0, nblk = 0, max_tiles = 0;
  int tb = kRouteBlock;
  size_t logits = 0, blk_counts = 0, blk_base = 0, blk_psum = 0, psum_tot = 0, plan = 0;
  size_t h = 0, h_sh = 0, y_perm = 0, y_sh = 0;
  // fp8 experts: quantised rows and their scales
  size_t xq = 0, xs = 0, xq_sh = 0, xs_sh = 0, hq = 0, hs = 0, hq_sh = 0, hs_sh = 0;
  size_t total = 0;
};

int64_t max_rows(const moe_config* c, int64_t T) {
  const int64_t tk = T * c->top_k;
  if (c->capacity > 0) return std::min<int64_t>(tk, (int64_t)c->n_routed * c->capacity);
  return tk;
}

Layout make_layout(const moe_config* c, int64_t T) {
  Layout L;
  const int64_t E = c->n_routed, d = c->hidden, F = c->ffn, S = c->n_shared;
  const size_t es = elem_size(c);
  L.T = T;
  L.R = max_rows(c, T);
  L.tb = route_tb(c, T);
  L.nblk = ceil_div(T, L.tb);
  L.max_tiles = ceil_div(L.R, plan_bm(c)) + E;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  L.logits = take((size_t)T * E * 4);
  L.blk_counts = take((size_t)L.nblk * E * 4);
  L.blk_base = take((size_t)L.nblk * E * 4);
  L.blk_psum = take((size_t)L.nblk * E * 4);
  L.psum_tot = take((size_t)E * 4);
  L.plan = take((size_t)(1 + 2 * L.max_tiles) * 4);
  // low-rank experts keep their h on chip: no routed h rows
  L.h = take(c->rank > 0 ? 0 : (size_t)L.R * F * es);
  L.h_sh = take((size_t)T * S * F * es);
  L.y_perm = take((size_t)L.R * d * 4);
  L.y_sh = take(S > 0 ? (size_t)T * d * 4 : 0);
  if (c->dtype == MOE_FP8) {
    // x rows (layer) or x_perm rows (stage); low-rank experts quantise no
    // routed activations (only their factors are fp8)
    const int64_t xr = c->rank > 0 ? 0 : std::max<int64_t>(L.R, T);
    const int64_t hr = c->rank > 0 ? 0 : L.R;
    L.xq = take((size_t)xr * d);
    L.xs = take((size_t)xr * 4);
    L.xq_sh = take((size_t)T * d);
    L.xs_sh = take((size_t)T * 4);
    L.hq = take((size_t)hr * F);
    L.hs = take((size_t)hr * 4);
    L.hq_sh = take((size_t)T * S * F);
    L.hs_sh = take((size_t)T * 4);
  }
  L.total = off;
  return L;
}

template <class T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<unsigned char*>(ws) + off);
}

// Launch bookkeeping shared by the streams of one call: stage names for
// moe_stage_name() and, when timing, a start and an end event per stage
// recorded on the stream the stage runs on.
struct Timeline {
  void** events = nullptr;
  int n_events = 0;
  int n = 0;
  hipError_t err = hipSuccess;
};

struct Runner {
  hipStream_t stream;
  Timeline* tl;

  // Launches one kernel (launch() returns its hipError_t) as stage `name`.
  template <class F>
  void run(const char* name, F&& launch) {
    const int i = tl->n++;
    if (i < 64) g_stage_names[i] = name;
    hipEvent_t* ev = reinterpret_cast<hipEvent_t*>(tl->events);
    const bool timed = ev && 2 * i + 1 < tl->n_events;
    if (timed) check(hipEventRecord(ev[2 * i], stream));
    check(launch());
    if (timed) check(hipEventRecord(ev[2 * i + 1], stream));
  }
  bool check(hipError_t e) {
    if (e != hipSuccess && tl->err == hipSuccess) tl->err = e;
    return e == hipSuccess;
  }
};

int hip_fail(hipError_t e) {
  g_last_error = hipGetErrorString(e);
  return MOE_EHIP;
}

int check_ws(const moe_config* c, int64_t T, void* ws, size_t ws_bytes, Layout& L) {
  L = make_layout(c, T);
  if (L.total > 0 && !ws) return MOE_EWORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % kAlign) return MOE_EWORKSPACE;
  if (ws_bytes < L.total) return MOE_EWORKSPACE;
  return MOE_OK;
}

int check_common(const moe_config* c, int64_t T) {
  if (!valid_config(c)) return MOE_EINVAL;
  if (T < 0 || T * c->top_k >= ((int64_t)1 << 31)) return MOE_EINVAL;
  if (max_rows(c, T) * std::max(c->hidden, c->ffn) >= ((int64_t)1 << 40)) return MOE_EINVAL;
  if (!supported_config(c)) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

// Per-token arrays may be NULL when T == 0 (empty tensors have no storage).
bool route_outputs_ok(const moe_outputs* o, int64_t T) {
  return o && o->counts && o->kept && o->offsets && o->n_dropped && o->aux &&
         (T == 0 || (o->topk_idx && o->topk_gate));
}
bool permute_outputs_ok(const moe_outputs* o, int64_t T) {
  return o && (T == 0 || (o->row_of_slot && o->sorted_token));
}
bool expert_weights_ok(const moe_config* c, const moe_weights* w, bool routed, bool shared) {
  if (!w) return false;
  if (c->dtype == MOE_FP8) {
    if (routed && c->rank == 0 && (!w->w_gate_scale || !w->w_up_scale || !w->w_down_scale))
      return false;
    if (routed && c->rank > 0 &&
        (!w->u_gate_scale || !w->u_up_scale || !w->u_down_scale || !w->v_gate_scale ||
         !w->v_up_scale || !w->v_down_scale))
      return false;
    if (shared && c->n_shared > 0 && (!w->sh_gate_scale || !w->sh_up_scale || !w->sh_down_scale))
      return false;
  }
  if (routed) {
    if (c->rank == 0) {
      if (!w->w_gate || !w->w_up || !w->w_down) return false;
    } else {
      if (!w->u_gate || !w->s_gate || !w->v_gate || !w->u_up || !w->s_up || !w->v_up ||
          !w->u_down || !w->s_down || !w->v_down)
        return false;
    }
  }
  if (shared && c->n_shared > 0 && (!w->sh_gate || !w->sh_up || !w->sh_down)) return false;
  return true;
}

// ---- stage bodies (no validation) ------------------------------------------
ScanArgs scan_args(const moe_config* c, const Layout& L, moe_outputs* o, void* ws,
                   bool with_plan) {
  ScanArgs s{};
  s.blk_counts = at<int32_t>(ws, L.blk_counts);
  s.blk_psum = at<float>(ws, L.blk_psum);
  s.blk_base = at<int32_t>(ws, L.blk_base);
  s.counts = o->counts;
  s.kept = o->kept;
  s.offsets = o->offsets;
  s.n_dropped = o->n_dropped;
  s.aux = o->aux;
  s.f = o->f;
  s.P = o->P;
  s.psum_tot = at<float>(ws, L.psum_tot);
  s.plan = with_plan ? at<int32_t>(ws, L.plan) : nullptr;
  s.plan_bm = plan_bm(c);
  s.nblk = (int32_t)L.nblk;
  s.E = c->n_routed;
  s.k = c->top_k;
  s.capacity = c->capacity;
  s.T = L.T;
  s.aux_coef = c->aux_coef;
  return s;
}

RankArgs rank_args(const moe_config* c, const Layout& L, moe_outputs* o, void* ws) {
  RankArgs r{};
  r.topk_idx = o->topk_idx;
  r.blk_base = at<int32_t>(ws, L.blk_base);
  r.offsets = o->offsets;
  r.row_of_slot = o->row_of_slot;
  r.sorted_token = o->sorted_token;
  r.dropped = o->dropped;
  r.T = L.T;
  r.E = c->n_routed;
  r.k = c->top_k;
  r.capacity = c->capacity;
  r.nblk = (int32_t)L.nblk;
  r.tb = L.tb;
  return r;
}

// The layer call ranks in the scan's launch when the fused router made few
// blocks of few experts.
bool scan_rank_fused(const moe_config* c, const Layout& L) {
  return fused_router(c) && L.T > 0 && L.nblk <= 256;
}

// One routing block for the whole batch in the layer call: the fused router
// also scans and ranks it.
bool route_tail_fused(const moe_config* c, const Layout& L) {
  return fused_router(c) && L.T > 0 && L.nblk == 1;
}

void run_route(Runner& R, const moe_config* c, const Layout& L, const void* x,
               const moe_weights* w, moe_outputs* o, void* ws, bool with_plan,
               bool scan = true, bool tail = false) {
  const int64_t T = L.T;
  const int E = c->n_routed;
  float* logits = at<float>(ws, L.logits);
  if (T > 0 && fused_router(c)) {
    RouteSmallArgs r{};
    r.x = x;
    r.w_router = w->w_router;
    r.logit_bias = w->logit_bias;
    r.select_bias = c->score == MOE_SIGMOID ? w->select_bias : nullptr;
    r.topk_idx = o->topk_idx;
    r.topk_gate = o->topk_gate;
    r.topk_margin = o->topk_margin;
    r.blk_counts = at<int32_t>(ws, L.blk_counts);
    r.blk_psum = at<float>(ws, L.blk_psum);
    r.logits = logits;
    r.T = T;
    r.d = c->hidden;
    r.E = E;
    r.k = c->top_k;
    r.score = c->score;
    r.renorm = c->renorm_topk;
    if (tail) {
      const ScanArgs sa = scan_args(c, L, o, ws, with_plan);
      const RankArgs ra = rank_args(c, L, o, ws);
      R.run("route_scan_rank", [&] {
        return launch_route_small(r, L.tb / kRouteBlockSmall, R.stream, &sa, &ra);
      });
      return;
    }
    R.run("route", [&] {
      return launch_route_small(r, L.tb / kRouteBlockSmall, R.stream);
    });
  } else if (T > 0) {
    GemmLaunch G{};
    GemmProblem& p = G.p[0];
    p.A = x;
    p.lda = c->hidden;
    p.B0 = w->w_router;
    p.ldb = E;
    p.C = logits;
    p.ldc = E;
    p.col_bias = w->logit_bias;
    p.M = (int32_t)T;
    p.N = E;
    p.K = c->hidden;
    p.G = 1;
    const int bn = act_bf16(c) ? 128 : 64;
    const int bm = act_bf16(c) ? kGemmBM : kGemmBM_F32;
    p.n_tiles_n = (int32_t)ceil_div(E, bn);
    p.max_m_tiles = (int32_t)ceil_div(T, bm);
    G.n_problems = 1;
    G.tiles0 = p.max_m_tiles * p.n_tiles_n;
    if (act_bf16(c) && E % 8 == 0) {
      // many experts: the large-tile kernel (256 x 128 tiles)
      p.n_tiles_n = (int32_t)ceil_div(E, 128);
      p.max_m_tiles = (int32_t)ceil_div(T, kGemmBigBM);
      G.tiles0 = p.max_m_tiles * p.n_tiles_n;
      R.run("router_gemm", [&] { return launch_gemm_big(G, kEpiStoreF32, R.stream); });
    } else {
      R.run("router_gemm", [&] {
        return act_bf16(c) ? launch_gemm_bf16(G, kEpiStoreF32, R.stream)
                                    : launch_gemm_f32(G, kEpiStoreF32, R.stream);
      });
    }

    TopkArgs t{};
    t.logits = logits;
    t.select_bias = c->score == MOE_SIGMOID ? w->select_bias : nullptr;
    t.topk_idx = o->topk_idx;
    t.topk_gate = o->topk_gate;
    t.topk_margin = o->topk_margin;
    t.blk_counts = at<int32_t>(ws, L.blk_counts);
    t.blk_psum = at<float>(ws, L.blk_psum);
    t.T = T;
    t.E = E;
    t.k = c->top_k;
    t.score = c->score;
    t.renorm = c->renorm_topk;
    t.tb = L.tb;
    R.run("topk", [&] { return launch_topk(t, R.stream); });
  }
  if (!scan) return;
  const ScanArgs s = scan_args(c, L, o, ws, with_plan);
  R.run("scan", [&] { return launch_scan(s, R.stream); });
}

void run_rank(Runner& R, const moe_config* c, const Layout& L, moe_outputs* o, void* ws) {
  if (L.T == 0) return;
  const RankArgs r = rank_args(c, L, o, ws);
  R.run("rank", [&] { return launch_rank(r, R.stream); });
}

void run_scan_rank(Runner& R, const moe_config* c, const Layout& L, moe_outputs* o, void* ws) {
  const ScanArgs s = scan_args(c, L, o, ws, true);
  const RankArgs r = rank_args(c, L, o, ws);
  R.run("scan_rank", [&] { return launch_scan_rank(s, r, R.stream); });
}


// fp8 expert FFN: quantise the rows entering the gate/up products, the fp8
// gate/up GEMM with SwiGLU (h in bf16, as in the bf16 path), quantise h rows,
// the fp8 down GEMM. Routed rows A = a_routed gathered through a_rows (token
// rows) or the dispatched rows themselves; shared rows A = a_shared.
void run_ffn_fp8(Runner& R, const moe_config* c, const Layout& L, bool routed, bool shared,
                 const void* a_routed, const int32_t* a_rows, const int32_t* offsets,
                 const void* a_shared, const moe_weights* w, float* y_routed, float* y_shared,
                 void* ws) {
  const int64_t T = L.T, d = c->hidden, F = c->ffn, S = c->n_shared, E = c->n_routed;
  void* h = at<void>(ws, L.h);
  void* h_sh = at<void>(ws, L.h_sh);
  const int32_t* plan = at<int32_t>(ws, L.plan);
  uint8_t* xq = at<uint8_t>(ws, L.xq);
  float* xs = at<float>(ws, L.xs);
  uint8_t* xq_sh = at<uint8_t>(ws, L.xq_sh);
  float* xs_sh = at<float>(ws, L.xs_sh);
  const uint16_t* src_r = static_cast<const uint16_t*>(a_routed);
  const uint16_t* src_s = static_cast<const uint16_t*>(a_shared);
  // token rows gathered by the GEMM (the layer call): one quantisation of x
  // serves the routed and the shared products
  const bool same_rows = routed && shared && a_rows && src_r == src_s;
  if (routed) {
    R.run("quant_x", [&] {
      return a_rows ? launch_quant_rows(src_r, d, T, (int32_t)d, nullptr, xq, xs, R.stream)
                    : launch_quant_rows(src_r, d, L.R, (int32_t)d, offsets + E, xq, xs, R.stream);
    });
  }
  if (shared && !same_rows) {
    R.run("quant_x_shared", [&] {
      return launch_quant_rows(src_s, d, T, (int32_t)d, nullptr, xq_sh, xs_sh, R.stream);
    });
  }
  const uint8_t* xq_shared = same_rows ? xq : xq_sh;
  const float* xs_shared = same_rows ? xs : xs_sh;
  const bool both = routed && shared;
  {
    GemmLaunch G{};
    int np = 0;
    if (shared) {
      GemmProblem& p = G.p[np++];
      p.A = xq_shared;
      p.lda = d;
      p.a_scale = xs_shared;
      p.B0 = w->sh_gate;
      p.B1 = w->sh_up;
      p.b_group_stride = F * d;
      p.ldb = d;
      p.b_scale0 = w->sh_gate_scale;
      p.b_scale1 = w->sh_up_scale;
      p.b_scale_group = F;
      p.C = h_sh;
      p.ldc = S * F;
      p.c_group_col = F;
      p.M = (int32_t)T;
      p.N = (int32_t)F;
      p.K = (int32_t)d;
      p.G = (int32_t)S;
      p.n_tiles_n = (int32_t)(F / 64);
      p.max_m_tiles = (int32_t)(S * ceil_div(T, kGemmBigBM));
    }
    if (routed) {
      GemmProblem& p = G.p[np++];
      p.A = xq;
      p.a_rows = a_rows;
      p.lda = d;
      p.a_scale = xs;
      p.B0 = w->w_gate;
      p.B1 = w->w_up;
      p.b_group_stride = F * d;
      p.ldb = d;
      p.b_scale0 = w->w_gate_scale;
      p.b_scale1 = w->w_up_scale;
      p.b_scale_group = F;
      p.C = h;
      p.ldc = F;
      p.row_off = offsets;
      p.plan = plan;
      p.N = (int32_t)F;
      p.K = (int32_t)d;
      p.G = (int32_t)E;
      p.n_tiles_n = (int32_t)(F / 64);
      p.max_m_tiles = (int32_t)L.max_tiles;
    }
    G.n_problems = np;
    G.tiles0 = G.p[0].max_m_tiles * G.p[0].n_tiles_n;
    R.run(both || routed ? "gate_up_gemm" : "shared_gate_up_gemm",
          [&] { return launch_gemm_fp8(G, kEpiSwiGLU, R.stream); });
  }
  uint8_t* hq = at<uint8_t>(ws, L.hq);
  float* hs = at<float>(ws, L.hs);
  uint8_t* hq_sh = at<uint8_t>(ws, L.hq_sh);
  float* hs_sh = at<float>(ws, L.hs_sh);
  R.run("quant_h", [&] {
    hipError_t e = hipSuccess;
    if (routed)
      e = launch_quant_rows(static_cast<const uint16_t*>(h), F, L.R, (int32_t)F, offsets + E, hq,
                            hs, R.stream);
    if (e == hipSuccess && shared)
      e = launch_quant_rows(static_cast<const uint16_t*>(h_sh), S * F, T, (int32_t)(S * F),
                            nullptr, hq_sh, hs_sh, R.stream);
    return e;
  });
  {
    GemmLaunch G{};
    int np = 0;
    if (shared) {
      GemmProblem& p = G.p[np++];
      p.A = hq_sh;
      p.lda = S * F;
      p.a_scale = hs_sh;
      p.B0 = w->sh_down;          // [d, S F]: the S experts' down projections summed
      p.ldb = S * F;
      p.b_scale0 = w->sh_down_scale;
      p.C = y_shared;
      p.ldc = d;
      p.M = (int32_t)T;
      p.N = (int32_t)d;
      p.K = (int32_t)(S * F);
      p.G = 1;
      p.n_tiles_n = (int32_t)ceil_div(d, 128);
      p.max_m_tiles = (int32_t)ceil_div(T, kGemmBigBM);
    }
    if (routed) {
      GemmProblem& p = G.p[np++];
      p.A = hq;
      p.lda = F;
      p.a_scale = hs;
      p.B0 = w->w_down;
      p.b_group_stride = d * F;
      p.ldb = F;
      p.b_scale0 = w->w_down_scale;
      p.b_scale_group = d;
      p.C = y_routed;
      p.ldc = d;
      p.row_off = offsets;
      p.plan = plan;
      p.N = (int32_t)d;
      p.K = (int32_t)F;
      p.G = (int32_t)E;
      p.n_tiles_n = (int32_t)ceil_div(d, 128);
      p.max_m_tiles = (int32_t)L.max_tiles;
      // streaming stores for routed rows that cannot stay in the Infinity
      // Cache, as in the bf16 down product
      p.c_stream = L.R * d * 4 > kInfinityCacheBytes ? 1 : 0;
    }
    G.n_problems = np;
    G.tiles0 = G.p[0].max_m_tiles * G.p[0].n_tiles_n;
    R.run(both || routed ? "down_gemm" : "shared_down_gemm",
          [&] { return launch_gemm_fp8(G, kEpiStoreF32, R.stream); });
  }
}

// Expert FFN launches. Routed rows: A = a_routed with optional row gather;
// shared rows: A = a_shared (T rows).
void run_ffn(Runner& R, const moe_config* c, const Layout& L, bool routed, bool shared,
             const void* a_routed, const int32_t* a_rows, const int32_t* offsets,
             const void* a_shared, const moe_weights* w, float* y_routed, float* y_shared,
             void* ws, float* saved_ab = nullptr) {
  const int64_t T = L.T, d = c->hidden, F = c->ffn, S = c->n_shared;
  const bool bf = c->dtype == MOE_BF16;
  // tile shapes: bf16 256 x 128 (gate/up: 256 x (64 + 64)); fp32 64 x 64
  const int bm = bf ? kGemmBigBM : kGemmBM_F32;
  const int bn_dual = 64, bn = bf ? 128 : 64;
  shared = shared && S > 0 && T > 0;
  routed = routed && L.R > 0;
  if (!routed && !shared) return;
  void* h = at<void>(ws, L.h);
  void* h_sh = at<void>(ws, L.h_sh);
  const int32_t* plan = at<int32_t>(ws, L.plan);

  // decode-sized batches: the weight-streaming skinny kernel
  const bool skinny = bf && T <= kSkinnyMaxT;
  auto launch = [&](const GemmLaunch& G, int epi, const char* name) {
    R.run(name, [&] {
      if (skinny) return launch_gemm_skinny(G, epi, R.stream, T <= 2, (int)T);
      return bf ? launch_gemm_big(G, epi, R.stream) : launch_gemm_f32(G, epi, R.stream);
    });
  };

  if (routed && c->rank > 0) {
    LowRankArgs lr{};
    lr.A = a_routed;
    lr.a_rows = a_rows;
    lr.lda = d;
    lr.u_gate = w->u_gate;
    lr.s_gate = w->s_gate;
    lr.v_gate = w->v_gate;
    lr.u_up = w->u_up;
    lr.s_up = w->s_up;
    lr.v_up = w->v_up;
    lr.u_down = w->u_down;
    lr.s_down = w->s_down;
    lr.v_down = w->v_down;
    lr.offsets = offsets;
    lr.plan = plan;
    lr.y = y_routed;
    lr.d = (int32_t)d;
    lr.F = (int32_t)F;
    lr.E = c->n_routed;
    lr.max_tiles = (int32_t)L.max_tiles;
    lr.rank = c->rank;
    if (fp8(c)) {
      lr.fp8 = 1;
      lr.u_gate_scale = w->u_gate_scale;
      lr.u_up_scale = w->u_up_scale;
      lr.u_down_scale = w->u_down_scale;
      lr.v_gate_scale = w->v_gate_scale;
      lr.v_up_scale = w->v_up_scale;
      lr.v_down_scale = w->v_down_scale;
    }
    R.run("lowrank_experts", [&] { return launch_lowrank(lr, R.stream); });
  }
  if (c->rank > 0) routed = false;   // the dense launches below serve the shared experts
  if (!routed && !shared) return;
  if (fp8(c)) {
    run_ffn_fp8(R, c, L, routed, shared, a_routed, a_rows, offsets, a_shared, w, y_routed,
                y_shared, ws);
    return;
  }
  // stage names: routed and shared launches are told apart when only one
  // group is present
  const bool both = routed && shared;
  // gate/up with fused SiLU * up
  {
    GemmLaunch G{};
    int np = 0;
    if (shared) {
      GemmProblem& p = G.p[np++];
      p.A = a_shared;
      p.lda = d;
      p.B0 = w->sh_gate;
      p.B1 = w->sh_up;
      p.b_group_stride = d * F;
      p.ldb = F;
      p.C = h_sh;
      p.ldc = S * F;
      p.c_group_col = F;
      if (saved_ab) {
        p.ab = saved_ab + L.R * 2 * F;
        p.ab_ld = S * 2 * F;
        p.ab_group_col = 2 * F;
      }
      p.M = (int32_t)T;
      p.N = (int32_t)F;
      p.K = (int32_t)d;
      p.G = (int32_t)S;
      p.n_tiles_n = (int32_t)ceil_div(F, bn_dual);
      p.max_m_tiles = (int32_t)(S * ceil_div(T, bm));
    }
    if (routed) {
      GemmProblem& p = G.p[np++];
      p.A = a_routed;
      p.a_rows = a_rows;
      p.lda = d;
      p.B0 = w->w_gate;
      p.B1 = w->w_up;
      p.b_group_stride = d * F;
      p.ldb = F;
      p.C = h;
      p.ldc = F;
      if (saved_ab) {
        p.ab = saved_ab;
        p.ab_ld = 2 * F;
      }
      p.row_off = offsets;
      p.plan = plan;
      p.N = (int32_t)F;
      p.K = (int32_t)d;
      p.G = c->n_routed;
      p.n_tiles_n = (int32_t)ceil_div(F, bn_dual);
      p.max_m_tiles = (int32_t)L.max_tiles;
    }
    G.n_problems = np;
    G.tiles0 = G.p[0].max_m_tiles * G.p[0].n_tiles_n;
    launch(G, kEpiSwiGLU, both || routed ? "gate_up_gemm" : "shared_gate_up_gemm");
  }
  // down projection
  {
    GemmLaunch G{};
    int np = 0;
    if (shared) {
      GemmProblem& p = G.p[np++];
      p.A = h_sh;
      p.lda = S * F;
      p.B0 = w->sh_down;        // [S, F, d] read as [S*F, d]: the S experts summed
      p.ldb = d;
      p.C = y_shared;
      p.ldc = d;
      p.M = (int32_t)T;
      p.N = (int32_t)d;
      p.K = (int32_t)(S * F);
      p.G = 1;
      p.n_tiles_n = (int32_t)ceil_div(d, bn);
      p.max_m_tiles = (int32_t)ceil_div(T, bm);
    }
    if (routed) {
      GemmProblem& p = G.p[np++];
      p.A = h;
      p.lda = F;
      p.B0 = w->w_down;
      p.b_group_stride = F * d;
      p.ldb = d;
      p.C = y_routed;
      p.ldc = d;
      p.row_off = offsets;
      p.plan = plan;
      p.N = (int32_t)d;
      p.K = (int32_t)F;
      p.G = c->n_routed;
      p.n_tiles_n = (int32_t)ceil_div(d, bn);
      p.max_m_tiles = (int32_t)L.max_tiles;
      // the routed rows (k fp32 rows per token, read once by the combine) go
      // out as streaming stores when they cannot stay in the 256 MiB Infinity
      // Cache anyway (Sutra: 805 MB, -2% per call with warm or cold weights).
      // Rows that fit are stored normally, for the combine to find there:
      // streaming them made the Quartz layer 4% faster while its weights sat
      // in that cache, but 3-7% slower once they had been evicted.
      p.c_stream = bf && L.R * d * 4 > kInfinityCacheBytes ? 1 : 0;
    }
    G.n_problems = np;
    G.tiles0 = G.p[0].max_m_tiles * G.p[0].n_tiles_n;
    launch(G, kEpiStoreF32, both || routed ? "down_gemm" : "shared_down_gemm");
  }
}

void run_combine(Runner& R, const moe_config* c, int64_t T, const float* y_routed,
                 const float* y_shared, moe_outputs* o) {
  if (T == 0) return;
  CombineArgs a{};
  a.y_routed = y_routed;
  a.y_shared = y_shared;
  a.row_of_slot = o->row_of_slot;
  a.topk_gate = o->topk_gate;
  a.y = o->y;
  a.y_lowp = o->y_lowp;
  a.T = T;
  a.d = c->hidden;
  a.k = c->top_k;
  a.dtype = act_bf16(c) ? MOE_BF16 : MOE_F32;
  R.run("combine", [&] { return launch_combine(a, R.stream); });
}

int finish(Timeline& tl) {
  g_n_stages = tl.n;
  if (tl.err != hipSuccess) return hip_fail(tl.err);
  return MOE_OK;
}

int layer_forward(const moe_config* c, int64_t T, const void* x, const moe_weights* w,
                  moe_outputs* o, void* ws, size_t ws_bytes, void* stream, void** events,
                  int n_events) {
  int st = check_common(c, T);
  if (st) return st;
  if (!x && T > 0) return MOE_EINVAL;
  if (!w || !w->w_router || !expert_weights_ok(c, w, true, true)) return MOE_EINVAL;
  if (c->score == MOE_SOFTMAX && w->select_bias) return MOE_EINVAL;
  if (!route_outputs_ok(o, T) || !permute_outputs_ok(o, T) || (T > 0 && !o->y))
    return MOE_EINVAL;
  Layout L;
  if ((st = check_ws(c, T, ws, ws_bytes, L))) return st;
  Timeline tl{events, n_events};
  Runner R{static_cast<hipStream_t>(stream), &tl};
  float* y_perm = at<float>(ws, L.y_perm);
  float* y_sh = c->n_shared > 0 ? at<float>(ws, L.y_sh) : nullptr;
  if (route_tail_fused(c, L)) {
    run_route(R, c, L, x, w, o, ws, true, false, true);
  } else if (scan_rank_fused(c, L)) {
    run_route(R, c, L, x, w, o, ws, true, false);
    run_scan_rank(R, c, L, o, ws);
  } else {
    run_route(R, c, L, x, w, o, ws, true);
    run_rank(R, c, L, o, ws);
  }
  float* saved_ab = c->dtype == MOE_BF16 && c->rank == 0 ? o->saved_ab : nullptr;
  run_ffn(R, c, L, true, true, x, o->sorted_token, o->offsets, x, w, y_perm, y_sh, ws, saved_ab);
  run_combine(R, c, T, y_perm, y_sh, o);
  st = finish(tl);
  return st ? st : tl.n;
}


// ---- backward ---------------------------------------------------------------
// Rows of the split-K chunks of the products summed over all tokens.
constexpr int kRouterKChunk = 512;
constexpr int kSharedKChunk = 4096;

// bf16 layers with E a multiple of 8 (the router's gradient products read E
// in 16-byte pieces); rank-r experts with r a multiple of 32 (a K-step of the
// backward products) and no shared experts.
bool backward_supported(const moe_config* c) {
  if (c->dtype == MOE_F32) return c->rank == 0;   // the fp32 FMA products
  if (c->dtype != MOE_BF16 || c->n_routed % 8) return false;
  if (c->rank == 0) return true;
  return c->rank % 32 == 0 && c->rank <= 64;
}

struct BwdLayout {
  int64_t T = 0, R = 0, nch_r = 1, nch_s = 1, lr_tiles = 0;
  int32_t kch_r = 1;   // tokens per chunk of the router's weight gradient
  size_t dyr = 0, dysh = 0, dg = 0, dl = 0, dab = 0, dabsh = 0, xperm = 0, dxp = 0,
         dxsh = 0, part_r = 0, part_g = 0, part_u = 0, part_d = 0, total = 0;
  // float32 layers: the recomputed gate and up products (routed, shared)
  size_t ab32 = 0, absh32 = 0;
  // rank-r experts: the 256-row tile list, the recomputed forward chain
  // (x U, its scaled and rounded z, the gate and up products, h, h U_d, z_d)
  // and the backward's (dz_d, dz_d s_d rounded, dz_g | dz_u, their scaled
  // and rounded forms)
  size_t lr_plan = 0, ug = 0, uu = 0, dzd = 0, ud = 0, dzg = 0, dzu = 0, zgu = 0, zd = 0,
         dud = 0, dugu = 0, ab = 0, hh = 0;
};

BwdLayout make_bwd_layout(const moe_config* c, int64_t T) {
  BwdLayout B;
  const int64_t E = c->n_routed, d = c->hidden, F = c->ffn, S = c->n_shared, k = c->top_k;
  B.T = T;
  B.R = max_rows(c, T);
  // the router's weight gradient x^T dl: its (d / 256) x (E / 128) tiles split
  // over token chunks of at least kRouterKChunk, about one round of
  // workgroups in all (fewer chunks, fewer partials to write and reduce)
  {
    const int64_t tiles = ceil_div(d, kGemmBigBM) * ceil_div(E, 128);
    const int64_t most = std::max<int64_t>(1, ceil_div(T, kRouterKChunk));
    const int64_t want = std::min<int64_t>(most, std::max<int64_t>(1, ceil_div(512, tiles)));
    B.kch_r = (int32_t)(ceil_div(ceil_div(std::max<int64_t>(T, 1), want), 32) * 32);
    B.nch_r = std::max<int64_t>(1, ceil_div(T, B.kch_r));
  }
  B.nch_s = std::max<int64_t>(1, ceil_div(T, kSharedKChunk));
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  // operands of the backward products in the activation type (bf16, or
  // float32 for float32 layers, whose shared upstream rows are dy itself)
  const bool f32 = c->dtype == MOE_F32;
  const size_t es = f32 ? 4 : 2;
  B.dyr = take((size_t)B.R * d * es);
  B.dysh = take((size_t)T * d * 2 * (S > 0 && !f32));
  B.dg = take((size_t)T * k * 4);
  B.dl = take((size_t)T * E * es);
  B.dab = take((size_t)B.R * 2 * F * es);
  B.dabsh = take((size_t)T * S * 2 * F * es);
  B.xperm = take((size_t)B.R * d * es);
  B.dxp = take((size_t)B.R * d * 4);
  B.dxsh = take((size_t)T * d * 4 * (S > 0));
  B.part_r = take(B.nch_r > 1 ? (size_t)B.nch_r * d * E * 4 : 0);
  const size_t shp = (S > 0 && B.nch_s > 1) ? (size_t)S * B.nch_s * d * F * 4 : 0;
  B.part_g = take(shp);
  B.part_u = take(shp);
  B.part_d = take(shp);
  if (f32) {
    B.ab32 = take((size_t)B.R * 2 * F * 4);
    B.absh32 = take((size_t)T * S * 2 * F * 4);
  }
  if (c->rank > 0) {
    const int64_t r = c->rank, R = B.R;
    B.lr_tiles = ceil_div(R, kGemmBigBM) + E;
    B.lr_plan = take((size_t)(1 + 2 * B.lr_tiles) * 4);
    B.ug = take((size_t)R * r * 4);
    B.uu = take((size_t)R * r * 4);
    B.dzd = take((size_t)R * r * 4);
    B.ud = take((size_t)R * r * 4);
    B.dzg = take((size_t)R * r * 4);
    B.dzu = take((size_t)R * r * 4);
    B.zgu = take((size_t)R * 2 * r * 2);
    B.zd = take((size_t)R * r * 2);
    B.dud = take((size_t)R * r * 2);
    B.dugu = take((size_t)R * 2 * r * 2);
    B.ab = take((size_t)R * 2 * F * 4);
    B.hh = take((size_t)R * F * 2);
  }
  B.total = off;
  return B;
}

BwdGemm bwd_problem() {
  BwdGemm p{};
  p.n_chunks = 1;
  p.G = 1;
  p.c_split = INT32_MAX;
  return p;
}

// Backward of a layer of rank-r experts (no shared experts): the upstream
// rows, gate gradients and router gradient as for dense experts; then, per
// dispatched row of expert e (W[in, out] = U[in, r] diag(s) V[out, r]^T),
// the forward chain recomputed and the chain rule back through it:
//   ug = x U_g, zg = bf16(ug s_g), a = zg V_g^T (same for up), h = bf16(SiLU(a) b),
//   ud = h U_d, zd = bf16(ud s_d); with dY = bf16(gate dy):
//   dzd = dY V_d, dud = bf16(dzd s_d), dh = dud U_d^T -> da, db (bf16),
//   dzg = da V_g, dzu = db V_u, dug = bf16(dzg s_g), duu = bf16(dzu s_u),
//   dx rows = dug U_g^T + duu U_u^T;
//   dV_d = dY^T zd, dU_d = h^T dud, dV_g = da^T zg, dV_u = db^T zu,
//   dU_g = x^T dug, dU_u = x^T duu (summed over the expert's rows), and
//   ds = the row sums of dz * u.
void lowrank_backward(Runner& Rn, const moe_config* c, int64_t T, const void* x,
                      const moe_weights* w, const moe_outputs* o, const float* dy,
                      float aux_grad, moe_grads* g, const Layout& L, const BwdLayout& B,
                      void* fws, void* bws) {
  const int64_t E = c->n_routed, d = c->hidden, F = c->ffn, k = c->top_k, r = c->rank;
  const int64_t S = c->n_shared;
  const int64_t R = B.R;
  uint16_t* dyr = at<uint16_t>(bws, B.dyr);
  // shared experts (dense, beside the rank-r ones): their upstream rows bf16(dy),
  // da | db, input-gradient rows, and the forward's h of theirs
  uint16_t* dysh = S > 0 ? at<uint16_t>(bws, B.dysh) : nullptr;
  void* dabsh = at<void>(bws, B.dabsh);
  float* dxsh = S > 0 ? at<float>(bws, B.dxsh) : nullptr;
  const void* h_sh = at<void>(fws, L.h_sh);
  float* dg = at<float>(bws, B.dg);
  uint16_t* dl = at<uint16_t>(bws, B.dl);
  uint16_t* dab = at<uint16_t>(bws, B.dab);
  uint16_t* xperm = at<uint16_t>(bws, B.xperm);
  float* dxp = at<float>(bws, B.dxp);
  int32_t* plan = at<int32_t>(bws, B.lr_plan);
  float *ug = at<float>(bws, B.ug), *uu = at<float>(bws, B.uu), *dzd = at<float>(bws, B.dzd);
  float *ud = at<float>(bws, B.ud), *dzg = at<float>(bws, B.dzg), *dzu = at<float>(bws, B.dzu);
  uint16_t *zgu = at<uint16_t>(bws, B.zgu), *zd = at<uint16_t>(bws, B.zd);
  uint16_t *dud = at<uint16_t>(bws, B.dud), *dugu = at<uint16_t>(bws, B.dugu);
  float* ab = at<float>(bws, B.ab);
  uint16_t* hh = at<uint16_t>(bws, B.hh);
  const float* y_perm = at<float>(fws, L.y_perm);
  const float* logits = at<float>(fws, L.logits);
  const int32_t* offs = o->offsets;
  const int32_t* rows = o->offsets + E;

  // a product over the dispatched rows of each expert (the 256-row tile list)
  auto rows_problem = [&](const void* A, int64_t lda, const void* B0, int64_t ldb, int64_t bgrp,
                          float* C, int64_t ldc, int64_t N, int64_t K) {
    BwdGemm p = bwd_problem();
    p.A = A;
    p.lda = lda;
    p.B0 = B0;
    p.ldb = ldb;
    p.b_group = bgrp;
    p.C0 = C;
    p.ldc = ldc;
    p.m_off = offs;
    p.plan = plan;
    p.N = (int32_t)N;
    p.K = (int32_t)K;
    p.G = (int32_t)E;
    p.n_tiles_n = (int32_t)ceil_div(N, 128);
    p.max_m_tiles = (int32_t)B.lr_tiles;
    return p;
  };
  // a weight gradient: sum over each expert's rows of A^T B
  auto wgrad_problem = [&](const void* A, int64_t lda, const void* B0, int64_t ldb, float* C,
                           int64_t M, int64_t N) {
    BwdGemm p = bwd_problem();
    p.A = A;
    p.lda = lda;
    p.B0 = B0;
    p.ldb = ldb;
    p.C0 = C;
    p.ldc = N;
    p.c_group = M * N;
    p.k_off = offs;
    p.M = (int32_t)M;
    p.N = (int32_t)N;
    p.K = (int32_t)R;
    p.G = (int32_t)E;
    p.n_tiles_m = (int32_t)ceil_div(M, kGemmBigBM);
    p.n_tiles_n = (int32_t)ceil_div(N, 128);
    return p;
  };
  // the product's bf16 copy scaled by s of the row's expert (its rounding point)
  auto scaled = [&](BwdGemm& p, uint16_t* out, int64_t ldo, const void* s_vec) {
    p.C2 = out;
    p.ldc2 = ldo;
    p.c2_scale = static_cast<const uint16_t*>(s_vec);
    p.c2_scale_group = r;
  };

  if (T > 0) {
    CombineBwdArgs cb{};
    cb.dy = dy;
    cb.x = static_cast<const uint16_t*>(x);
    cb.x_perm = xperm;
    cb.y_routed = y_perm;
    cb.row_of_slot = o->row_of_slot;
    cb.topk_gate = o->topk_gate;
    cb.dy_routed = dyr;
    cb.dy_shared = dysh;
    cb.dgate = dg;
    cb.T = T;
    cb.d = (int32_t)d;
    cb.k = (int32_t)k;
    Rn.run("combine_bwd", [&] { return launch_combine_bwd(cb, Rn.stream); });

    if (S > 0) {
      // the shared experts' SwiGLU backward, their gate and up products recomputed
      SwigluBwdLaunch SL{};
      SwigluBwdProblem& p = SL.p[0];
      p.X = x;
      p.ldx = d;
      p.DY = dysh;
      p.ldy = d;
      p.Wg = w->sh_gate;
      p.Wu = w->sh_up;
      p.Wd = w->sh_down;
      p.w_group = d * F;
      p.DAB = dabsh;
      p.ldab = S * 2 * F;
      p.ab_group = 2 * F;
      p.M = (int32_t)T;
      p.d = (int32_t)d;
      p.F = (int32_t)F;
      p.G = (int32_t)S;
      p.n_tiles_n = (int32_t)(F / 64);
      SL.n = 1;
      SL.tiles0 = p.G * (int32_t)ceil_div(p.M, kSwigluBwdBM) * p.n_tiles_n;
      Rn.run("swiglu_bwd", [&] { return launch_swiglu_bwd(SL, Rn.stream); });
    }

    RouterBwdArgs rb{};
    rb.logits = logits;
    rb.topk_idx = o->topk_idx;
    rb.topk_gate = o->topk_gate;
    rb.dgate = dg;
    rb.counts = o->counts;
    rb.dl = dl;
    rb.T = T;
    rb.E = (int32_t)E;
    rb.k = (int32_t)k;
    rb.score = c->score;
    rb.renorm = c->renorm_topk;
    rb.aux_scale = (float)((double)aux_grad * c->aux_coef * (double)E / (double)T);
    Rn.run("router_bwd", [&] { return launch_router_bwd(rb, Rn.stream); });
    Rn.run("plan", [&] { return launch_plan(offs, (int32_t)E, kGemmBigBM, plan, Rn.stream); });

    {  // x U_g, x U_u and dY V_d, with zg = bf16(x U_g s_g), zu and dud = bf16(dzd s_d)
      BwdLaunch BL{};
      BL.p[0] = rows_problem(xperm, d, w->u_gate, r, d * r, ug, r, r, d);
      scaled(BL.p[0], zgu, 2 * r, w->s_gate);
      BL.p[1] = rows_problem(xperm, d, w->u_up, r, d * r, uu, r, r, d);
      scaled(BL.p[1], zgu + r, 2 * r, w->s_up);
      BL.p[2] = rows_problem(dyr, d, w->v_down, r, d * r, dzd, r, r, d);
      scaled(BL.p[2], dud, r, w->s_down);
      BL.n = 3;
      Rn.run("lr_in_gemm", [&] { return launch_gemm_bwd(BL, true, false, kBwdStoreF32, Rn.stream); });
    }
    {  // a = zg V_g^T, b = zu V_u^T
      BwdLaunch BL{};
      BL.p[0] = rows_problem(zgu, 2 * r, w->v_gate, r, F * r, ab, 2 * F, F, r);
      BL.p[1] = rows_problem(zgu + r, 2 * r, w->v_up, r, F * r, ab + F, 2 * F, F, r);
      BL.n = 2;
      Rn.run("lr_ab_gemm", [&] { return launch_gemm_bwd(BL, true, true, kBwdStoreF32, Rn.stream); });
    }
    Rn.run("lr_h", [&] { return launch_swiglu_h(ab, hh, rows, R, (int)F, Rn.stream); });
    {  // ud = h U_d, with zd = bf16(ud s_d)
      BwdLaunch BL{};
      BL.p[0] = rows_problem(hh, F, w->u_down, r, F * r, ud, r, r, F);
      scaled(BL.p[0], zd, r, w->s_down);
      BL.n = 1;
      Rn.run("lr_ud_gemm", [&] { return launch_gemm_bwd(BL, true, false, kBwdStoreF32, Rn.stream); });
    }
    {  // dh = dud U_d^T with the SwiGLU backward in the epilogue
      BwdLaunch BL{};
      BwdGemm& p = BL.p[0] = rows_problem(dud, r, w->u_down, r, F * r,
                                          reinterpret_cast<float*>(dab), 2 * F, F, r);
      p.ab = ab;
      p.ab_ld = 2 * F;
      p.half = (int32_t)F;
      BL.n = 1;
      Rn.run("lr_dh_gemm", [&] { return launch_gemm_bwd(BL, true, true, kBwdSwiGLU, Rn.stream); });
    }
    {  // dz_g = da V_g, dz_u = db V_u, with dug = bf16(dz_g s_g) and duu
      BwdLaunch BL{};
      BL.p[0] = rows_problem(dab, 2 * F, w->v_gate, r, F * r, dzg, r, r, F);
      scaled(BL.p[0], dugu, 2 * r, w->s_gate);
      BL.p[1] = rows_problem(dab + F, 2 * F, w->v_up, r, F * r, dzu, r, r, F);
      scaled(BL.p[1], dugu + r, 2 * r, w->s_up);
      BL.n = 2;
      Rn.run("lr_dz_gemm", [&] { return launch_gemm_bwd(BL, true, false, kBwdStoreF32, Rn.stream); });
    }
    {  // input-gradient rows [dug | duu] [U_g; U_u]^T, and the router's dl W_r^T
      BwdLaunch BL{};
      BwdGemm& p = BL.p[0] = rows_problem(dugu, 2 * r, w->u_gate, r, d * r, dxp, d, d, 2 * r);
      p.B1 = w->u_up;
      p.k_seg = (int32_t)r;
      BwdGemm& q = BL.p[1] = bwd_problem();
      q.A = dl;
      q.lda = E;
      q.B0 = w->w_router;
      q.ldb = E;
      q.C0 = g->dx;
      q.ldc = d;
      q.M = (int32_t)T;
      q.N = (int32_t)d;
      q.K = (int32_t)E;
      q.k_chunk = q.K;
      q.n_tiles_m = (int32_t)ceil_div(T, kGemmBigBM);
      q.n_tiles_n = (int32_t)ceil_div(d, 128);
      BL.n = 2;
      if (S > 0) {   // the shared experts' [da | db] [W_gate; W_up]^T
        BwdGemm& u = BL.p[BL.n++] = bwd_problem();
        u.A = dabsh;
        u.lda = S * 2 * F;
        u.B0 = w->sh_gate;
        u.B1 = w->sh_up;
        u.ldb = F;
        u.k_seg = (int32_t)F;
        u.b_seg = d * F;
        u.C0 = dxsh;
        u.ldc = d;
        u.M = (int32_t)T;
        u.N = (int32_t)d;
        u.K = (int32_t)(S * 2 * F);
        u.k_chunk = u.K;
        u.n_tiles_m = (int32_t)ceil_div(T, kGemmBigBM);
        u.n_tiles_n = (int32_t)ceil_div(d, 128);
      }
      Rn.run("dgrad_gemm", [&] { return launch_gemm_bwd(BL, true, true, kBwdStoreF32, Rn.stream); });
    }
    DxGatherArgs dxa{};
    dxa.dx_rows = dxp;
    dxa.dx_shared = dxsh;
    dxa.row_of_slot = o->row_of_slot;
    dxa.dx = g->dx;
    dxa.T = T;
    dxa.d = (int32_t)d;
    dxa.k = (int32_t)k;
    Rn.run("dx_gather", [&] { return launch_dx_gather(dxa, Rn.stream); });
  }

  {  // factor gradients, each summed over its expert's rows
    BwdLaunch BL{};
    BL.p[0] = wgrad_problem(dyr, d, zd, r, g->dv_down, d, r);
    BL.p[1] = wgrad_problem(hh, F, dud, r, g->du_down, F, r);
    BL.p[2] = wgrad_problem(dab, 2 * F, zgu, 2 * r, g->dv_gate, F, r);
    BL.p[3] = wgrad_problem(dab + F, 2 * F, zgu + r, 2 * r, g->dv_up, F, r);
    BL.p[4] = wgrad_problem(xperm, d, dugu, 2 * r, g->du_gate, d, r);
    BL.n = 5;
    Rn.run("wgrad_gemm", [&] { return launch_gemm_bwd(BL, false, false, kBwdStoreF32, Rn.stream); });
  }
  {  // du_up and the router's x^T dl (split over tokens when long)
    BwdLaunch BL{};
    BL.p[0] = wgrad_problem(xperm, d, dugu + r, 2 * r, g->du_up, d, r);
    BwdGemm& p = BL.p[1] = bwd_problem();
    p.A = x;
    p.lda = d;
    p.B0 = dl;
    p.ldb = E;
    p.C0 = B.nch_r > 1 ? at<float>(bws, B.part_r) : g->dw_router;
    p.ldc = E;
    p.c_chunk = d * E;
    p.M = (int32_t)d;
    p.N = (int32_t)E;
    p.K = (int32_t)T;
    p.k_chunk = B.nch_r > 1 ? B.kch_r : (int32_t)std::max<int64_t>(T, 1);
    p.n_chunks = (int32_t)B.nch_r;
    p.n_tiles_m = (int32_t)ceil_div(d, kGemmBigBM);
    p.n_tiles_n = (int32_t)ceil_div(E, 128);
    BL.n = 2;
    // the shared experts over all tokens (split over tokens when long)
    const bool split_s = S > 0 && B.nch_s > 1;
    const int32_t kch_s = (int32_t)(split_s ? kSharedKChunk : std::max<int64_t>(T, 1));
    if (S > 0) {
      BwdGemm& u = BL.p[BL.n++] = bwd_problem();
      u.A = h_sh;
      u.lda = S * F;
      u.a_group = F;
      u.B0 = dysh;
      u.ldb = d;
      u.C0 = split_s ? at<float>(bws, B.part_d) : g->dsh_down;
      u.ldc = d;
      u.c_group = (int64_t)B.nch_s * F * d;
      u.c_chunk = F * d;
      u.M = (int32_t)F;
      u.N = (int32_t)d;
      u.K = (int32_t)T;
      u.G = (int32_t)S;
      u.k_chunk = kch_s;
      u.n_chunks = (int32_t)B.nch_s;
      u.n_tiles_m = (int32_t)ceil_div(F, kGemmBigBM);
      u.n_tiles_n = (int32_t)ceil_div(d, 128);
      BwdGemm& v = BL.p[BL.n++] = bwd_problem();
      v.A = x;
      v.lda = d;
      v.B0 = dabsh;
      v.ldb = S * 2 * F;
      v.b_group = 2 * F;
      v.C0 = split_s ? at<float>(bws, B.part_g) : g->dsh_gate;
      v.C1 = split_s ? at<float>(bws, B.part_u) : g->dsh_up;
      v.c_split = (int32_t)F;
      v.ldc = F;
      v.c_group = (int64_t)B.nch_s * d * F;
      v.c_chunk = d * F;
      v.M = (int32_t)d;
      v.N = (int32_t)(2 * F);
      v.K = (int32_t)T;
      v.G = (int32_t)S;
      v.k_chunk = kch_s;
      v.n_chunks = (int32_t)B.nch_s;
      v.n_tiles_m = (int32_t)ceil_div(d, kGemmBigBM);
      v.n_tiles_n = (int32_t)ceil_div(2 * F, 128);
    }
    Rn.run("wgrad_gemm2", [&] { return launch_gemm_bwd(BL, false, false, kBwdStoreF32, Rn.stream); });
    if (B.nch_r > 1) {
      Rn.run("reduce_router", [&] {
        return launch_reduce_chunks(at<float>(bws, B.part_r), g->dw_router, 1, B.nch_r, d * E,
                                    Rn.stream);
      });
    }
    if (split_s) {
      Rn.run("reduce_shared", [&] {
        hipError_t e = launch_reduce_chunks(at<float>(bws, B.part_g), g->dsh_gate, S, B.nch_s,
                                            d * F, Rn.stream);
        if (e == hipSuccess)
          e = launch_reduce_chunks(at<float>(bws, B.part_u), g->dsh_up, S, B.nch_s, d * F,
                                   Rn.stream);
        if (e == hipSuccess)
          e = launch_reduce_chunks(at<float>(bws, B.part_d), g->dsh_down, S, B.nch_s, F * d,
                                   Rn.stream);
        return e;
      });
    }
  }
  {  // ds = row sums of dz * u per expert
    LowRankDsJobs J{};
    J.job[0] = LowRankDsJob{dzg, r, ug, r, g->ds_gate};
    J.job[1] = LowRankDsJob{dzu, r, uu, r, g->ds_up};
    J.job[2] = LowRankDsJob{dzd, r, ud, r, g->ds_down};
    J.n = 3;
    J.offsets = offs;
    J.E = (int32_t)E;
    J.r = (int32_t)r;
    Rn.run("lr_ds", [&] { return launch_ds_sum(J, Rn.stream); });
  }
}

int layer_backward(const moe_config* c, int64_t T, const void* x, const moe_weights* w,
                   const moe_outputs* o, const float* dy, float aux_grad, moe_grads* g,
                   const void* ws, size_t ws_bytes, void* bws, size_t bws_bytes, void* stream,
                   void** events, int n_events) {
  int st = check_common(c, T);
  if (st) return st;
  if (!backward_supported(c)) return MOE_EUNSUPPORTED;
  if (!isfinite(aux_grad)) return MOE_EINVAL;
  if (!w || !w->w_router || !expert_weights_ok(c, w, true, true)) return MOE_EINVAL;
  if (!o || !o->counts || !o->offsets) return MOE_EINVAL;
  if (T > 0 && (!x || !dy || !o->topk_idx || !o->topk_gate || !o->row_of_slot ||
                !o->sorted_token))
    return MOE_EINVAL;
  if (!g || !g->dw_router || (T > 0 && !g->dx)) return MOE_EINVAL;
  if (c->rank == 0 && (!g->dw_gate || !g->dw_up || !g->dw_down)) return MOE_EINVAL;
  if (c->rank > 0 && (!g->du_gate || !g->ds_gate || !g->dv_gate || !g->du_up || !g->ds_up ||
                      !g->dv_up || !g->du_down || !g->ds_down || !g->dv_down))
    return MOE_EINVAL;
  if (c->n_shared > 0 && (!g->dsh_gate || !g->dsh_up || !g->dsh_down)) return MOE_EINVAL;
  Layout L;
  if ((st = check_ws(c, T, const_cast<void*>(ws), ws_bytes, L))) return st;
  const BwdLayout B = make_bwd_layout(c, T);
  if (B.total > 0 && !bws) return MOE_EWORKSPACE;
  if (reinterpret_cast<uintptr_t>(bws) % kAlign || bws_bytes < B.total) return MOE_EWORKSPACE;

  void* fws = const_cast<void*>(ws);
  const int64_t E = c->n_routed, d = c->hidden, F = c->ffn, S = c->n_shared, k = c->top_k;
  const int64_t R = B.R;
  Timeline tl{events, n_events};
  Runner Rn{static_cast<hipStream_t>(stream), &tl};
  const bool f32 = c->dtype == MOE_F32;
  void* dyr = at<void>(bws, B.dyr);
  // shared upstream rows: bf16(dy), or dy itself in a float32 layer
  void* dysh = S > 0 ? (f32 ? const_cast<float*>(dy) : at<void>(bws, B.dysh)) : nullptr;
  float* dg = at<float>(bws, B.dg);
  const float* logits = at<float>(fws, L.logits);   // the forward router's
  void* dl = at<void>(bws, B.dl);
  // the products: MFMA on bf16 operands, or fp32 FMA for float32 layers
  auto gemm = [&](BwdLaunch& BL, bool akc, bool bkc, int epi) {
    return f32 ? launch_gemm_bwd_f32(BL, akc, bkc, epi, Rn.stream)
               : launch_gemm_bwd(BL, akc, bkc, epi, Rn.stream);
  };
  void* dab = at<void>(bws, B.dab);
  void* dabsh = at<void>(bws, B.dabsh);
  void* xperm = at<void>(bws, B.xperm);
  float* dxp = at<float>(bws, B.dxp);
  float* dxsh = S > 0 ? at<float>(bws, B.dxsh) : nullptr;
  const float* y_perm = at<float>(fws, L.y_perm);
  const void* h = at<void>(fws, L.h);
  const void* h_sh = at<void>(fws, L.h_sh);
  const int32_t* plan256 = at<int32_t>(fws, L.plan);
  if (c->rank > 0) {
    lowrank_backward(Rn, c, T, x, w, o, dy, aux_grad, g, L, B, fws, bws);
    st = finish(tl);
    return st ? st : tl.n;
  }

  if (T > 0) {
    // upstream rows of the expert products and the gate gradients
    CombineBwdArgs cb{};
    cb.dy = dy;
    cb.x = x;
    cb.x_perm = xperm;
    cb.y_routed = y_perm;
    cb.row_of_slot = o->row_of_slot;
    cb.topk_gate = o->topk_gate;
    cb.dy_routed = dyr;
    cb.dy_shared = f32 ? nullptr : static_cast<uint16_t*>(dysh);
    cb.dgate = dg;
    cb.T = T;
    cb.d = (int32_t)d;
    cb.k = (int32_t)k;
    cb.f32 = f32;
    Rn.run("combine_bwd", [&] { return launch_combine_bwd(cb, Rn.stream); });

    RouterBwdArgs rb{};
    rb.logits = logits;
    rb.topk_idx = o->topk_idx;
    rb.topk_gate = o->topk_gate;
    rb.dgate = dg;
    rb.counts = o->counts;
    rb.dl = dl;
    rb.T = T;
    rb.E = (int32_t)E;
    rb.k = (int32_t)k;
    rb.score = c->score;
    rb.renorm = c->renorm_topk;
    rb.aux_scale = (float)((double)aux_grad * c->aux_coef * (double)E / (double)T);
    rb.f32_out = f32;
    Rn.run("router_bwd", [&] { return launch_router_bwd(rb, Rn.stream); });

    // float32 layers (the forward keeps no products): a | b recomputed, x W_gate
    // and x W_up as one problem per weight (routed rows, then the shared
    // experts over all tokens)
    float* ab32 = f32 ? at<float>(bws, B.ab32) : nullptr;
    float* absh32 = f32 ? at<float>(bws, B.absh32) : nullptr;
    if (f32) {
      BwdLaunch BL{};
      int np = 0;
      for (int half = 0; half < 2; ++half) {
        {
          BwdGemm& p = BL.p[np++] = bwd_problem();
          p.A = xperm;
          p.lda = d;
          p.B0 = half ? w->w_up : w->w_gate;
          p.ldb = F;
          p.b_group = d * F;
          p.C0 = ab32 + half * F;
          p.ldc = 2 * F;
          p.m_off = o->offsets;
          p.plan = plan256;
          p.N = (int32_t)F;
          p.K = (int32_t)d;
          p.G = (int32_t)E;
          p.n_tiles_n = (int32_t)ceil_div(F, 128);
          p.max_m_tiles = (int32_t)L.max_tiles;
        }
        if (S > 0) {
          BwdGemm& p = BL.p[np++] = bwd_problem();
          p.A = x;
          p.lda = d;
          p.B0 = half ? w->sh_up : w->sh_gate;
          p.ldb = F;
          p.b_group = d * F;
          p.C0 = absh32 + half * F;
          p.ldc = S * 2 * F;
          p.c_group = 2 * F;
          p.M = (int32_t)T;
          p.N = (int32_t)F;
          p.K = (int32_t)d;
          p.G = (int32_t)S;
          p.k_chunk = p.K;
          p.n_tiles_m = (int32_t)ceil_div(T, kGemmBigBM);
          p.n_tiles_n = (int32_t)ceil_div(F, 128);
        }
      }
      BL.n = np;
      Rn.run("ab_gemm", [&] { return gemm(BL, true, false, kBwdStoreF32); });
    }
    const float* ab_routed = f32 ? ab32 : o->saved_ab;
    const float* ab_shared = f32 ? absh32 : (o->saved_ab ? o->saved_ab + R * 2 * F : nullptr);

    if (ab_routed) {
      // dh = dy W_down^T with the SwiGLU backward in the epilogue, on the
      // forward's saved gate and up products (shared experts, then routed)
      BwdLaunch BL{};
      int np = 0;
      if (S > 0) {
        BwdGemm& p = BL.p[np++] = bwd_problem();
        p.A = dysh;
        p.lda = d;
        p.B0 = w->sh_down;
        p.ldb = d;
        p.b_group = F * d;
        p.C0 = static_cast<float*>(dabsh);   // output in the activation type
        p.ldc = S * 2 * F;
        p.c_group = 2 * F;
        p.ab = ab_shared;
        p.ab_ld = S * 2 * F;
        p.ab_group = 2 * F;
        p.half = (int32_t)F;
        p.M = (int32_t)T;
        p.N = (int32_t)F;
        p.K = (int32_t)d;
        p.G = (int32_t)S;
        p.k_chunk = p.K;
        p.n_tiles_m = (int32_t)ceil_div(T, kGemmBigBM);
        p.n_tiles_n = (int32_t)ceil_div(F, 128);
      }
      {
        BwdGemm& p = BL.p[np++] = bwd_problem();
        p.A = dyr;
        p.lda = d;
        p.B0 = w->w_down;
        p.ldb = d;
        p.b_group = F * d;
        p.C0 = static_cast<float*>(dab);     // output in the activation type
        p.ldc = 2 * F;
        p.ab = ab_routed;
        p.ab_ld = 2 * F;
        p.half = (int32_t)F;
        p.m_off = o->offsets;
        p.plan = plan256;
        p.N = (int32_t)F;
        p.K = (int32_t)d;
        p.G = (int32_t)E;
        p.n_tiles_n = (int32_t)ceil_div(F, 128);
        p.max_m_tiles = (int32_t)L.max_tiles;
      }
      BL.n = np;
      Rn.run("dh_gemm", [&] { return gemm(BL, true, true, kBwdSwiGLU); });
    } else {
    // SwiGLU backward with the gate and up products recomputed (shared
    // experts, then routed)
      SwigluBwdLaunch SL{};
      int np = 0;
      if (S > 0) {
        SwigluBwdProblem& p = SL.p[np++];
        p.X = x;
        p.ldx = d;
        p.DY = dysh;
        p.ldy = d;
        p.Wg = w->sh_gate;
        p.Wu = w->sh_up;
        p.Wd = w->sh_down;
        p.w_group = d * F;
        p.DAB = dabsh;
        p.ldab = S * 2 * F;
        p.ab_group = 2 * F;
        p.M = (int32_t)T;
        p.d = (int32_t)d;
        p.F = (int32_t)F;
        p.G = (int32_t)S;
        p.n_tiles_n = (int32_t)(F / 64);
      }
      {
        SwigluBwdProblem& p = SL.p[np++];
        p.X = xperm;
        p.ldx = d;
        p.DY = dyr;
        p.ldy = d;
        p.Wg = w->w_gate;
        p.Wu = w->w_up;
        p.Wd = w->w_down;
        p.w_group = d * F;
        p.DAB = dab;
        p.ldab = 2 * F;
        p.m_off = o->offsets;
        p.plan = plan256;
        p.d = (int32_t)d;
        p.F = (int32_t)F;
        p.G = (int32_t)E;
        p.n_tiles_n = (int32_t)(F / 64);
        p.max_m_tiles = (int32_t)L.max_tiles;
      }
      SL.n = np;
      const SwigluBwdProblem& p0 = SL.p[0];
      SL.tiles0 = p0.plan ? 2 * p0.max_m_tiles * p0.n_tiles_n
                          : p0.G * (int32_t)ceil_div(p0.M, kSwigluBwdBM) * p0.n_tiles_n;
      Rn.run("swiglu_bwd", [&] { return launch_swiglu_bwd(SL, Rn.stream); });
    }

    // input gradient products: shared experts, router, routed experts
    {
      BwdLaunch BL{};
      int np = 0;
      const int32_t ntn = (int32_t)ceil_div(d, 128), ntm = (int32_t)ceil_div(T, kGemmBigBM);
      if (S > 0) {
        BwdGemm& p = BL.p[np++] = bwd_problem();
        p.A = dabsh;
        p.lda = S * 2 * F;
        p.B0 = w->sh_gate;
        p.B1 = w->sh_up;
        p.ldb = F;
        p.k_seg = (int32_t)F;
        p.b_seg = d * F;
        p.C0 = dxsh;
        p.ldc = d;
        p.M = (int32_t)T;
        p.N = (int32_t)d;
        p.K = (int32_t)(S * 2 * F);
        p.k_chunk = p.K;
        p.n_tiles_m = ntm;
        p.n_tiles_n = ntn;
      }
      {
        BwdGemm& p = BL.p[np++] = bwd_problem();
        p.A = dl;
        p.lda = E;
        p.B0 = w->w_router;
        p.ldb = E;
        p.C0 = g->dx;
        p.ldc = d;
        p.M = (int32_t)T;
        p.N = (int32_t)d;
        p.K = (int32_t)E;
        p.k_chunk = p.K;
        p.n_tiles_m = ntm;
        p.n_tiles_n = ntn;
      }
      {
        BwdGemm& p = BL.p[np++] = bwd_problem();
        p.A = dab;
        p.lda = 2 * F;
        p.B0 = w->w_gate;
        p.B1 = w->w_up;
        p.ldb = F;
        p.b_group = d * F;
        p.k_seg = (int32_t)F;
        p.C0 = dxp;
        p.ldc = d;
        p.m_off = o->offsets;
        p.plan = plan256;
        p.N = (int32_t)d;
        p.K = (int32_t)(2 * F);
        p.G = (int32_t)E;
        p.n_tiles_n = ntn;
        p.max_m_tiles = (int32_t)L.max_tiles;
      }
      BL.n = np;
      Rn.run("dgrad_gemm", [&] { return gemm(BL, true, true, kBwdStoreF32); });
    }
    DxGatherArgs dx{};
    dx.dx_rows = dxp;
    dx.dx_shared = dxsh;
    dx.row_of_slot = o->row_of_slot;
    dx.dx = g->dx;
    dx.T = T;
    dx.d = (int32_t)d;
    dx.k = (int32_t)k;
    Rn.run("dx_gather", [&] { return launch_dx_gather(dx, Rn.stream); });
  }

  // weight gradient products: shared experts (split over tokens), routed
  // experts (their own rows), router (split over tokens)
  {
    BwdLaunch BL{};
    int np = 0;
    const bool split_s = S > 0 && B.nch_s > 1;
    const int32_t kch_s = (int32_t)(split_s ? kSharedKChunk : std::max<int64_t>(T, 1));
    if (S > 0) {
      BwdGemm& p = BL.p[np++] = bwd_problem();
      p.A = h_sh;
      p.lda = S * F;
      p.a_group = F;
      p.B0 = dysh;
      p.ldb = d;
      p.C0 = split_s ? at<float>(bws, B.part_d) : g->dsh_down;
      p.ldc = d;
      p.c_group = (int64_t)B.nch_s * F * d;
      p.c_chunk = F * d;
      p.M = (int32_t)F;
      p.N = (int32_t)d;
      p.K = (int32_t)T;
      p.G = (int32_t)S;
      p.k_chunk = kch_s;
      p.n_chunks = (int32_t)B.nch_s;
      p.n_tiles_m = (int32_t)ceil_div(F, kGemmBigBM);
      p.n_tiles_n = (int32_t)ceil_div(d, 128);
    }
    if (S > 0) {
      BwdGemm& p = BL.p[np++] = bwd_problem();
      p.A = x;
      p.lda = d;
      p.B0 = dabsh;
      p.ldb = S * 2 * F;
      p.b_group = 2 * F;
      p.C0 = split_s ? at<float>(bws, B.part_g) : g->dsh_gate;
      p.C1 = split_s ? at<float>(bws, B.part_u) : g->dsh_up;
      p.c_split = (int32_t)F;
      p.ldc = F;
      p.c_group = (int64_t)B.nch_s * d * F;
      p.c_chunk = d * F;
      p.M = (int32_t)d;
      p.N = (int32_t)(2 * F);
      p.K = (int32_t)T;
      p.G = (int32_t)S;
      p.k_chunk = kch_s;
      p.n_chunks = (int32_t)B.nch_s;
      p.n_tiles_m = (int32_t)ceil_div(d, kGemmBigBM);
      p.n_tiles_n = (int32_t)ceil_div(2 * F, 128);
    }
    {
      BwdGemm& p = BL.p[np++] = bwd_problem();
      p.A = h;
      p.lda = F;
      p.B0 = dyr;
      p.ldb = d;
      p.C0 = g->dw_down;
      p.ldc = d;
      p.c_group = F * d;
      p.k_off = o->offsets;
      p.M = (int32_t)F;
      p.N = (int32_t)d;
      p.K = (int32_t)R;
      p.G = (int32_t)E;
      p.n_tiles_m = (int32_t)ceil_div(F, kGemmBigBM);
      p.n_tiles_n = (int32_t)ceil_div(d, 128);
    }
    {
      BwdGemm& p = BL.p[np++] = bwd_problem();
      p.A = xperm;
      p.lda = d;
      p.B0 = dab;
      p.ldb = 2 * F;
      p.C0 = g->dw_gate;
      p.C1 = g->dw_up;
      p.c_split = (int32_t)F;
      p.ldc = F;
      p.c_group = d * F;
      p.k_off = o->offsets;
      p.M = (int32_t)d;
      p.N = (int32_t)(2 * F);
      p.K = (int32_t)R;
      p.G = (int32_t)E;
      p.n_tiles_m = (int32_t)ceil_div(d, kGemmBigBM);
      p.n_tiles_n = (int32_t)ceil_div(2 * F, 128);
    }
    {
      BwdGemm& p = BL.p[np++] = bwd_problem();
      p.A = x;
      p.lda = d;
      p.B0 = dl;
      p.ldb = E;
      p.C0 = B.nch_r > 1 ? at<float>(bws, B.part_r) : g->dw_router;
      p.ldc = E;
      p.c_chunk = d * E;
      p.M = (int32_t)d;
      p.N = (int32_t)E;
      p.K = (int32_t)T;
      p.k_chunk = B.nch_r > 1 ? B.kch_r : (int32_t)std::max<int64_t>(T, 1);
      p.n_chunks = (int32_t)B.nch_r;
      p.n_tiles_m = (int32_t)ceil_div(d, kGemmBigBM);
      p.n_tiles_n = (int32_t)ceil_div(E, 128);
    }
    BL.n = np;
    Rn.run("wgrad_gemm", [&] { return gemm(BL, false, false, kBwdStoreF32); });
    if (B.nch_r > 1) {
      Rn.run("reduce_router", [&] {
        return launch_reduce_chunks(at<float>(bws, B.part_r), g->dw_router, 1, B.nch_r, d * E,
                                    Rn.stream);
      });
    }
    if (split_s) {
      Rn.run("reduce_shared", [&] {
        hipError_t e = launch_reduce_chunks(at<float>(bws, B.part_g), g->dsh_gate, S, B.nch_s,
                                            d * F, Rn.stream);
        if (e == hipSuccess)
          e = launch_reduce_chunks(at<float>(bws, B.part_u), g->dsh_up, S, B.nch_s, d * F,
                                   Rn.stream);
        if (e == hipSuccess)
          e = launch_reduce_chunks(at<float>(bws, B.part_d), g->dsh_down, S, B.nch_s, F * d,
                                   Rn.stream);
        return e;
      });
    }
  }
  st = finish(tl);
  return st ? st : tl.n;
}
}  // namespace

int report_hip_error(hipError_t e) { return hip_fail(e); }

// The layer forward for callers that bring their own workspace pointer from
// elsewhere (the allocation-free entry point's device scratch array).
int layer_forward_on(const moe_config* c, int64_t T, const void* x, const moe_weights* w,
                     moe_outputs* o, void* ws, size_t ws_bytes, void* stream) {
  const int r = layer_forward(c, T, x, w, o, ws, ws_bytes, stream, nullptr, 0);
  return r < 0 ? r : MOE_OK;
}

// Validation of a forward call that does not touch the device: MOE_OK, or the
// status the call would return before launching anything. ws_bytes_out gets
// the workspace the call needs.
int layer_forward_check(const moe_config* c, int64_t T, const void* x, const moe_weights* w,
                        const moe_outputs* o, size_t* ws_bytes_out) {
  int st = check_common(c, T);
  if (st) return st;
  if (!x && T > 0) return MOE_EINVAL;
  if (!w || !w->w_router || !expert_weights_ok(c, w, true, true)) return MOE_EINVAL;
  if (c->score == MOE_SOFTMAX && w->select_bias) return MOE_EINVAL;
  if (!route_outputs_ok(o, T) || !permute_outputs_ok(o, T) || (T > 0 && !o->y))
    return MOE_EINVAL;
  *ws_bytes_out = make_layout(c, T).total;
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" {

int32_t moe_capacity(int64_t num, int64_t den, int64_t T, int32_t k, int32_t E) {
  if (num <= 0 || den <= 0 || T < 0 || k <= 0 || E <= 0) return -1;
  const __int128 n = (__int128)num * T * k;
  const __int128 q = (__int128)den * E;
  const __int128 c = (n + q - 1) / q;
  if (c > INT32_MAX) return -1;
  return (int32_t)c;
}

int64_t moe_max_rows(const moe_config* cfg, int64_t T) {
  if (!valid_config(cfg) || T < 0) return -1;
  return max_rows(cfg, T);
}

size_t moe_workspace_bytes(const moe_config* cfg, int64_t T) {
  if (!valid_config(cfg) || T < 0) return 0;
  return make_layout(cfg, T).total;
}

int moe_route(const moe_config* c, int64_t T, const void* x, const moe_weights* w,
              moe_outputs* o, void* ws, size_t ws_bytes, void* stream) {
  int st = check_common(c, T);
  if (st) return st;
  if ((!x && T > 0) || !w || !w->w_router || !route_outputs_ok(o, T)) return MOE_EINVAL;
  if (c->score == MOE_SOFTMAX && w->select_bias) return MOE_EINVAL;
  Layout L;
  if ((st = check_ws(c, T, ws, ws_bytes, L))) return st;
  Timeline tl;
  Runner R{static_cast<hipStream_t>(stream), &tl};
  run_route(R, c, L, x, w, o, ws, false);
  return finish(tl);
}

int moe_permute(const moe_config* c, int64_t T, const void* x, moe_outputs* o, void* x_perm,
                void* ws, size_t ws_bytes, void* stream) {
  int st = check_common(c, T);
  if (st) return st;
  if (!o || !o->offsets || !permute_outputs_ok(o, T) || (T > 0 && !o->topk_idx))
    return MOE_EINVAL;
  if (x_perm && !x && T > 0) return MOE_EINVAL;
  Layout L;
  if ((st = check_ws(c, T, ws, ws_bytes, L))) return st;
  Timeline tl;
  Runner R{static_cast<hipStream_t>(stream), &tl};
  run_rank(R, c, L, o, ws);
  if (x_perm && L.R > 0) {
    R.run("gather", [&] {
      return launch_gather(x, o->sorted_token, o->offsets, c->n_routed, L.R,
                           (int64_t)c->hidden * elem_size(c), x_perm, R.stream);
    });
  }
  return finish(tl);
}

int moe_grouped_ffn(const moe_config* c, int64_t T, int32_t groups, const void* x_perm,
                    const int32_t* offsets, const void* x_shared, const moe_weights* w,
                    float* y_routed, float* y_shared, void* ws, size_t ws_bytes, void* stream) {
  int st = check_common(c, T);
  if (st) return st;
  if (groups & ~(MOE_GROUPS_ROUTED | MOE_GROUPS_SHARED)) return MOE_EINVAL;
  const bool routed = groups & MOE_GROUPS_ROUTED;
  const bool shared = (groups & MOE_GROUPS_SHARED) && c->n_shared > 0;
  if (!expert_weights_ok(c, w, routed, shared)) return MOE_EINVAL;
  if (routed && (!x_perm || !offsets || !y_routed)) return MOE_EINVAL;
  if (shared && T > 0 && (!x_shared || !y_shared)) return MOE_EINVAL;
  Layout L;
  if ((st = check_ws(c, T, ws, ws_bytes, L))) return st;
  Timeline tl;
  Runner R{static_cast<hipStream_t>(stream), &tl};
  if (routed && L.R > 0) {
    R.run("plan", [&] {
      return launch_plan(offsets, c->n_routed, plan_bm(c), at<int32_t>(ws, L.plan), R.stream);
    });
  }
  run_ffn(R, c, L, routed, shared, x_perm, nullptr, offsets, x_shared, w, y_routed, y_shared,
          ws);
  return finish(tl);
}

int moe_combine(const moe_config* c, int64_t T, const float* y_routed, const float* y_shared,
                moe_outputs* o, void* stream) {
  int st = check_common(c, T);
  if (st) return st;
  if (!o || (T > 0 && (!o->row_of_slot || !o->topk_gate || !o->y))) return MOE_EINVAL;
  if (T > 0 && !y_routed) return MOE_EINVAL;
  if (c->n_shared > 0 && T > 0 && !y_shared) return MOE_EINVAL;
  Timeline tl;
  Runner R{static_cast<hipStream_t>(stream), &tl};
  run_combine(R, c, T, y_routed, c->n_shared > 0 ? y_shared : nullptr, o);
  return finish(tl);
}

int moe_quantize_fp8(const moe_config* c, const moe_weights* src, moe_weights* dst,
                     void* stream) {
  if (!valid_config(c) || c->dtype != MOE_FP8) return MOE_EINVAL;
  if (!supported_config(c)) return MOE_EUNSUPPORTED;
  if (!src || !dst) return MOE_EINVAL;
  moe_config bc = *c;
  bc.dtype = MOE_BF16;
  if (!expert_weights_ok(&bc, src, true, true) || !expert_weights_ok(c, dst, true, true))
    return MOE_EINVAL;
  const int64_t d = c->hidden, F = c->ffn, S = c->n_shared, E = c->n_routed;
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto q = [&](const void* w, int64_t G, int64_t K, int64_t N, const void* out,
               const float* scale) {
    return launch_quant_cols(static_cast<const uint16_t*>(w), G, (int32_t)K, (int32_t)N,
                             static_cast<uint8_t*>(const_cast<void*>(out)),
                             const_cast<float*>(scale), s);
  };
  hipError_t e = hipSuccess;
  if (c->rank == 0) {
    e = q(src->w_gate, E, d, F, dst->w_gate, dst->w_gate_scale);
    if (e == hipSuccess) e = q(src->w_up, E, d, F, dst->w_up, dst->w_up_scale);
    if (e == hipSuccess) e = q(src->w_down, E, F, d, dst->w_down, dst->w_down_scale);
  } else {
    const int64_t r = c->rank;
    // U [in, r] per column r, written transposed [r, in]
    e = q(src->u_gate, E, d, r, dst->u_gate, dst->u_gate_scale);
    if (e == hipSuccess) e = q(src->u_up, E, d, r, dst->u_up, dst->u_up_scale);
    if (e == hipSuccess) e = q(src->u_down, E, F, r, dst->u_down, dst->u_down_scale);
    // V [out, r] per row: rows of r values
    auto qr = [&](const void* v, int64_t rows, const void* out, const float* scale) {
      return launch_quant_rows(static_cast<const uint16_t*>(v), r, rows, (int32_t)r, nullptr,
                               static_cast<uint8_t*>(const_cast<void*>(out)),
                               const_cast<float*>(scale), s);
    };
    if (e == hipSuccess) e = qr(src->v_gate, E * F, dst->v_gate, dst->v_gate_scale);
    if (e == hipSuccess) e = qr(src->v_up, E * F, dst->v_up, dst->v_up_scale);
    if (e == hipSuccess) e = qr(src->v_down, E * d, dst->v_down, dst->v_down_scale);
  }
  if (S > 0) {
    if (e == hipSuccess) e = q(src->sh_gate, S, d, F, dst->sh_gate, dst->sh_gate_scale);
    if (e == hipSuccess) e = q(src->sh_up, S, d, F, dst->sh_up, dst->sh_up_scale);
    // the S down projections as one [S F, d] matrix
    if (e == hipSuccess) e = q(src->sh_down, 1, S * F, d, dst->sh_down, dst->sh_down_scale);
  }
  return e == hipSuccess ? MOE_OK : hip_fail(e);
}

int moe_workspace_region(const moe_config* c, int64_t T, int32_t which, size_t* offset,
                         size_t* bytes) {
  if (!valid_config(c) || T < 0 || !offset || !bytes) return MOE_EINVAL;
  const Layout L = make_layout(c, T);
  const int64_t d = c->hidden, F = c->ffn, S = c->n_shared;
  const size_t es = elem_size(c);
  const bool q = fp8(c) && c->rank == 0;
  size_t at = 0, n = 0;
  switch (which) {
    case MOE_WS_H: at = L.h; n = c->rank > 0 ? 0 : (size_t)L.R * F * es; break;
    case MOE_WS_H_SHARED: at = L.h_sh; n = (size_t)T * S * F * es; break;
    case MOE_WS_Y_ROUTED: at = L.y_perm; n = (size_t)L.R * d * 4; break;
    case MOE_WS_Y_SHARED: at = L.y_sh; n = S > 0 ? (size_t)T * d * 4 : 0; break;
    case MOE_WS_HQ: at = L.hq; n = q ? (size_t)L.R * F : 0; break;
    case MOE_WS_HQ_SCALE: at = L.hs; n = q ? (size_t)L.R * 4 : 0; break;
    case MOE_WS_HQ_SHARED: at = L.hq_sh; n = fp8(c) ? (size_t)T * S * F : 0; break;
    case MOE_WS_HQ_SHARED_SCALE: at = L.hs_sh; n = fp8(c) && S > 0 ? (size_t)T * 4 : 0; break;
    default: return MOE_EINVAL;
  }
  *offset = n ? at : 0;
  *bytes = n;
  return MOE_OK;
}

int moe_backward_workspace_region(const moe_config* c, int64_t T, int32_t which, size_t* offset,
                                  size_t* bytes) {
  if (!valid_config(c) || T < 0 || !offset || !bytes) return MOE_EINVAL;
  const BwdLayout B = make_bwd_layout(c, T);
  const int64_t d = c->hidden, F = c->ffn, E = c->n_routed, R = B.R;
  const int64_t r = c->rank;
  const bool lr = r > 0;
  const size_t es = c->dtype == MOE_F32 ? 4 : 2;
  size_t at = 0, n = 0;
  switch (which) {
    case MOE_BWS_DY_ROUTED: at = B.dyr; n = (size_t)R * d * es; break;
    case MOE_BWS_X_PERM: at = B.xperm; n = (size_t)R * d * es; break;
    case MOE_BWS_DAB: at = B.dab; n = (size_t)R * 2 * F * es; break;
    case MOE_BWS_DL: at = B.dl; n = (size_t)T * E * es; break;
    case MOE_BWS_DAB_SHARED: at = B.dabsh; n = (size_t)T * c->n_shared * 2 * F * es; break;
    case MOE_BWS_LR_UG: at = B.ug; n = lr ? (size_t)R * r * 4 : 0; break;
    case MOE_BWS_LR_UU: at = B.uu; n = lr ? (size_t)R * r * 4 : 0; break;
    case MOE_BWS_LR_Z_GU: at = B.zgu; n = lr ? (size_t)R * 2 * r * 2 : 0; break;
    case MOE_BWS_LR_AB: at = B.ab; n = lr ? (size_t)R * 2 * F * 4 : 0; break;
    case MOE_BWS_LR_H: at = B.hh; n = lr ? (size_t)R * F * 2 : 0; break;
    case MOE_BWS_LR_UD: at = B.ud; n = lr ? (size_t)R * r * 4 : 0; break;
    case MOE_BWS_LR_ZD: at = B.zd; n = lr ? (size_t)R * r * 2 : 0; break;
    case MOE_BWS_LR_DZD: at = B.dzd; n = lr ? (size_t)R * r * 4 : 0; break;
    case MOE_BWS_LR_DUD: at = B.dud; n = lr ? (size_t)R * r * 2 : 0; break;
    case MOE_BWS_LR_DZG: at = B.dzg; n = lr ? (size_t)R * r * 4 : 0; break;
    case MOE_BWS_LR_DZU: at = B.dzu; n = lr ? (size_t)R * r * 4 : 0; break;
    case MOE_BWS_LR_DU_GU: at = B.dugu; n = lr ? (size_t)R * 2 * r * 2 : 0; break;
    default: return MOE_EINVAL;
  }
  *offset = n ? at : 0;
  *bytes = n;
  return MOE_OK;
}

int moe_bias_update(const moe_config* c, int64_t T, const int32_t* counts, float* select_bias,
                    float gamma, void* stream) {
  if (!valid_config(c) || T < 0 || !isfinite(gamma)) return MOE_EINVAL;
  if (!counts || !select_bias) return MOE_EINVAL;
  const hipError_t e = launch_bias_update(counts, select_bias, c->n_routed, T * c->top_k, gamma,
                                          static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e);
}

int moe_layer_forward(const moe_config* c, int64_t T, const void* x, const moe_weights* w,
                      moe_outputs* o, void* ws, size_t ws_bytes, void* stream) {
  const int r = layer_forward(c, T, x, w, o, ws, ws_bytes, stream, nullptr, 0);
  return r < 0 ? r : MOE_OK;
}

int moe_layer_forward_timed(const moe_config* c, int64_t T, const void* x, const moe_weights* w,
                            moe_outputs* o, void* ws, size_t ws_bytes, void* stream,
                            void** events, int n_events) {
  if (n_events < 0 || (n_events > 0 && !events)) return MOE_EINVAL;
  return layer_forward(c, T, x, w, o, ws, ws_bytes, stream, events, n_events);
}

size_t moe_backward_workspace_bytes(const moe_config* cfg, int64_t T) {
  if (!valid_config(cfg) || T < 0) return 0;
  return make_bwd_layout(cfg, T).total;
}

int moe_layer_backward(const moe_config* c, int64_t T, const void* x, const moe_weights* w,
                       const moe_outputs* o, const float* dy, float aux_grad, moe_grads* g,
                       const void* ws, size_t ws_bytes, void* bwd_ws, size_t bwd_ws_bytes,
                       void* stream) {
  const int r = layer_backward(c, T, x, w, o, dy, aux_grad, g, ws, ws_bytes, bwd_ws,
                               bwd_ws_bytes, stream, nullptr, 0);
  return r < 0 ? r : MOE_OK;
}

int moe_layer_backward_timed(const moe_config* c, int64_t T, const void* x, const moe_weights* w,
                             const moe_outputs* o, const float* dy, float aux_grad, moe_grads* g,
                             const void* ws, size_t ws_bytes, void* bwd_ws, size_t bwd_ws_bytes,
                             void* stream, void** events, int n_events) {
  if (n_events < 0 || (n_events > 0 && !events)) return MOE_EINVAL;
  return layer_backward(c, T, x, w, o, dy, aux_grad, g, ws, ws_bytes, bwd_ws, bwd_ws_bytes,
                        stream, events, n_events);
}

const char* moe_stage_name(int i) {
  if (i < 0 || i >= g_n_stages || i >= 64) return nullptr;
  return g_stage_names[i];
}

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "configuration not supported by this library";
    case MOE_EWORKSPACE: return "workspace missing, misaligned or too small";
    case MOE_EHIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
