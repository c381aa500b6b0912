/*
 * moe.h -- C ABI of the fine-grained mixture-of-experts feed-forward layer,
 * built from hand-written HIP kernels for MI355X (gfx950, CDNA4).
 *
 * The layer (DeepSeek-style fine-grained MoE, as on the Vertex AGI research
 * page "Architecture" section, the Quartz Micro Preview Base model card
 * "Architecture" table, the Moonfrost site MoE and stacking cards, the
 * Sutra-1.3B "48 + 1 experts" card and the dormouse "dropless MoE" and
 * "TSCT low-rank experts" cards), for T tokens x[T,d]:
 *
 *   l    = x W_r + logit_bias                       router projection
 *   key  = l (softmax rule)  |  sigmoid(l) + select_bias (sigmoid rule)
 *   idx  = the k experts of largest key, equal keys -> lower id first
 *   gate = softmax(l)[idx] (optionally / their sum)  |  sigmoid(l)[idx] / their sum
 *   dispatch: each expert's slots in token order; with capacity C > 0 only the
 *             first C slots of an expert are kept (the rest are dropped)
 *   y[t] = sum_{s<S} SwiGLU_s(x[t]) + sum_{kept j} gate[t,j] SwiGLU_{idx[t,j]}(x[t])
 *   SwiGLU(v) = (SiLU(v W_gate) * (v W_up)) W_down,  h = SiLU(.)*(.) rounded to
 *             the storage type before W_down; low-rank experts use
 *             W = U diag(s) V^T for each of the three matrices
 *   aux_raw = E * sum_i f_i P_i,  f_i = counts_i/(T k),  P_i = mean_t prob[t,i]
 *             (prob = full softmax, or sigmoid / row sum); aux = aux_coef * aux_raw
 *
 * Conventions for every entry point
 *   - Pointers named "device" are HIP device pointers; every array is dense
 *     row-major with the shape given. The caller owns and allocates all of them
 *     and the workspace; the library never allocates or frees device memory and
 *     keeps nothing between calls.
 *   - `stream` is a hipStream_t (NULL = the default stream). Every call only
 *     enqueues work on it and returns; results are valid after the stream
 *     synchronises. No call reads device memory from the host.
 *   - Errors are returned as moe_status codes; arguments are validated before
 *     anything is enqueued, so an error return means nothing was launched
 *     (except MOE_EHIP, reported when a launch itself fails).
 *   - Calls that share a workspace on different streams race; calls on one
 *     stream are ordered.
 *   - A legal layer (else MOE_EINVAL): 1 <= k <= E <= 4096; d and F positive
 *     multiples of 8; 0 <= S <= 64; T*k < 2^31; sigmoid scoring requires
 *     renorm_topk == 1.
 *   - Legal layers outside this library's kernels return MOE_EUNSUPPORTED:
 *     k > 15; d or F not a multiple of 64; d >= 2^21 with bf16 or fp8
 *     activations; rank other than 0, 16, 32, 48 or 64
 *     with bf16, or 64 with fp8 (low-rank float32 experts are unsupported);
 *     MOE_FP8 with d, F or S*F above 4096. MOE_FP8 runs in moe_layer_forward
 *     and moe_grouped_ffn.
 */
#ifndef FGM_MOE_H
#define FGM_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,        /* NULL required pointer or a size/setting out of range   */
  MOE_EUNSUPPORTED = -2,  /* legal layer this library does not implement (see limits) */
  MOE_EWORKSPACE = -3,    /* ws is NULL/misaligned or ws_bytes < moe_workspace_bytes */
  MOE_EHIP = -4           /* a HIP call failed; moe_last_error() holds its text      */
} moe_status;

/* type of x and weights. MOE_FP8: x, W_r, biases and the layer's activations as
   for MOE_BF16; the dense expert weights are fp8 codes (see moe_weights). */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8 = 2 } moe_dtype;
typedef enum { MOE_SOFTMAX = 0, MOE_SIGMOID = 1 } moe_score;  /* router scoring rule   */

/* moe_grouped_ffn `groups` bits */
enum { MOE_GROUPS_ROUTED = 1, MOE_GROUPS_SHARED = 2 };

typedef struct {
  int32_t hidden;       /* d, multiple of 8 (this library: of 64)                  */
  int32_t n_routed;     /* E, routed experts                                       */
  int32_t top_k;        /* k, active routed experts per token                      */
  int32_t n_shared;     /* S, always-on ungated shared experts (0 allowed)         */
  int32_t ffn;          /* F, width of every expert, multiple of 8 (library: 64)   */
  int32_t rank;         /* 0: dense experts; r > 0: U diag(s) V^T factors of rank r */
  int32_t score;        /* moe_score                                               */
  int32_t renorm_topk;  /* softmax: 1 = gates divided by their top-k sum, 0 = raw
                           probabilities; sigmoid: must be 1                       */
  int32_t capacity;     /* 0: dropless; C > 0: at most C slots per expert, later
                           tokens' slots dropped (see moe_capacity)               */
  float   aux_coef;     /* alpha of the aux statistic (0.01 for Quartz)            */
  int32_t dtype;        /* moe_dtype of x, every weight and the x_perm/h buffers   */
} moe_config;

/* Device pointers to one layer's weights, element type = cfg.dtype unless noted.
   All read-only. */
typedef struct {
  const void  *w_router;     /* [d, E]                                              */
  const float *logit_bias;   /* [E] float32 or NULL; added to the logits (moves gates) */
  const float *select_bias;  /* [E] float32 or NULL; sigmoid rule only: added to the
                                selection key, never to the gates                   */
  /* dense experts (rank == 0): stacked expert tensors                              */
  const void *w_gate;        /* [E, d, F] */
  const void *w_up;          /* [E, d, F] */
  const void *w_down;        /* [E, F, d] */
  /* low-rank experts (rank == r > 0): W[in,out] = U[in,r] diag(s[r]) V[out,r]^T    */
  const void *u_gate, *s_gate, *v_gate;   /* [E,d,r], [E,r], [E,F,r] */
  const void *u_up,   *s_up,   *v_up;     /* [E,d,r], [E,r], [E,F,r] */
  const void *u_down, *s_down, *v_down;   /* [E,F,r], [E,r], [E,d,r] */
  /* shared experts (S > 0), NULL when S == 0                                      */
  const void *sh_gate;       /* [S, d, F] */
  const void *sh_up;         /* [S, d, F] */
  const void *sh_down;       /* [S, F, d] */
  /* MOE_FP8 (the storage ladder's fp8 rung, dormouse "TSCT low-rank experts"
     card): every expert matrix W[in, out] is stored as OCP E4M3 codes (one byte)
     in the transposed order q[out, in], with one float32 power-of-two scale per
     output column, W[i, o] ~= code(q[o, i]) * scale[o] (moe_quantize_fp8). The
     pointers above then hold the codes:
       w_gate, w_up [E, F, d]; w_down [E, d, F]; sh_gate, sh_up [S, F, d];
       sh_down [d, S*F]: the S shared down projections as one [S*F, d] matrix
       (they are summed), so one scale per output column over all S*F rows. */
  const float *w_gate_scale;   /* [E, F] */
  const float *w_up_scale;     /* [E, F] */
  const float *w_down_scale;   /* [E, d] */
  const float *sh_gate_scale;  /* [S, F] */
  const float *sh_up_scale;    /* [S, F] */
  const float *sh_down_scale;  /* [d]    */
  /* MOE_FP8 with rank r: the factor pointers above hold E4M3 codes, U stored
     transposed (u_gate, u_up [E, r, d]; u_down [E, r, F]) and V as in bf16
     (v_gate, v_up [E, F, r]; v_down [E, d, r]), with power-of-two scales per
     column of U and per row of V; s_gate, s_up, s_down stay bf16. */
  const float *u_gate_scale;   /* [E, r] */
  const float *u_up_scale;     /* [E, r] */
  const float *u_down_scale;   /* [E, r] */
  const float *v_gate_scale;   /* [E, F] */
  const float *v_up_scale;     /* [E, F] */
  const float *v_down_scale;   /* [E, d] */
} moe_weights;

/* Device output buffers, caller-allocated. R_max = T*k (dropless) or
   min(T*k, E*C). "optional" pointers may be NULL. */
typedef struct {
  int32_t *topk_idx;      /* [T, k] selected expert ids, descending key          */
  float   *topk_gate;     /* [T, k] gate weights                                  */
  float   *topk_margin;   /* [T] optional: key of k-th minus key of (k+1)-th
                             expert (+inf when k == E)                            */
  int32_t *counts;        /* [E] slots per expert before capacity                 */
  int32_t *kept;          /* [E] min(counts, C) (counts when dropless)             */
  int32_t *offsets;       /* [E+1] exclusive prefix sum of kept; offsets[E] = rows  */
  int32_t *sorted_token;  /* [R_max] token of each dispatched row, rows grouped by
                             expert, ascending token within an expert; entries at
                             and beyond offsets[E] are left untouched              */
  int32_t *row_of_slot;   /* [T, k] dispatched row of slot (t, j), -1 if dropped  */
  uint8_t *dropped;       /* [T, k] optional: 1 if slot dropped by capacity       */
  int32_t *n_dropped;     /* [1] number of dropped slots                          */
  float   *aux;           /* [2] {aux_raw, aux_coef * aux_raw}                    */
  float   *f;             /* [E] optional: counts / (T k)                          */
  float   *P;             /* [E] optional: mean routing probability per expert    */
  float   *y;             /* [T, d] float32 layer output                          */
  void    *y_lowp;        /* [T, d] optional copy of y in cfg.dtype               */
  float   *saved_ab;      /* optional, bf16 dense layers (ignored otherwise): the
                             gate and up products a = x W_gate, b = x W_up that
                             moe_layer_forward computes, float32, for
                             moe_layer_backward to read instead of recomputing:
                             [R_max, 2F] (dispatched row r: a at columns [0, F),
                             b at [F, 2F)), then [T, S, 2F] (token t, shared
                             expert s). Rows at and beyond offsets[E] of the
                             first block are left untouched.                  */
} moe_outputs;

/* Capacity C = ceil(num * T * k / (den * E)) in exact integer arithmetic, as for
   a capacity factor num/den (Moonfrost stacking card: capacity-based routing;
   factor 5/4 gives C = 1920 at T = 16384, k = 3, E = 32). Returns -1 on bad input. */
int32_t moe_capacity(int64_t num, int64_t den, int64_t T, int32_t k, int32_t E);

/* Largest number of dispatched rows: T*k dropless, else min(T*k, E*C). */
int64_t moe_max_rows(const moe_config *cfg, int64_t T);

/* Workspace bytes every entry point below needs for this config and T (the same
   workspace serves all of them). 0 if cfg is invalid. */
size_t moe_workspace_bytes(const moe_config *cfg, int64_t T);

/* Intermediates of the expert FFN that moe_layer_forward and moe_grouped_ffn
   leave in ws, for inspection after the call (parity checks, debugging); valid
   until the next call on the same ws. moe_workspace_region gives the byte
   offset into ws and the size of region `which` for this config and T; a size
   of 0 means the config has no such region. Returns MOE_EINVAL for an invalid
   config, T < 0, NULL outputs or an unknown region.
     MOE_WS_H                h [R_max, F] in cfg.dtype's activation type
                             (bf16 for MOE_FP8): SiLU(a) * b of each dispatched
                             row, rounded, before the down projection (dense
                             experts; low-rank experts keep h on chip)
     MOE_WS_H_SHARED         [T, S*F]: the same for the shared experts
     MOE_WS_Y_ROUTED         [R_max, d] float32: each dispatched row's expert output
     MOE_WS_Y_SHARED         [T, d] float32: the shared experts' summed output
     MOE_WS_HQ, _HQ_SCALE    MOE_FP8 dense experts: E4M3 codes of h [R_max, F] and
                             each row's float32 power-of-two scale [R_max]
     MOE_WS_HQ_SHARED, _HQ_SHARED_SCALE   MOE_FP8: codes [T, S*F], scales [T]
   Rows at and beyond offsets[E] of the routed regions hold no data.          */
enum {
  MOE_WS_H = 0, MOE_WS_H_SHARED = 1, MOE_WS_Y_ROUTED = 2, MOE_WS_Y_SHARED = 3,
  MOE_WS_HQ = 4, MOE_WS_HQ_SCALE = 5, MOE_WS_HQ_SHARED = 6, MOE_WS_HQ_SHARED_SCALE = 7
};
int moe_workspace_region(const moe_config *cfg, int64_t T, int32_t which, size_t *offset,
                         size_t *bytes);

/* Router projection, scores, top-k, gates, per-expert histogram, capacity,
   prefix sum and aux statistic (steps: a learned router picks the top k of E
   routed experts per token -- Vertex AGI research page "Architecture", Quartz
   model card "Architecture" table, Moonfrost MoE card; sigmoid scores with a
   selection-only balancing bias -- Sutra-1.3B "48 + 1 experts" card; the
   0.01-weighted load-balancing statistic -- research page "Architecture";
   capacity, 0 = dropless -- Moonfrost stacking card, dormouse terminal block).
   In:  x [T,d] device; w->w_router, w->logit_bias, w->select_bias.
   Out: o->topk_idx, topk_gate, (topk_margin), counts, kept, offsets, n_dropped,
        aux, (f), (P); per-block tables kept in ws for moe_permute.           */
int moe_route(const moe_config *cfg, int64_t T, const void *x, const moe_weights *w,
              moe_outputs *o, void *ws, size_t ws_bytes, void *stream);

/* Token permutation: each kept slot's row in token order per expert, drops,
   and optionally the gathered rows x_perm[row] = x[sorted_token[row]]
   (grouping the tokens by expert so that each expert runs once over its rows:
   Moonfrost stacking card, stacked (E, hidden, ffn) expert tensors with
   capacity-based routing; capacity queues in token order).
   Must follow moe_route with the same cfg, T, outputs and ws on the same stream.
   In:  x [T,d] device (read only if x_perm != NULL).
   Out: o->row_of_slot, sorted_token, (dropped); x_perm [R_max, d] cfg.dtype or NULL. */
int moe_permute(const moe_config *cfg, int64_t T, const void *x, moe_outputs *o,
                void *x_perm, void *ws, size_t ws_bytes, void *stream);

/* Grouped SwiGLU expert FFN (the experts' gated feed-forward blocks over the
   stacked expert tensors -- Moonfrost stacking card; two always-on shared
   experts -- research page "Architecture"; rank-64 U diag(s) V^T experts --
   dormouse "TSCT low-rank experts" card).
   groups & MOE_GROUPS_ROUTED: for every routed expert e, the rows
     x_perm[offsets[e] : offsets[e+1]] of x_or_xperm ([R_max, d]) go through
     expert e; result rows written to y_routed [R_max, d] float32 (rows at and
     beyond offsets[E] untouched). offsets [E+1] device, as from moe_route.
   groups & MOE_GROUPS_SHARED: every row of x_shared [T, d] goes through all S
     shared experts, summed, into y_shared [T, d] float32.
   Unused inputs/outputs may be NULL.                                         */
int moe_grouped_ffn(const moe_config *cfg, int64_t T, int32_t groups,
                    const void *x_perm, const int32_t *offsets, const void *x_shared,
                    const moe_weights *w, float *y_routed, float *y_shared,
                    void *ws, size_t ws_bytes, void *stream);

/* Gate-weighted combine (each token's output is its shared experts' sum plus
   its routed experts' outputs weighted by their gates -- research page
   "Architecture", Moonfrost MoE card; dropped slots add nothing -- Moonfrost
   stacking card): y[t] = y_shared[t] + sum_{j kept, ascending j}
   topk_gate[t,j] * y_routed[row_of_slot[t,j]], in float32 in that order.
   y_shared may be NULL (S == 0). Writes o->y and (o->y_lowp).               */
int moe_combine(const moe_config *cfg, int64_t T, const float *y_routed,
                const float *y_shared, moe_outputs *o, void *stream);

/* fp8 expert weights from bf16 ones (cfg->dtype == MOE_FP8). For every expert
   matrix of src (bf16, the MOE_BF16 layouts) writes dst's codes and scales
   (layouts in moe_weights): per output column o of the product the matrix
   enters, the scale is the smallest power of two s with max |W[., o]| / s <= 448,
   and each code is W / s rounded to the nearest E4M3 value, ties to even.
   Dense experts (rank 0) then run on the fp8 MFMA: the activations entering
   each product (x rows over d, h rows over F -- for the shared experts one row
   of S*F) are quantised the same way, per row, inside moe_layer_forward.
   Low-rank experts (rank 64) store only their factors in fp8: U per column,
   V per row (its product z V^T sums over r); the products stay bf16 and
   dst->s_gate, s_up, s_down must point to the bf16 s vectors. dst's arrays
   are caller-allocated device memory; src->w_router is not touched.          */
int moe_quantize_fp8(const moe_config *cfg, const moe_weights *src, moe_weights *dst,
                     void *stream);

/* Loss-free balancing step (dormouse site, stack list "dropless MoE + LFB":
   balancing by a router bias instead of an auxiliary loss; Sutra-1.3B site,
   "48 + 1 experts" card: bias-based load balancing). For every routed expert e:
     select_bias[e] += gamma * sign(T * top_k - n_routed * counts[e])
   i.e. the bias of an expert with fewer pre-drop slots than the mean T k / E
   rises by gamma, above the mean it falls by gamma, at the mean it stays; one
   float32 addition per expert. counts [E] int32 device (o->counts of the
   routing call, before capacity); select_bias [E] float32 device, updated in
   place (the array moe_route reads for the sigmoid rule). gamma must be
   finite. Enqueued on `stream`; returns MOE_EINVAL for a bad configuration,
   T < 0, a null pointer or a non-finite gamma.                              */
int moe_bias_update(const moe_config *cfg, int64_t T, const int32_t *counts,
                    float *select_bias, float gamma, void *stream);

/* The whole layer forward (route, permute, grouped FFN for routed and shared
   experts, combine), as defined at the top of this file from the research
   page "Architecture" section, the Quartz model card "Architecture" table,
   the Moonfrost MoE and stacking cards, the Sutra-1.3B "48 + 1 experts" card
   and the dormouse "dropless MoE" and "TSCT low-rank experts" cards.
   In: x [T, d] device (cfg.dtype; bf16 for MOE_FP8); w as above. Out: every
   output of o (optional ones when non-NULL). Intermediates live in ws
   (moe_workspace_bytes, 256-byte aligned); errors as for every entry point. */
int moe_layer_forward(const moe_config *cfg, int64_t T, const void *x,
                      const moe_weights *w, moe_outputs *o, void *ws, size_t ws_bytes,
                      void *stream);

/* For callers that cannot allocate device memory or pass a workspace (code
   under HIP graph capture, tight serving loops, harnesses that forbid
   allocation): moe_layer_forward with its workspace in a device array of
   MOE_NOALLOC_SCRATCH_BYTES that the library itself holds, one copy per GPU,
   kept until the process ends. The caller still passes x, w and o. A call
   whose moe_workspace_bytes(cfg, T) exceeds the array returns
   MOE_EWORKSPACE before anything is launched (the Quartz-shaped layer fits
   up to 1,719 tokens, the Sutra-shaped one 1,737). Nothing in the array has to start at zero:
   every call writes what it reads there. Every call on one GPU shares that
   GPU's array, so calls that may overlap on one GPU (different streams, or
   different host threads) race; calls on one stream are ordered. The
   device address of each GPU's array is looked up on the first call with
   that GPU current (hipGetSymbolAddress); no call allocates or frees.     */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int moe_layer_forward_noalloc(const moe_config *cfg, int64_t T, const void *x,
                              const moe_weights *w, moe_outputs *o, void *stream);

/* Same as moe_layer_forward, and records events[2i] and events[2i+1]
   (hipEvent_t, caller-created) immediately before and after the launch of
   kernel i, on the stream that kernel runs on, for 2i+1 < n_events; returns
   the number of kernels launched (>= 0) or a moe_status. moe_stage_name(i)
   names kernel i of the last such call.                                     */
int moe_layer_forward_timed(const moe_config *cfg, int64_t T, const void *x,
                            const moe_weights *w, moe_outputs *o, void *ws,
                            size_t ws_bytes, void *stream, void **events, int n_events);
const char *moe_stage_name(int i);

/* ---- backward --------------------------------------------------------------
   Gradients of  L = sum(dy * y) + aux_grad * aux  for the layer above (every
   page trains it: the Quartz card's training setup, the Moonfrost stacking and
   training cards, the Sutra-1.3B and dormouse training notes). The top-k
   choice, the capacity drops and the counts in f are held fixed (they carry
   no gradient); the selection bias of the sigmoid rule gets none. h is taken
   as rounded in the forward (straight through). In bf16 layers the operands
   of the backward products are rounded to bf16 where they are formed: the
   routed upstream rows gate * dy, the shared upstream rows dy, the SwiGLU
   gradients da = dh * b * SiLU'(a) and db = dh * SiLU(a), and the router-logit
   gradient; every sum is float32.
   Outputs, float32 device arrays, overwritten (not accumulated):            */
typedef struct {
  float *dx;          /* [T, d]                                              */
  float *dw_router;   /* [d, E]                                              */
  float *dw_gate;     /* [E, d, F]                                           */
  float *dw_up;       /* [E, d, F]                                           */
  float *dw_down;     /* [E, F, d]                                           */
  float *dsh_gate;    /* [S, d, F]  (NULL allowed when S == 0)               */
  float *dsh_up;      /* [S, d, F]                                           */
  float *dsh_down;    /* [S, F, d]                                           */
  /* rank-r experts (rank > 0): the gradients of their factors, in the
     factors' own shapes (dw_gate, dw_up, dw_down are then unused, NULL
     allowed); the dormouse "TSCT low-rank experts" card's U diag(s) V^T      */
  float *du_gate, *ds_gate, *dv_gate;   /* [E, d, r], [E, r], [E, F, r]      */
  float *du_up,   *ds_up,   *dv_up;     /* [E, d, r], [E, r], [E, F, r]      */
  float *du_down, *ds_down, *dv_down;   /* [E, F, r], [E, r], [E, d, r]      */
} moe_grads;

/* Bytes of the backward's own workspace for this config and T (0 if cfg is
   invalid). */
size_t moe_backward_workspace_bytes(const moe_config *cfg, int64_t T);

/* Intermediates that moe_layer_backward leaves in bwd_ws, for inspection after
   the call (parity checks, debugging); valid until the next call on the same
   bwd_ws. Rows are the dispatched rows in the forward's expert-sorted order
   (rows at and beyond offsets[E] hold no data). moe_backward_workspace_region
   gives the byte offset into bwd_ws and the size of region `which`; a size of
   0 means the config has no such region. Returns MOE_EINVAL for an invalid
   config, T < 0, NULL outputs or an unknown region.
     MOE_BWS_DY_ROUTED   [R_max, d]: gate * dy of each row (bf16, rounded; float32
                         in a MOE_F32 layer, as the next three)
     MOE_BWS_X_PERM      [R_max, d]: x of each row's token
     MOE_BWS_DAB         [R_max, 2F]: da | db of each row
     MOE_BWS_DL          [T, E]: the router-logit gradient
     MOE_BWS_DAB_SHARED  [T, S*2F]: the shared experts' da | db of each token
   rank-r experts (W = U diag(s) V^T of the dormouse "TSCT low-rank experts"
   card), per row, the recomputed forward chain and the backward's:
     MOE_BWS_LR_UG, _UU  float32 [R_max, r]: x U_gate, x U_up
     MOE_BWS_LR_Z_GU     bf16 [R_max, 2r]: zg | zu = bf16(x U s) of gate, up
     MOE_BWS_LR_AB       float32 [R_max, 2F]: a | b = zg V_gate^T | zu V_up^T
     MOE_BWS_LR_H        bf16 [R_max, F]: h = bf16(SiLU(a) b)
     MOE_BWS_LR_UD       float32 [R_max, r]: h U_down
     MOE_BWS_LR_ZD       bf16 [R_max, r]: bf16(h U_down s_down)
     MOE_BWS_LR_DZD      float32 [R_max, r]: (gate dy) V_down
     MOE_BWS_LR_DUD      bf16 [R_max, r]: bf16(dzd s_down)
     MOE_BWS_LR_DZG, _DZU float32 [R_max, r]: da V_gate, db V_up
     MOE_BWS_LR_DU_GU    bf16 [R_max, 2r]: bf16(dzg s_gate) | bf16(dzu s_up)  */
enum {
  MOE_BWS_DY_ROUTED = 0, MOE_BWS_X_PERM = 1, MOE_BWS_DAB = 2, MOE_BWS_DL = 3,
  MOE_BWS_LR_UG = 4, MOE_BWS_LR_UU = 5, MOE_BWS_LR_Z_GU = 6, MOE_BWS_LR_AB = 7,
  MOE_BWS_LR_H = 8, MOE_BWS_LR_UD = 9, MOE_BWS_LR_ZD = 10, MOE_BWS_LR_DZD = 11,
  MOE_BWS_LR_DUD = 12, MOE_BWS_LR_DZG = 13, MOE_BWS_LR_DZU = 14, MOE_BWS_LR_DU_GU = 15,
  MOE_BWS_DAB_SHARED = 16
};
int moe_backward_workspace_region(const moe_config *cfg, int64_t T, int32_t which,
                                  size_t *offset, size_t *bytes);

/* Layer backward. Must follow moe_layer_forward on the same stream with the
   same cfg, T, x and w; o and ws are that call's outputs and workspace, read
   here and not modified (h, the shared h and the expert output rows of the
   forward live in ws). dy [T, d] float32 device: the loss gradient of o->y;
   aux_grad: the loss gradient of aux (o->aux[1]), finite. bwd_ws: device,
   256-byte aligned, at least moe_backward_workspace_bytes. This library: bf16
   layers with n_routed a multiple of 8, of dense experts, or of rank-32 or
   rank-64 experts (beside dense shared experts or none); MOE_F32 layers of dense experts
   (every operand and sum in float32, no rounding points); otherwise
   MOE_EUNSUPPORTED.
   The result does not depend on scheduling (fixed summation orders, no
   atomics).                                                                 */
int moe_layer_backward(const moe_config *cfg, int64_t T, const void *x, const moe_weights *w,
                       const moe_outputs *o, const float *dy, float aux_grad, moe_grads *g,
                       const void *ws, size_t ws_bytes, void *bwd_ws, size_t bwd_ws_bytes,
                       void *stream);
/* Same, recording events around each kernel as moe_layer_forward_timed does. */
int moe_layer_backward_timed(const moe_config *cfg, int64_t T, const void *x,
                             const moe_weights *w, const moe_outputs *o, const float *dy,
                             float aux_grad, moe_grads *g, const void *ws, size_t ws_bytes,
                             void *bwd_ws, size_t bwd_ws_bytes, void *stream, void **events,
                             int n_events);

/* Static text for a status code, and the text of the last MOE_EHIP error of the
   calling thread. */
const char *moe_status_str(int status);
const char *moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* FGM_MOE_H */
