"""Plain, slow CPU oracle of the fine-grained MoE feed-forward layer.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The product path
(the HIP library and its Python binding) never imports, links or calls it, and
this module imports nothing from the product path.

Everything is evaluated in float64 on the exact input values. The layer is a
per-token definition; the GPU reaches the same result by regrouping tokens by
expert, so this oracle simply evaluates the definition token by token over the
experts each token selected.

Sources (pages as cited; the formulas not printed on any page are readings,
listed in the design notes of this repository):
  * Router with top-k of E routed experts plus always-on shared experts: Vertex
    AGI research page, Architecture ("Router", "Routed experts", "Shared
    experts"); Quartz Micro Preview Base model card, Architecture table; Moonfrost
    site, MoE card (top 3 of 32 plus one shared expert, so 4 of 33 run).
  * Sigmoid scoring with a bias used for balancing: Sutra-1.3B site, "48 + 1
    experts" card; dormouse site, stack list ("dropless MoE + LFB": balancing by a
    router bias rather than an auxiliary loss).
  * 0.01-weighted load-balancing loss: research page Architecture, model card
    Architecture table. Its form E * sum_i f_i * P_i is the reading used here.
  * Capacity-based routing over stacked (E, hidden, ffn) expert tensors: Moonfrost
    site, stacking card. Dropless routing (every token keeps every expert it
    chose, capacity 0 meaning dropless): dormouse site, "dropless MoE" card and
    terminal block.
  * Low-rank experts, each matrix U diag(s) V^T of rank 64: dormouse site, "TSCT
    low-rank experts" card.
  * Gated (three-matrix) experts of width F: consistent with the parameter totals
    on the research page and model card (see tests/golden).

Readings where the pages are silent: SwiGLU experts without biases; softmax
ranking by logit with ties to the lower expert id; gates renormalised over the
top-k when the workload says so; sigmoid gates are the selected sigmoid scores
normalised to sum 1 and the selection bias moves selection only; capacity queues
are in token order; the bf16 rounding points rho are the SwiGLU product h and the
rank-r intermediates z (identity for float32 workloads).

Parity unpinned: no page prints layer inputs or outputs, so no function here is
checked against page values; every function is pinned by brute force on tiny
inputs, closed forms, invariants and textbook reductions instead (tests/).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

SOFTMAX = "softmax"
SIGMOID = "sigmoid"


@dataclass(frozen=True)
class LayerSpec:
    """The layer's hyper-parameters, as the pages state a model's MoE block."""

    hidden: int          # d
    n_routed: int        # E
    top_k: int           # k
    n_shared: int        # S
    ffn: int             # F
    rank: int = 0        # 0: dense experts
    score: str = SOFTMAX
    renorm: bool = True  # softmax: divide the selected probabilities by their sum
    capacity: int = 0    # 0: dropless
    aux_coef: float = 0.01
    bf16: bool = True    # rho rounds to bf16 (bf16 workloads); identity for float32
    fp8: bool = False    # expert products on fp8 (e4m3) codes: weights per column, rows per row


# ---------------------------------------------------------------------------
# rho: round to the nearest bf16 value, ties to even, from float64 directly.
# bf16 keeps 8 significant bits and float32's exponent range.
# ---------------------------------------------------------------------------
_BF16_MAX = float.fromhex("0x1.fep127")
_BF16_MIN_NORMAL = 2.0 ** -126


def round_bf16(a) -> np.ndarray:
    a = np.asarray(a, dtype=np.float64)
    out = np.empty_like(a)
    fin = np.isfinite(a)
    mant, expo = np.frexp(np.where(fin, a, 0.0))         # a = mant * 2**expo, |mant| in [0.5, 1)
    normal = np.abs(a) >= _BF16_MIN_NORMAL
    # normal range: 8 significant bits -> mant * 256 rounded half-to-even
    rn = np.ldexp(np.rint(mant * 256.0), expo - 8)
    # subnormal range: fixed spacing 2**-133
    rs = np.ldexp(np.rint(np.ldexp(np.where(fin, a, 0.0), 133)), -133)
    out[...] = np.where(normal, rn, rs)
    # anything that rounds beyond the largest finite bf16 overflows
    big = np.abs(out) > _BF16_MAX
    out[big] = np.copysign(np.inf, a[big])
    out[~fin] = a[~fin]
    return out


# ---------------------------------------------------------------------------
# fp8 (the storage ladder's first rung, dormouse "TSCT low-rank experts" card):
# OCP E4M3 -- sign, 4 exponent bits (bias 7), 3 mantissa bits; normal values
# (1 + m/8) 2^(e-7) for e = 1..15 except the all-ones code (NaN), subnormals
# (m/8) 2^-6; largest finite 448. A vector is stored as codes times one power of
# two 2^s per row (activations) or per output column (weights), s the smallest
# integer with amax 2^-s <= 448, so that scaling is exact and the only rounding
# is round-to-nearest-even of v 2^-s onto the E4M3 grid.
# ---------------------------------------------------------------------------
E4M3_MAX = 448.0


def e4m3_round(v) -> np.ndarray:
    """Nearest E4M3 value to v (|v| <= 448), ties to the even mantissa."""
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    frac, ex = np.frexp(np.where(a > 0, a, 1.0))       # a = frac 2^ex, frac in [0.5, 1)
    e = ex - 1                                          # a = (2 frac) 2^e, 2 frac in [1, 2)
    normal = a >= 2.0 ** -6
    qn = np.ldexp(np.rint(np.ldexp(a, 3 - e)), e - 3)   # 3 fraction bits at exponent e
    qs = np.ldexp(np.rint(np.ldexp(a, 9)), -9)          # subnormal spacing 2^-9
    q = np.where(normal, qn, qs)
    return np.copysign(q, v)


def fp8_scale_exp(amax) -> np.ndarray:
    """Smallest integer s with amax 2^-s <= 448 (0 where amax is 0)."""
    amax = np.asarray(amax, np.float64)
    frac, ex = np.frexp(np.where(amax > 0, amax, 1.0))  # amax = frac 2^ex
    s = np.where(frac <= 0.875, ex - 9, ex - 8)          # 448 = 0.875 2^9
    return np.where(amax > 0, s, 0).astype(np.int64)


def fp8_quantize(m, axis):
    """Quantise m along `axis` (the summed dimension of its product): one
    scale per slice. Returns (the dequantised values q 2^s, s)."""
    m = np.asarray(m, np.float64)
    s = fp8_scale_exp(np.max(np.abs(m), axis=axis, keepdims=True))
    return np.ldexp(e4m3_round(np.ldexp(m, -s)), s), np.squeeze(s, axis)


def _rho(spec: LayerSpec):
    return round_bf16 if spec.bf16 else (lambda v: np.asarray(v, dtype=np.float64))


def silu(z):
    """SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def sigmoid(z):
    z = np.asarray(z, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-z))


# ---------------------------------------------------------------------------
# Router: projection, scores, top-k selection, gates
# ---------------------------------------------------------------------------
def router_logits(x, w_router, logit_bias=None) -> np.ndarray:
    """l[t, i] = sum_c x[t, c] * W_r[c, i] + logit_bias[i]   (float64)."""
    l = np.asarray(x, np.float64) @ np.asarray(w_router, np.float64)
    if logit_bias is not None:
        l = l + np.asarray(logit_bias, np.float64)[None, :]
    return l


def router_scores(l, spec: LayerSpec, select_bias=None):
    """Returns (key, prob, sig).

    key  -- what top-k ranks by: the logit (softmax rule), or sigmoid + selection
            bias (sigmoid rule);
    prob -- the full per-token distribution over experts used by the aux
            statistic: softmax(l), or s / sum(s) for the sigmoid rule;
    sig  -- sigmoid scores (sigmoid rule) or None.
    """
    l = np.asarray(l, np.float64)
    if spec.score == SOFTMAX:
        m = l.max(axis=1, keepdims=True)
        ex = np.exp(l - m)
        prob = ex / ex.sum(axis=1, keepdims=True)
        return l.copy(), prob, None
    if spec.score == SIGMOID:
        s = sigmoid(l)
        key = s + (0.0 if select_bias is None else np.asarray(select_bias, np.float64)[None, :])
        prob = s / s.sum(axis=1, keepdims=True)
        return key, prob, s
    raise ValueError(spec.score)


def select_topk(key, k):
    """Experts ordered by descending key, equal keys to the lower id first.

    Returns idx [T, k] and margin [T] = key of the k-th minus key of the
    (k+1)-th expert (+inf when k == E).
    """
    key = np.asarray(key, np.float64)
    T, E = key.shape
    order = np.argsort(-key, axis=1, kind="stable")
    idx = order[:, :k].astype(np.int64)
    if k < E:
        rows = np.arange(T)
        margin = key[rows, order[:, k - 1]] - key[rows, order[:, k]]
    else:
        margin = np.full(T, np.inf)
    return idx, margin


def token_gates(t, sel, prob, sig, spec: LayerSpec) -> np.ndarray:
    """Gate weights of token t's selected experts, in selection order."""
    sel = np.asarray(sel)
    if spec.score == SOFTMAX:
        g = prob[t, sel].astype(np.float64)
        if spec.renorm:
            g = g / g.sum()
        return g
    s = sig[t, sel].astype(np.float64)
    return s / s.sum()


# ---------------------------------------------------------------------------
# Dispatch: histogram, capacity, prefix sum, permutation
# ---------------------------------------------------------------------------
def dispatch(idx, n_routed, capacity):
    """Group the T*k slots by expert in token order.

    Visiting tokens in ascending order (and each token's k choices in list
    order), a slot's position is the number of earlier slots on the same
    expert. With capacity C > 0 a slot is kept iff its position is below C;
    capacity 0 keeps every slot. Kept slots of expert e occupy rows
    offsets[e] + position, offsets being the exclusive prefix sum of the kept
    counts.
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    E = n_routed
    running = [0] * E
    pos = np.zeros((T, k), np.int64)
    keep = np.zeros((T, k), bool)
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            p = running[e]
            running[e] = p + 1
            pos[t, j] = p
            keep[t, j] = capacity == 0 or p < capacity
    counts = np.array(running, np.int64)
    kept = np.minimum(counts, capacity) if capacity > 0 else counts.copy()
    offsets = np.zeros(E + 1, np.int64)
    offsets[1:] = np.cumsum(kept)
    row_of_slot = np.full((T, k), -1, np.int64)
    sorted_token = np.full(int(offsets[E]), -1, np.int64)
    for t in range(T):
        for j in range(k):
            if keep[t, j]:
                row = int(offsets[idx[t, j]] + pos[t, j])
                row_of_slot[t, j] = row
                sorted_token[row] = t
    dropped = ~keep
    return dict(counts=counts, kept=kept, offsets=offsets, pos=pos,
                row_of_slot=row_of_slot, sorted_token=sorted_token,
                dropped=dropped, n_dropped=int(dropped.sum()))


# ---------------------------------------------------------------------------
# Experts
# ---------------------------------------------------------------------------
class _Bank:
    """float64 views of one expert bank, converted lazily per expert."""

    def __init__(self, arr):
        self.arr = arr
        self.cache = {}

    def __getitem__(self, e):
        m = self.cache.get(e)
        if m is None:
            m = np.asarray(self.arr[e], np.float64)
            self.cache[e] = m
        return m


def swiglu(xrow, w_gate, w_up, w_down, rho):
    """W_down^T applied to rho(SiLU(x W_gate) * (x W_up)) for one token row."""
    a = xrow @ w_gate
    b = xrow @ w_up
    h = rho(silu(a) * b)
    return h @ w_down


def lowrank_apply(v, u, s, vmat, rho):
    """v W with W = U diag(s) V^T: z = rho((v U) * s), then z V^T."""
    z = rho((v @ u) * s)
    return z @ vmat.T


def lowrank_swiglu(xrow, f, rho):
    """SwiGLU expert whose three matrices are each rank-r factorised."""
    a = lowrank_apply(xrow, f["u_gate"], f["s_gate"], f["v_gate"], rho)
    b = lowrank_apply(xrow, f["u_up"], f["s_up"], f["v_up"], rho)
    h = rho(silu(a) * b)
    return lowrank_apply(h, f["u_down"], f["s_down"], f["v_down"], rho)


class _Fp8Bank:
    """float64 values of an expert bank quantised to fp8, one scale per output
    column of the product the matrix enters: reduced over `axis` (0 for
    W[in, out], 1 for a factor V[out, r] entering z V^T)."""

    def __init__(self, arr, axis=0):
        self.arr = arr
        self.axis = axis
        self.cache = {}

    def __getitem__(self, e):
        m = self.cache.get(e)
        if m is None:
            m = fp8_quantize(np.asarray(self.arr[e], np.float64), axis=self.axis)[0]
            self.cache[e] = m
        return m


def swiglu_fp8(xrow, w_gate, w_up, w_down, rho, with_max=False):
    """SwiGLU with fp8 products: the row entering each product is quantised
    (x over d, h = rho(SiLU(a) b) over F); the weights come quantised. With
    ``with_max`` also returns, per output column, the largest magnitude of one
    term of the down product (the error scale of a quantised h entry).
    ``xrow`` may also be a matrix of rows (each quantised on its own; not with
    ``with_max``)."""
    xq = fp8_quantize(xrow, axis=-1)[0]
    h = rho(silu(xq @ w_gate) * (xq @ w_up))
    hq = fp8_quantize(h, axis=-1)[0]
    y = hq @ w_down
    if not with_max:
        return y
    return y, (np.abs(hq)[:, None] * np.abs(w_down)).max(axis=0)


class Experts:
    """Routed and shared expert weights of one layer in float64."""

    def __init__(self, weights: dict, spec: LayerSpec):
        self.spec = spec
        self.rho = _rho(spec)
        if spec.fp8:
            if not spec.bf16:
                raise ValueError("fp8 experts: bf16 layers only")
            if spec.rank == 0:
                self.gate = _Fp8Bank(weights["w_gate"])
                self.up = _Fp8Bank(weights["w_up"])
                self.down = _Fp8Bank(weights["w_down"])
            else:
                # low-rank factors stored in fp8: U[in, r] per column r, V[out, r]
                # per row (its product z V^T sums over r); s stays bf16; the
                # products and their rounding points are the bf16 ones
                self.lr = {n: _Fp8Bank(weights[n], axis=0)
                           for n in ("u_gate", "u_up", "u_down")}
                self.lr.update({n: _Fp8Bank(weights[n], axis=1)
                                for n in ("v_gate", "v_up", "v_down")})
                self.lr.update({n: _Bank(weights[n]) for n in ("s_gate", "s_up", "s_down")})
            self.S = spec.n_shared
            if self.S > 0:
                S, F, d = self.S, spec.ffn, spec.hidden
                # the shared experts' down projections are one product over
                # their stacked S F rows (summed experts): one scale per column
                self.sh = [_Fp8Bank(weights["sh_gate"]), _Fp8Bank(weights["sh_up"])]
                self.sh_down = fp8_quantize(
                    np.asarray(weights["sh_down"], np.float64).reshape(S * F, d), axis=0)[0]
            return
        if spec.rank == 0:
            self.gate = _Bank(weights["w_gate"])
            self.up = _Bank(weights["w_up"])
            self.down = _Bank(weights["w_down"])
        else:
            self.lr = {n: _Bank(weights[n]) for n in (
                "u_gate", "s_gate", "v_gate", "u_up", "s_up", "v_up",
                "u_down", "s_down", "v_down")}
        self.S = spec.n_shared
        if self.S > 0:
            self.sh = [_Bank(weights["sh_gate"]), _Bank(weights["sh_up"]),
                       _Bank(weights["sh_down"])]

    def routed(self, xrow, e, with_max=False):
        if self.spec.fp8 and self.spec.rank == 0:
            return swiglu_fp8(xrow, self.gate[e], self.up[e], self.down[e], self.rho, with_max)
        if self.spec.fp8:
            f = {n: b[e] for n, b in self.lr.items()}
            y = lowrank_swiglu(xrow, f, self.rho)
            return (y, np.zeros_like(y)) if with_max else y
        if self.spec.rank == 0:
            return swiglu(xrow, self.gate[e], self.up[e], self.down[e], self.rho)
        f = {n: b[e] for n, b in self.lr.items()}
        return lowrank_swiglu(xrow, f, self.rho)

    def shared(self, xrow, with_max=False):
        """Sum of the shared experts on one token row (or on a matrix of rows,
        without ``with_max``)."""
        if self.spec.fp8:
            # h of every shared expert, quantised as one row of S F values
            xq = fp8_quantize(xrow, axis=-1)[0]
            h = np.concatenate([self.rho(silu(xq @ self.sh[0][s]) * (xq @ self.sh[1][s]))
                                for s in range(self.S)], axis=-1)
            hq = fp8_quantize(h, axis=-1)[0]
            y = hq @ self.sh_down
            if not with_max:
                return y
            return y, (np.abs(hq)[:, None] * np.abs(self.sh_down)).max(axis=0)
        out = np.zeros(np.shape(xrow)[:-1] + (self.spec.hidden,))
        for s in range(self.S):
            out = out + swiglu(xrow, self.sh[0][s], self.sh[1][s], self.sh[2][s], self.rho)
        return out


# ---------------------------------------------------------------------------
# Aux load-balancing statistic
# ---------------------------------------------------------------------------
def aux_statistic(counts, prob, T, k, spec: LayerSpec):
    """f_i = counts_i / (T k) (pre-drop), P_i = mean_t prob[t, i],
    aux_raw = E * sum_i f_i P_i, aux = aux_coef * aux_raw."""
    f = np.asarray(counts, np.float64) / float(T * k)
    P = np.asarray(prob, np.float64).sum(axis=0) / float(T)
    aux_raw = spec.n_routed * float(np.sum(f * P))
    return dict(f=f, P=P, aux_raw=aux_raw, aux=spec.aux_coef * aux_raw)


# ---------------------------------------------------------------------------
# Loss-free balancing: one update of the selection bias
# ---------------------------------------------------------------------------
def bias_update(select_bias, counts, T, k, gamma):
    """Bias-based balancing in place of an auxiliary loss (dormouse site, stack
    list "dropless MoE + LFB", which points to the auxiliary-loss-free balancing
    method; Sutra-1.3B site, "48 + 1 experts" card: bias-based load balancing).

    Each expert's selection bias moves by gamma toward balance: up when its
    pre-drop slot count is below the mean T k / E, down when above, unchanged
    when equal. The comparison is made in integers (T k against E counts_i).
    The new bias is the float32 value nearest to b_i + gamma sign(T k - E c_i);
    with float32 inputs the float64 sum is exact whenever the binary exponents
    of b_i and gamma differ by at most 29, so that single rounding is the float32
    addition's own.
    """
    b = np.asarray(select_bias, np.float32).astype(np.float64)
    c = np.asarray(counts, np.int64)
    n_routed = c.shape[0]
    direction = np.sign(int(T) * int(k) - n_routed * c).astype(np.float64)
    g = float(np.float32(gamma))
    return (b + g * direction).astype(np.float32)


# ---------------------------------------------------------------------------
# The layer
# ---------------------------------------------------------------------------
def route(x, w_router, spec: LayerSpec, logit_bias=None, select_bias=None,
          override_idx=None, override_mask=None):
    """Router projection, scores, top-k and gates for every token.

    override_idx/override_mask force the selection of the masked tokens (used
    for near-tie tokens, where either choice is correct); their gates are then
    computed by the same formulas from the forced set.
    """
    l = router_logits(x, w_router, logit_bias)
    key, prob, sig = router_scores(l, spec, select_bias)
    idx, margin = select_topk(key, spec.top_k)
    if override_mask is not None:
        mask = np.asarray(override_mask, bool)
        idx = idx.copy()
        idx[mask] = np.asarray(override_idx)[mask]
    T = idx.shape[0]
    gates = np.zeros(idx.shape)
    for t in range(T):
        gates[t] = token_gates(t, idx[t], prob, sig, spec)
    return dict(logits=l, key=key, prob=prob, sig=sig, idx=idx, margin=margin,
                gates=gates)


def layer_forward(x, weights: dict, spec: LayerSpec, tokens=None,
                  override_idx=None, override_mask=None, scales=False):
    """The whole layer. y is evaluated for ``tokens`` (default: all tokens),
    routing and dispatch for every token (capacity decisions need them all).

    Returns a dict with the router outputs, the dispatch tables, the aux
    statistic and ``y`` [len(tokens), d] in float64. With ``scales`` (fp8
    experts), also ``M_y``: per element of y the largest magnitude of one term
    g h_f W_down[f, c] of its down products.
    """
    x = np.asarray(x)
    T = x.shape[0]
    r = route(x, weights["w_router"], spec, weights.get("logit_bias"),
              weights.get("select_bias"), override_idx, override_mask)
    dsp = dispatch(r["idx"], spec.n_routed, spec.capacity)
    aux = aux_statistic(dsp["counts"], r["prob"], T, spec.top_k, spec)
    experts = Experts(weights, spec)
    toks = np.arange(T) if tokens is None else np.asarray(tokens, np.int64)
    y = np.zeros((len(toks), spec.hidden))
    want_max = scales and spec.fp8
    m_y = np.zeros((len(toks), spec.hidden)) if want_max else None
    for n, t in enumerate(toks):
        xrow = np.asarray(x[t], np.float64)
        acc = np.zeros(spec.hidden)
        if spec.n_shared > 0:
            if want_max:
                ys, ms = experts.shared(xrow, True)
                acc = acc + ys
                m_y[n] = ms
            else:
                acc = acc + experts.shared(xrow)
        for j in range(spec.top_k):
            if dsp["row_of_slot"][t, j] < 0:
                continue                      # dropped slot contributes nothing
            g = r["gates"][t, j]
            if want_max:
                yr, mr = experts.routed(xrow, int(r["idx"][t, j]), True)
                acc = acc + g * yr
                m_y[n] = np.maximum(m_y[n], g * mr)
            else:
                acc = acc + g * experts.routed(xrow, int(r["idx"][t, j]))
        y[n] = acc
    out = dict(r)
    out.update(dsp)
    out.update(aux)
    out["tokens"] = toks
    out["y"] = y
    if want_max:
        out["M_y"] = m_y
    return out


def layer_forward_batched(x, weights: dict, spec: LayerSpec, override_idx=None,
                          override_mask=None):
    """The same layer as layer_forward (same readings, same rounding points,
    the same order of the per-token sum: shared experts in ascending order,
    then the kept slots in list order), with every expert evaluated once over
    all of its rows with matrix products instead of token by token. For
    full-size checks; routing, dispatch and the aux statistic are
    layer_forward's own. y [T, d] covers every token."""
    x = np.asarray(x)
    T = x.shape[0]
    out = layer_forward(x, weights, spec, tokens=[], override_idx=override_idx,
                        override_mask=override_mask)
    x64 = np.asarray(x, np.float64)
    ex = Experts(weights, spec)
    k, d = spec.top_k, spec.hidden
    idx, gates, rows = out["idx"], out["gates"], out["row_of_slot"]
    y = np.zeros((T, d))
    if spec.n_shared > 0 and T > 0:
        y = y + ex.shared(x64)
    # one output row per kept (token, slot), every expert over its own rows
    o = np.zeros((T, k, d))
    for e in range(spec.n_routed):
        ts, js = np.nonzero((idx == e) & (rows >= 0))
        if len(ts):
            o[ts, js] = ex.routed(x64[ts], e)
    for j in range(k):
        kept = rows[:, j] >= 0
        y[kept] = y[kept] + gates[kept, j, None] * o[kept, j]
    out["tokens"] = np.arange(T)
    out["y"] = y
    return out


# ---------------------------------------------------------------------------
# Backward of the layer
# ---------------------------------------------------------------------------
def dsilu(z):
    """d/dz of z * sigmoid(z)."""
    s = sigmoid(z)
    return s * (1.0 + z * (1.0 - s))


def _expert_backward(xrow, wg, wu, wd, dyrow, rho, grads, key, scales=None):
    """One SwiGLU expert on one token: y = rho(SiLU(x Wg) * (x Wu)) Wd with the
    upstream gradient dyrow (already rounded where the layer rounds it).
    Adds to grads[key] = [dWg, dWu, dWd] and returns dx. rho is straight-through
    on h; the gradients entering the two gate/up products, da and db, are
    rounded with rho (they are the bf16 operands of those products).

    With ``scales`` (a dict), also accumulates for every gradient element the
    largest single product term and the sum of the terms' magnitudes, in
    scales[key] = [(M, S) for dWg, dWu, dWd], and returns (dx, M_dx, S_dx)."""
    a = xrow @ wg
    b = xrow @ wu
    h = rho(silu(a) * b)
    dWg, dWu, dWd = grads[key]
    dWd += np.outer(h, dyrow)
    dh = wd @ dyrow
    da = rho(dh * b * dsilu(a))
    db = rho(dh * silu(a))
    dWg += np.outer(xrow, da)
    dWu += np.outer(xrow, db)
    dx = wg @ da + wu @ db
    if scales is None:
        return dx
    ax = np.abs(xrow)
    for (M, S), (u, v) in zip(scales[key], ((ax, np.abs(da)), (ax, np.abs(db)),
                                             (np.abs(h), np.abs(dyrow)))):
        t = np.outer(u, v)
        np.maximum(M, t, out=M)
        S += t
    tg = np.abs(wg) * np.abs(da)
    tu = np.abs(wu) * np.abs(db)
    return dx, np.maximum(tg.max(axis=1), tu.max(axis=1)), tg.sum(axis=1) + tu.sum(axis=1)


LOWRANK_GRADS = ("du_gate", "ds_gate", "dv_gate", "du_up", "ds_up", "dv_up",
                 "du_down", "ds_down", "dv_down")


def _lowrank_expert_backward(xrow, f, dyrow, rho, grads, key):
    """One rank-r SwiGLU expert (each matrix W[in, out] = U[in, r] diag(s) V[out, r]^T,
    dormouse "TSCT low-rank experts" card) on one token row, with the
    upstream gradient dyrow of its output (already rounded where the layer
    rounds it). The forward is re-evaluated with its rounding points:
    z_g = rho((x U_g) s_g), a = z_g V_g^T, the same for up, h = rho(SiLU(a) b),
    z_d = rho((h U_d) s_d), o = z_d V_d^T; rho is straight-through. The
    gradients entering the backward's products are rounded with rho where
    those products take bf16 operands: da and db (as for dense experts) and,
    in the factor chains, dz_d s_d, dz_g s_g and dz_u s_u. Adds to
    grads[key][name] for the nine factor gradients and returns dx."""
    ug = xrow @ f["u_gate"]
    zg = rho(ug * f["s_gate"])
    a = zg @ f["v_gate"].T
    uu = xrow @ f["u_up"]
    zu = rho(uu * f["s_up"])
    b = zu @ f["v_up"].T
    h = rho(silu(a) * b)
    ud = h @ f["u_down"]
    zd = rho(ud * f["s_down"])
    G = grads[key]
    dzd = f["v_down"].T @ dyrow            # sum over the output columns c of dy_c V_d[c, i]
    G["dv_down"] += np.outer(dyrow, zd)
    G["ds_down"] += dzd * ud
    dud = rho(dzd * f["s_down"])
    G["du_down"] += np.outer(h, dud)
    dh = f["u_down"] @ dud
    da = rho(dh * b * dsilu(a))
    db = rho(dh * silu(a))
    dzg = f["v_gate"].T @ da
    dzu = f["v_up"].T @ db
    G["dv_gate"] += np.outer(da, zg)
    G["dv_up"] += np.outer(db, zu)
    G["ds_gate"] += dzg * ug
    G["ds_up"] += dzu * uu
    dug = rho(dzg * f["s_gate"])
    duu = rho(dzu * f["s_up"])
    G["du_gate"] += np.outer(xrow, dug)
    G["du_up"] += np.outer(xrow, duu)
    return f["u_gate"] @ dug + f["u_up"] @ duu


def layer_backward(x, weights: dict, spec: LayerSpec, dy, aux_grad=0.0, fwd=None,
                   scales=False):
    """Gradients of L = sum(dy * y) + aux_grad * aux with respect to x, the
    router weight and every expert weight (dense experts).

    Readings (the pages train the layer but print no backward): the top-k
    choice and the capacity drops are held fixed (no gradient through the
    selection), as are the counts in f; rho on h is straight-through; the
    selection bias of the sigmoid rule receives no gradient. Where the layer
    works in bf16 the gradients entering the expert products are rounded with
    rho at the points where the products take bf16 operands: the routed
    upstream rows rho(g * dy), the shared upstream rows rho(dy), da and db, and
    the router-logit gradient rho(dl). Everything else is float64.

    Rank-r experts: their factor gradients du_gate, ds_gate, dv_gate, ... (the
    factors' own shapes) in place of dw_gate/up/down, with the rounding points
    of _lowrank_expert_backward.

    Returns dict dx [T, d], dw_router [d, E], dw_gate/up/down [E, ...] and
    dsh_gate/up/down [S, ...]. With ``scales``, also M_<name> and S_<name> for
    each of them: per element, the largest magnitude of a single product term
    of its sums, and the sum of those magnitudes (error scales of a result
    formed from rounded operands; the terms of dx are its products' terms
    with the weights).
    """
    if spec.fp8 or (spec.rank != 0 and scales):
        raise NotImplementedError("backward of fp8 experts; scales of low-rank experts")
    x = np.asarray(x)
    T, d = x.shape
    E, k, S, F = spec.n_routed, spec.top_k, spec.n_shared, spec.ffn
    rho = _rho(spec)
    if fwd is None:
        fwd = layer_forward(x, weights, spec)
    dy = np.asarray(dy, np.float64)
    ex = Experts(weights, spec)
    if spec.rank == 0:
        grads = {("r", e): [np.zeros((d, F)), np.zeros((d, F)), np.zeros((F, d))]
                 for e in range(E)}
    else:
        grads = {}
        lr_grads = {e: {n: np.zeros(np.shape(ex.lr[n[1:]][e])) for n in LOWRANK_GRADS}
                    for e in range(E)}
    for s in range(S):
        grads[("s", s)] = [np.zeros((d, F)), np.zeros((d, F)), np.zeros((F, d))]
    dx = np.zeros((T, d))
    dg = np.zeros((T, k))
    sc = None
    if scales:
        sc = {key: [(np.zeros_like(m), np.zeros_like(m)) for m in mats]
              for key, mats in grads.items()}
        mdx, sdx = np.zeros((T, d)), np.zeros((T, d))

    def run_expert(t, xrow, w3, dyrow, key):
        r = _expert_backward(xrow, *w3, dyrow, rho, grads, key, sc)
        if sc is None:
            dx[t] += r
        else:
            dx[t] += r[0]
            np.maximum(mdx[t], r[1], out=mdx[t])
            sdx[t] += r[2]

    idx, gates, rows = fwd["idx"], fwd["gates"], fwd["row_of_slot"]
    for t in range(T):
        xrow = np.asarray(x[t], np.float64)
        for s in range(S):
            run_expert(t, xrow, (ex.sh[0][s], ex.sh[1][s], ex.sh[2][s]), rho(dy[t]), ("s", s))
        for j in range(k):
            if rows[t, j] < 0:
                continue                      # dropped slot: no gradient
            e = int(idx[t, j])
            dg[t, j] = float(dy[t] @ ex.routed(xrow, e))
            if spec.rank == 0:
                run_expert(t, xrow, (ex.gate[e], ex.up[e], ex.down[e]),
                           rho(gates[t, j] * dy[t]), ("r", e))
            else:
                f = {n: b[e] for n, b in ex.lr.items()}
                dx[t] += _lowrank_expert_backward(xrow, f, rho(gates[t, j] * dy[t]), rho,
                                                  lr_grads, e)

    # router: gates -> logits, plus the aux statistic's dependence on the
    # routing distribution (f held fixed)
    l = router_logits(x, weights["w_router"], weights.get("logit_bias"))
    _, prob, sig = router_scores(l, spec)
    dl = np.zeros((T, E))
    f = np.asarray(fwd["f"], np.float64)
    c = aux_grad * spec.aux_coef * E / T
    for t in range(T):
        sel = idx[t]
        g = gates[t]
        if spec.score == SOFTMAX and spec.renorm:
            dl[t, sel] += g * (dg[t] - np.dot(g, dg[t]))
        elif spec.score == SOFTMAX:
            p = prob[t]
            dl[t] += -p * np.dot(p[sel], dg[t])
            dl[t, sel] += p[sel] * dg[t]
        else:
            st = sig[t, sel]
            dsig = (dg[t] - np.dot(g, dg[t])) / st.sum()
            dl[t, sel] += dsig * st * (1.0 - st)
        if spec.score == SOFTMAX:
            p = prob[t]
            dl[t] += c * p * (f - np.dot(f, p))
        else:
            st = sig[t]
            pr = prob[t]
            dl[t] += c * (f - np.dot(f, pr)) / st.sum() * st * (1.0 - st)
    wr = np.asarray(weights["w_router"], np.float64)
    dl = rho(dl)            # the operand of the two router products
    dx += dl @ wr.T
    out = dict(dx=dx, dw_router=np.asarray(x, np.float64).T @ dl, dl=dl, dg=dg)
    if spec.rank == 0:
        names = [("dw_gate", "r", E, 0), ("dw_up", "r", E, 1), ("dw_down", "r", E, 2)]
    else:
        names = []
        for n in LOWRANK_GRADS:
            out[n] = np.stack([lr_grads[e][n] for e in range(E)])
    if S > 0:
        names += [("dsh_gate", "s", S, 0), ("dsh_up", "s", S, 1), ("dsh_down", "s", S, 2)]
    for name, kind, n, i in names:
        out[name] = np.stack([grads[(kind, g)][i] for g in range(n)])
        if scales:
            out["M_" + name] = np.stack([sc[(kind, g)][i][0] for g in range(n)])
            out["S_" + name] = np.stack([sc[(kind, g)][i][1] for g in range(n)])
    if scales:
        ax, adl, awr = np.abs(np.asarray(x, np.float64)), np.abs(dl), np.abs(wr)
        tr = adl[:, None, :] * awr[None, :, :]          # [T, d, E] router terms of dx
        out["M_dx"] = np.maximum(mdx, tr.max(axis=2))
        out["S_dx"] = sdx + tr.sum(axis=2)
        out["M_dw_router"] = (ax[:, :, None] * adl[:, None, :]).max(axis=0)
        out["S_dw_router"] = ax.T @ adl
    return out


def _router_dl(l, idx, gates, dg, f, spec: LayerSpec, aux_grad, T):
    """Gradient of the loss with respect to the logits l [T, E] (unrounded):
    the gate terms of the selected experts and the aux statistic's term,
    vectorised over tokens (the same formulas as layer_backward's token loop)."""
    E, k = spec.n_routed, spec.top_k
    _, prob, sig = router_scores(l, spec)
    dl = np.zeros((T, E))
    ar = np.arange(T)[:, None]
    c = aux_grad * spec.aux_coef * E / T
    if spec.score == SOFTMAX and spec.renorm:
        gd = np.sum(gates * dg, axis=1, keepdims=True)
        np.add.at(dl, (ar, idx), gates * (dg - gd))
    elif spec.score == SOFTMAX:
        psel = np.take_along_axis(prob, idx, 1)
        dl -= prob * np.sum(psel * dg, axis=1, keepdims=True)
        np.add.at(dl, (ar, idx), psel * dg)
    else:
        st = np.take_along_axis(sig, idx, 1)
        gd = np.sum(gates * dg, axis=1, keepdims=True)
        dsig = (dg - gd) / st.sum(axis=1, keepdims=True)
        np.add.at(dl, (ar, idx), dsig * st * (1.0 - st))
    if spec.score == SOFTMAX:
        dl += c * prob * (f[None, :] - (prob @ f)[:, None])
    else:
        ssum = sig.sum(axis=1, keepdims=True)
        dl += c * (f[None, :] - (prob @ f)[:, None]) / ssum * sig * (1.0 - sig)
    return dl


def layer_backward_batched(x, weights: dict, spec: LayerSpec, dy, aux_grad=0.0, fwd=None):
    """The same gradients as layer_backward (same readings, same rounding
    points; dense or rank-r experts), computed per expert over all of its rows
    at once with matrix products instead of token by token, for full-size
    checks.

    Returns the gradients, their S_<name> (sum of the product terms'
    magnitudes, as in layer_backward) and B_<name>, an upper bound of
    layer_backward's M_<name>: the product of the largest magnitudes of the two
    operands over the summed index.
    """
    if spec.fp8:
        raise NotImplementedError("backward of fp8 experts")
    x64 = np.asarray(x, np.float64)
    T, d = x64.shape
    E, k, S, F = spec.n_routed, spec.top_k, spec.n_shared, spec.ffn
    rho = _rho(spec)
    if fwd is None:
        fwd = layer_forward(x, weights, spec, tokens=[])
    dy = np.asarray(dy, np.float64)
    idx, gates, rows = fwd["idx"], fwd["gates"], fwd["row_of_slot"]
    out = {"dx": np.zeros((T, d)), "S_dx": np.zeros((T, d)), "B_dx": np.zeros((T, d))}
    dg = np.zeros((T, k))

    def colmax(m):
        return np.abs(m).max(axis=0) if m.shape[0] else np.zeros(m.shape[1])

    def expert(tok, g, wg, wu, wd):
        X = x64[tok]
        DY = rho(g[:, None] * dy[tok])
        A = X @ wg
        Bv = X @ wu
        Hh = rho(silu(A) * Bv)
        DH = DY @ wd.T
        DA = rho(DH * Bv * dsilu(A))
        DB = rho(DH * silu(A))
        aX, aDA, aDB, aH, aDY = np.abs(X), np.abs(DA), np.abs(DB), np.abs(Hh), np.abs(DY)
        res = {
            "gate": (X.T @ DA, aX.T @ aDA, np.outer(colmax(X), colmax(DA))),
            "up": (X.T @ DB, aX.T @ aDB, np.outer(colmax(X), colmax(DB))),
            "down": (Hh.T @ DY, aH.T @ aDY, np.outer(colmax(Hh), colmax(DY))),
        }
        DX = DA @ wg.T + DB @ wu.T
        SDX = aDA @ np.abs(wg).T + aDB @ np.abs(wu).T
        rmax = np.maximum(aDA.max(axis=1, initial=0.0)[:, None] * np.abs(wg).max(axis=1)[None, :],
                          aDB.max(axis=1, initial=0.0)[:, None] * np.abs(wu).max(axis=1)[None, :])
        out["dx"][tok] += DX
        out["S_dx"][tok] += SDX
        np.maximum(out["B_dx"][tok], rmax, out=rmax)
        out["B_dx"][tok] = rmax
        return Hh @ wd, res

    ex = Experts(weights, spec)

    def put(name, val, sabs, bmax):
        out[name], out["S_" + name], out["B_" + name] = val, sabs, bmax

    def lowrank_expert(tok, g, f):
        """The rank-r expert backward of _lowrank_expert_backward over the
        expert's rows at once; returns its output rows and the gradients with
        their scales."""
        X = x64[tok]
        DY = rho(g[:, None] * dy[tok])
        UG = X @ f["u_gate"]
        ZG = rho(UG * f["s_gate"])
        A = ZG @ f["v_gate"].T
        UU = X @ f["u_up"]
        ZU = rho(UU * f["s_up"])
        Bv = ZU @ f["v_up"].T
        Hh = rho(silu(A) * Bv)
        UD = Hh @ f["u_down"]
        ZD = rho(UD * f["s_down"])
        DZD = DY @ f["v_down"]
        DUD = rho(DZD * f["s_down"])
        DH = DUD @ f["u_down"].T
        DA = rho(DH * Bv * dsilu(A))
        DB = rho(DH * silu(A))
        DZG = DA @ f["v_gate"]
        DZU = DB @ f["v_up"]
        DUG = rho(DZG * f["s_gate"])
        DUU = rho(DZU * f["s_up"])

        def outer_sum(P, Q):       # P^T Q with its scales
            aP, aQ = np.abs(P), np.abs(Q)
            return P.T @ Q, aP.T @ aQ, np.outer(colmax(P), colmax(Q))

        def col_sum(P, Q):         # sum over rows of P * Q, per column
            t = P * Q
            return t.sum(axis=0), np.abs(t).sum(axis=0), (np.abs(t).max(axis=0) if len(t)
                                                          else np.zeros(t.shape[1]))
        res = {"dv_down": outer_sum(DY, ZD), "ds_down": col_sum(DZD, UD),
               "du_down": outer_sum(Hh, DUD), "dv_gate": outer_sum(DA, ZG),
               "dv_up": outer_sum(DB, ZU), "ds_gate": col_sum(DZG, UG),
               "ds_up": col_sum(DZU, UU), "du_gate": outer_sum(X, DUG),
               "du_up": outer_sum(X, DUU)}
        DX = DUG @ f["u_gate"].T + DUU @ f["u_up"].T
        SDX = np.abs(DUG) @ np.abs(f["u_gate"]).T + np.abs(DUU) @ np.abs(f["u_up"]).T
        rmax = np.maximum(
            np.abs(DUG).max(axis=1, initial=0.0)[:, None] * np.abs(f["u_gate"]).max(axis=1)[None, :],
            np.abs(DUU).max(axis=1, initial=0.0)[:, None] * np.abs(f["u_up"]).max(axis=1)[None, :])
        out["dx"][tok] += DX
        out["S_dx"][tok] += SDX
        out["B_dx"][tok] = np.maximum(out["B_dx"][tok], rmax)
        return ZD @ f["v_down"].T, res

    if spec.rank > 0:
        acc = {n: [] for n in LOWRANK_GRADS}
        for e in range(E):
            ts, js = np.nonzero((idx == e) & (rows >= 0))
            f = {n: b[e] for n, b in ex.lr.items()}
            Y, res = lowrank_expert(ts, gates[ts, js], f)
            dg[ts, js] = np.sum(dy[ts] * Y, axis=1)
            for n in LOWRANK_GRADS:
                acc[n].append(res[n])
        for n in LOWRANK_GRADS:
            put(n, *(np.stack([r[i] for r in acc[n]]) for i in range(3)))
    for kind, n in (("w", E if spec.rank == 0 else 0), ("sh", S)):
        if n == 0:
            continue
        acc = {p: [] for p in ("gate", "up", "down")}
        for e in range(n):
            if kind == "w":
                ts, js = np.nonzero((idx == e) & (rows >= 0))
                Y, res = expert(ts, gates[ts, js], ex.gate[e], ex.up[e], ex.down[e])
                dg[ts, js] = np.sum(dy[ts] * Y, axis=1)
            else:
                _, res = expert(np.arange(T), np.ones(T), ex.sh[0][e], ex.sh[1][e], ex.sh[2][e])
            for p in acc:
                acc[p].append(res[p])
        pre = "dw_" if kind == "w" else "dsh_"
        for p, lst in acc.items():
            out[pre + p] = np.stack([r[0] for r in lst])
            out["S_" + pre + p] = np.stack([r[1] for r in lst])
            out["B_" + pre + p] = np.stack([r[2] for r in lst])

    l = router_logits(x, weights["w_router"], weights.get("logit_bias"))
    dl = rho(_router_dl(l, idx, gates, dg, np.asarray(fwd["f"], np.float64), spec, aux_grad, T))
    wr = np.asarray(weights["w_router"], np.float64)
    out["dx"] += dl @ wr.T
    out["S_dx"] += np.abs(dl) @ np.abs(wr).T
    out["B_dx"] = np.maximum(out["B_dx"], np.abs(dl).max(axis=1, initial=0.0)[:, None]
                             * np.abs(wr).max(axis=1)[None, :])
    out["dw_router"] = x64.T @ dl
    out["S_dw_router"] = np.abs(x64).T @ np.abs(dl)
    out["B_dw_router"] = np.outer(colmax(x64), colmax(dl))
    out["dl"], out["dg"] = dl, dg
    return out
