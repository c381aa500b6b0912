"""The parity checks of tests/_parity.py on the CPU: the dense experts' chain
(dense_chain), fed the oracle's own intermediates, passes, and each kind of
planted mistake (a code that is not the quantised h, an h entry outside its
window, a y element off the product of the GPU's h) makes it fail; the
low-rank allowance covers a float32 evaluation of the chain and catches a
systematic slip. The mistakes are planted in copies of the oracle's values;
nothing here runs on a GPU.
"""
import numpy as np
import pytest

import oracle
from fine_grained_mixture_amd import synth
from tests import _parity as P


def _oracle_as_gpu(wl):
    """Outputs shaped like run_gpu's, with the workspace intermediates the
    oracle itself forms (h, its codes and row scales)."""
    inp = synth.make_inputs(wl)
    spec = P.spec_of(wl)
    ref = oracle.layer_forward_batched(inp["x"], inp, spec)
    x = np.asarray(inp["x"], np.float64)
    ex = oracle.Experts(inp, spec)
    rho = oracle.round_bf16
    xq = oracle.fp8_quantize(x, axis=-1)[0] if spec.fp8 else x

    def h_of(X, wg, wu):
        return rho(oracle.silu(X @ wg) * (X @ wu))

    def codes(h):
        if not spec.fp8:
            return None, None
        q, s = oracle.fp8_quantize(h, axis=-1)
        return np.ldexp(q, -s[:, None]), np.ldexp(1.0, s)

    T, R, F, S = wl.T, int(ref["offsets"][-1]), wl.ffn, wl.n_shared
    ws = {}
    if wl.rank == 0:
        h = np.zeros((R, F))
        for e in range(wl.n_routed):
            a, b = int(ref["offsets"][e]), int(ref["offsets"][e + 1])
            if a < b:
                h[a:b] = h_of(xq[ref["sorted_token"][a:b]], ex.gate[e], ex.up[e])
        ws["h"] = h
        ws["hq"], ws["hs"] = codes(h)
    if S:
        ws["h_sh"] = np.concatenate([h_of(xq, ex.sh[0][s], ex.sh[1][s]) for s in range(S)], axis=-1)
        ws["hq_sh"], ws["hs_sh"] = codes(ws["h_sh"])
    g = dict(sorted_token=ref["sorted_token"], ws=ws)
    return inp, spec, ref, g


@pytest.mark.parametrize("S,rank,dtype", [(0, 0, "fp8"), (1, 0, "fp8"), (2, 0, "fp8"),
                                          (2, 64, "fp8"), (0, 0, "bf16"), (2, 0, "bf16"),
                                          (1, 64, "bf16")])
def test_chain_accepts_the_oracle_and_rejects_planted_mistakes(S, rank, dtype):
    wl = synth.QUARTZ.replace(T=40, hidden=128, ffn=64, n_shared=S, dtype=dtype, seed=S,
                              rank=rank)
    inp, spec, ref, g = _oracle_as_gpu(wl)
    y = ref["y"]
    rms = float(np.sqrt(np.mean(y ** 2)))
    r_lr = P.lowrank_zd_allowance(inp, spec, ref) if rank else None
    rep = P.dense_chain(inp, spec, ref, g, y, rms, r_lr)
    assert rep["y_rel_to_gpu_h"] < 1e-12 and rep.get("codes_moved", 0) == 0
    assert rep["h_window_ratio"] == 0.0

    def fails(mutate):
        g2 = dict(g, ws={k: None if v is None else v.copy() for k, v in g["ws"].items()})
        y2 = y.copy()
        mutate(g2["ws"], y2)
        with pytest.raises(AssertionError):
            P.dense_chain(inp, spec, ref, g2, y2, rms, r_lr)

    hk, qk, sk = ("h", "hq", "hs") if rank == 0 else ("h_sh", "hq_sh", "hs_sh")

    def bump_code(ws, y2):            # a code one E4M3 step off its h
        r = 3
        f = int(np.argmax(np.abs(ws[qk][r])))
        ws[qk][r, f] = oracle.e4m3_round(ws[qk][r, f] * (1 - 2.0 ** -3))

    def move_h(ws, y2):               # h (and its codes) 20% off the oracle's
        ws[hk][5] = oracle.round_bf16(ws[hk][5] * 1.2)
        if spec.fp8:
            q, s = oracle.fp8_quantize(ws[hk][5:6], axis=-1)
            ws[qk][5], ws[sk][5] = np.ldexp(q, -s[:, None])[0], np.ldexp(1.0, s)[0]

    def bump_y(ws, y2):               # one output element 2e-2 RMS off
        y2[7, 11] += 2e-2 * rms

    for m in ((bump_code, move_h, bump_y) if spec.fp8 else (move_h, bump_y)):
        fails(m)
    if S and rank == 0 and spec.fp8:
        def bump_shared_scale(ws, y2):   # the shared row's scale doubled
            ws["hs_sh"][2] *= 2.0
        fails(bump_shared_scale)


def _float32_lowrank_y(inp, spec, ref):
    """The low-rank layer evaluated in float32 (NumPy's float32 products: fp32
    sums in an order of their own), rounded to bf16 at the layer's points."""
    ex = oracle.Experts(inp, spec)
    x = np.asarray(inp["x"], np.float32)

    def r32(v):
        return oracle.round_bf16(v.astype(np.float64)).astype(np.float32)

    def apply(v, u, s, vmat):
        return r32((v @ u) * s) @ vmat.T

    y = np.zeros(x.shape)
    idx, gates, rows = ref["idx"], ref["gates"], ref["row_of_slot"]
    for e in range(spec.n_routed):
        ts, js = np.nonzero((idx == e) & (rows >= 0))
        if not len(ts):
            continue
        f = {n: np.asarray(b[e], np.float32) for n, b in ex.lr.items()}
        a = apply(x[ts], f["u_gate"], f["s_gate"], f["v_gate"])
        b = apply(x[ts], f["u_up"], f["s_up"], f["v_up"])
        h = r32(a / (1 + np.exp(-a)) * b)
        np.add.at(y, ts, gates[ts, js][:, None] * apply(h, f["u_down"], f["s_down"], f["v_down"]))
    return y


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_lowrank_allowance_covers_a_float32_chain_and_catches_a_slip(dtype):
    """A float32 evaluation of the low-rank chain (another summation order,
    tipping rounding decisions all along the chain) meets the low-rank
    acceptance against the oracle; the same evaluation with s_down off by
    2^-6 (a systematic slip) fails it."""
    wl = synth.DORMOUSE.replace(T=1500, dtype=dtype, seed=5)
    inp = synth.make_inputs(wl)
    spec = P.spec_of(wl)
    ref = oracle.layer_forward_batched(inp["x"], inp, spec)
    y = ref["y"]
    rms = np.sqrt(np.mean(y ** 2))
    r_y = P.lowrank_zd_allowance(inp, spec, ref)
    y32 = _float32_lowrank_y(inp, spec, ref)
    dev = np.abs(y32 - y)
    assert np.count_nonzero(dev) > 0.1 * dev.size          # the orders differ
    assert np.max(dev / (P.Y_TOL * rms + r_y)) <= 0.5
    assert np.sqrt(np.mean(dev ** 2)) / rms <= 0.5 * P.LOWRANK_ERR_RMS
    bad = dict(inp)
    bad["s_down"] = (np.asarray(inp["s_down"], np.float64) * (1 + 2.0 ** -6)).astype(np.float32)
    dev = np.abs(_float32_lowrank_y(bad, spec, ref) - y)
    assert np.sqrt(np.mean(dev ** 2)) / rms > P.LOWRANK_ERR_RMS


def _emulate_lowrank_backward(inp, spec, ref, dy, dl, s_gate_scale=1.0, dsilu=None):
    """A GPU-like evaluation of the rank-r experts' backward on the CPU: the
    forward chain recomputed and the chain rule back through it, products in
    float32 (NumPy's own summation order), bf16 rounding at the layer's
    points, laid out as the GPU leaves it: the forward's routing (fwd), the
    gradients (g) and the backward workspace's intermediates (I, rows in
    expert-sorted order). dl is the router-logit gradient taken as given.
    s_gate_scale and dsilu plant mistakes."""
    f32 = np.float32
    ex = oracle.Experts(inp, spec)

    def r32(v):
        return oracle.round_bf16(np.asarray(v, np.float64)).astype(f32)

    x = np.asarray(inp["x"], f32)
    dy = np.asarray(dy, f32)
    T, d = x.shape
    E, F, r, k = spec.n_routed, spec.ffn, spec.rank, spec.top_k
    offs = np.asarray(ref["offsets"][:E + 1], np.int64)
    R = int(offs[-1])
    rows = np.asarray(ref["row_of_slot"], np.int64)
    tok = np.zeros(R, np.int64)
    slot = np.zeros(R, np.int64)
    ts, js = np.nonzero(rows >= 0)
    tok[rows[ts, js]], slot[rows[ts, js]] = ts, js
    gate32 = np.asarray(ref["gates"], f32)
    shapes = dict(dy=d, xperm=d, dab=2 * F, ug=r, uu=r, zgu=2 * r, ab=2 * F, h=F, ud=r, zd=r,
                  dzd=r, dud=r, dzg=r, dzu=r, dugu=2 * r)
    I = {n: np.zeros((R, w), f32) for n, w in shapes.items()}
    g = {n: np.zeros((E,) + np.shape(ex.lr[n[1:]][0]), f32) for n in oracle.LOWRANK_GRADS}
    dxe = np.zeros((R, d), f32)
    for e in range(E):
        a, b = int(offs[e]), int(offs[e + 1])
        if a == b:
            continue
        f = {n: np.asarray(bk[e], f32) for n, bk in ex.lr.items()}
        sg = (f["s_gate"] * f32(s_gate_scale)).astype(f32)
        X = x[tok[a:b]]
        UG, UU = X @ f["u_gate"], X @ f["u_up"]
        ZG, ZU = r32(UG * sg), r32(UU * f["s_up"])
        A, B = ZG @ f["v_gate"].T, ZU @ f["v_up"].T
        sgm = f32(1) / (f32(1) + np.exp(-A))
        H = r32(A * sgm * B)
        UD = H @ f["u_down"]
        ZD = r32(UD * f["s_down"])
        DY = r32(gate32[tok[a:b], slot[a:b]][:, None] * dy[tok[a:b]])
        DZD = DY @ f["v_down"]
        DUD = r32(DZD * f["s_down"])
        DH = DUD @ f["u_down"].T
        dsA = sgm * (f32(1) + A * (f32(1) - sgm)) if dsilu is None else dsilu(A)
        DA, DB = r32(DH * B * dsA), r32(DH * (A * sgm))
        DZG, DZU = DA @ f["v_gate"], DB @ f["v_up"]
        DUG, DUU = r32(DZG * sg), r32(DZU * f["s_up"])
        for n, v in (("dy", DY), ("xperm", X), ("dab", np.concatenate([DA, DB], 1)),
                     ("ug", UG), ("uu", UU), ("zgu", np.concatenate([ZG, ZU], 1)),
                     ("ab", np.concatenate([A, B], 1)), ("h", H), ("ud", UD), ("zd", ZD),
                     ("dzd", DZD), ("dud", DUD), ("dzg", DZG), ("dzu", DZU),
                     ("dugu", np.concatenate([DUG, DUU], 1))):
            I[n][a:b] = v
        g["dv_down"][e], g["du_down"][e] = DY.T @ ZD, H.T @ DUD
        g["dv_gate"][e], g["dv_up"][e] = DA.T @ ZG, DB.T @ ZU
        g["du_gate"][e], g["du_up"][e] = X.T @ DUG, X.T @ DUU
        g["ds_gate"][e] = (DZG * UG).sum(axis=0)
        g["ds_up"][e] = (DZU * UU).sum(axis=0)
        g["ds_down"][e] = (DZD * UD).sum(axis=0)
        dxe[a:b] = DUG @ f["u_gate"].T + DUU @ f["u_up"].T
    dl32 = np.asarray(dl, f32)
    dx = dl32 @ np.asarray(inp["w_router"], f32).T
    for j in range(k):
        m = rows[:, j] >= 0
        dx[m] += dxe[rows[m, j]]
    S = spec.n_shared
    if S:
        # dense shared experts over all tokens, as the GPU runs them
        dysh = r32(dy)
        dab_sh = np.zeros((T, S * 2 * F), f32)
        h_sh = np.zeros((T, S * F), f32)
        for n in ("dsh_gate", "dsh_up", "dsh_down"):
            g[n] = np.zeros((S, F, d) if n == "dsh_down" else (S, d, F), f32)
        for e in range(S):
            wg, wu, wd = (np.asarray(ex.sh[i][e], f32) for i in range(3))
            A, B = x @ wg, x @ wu
            sgm = f32(1) / (f32(1) + np.exp(-A))
            h_sh[:, e * F:(e + 1) * F] = r32(A * sgm * B)
            dh = dysh @ wd.T
            DA = r32(dh * B * (sgm * (f32(1) + A * (f32(1) - sgm))))
            DB = r32(dh * (A * sgm))
            dab_sh[:, e * 2 * F:e * 2 * F + F], dab_sh[:, e * 2 * F + F:(e + 1) * 2 * F] = DA, DB
            dx += DA @ wg.T + DB @ wu.T
            g["dsh_down"][e] = h_sh[:, e * F:(e + 1) * F].T @ dysh
            g["dsh_gate"][e], g["dsh_up"][e] = x.T @ DA, x.T @ DB
        I["dab_sh"], I["h_sh"] = dab_sh, h_sh
    g["dx"], g["dw_router"] = dx, x.T @ dl32
    I = {n: v.astype(np.float64) for n, v in I.items()}
    I["dl"] = dl32.astype(np.float64)
    fwd = dict(offsets=offs, row_of_slot=rows, sorted_token=np.asarray(ref["sorted_token"]),
               topk_gate=gate32)
    return fwd, g, I


def _lowrank_bwd_case():
    wl = synth.DORMOUSE.replace(T=1500, hidden=384, ffn=256, seed=5)
    inp = synth.make_inputs(wl)
    dy = synth.make_upstream(wl)
    spec = P.spec_of(wl)
    ref = oracle.layer_forward(inp["x"], inp, spec, tokens=[])
    orc = oracle.layer_backward_batched(inp["x"], inp, spec, dy, aux_grad=1.0, fwd=ref)
    return inp, spec, dy, ref, orc


def test_lowrank_backward_check_accepts_a_float32_chain_and_rejects_planted_mistakes():
    """A float32 evaluation of the rank-r backward, laid out as the GPU leaves
    it, passes lowrank_backward_check (its fp32 sums tip bf16 roundings all
    along the chain, which the oracle comparison tolerates); each planted
    mistake fails it: an intermediate two ulps off its rounding, one gradient
    element 2^-10 off its sum, a SwiGLU derivative that drops a term, s_gate
    2^-6 off, two x rows swapped, a router-logit gradient entry changed after
    use, the router's share of dx left out."""
    inp, spec, dy, ref, orc = _lowrank_bwd_case()
    fwd, g, I = _emulate_lowrank_backward(inp, spec, ref, dy, orc["dl"])
    rep = P.lowrank_backward_check(inp, spec, dy, fwd, g, I, orc)
    print(rep)
    assert sum(rep["tipped"].values()) > 0                 # the orders differ

    def fails(fwd2, g2, I2, what):
        with pytest.raises(AssertionError):
            P.lowrank_backward_check(inp, spec, dy, fwd2, g2, I2, orc)

    r = spec.rank
    I2 = {n: v.copy() for n, v in I.items()}
    i = int(np.argmax(np.abs(I2["dugu"][:, 3])))
    v = I2["dugu"][i, 3]
    I2["dugu"][i, 3] = v + 2 * np.ldexp(1.0, int(np.frexp(abs(v))[1]) - 8) * np.sign(v)
    fails(fwd, g, I2, "dug two ulps off")
    g2 = {n: v.copy() for n, v in g.items()}
    e = int(np.argmax(np.diff(fwd["offsets"])))
    g2["du_gate"][e, 5, 7] *= 1 + 2.0 ** -10
    fails(fwd, g2, I, "du_gate element")
    fails(*_emulate_lowrank_backward(inp, spec, ref, dy, orc["dl"],
                                     dsilu=lambda A: 1 / (1 + np.exp(-A))), "dsilu")
    fails(*_emulate_lowrank_backward(inp, spec, ref, dy, orc["dl"], s_gate_scale=1 + 2.0 ** -6),
          "s_gate")
    I2 = {n: v.copy() for n, v in I.items()}
    I2["xperm"][[0, 1]] = I2["xperm"][[1, 0]]
    fails(fwd, g, I2, "x rows")
    I2 = {n: v.copy() for n, v in I.items()}
    t = int(np.argmax(np.abs(I2["dl"]).max(axis=1)))
    I2["dl"][t] *= 1.5
    fails(fwd, g, I2, "dl")
    g2 = {n: v.copy() for n, v in g.items()}
    g2["dx"] = g2["dx"] - (np.asarray(orc["dl"], np.float32) @
                           np.asarray(inp["w_router"], np.float32).T)
    fails(fwd, g2, I, "router share of dx")
    assert r == 64


def test_lowrank_backward_check_covers_shared_experts():
    """With dense shared experts beside the rank-r ones, the float32
    evaluation still passes the check, and mistakes planted in the shared
    part fail it: a shared da entry two ulps off its rounding, a shared down
    gradient element 2^-10 off its sum, the shared experts' share of dx left
    out."""
    wl = synth.DORMOUSE.replace(T=700, hidden=192, ffn=128, rank=32, n_routed=64, n_shared=2,
                                renorm=1, seed=22)
    inp = synth.make_inputs(wl)
    dy = synth.make_upstream(wl)
    spec = P.spec_of(wl)
    ref = oracle.layer_forward(inp["x"], inp, spec, tokens=[])
    orc = oracle.layer_backward_batched(inp["x"], inp, spec, dy, aux_grad=1.0, fwd=ref)
    fwd, g, I = _emulate_lowrank_backward(inp, spec, ref, dy, orc["dl"])
    rep = P.lowrank_backward_check(inp, spec, dy, fwd, g, I, orc)
    assert "da_shared1" in rep["tipped"] and "dsh_down[1]" in rep["worst_sum"]

    def fails(g2, I2):
        with pytest.raises(AssertionError):
            P.lowrank_backward_check(inp, spec, dy, fwd, g2, I2, orc)

    I2 = {n: v.copy() for n, v in I.items()}
    t, c = np.unravel_index(int(np.argmax(np.abs(I2["dab_sh"][:, 5:6]))), (wl.T, 1))
    v = I2["dab_sh"][t, 5]
    I2["dab_sh"][t, 5] = v + 2 * np.ldexp(1.0, int(np.frexp(abs(v))[1]) - 8) * np.sign(v)
    fails(g, I2)
    g2 = {n: v.copy() for n, v in g.items()}
    g2["dsh_down"][1, 3, 4] *= 1 + 2.0 ** -10
    fails(g2, I)
    g2 = {n: v.copy() for n, v in g.items()}
    F = wl.ffn
    for e in range(wl.n_shared):
        wg, wu = (np.asarray(oracle.Experts(inp, spec).sh[i][e], np.float32) for i in range(2))
        g2["dx"] = g2["dx"] - (I["dab_sh"][:, e * 2 * F:e * 2 * F + F].astype(np.float32) @ wg.T +
                               I["dab_sh"][:, e * 2 * F + F:(e + 1) * 2 * F].astype(np.float32)
                               @ wu.T)
    fails(g2, I)
