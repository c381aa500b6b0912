"""GPU-vs-oracle parity helpers (test infrastructure).

Acceptance (what the layer must reproduce, per token whose k-th vs (k+1)-th
key margin exceeds 1e-4 in the oracle):
  * selected expert sets, per-expert counts, kept counts, offsets,
    sorted_token, the (token, expert) -> row map, drop flags and n_dropped:
    bit-exact, after the oracle is re-run with near-tie tokens forced to the
    GPU's selection (either choice is correct for them); sorted_token rows at
    and past offsets[E] keep the caller's fill;
  * gates within 1e-5 absolute, aux within 1e-4 relative;
  * max |y_gpu - y_oracle| <= 1e-2 * RMS(y_oracle) over every element of y
    (all T tokens; the oracle's per-expert batched form at full size);
  * low-rank experts, whose chain has four bf16 rounding points (z_g, z_u, h,
    z_d): per element 1e-2 * RMS(y_oracle) plus one bf16 ulp of every entry
    of the last rounding point z_d carried through |V_d| and the gate
    (lowrank_zd_allowance), and the error's RMS over all of y at most
    1e-3 RMS(y_oracle);
  * bf16 and fp8 layers with dense experts, from the GPU's own
    intermediates (read from the workspace): its h is within one bf16 ulp
    plus its products' fp32 window of the oracle's h, per entry; fp8: its
    E4M3 codes are the oracle's quantisation of its own h, exactly; y is
    within 1e-2 RMS of the oracle's down projections and combine of the GPU's
    h (or codes), everywhere; and y against the oracle's y is within 1e-2 RMS
    plus exactly what the two sides' h differ by, carried through |W_down|
    (dense_chain). An h rounding decision taken differently by the two
    summation orders (h has heavy tails, so one ulp at a large entry can
    move an output by a percent of RMS(y)) is thus accounted for exactly, at
    any batch size.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from fine_grained_mixture_amd.layer import (DeviceWeights, allocate_outputs, allocate_workspace,
                                            config_from_workload)
from fine_grained_mixture_amd import _lib
from fine_grained_mixture_amd import layer as L

NEAR_TIE = 1e-4
Y_TOL = 1e-2
GATE_TOL = 1e-5
AUX_RTOL = 1e-4
# bound on |gpu - exact| of one fp8 gate/up product entry, relative to the sum
# of its terms' magnitudes (fp8 MFMA with fp32 sums; about 1e-4 measured)
FP8_PRODUCT_REL = 2.0 ** -10
# the same for a bf16 MFMA product with fp32 sums over K <= 4096 terms: at most
# K/16 + 16 fp32 roundings of partial sums, each <= 2^-24 of the running sum's
# terms (<= 2^-16 for K = 4096); four times that
BF16_PRODUCT_REL = 2.0 ** -14
# low-rank experts: largest RMS of (gpu - oracle) over all of y, relative to
# RMS(y) (a float32 evaluation of the chain on the CPU gives 1.8e-4 at the
# Dormouse widths)
LOWRANK_ERR_RMS = 1e-3


def spec_of(wl) -> oracle.LayerSpec:
    return oracle.LayerSpec(hidden=wl.hidden, n_routed=wl.n_routed, top_k=wl.top_k,
                            n_shared=wl.n_shared, ffn=wl.ffn, rank=wl.rank, score=wl.score,
                            renorm=bool(wl.renorm), capacity=wl.capacity,
                            aux_coef=wl.aux_coef, bf16=wl.dtype in ("bf16", "fp8"),
                            fp8=wl.dtype == "fp8")


def upload(wl, inp, device="cuda"):
    cfg = config_from_workload(wl)
    dt = torch.bfloat16 if wl.dtype in ("bf16", "fp8") else torch.float32
    x = torch.from_numpy(inp["x"]).to(device=device, dtype=dt)
    w = DeviceWeights.from_numpy(inp, cfg, device)
    return cfg, x, w


def to_numpy(out) -> dict:
    res = {}
    for k, v in out.t.items():
        if v is not None:
            if v.dtype == torch.bfloat16:
                v = v.float()
            res[k] = v.cpu().numpy()
    return res


def workspace_intermediates(cfg, T, ws, rows) -> dict:
    """The layer's h (and for fp8 its E4M3 codes and row scales), read from
    the workspace after a call (regions from moe_workspace_region), as numpy;
    routed regions up to the `rows` dispatched rows."""
    R, F, S = _lib.moe_max_rows(cfg, T), cfg.ffn, cfg.n_shared

    def region(which, dtype, shape):
        off, n = _lib.moe_workspace_region(cfg, T, which)
        if n == 0:
            return None
        t = ws[off:off + n].view(dtype).reshape(shape)
        if shape[0] == R:
            t = t[:rows]
        if dtype == torch.bfloat16:
            t = t.float()
        if dtype == torch.uint8:
            t = t.view(torch.float8_e4m3fn).to(torch.float32)
        return t.cpu().numpy().astype(np.float64)

    return dict(h=region(_lib.MOE_WS_H, torch.bfloat16, (R, F)),
                h_sh=region(_lib.MOE_WS_H_SHARED, torch.bfloat16, (T, S * F)),
                hq=region(_lib.MOE_WS_HQ, torch.uint8, (R, F)),
                hs=region(_lib.MOE_WS_HQ_SCALE, torch.float32, (R,)),
                hq_sh=region(_lib.MOE_WS_HQ_SHARED, torch.uint8, (T, S * F)),
                hs_sh=region(_lib.MOE_WS_HQ_SHARED_SCALE, torch.float32, (T,)))


def run_gpu(wl, inp, *, y_lowp=False, intermediates=True):
    cfg, x, w = upload(wl, inp)
    out = allocate_outputs(cfg, wl.T, x.device, y_lowp=y_lowp)
    ws = allocate_workspace(cfg, wl.T, x.device)
    L.layer_forward(cfg, x, w, out, ws)
    torch.cuda.synchronize()
    res = to_numpy(out)
    return with_intermediates(wl, cfg, res, ws) if intermediates else res


def with_intermediates(wl, cfg, res: dict, ws) -> dict:
    """Adds the workspace intermediates that check_parity's chain check reads
    (bf16 or fp8 layers with dense experts, routed or shared)."""
    if wl.dtype in ("bf16", "fp8") and (wl.rank == 0 or wl.n_shared > 0) and wl.T > 0:
        res["ws"] = workspace_intermediates(cfg, wl.T, ws, int(res["offsets"][-1]))
    return res


def slot_map(idx, rows):
    """(token, expert) -> row (or -1)."""
    T, k = idx.shape
    return {(t, int(idx[t, j])): int(rows[t, j]) for t in range(T) for j in range(k)}


def check_parity(wl, inp, g, *, check_y=True, no_rho=True):
    """Compare GPU outputs g (numpy dict) with the oracle on every token and
    every element of y. Returns a report. ``no_rho`` also reports (not gated)
    the error against the oracle without bf16 rounding points."""
    spec = spec_of(wl)
    T, k = wl.T, wl.top_k
    r0 = oracle.route(inp["x"], inp["w_router"], spec, inp.get("logit_bias"),
                      inp.get("select_bias"))
    near = r0["margin"] <= NEAR_TIE
    gi = g["topk_idx"].astype(np.int64)
    assert gi.shape == (T, k)
    assert np.all((gi >= 0) & (gi < wl.n_routed))
    # every token's selection holds k distinct experts
    assert np.all(np.diff(np.sort(gi, 1), axis=1) > 0) if k > 1 else True
    same = np.all(np.sort(gi, 1) == np.sort(r0["idx"], 1), axis=1)
    bad = ~same & ~near
    assert not bad.any(), (f"{int(bad.sum())} tokens with margin > {NEAR_TIE} select different "
                           f"experts, e.g. token {int(np.nonzero(bad)[0][0])}")
    # the in-list order follows the key, unless two selected keys are within the tie margin
    srt = np.take_along_axis(r0["key"], r0["idx"], 1)
    close = np.any(np.abs(np.diff(srt, axis=1)) <= NEAR_TIE, axis=1) if k > 1 else np.zeros(T, bool)
    chk = ~near & ~close
    assert np.array_equal(gi[chk], r0["idx"][chk])

    # oracle with the near-tie tokens forced to the GPU's choice
    ov = near & ~same
    if check_y:
        ref = oracle.layer_forward_batched(inp["x"], inp, spec, override_idx=gi, override_mask=ov)
    else:
        ref = oracle.layer_forward(inp["x"], inp, spec, tokens=[], override_idx=gi,
                                   override_mask=ov)
    for key in ("counts", "kept", "offsets"):
        np.testing.assert_array_equal(g[key], ref[key], err_msg=key)
    assert int(g["n_dropped"][0]) == ref["n_dropped"]
    R = int(ref["offsets"][-1])
    np.testing.assert_array_equal(g["sorted_token"][:R], ref["sorted_token"], err_msg="sorted_token")
    # rows past the routed total are not the layer's: they keep the caller's fill (-1)
    assert np.all(g["sorted_token"][R:] == -1), "sorted_token written past offsets[E]"
    assert slot_map(gi, g["row_of_slot"]) == slot_map(ref["idx"], ref["row_of_slot"])
    if "dropped" in g:
        gd = {(t, int(gi[t, j])): bool(g["dropped"][t, j]) for t in range(T) for j in range(k)}
        rd = {(t, int(ref["idx"][t, j])): bool(ref["dropped"][t, j]) for t in range(T) for j in range(k)}
        assert gd == rd
    # gates per (token, expert)
    gg = {(t, int(gi[t, j])): float(g["topk_gate"][t, j]) for t in range(T) for j in range(k)}
    rg = {(t, int(ref["idx"][t, j])): float(ref["gates"][t, j]) for t in range(T) for j in range(k)}
    gate_err = max(abs(gg[key] - rg[key]) for key in rg) if rg else 0.0
    assert gate_err <= GATE_TOL, gate_err
    aux_rel = abs(float(g["aux"][0]) - ref["aux_raw"]) / max(abs(ref["aux_raw"]), 1e-30)
    assert aux_rel <= AUX_RTOL, aux_rel
    assert abs(float(g["aux"][1]) - ref["aux"]) <= AUX_RTOL * abs(ref["aux"]) + 1e-12
    if "f" in g:
        np.testing.assert_allclose(g["f"], ref["f"], rtol=1e-6, atol=1e-9)
        np.testing.assert_allclose(g["P"], ref["P"], rtol=1e-4, atol=1e-7)
    if "topk_margin" in g and k < wl.n_routed:
        m_err = np.max(np.abs(g["topk_margin"][~near] - r0["margin"][~near])) if (~near).any() else 0
        assert m_err <= 1e-4, m_err
    rep = dict(near_ties=int(near.sum()), forced=int(ov.sum()), gate_err=gate_err,
               aux_rel=aux_rel, rows=R, n_dropped=ref["n_dropped"])
    if not check_y:
        return rep
    yg = g["y"].astype(np.float64)
    yr = ref["y"]
    assert yg.shape == yr.shape == (T, wl.hidden)
    assert np.all(np.isfinite(yg))
    rms = float(np.sqrt(np.mean(yr ** 2))) if T else 0.0
    diff = np.abs(yg - yr)
    err = float(diff.max()) if T else 0.0
    rep.update(y_err=err, y_rms=rms, y_rel=err / rms if rms else 0.0, checked=T)
    # low-rank experts: bf16 rounding points z_g, z_u, h, z_d in a chain
    r_y = lowrank_zd_allowance(inp, spec, ref) if spec.rank > 0 and spec.bf16 and T else None
    if spec.bf16 and (spec.rank == 0 or spec.n_shared > 0) and T:
        rep.update(dense_chain(inp, spec, ref, g, yg, rms, r_y))
    elif r_y is not None:
        # the error's RMS over all elements stays at accumulation-order level
        err_rms = float(np.sqrt(np.mean(diff ** 2))) / rms if rms else 0.0
        rep.update(y_err_rms_rel=err_rms,
                   elements_beyond_rms_bound=int(np.count_nonzero(diff > Y_TOL * rms)))
        assert err_rms <= LOWRANK_ERR_RMS, f"error RMS {err_rms:.2e} of RMS(y)"
        ratio = float(np.max(diff / (Y_TOL * rms + r_y)))
        rep.update(y_tol_ratio=ratio)
        assert ratio <= 1.0, (f"max |dy| / (1e-2 RMS + z_d ulps) = {ratio:.3f} at "
                              f"{np.unravel_index(np.argmax(diff / (Y_TOL * rms + r_y)), diff.shape)}")
    else:
        assert err <= Y_TOL * rms, f"max|dy| {err:.3e} > {Y_TOL} * RMS {rms:.3e}"
    if no_rho and spec.bf16 and not spec.fp8 and T:
        # informative: against float64 with no bf16 rounding point at all
        import dataclasses
        y0 = oracle.layer_forward_batched(inp["x"], inp, dataclasses.replace(spec, bf16=False),
                                          override_idx=gi, override_mask=ov)["y"]
        rms0 = float(np.sqrt(np.mean(y0 ** 2)))
        rep.update(y_rel_no_rho=float(np.max(np.abs(yg - y0))) / rms0 if rms0 else 0.0)
    return rep


def lowrank_zd_allowance(inp, spec, ref):
    """Per element of y, one bf16 ulp of every entry of z_d = rho((h U_d) s_d)
    of the token's low-rank experts, carried to the output by |V_d| and the
    gate: sum_j g_j sum_i ulp(z_d[i]) |V_d[c, i]|.

    z_d is the chain's last rounding point, one product before the output.
    Its unrounded value is a sum over all F entries of h, each itself rounded
    after two rounded rank-r intermediates, so a different fp32 summation
    order upstream tips some of its rounding decisions (a float32 evaluation
    of the chain on the CPU tips several per row); each tipped decision moves
    the output row by one ulp of that entry times the V_d row."""
    x = np.asarray(inp["x"], np.float64)
    T, d = x.shape
    ex = oracle.Experts(inp, spec)
    rho = oracle.round_bf16
    out = np.zeros((T, d))
    idx, gates, rows = ref["idx"], ref["gates"], ref["row_of_slot"]
    for e in range(spec.n_routed):
        ts, js = np.nonzero((idx == e) & (rows >= 0))
        if not len(ts):
            continue
        f = {n: b[e] for n, b in ex.lr.items()}
        X = x[ts]
        a = oracle.lowrank_apply(X, f["u_gate"], f["s_gate"], f["v_gate"], rho)
        b = oracle.lowrank_apply(X, f["u_up"], f["s_up"], f["v_up"], rho)
        h = rho(oracle.silu(a) * b)
        zd = rho((h @ f["u_down"]) * f["s_down"])
        _, ex2 = np.frexp(zd)                        # |zd| in [2^(ex2-1), 2^ex2)
        ulp = np.where(zd != 0, np.ldexp(1.0, ex2 - 8), 0.0)
        np.add.at(out, ts, gates[ts, js][:, None] * (ulp @ np.abs(f["v_down"]).T))
    return out


def _worst(diff, tol, what):
    """Message naming the worst elements of diff / tol."""
    r = diff / tol
    flat = np.argsort(r, axis=None)[::-1][:3]
    parts = [f"{what}: max ratio {float(r.max()):.3f}"]
    for f in flat:
        t, c = np.unravel_index(f, r.shape)
        parts.append(f"(token {t}, col {c}: |d| {diff[t, c]:.3e}, tol {tol[t, c]:.3e})")
    return " ".join(parts)


def dense_chain(inp, spec, ref, g, yg, rms, r_lowrank=None):
    """Dense experts of a bf16 or fp8 layer (routed, or the shared experts
    beside low-rank routed ones), checked link by link on every element from
    the GPU's own intermediates (read from the workspace):

      1. its h is the oracle's rho(SiLU(a) b), per entry within one bf16 ulp
         plus what the gate and up products' fp32 sums can move it
         (BF16_PRODUCT_REL, or FP8_PRODUCT_REL for the fp8 MFMA, of the sum of
         their terms' magnitudes, first and second order through SiLU(a) b);
      2. fp8: its E4M3 codes and row scales are the oracle's quantisation of
         its own h, exactly (routed rows; the shared experts' S F rows);
      3. y is the oracle's down projections and gate-weighted combine of the
         GPU's own h (or codes), in float64, within 1e-2 RMS(y) everywhere;
      4. y against the oracle's own y: within 1e-2 RMS(y) plus exactly what
         the two sides' h (or codes) differ by, carried through |W_down| and
         the gates (sum_f |dh_f| |W_down[f, c]|).

    A bf16 rounding decision of h that the two summation orders take
    differently (one ulp at an entry that may be large: h has heavy tails),
    or the E4M3 code step it can cause, is thus accounted for exactly, at any
    batch size. Low-rank routed experts enter with the oracle's own rows and
    the allowance ``r_lowrank``."""
    w = g["ws"]
    x = np.asarray(inp["x"], np.float64)
    T, d = x.shape
    F, S, E, k = spec.ffn, spec.n_shared, spec.n_routed, spec.top_k
    ex = oracle.Experts(inp, spec)
    rho = oracle.round_bf16
    xa = oracle.fp8_quantize(x, axis=-1)[0] if spec.fp8 else x
    axa = np.abs(xa)
    eps = FP8_PRODUCT_REL if spec.fp8 else BF16_PRODUCT_REL
    offs = ref["offsets"]
    R = int(offs[-1])
    rep = {}

    def h_window(X, aX, wg, wu):
        A, Bv = X @ wg, X @ wu
        ea = eps * (aX @ np.abs(wg))
        eb = eps * (aX @ np.abs(wu))
        sa = oracle.silu(A)
        H = rho(sa * Bv)
        # one bf16 ulp (at most 2^-7 of |h|), the first-order move, and the
        # second-order terms (|SiLU'| < 1.1, |SiLU''| <= 1/2)
        tol = (2.0 ** -7 * np.abs(H) + np.abs(oracle.dsilu(A)) * ea * np.abs(Bv)
               + np.abs(sa) * eb + 1.1 * ea * eb + 0.5 * ea ** 2 * np.abs(Bv) + 2.0 ** -133)
        return H, tol

    stats = dict(worst_h=0.0, h_moved=0, h_n=0, code_moved=0)

    def check_rows(h_gpu, hq_gpu, hs_gpu, H_or, tol, what):
        dev = np.abs(h_gpu - H_or)
        r = float(np.max(dev / tol)) if dev.size else 0.0
        assert r <= 1.0, f"{what}: h beyond its window ({r:.2f})"
        stats["worst_h"] = max(stats["worst_h"], r)
        stats["h_moved"] += int(np.count_nonzero(dev))
        stats["h_n"] += dev.size
        if not spec.fp8:
            return h_gpu, H_or
        codes = hq_gpu * hs_gpu[:, None]
        want = oracle.fp8_quantize(h_gpu, axis=-1)[0]
        assert np.array_equal(codes, want), f"{what}: codes are not the quantised h"
        c_or = oracle.fp8_quantize(H_or, axis=-1)[0]
        stats["code_moved"] += int(np.count_nonzero(codes != c_or))
        return codes, c_or

    y_codes = np.zeros((T, d))
    b_y = np.zeros((T, d))       # |h_gpu - h_oracle| carried to y
    if S > 0:
        parts = [h_window(xa, axa, ex.sh[0][s], ex.sh[1][s]) for s in range(S)]
        H_or = np.concatenate([p[0] for p in parts], axis=-1)
        tol = np.concatenate([p[1] for p in parts], axis=-1)
        c, c_or = check_rows(w["h_sh"], w.get("hq_sh"), w.get("hs_sh"), H_or, tol, "shared")
        wd = ex.sh_down if spec.fp8 else np.concatenate([ex.sh[2][s] for s in range(S)], axis=0)
        y_codes = y_codes + c @ wd
        b_y += np.abs(c - c_or) @ np.abs(wd)
    yr = np.zeros((R, d))
    br = np.zeros((R, d))
    st = g["sorted_token"][:R].astype(np.int64)
    for e in range(E):
        a, b = int(offs[e]), int(offs[e + 1])
        if a == b:
            continue
        toks = st[a:b]
        if spec.rank > 0:
            # low-rank experts: their rows are the oracle's own
            yr[a:b] = ex.routed(x[toks], e)
            continue
        H_or, tol = h_window(xa[toks], axa[toks], ex.gate[e], ex.up[e])
        if spec.fp8:
            c, c_or = check_rows(w["h"][a:b], w["hq"][a:b], w["hs"][a:b], H_or, tol,
                                 f"expert {e}")
        else:
            c, c_or = check_rows(w["h"][a:b], None, None, H_or, tol, f"expert {e}")
        yr[a:b] = c @ ex.down[e]
        br[a:b] = np.abs(c - c_or) @ np.abs(ex.down[e])
    # the combine in slot order, as the oracle's
    rows, gates = ref["row_of_slot"], ref["gates"]
    for j in range(k):
        kept = rows[:, j] >= 0
        rj = rows[kept, j]
        y_codes[kept] = y_codes[kept] + gates[kept, j, None] * yr[rj]
        b_y[kept] = b_y[kept] + gates[kept, j, None] * br[rj]
    r_lr = 0.0 if r_lowrank is None else r_lowrank
    diff_c = np.abs(yg - y_codes)
    tol_c = Y_TOL * rms + r_lr
    rel_c = float(np.max(diff_c / tol_c)) * Y_TOL if rms else 0.0
    rep.update(h_window_ratio=stats["worst_h"], h_entries_moved=stats["h_moved"],
               h_entries=stats["h_n"], y_rel_to_gpu_h=rel_c)
    if spec.fp8:
        rep.update(codes_moved=stats["code_moved"])
    assert rel_c <= Y_TOL, _worst(diff_c, np.broadcast_to(tol_c, diff_c.shape),
                                  "y against the GPU's own h")
    if r_lowrank is not None:
        # low-rank routed rows: the error's RMS at accumulation-order level
        err_rms = float(np.sqrt(np.mean(diff_c ** 2))) / rms if rms else 0.0
        rep.update(y_err_rms_rel_to_gpu_h=err_rms)
        assert err_rms <= LOWRANK_ERR_RMS, f"error RMS {err_rms:.2e} of RMS(y)"
    diff = np.abs(yg - ref["y"])
    tol = Y_TOL * rms + b_y + r_lr
    ratio = float(np.max(diff / tol))
    rep.update(y_tol_ratio=ratio, max_h_term_rel=float(b_y.max()) / rms if rms else 0.0,
               tokens_beyond_rms_bound=int(np.count_nonzero(np.any(diff > Y_TOL * rms, axis=1))))
    assert ratio <= 1.0, _worst(diff, tol, "y against the oracle")
    return rep
