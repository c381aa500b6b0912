"""GPU-vs-oracle parity helpers (test infrastructure).

Acceptance (what the layer must reproduce, per token whose k-th vs (k+1)-th
key margin exceeds 1e-4 in the oracle):
  * selected expert sets, per-expert counts, kept counts, offsets,
    sorted_token, the (token, expert) -> row map, drop flags and n_dropped:
    bit-exact, after the oracle is re-run with near-tie tokens forced to the
    GPU's selection (either choice is correct for them);
  * gates within 1e-5 absolute, aux within 1e-4 relative;
  * max |y_gpu - y_oracle| <= 1e-2 * RMS(y_oracle) over the checked tokens;
    for fp8 experts per element 1e-2 * RMS(y_oracle) + 2^-2 M_y, M_y the
    largest single term g h_f W_down[f, c] of that element's down products:
    both sides quantise h from their own bf16 h, and where those differ by one
    bf16 ulp the E4M3 code can differ by one step (at most 2^-3 of h), which
    the bound allows twice at the largest term; and at most max(2, 10%) of the
    checked tokens may have any element beyond the plain 1e-2 RMS bound.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from fine_grained_mixture_amd.layer import (DeviceWeights, allocate_outputs, allocate_workspace,
                                            config_from_workload)
from fine_grained_mixture_amd import layer as L

NEAR_TIE = 1e-4
Y_TOL = 1e-2
GATE_TOL = 1e-5
AUX_RTOL = 1e-4
FP8_FLIP_TOKENS = 0.1


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


def run_gpu(wl, inp, *, y_lowp=False):
    cfg, x, w = upload(wl, inp)
    out = allocate_outputs(cfg, wl.T, x.device, y_lowp=y_lowp)
    ws = allocate_workspace(cfg, wl.T, x.device)
    L.layer_forward(cfg, x, w, out, ws)
    torch.cuda.synchronize()
    return to_numpy(out)


def slot_map(idx, rows):
    """(token, expert) -> row (or -1)."""
    T, k = idx.shape
    return {(t, int(idx[t, j])): int(rows[t, j]) for t in range(T) for j in range(k)}


def check_parity(wl, inp, g, tokens=None, *, check_y=True):
    """Compare GPU outputs g (numpy dict) with the oracle. Returns a report."""
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
    ref = oracle.layer_forward(inp["x"], inp, spec, tokens=[] if not check_y else tokens,
                               override_idx=gi, override_mask=ov, scales=spec.fp8)
    for key in ("counts", "kept", "offsets"):
        np.testing.assert_array_equal(g[key], ref[key], err_msg=key)
    assert int(g["n_dropped"][0]) == ref["n_dropped"]
    R = int(ref["offsets"][-1])
    np.testing.assert_array_equal(g["sorted_token"][:R], ref["sorted_token"], err_msg="sorted_token")
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
    if check_y:
        toks = ref["tokens"]
        yg = g["y"][toks].astype(np.float64)
        yr = ref["y"]
        rms = float(np.sqrt(np.mean(yr ** 2)))
        err = float(np.max(np.abs(yg - yr))) if len(toks) else 0.0
        rep.update(y_err=err, y_rms=rms, y_rel=err / rms if rms else 0.0, checked=len(toks))
        assert np.all(np.isfinite(yg))
        if spec.fp8:
            tol = Y_TOL * rms + 2.0 ** -2 * ref["M_y"]
            ratio = float(np.max(np.abs(yg - yr) / tol)) if len(toks) else 0.0
            # flips touch only the tokens whose h row had one: the share of
            # tokens with any element beyond the plain bound stays small
            beyond = np.any(np.abs(yg - yr) > Y_TOL * rms, axis=1) if len(toks) else np.zeros(0)
            frac = float(np.mean(beyond)) if len(toks) else 0.0
            rep.update(y_tol_ratio=ratio, tokens_beyond_rms_bound=frac)
            assert ratio <= 1.0, f"max |dy| / (1e-2 RMS + 2^-2 M_y) = {ratio:.3f}"
            # (at least two tokens allowed, so that tiny batches are not judged by share)
            allowed = max(2, int(FP8_FLIP_TOKENS * len(toks)))
            assert int(beyond.sum()) <= allowed, f"{frac:.3f} of tokens beyond 1e-2 RMS"
        else:
            assert err <= Y_TOL * rms, f"max|dy| {err:.3e} > {Y_TOL} * RMS {rms:.3e}"
    return rep


def sample_tokens(T, n, seed=0, extra=()):
    rng = np.random.default_rng(seed)
    base = {0, T - 1, T // 2}
    base.update(int(t) for t in extra)
    base.update(int(t) for t in rng.choice(T, size=min(n, T), replace=False))
    return np.array(sorted(t for t in base if 0 <= t < T))
