"""fp8 (E4M3) experts on the GPU against the oracle, through the C ABI.

The device quantisation of the expert weights must give the oracle's codes and
power-of-two scales exactly (both round v / 2^s to the nearest E4M3 value, ties
to even). The layer then meets the forward's acceptance: routing bit-exact
after the near-tie override, gates and aux as for bf16; for dense experts the
chain of tests/_parity.py (fp8_chain): the GPU's h codes are the oracle's
quantisation of its own bf16 h, its h is within one ulp and the fp8 products'
window of the oracle's, and y is within 1e-2 RMS of the oracle's down
projections of those codes, on every element. Low-rank experts keep only
their factors in fp8 (products bf16), so the bound there is the bf16 one.
"""
import numpy as np
import pytest
import torch

import oracle
from fine_grained_mixture_amd import _lib, synth
from fine_grained_mixture_amd import layer as L
from tests import _parity as P

pytestmark = pytest.mark.gpu


def _decode(codes: torch.Tensor) -> np.ndarray:
    return codes.view(torch.float8_e4m3fn).to(torch.float64).cpu().numpy()


def test_weight_quantization_matches_oracle():
    wl = synth.QUARTZ.replace(T=8, hidden=256, ffn=192, n_shared=3, dtype="fp8", seed=21)
    inp = synth.make_inputs(wl)
    cfg = L.config_from_workload(wl)
    w = L.DeviceWeights.from_numpy(inp, cfg)
    torch.cuda.synchronize()
    E, d, F, S = wl.n_routed, wl.hidden, wl.ffn, wl.n_shared
    cases = [("w_gate", inp["w_gate"], (E, F, d)), ("w_up", inp["w_up"], (E, F, d)),
             ("w_down", inp["w_down"], (E, d, F)), ("sh_gate", inp["sh_gate"], (S, F, d)),
             ("sh_up", inp["sh_up"], (S, F, d)),
             ("sh_down", inp["sh_down"].reshape(1, S * F, d), (1, d, S * F))]
    for name, src, shape in cases:
        codes = w.t[name].reshape(shape)
        scale = w.t[name + "_scale"].reshape(shape[0], shape[1]).cpu().numpy().astype(np.float64)
        got = _decode(codes) * scale[:, :, None]            # [G, out, in]
        for g in range(shape[0]):
            ref, s = oracle.fp8_quantize(np.asarray(src[g], np.float64), axis=0)   # [in, out]
            np.testing.assert_array_equal(scale[g], np.ldexp(1.0, s), err_msg=name)
            np.testing.assert_array_equal(got[g], ref.T, err_msg=name)


def test_factor_quantization_matches_oracle():
    """Low-rank experts: U codes (written transposed, [E, r, in]) with one scale
    per column r, V codes [E, out, r] with one scale per row; s is left bf16."""
    wl = synth.DORMOUSE.replace(T=8, hidden=256, ffn=192, n_routed=12, dtype="fp8", seed=23)
    inp = synth.make_inputs(wl)
    cfg = L.config_from_workload(wl)
    w = L.DeviceWeights.from_numpy(inp, cfg)
    torch.cuda.synchronize()
    E, d, F, r = wl.n_routed, wl.hidden, wl.ffn, wl.rank
    for name, n_in in (("u_gate", d), ("u_up", d), ("u_down", F)):
        codes = w.t[name].reshape(E, r, n_in)
        scale = w.t[name + "_scale"].reshape(E, r).cpu().numpy().astype(np.float64)
        got = _decode(codes) * scale[:, :, None]            # [E, r, in]
        for e in range(E):
            ref, s = oracle.fp8_quantize(np.asarray(inp[name][e], np.float64), axis=0)
            np.testing.assert_array_equal(scale[e], np.ldexp(1.0, s), err_msg=name)
            np.testing.assert_array_equal(got[e], ref.T, err_msg=name)
    for name, n_out in (("v_gate", F), ("v_up", F), ("v_down", d)):
        codes = w.t[name].reshape(E, n_out, r)
        scale = w.t[name + "_scale"].reshape(E, n_out).cpu().numpy().astype(np.float64)
        got = _decode(codes) * scale[:, :, None]
        for e in range(E):
            ref, s = oracle.fp8_quantize(np.asarray(inp[name][e], np.float64), axis=1)
            np.testing.assert_array_equal(scale[e], np.ldexp(1.0, s), err_msg=name)
            np.testing.assert_array_equal(got[e], ref, err_msg=name)
    for name in ("s_gate", "s_up", "s_down"):
        np.testing.assert_array_equal(w.t[name].float().cpu().numpy(),
                                      np.asarray(inp[name], np.float32), err_msg=name)


SMALL = {
    "quartz_small": synth.QUARTZ.replace(T=517, hidden=256, ffn=128, dtype="fp8"),
    "moonfrost_small_capacity": synth.MOONFROST.replace(T=1000, hidden=256, ffn=128,
                                                        dtype="fp8"),
    "sutra_small_sigmoid": synth.SUTRA.replace(T=700, hidden=384, ffn=192, dtype="fp8"),
    "no_shared": synth.QUARTZ.replace(T=300, hidden=128, ffn=64, n_shared=0, dtype="fp8",
                                      seed=2),
    "one_token": synth.QUARTZ.replace(T=1, hidden=128, ffn=64, dtype="fp8"),
    "three_shared": synth.Workload("s3", T=260, hidden=192, n_routed=16, top_k=3, n_shared=3,
                                   ffn=192, dtype="fp8", seed=6),
    "capacity_one": synth.QUARTZ.replace(T=200, hidden=128, ffn=64, capacity_factor="1/200",
                                         dtype="fp8"),
    "decode_t2": synth.QUARTZ.replace(T=2, dtype="fp8", seed=5),
    "decode_t4": synth.SUTRA.replace(T=4, dtype="fp8", seed=8),
    "dormouse_small": synth.DORMOUSE.replace(T=600, hidden=256, ffn=128, dtype="fp8"),
    "dormouse_small_shared": synth.DORMOUSE.replace(T=333, hidden=256, ffn=192, n_shared=2,
                                                    renorm=1, dtype="fp8", seed=4),
    "dormouse_decode": synth.DORMOUSE.replace(T=3, dtype="fp8", seed=9),
}


def _run(wl):
    print(f"\n[case] {wl}", flush=True)
    inp = synth.make_inputs(wl)
    g = P.run_gpu(wl, inp)
    rep = P.check_parity(wl, inp, g)
    print(f"[report] {wl.name} fp8 T={wl.T}: {rep}", flush=True)
    return rep


@pytest.mark.parametrize("name", list(SMALL))
def test_fp8_small_parity(name):
    _run(SMALL[name])


FULL = {
    "quartz": synth.QUARTZ.replace(dtype="fp8"),
    "moonfrost": synth.MOONFROST.replace(dtype="fp8"),
    "sutra": synth.SUTRA.replace(dtype="fp8"),
    "dormouse": synth.DORMOUSE.replace(dtype="fp8"),
}


@pytest.mark.parametrize("name", list(FULL))
def test_fp8_full_size_parity(name):
    """Every output element; for dense experts every h entry, code and row
    scale of the GPU's intermediates too."""
    _run(FULL[name])


def test_fp8_stage_entry_points_match_layer():
    """moe_route -> moe_permute (x_perm) -> moe_grouped_ffn -> moe_combine gives
    the whole-layer result: the x_perm rows quantise to the same codes as the
    token rows they copy."""
    wl = synth.QUARTZ.replace(T=333, hidden=256, ffn=128, dtype="fp8", seed=8)
    inp = synth.make_inputs(wl)
    cfg, x, w = P.upload(wl, inp)
    out = L.allocate_outputs(cfg, wl.T, x.device)
    ws = L.allocate_workspace(cfg, wl.T, x.device)
    L.layer_forward(cfg, x, w, out, ws)
    out2 = L.allocate_outputs(cfg, wl.T, x.device)
    ws2 = L.allocate_workspace(cfg, wl.T, x.device)
    R = _lib.moe_max_rows(cfg, wl.T)
    x_perm = torch.empty((R, wl.hidden), dtype=torch.bfloat16, device=x.device)
    y_r = torch.empty((R, wl.hidden), dtype=torch.float32, device=x.device)
    y_s = torch.empty((wl.T, wl.hidden), dtype=torch.float32, device=x.device)
    L.route(cfg, x, w, out2, ws2)
    L.permute(cfg, x, out2, ws2, x_perm)
    L.grouped_ffn(cfg, wl.T, _lib.MOE_GROUPS_ROUTED | _lib.MOE_GROUPS_SHARED, w, ws2,
                  x_perm=x_perm, offsets=out2["offsets"], x_shared=x, y_routed=y_r, y_shared=y_s)
    L.combine(cfg, wl.T, y_r, y_s, out2)
    torch.cuda.synchronize()
    assert torch.equal(out["y"], out2["y"])
