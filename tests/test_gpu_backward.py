"""Layer backward on the GPU against the oracle's backward, through the C ABI.

The forward runs first (its workspace holds what the backward reads); the
oracle's backward then takes the GPU's expert selection for every token (it is
the oracle's own for tokens away from near-ties, and either choice is correct
within them) and the same upstream gradient.

Dense experts give dW of every expert matrix; rank-r experts give the
gradients of their factors U, s and V (and dW of dense shared experts beside
them).

Tolerance, per element of every gradient tensor. Each element is a sum of
products whose bf16 operands both sides round at the same points; the GPU
forms the unrounded operand in float32, the oracle in float64, so an operand
lying within that difference of a bf16 rounding boundary rounds one ulp apart
on the two sides (a change of at most 2^-7 of the operand). Allowing four such
operands per sum, plus float32 summation:
    |gpu - oracle| <= 2^-5 M + 2^-16 S,
M the largest single term's magnitude and S the sum of the terms' magnitudes,
both computed by the oracle. The error relative to the tensor's RMS is
reported as well.
"""
import numpy as np
import pytest
import torch

import oracle
from fine_grained_mixture_amd import layer as L
from fine_grained_mixture_amd import synth
from tests import _parity as P

pytestmark = pytest.mark.gpu

NAMES = ("dx", "dw_router", "dw_gate", "dw_up", "dw_down", "dsh_gate", "dsh_up", "dsh_down",
         *oracle.LOWRANK_GRADS)


def _gpu_fwd_bwd(wl, inp, dy, aux_grad, saved=False):
    cfg, x, w = P.upload(wl, inp)
    out = L.allocate_outputs(cfg, wl.T, x.device, saved_ab=saved)
    ws = L.allocate_workspace(cfg, wl.T, x.device)
    L.layer_forward(cfg, x, w, out, ws)
    dyt = torch.from_numpy(dy).to(x.device)
    g = L.layer_backward(cfg, x, w, out, ws, dyt, aux_grad)
    torch.cuda.synchronize()
    fwd = P.to_numpy(out)
    grads = {n: v.cpu().numpy() for n, v in g.t.items() if v is not None}
    return fwd, grads


def _check(wl, *, aux_grad=1.0, zero_dy=False, saved=False):
    print(f"\n[case] {wl} aux_grad={aux_grad} zero_dy={zero_dy} saved={saved}", flush=True)
    inp = synth.make_inputs(wl)
    dy = np.zeros((wl.T, wl.hidden), np.float32) if zero_dy else synth.make_upstream(wl)
    fwd, g = _gpu_fwd_bwd(wl, inp, dy, aux_grad, saved)
    P.check_parity(wl, inp, fwd, check_y=False)
    spec = P.spec_of(wl)
    gi = fwd["topk_idx"].astype(np.int64)
    ref_f = oracle.layer_forward(inp["x"], inp, spec, tokens=[], override_idx=gi,
                                 override_mask=np.ones(wl.T, bool))
    ref = oracle.layer_backward(inp["x"], inp, spec, dy, aux_grad=aux_grad, fwd=ref_f,
                                scales=True)
    rep = {}
    for n in NAMES:
        if n not in ref:
            continue
        r, v = ref[n], g[n].astype(np.float64)
        assert v.shape == r.shape, n
        assert np.all(np.isfinite(v)), n
        rms = float(np.sqrt(np.mean(r ** 2)))
        err = np.abs(v - r)
        tol = 2.0 ** -5 * ref["M_" + n] + 2.0 ** -16 * ref["S_" + n]
        worst = float(np.max(err / np.maximum(tol, 1e-300))) if r.size else 0.0
        rep[n] = (float(err.max()) / rms if rms else float(err.max(initial=0.0)), worst)
        bad = err > tol
        if bad.any():
            i = np.unravel_index(int(np.argmax(err - tol)), err.shape)
            raise AssertionError(f"{n}: {int(bad.sum())} elements beyond 2^-5 M + 2^-16 S, "
                                 f"e.g. {i}: gpu {v[i]:.6e} oracle {r[i]:.6e} tol {tol[i]:.3e}")
        if wl.dtype == "f32" and rms > 0:
            # no rounding points: only fp32 sums separate the two sides (a bf16
            # rounding anywhere would leave about 1e-3 of the RMS)
            e_rms = float(np.sqrt(np.mean(err ** 2))) / rms
            assert e_rms <= F32_ERR_RMS, f"{n}: error RMS {e_rms:.2e} of its RMS"
    print(f"[report] {wl.name} T={wl.T}: " + ", ".join(
        f"{k}: {a:.2e} rms, {b:.2f} tol" for k, (a, b) in rep.items()), flush=True)
    return rep


# float32 layers: largest RMS of (gpu - oracle) over a gradient tensor,
# relative to its RMS
F32_ERR_RMS = 1e-5

CASES = {
    "quartz_small": synth.QUARTZ.replace(T=517, hidden=256, ffn=128),
    "moonfrost_small_capacity": synth.MOONFROST.replace(T=1000, hidden=256, ffn=128),
    "sutra_small_sigmoid": synth.SUTRA.replace(T=700, hidden=384, ffn=192),
    "quartz_no_shared": synth.QUARTZ.replace(T=300, hidden=128, ffn=64, n_shared=0, seed=2),
    "split_k_tokens": synth.Workload("sk", T=2500, hidden=128, n_routed=8, top_k=2,
                                     n_shared=1, ffn=64, logit_offset_std=0.5, seed=4),
    "one_token": synth.QUARTZ.replace(T=1, hidden=128, ffn=64),
    "wide_ffn_k1": synth.Workload("wk", T=260, hidden=192, n_routed=8, top_k=1, n_shared=3,
                                  ffn=320, seed=6),
    # edge cases: nearly every slot dropped; every expert selected with raw
    # softmax gates; sigmoid without shared experts; widths that leave partial
    # column tiles in every product; a handful of tokens
    "capacity_one": synth.QUARTZ.replace(T=200, hidden=128, ffn=64,
                                         capacity_factor="1/200"),
    "all_experts_raw_softmax": synth.Workload("ak", T=150, hidden=128, n_routed=8, top_k=8,
                                              n_shared=1, ffn=64, renorm=0, seed=7),
    "sigmoid_no_shared": synth.SUTRA.replace(T=333, hidden=128, ffn=64, n_shared=0),
    "odd_widths": synth.Workload("ow", T=257, hidden=192, n_routed=16, top_k=3, n_shared=3,
                                 ffn=192, logit_offset_std=0.3, seed=11),
    "three_tokens": synth.QUARTZ.replace(T=3, hidden=256, ffn=128, seed=12),
    # Quartz widths at T = 1 and 2: the forward keeps its products from the
    # 512-thread decode kernels
    "quartz_widths_t1": synth.QUARTZ.replace(T=1, seed=21),
    "quartz_widths_t2": synth.QUARTZ.replace(T=2, seed=22),
    # float32 layers (the fp32 FMA products, a | b recomputed): the Tiny layer
    # and wider ones with capacity drops, sigmoid gates, no or three shared
    # experts, top-1, and more rows than one tile per expert
    "tiny_f32": synth.TINY,
    "f32_rows": synth.TINY.replace(T=1500, hidden=192, ffn=128, n_routed=12, top_k=3,
                                   n_shared=2, seed=31),
    "f32_capacity_sigmoid": synth.Workload("fc", T=600, hidden=128, n_routed=16, top_k=2,
                                           n_shared=0, ffn=64, score="sigmoid", renorm=1,
                                           select_bias_std=0.1, capacity_factor="1/2",
                                           dtype="f32", seed=32),
    "f32_k1_three_shared": synth.Workload("f1", T=257, hidden=128, n_routed=8, top_k=1,
                                          n_shared=3, ffn=192, dtype="f32", seed=33),
    # many experts: the router backward holding a token's logits in registers
    # (E >= 256), raw softmax gates, the last lanes partly filled
    "many_experts_raw_softmax": synth.Workload("me", T=300, hidden=128, n_routed=264, top_k=4,
                                               n_shared=1, ffn=64, renorm=0,
                                               logit_offset_std=0.3, seed=21),
}


@pytest.mark.parametrize("name", list(CASES))
def test_backward_parity(name):
    _check(CASES[name])


# the forward keeps its gate and up products; the backward then runs dh alone
SAVED = ["quartz_small", "moonfrost_small_capacity", "sutra_small_sigmoid", "quartz_no_shared",
         "one_token", "wide_ffn_k1", "quartz_widths_t1", "quartz_widths_t2"]


@pytest.mark.parametrize("name", SAVED)
def test_backward_parity_saved_products(name):
    _check(CASES[name], saved=True)


def test_saving_products_leaves_forward_unchanged():
    """y and the routing are bitwise the same with saved_ab; the saved gate and
    up products match the oracle's x W_gate and x W_up on sampled rows."""
    for wl in (synth.QUARTZ.replace(T=300, hidden=256, ffn=128, seed=12),
               synth.QUARTZ.replace(T=3, hidden=256, ffn=128, seed=13),
               synth.QUARTZ.replace(T=2, seed=14)):
        inp = synth.make_inputs(wl)
        cfg, x, w = P.upload(wl, inp)
        outs = []
        for saved in (False, True):
            out = L.allocate_outputs(cfg, wl.T, x.device, saved_ab=saved)
            ws = L.allocate_workspace(cfg, wl.T, x.device)
            L.layer_forward(cfg, x, w, out, ws)
            torch.cuda.synchronize()
            outs.append(out)
        for key in ("y", "topk_idx", "topk_gate", "row_of_slot", "sorted_token"):
            assert torch.equal(outs[0][key], outs[1][key]), key
        ab = outs[1]["saved_ab"].cpu().numpy().astype(np.float64)
        F, S, k = wl.ffn, wl.n_shared, wl.top_k
        R = wl.T * k
        rows = outs[1]["row_of_slot"].cpu().numpy()
        idx = outs[1]["topk_idx"].cpu().numpy()
        xs = inp["x"].astype(np.float64)
        for t in sorted({0, wl.T // 2, wl.T - 1}):
            for j in range(k):
                e, r = int(idx[t, j]), int(rows[t, j])
                want = np.concatenate([xs[t] @ inp["w_gate"][e], xs[t] @ inp["w_up"][e]])
                got = ab[r * 2 * F:(r + 1) * 2 * F]
                scale = np.abs(xs[t]) @ np.abs(np.concatenate([inp["w_gate"][e], inp["w_up"][e]], 1))
                assert np.all(np.abs(got - want) <= 1e-5 * scale + 1e-30), (t, j)
            for s_ in range(S):
                want = np.concatenate([xs[t] @ inp["sh_gate"][s_], xs[t] @ inp["sh_up"][s_]])
                o = R * 2 * F + (t * S + s_) * 2 * F
                got = ab[o:o + 2 * F]
                scale = np.abs(xs[t]) @ np.abs(np.concatenate([inp["sh_gate"][s_], inp["sh_up"][s_]], 1))
                assert np.all(np.abs(got - want) <= 1e-5 * scale + 1e-30), (t, s_)


def test_backward_aux_only():
    """dy = 0: only the aux statistic's gradient reaches the router and x."""
    rep = _check(synth.QUARTZ.replace(T=400, hidden=128, ffn=64, logit_offset_std=0.5, seed=3),
                 aux_grad=3.0, zero_dy=True)
    assert rep["dw_gate"][0] == 0.0


def test_backward_empty_batch_zeroes_weight_grads():
    wl = synth.QUARTZ.replace(T=0, hidden=128, ffn=64)
    inp = synth.make_inputs(wl)
    cfg, x, w = P.upload(wl, inp)
    out = L.allocate_outputs(cfg, 0, x.device)
    ws = L.allocate_workspace(cfg, 0, x.device)
    L.layer_forward(cfg, x, w, out, ws)
    grads = L.allocate_grads(cfg, 0, x.device)
    for n, v in grads.t.items():
        if v is not None:
            v.fill_(7.0)
    L.layer_backward(cfg, x, w, out, ws, torch.zeros((0, wl.hidden), device=x.device),
                     1.0, grads)
    torch.cuda.synchronize()
    for n, v in grads.t.items():
        if v is not None and v.numel():
            assert float(v.abs().max()) == 0.0, n


def test_backward_deterministic():
    wl = synth.QUARTZ.replace(T=700, hidden=256, ffn=128, seed=9)
    inp = synth.make_inputs(wl)
    dy = synth.make_upstream(wl)
    _, g1 = _gpu_fwd_bwd(wl, inp, dy, 1.0)
    _, g2 = _gpu_fwd_bwd(wl, inp, dy, 1.0)
    for n in g1:
        assert np.array_equal(g1[n], g2[n]), n


# Full sizes: every element of every gradient against the per-expert batched
# oracle (pinned to the token loop on small inputs), with its bound B >= M of
# the largest term: |gpu - oracle| <= 2^-5 B + 2^-16 S. Sutra runs at its full
# widths with a quarter of its tokens (the oracle's time at 32768 tokens).
FULL = {
    "quartz_saved": (synth.QUARTZ, True),
    "quartz_recompute": (synth.QUARTZ, False),
    "moonfrost_saved": (synth.MOONFROST, True),
    "sutra_t8192_saved": (synth.SUTRA.replace(T=8192), True),
}


@pytest.mark.parametrize("name", list(FULL))
def test_full_size_backward(name):
    wl, saved = FULL[name]
    print(f"\n[case] {name}: {wl}", flush=True)
    inp = synth.make_inputs(wl)
    dy = synth.make_upstream(wl)
    fwd, g = _gpu_fwd_bwd(wl, inp, dy, 1.0, saved)
    P.check_parity(wl, inp, fwd, check_y=False)
    spec = P.spec_of(wl)
    gi = fwd["topk_idx"].astype(np.int64)
    ref_f = oracle.layer_forward(inp["x"], inp, spec, tokens=[], override_idx=gi,
                                 override_mask=np.ones(wl.T, bool))
    ref = oracle.layer_backward_batched(inp["x"], inp, spec, dy, aux_grad=1.0, fwd=ref_f)
    rep = {}
    for n in NAMES:
        if n not in ref:
            continue
        r, v = ref[n], g[n].astype(np.float64)
        assert v.shape == r.shape and np.all(np.isfinite(v)), n
        err = np.abs(v - r)
        tol = 2.0 ** -5 * ref["B_" + n] + 2.0 ** -16 * ref["S_" + n]
        rms = float(np.sqrt(np.mean(r ** 2)))
        rep[n] = (float(err.max()) / rms, float(np.max(err / np.maximum(tol, 1e-300))))
        bad = err > tol
        assert not bad.any(), f"{n}: {int(bad.sum())} elements beyond 2^-5 B + 2^-16 S"
    print(f"[report] {name}: " + ", ".join(
        f"{k}: {a:.2e} rms, {b:.2f} tol" for k, (a, b) in rep.items()), flush=True)


# Rank-64 (and rank-32) experts: the factor gradients of U diag(s) V^T,
# checked link by link on every element from the GPU's own intermediates (the
# backward workspace) and then against the per-expert batched oracle
# (_parity.lowrank_backward_check).
def _check_lowrank(wl, aux_grad=1.0):
    print(f"\n[case] low-rank backward {wl}", flush=True)
    inp = synth.make_inputs(wl)
    dy = synth.make_upstream(wl)
    cfg, x, w = P.upload(wl, inp)
    out = L.allocate_outputs(cfg, wl.T, x.device)
    ws = L.allocate_workspace(cfg, wl.T, x.device)
    L.layer_forward(cfg, x, w, out, ws)
    bws = L.allocate_backward_workspace(cfg, wl.T, x.device)
    g = L.layer_backward(cfg, x, w, out, ws, torch.from_numpy(dy).to(x.device), aux_grad,
                         bws=bws)
    torch.cuda.synchronize()
    fwd = P.to_numpy(out)
    grads = {n: v.cpu().numpy() for n, v in g.t.items() if v is not None}
    rows = int(fwd["offsets"][wl.n_routed])
    I = P.backward_intermediates(cfg, wl.T, bws, rows)
    I["h_sh"] = P.workspace_intermediates(cfg, wl.T, ws, rows)["h_sh"]
    P.check_parity(wl, inp, fwd, check_y=False)
    spec = P.spec_of(wl)
    gi = fwd["topk_idx"].astype(np.int64)
    ref_f = oracle.layer_forward(inp["x"], inp, spec, tokens=[], override_idx=gi,
                                 override_mask=np.ones(wl.T, bool))
    ref = oracle.layer_backward_batched(inp["x"], inp, spec, dy, aux_grad=aux_grad, fwd=ref_f)
    rep = P.lowrank_backward_check(inp, spec, dy, fwd, grads, I, ref)
    print(f"[report] low-rank {wl.name} T={wl.T}: tipped {rep['tipped']}; "
          f"worst sum/bound {max(rep['worst_sum'].values()):.3f}; error RMS " +
          ", ".join(f"{k}: {v:.1e}" for k, v in rep["err_rms"].items()), flush=True)
    return rep


LOWRANK = {
    "dormouse_small": synth.DORMOUSE.replace(T=600, hidden=256, ffn=128),
    "dormouse_small_renorm": synth.DORMOUSE.replace(T=500, hidden=256, ffn=192, renorm=1,
                                                    seed=3),
    "rank32": synth.DORMOUSE.replace(T=420, hidden=256, ffn=128, rank=32, n_routed=64, seed=4),
    "capacity": synth.DORMOUSE.replace(T=900, hidden=128, ffn=128, n_routed=64,
                                       capacity_factor="3/2", logit_offset_std=0.5, seed=13),
    "sigmoid": synth.DORMOUSE.replace(T=333, hidden=192, ffn=128, n_routed=200, score="sigmoid",
                                      renorm=1, select_bias_std=0.1, seed=14),
    "sigmoid_many": synth.DORMOUSE.replace(T=700, hidden=128, ffn=64, n_routed=520,
                                           score="sigmoid", renorm=1, select_bias_std=0.1,
                                           seed=15),
    "zipf_skew": synth.DORMOUSE.replace(T=1500, hidden=256, ffn=128, n_routed=64, zipf_s=1.1,
                                        seed=11),
    "one_token": synth.DORMOUSE.replace(T=1, hidden=128, ffn=64, seed=2),
    # dense shared experts beside the rank-r ones: one, two with r = 32 and
    # renormalised gates, and one over more tokens than a shared-expert chunk
    # (4096: the weight gradients split over tokens and reduced in order)
    "shared": synth.DORMOUSE.replace(T=500, hidden=256, ffn=128, n_shared=1, seed=21),
    "rank32_two_shared": synth.DORMOUSE.replace(T=700, hidden=192, ffn=128, rank=32,
                                                n_routed=64, n_shared=2, renorm=1, seed=22),
    "shared_split": synth.DORMOUSE.replace(T=5000, hidden=128, ffn=64, n_routed=64, n_shared=1,
                                           seed=23),
    "full_dormouse": synth.DORMOUSE,
}


@pytest.mark.parametrize("name", list(LOWRANK))
def test_lowrank_backward_parity(name):
    _check_lowrank(LOWRANK[name])


def test_lowrank_backward_deterministic_and_empty_batch():
    wl = LOWRANK["dormouse_small"]
    inp = synth.make_inputs(wl)
    dy = synth.make_upstream(wl)
    _, g1 = _gpu_fwd_bwd(wl, inp, dy, 1.0)
    _, g2 = _gpu_fwd_bwd(wl, inp, dy, 1.0)
    for n in g1:
        assert np.array_equal(g1[n], g2[n]), n
    wl0 = wl.replace(T=0)
    cfg, x, w = P.upload(wl0, synth.make_inputs(wl0))
    out = L.allocate_outputs(cfg, 0, x.device)
    ws = L.allocate_workspace(cfg, 0, x.device)
    L.layer_forward(cfg, x, w, out, ws)
    grads = L.allocate_grads(cfg, 0, x.device)
    for v in grads.t.values():
        if v is not None:
            v.fill_(7.0)
    L.layer_backward(cfg, x, w, out, ws, torch.zeros((0, wl.hidden), device=x.device), 1.0,
                     grads)
    torch.cuda.synchronize()
    for n, v in grads.t.items():
        if v is not None and v.numel():
            assert float(v.abs().max()) == 0.0, n
