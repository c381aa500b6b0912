"""Pins of the CPU oracle against things other than itself.

No page prints layer inputs or outputs, so the oracle is pinned by: brute force
on tiny inputs (tests/_brute.py, independent code), closed forms, invariants,
textbook reductions, exact rounding values, a library rounding routine, and the
parameter totals the pages print for Quartz.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import LayerSpec
from fine_grained_mixture_amd import synth
from tests import _brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _inputs(T, d, E, k, S, F, seed, *, rank=0, score="softmax", bf16=False,
            logit_std=0.0, select_std=0.0, w_std=0.3, zero_router=False):
    wl = synth.Workload("t", T=T, hidden=d, n_routed=E, top_k=k, n_shared=S, ffn=F,
                        rank=rank, score=score, dtype="bf16" if bf16 else "f32",
                        logit_offset_std=logit_std, select_bias_std=select_std,
                        w_std=w_std, seed=seed)
    w = synth.make_inputs(wl)
    if zero_router:
        w["w_router"] = np.zeros_like(w["w_router"])
    return w


def _spec(d, E, k, S, F, **kw):
    return LayerSpec(hidden=d, n_routed=E, top_k=k, n_shared=S, ffn=F, **kw)


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ---------------------------------------------------------------- rho (bf16)
def test_round_bf16_exact_values():
    r = oracle.round_bf16
    one = 1.0
    assert r(one) == 1.0
    assert r(1 + 2 ** -8) == 1.0                        # halfway, ties to even (down)
    assert r(1 + 3 * 2 ** -8) == 1 + 2 ** -6            # halfway, ties to even (up)
    assert r(1 + 2 ** -8 + 2 ** -30) == 1 + 2 ** -7     # just above halfway
    assert r(1 + 2 ** -8 - 2 ** -30) == 1.0             # just below halfway
    assert r(-(1 + 3 * 2 ** -8)) == -(1 + 2 ** -6)
    assert r(255.5) == 256.0 and r(254.5) == 254.0
    assert r(3.0) == 3.0 and r(0.0) == 0.0
    assert r(2.0 ** -130) == 2.0 ** -130                 # bf16 subnormal, exact
    assert r(2.0 ** -134) == 0.0                         # half of min subnormal -> even (0)
    assert math.isinf(r(1e39)) and r(1e39) > 0


def test_round_bf16_matches_library_on_float32_values():
    # Each float32 value rounds once to bf16: torch's float32->bfloat16
    # conversion is round-to-nearest-even, so it is a valid library reference.
    rng = np.random.default_rng(1)
    a = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 3,
                        rng.standard_normal(2000).astype(np.float32) * 1e-20,
                        rng.standard_normal(2000).astype(np.float32) * 1e20])
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.round_bf16(a.astype(np.float64)), ref)
    # the input generator's own rounding agrees with the library as well
    np.testing.assert_array_equal(synth.bf16_round_f32(a).astype(np.float64), ref)


def test_round_bf16_matches_exact_fraction_rounding():
    rng = np.random.default_rng(2)
    a = rng.standard_normal(3000) * np.exp(rng.uniform(-20, 20, 3000))
    got = oracle.round_bf16(a)
    ref = np.array([_brute.bf16_exact(float(v)) for v in a])
    np.testing.assert_array_equal(got, ref)


# ---------------------------------------------------------------- brute force
CASES = [
    # T, d, E, k, S, F, kwargs
    (16, 12, 8, 2, 1, 8, dict(score="softmax", renorm=True)),
    (16, 12, 8, 2, 0, 8, dict(score="softmax", renorm=False)),
    (12, 10, 6, 3, 2, 6, dict(score="softmax", renorm=True, capacity=5)),
    (14, 10, 7, 2, 1, 8, dict(score="sigmoid", renorm=True)),
    (14, 10, 7, 3, 0, 8, dict(score="sigmoid", renorm=True, capacity=4)),
    (10, 16, 5, 2, 1, 16, dict(score="softmax", renorm=True, rank=4)),
]


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_oracle_equals_bruteforce(case, bf16):
    T, d, E, k, S, F, kw = CASES[case]
    rank = kw.get("rank", 0)
    w = _inputs(T, d, E, k, S, F, seed=10 + case, rank=rank, score=kw["score"],
                bf16=bf16, logit_std=0.7, select_std=0.2 if kw["score"] == "sigmoid" else 0)
    spec = _spec(d, E, k, S, F, bf16=bf16, **kw)
    out = oracle.layer_forward(w["x"], w, spec)
    bf = _brute.layer_bruteforce(w["x"], w, E=E, k=k, S=S, F=F, d=d, bf16=bf16,
                                 score=kw["score"], renorm=kw["renorm"],
                                 capacity=kw.get("capacity", 0), rank=rank)
    for t in range(T):
        assert tuple(sorted(out["idx"][t])) == bf["sel"][t]
        np.testing.assert_allclose(out["gates"][t], bf["G"][t, out["idx"][t]], rtol=1e-12)
        for j in range(k):
            assert (out["row_of_slot"][t, j] >= 0) == bf["keep"][t, out["idx"][t, j]]
    np.testing.assert_array_equal(out["counts"], bf["counts"])
    assert _rel(out["y"], bf["y"]) < 1e-12
    assert abs(out["aux_raw"] - bf["aux_raw"]) < 1e-12
    np.testing.assert_allclose(out["P"], bf["P"], rtol=1e-12)
    # margins: the k-th minus the (k+1)-th key
    key = out["key"]
    for t in range(T):
        srt = np.sort(key[t])[::-1]
        assert abs(out["margin"][t] - (srt[k - 1] - srt[k])) < 1e-15


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_batched_forward_equals_bruteforce(case, bf16):
    """The per-expert batched forward (the full-size checks' oracle) against
    the brute-force evaluation of every expert on every token."""
    T, d, E, k, S, F, kw = CASES[case]
    rank = kw.get("rank", 0)
    w = _inputs(T, d, E, k, S, F, seed=10 + case, rank=rank, score=kw["score"],
                bf16=bf16, logit_std=0.7, select_std=0.2 if kw["score"] == "sigmoid" else 0)
    spec = _spec(d, E, k, S, F, bf16=bf16, **kw)
    out = oracle.layer_forward_batched(w["x"], w, spec)
    bf = _brute.layer_bruteforce(w["x"], w, E=E, k=k, S=S, F=F, d=d, bf16=bf16,
                                 score=kw["score"], renorm=kw["renorm"],
                                 capacity=kw.get("capacity", 0), rank=rank)
    assert out["y"].shape == (T, d)
    assert _rel(out["y"], bf["y"]) < 1e-12


BATCHED_CASES = [
    # T, d, E, k, S, F, workload extras
    (40, 24, 8, 3, 2, 16, dict(logit_std=0.5)),
    (33, 16, 6, 2, 0, 8, dict(score="sigmoid", select_std=0.2)),
    (50, 16, 5, 2, 1, 8, dict(logit_std=1.0, capacity=7)),
    (30, 32, 6, 2, 1, 32, dict(rank=16)),
    (24, 32, 4, 2, 2, 16, dict(fp8=True)),
    (20, 64, 4, 2, 1, 64, dict(fp8=True, rank=64)),
]


@pytest.mark.parametrize("case", range(len(BATCHED_CASES)))
def test_batched_forward_equals_token_loop(case):
    """The batched forward gives the token loop's y on every token (bf16
    rounding points, capacity drops, low-rank and fp8 experts), with a forced
    selection too."""
    T, d, E, k, S, F, kw = BATCHED_CASES[case]
    kw = dict(kw)
    score, cap = kw.pop("score", "softmax"), kw.pop("capacity", 0)
    fp8, rank = kw.pop("fp8", False), kw.pop("rank", 0)
    w = _inputs(T, d, E, k, S, F, seed=70 + case, rank=rank, score=score, bf16=True, **kw)
    spec = _spec(d, E, k, S, F, score=score, capacity=cap, rank=rank, bf16=True, fp8=fp8)
    a = oracle.layer_forward(w["x"], w, spec)
    b = oracle.layer_forward_batched(w["x"], w, spec)
    assert _rel(b["y"], a["y"]) < 1e-12
    for n in ("idx", "gates", "row_of_slot", "counts", "offsets", "sorted_token"):
        np.testing.assert_array_equal(b[n], a[n], err_msg=n)
    # forced selection of a third of the tokens
    mask = np.arange(T) % 3 == 0
    forced = np.tile(np.arange(E - k, E)[::-1], (T, 1))
    a = oracle.layer_forward(w["x"], w, spec, override_idx=forced, override_mask=mask)
    b = oracle.layer_forward_batched(w["x"], w, spec, override_idx=forced, override_mask=mask)
    assert _rel(b["y"], a["y"]) < 1e-12


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("score,renorm", [("softmax", True), ("softmax", False),
                                          ("sigmoid", True)])
def test_zero_router_closed_form(score, renorm):
    T, d, E, k, S, F, C = 40, 16, 8, 3, 1, 8, 13
    w = _inputs(T, d, E, k, S, F, seed=3, score=score, zero_router=True)
    spec = _spec(d, E, k, S, F, score=score, renorm=renorm, capacity=C, bf16=False)
    out = oracle.layer_forward(w["x"], w, spec)
    np.testing.assert_array_equal(out["idx"], np.tile(np.arange(k), (T, 1)))
    want_gate = 1.0 / k if (renorm or score == "sigmoid") else 1.0 / E
    np.testing.assert_allclose(out["gates"], want_gate, rtol=1e-15)
    np.testing.assert_array_equal(out["counts"], [T] * k + [0] * (E - k))
    np.testing.assert_array_equal(out["kept"], [C] * k + [0] * (E - k))
    assert out["n_dropped"] == k * (T - C)
    np.testing.assert_array_equal(out["dropped"], np.repeat((np.arange(T) >= C)[:, None], k, 1))
    assert out["aux_raw"] == pytest.approx(1.0, abs=1e-14)
    assert out["aux"] == pytest.approx(0.01, abs=1e-16)
    # y: shared plus the first C tokens' equal-weight mixture of experts 0..k-1
    x = np.asarray(w["x"], np.float64)

    def swiglu(xr, g, u, dn):
        a = xr @ g
        return (a / (1 + np.exp(-a)) * (xr @ u)) @ dn

    for t in (0, C - 1, C, T - 1):
        want = swiglu(x[t], w["sh_gate"][0], w["sh_up"][0], w["sh_down"][0]).astype(np.float64)
        if t < C:
            for e in range(k):
                want += want_gate * swiglu(x[t], w["w_gate"][e], w["w_up"][e], w["w_down"][e])
        assert _rel(out["y"][t], want) < 1e-12


def test_aux_closed_forms():
    spec = _spec(2, 4, 2, 0, 2, bf16=False)
    # perfectly balanced routing: tokens pick {0,1} and {2,3}, so f_i = 1/4 and
    # aux_raw = sum_i P_i = 1
    x = np.array([[1.0, 0.0], [0.0, 1.0]])
    wr = np.array([[5.0, 5.0, 0.0, 0.0], [0.0, 0.0, 5.0, 5.0]])
    r = oracle.route(x, wr, spec)
    d = oracle.dispatch(r["idx"], 4, 0)
    np.testing.assert_array_equal(d["counts"], [1, 1, 1, 1])
    a = oracle.aux_statistic(d["counts"], r["prob"], 2, 2, spec)
    assert a["aux_raw"] == pytest.approx(1.0, abs=1e-15)
    # one token, two experts, top-1: aux_raw = 2 * sigmoid(a)
    spec1 = _spec(1, 2, 1, 0, 2, bf16=False)
    for av in (0.3, 2.0):
        r = oracle.route(np.array([[1.0]]), np.array([[av, 0.0]]), spec1)
        d = oracle.dispatch(r["idx"], 2, 0)
        a = oracle.aux_statistic(d["counts"], r["prob"], 1, 1, spec1)
        assert a["aux_raw"] == pytest.approx(2.0 / (1.0 + math.exp(-av)), rel=1e-15)


# ---------------------------------------------------------------- invariants
def test_gates_sum_to_one_and_bounds():
    for score in ("softmax", "sigmoid"):
        w = _inputs(200, 32, 12, 4, 0, 8, seed=4, score=score, logit_std=1.0,
                    select_std=0.3 if score == "sigmoid" else 0)
        spec = _spec(32, 12, 4, 0, 8, score=score, renorm=True, bf16=False)
        r = oracle.route(w["x"], w["w_router"], spec, w["logit_bias"], w["select_bias"])
        assert np.max(np.abs(r["gates"].sum(axis=1) - 1.0)) < 1e-15
        assert np.all(r["gates"] > 0) and np.all(r["gates"] <= 1.0)


def test_softmax_shift_invariance_and_sigmoid_not():
    w = _inputs(64, 16, 10, 3, 0, 8, seed=5)
    spec = _spec(16, 10, 3, 0, 8, renorm=False, bf16=False)
    r0 = oracle.route(w["x"], w["w_router"], spec, None)
    r1 = oracle.route(w["x"], w["w_router"], spec, np.full(10, 2.5))
    np.testing.assert_array_equal(r0["idx"], r1["idx"])
    np.testing.assert_allclose(r0["gates"], r1["gates"], rtol=1e-12)
    specs = _spec(16, 10, 3, 0, 8, score="sigmoid", bf16=False)
    s0 = oracle.route(w["x"], w["w_router"], specs, None)
    s1 = oracle.route(w["x"], w["w_router"], specs, np.full(10, 2.5))
    assert np.max(np.abs(s0["gates"] - s1["gates"])) > 1e-3


def test_sigmoid_selection_bias_moves_selection_only():
    T, d, E, k = 50, 16, 8, 2
    w = _inputs(T, d, E, k, 0, 8, seed=6, score="sigmoid")
    spec = _spec(d, E, k, 0, 8, score="sigmoid", bf16=False)
    bias = np.zeros(E)
    bias[E - 1] = 10.0                     # forces expert E-1 into every selection
    r = oracle.route(w["x"], w["w_router"], spec, None, bias)
    assert np.all(r["idx"][:, 0] == E - 1)
    l = np.asarray(w["x"], np.float64) @ np.asarray(w["w_router"], np.float64)
    s = 1 / (1 + np.exp(-l))
    for t in range(T):
        sel = r["idx"][t]
        np.testing.assert_allclose(r["gates"][t], s[t, sel] / s[t, sel].sum(), rtol=1e-14)


def test_dispatch_conservation_and_token_order_drops():
    T, E, k = 300, 16, 3
    rng = np.random.default_rng(7)
    # skewed random selections with distinct experts per token
    p = np.exp(-0.3 * np.arange(E))
    p /= p.sum()
    idx = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)])
    for C in (0, 1, 7, 40, 10 ** 6):
        d = oracle.dispatch(idx, E, C)
        assert d["counts"].sum() == T * k
        assert d["kept"].sum() == d["offsets"][E] == T * k - d["n_dropped"]
        rows = d["row_of_slot"][d["row_of_slot"] >= 0]
        np.testing.assert_array_equal(np.sort(rows), np.arange(d["offsets"][E]))
        for e in range(E):
            seg = d["sorted_token"][d["offsets"][e]:d["offsets"][e + 1]]
            assert np.all(np.diff(seg) > 0)
            toks = [t for t in range(T) if e in idx[t]]     # token-order queue
            keep = toks if C == 0 else toks[:C]
            np.testing.assert_array_equal(seg, keep)
            for t in toks:
                j = int(np.nonzero(idx[t] == e)[0][0])
                assert d["dropped"][t, j] == (t not in keep)
    d1 = oracle.dispatch(idx, E, 1)
    assert np.all(d1["kept"] == np.minimum(d1["counts"], 1))


def test_capacity_at_least_max_count_equals_dropless():
    T, d, E, k, S, F = 48, 16, 6, 2, 1, 8
    w = _inputs(T, d, E, k, S, F, seed=8, bf16=True, logit_std=0.5)
    a = oracle.layer_forward(w["x"], w, _spec(d, E, k, S, F, bf16=True))
    cmax = int(a["counts"].max())
    b = oracle.layer_forward(w["x"], w, _spec(d, E, k, S, F, bf16=True, capacity=cmax))
    for key in ("idx", "counts", "kept", "offsets", "row_of_slot", "sorted_token", "dropped"):
        np.testing.assert_array_equal(a[key], b[key])
    np.testing.assert_array_equal(a["y"], b["y"])
    c = oracle.layer_forward(w["x"], w, _spec(d, E, k, S, F, bf16=True, capacity=cmax - 1))
    assert c["n_dropped"] == int(np.sum(a["counts"] == cmax))


# ---------------------------------------------------------------- reductions
def test_single_expert_is_plain_swiglu():
    T, d, F = 20, 16, 12
    w = _inputs(T, d, 1, 1, 0, F, seed=9)
    out = oracle.layer_forward(w["x"], w, _spec(d, 1, 1, 0, F, bf16=False))
    x = np.asarray(w["x"], np.float64)
    a = x @ w["w_gate"][0]
    want = (a / (1 + np.exp(-a)) * (x @ w["w_up"][0])) @ w["w_down"][0]
    assert _rel(out["y"], want) < 1e-12
    np.testing.assert_array_equal(out["gates"], 1.0)


def test_all_experts_active_is_dense_softmax_mixture():
    T, d, E, F = 15, 12, 5, 8
    w = _inputs(T, d, E, E, 0, F, seed=11)
    for renorm in (True, False):
        out = oracle.layer_forward(w["x"], w, _spec(d, E, E, 0, F, renorm=renorm, bf16=False))
        x = np.asarray(w["x"], np.float64)
        l = x @ w["w_router"]
        p = np.exp(l) / np.exp(l).sum(1, keepdims=True)
        want = np.zeros((T, d))
        for e in range(E):
            a = x @ w["w_gate"][e]
            want += p[:, e:e + 1] * ((a / (1 + np.exp(-a)) * (x @ w["w_up"][e])) @ w["w_down"][e])
        assert _rel(out["y"], want) < 1e-12
        assert np.all(np.isinf(out["margin"]))


def test_zero_routed_down_gives_shared_only():
    T, d, E, k, S, F = 20, 16, 6, 2, 2, 8
    w = _inputs(T, d, E, k, S, F, seed=12, bf16=True)
    w["w_down"] = np.zeros_like(w["w_down"])
    out = oracle.layer_forward(w["x"], w, _spec(d, E, k, S, F, bf16=True))
    x = np.asarray(w["x"], np.float64)
    want = np.zeros((T, d))
    for s in range(S):
        a = x @ w["sh_gate"][s]
        h = np.array([[_brute.bf16_exact(v) for v in row] for row in a / (1 + np.exp(-a)) * (x @ w["sh_up"][s])])
        want += h @ w["sh_down"][s]
    assert _rel(out["y"], want) < 1e-12


def test_lowrank_equals_materialised_dense():
    T, d, E, k, S, F, r = 24, 32, 6, 2, 1, 16, 4
    w = _inputs(T, d, E, k, S, F, seed=13, rank=r)
    out = oracle.layer_forward(w["x"], w, _spec(d, E, k, S, F, rank=r, bf16=False))
    dense = dict(w)

    def mat(u, s, v):
        return np.einsum("eir,er,eor->eio", np.asarray(u, np.float64),
                         np.asarray(s, np.float64), np.asarray(v, np.float64))

    dense["w_gate"] = mat(w["u_gate"], w["s_gate"], w["v_gate"])
    dense["w_up"] = mat(w["u_up"], w["s_up"], w["v_up"])
    dense["w_down"] = mat(w["u_down"], w["s_down"], w["v_down"])
    ref = oracle.layer_forward(w["x"], dense, _spec(d, E, k, S, F, bf16=False))
    assert _rel(out["y"], ref["y"]) < 1e-12


def test_token_permutation_equivariance_dropless():
    T, d, E, k, S, F = 40, 16, 8, 3, 1, 8
    w = _inputs(T, d, E, k, S, F, seed=14, bf16=True)
    spec = _spec(d, E, k, S, F, bf16=True)
    a = oracle.layer_forward(w["x"], w, spec)
    perm = np.random.default_rng(0).permutation(T)
    w2 = dict(w)
    w2["x"] = w["x"][perm]
    b = oracle.layer_forward(w2["x"], w2, spec)
    np.testing.assert_array_equal(b["idx"], a["idx"][perm])
    np.testing.assert_array_equal(b["y"], a["y"][perm])


def test_down_projection_linearity():
    T, d, E, k, S, F = 30, 16, 6, 2, 1, 8
    w = _inputs(T, d, E, k, S, F, seed=15, bf16=True)
    spec = _spec(d, E, k, S, F, bf16=True)
    a = oracle.layer_forward(w["x"], w, spec)
    w2 = dict(w)
    w2["w_down"] = w["w_down"] * 2
    w2["sh_down"] = w["sh_down"] * 2
    b = oracle.layer_forward(w["x"], w2, spec)
    np.testing.assert_array_equal(b["y"], 2 * a["y"])


def test_override_forces_selection():
    T, d, E, k = 10, 8, 6, 2
    w = _inputs(T, d, E, k, 0, 8, seed=16)
    spec = _spec(d, E, k, 0, 8, bf16=False)
    forced = np.tile(np.array([5, 4]), (T, 1))
    mask = np.zeros(T, bool)
    mask[[1, 7]] = True
    r = oracle.route(w["x"], w["w_router"], spec, override_idx=forced, override_mask=mask)
    base = oracle.route(w["x"], w["w_router"], spec)
    np.testing.assert_array_equal(r["idx"][1], [5, 4])
    np.testing.assert_array_equal(r["idx"][~mask], base["idx"][~mask])
    p = base["prob"][1, [5, 4]]
    np.testing.assert_allclose(r["gates"][1], p / p.sum(), rtol=1e-14)


# ---------------------------------------------------------------- page numbers
def test_quartz_parameter_totals_pin_gated_experts():
    """With three d x F matrices per expert (as the oracle's experts take), the
    Quartz architecture reproduces the printed totals; two matrices do not."""
    g = json.load(open(os.path.join(GOLDEN, "quartz_param_counts.json")))
    P = g["printed"]
    d, F = P["hidden"], P["expert_ffn"]
    w = synth.make_inputs(synth.QUARTZ.replace(T=1, hidden=8, ffn=8))   # key names only
    expert_mats = [k for k in ("w_gate", "w_up", "w_down") if k in w]
    per_expert = len(expert_mats) * d * F
    hd = P["head_dim"]
    attn = d * P["query_heads"] * hd * 2 + d * P["kv_heads"] * hd * 2
    norms = 2 * d * P["layers"] + d
    dense_ffn = 3 * d * g["inferred_not_printed"]["dense_ffn_width"]
    router = d * P["routed_experts"]
    n_moe = P["layers"] - P["dense_layers"]
    emb = P["vocab"] * d
    common = emb + attn * P["layers"] + norms + dense_ffn * P["dense_layers"]
    total = common + n_moe * ((P["routed_experts"] + P["shared_experts"]) * per_expert + router)
    active = common + n_moe * ((P["active_routed"] + P["shared_experts"]) * per_expert + router)
    assert round(total / 1e6, 1) == P["total_params_millions"]
    assert round(active / 1e6, 1) == P["active_params_per_token_millions"]
    two = common + n_moe * ((P["routed_experts"] + P["shared_experts"]) * 2 * d * F + router)
    assert round(two / 1e6, 1) != P["total_params_millions"]


# ---------------------------------------------------------------- bias update
def test_bias_update_closed_forms():
    """Balanced counts leave the bias unchanged; above-mean experts move down
    by exactly gamma, below-mean up, at-mean not at all (integer comparison:
    here T k / E = 3 exactly)."""
    T, k, E = 12, 2, 8                    # mean slots per expert: 3
    b = np.array([0.25, -0.5, 0.0, 1.0, 0.125, -2.0, 0.75, 3.0], np.float32)
    g = np.float32(0.03125)               # a power of two: every result is exact
    same = oracle.bias_update(b, np.full(E, 3), T, k, g)
    np.testing.assert_array_equal(same, b)
    counts = np.array([9, 0, 3, 4, 2, 3, 1, 2])
    assert counts.sum() == T * k
    out = oracle.bias_update(b, counts, T, k, g)
    want = b + g * np.array([-1, 1, 0, -1, 1, 0, 1, 1], np.float32)
    np.testing.assert_array_equal(out, want)
    assert out.dtype == np.float32


def test_bias_update_rounds_once_in_float32():
    """The result is the float32 addition b + gamma (or b - gamma)."""
    rng = np.random.default_rng(1)
    b = rng.standard_normal(64).astype(np.float32)
    counts = rng.integers(0, 40, 64)
    T, k = 100, 8
    g = np.float32(1e-3)
    out = oracle.bias_update(b, counts, T, k, g)
    d = np.sign(T * k - 64 * counts.astype(np.int64))
    want = np.where(d > 0, b + g, np.where(d < 0, b - g, b)).astype(np.float32)
    np.testing.assert_array_equal(out, want)


def test_bias_update_balances_a_skewed_router():
    """Repeated updates on a router with a strong per-expert offset drive the
    per-expert loads toward the mean; the reverse sign would drive them apart."""
    T, d, E, k = 256, 16, 8, 2
    w = _inputs(T, d, E, k, 0, 8, seed=11, score="sigmoid")
    spec = _spec(d, E, k, 0, 8, score="sigmoid", bf16=False)
    logit_bias = -1.5 * np.log(np.arange(E) + 1.0)      # Zipf-like skew by expert id

    def max_over_mean(bias):
        r = oracle.route(w["x"], w["w_router"], spec, logit_bias, bias)
        c = np.bincount(r["idx"].ravel(), minlength=E)
        return c.max() / (T * k / E), c

    bias = np.zeros(E, np.float32)
    start, _ = max_over_mean(bias)
    for _ in range(150):
        _, c = max_over_mean(bias)
        bias = oracle.bias_update(bias, c, T, k, 0.02)
    end, _ = max_over_mean(bias)
    assert start > 2.5
    assert end < 1.4, (start, end)

    flipped = np.zeros(E, np.float32)
    for _ in range(20):
        _, c = max_over_mean(flipped)
        flipped = 2 * flipped - oracle.bias_update(flipped, c, T, k, 0.02)   # opposite sign
    worse, _ = max_over_mean(flipped)
    assert worse >= start


# ---------------------------------------------------------------- backward
def _f64(w):
    return {n: (None if v is None else np.asarray(v, np.float64)) for n, v in w.items()}


def _loss(x, w, spec, dy, aux_grad, idx):
    """sum(dy * y) + aux_grad * aux with the selection held at idx."""
    T = x.shape[0]
    f = oracle.layer_forward(x, w, spec, override_idx=idx, override_mask=np.ones(T, bool))
    return float(np.sum(dy * f["y"])) + aux_grad * f["aux"]


def _fd_grad(fn, arr, h=1e-6):
    g = np.zeros(arr.shape)
    it = np.nditer(arr, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        keep = arr[i]
        arr[i] = keep + h
        lp = fn()
        arr[i] = keep - h
        lm = fn()
        arr[i] = keep
        g[i] = (lp - lm) / (2 * h)
    return g


BWD_CASES = [
    # T, d, E, k, S, F, score, renorm, capacity
    (5, 6, 4, 2, 1, 3, "softmax", True, 0),
    (6, 5, 5, 3, 0, 4, "softmax", False, 0),
    (5, 4, 6, 2, 2, 3, "sigmoid", True, 0),
    (8, 4, 3, 2, 1, 3, "softmax", True, 3),     # capacity drops some slots
]


@pytest.mark.parametrize("case", BWD_CASES)
def test_backward_matches_finite_differences(case):
    """Every gradient the backward returns agrees with central differences of
    the forward oracle, selection held fixed, in float64 (rho = identity)."""
    T, d, E, k, S, F, score, renorm, cap = case
    w = _inputs(T, d, E, k, S, F, seed=40 + T, score=score, logit_std=0.5,
                select_std=0.2 if score == "sigmoid" else 0.0)
    w = _f64(w)
    spec = _spec(d, E, k, S, F, score=score, renorm=renorm, capacity=cap, bf16=False,
                 aux_coef=0.05)
    x = w.pop("x")
    rng = np.random.default_rng(7)
    dy = rng.standard_normal((T, d))
    aux_grad = 1.7
    base = oracle.layer_forward(x, w, spec)
    if cap:
        assert base["n_dropped"] > 0
    idx = base["idx"]
    g = oracle.layer_backward(x, w, spec, dy, aux_grad=aux_grad)
    fn = lambda: _loss(x, w, spec, dy, aux_grad, idx)
    assert _rel(g["dx"], _fd_grad(fn, x)) < 1e-7
    assert _rel(g["dw_router"], _fd_grad(fn, w["w_router"])) < 1e-7
    for name, key in (("dw_gate", "w_gate"), ("dw_up", "w_up"), ("dw_down", "w_down")):
        assert _rel(g[name], _fd_grad(fn, w[key])) < 1e-7, name
    if S:
        for name, key in (("dsh_gate", "sh_gate"), ("dsh_up", "sh_up"), ("dsh_down", "sh_down")):
            assert _rel(g[name], _fd_grad(fn, w[key])) < 1e-7, name


LR_BWD_CASES = [
    # T, d, E, k, S, F, r, score, renorm, capacity
    (5, 6, 4, 2, 0, 5, 3, "softmax", False, 0),
    (6, 5, 3, 2, 1, 4, 2, "softmax", True, 0),
    (5, 4, 5, 2, 0, 3, 2, "sigmoid", True, 0),
    (8, 4, 3, 2, 0, 3, 2, "softmax", True, 3),     # capacity drops some slots
]


@pytest.mark.parametrize("case", LR_BWD_CASES)
def test_lowrank_backward_matches_finite_differences(case):
    """Rank-r experts: every factor gradient (U, s, V of gate, up and down),
    dx and dW_r against central differences of the forward oracle, selection
    held fixed, in float64 (rho = identity)."""
    T, d, E, k, S, F, r, score, renorm, cap = case
    w = _f64(_inputs(T, d, E, k, S, F, seed=80 + T, rank=r, score=score, logit_std=0.5,
                     select_std=0.2 if score == "sigmoid" else 0.0))
    spec = _spec(d, E, k, S, F, rank=r, score=score, renorm=renorm, capacity=cap, bf16=False,
                 aux_coef=0.05)
    x = w.pop("x")
    dy = np.random.default_rng(9).standard_normal((T, d))
    base = oracle.layer_forward(x, w, spec)
    if cap:
        assert base["n_dropped"] > 0
    g = oracle.layer_backward(x, w, spec, dy, aux_grad=1.3)
    fn = lambda: _loss(x, w, spec, dy, 1.3, base["idx"])
    assert _rel(g["dx"], _fd_grad(fn, x)) < 1e-7
    assert _rel(g["dw_router"], _fd_grad(fn, w["w_router"])) < 1e-7
    for name in oracle.LOWRANK_GRADS:
        assert _rel(g[name], _fd_grad(fn, w[name[1:]])) < 1e-7, name
    if S:
        for name, key in (("dsh_gate", "sh_gate"), ("dsh_up", "sh_up"), ("dsh_down", "sh_down")):
            assert _rel(g[name], _fd_grad(fn, w[key])) < 1e-7, name


def test_lowrank_backward_equals_the_dense_backward_of_the_product():
    """With rho = identity a rank-r expert is the dense expert W = U diag(s) V^T,
    so its factor gradients follow from the dense backward's dW:
    dU = dW V diag(s), ds = diag(U^T dW V), dV = dW^T U diag(s); dx and dW_r
    are the dense ones."""
    T, d, E, k, S, F, r = 12, 10, 5, 2, 1, 7, 4
    w = _f64(_inputs(T, d, E, k, S, F, seed=5, rank=r, logit_std=0.4))
    x = w.pop("x")
    spec = _spec(d, E, k, S, F, rank=r, bf16=False)
    dense = {n: v for n, v in w.items() if not n[:2] in ("u_", "s_", "v_")}
    for m, (din, dout) in (("gate", (d, F)), ("up", (d, F)), ("down", (F, d))):
        dense["w_" + m] = np.stack([w["u_" + m][e] @ np.diag(w["s_" + m][e]) @ w["v_" + m][e].T
                                    for e in range(E)])
    dy = np.random.default_rng(2).standard_normal((T, d))
    g = oracle.layer_backward(x, w, spec, dy, aux_grad=0.9)
    h = oracle.layer_backward(x, dense, _spec(d, E, k, S, F, bf16=False), dy, aux_grad=0.9)
    assert _rel(g["dx"], h["dx"]) < 1e-12 and _rel(g["dw_router"], h["dw_router"]) < 1e-12
    for m in ("gate", "up", "down"):
        U, s_, V, dW = w["u_" + m], w["s_" + m], w["v_" + m], h["dw_" + m]
        du = np.stack([dW[e] @ V[e] * s_[e][None, :] for e in range(E)])
        ds = np.stack([np.einsum("ci,cf,fi->i", U[e], dW[e], V[e]) for e in range(E)])
        dv = np.stack([dW[e].T @ U[e] * s_[e][None, :] for e in range(E)])
        assert _rel(g["du_" + m], du) < 1e-12, m
        assert _rel(g["ds_" + m], ds) < 1e-12, m
        assert _rel(g["dv_" + m], dv) < 1e-12, m


@pytest.mark.parametrize("case", LR_BWD_CASES)
@pytest.mark.parametrize("bf16", [False, True])
def test_lowrank_batched_backward_equals_token_loop(case, bf16):
    """The per-expert batched low-rank backward (full-size checks) gives the
    token loop's gradients, with the same bf16 rounding points."""
    T, d, E, k, S, F, r, score, renorm, cap = case
    w = _f64(_inputs(T + 20, d + 4, E, k, S, F + 8, seed=90 + T, rank=r, score=score,
                     logit_std=0.5, select_std=0.2 if score == "sigmoid" else 0.0))
    spec = _spec(d + 4, E, k, S, F + 8, rank=r, score=score, renorm=renorm, capacity=cap,
                 bf16=bf16, aux_coef=0.05)
    x = w.pop("x")
    dy = np.random.default_rng(3).standard_normal((T + 20, d + 4))
    a = oracle.layer_backward(x, w, spec, dy, aux_grad=1.1)
    b = oracle.layer_backward_batched(x, w, spec, dy, aux_grad=1.1)
    names = ["dx", "dw_router", *oracle.LOWRANK_GRADS]
    if S:
        names += ["dsh_gate", "dsh_up", "dsh_down"]
    for n in names:
        assert _rel(b[n], a[n]) < 1e-10, n
        assert np.all(b["S_" + n] >= np.abs(b[n]) * (1 - 1e-12)), n
        assert np.all(b["B_" + n] >= 0), n


def test_lowrank_backward_bf16_rounding_points_are_small_perturbations():
    """The bf16 rounding points move the low-rank gradients by rounding-level
    amounts only (against the same layer with rho = identity)."""
    T, d, E, k, S, F, r = 30, 64, 6, 2, 0, 48, 16
    w = _inputs(T, d, E, k, S, F, seed=12, rank=r, bf16=True, logit_std=0.3)
    x = w.pop("x")
    dy = np.random.default_rng(4).standard_normal((T, d))
    g1 = oracle.layer_backward_batched(x, w, _spec(d, E, k, S, F, rank=r, bf16=True), dy)
    g0 = oracle.layer_backward_batched(x, w, _spec(d, E, k, S, F, rank=r, bf16=False), dy)
    for n in ["dx", *oracle.LOWRANK_GRADS]:
        rel = _rel(g1[n], g0[n])
        assert 0 < rel < 5e-2, (n, rel)


def test_backward_aux_term_alone():
    """With dy = 0 only the aux statistic carries gradient: the expert weights
    get none, and the router gradient matches differences of aux alone."""
    T, d, E, k, S, F = 7, 5, 4, 2, 1, 3
    w = _f64(_inputs(T, d, E, k, S, F, seed=3, logit_std=0.4))
    spec = _spec(d, E, k, S, F, bf16=False, aux_coef=0.1)
    x = w.pop("x")
    dy = np.zeros((T, d))
    g = oracle.layer_backward(x, w, spec, dy, aux_grad=1.0)
    for name in ("dw_gate", "dw_up", "dw_down", "dsh_gate", "dsh_up", "dsh_down"):
        assert not np.any(g[name]), name
    assert np.any(g["dw_router"])
    idx = oracle.layer_forward(x, w, spec)["idx"]
    fn = lambda: _loss(x, w, spec, dy, 1.0, idx)
    assert _rel(g["dw_router"], _fd_grad(fn, w["w_router"])) < 1e-7


def test_backward_single_expert_is_textbook_swiglu():
    """E = 1, k = 1, no shared expert, no aux: the layer is one SwiGLU MLP with
    gate one, so its gradients are those torch autograd gives for
    SiLU(x Wg) * (x Wu) Wd, and the router gets none."""
    T, d, F = 6, 5, 7
    w = _f64(_inputs(T, d, 1, 1, 0, F, seed=11))
    spec = _spec(d, 1, 1, 0, F, bf16=False)
    x = w.pop("x")
    dy = np.random.default_rng(1).standard_normal((T, d))
    g = oracle.layer_backward(x, w, spec, dy, aux_grad=0.0)
    xt = torch.tensor(x, requires_grad=True)
    wg = torch.tensor(w["w_gate"][0], requires_grad=True)
    wu = torch.tensor(w["w_up"][0], requires_grad=True)
    wd = torch.tensor(w["w_down"][0], requires_grad=True)
    y = (torch.nn.functional.silu(xt @ wg) * (xt @ wu)) @ wd
    (y * torch.tensor(dy)).sum().backward()
    assert _rel(g["dx"], xt.grad.numpy()) < 1e-12
    assert _rel(g["dw_gate"][0], wg.grad.numpy()) < 1e-12
    assert _rel(g["dw_up"][0], wu.grad.numpy()) < 1e-12
    assert _rel(g["dw_down"][0], wd.grad.numpy()) < 1e-12
    assert not np.any(g["dw_router"])


def test_backward_bf16_rounding_points_are_small_perturbations():
    """Rounding the expert-product operands to bf16 moves each gradient by
    rounding-level amounts only (a misplaced rho on a whole tensor, or a
    missing gate, would move it by O(1))."""
    T, d, E, k, S, F = 12, 16, 6, 2, 1, 8
    w = _f64(_inputs(T, d, E, k, S, F, seed=5, logit_std=0.5))
    x = w.pop("x")
    dy = np.random.default_rng(2).standard_normal((T, d))
    g64 = oracle.layer_backward(x, w, _spec(d, E, k, S, F, bf16=False), dy, aux_grad=0.3)
    g16 = oracle.layer_backward(x, w, _spec(d, E, k, S, F, bf16=True), dy, aux_grad=0.3)
    for name in ("dx", "dw_router", "dw_gate", "dw_up", "dw_down", "dsh_gate", "dsh_up",
                 "dsh_down"):
        r = _rel(g16[name], g64[name])
        assert 0 < r < 3e-2, (name, r)


def test_backward_error_scales_bound_the_gradients():
    """M (largest term) and S (sum of term magnitudes) satisfy
    |C| <= S, M <= S <= n M for a sum of n terms; a one-token, one-expert layer
    has single-term weight gradients, where M = S = |C|."""
    T, d, E, k, S_, F = 9, 6, 4, 2, 1, 5
    w = _f64(_inputs(T, d, E, k, S_, F, seed=21, logit_std=0.3))
    x = w.pop("x")
    spec = _spec(d, E, k, S_, F, bf16=True)
    dy = np.random.default_rng(4).standard_normal((T, d))
    g = oracle.layer_backward(x, w, spec, dy, aux_grad=0.5, scales=True)
    for name in ("dx", "dw_router", "dw_gate", "dw_up", "dw_down", "dsh_gate", "dsh_up",
                 "dsh_down"):
        c, m, s = g[name], g["M_" + name], g["S_" + name]
        assert np.all(np.abs(c) <= s * (1 + 1e-12) + 1e-300), name
        assert np.all(m <= s * (1 + 1e-12)), name
        assert np.all(s <= T * 64 * m + 1e-300), name
    w1 = _f64(_inputs(1, d, 1, 1, 0, F, seed=22))
    x1 = w1.pop("x")
    g1 = oracle.layer_backward(x1, w1, _spec(d, 1, 1, 0, F, bf16=False), dy[:1], scales=True)
    for name in ("dw_gate", "dw_up", "dw_down"):
        np.testing.assert_allclose(g1["M_" + name], np.abs(g1[name]), rtol=1e-12)
        np.testing.assert_allclose(g1["S_" + name], np.abs(g1[name]), rtol=1e-12)


@pytest.mark.parametrize("case", BWD_CASES)
@pytest.mark.parametrize("bf16", [False, True])
def test_batched_backward_equals_token_loop(case, bf16):
    """The per-expert batched backward (full-size checks) gives the token
    loop's gradients and error sums S, and bounds its largest terms M."""
    T, d, E, k, S, F, score, renorm, cap = case
    w = _f64(_inputs(T, d, E, k, S, F, seed=60 + T, score=score, logit_std=0.5,
                     select_std=0.2 if score == "sigmoid" else 0.0))
    spec = _spec(d, E, k, S, F, score=score, renorm=renorm, capacity=cap, bf16=bf16,
                 aux_coef=0.05)
    x = w.pop("x")
    dy = np.random.default_rng(8).standard_normal((T, d))
    a = oracle.layer_backward(x, w, spec, dy, aux_grad=1.3, scales=True)
    b = oracle.layer_backward_batched(x, w, spec, dy, aux_grad=1.3)
    names = ["dx", "dw_router", "dw_gate", "dw_up", "dw_down"]
    if S:
        names += ["dsh_gate", "dsh_up", "dsh_down"]
    for n in names:
        assert _rel(b[n], a[n]) < 1e-10, n
        assert _rel(b["S_" + n], a["S_" + n]) < 1e-10, n
        assert np.all(b["B_" + n] >= a["M_" + n] * (1 - 1e-12)), n


# ---------------------------------------------------------------- fp8 (E4M3)
def _e4m3_codes():
    """Every finite E4M3 value from the bit layout, by brute enumeration."""
    vals = []
    for c in range(256):
        sgn, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            continue
        v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        vals.append((-v if sgn else v, c))
    return vals


def test_e4m3_round_matches_torch_on_every_bf16_value():
    bits = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    v = bits[np.isfinite(bits) & (np.abs(bits) <= 448)].astype(np.float64)
    ours = oracle.e4m3_round(v)
    ref = torch.tensor(v, dtype=torch.float32).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_e4m3_round_is_nearest_with_ties_to_even():
    codes = _e4m3_codes()
    pos = sorted({abs(v) for v, _ in codes})
    assert len(pos) == 127 and pos[-1] == 448.0 and pos[1] == 2.0 ** -9
    grid = np.array(pos)
    rng = np.random.default_rng(0)
    mids = (grid[:-1] + grid[1:]) / 2
    v = np.concatenate([mids, -mids, rng.uniform(-448, 448, 5000),
                        rng.uniform(-1, 1, 5000) * 2.0 ** -5])
    q = oracle.e4m3_round(v)
    code_of = {val: c for val, c in codes if val >= 0}
    for x, y in zip(v, q):
        d = np.abs(grid - abs(x))
        best = grid[d == d.min()]
        if len(best) == 2:   # tie: the even code (even mantissa)
            best = [b for b in best if code_of[b] % 2 == 0]
        assert abs(y) == best[0] and (y == 0 or (x > 0) == (y > 0))


def test_fp8_scale_rule():
    s = oracle.fp8_scale_exp
    assert s(448.0) == 0 and s(448.0 * 2 ** -5) == -5 and s(449.0) == 1 and s(0.0) == 0
    assert s(1.0) == -8 and s(0.875) == -9 and s(2.0 ** -20) == -28
    rng = np.random.default_rng(1)
    amax = np.exp(rng.uniform(-30, 30, 2000))
    e = s(amax)
    assert np.all(np.ldexp(amax, -e) <= 448.0)          # fits
    assert np.all(np.ldexp(amax, -(e - 1)) > 448.0)     # and is the smallest that fits


def test_fp8_quantize_error_and_exact_cases():
    rng = np.random.default_rng(2)
    m = rng.standard_normal((40, 30)) * np.exp(rng.uniform(-5, 5, (1, 30)))
    q, s = oracle.fp8_quantize(m, axis=0)
    assert s.shape == (30,)
    scale = np.ldexp(1.0, s)[None, :]
    # relative error <= 2^-4 where normal, absolute <= 2^-10 scale where subnormal
    err = np.abs(q - m)
    assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(m), 2.0 ** -10 * scale) * (1 + 1e-12))
    assert np.all(np.abs(q) <= 448 * scale)
    # values already on the grid (with a column maximum that keeps the scale) stay
    grid = np.array(sorted({abs(v) for v, _ in _e4m3_codes()}))
    g = rng.choice(grid, (20, 6)) * rng.choice([-1, 1], (20, 6))
    g[0] = 448.0
    g = np.ldexp(g, np.array([-12, -3, 0, 2, 5, 9])[None, :])
    np.testing.assert_array_equal(oracle.fp8_quantize(g, axis=0)[0], g)


@pytest.mark.parametrize("S", [1, 2])
def test_fp8_layer_reduces_to_quantised_h_on_grid_inputs(S):
    """With x rows and weight columns already on their E4M3 grids (scales
    preserved), the fp8 layer is the bf16 layer with h quantised; h's
    quantisation here goes through torch's float8_e4m3fn. With two shared
    experts the second one's h is made about 2^16 times larger than the
    first's, so under the shared h row's one joint scale (the S experts form
    one product over their stacked S F rows) the first expert's h falls into
    E4M3's subnormal range, far coarser than under a scale of its own: the
    check tells the two readings apart (E4M3 is a floating-point grid, so a
    smaller ratio would leave the first expert's codes unchanged)."""
    T, d, E, k, F = 6, 32, 4, 2, 16
    rng = np.random.default_rng(3)
    grid = np.array(sorted({abs(v) for v, _ in _e4m3_codes()}))
    def ongrid(shape, sc):
        a = rng.choice(grid[grid <= 240], shape) * rng.choice([-1, 1], shape)
        return np.ldexp(a, sc)
    x = ongrid((T, d), 0)
    x[:, 0] = 448.0                       # every row's scale is 1
    w = _inputs(T, d, E, k, S, F, seed=4, bf16=True)
    for n in ("w_gate", "w_up", "w_down", "sh_gate", "sh_up", "sh_down"):
        a = ongrid(w[n].shape, -9)
        a[..., 0, :] = 448.0 * 2.0 ** -9  # every column's scale is 2^-9
        w[n] = a
    if S == 2:
        # the second shared expert's gate and up columns 2^8 larger (scale
        # 2^-1, still on their grids): its h is ~2^16 times the first's
        w["sh_gate"][1] *= 256.0
        w["sh_up"][1] *= 256.0
    w["x"] = x
    spec8 = _spec(d, E, k, S, F, bf16=True, fp8=True)
    got = oracle.layer_forward(x, w, spec8)
    ref = oracle.layer_forward(x, w, _spec(d, E, k, S, F, bf16=True), tokens=[])
    rho = oracle.round_bf16
    def q_torch(h):
        s = oracle.fp8_scale_exp(np.max(np.abs(h)))
        t = torch.tensor(np.ldexp(h, -s), dtype=torch.float32).to(torch.float8_e4m3fn)
        return np.ldexp(t.to(torch.float64).numpy(), s)
    y = np.zeros((T, d))
    y_apart = np.zeros((T, d))         # the other reading: one scale per shared expert
    for t in range(T):
        hs = [rho(oracle.silu(x[t] @ w["sh_gate"][s_]) * (x[t] @ w["sh_up"][s_]))
              for s_ in range(S)]
        y[t] = q_torch(np.concatenate(hs)) @ w["sh_down"].reshape(S * F, d)
        y_apart[t] = np.concatenate([q_torch(h) for h in hs]) @ w["sh_down"].reshape(S * F, d)
        for j in range(k):
            e = int(ref["idx"][t, j])
            h = rho(oracle.silu(x[t] @ w["w_gate"][e]) * (x[t] @ w["w_up"][e]))
            yr = ref["gates"][t, j] * (q_torch(h) @ w["w_down"][e])
            y[t] += yr
            y_apart[t] += yr
    np.testing.assert_allclose(got["y"], y, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.layer_forward_batched(x, w, spec8)["y"], y,
                               rtol=1e-12, atol=1e-12)
    if S == 2:
        # the readings differ by far more than the tolerance of the check above
        assert np.max(np.abs(y_apart - y)) > 1e6 * 1e-12 * np.max(np.abs(y))


def test_fp8_term_maxima_bound_the_output():
    """M_y (the largest single down-product term of each output element) is
    positive and bounds y by the term count: |y| <= (k + S) F M_y."""
    T, d, E, k, S, F = 7, 32, 4, 2, 2, 16
    w = _inputs(T, d, E, k, S, F, seed=9, bf16=True)
    spec = _spec(d, E, k, S, F, bf16=True, fp8=True)
    f = oracle.layer_forward(w["x"], w, spec, scales=True)
    assert f["M_y"].shape == f["y"].shape and np.all(f["M_y"] > 0)
    assert np.all(np.abs(f["y"]) <= (k + S) * F * f["M_y"] * (1 + 1e-12))
    g = oracle.layer_forward(w["x"], w, spec)
    np.testing.assert_array_equal(g["y"], f["y"])


def test_fp8_lowrank_factors_are_the_bf16_layer_on_quantised_factors():
    """fp8 low-rank experts: the bf16 low-rank layer evaluated on factors
    quantised by the stated rule (U per column, V per row), which equals the
    scales folded where the kernel applies them: U's into s, V's onto the
    product's output columns."""
    T, d, E, k, S, F, r = 5, 64, 4, 2, 0, 64, 64
    w = _inputs(T, d, E, k, S, F, seed=31, rank=r, bf16=True)
    spec8 = _spec(d, E, k, S, F, rank=r, bf16=True, fp8=True)
    got = oracle.layer_forward(w["x"], w, spec8)
    wq = dict(w)
    for n in ("u_gate", "u_up", "u_down"):
        wq[n] = np.stack([oracle.fp8_quantize(np.asarray(w[n][e], np.float64), 0)[0]
                          for e in range(E)])
    for n in ("v_gate", "v_up", "v_down"):
        wq[n] = np.stack([oracle.fp8_quantize(np.asarray(w[n][e], np.float64), 1)[0]
                          for e in range(E)])
    ref = oracle.layer_forward(w["x"], wq, _spec(d, E, k, S, F, rank=r, bf16=True))
    np.testing.assert_array_equal(got["y"], ref["y"])
    # folding: (x U_q 2^su) * s = (x U_q) * (s 2^su) exactly; V's scale per output
    e = 1
    u, su = oracle.fp8_quantize(np.asarray(w["u_gate"][e], np.float64), 0)
    v, sv = oracle.fp8_quantize(np.asarray(w["v_gate"][e], np.float64), 1)
    uq, vq = np.ldexp(u, -su[None, :]), np.ldexp(v, -sv[:, None])
    assert np.all(np.abs(uq) <= 448) and np.all(np.abs(vq) <= 448)
    xr = np.asarray(w["x"][0], np.float64)
    np.testing.assert_array_equal((xr @ u) * w["s_gate"][e],
                                  (xr @ uq) * (np.asarray(w["s_gate"][e], np.float64) * np.ldexp(1.0, su)))
