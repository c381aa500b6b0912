"""HIP path vs the CPU oracle on the same seeded inputs, through the C ABI.

Small shapes (several tiles and ragged tails), the five workloads at full
size, edge cases, determinism, and the stage entry points against the
whole-layer entry point. Every output element of every case is checked: y
against the oracle's per-expert batched form, routing on every token.
"""
import numpy as np
import pytest
import torch

import oracle

from fine_grained_mixture_amd import layer as L
from fine_grained_mixture_amd import synth
from fine_grained_mixture_amd._lib import MOE_GROUPS_ROUTED, MOE_GROUPS_SHARED
from tests import _parity as P

pytestmark = pytest.mark.gpu


def _run_and_check(wl, **kw):
    print(f"\n[case] {wl}", flush=True)
    inp = synth.make_inputs(wl)
    g = P.run_gpu(wl, inp)
    rep = P.check_parity(wl, inp, g, **kw)
    print(f"[report] {wl.name} T={wl.T}: {rep}", flush=True)
    return rep


SMALL = {
    "tiny": synth.TINY,
    "tiny_ragged": synth.TINY.replace(T=77, seed=1),
    "quartz_small": synth.QUARTZ.replace(T=517, hidden=256, ffn=128),
    "moonfrost_small": synth.MOONFROST.replace(T=1000, hidden=256, ffn=128),
    "moonfrost_small_renorm": synth.MOONFROST.replace(T=1000, hidden=256, ffn=128, renorm=1),
    "sutra_small": synth.SUTRA.replace(T=700, hidden=384, ffn=192),
    "dormouse_small": synth.DORMOUSE.replace(T=600, hidden=256, ffn=128),
    "dormouse_small_renorm": synth.DORMOUSE.replace(T=600, hidden=256, ffn=128, renorm=1),
    # ranks below 64: the kernel's rank-64 tiles with the factor entries past r read as zero
    "dormouse_small_rank16": synth.DORMOUSE.replace(T=300, hidden=192, ffn=320, rank=16, seed=3),
    "dormouse_small_rank32": synth.DORMOUSE.replace(T=420, hidden=256, ffn=128, rank=32,
                                                    n_shared=1, seed=4),
    "dormouse_small_rank48": synth.DORMOUSE.replace(T=500, hidden=128, ffn=192, rank=48, seed=5),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_parity(name):
    _run_and_check(SMALL[name])


EDGE = {
    "single_expert": synth.Workload("e1", T=130, hidden=128, n_routed=1, top_k=1, n_shared=0,
                                    ffn=64),
    "all_experts_active": synth.Workload("ek", T=150, hidden=128, n_routed=4, top_k=4,
                                         n_shared=1, ffn=64, renorm=0),
    "capacity_one": synth.QUARTZ.replace(T=200, hidden=128, ffn=64, capacity_factor="1/200"),
    "capacity_large": synth.MOONFROST.replace(T=300, hidden=128, ffn=64, capacity_factor="10"),
    "no_shared_sigmoid": synth.SUTRA.replace(T=333, hidden=128, ffn=64, n_shared=0),
    "one_token": synth.QUARTZ.replace(T=1, hidden=128, ffn=64),
    "odd_experts": synth.Workload("odd", T=257, hidden=192, n_routed=13, top_k=3, n_shared=3,
                                  ffn=192, logit_offset_std=0.3),
    "many_experts_k8": synth.Workload("k8", T=190, hidden=128, n_routed=300, top_k=8,
                                      n_shared=1, ffn=64, renorm=0),
    "tiny_f32_capacity": synth.TINY.replace(T=200, capacity_factor="1/2", seed=3),
    # rank-64 experts under extreme skew (one expert takes almost every token,
    # 24 row chunks) and under capacity drops
    "lowrank_zipf_skew": synth.DORMOUSE.replace(T=1500, hidden=256, ffn=128, zipf_s=1.1, seed=11),
    "lowrank_capacity": synth.DORMOUSE.replace(T=900, hidden=128, ffn=128, capacity_factor="3/2",
                                               logit_offset_std=0.5, seed=13),
    # 3000 experts: the top-k workgroup's probability sums take the one-row LDS path
    "experts_3000": synth.Workload("e3000", T=100, hidden=128, n_routed=3000, top_k=4,
                                   n_shared=0, ffn=64, seed=14),
    # 520 to 1,000 experts (the top-k kernel with 16 experts per lane, the
    # last lanes partly past E): sigmoid keys with a selection bias beside a
    # shared expert; k = 15 with capacity drops and a last routing block of
    # one token; a single token at the Dormouse expert count
    "experts_1000_sigmoid_k7": synth.Workload("w7", T=300, hidden=128, n_routed=1000, top_k=7,
                                             n_shared=1, ffn=64, score="sigmoid", renorm=1,
                                             select_bias_std=0.1, seed=15),
    "experts_520_k15_capacity": synth.Workload("w15", T=129, hidden=192, n_routed=520,
                                               top_k=15, n_shared=0, ffn=64, renorm=0,
                                               capacity_factor="1", logit_offset_std=0.3,
                                               seed=16),
    "experts_1024_one_token": synth.DORMOUSE.replace(T=1, hidden=256, ffn=128, seed=17),
    # many experts, two active: routing blocks of one 64-slot chunk, with drops
    "many_experts_k2_capacity": synth.Workload("mc", T=333, hidden=128, n_routed=128, top_k=2,
                                               n_shared=0, ffn=64, capacity_factor="3/2",
                                               logit_offset_std=0.5),
}


# exact ties: a zero router leaves the logits equal to an integer-valued bias
# (few distinct values, so most experts tie with others); the selection is
# then the k largest biases with lower expert ids first among equals, in that
# order, the same for every token. The many-expert cases take the top-k
# kernel's tie path in every round.
TIES = {
    "many_softmax": synth.Workload("tie_m", T=150, hidden=128, n_routed=300, top_k=5,
                                   n_shared=0, ffn=64, renorm=1),
    "many_softmax_k15": synth.Workload("tie_k", T=70, hidden=128, n_routed=100, top_k=15,
                                       n_shared=0, ffn=64, renorm=0),
    "many_sigmoid": synth.Workload("tie_s", T=150, hidden=128, n_routed=200, top_k=6,
                                   n_shared=0, ffn=64, score="sigmoid", renorm=1),
    "few_softmax": synth.Workload("tie_f", T=150, hidden=128, n_routed=24, top_k=6,
                                  n_shared=0, ffn=64, renorm=1),
    # 600 and 1,024 experts
    "wide_softmax": synth.Workload("tie_w", T=100, hidden=128, n_routed=1024, top_k=4,
                                   n_shared=0, ffn=64, renorm=1),
    "wide_sigmoid_k15": synth.Workload("tie_ws", T=70, hidden=128, n_routed=600, top_k=15,
                                       n_shared=0, ffn=64, score="sigmoid", renorm=1),
}


@pytest.mark.parametrize("name", list(TIES))
def test_exact_ties_take_lower_ids(name):
    wl = TIES[name]
    print(f"\n[case] ties {wl}", flush=True)
    inp = synth.make_inputs(wl)
    inp["w_router"] = np.zeros_like(inp["w_router"])
    bias = np.random.default_rng(17).integers(-2, 3, size=wl.n_routed).astype(np.float32)
    if wl.score == "sigmoid":
        inp["select_bias"] = bias
    else:
        inp["logit_bias"] = bias
    g = P.run_gpu(wl, inp)
    order = np.argsort(-bias, kind="stable")[:wl.top_k]
    np.testing.assert_array_equal(g["topk_idx"], np.broadcast_to(order, (wl.T, wl.top_k)))
    r0 = oracle.route(inp["x"], inp["w_router"], P.spec_of(wl), inp.get("logit_bias"),
                      inp.get("select_bias"))
    np.testing.assert_array_equal(g["topk_idx"], r0["idx"])
    np.testing.assert_allclose(g["topk_gate"], r0["gates"], rtol=0, atol=1e-6)


# decode-sized batches (T <= 4 take the weight-streaming skinny expert kernel,
# T = 1 with only k + S experts busy, T <= 2 with 512 threads where K > 512;
# the larger ones check the tile kernel at few rows per expert)
DECODE = {
    "quartz_t1": synth.QUARTZ.replace(T=1, seed=4),
    "quartz_t2": synth.QUARTZ.replace(T=2, seed=5),
    "sutra_t1": synth.SUTRA.replace(T=1, seed=17),
    "sutra_t2": synth.SUTRA.replace(T=2, seed=18),
    # K = 512 for the down product: its 256-thread kernel beside the 512-thread gate/up
    "moonfrost_t2": synth.MOONFROST.replace(T=2, seed=19),
    "quartz_t4": synth.QUARTZ.replace(T=4, seed=10),
    # the first batch past the skinny kernel, and the first with two routing blocks
    "quartz_t5": synth.QUARTZ.replace(T=5, seed=13),
    "quartz_t33": synth.QUARTZ.replace(T=33, seed=14),
    "quartz_t17": synth.QUARTZ.replace(T=17, seed=6),
    "quartz_t64": synth.QUARTZ.replace(T=64, seed=7),
    # tens of rows per expert, softmax and sigmoid
    "quartz_t256": synth.QUARTZ.replace(T=256, seed=15),
    "sutra_t200": synth.SUTRA.replace(T=200, seed=16),
    "sutra_t3": synth.SUTRA.replace(T=3, seed=8),
    "sutra_t9": synth.SUTRA.replace(T=9, seed=8),
    "moonfrost_t40_capacity": synth.MOONFROST.replace(T=40, seed=9),
}


@pytest.mark.parametrize("name", list(DECODE))
def test_decode_parity(name):
    _run_and_check(DECODE[name])


@pytest.mark.parametrize("name", list(EDGE))
def test_edge_parity(name):
    wl = EDGE[name]
    rep = _run_and_check(wl)
    if name == "capacity_one":
        assert wl.capacity == 1 and rep["rows"] <= wl.n_routed


def test_empty_batch():
    wl = synth.QUARTZ.replace(T=0, hidden=128, ffn=64)
    cfg = L.config_from_workload(wl)
    x = torch.empty((0, wl.hidden), dtype=torch.bfloat16, device="cuda")
    inp = synth.make_inputs(wl.replace(T=1))
    w = L.DeviceWeights.from_numpy(inp, cfg, "cuda")
    out = L.allocate_outputs(cfg, 0, "cuda")
    ws = L.allocate_workspace(cfg, 0, "cuda")
    L.layer_forward(cfg, x, w, out, ws)
    torch.cuda.synchronize()
    assert out["counts"].sum().item() == 0
    assert out["offsets"].sum().item() == 0
    assert out["n_dropped"].item() == 0


FULL = {
    "tiny": synth.TINY,
    "quartz": synth.QUARTZ,
    "moonfrost": synth.MOONFROST,
    "moonfrost_renorm": synth.MOONFROST.replace(renorm=1),
    "sutra": synth.SUTRA,
    "dormouse": synth.DORMOUSE,
    "dormouse_renorm": synth.DORMOUSE.replace(renorm=1),
}


@pytest.mark.parametrize("name", list(FULL))
def test_full_size_parity(name):
    """Every one of the T x d outputs against the oracle (and, reported, the
    error against the oracle without bf16 rounding points)."""
    _run_and_check(FULL[name])


def test_determinism_bitwise():
    wl = synth.MOONFROST.replace(T=3000, hidden=256, ffn=128)
    inp = synth.make_inputs(wl)
    a = P.run_gpu(wl, inp, intermediates=False)
    b = P.run_gpu(wl, inp, intermediates=False)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


STAGED = {
    "quartz": synth.QUARTZ.replace(T=700, hidden=256, ffn=128),
    "tiny": synth.TINY.replace(T=150),
    # many experts and low-rank experts: top-k kernel, column scan, one-chunk rank
    "dormouse": synth.DORMOUSE.replace(T=500, hidden=256, ffn=128),
    "dormouse_rank32_shared": synth.DORMOUSE.replace(T=300, hidden=128, ffn=192, rank=32,
                                                     n_shared=1, seed=7),
    # one routing block: the layer call scans and ranks inside the router's launch
    "quartz_decode": synth.QUARTZ.replace(T=4, seed=12),
}


@pytest.mark.parametrize("base", list(STAGED))
def test_stage_entry_points_match_layer(base):
    wl = STAGED[base]
    inp = synth.make_inputs(wl)
    whole = P.run_gpu(wl, inp, y_lowp=True, intermediates=False)
    cfg, x, w = P.upload(wl, inp)
    T = wl.T
    out = L.allocate_outputs(cfg, T, x.device, y_lowp=True)
    ws = L.allocate_workspace(cfg, T, x.device)
    R = max(1, int(L._lib.moe_max_rows(cfg, T)))
    x_perm = torch.empty((R, wl.hidden), dtype=x.dtype, device=x.device)
    y_routed = torch.empty((R, wl.hidden), dtype=torch.float32, device=x.device)
    y_shared = torch.empty((T, wl.hidden), dtype=torch.float32, device=x.device)
    L.route(cfg, x, w, out, ws)
    L.permute(cfg, x, out, ws, x_perm)
    L.grouped_ffn(cfg, T, MOE_GROUPS_ROUTED, w, ws, x_perm=x_perm, offsets=out["offsets"],
                  y_routed=y_routed)
    L.grouped_ffn(cfg, T, MOE_GROUPS_SHARED, w, ws, x_shared=x, y_shared=y_shared)
    L.combine(cfg, T, y_routed, y_shared, out)
    torch.cuda.synchronize()
    staged = P.to_numpy(out)
    for k in whole:
        np.testing.assert_array_equal(staged[k], whole[k], err_msg=k)
    # the gathered rows are the token rows
    rows = int(staged["offsets"][-1])
    st = torch.from_numpy(staged["sorted_token"][:rows]).long().to(x.device)
    assert torch.equal(x_perm[:rows], x[st])
    # y_lowp is y rounded to the storage type
    yl = torch.from_numpy(whole["y"]).to(x.dtype).float().numpy()
    np.testing.assert_array_equal(whole["y_lowp"], yl)



# one case per shape of the stand-alone gather: 16-byte pieces per row 96 (bf16
# d = 768), 192 (1536), 512 (fp32 2048) and 1024 (bf16 8192, two passes per
# row), and a capacity that drops slots
GATHER = {
    "d768": synth.QUARTZ.replace(T=400, hidden=768, ffn=64, seed=21),
    "d1536_sigmoid": synth.SUTRA.replace(T=333, ffn=64, seed=22),
    "f32_d2048": synth.TINY.replace(T=257, hidden=2048, dtype="f32", seed=23),
    "d8192": synth.QUARTZ.replace(T=129, hidden=8192, ffn=64, seed=24),
    "capacity_drops": synth.MOONFROST.replace(T=600, ffn=64, seed=25),
}


@pytest.mark.parametrize("base", list(GATHER))
def test_permute_gathers_token_rows(base):
    """moe_permute's x_perm holds x[sorted_token[row]] for every kept row, bit
    for bit, and leaves the rows past offsets[E] as they were."""
    wl = GATHER[base]
    inp = synth.make_inputs(wl)
    cfg, x, w = P.upload(wl, inp)
    T = wl.T
    out = L.allocate_outputs(cfg, T, x.device)
    ws = L.allocate_workspace(cfg, T, x.device)
    R = max(1, int(L._lib.moe_max_rows(cfg, T)))
    x_perm = torch.full((R + 3, wl.hidden), 7.0, dtype=x.dtype, device=x.device)
    L.route(cfg, x, w, out, ws)
    L.permute(cfg, x, out, ws, x_perm)
    torch.cuda.synchronize()
    rows = int(out["offsets"][-1].item())
    assert 0 < rows <= R
    st = out["sorted_token"][:rows].long()
    assert torch.equal(x_perm[:rows], x[st])
    assert bool((x_perm[rows:] == 7).all())

def test_bias_update_matches_oracle():
    """moe_bias_update against the oracle, bit for bit: counts from a real
    routing call on the GPU (Sutra-shaped skew), then hand-made patterns with
    experts exactly at the mean, an empty expert, and signed zeros."""
    import oracle
    wl = SMALL["sutra_small"]
    print(f"\n[case] bias update after {wl}", flush=True)
    inp = synth.make_inputs(wl)
    cfg, x, w = P.upload(wl, inp)
    out = L.allocate_outputs(cfg, wl.T, x.device)
    ws = L.allocate_workspace(cfg, wl.T, x.device)
    L.layer_forward(cfg, x, w, out, ws)
    torch.cuda.synchronize()
    counts = out.t["counts"].clone()
    E = wl.n_routed
    cases = [(wl.T, wl.top_k, counts, w.t["select_bias"].clone(), 1e-3)]
    # T k / E = 2 exactly: experts at, above and below the mean, one empty
    hand = torch.tensor([2, 5, 0, 2, 1, 2, 3, 1], dtype=torch.int32, device=x.device)
    bias = torch.tensor([0.5, -0.0, 0.0, -0.25, 3.0, -1e-8, 7.5, 1e-3], dtype=torch.float32,
                        device=x.device)
    cfg8 = L.make_config(hidden=128, n_routed=8, top_k=2, n_shared=0, ffn=64, score="sigmoid")
    for T, k, c, b, g in cases + [(8, 2, hand, bias, 0.0625)]:
        cf = cfg if c.numel() == E else cfg8
        want = oracle.bias_update(b.cpu().numpy(), c.cpu().numpy(), T, k, g)
        got = b.clone()
        L.bias_update(cf, T, c, got, g)
        torch.cuda.synchronize()
        got = got.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (got, want)
    # repeated on the device: the largest load falls toward the mean
    sb = w.t["select_bias"]
    first = int(counts.max())
    for _ in range(60):
        L.layer_forward(cfg, x, w, out, ws)
        L.bias_update(cfg, wl.T, out.t["counts"], sb, 0.05)
    torch.cuda.synchronize()
    last = int(out.t["counts"].max())
    print(f"[report] bias update: max count {first} -> {last} (mean {wl.T * wl.top_k / E:.1f})",
          flush=True)
    assert last < first
