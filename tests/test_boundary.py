"""The C ABI library loads, exports every function include/moe.h declares, and
its host-side logic (capacity, sizes, argument validation) behaves as
documented. Nothing here launches a kernel, so it runs without a GPU: every
invalid call must return before anything is enqueued.
"""
import ctypes
import os
import re
import subprocess

import pytest

from fine_grained_mixture_amd import _lib
from fine_grained_mixture_amd.synth import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__  # noqa: F401
        from fine_grained_mixture_amd import build
        build.build()
    return _lib.load()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("moe_route", "moe_permute", "moe_grouped_ffn", "moe_combine", "moe_layer_forward",
              "moe_workspace_bytes", "moe_status_str", "moe_capacity"):
        assert n in names
    assert set(names) == set(_lib.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(\w+)$", out, flags=re.M))
    for n in declared_functions():
        assert n in exported, n
        assert getattr(lib, n) is not None


def test_capacity_exact_ceiling(lib):
    # capacity factor 5/4 at the Moonfrost shape gives exactly 1920 slots
    assert _lib.moe_capacity(5, 4, 16384, 3, 32) == 1920
    assert _lib.moe_capacity(5, 4, 16385, 3, 32) == 1921
    assert _lib.moe_capacity(1, 1, 10, 2, 4) == 5
    assert _lib.moe_capacity(1, 1, 11, 2, 4) == 6
    assert _lib.moe_capacity(5, 4, 1000, 3, 32) == WORKLOADS["moonfrost"].replace(T=1000).capacity
    assert _lib.moe_capacity(0, 1, 10, 2, 4) == -1


def test_max_rows_and_workspace(lib):
    from fine_grained_mixture_amd.layer import config_from_workload
    for wl in WORKLOADS.values():
        cfg = config_from_workload(wl)
        r = _lib.moe_max_rows(cfg, wl.T)
        want = wl.T * wl.top_k if wl.capacity == 0 else min(wl.T * wl.top_k,
                                                            wl.n_routed * wl.capacity)
        assert r == want
        ws = _lib.moe_workspace_bytes(cfg, wl.T)
        es = 2 if wl.dtype in ("bf16", "fp8") else 4
        # at least the routed intermediates and the fp32 routed outputs
        assert ws >= r * wl.ffn * es + r * wl.hidden * 4
        assert ws % 256 == 0 or ws > 0


def _cfg(**kw):
    from fine_grained_mixture_amd.layer import make_config
    base = dict(hidden=128, n_routed=8, top_k=2, n_shared=1, ffn=64)
    base.update(kw)
    return make_config(**base)


@pytest.mark.parametrize("bad", [
    dict(hidden=100), dict(ffn=44), dict(top_k=0), dict(top_k=9), dict(top_k=33, n_routed=32),
    dict(n_routed=5000), dict(score="sigmoid", renorm=False), dict(capacity=-1),
    dict(n_shared=-1),
])
def test_invalid_config_rejected(lib, bad):
    cfg = _cfg(**bad)
    assert _lib.moe_workspace_bytes(cfg, 64) == 0
    w = _lib.MoeWeights(w_router=0x1000)
    o = _lib.MoeOutputs(**{n: 0x1000 for n in _lib.OUTPUT_FIELDS})
    st = lib.moe_layer_forward(ctypes.byref(cfg), 64, 0x1000, ctypes.byref(w), ctypes.byref(o),
                               0x1000, 1 << 30, None)
    assert st == _lib.MOE_EINVAL


@pytest.mark.parametrize("legal", [
    dict(hidden=104), dict(ffn=48), dict(hidden=136, ffn=200), dict(top_k=16, n_routed=32),
    dict(top_k=32, n_routed=32), dict(hidden=1 << 21),
])
def test_legal_but_unimplemented_layer_is_unsupported(lib, legal):
    """Layers the layer's definition allows (d, F multiples of 8; k <= E) but
    the kernels do not cover: MOE_EUNSUPPORTED, before any launch; their
    sizes are still reported."""
    cfg = _cfg(**legal)
    assert _lib.moe_workspace_bytes(cfg, 64) > 0
    assert _lib.moe_max_rows(cfg, 64) == 64 * cfg.top_k
    w = _lib.MoeWeights(**{n: 0x1000 for n in _lib.WEIGHT_FIELDS if n != "select_bias"})
    o = _lib.MoeOutputs(**{n: 0x1000 for n in _lib.OUTPUT_FIELDS})
    st = lib.moe_layer_forward(ctypes.byref(cfg), 64, 0x1000, ctypes.byref(w), ctypes.byref(o),
                               0x1000, 1 << 30, None)
    assert st == _lib.MOE_EUNSUPPORTED
    st = lib.moe_route(ctypes.byref(cfg), 64, 0x1000, ctypes.byref(w), ctypes.byref(o), 0x1000,
                       1 << 30, None)
    assert st == _lib.MOE_EUNSUPPORTED


def test_workspace_regions(lib):
    """Intermediate regions lie inside the workspace, do not overlap, and have
    the documented sizes; fp8-only regions are empty otherwise."""
    from fine_grained_mixture_amd.layer import config_from_workload
    for wl in list(WORKLOADS.values()) + [WORKLOADS["quartz"].replace(dtype="fp8"),
                                          WORKLOADS["dormouse"].replace(dtype="fp8", n_shared=2)]:
        cfg = config_from_workload(wl)
        T, R = wl.T, _lib.moe_max_rows(cfg, wl.T)
        total = _lib.moe_workspace_bytes(cfg, T)
        es = 2 if wl.dtype in ("bf16", "fp8") else 4
        S, F, d = wl.n_shared, wl.ffn, wl.hidden
        q = wl.dtype == "fp8" and wl.rank == 0
        want = {_lib.MOE_WS_H: R * F * es * (wl.rank == 0), _lib.MOE_WS_H_SHARED: T * S * F * es,
                _lib.MOE_WS_Y_ROUTED: R * d * 4, _lib.MOE_WS_Y_SHARED: T * d * 4 * (S > 0),
                _lib.MOE_WS_HQ: R * F * q, _lib.MOE_WS_HQ_SCALE: R * 4 * q,
                _lib.MOE_WS_HQ_SHARED: T * S * F * (wl.dtype == "fp8"),
                _lib.MOE_WS_HQ_SHARED_SCALE: T * 4 * (wl.dtype == "fp8" and S > 0)}
        spans = []
        for which, n in want.items():
            off, got = _lib.moe_workspace_region(cfg, T, which)
            assert got == n, (wl.name, which)
            assert off % 256 == 0 and off + got <= total
            if got:
                spans.append((off, off + got))
        spans.sort()
        assert all(a[1] <= b[0] for a, b in zip(spans, spans[1:]))
    with pytest.raises(_lib.MoeError):
        _lib.moe_workspace_region(_cfg(), 64, 99)


def test_backward_workspace_regions(lib):
    """The backward's intermediate regions lie inside its workspace, do not
    overlap, and have the documented sizes; rank-r regions are empty for
    dense experts."""
    from fine_grained_mixture_amd.layer import config_from_workload
    for wl in (WORKLOADS["quartz"], WORKLOADS["dormouse"], WORKLOADS["dormouse"].replace(T=1),
               WORKLOADS["dormouse"].replace(rank=32, T=777), WORKLOADS["tiny"]):
        cfg = config_from_workload(wl)
        T, R = wl.T, _lib.moe_max_rows(cfg, wl.T)
        total = _lib.moe_backward_workspace_bytes(cfg, T)
        d, F, E, r = wl.hidden, wl.ffn, wl.n_routed, wl.rank
        lr = r > 0
        es = 4 if wl.dtype == "f32" else 2
        m = _lib
        want = {m.MOE_BWS_DY_ROUTED: R * d * es, m.MOE_BWS_X_PERM: R * d * es,
                m.MOE_BWS_DAB: R * 2 * F * es, m.MOE_BWS_DL: T * E * es,
                m.MOE_BWS_LR_UG: R * r * 4 * lr, m.MOE_BWS_LR_UU: R * r * 4 * lr,
                m.MOE_BWS_LR_Z_GU: R * 2 * r * 2 * lr, m.MOE_BWS_LR_AB: R * 2 * F * 4 * lr,
                m.MOE_BWS_LR_H: R * F * 2 * lr, m.MOE_BWS_LR_UD: R * r * 4 * lr,
                m.MOE_BWS_LR_ZD: R * r * 2 * lr, m.MOE_BWS_LR_DZD: R * r * 4 * lr,
                m.MOE_BWS_LR_DUD: R * r * 2 * lr, m.MOE_BWS_LR_DZG: R * r * 4 * lr,
                m.MOE_BWS_LR_DZU: R * r * 4 * lr, m.MOE_BWS_LR_DU_GU: R * 2 * r * 2 * lr,
                m.MOE_BWS_DAB_SHARED: T * wl.n_shared * 2 * F * es}
        spans = []
        for which, n in want.items():
            off, got = _lib.moe_backward_workspace_region(cfg, T, which)
            assert got == n, (wl.name, which)
            assert off % 256 == 0 and off + got <= total
            if got:
                spans.append((off, off + got))
        spans.sort()
        assert all(a[1] <= b[0] for a, b in zip(spans, spans[1:]))
    with pytest.raises(_lib.MoeError):
        _lib.moe_backward_workspace_region(_cfg(), 64, 17)


@pytest.mark.parametrize("rank,dtype", [(8, "bf16"), (40, "bf16"), (80, "bf16"), (128, "bf16"),
                                        (32, "fp8"), (64, "f32")])
def test_unsupported_rank_rejected_before_any_launch(lib, rank, dtype):
    cfg = _cfg(rank=rank, dtype=dtype)
    w = _lib.MoeWeights(**{n: 0x1000 for n in _lib.WEIGHT_FIELDS})
    o = _lib.MoeOutputs(**{n: 0x1000 for n in _lib.OUTPUT_FIELDS})
    st = lib.moe_layer_forward(ctypes.byref(cfg), 64, 0x1000, ctypes.byref(w), ctypes.byref(o),
                               0x1000, 1 << 30, None)
    assert st == _lib.MOE_EUNSUPPORTED


@pytest.mark.parametrize("rank", [16, 32, 48, 64])
def test_low_ranks_accepted(lib, rank):
    assert _lib.moe_workspace_bytes(_cfg(rank=rank), 64) > 0


def test_null_pointers_and_workspace_rejected(lib):
    cfg = _cfg()
    full_w = _lib.MoeWeights(**{n: 0x1000 for n in ("w_router", "w_gate", "w_up", "w_down",
                                                      "sh_gate", "sh_up", "sh_down")})
    full_o = _lib.MoeOutputs(**{n: 0x1000 for n in _lib.OUTPUT_FIELDS})
    need = _lib.moe_workspace_bytes(cfg, 64)

    def call(w=full_w, o=full_o, x=0x1000, ws=0x1000, nbytes=need, T=64):
        return lib.moe_layer_forward(ctypes.byref(cfg), T, x, ctypes.byref(w), ctypes.byref(o),
                                     ws, nbytes, None)

    assert call(x=0) == _lib.MOE_EINVAL
    w = _lib.MoeWeights.from_buffer_copy(full_w)
    w.w_up = None
    assert call(w=w) == _lib.MOE_EINVAL
    w = _lib.MoeWeights.from_buffer_copy(full_w)
    w.sh_down = None
    assert call(w=w) == _lib.MOE_EINVAL
    w = _lib.MoeWeights.from_buffer_copy(full_w)
    w.select_bias = 0x1000          # selection bias only exists for the sigmoid rule
    assert call(w=w) == _lib.MOE_EINVAL
    o = _lib.MoeOutputs.from_buffer_copy(full_o)
    o.row_of_slot = None
    assert call(o=o) == _lib.MOE_EINVAL
    assert call(nbytes=need - 1) == _lib.MOE_EWORKSPACE
    assert call(ws=0) == _lib.MOE_EWORKSPACE
    assert call(ws=0x1001) == _lib.MOE_EWORKSPACE
    assert call(T=-1) == _lib.MOE_EINVAL
    # grouped FFN: unknown group bits, routed without offsets
    st = lib.moe_grouped_ffn(ctypes.byref(cfg), 64, 4, 0x1000, 0x1000, 0x1000,
                             ctypes.byref(full_w), 0x1000, 0x1000, 0x1000, need, None)
    assert st == _lib.MOE_EINVAL
    st = lib.moe_grouped_ffn(ctypes.byref(cfg), 64, _lib.MOE_GROUPS_ROUTED, 0x1000, None, None,
                             ctypes.byref(full_w), 0x1000, None, 0x1000, need, None)
    assert st == _lib.MOE_EINVAL


def test_bias_update_validation(lib):
    cfg = _cfg()
    call = lambda T=64, c=0x1000, b=0x1000, g=0.01: lib.moe_bias_update(  # noqa: E731
        ctypes.byref(cfg), T, c, b, g, None)
    assert call(c=None) == _lib.MOE_EINVAL
    assert call(b=None) == _lib.MOE_EINVAL
    assert call(T=-1) == _lib.MOE_EINVAL
    assert call(g=float("nan")) == _lib.MOE_EINVAL
    assert call(g=float("inf")) == _lib.MOE_EINVAL
    bad = _cfg()
    bad.top_k = 0
    assert lib.moe_bias_update(ctypes.byref(bad), 64, 0x1000, 0x1000, 0.01, None) == _lib.MOE_EINVAL


def test_status_strings(lib):
    for st in (0, -1, -2, -3, -4):
        assert lib.moe_status_str(st)
    assert lib.moe_stage_name(0) is None or isinstance(lib.moe_stage_name(0), bytes)


def test_backward_validation(lib):
    cfg = _cfg(dtype="bf16")
    T = 64
    full_w = _lib.MoeWeights(**{n: 0x1000 for n in ("w_router", "w_gate", "w_up", "w_down",
                                                      "sh_gate", "sh_up", "sh_down")})
    full_o = _lib.MoeOutputs(**{n: 0x1000 for n in _lib.OUTPUT_FIELDS})
    full_g = _lib.MoeGrads(**{n: 0x1000 for n in _lib.GRAD_FIELDS})
    need = _lib.moe_workspace_bytes(cfg, T)
    bneed = _lib.moe_backward_workspace_bytes(cfg, T)
    assert bneed > 0 and bneed % 256 == 0

    def call(c=cfg, w=full_w, o=full_o, g=full_g, x=0x1000, dy=0x1000, aux=1.0, ws=0x1000,
             nbytes=need, bws=0x1000, bbytes=bneed, T=T):
        return lib.moe_layer_backward(ctypes.byref(c), T, x, ctypes.byref(w), ctypes.byref(o),
                                      dy, aux, ctypes.byref(g), ws, nbytes, bws, bbytes, None)

    assert call(x=0) == _lib.MOE_EINVAL
    assert call(dy=0) == _lib.MOE_EINVAL
    assert call(aux=float("nan")) == _lib.MOE_EINVAL
    for field in ("dx", "dw_router", "dw_gate", "dsh_down"):
        g = _lib.MoeGrads.from_buffer_copy(full_g)
        setattr(g, field, None)
        assert call(g=g) == _lib.MOE_EINVAL, field
    o = _lib.MoeOutputs.from_buffer_copy(full_o)
    o.sorted_token = None
    assert call(o=o) == _lib.MOE_EINVAL
    assert call(nbytes=need - 1) == _lib.MOE_EWORKSPACE
    assert call(bbytes=bneed - 1) == _lib.MOE_EWORKSPACE
    assert call(bws=0) == _lib.MOE_EWORKSPACE
    assert call(bws=0x1001) == _lib.MOE_EWORKSPACE
    assert call(T=-1) == _lib.MOE_EINVAL
    # the library's backward: bf16 dense experts (expert count a multiple of 8)
    # or rank-32/64 experts, and float32 dense experts
    for bad in (_cfg(dtype="fp8"), _cfg(n_routed=12), _cfg(rank=16), _cfg(dtype="f32", rank=64)):
        nb = _lib.moe_backward_workspace_bytes(bad, T)
        st = call(c=bad, nbytes=_lib.moe_workspace_bytes(bad, T), bbytes=nb)
        assert st == _lib.MOE_EUNSUPPORTED


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the built library the binding raises; there is no fallback path."""
    monkeypatch.setattr(_lib, "_LIB", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libmoe.so"))
    with pytest.raises(RuntimeError, match="is missing"):
        _lib.load()


def test_binding_rejects_wrong_tensors():
    """The Python binding checks dtype, shape, device and layout of x and the
    weights before passing their addresses on (no GPU: CPU tensors are
    rejected as such, CUDA-less shape and dtype checks run first)."""
    import torch
    from fine_grained_mixture_amd import layer as L
    cfg = _cfg()
    x = torch.zeros((4, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        L.check_x(cfg, x)
    with pytest.raises(ValueError, match="2-d"):
        L.check_x(cfg, torch.zeros(128, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        L.check_device_tensor(torch.zeros((4, 64)), (4, 128), torch.float32, "x")
    want = L.expected_weight_shapes(cfg)
    assert want["w_gate"] == ((8, 128, 64), torch.bfloat16)
    assert want["sh_down"] == ((1, 64, 128), torch.bfloat16)
    w8 = L.expected_weight_shapes(L.make_config(128, 8, 2, 2, 64, dtype="fp8"))
    assert w8["w_gate"] == ((8, 64, 128), torch.uint8) and w8["sh_down"] == ((128, 128), torch.uint8)
    lr = L.expected_weight_shapes(L.make_config(128, 8, 2, 0, 64, rank=16))
    assert lr["u_down"] == ((8, 64, 16), torch.bfloat16) and "w_gate" not in lr
    # a weight set missing a matrix, or holding one the config does not read
    w = L.DeviceWeights({})
    with pytest.raises(ValueError, match="missing"):
        w.check(cfg)
    w = L.DeviceWeights({"u_gate": torch.zeros(1)})
    with pytest.raises(ValueError, match="not read"):
        w.check(cfg)


def test_noalloc_entry_point_refuses_before_touching_a_device(lib):
    """The allocation-free forward validates its arguments and the size of its
    device array before it looks anything up on a device (no GPU here)."""
    from fine_grained_mixture_amd.layer import config_from_workload
    cfg = config_from_workload(WORKLOADS["quartz"])
    w = _lib.MoeWeights(**{n: 0x1000 for n in ("w_router", "w_gate", "w_up", "w_down",
                                                 "sh_gate", "sh_up", "sh_down")})
    o = _lib.MoeOutputs(**{n: 0x1000 for n in _lib.OUTPUT_FIELDS})
    assert _lib.moe_workspace_bytes(cfg, 4096) > _lib.MOE_NOALLOC_SCRATCH_BYTES
    assert lib.moe_layer_forward_noalloc(ctypes.byref(cfg), 4096, 0x1000, ctypes.byref(w),
                                         ctypes.byref(o), None) == _lib.MOE_EWORKSPACE
    assert lib.moe_layer_forward_noalloc(ctypes.byref(cfg), 64, None, ctypes.byref(w),
                                         ctypes.byref(o), None) == _lib.MOE_EINVAL
    bad = _cfg(top_k=0)
    assert lib.moe_layer_forward_noalloc(ctypes.byref(bad), 64, 0x1000, ctypes.byref(w),
                                         ctypes.byref(o), None) == _lib.MOE_EINVAL
