"""moe_layer_forward_noalloc (workspace in the library's own device array)
against moe_layer_forward on a caller's workspace, through the C ABI: every
output bit for bit, on two calls in a row on the same array, the second with a
smaller batch (the array keeps the first call's contents); and a batch whose
workspace exceeds the array is refused before any launch.
"""
import numpy as np
import pytest
import torch

from fine_grained_mixture_amd import _lib, synth
from fine_grained_mixture_amd import layer as L
from tests import _parity as P

pytestmark = pytest.mark.gpu

CASES = {
    # Quartz widths: 600 then 77 tokens (several routing blocks, then fewer)
    "quartz": (synth.QUARTZ, (600, 77)),
    # capacity drops, raw softmax gates
    "moonfrost": (synth.MOONFROST.replace(hidden=512, ffn=256), (1000, 300)),
    # rank-64 experts over many experts
    "dormouse": (synth.DORMOUSE.replace(hidden=256, ffn=128), (900, 40)),
}


def _outputs(cfg, T, dev):
    return L.allocate_outputs(cfg, T, dev, y_lowp=True)


@pytest.mark.parametrize("name", list(CASES))
def test_noalloc_matches_layer_forward(name):
    base, sizes = CASES[name]
    for T in sizes:
        wl = base.replace(T=T, seed=T)
        print(f"\n[case] noalloc {name} T={T}", flush=True)
        inp = synth.make_inputs(wl)
        cfg, x, w = P.upload(wl, inp)
        assert _lib.moe_workspace_bytes(cfg, T) <= _lib.MOE_NOALLOC_SCRATCH_BYTES
        ref = _outputs(cfg, T, x.device)
        ws = L.allocate_workspace(cfg, T, x.device)
        L.layer_forward(cfg, x, w, ref, ws)
        got = _outputs(cfg, T, x.device)
        _lib.moe_layer_forward_noalloc(cfg, T, x.data_ptr(), w.struct, got.struct,
                                       L.current_stream())
        torch.cuda.synchronize()
        a, b = P.to_numpy(ref), P.to_numpy(got)
        assert a.keys() == b.keys()
        for k in a:
            np.testing.assert_array_equal(b[k], a[k], err_msg=f"{name} T={T} {k}")


def test_noalloc_refuses_a_batch_beyond_its_array():
    wl = synth.QUARTZ
    cfg = L.config_from_workload(wl)
    assert _lib.moe_workspace_bytes(cfg, wl.T) > _lib.MOE_NOALLOC_SCRATCH_BYTES
    inp = synth.make_inputs(wl.replace(T=1))
    w = L.DeviceWeights.from_numpy(inp, cfg, "cuda")
    x = torch.zeros((wl.T, wl.hidden), dtype=torch.bfloat16, device="cuda")
    out = L.allocate_outputs(cfg, wl.T, "cuda")
    with pytest.raises(_lib.MoeError) as e:
        _lib.moe_layer_forward_noalloc(cfg, wl.T, x.data_ptr(), w.struct, out.struct,
                                       L.current_stream())
    assert e.value.status == _lib.MOE_EWORKSPACE
