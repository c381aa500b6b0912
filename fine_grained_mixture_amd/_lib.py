"""ctypes binding of libmoe.so (include/moe.h). Argument marshalling only.

Every function takes plain integers (device pointers, sizes, the HIP stream
handle) or the ctypes structures below, and raises MoeError on a non-zero
status. The library is loaded from this package directory; if it is missing
the import of any entry point fails loudly -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP = 0, -1, -2, -3, -4
MOE_F32, MOE_BF16, MOE_FP8 = 0, 1, 2
MOE_SOFTMAX, MOE_SIGMOID = 0, 1
MOE_GROUPS_ROUTED, MOE_GROUPS_SHARED = 1, 2

MOE_WS_H, MOE_WS_H_SHARED, MOE_WS_Y_ROUTED, MOE_WS_Y_SHARED = 0, 1, 2, 3
MOE_WS_HQ, MOE_WS_HQ_SCALE, MOE_WS_HQ_SHARED, MOE_WS_HQ_SHARED_SCALE = 4, 5, 6, 7
MOE_BWS_DY_ROUTED, MOE_BWS_X_PERM, MOE_BWS_DAB, MOE_BWS_DL = 0, 1, 2, 3
(MOE_BWS_LR_UG, MOE_BWS_LR_UU, MOE_BWS_LR_Z_GU, MOE_BWS_LR_AB, MOE_BWS_LR_H, MOE_BWS_LR_UD,
 MOE_BWS_LR_ZD, MOE_BWS_LR_DZD, MOE_BWS_LR_DUD, MOE_BWS_LR_DZG, MOE_BWS_LR_DZU,
 MOE_BWS_LR_DU_GU) = range(4, 16)
MOE_BWS_DAB_SHARED = 16

EXPORTED = ("moe_capacity", "moe_max_rows", "moe_workspace_bytes", "moe_workspace_region",
            "moe_route", "moe_permute",
            "moe_grouped_ffn", "moe_combine", "moe_bias_update", "moe_quantize_fp8",
            "moe_layer_forward", "moe_layer_forward_noalloc",
            "moe_layer_forward_timed", "moe_backward_workspace_bytes",
            "moe_backward_workspace_region", "moe_layer_backward",
            "moe_layer_backward_timed", "moe_stage_name", "moe_status_str", "moe_last_error")


class MoeConfig(ctypes.Structure):
    _fields_ = [("hidden", c_int32), ("n_routed", c_int32), ("top_k", c_int32),
                ("n_shared", c_int32), ("ffn", c_int32), ("rank", c_int32),
                ("score", c_int32), ("renorm_topk", c_int32), ("capacity", c_int32),
                ("aux_coef", c_float), ("dtype", c_int32)]


WEIGHT_FIELDS = ("w_router", "logit_bias", "select_bias", "w_gate", "w_up", "w_down",
                 "u_gate", "s_gate", "v_gate", "u_up", "s_up", "v_up",
                 "u_down", "s_down", "v_down", "sh_gate", "sh_up", "sh_down",
                 "w_gate_scale", "w_up_scale", "w_down_scale", "sh_gate_scale", "sh_up_scale",
                 "sh_down_scale", "u_gate_scale", "u_up_scale", "u_down_scale", "v_gate_scale",
                 "v_up_scale", "v_down_scale")
OUTPUT_FIELDS = ("topk_idx", "topk_gate", "topk_margin", "counts", "kept", "offsets",
                 "sorted_token", "row_of_slot", "dropped", "n_dropped", "aux", "f", "P",
                 "y", "y_lowp", "saved_ab")


class MoeWeights(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in WEIGHT_FIELDS]


class MoeOutputs(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in OUTPUT_FIELDS]


GRAD_FIELDS = ("dx", "dw_router", "dw_gate", "dw_up", "dw_down", "dsh_gate", "dsh_up",
               "dsh_down", "du_gate", "ds_gate", "dv_gate", "du_up", "ds_up", "dv_up",
               "du_down", "ds_down", "dv_down")


class MoeGrads(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in GRAD_FIELDS]


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load()
        msg = lib.moe_status_str(status).decode()
        if status == MOE_EHIP:
            msg += ": " + lib.moe_last_error().decode()
        super().__init__(f"{where}: {msg} (status {status})")
        self.status = status


_LIB = None


def load():
    """Load libmoe.so once. Raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m fine_grained_mixture_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    cfgp, wp, op = POINTER(MoeConfig), POINTER(MoeWeights), POINTER(MoeOutputs)
    gp = POINTER(MoeGrads)
    sig = {
        "moe_capacity": (c_int32, [c_int64, c_int64, c_int64, c_int32, c_int32]),
        "moe_max_rows": (c_int64, [cfgp, c_int64]),
        "moe_workspace_bytes": (c_size_t, [cfgp, c_int64]),
        "moe_workspace_region": (c_int, [cfgp, c_int64, c_int32, POINTER(c_size_t),
                                         POINTER(c_size_t)]),
        "moe_backward_workspace_region": (c_int, [cfgp, c_int64, c_int32, POINTER(c_size_t),
                                                  POINTER(c_size_t)]),
        "moe_route": (c_int, [cfgp, c_int64, c_void_p, wp, op, c_void_p, c_size_t, c_void_p]),
        "moe_permute": (c_int, [cfgp, c_int64, c_void_p, op, c_void_p, c_void_p, c_size_t,
                                c_void_p]),
        "moe_grouped_ffn": (c_int, [cfgp, c_int64, c_int32, c_void_p, c_void_p, c_void_p, wp,
                                    c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
        "moe_combine": (c_int, [cfgp, c_int64, c_void_p, c_void_p, op, c_void_p]),
        "moe_bias_update": (c_int, [cfgp, c_int64, c_void_p, c_void_p, c_float, c_void_p]),
        "moe_quantize_fp8": (c_int, [cfgp, wp, wp, c_void_p]),
        "moe_layer_forward": (c_int, [cfgp, c_int64, c_void_p, wp, op, c_void_p, c_size_t,
                                      c_void_p]),
        "moe_layer_forward_noalloc": (c_int, [cfgp, c_int64, c_void_p, wp, op, c_void_p]),
        "moe_layer_forward_timed": (c_int, [cfgp, c_int64, c_void_p, wp, op, c_void_p,
                                            c_size_t, c_void_p, POINTER(c_void_p), c_int]),
        "moe_backward_workspace_bytes": (c_size_t, [cfgp, c_int64]),
        "moe_layer_backward": (c_int, [cfgp, c_int64, c_void_p, wp, op, c_void_p, c_float, gp,
                                       c_void_p, c_size_t, c_void_p, c_size_t, c_void_p]),
        "moe_layer_backward_timed": (c_int, [cfgp, c_int64, c_void_p, wp, op, c_void_p, c_float,
                                             gp, c_void_p, c_size_t, c_void_p, c_size_t,
                                             c_void_p, POINTER(c_void_p), c_int]),
        "moe_stage_name": (c_char_p, [c_int]),
        "moe_status_str": (c_char_p, [c_int]),
        "moe_last_error": (c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def _check(status: int, where: str) -> int:
    if status < 0:
        raise MoeError(status, where)
    return status


def moe_capacity(num: int, den: int, T: int, k: int, E: int) -> int:
    return load().moe_capacity(num, den, T, k, E)


def moe_max_rows(cfg: MoeConfig, T: int) -> int:
    return load().moe_max_rows(ctypes.byref(cfg), T)


def moe_workspace_bytes(cfg: MoeConfig, T: int) -> int:
    return load().moe_workspace_bytes(ctypes.byref(cfg), T)


def moe_workspace_region(cfg: MoeConfig, T: int, which: int) -> tuple[int, int]:
    """(byte offset into the workspace, bytes) of an intermediate region."""
    off, n = c_size_t(0), c_size_t(0)
    _check(load().moe_workspace_region(ctypes.byref(cfg), T, which, ctypes.byref(off),
                                       ctypes.byref(n)), "moe_workspace_region")
    return off.value, n.value


def moe_backward_workspace_region(cfg: MoeConfig, T: int, which: int) -> tuple[int, int]:
    """(byte offset into the backward workspace, bytes) of an intermediate region."""
    off, n = c_size_t(0), c_size_t(0)
    _check(load().moe_backward_workspace_region(ctypes.byref(cfg), T, which, ctypes.byref(off),
                                                ctypes.byref(n)),
           "moe_backward_workspace_region")
    return off.value, n.value


def moe_route(cfg, T, x, w, o, ws, ws_bytes, stream) -> None:
    _check(load().moe_route(ctypes.byref(cfg), T, x, ctypes.byref(w), ctypes.byref(o), ws,
                            ws_bytes, stream), "moe_route")


def moe_permute(cfg, T, x, o, x_perm, ws, ws_bytes, stream) -> None:
    _check(load().moe_permute(ctypes.byref(cfg), T, x, ctypes.byref(o), x_perm, ws, ws_bytes,
                              stream), "moe_permute")


def moe_grouped_ffn(cfg, T, groups, x_perm, offsets, x_shared, w, y_routed, y_shared, ws,
                    ws_bytes, stream) -> None:
    _check(load().moe_grouped_ffn(ctypes.byref(cfg), T, groups, x_perm, offsets, x_shared,
                                  ctypes.byref(w), y_routed, y_shared, ws, ws_bytes, stream),
           "moe_grouped_ffn")


def moe_bias_update(cfg, T, counts, select_bias, gamma, stream) -> None:
    _check(load().moe_bias_update(ctypes.byref(cfg), T, counts, select_bias, gamma, stream),
           "moe_bias_update")


def moe_quantize_fp8(cfg, src, dst, stream) -> None:
    _check(load().moe_quantize_fp8(ctypes.byref(cfg), ctypes.byref(src), ctypes.byref(dst),
                                   stream), "moe_quantize_fp8")


def moe_combine(cfg, T, y_routed, y_shared, o, stream) -> None:
    _check(load().moe_combine(ctypes.byref(cfg), T, y_routed, y_shared, ctypes.byref(o),
                              stream), "moe_combine")


def moe_layer_forward(cfg, T, x, w, o, ws, ws_bytes, stream) -> None:
    _check(load().moe_layer_forward(ctypes.byref(cfg), T, x, ctypes.byref(w), ctypes.byref(o),
                                    ws, ws_bytes, stream), "moe_layer_forward")


MOE_NOALLOC_SCRATCH_BYTES = 64 << 20


def moe_layer_forward_noalloc(cfg, T, x, w, o, stream) -> None:
    _check(load().moe_layer_forward_noalloc(ctypes.byref(cfg), T, x, ctypes.byref(w),
                                            ctypes.byref(o), stream), "moe_layer_forward_noalloc")


def moe_layer_forward_timed(cfg, T, x, w, o, ws, ws_bytes, stream, events) -> int:
    """events: list of hipEvent_t handles (ints). Returns the kernel count."""
    arr = (c_void_p * max(1, len(events)))(*events)
    n = load().moe_layer_forward_timed(ctypes.byref(cfg), T, x, ctypes.byref(w),
                                       ctypes.byref(o), ws, ws_bytes, stream, arr, len(events))
    return _check(n, "moe_layer_forward_timed")


def moe_backward_workspace_bytes(cfg: MoeConfig, T: int) -> int:
    return load().moe_backward_workspace_bytes(ctypes.byref(cfg), T)


def moe_layer_backward(cfg, T, x, w, o, dy, aux_grad, g, ws, ws_bytes, bws, bws_bytes,
                       stream) -> None:
    _check(load().moe_layer_backward(ctypes.byref(cfg), T, x, ctypes.byref(w), ctypes.byref(o),
                                     dy, aux_grad, ctypes.byref(g), ws, ws_bytes, bws, bws_bytes,
                                     stream), "moe_layer_backward")


def moe_layer_backward_timed(cfg, T, x, w, o, dy, aux_grad, g, ws, ws_bytes, bws, bws_bytes,
                             stream, events) -> int:
    arr = (c_void_p * max(1, len(events)))(*events)
    n = load().moe_layer_backward_timed(ctypes.byref(cfg), T, x, ctypes.byref(w),
                                        ctypes.byref(o), dy, aux_grad, ctypes.byref(g), ws,
                                        ws_bytes, bws, bws_bytes, stream, arr, len(events))
    return _check(n, "moe_layer_backward_timed")


def moe_stage_name(i: int) -> str | None:
    s = load().moe_stage_name(i)
    return None if s is None else s.decode()
