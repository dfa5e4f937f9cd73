"""Python binding of the C ABI in ``include/mxmoe.h`` (argument marshalling only).

Every step of the layer runs in the HIP library ``libmxmoe.so``; there is no
fallback.  If the library is missing this module raises on first use.
"""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_int, c_int32, c_int64, c_size_t, c_uint32, c_void_p
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmxmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_DEVICE = range(5)
MOE_SRC_BF16, MOE_SRC_FP32 = 0, 1

EXPORTED = ("moe_plan", "moe_plan_destroy", "moe_workspace_bytes", "moe_quantize_act",
            "moe_forward", "moe_forward_noalloc", "moe_profile_begin", "moe_profile_end", "moe_packed_scale_bytes",
            "moe_pack_mx4", "moe_latent_tail_workspace_bytes", "moe_latent_tail",
            "moe_router_bias_update",
            "moe_status_string", "moe_last_error")
STAGES = ("router", "topk", "permute", "gate_up", "down", "combine")


class MoeError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"mxmoe status {status}: {detail}")
        self.status = status
        self.detail = detail


class MoeConfig(ctypes.Structure):
    _fields_ = [("d_model", c_int32), ("d_ff", c_int32), ("num_experts", c_int32),
                ("top_k", c_int32), ("num_shared", c_int32), ("max_tokens", c_int64),
                ("flags", c_uint32)]


MOE_WEIGHTS_CANONICAL = 0x4E4E4143
MOE_WEIGHTS_PACKED = 0x3450584D


class MoeWeights(ctypes.Structure):
    """Device pointers of the layer's weights.  ``layout``:
    MOE_WEIGHTS_PACKED (expert matrices made by moe_pack_mx4) or
    MOE_WEIGHTS_CANONICAL (codes [N][K/2], scales [N][K/32])."""
    _fields_ = [(n, c_void_p) for n in ("gu_codes", "gu_scales", "dn_codes", "dn_scales",
                                         "sgu_codes", "sgu_scales", "sdn_codes", "sdn_scales",
                                         "router_w", "router_b")] + [("layout", c_uint32)]


TAP_FIELDS = ("logits", "topk_ids", "topk_w", "expert_offsets", "row_src", "token_row",
              "x_codes", "x_scales", "h_codes", "h_scales", "gu_acc", "y_routed", "y_shared",
              "h_bf16")
MOE_FLAG_A16W4 = 1


class MoeTaps(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in TAP_FIELDS]


class MoeTailWeights(ctypes.Structure):
    """W_up (MXFP4, packed with interleave 0 or canonical, as ``layout``
    says) and the RMSNorm gain."""
    _fields_ = [("up_codes", c_void_p), ("up_scales", c_void_p), ("gamma", c_void_p),
                ("layout", c_uint32)]


class MoeTailTaps(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("inv_rms", "a_codes", "a_scales")]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libmxmoe.so (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m mxfp4_expert_grouped_amd.build`")
    lib = ctypes.CDLL(path)
    lib.moe_plan.argtypes = [POINTER(MoeConfig), POINTER(c_void_p)]
    lib.moe_plan.restype = c_int
    lib.moe_plan_destroy.argtypes = [c_void_p]
    lib.moe_plan_destroy.restype = None
    lib.moe_workspace_bytes.argtypes = [c_void_p, c_int64, POINTER(c_size_t)]
    lib.moe_workspace_bytes.restype = c_int
    lib.moe_quantize_act.argtypes = [c_void_p, c_int, c_int64, c_int64, c_int64, c_void_p,
                                     c_void_p, c_void_p]
    lib.moe_quantize_act.restype = c_int
    lib.moe_forward.argtypes = [c_void_p, POINTER(MoeWeights), c_void_p, c_int64, c_void_p,
                                c_void_p, c_size_t, POINTER(MoeTaps), c_void_p]
    lib.moe_forward.restype = c_int
    lib.moe_forward_noalloc.argtypes = [c_void_p, POINTER(MoeWeights), c_void_p, c_int64, c_void_p,
                                        POINTER(MoeTaps), c_void_p]
    lib.moe_forward_noalloc.restype = c_int
    lib.moe_profile_begin.argtypes = [c_void_p, c_uint32, c_int32]
    lib.moe_profile_begin.restype = c_int
    lib.moe_profile_end.argtypes = [c_void_p, POINTER(ctypes.c_double), POINTER(c_int32)]
    lib.moe_profile_end.restype = c_int
    lib.moe_packed_scale_bytes.argtypes = [c_int64, c_int64]
    lib.moe_packed_scale_bytes.restype = c_size_t
    lib.moe_pack_mx4.argtypes = [c_void_p, c_void_p, c_int64, c_int64, c_int64, c_int, c_void_p,
                                 c_void_p, c_void_p]
    lib.moe_pack_mx4.restype = c_int
    lib.moe_latent_tail_workspace_bytes.argtypes = [c_int64, c_int32, c_int32, POINTER(c_size_t)]
    lib.moe_latent_tail_workspace_bytes.restype = c_int
    lib.moe_latent_tail.argtypes = [c_int64, c_int32, c_int32, ctypes.c_float, POINTER(MoeTailWeights),
                                    c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                    POINTER(MoeTailTaps), c_void_p]
    lib.moe_latent_tail.restype = c_int
    lib.moe_router_bias_update.argtypes = [c_void_p, c_void_p, c_int64, ctypes.c_float, c_void_p, c_void_p]
    lib.moe_router_bias_update.restype = c_int
    lib.moe_status_string.argtypes = [c_int]
    lib.moe_status_string.restype = c_char_p
    lib.moe_last_error.argtypes = []
    lib.moe_last_error.restype = c_char_p
    _lib = lib
    return lib


def _check(status: int):
    if status != MOE_OK:
        raise MoeError(status, load_library().moe_last_error().decode())


def moe_plan(d_model: int, d_ff: int, num_experts: int, top_k: int, num_shared: int,
             max_tokens: int, flags: int = 0) -> c_void_p:
    cfg = MoeConfig(d_model, d_ff, num_experts, top_k, num_shared, max_tokens, flags)
    h = c_void_p()
    _check(load_library().moe_plan(ctypes.byref(cfg), ctypes.byref(h)))
    return h


def moe_plan_destroy(plan: c_void_p) -> None:
    load_library().moe_plan_destroy(plan)


def moe_workspace_bytes(plan: c_void_p, num_tokens: int) -> int:
    out = c_size_t()
    _check(load_library().moe_workspace_bytes(plan, num_tokens, ctypes.byref(out)))
    return out.value


def moe_quantize_act(src: int, src_dtype: int, rows: int, cols: int, ld_src: int, codes: int,
                     scales: int, stream: Optional[int] = None) -> None:
    _check(load_library().moe_quantize_act(src, src_dtype, rows, cols, ld_src, codes, scales,
                                           stream))


def moe_forward(plan: c_void_p, weights: MoeWeights, x: int, num_tokens: int, y: int,
                workspace: int, workspace_bytes: int, taps: Optional[MoeTaps] = None,
                stream: Optional[int] = None) -> None:
    _check(load_library().moe_forward(plan, ctypes.byref(weights), x, num_tokens, y, workspace,
                                      workspace_bytes, ctypes.byref(taps) if taps else None,
                                      stream))


NOALLOC_SCRATCH_BYTES = 96 << 20  # MOE_NOALLOC_SCRATCH_BYTES


def moe_forward_noalloc(plan: c_void_p, weights: MoeWeights, x: int, num_tokens: int, y: int,
                        taps: Optional[MoeTaps] = None, stream: Optional[int] = None) -> None:
    _check(load_library().moe_forward_noalloc(plan, ctypes.byref(weights), x, num_tokens, y,
                                              ctypes.byref(taps) if taps else None, stream))


def moe_profile_begin(plan: c_void_p, stages, max_calls: int) -> None:
    """Record HIP events around the named stages of the next max_calls forwards."""
    mask = 0
    for st in stages:
        mask |= 1 << STAGES.index(st)
    _check(load_library().moe_profile_begin(plan, mask, max_calls))


def moe_profile_end(plan: c_void_p):
    """-> ({stage: summed ms}, recorded calls)"""
    ms = (ctypes.c_double * len(STAGES))()
    n = c_int32()
    _check(load_library().moe_profile_end(plan, ms, ctypes.byref(n)))
    return dict(zip(STAGES, list(ms))), n.value


def moe_packed_scale_bytes(rows: int, k: int) -> int:
    return load_library().moe_packed_scale_bytes(rows, k)


def moe_pack_mx4(codes: int, scales: int, mats: int, rows: int, k: int, interleave: int, codes_p: int,
                 scales_p: int, stream: Optional[int] = None) -> None:
    _check(load_library().moe_pack_mx4(codes, scales, mats, rows, k, interleave, codes_p, scales_p,
                                       stream))


def moe_latent_tail_workspace_bytes(num_tokens: int, latent: int, hidden: int) -> int:
    out = c_size_t()
    _check(load_library().moe_latent_tail_workspace_bytes(num_tokens, latent, hidden, ctypes.byref(out)))
    return out.value


def moe_latent_tail(num_tokens: int, latent: int, hidden: int, eps: float, weights: MoeTailWeights,
                    z: int, s: Optional[int], y: int, workspace: int, workspace_bytes: int,
                    taps: Optional[MoeTailTaps] = None, stream: Optional[int] = None) -> None:
    _check(load_library().moe_latent_tail(num_tokens, latent, hidden, eps, ctypes.byref(weights), z, s, y,
                                          workspace, workspace_bytes,
                                          ctypes.byref(taps) if taps else None, stream))


def moe_router_bias_update(plan: c_void_p, expert_offsets: int, num_tokens: int, rate: float,
                           router_b: int, stream: Optional[int] = None) -> None:
    _check(load_library().moe_router_bias_update(plan, expert_offsets, num_tokens, rate, router_b, stream))
