"""Seeded synthetic inputs placed on the GPU.

Dense inputs (x, W_r, bias) come from :mod:`.inputs` on the host and are
copied over.  The MXFP4 expert weights (21 GB for the full layer) are drawn on
the device by ``libmxmoe_inputs.so``, the GPU twin of the recipe in
:mod:`.inputs` (Philox uniforms, the same float32 normal-quantile table,
MXFP4 quantisation of each block), which produces the same canonical bytes as
the numpy generator; the layer library then packs them into its tile order.
"""

from __future__ import annotations

import ctypes
import os
from ctypes import c_float, c_int, c_int64, c_uint64, c_void_p
from typing import Optional, Tuple

import numpy as np
import torch

from . import inputs as I
from . import mxmoe as M
from .layer import DeviceWeights

_PKG = os.path.dirname(os.path.abspath(__file__))
GEN_LIB_PATH = os.path.join(_PKG, "libmxmoe_inputs.so")
_gen = None


def _genlib():
    global _gen
    if _gen is None:
        if not os.path.exists(GEN_LIB_PATH):
            raise ImportError(f"{GEN_LIB_PATH} is not built")
        lib = ctypes.CDLL(GEN_LIB_PATH)
        lib.mxmoe_gen_mx_matrix.argtypes = [c_void_p, c_void_p, c_int64, c_int64, c_uint64,
                                            c_uint64, c_void_p, c_float, c_void_p]
        lib.mxmoe_gen_mx_matrix.restype = c_int
        _gen = lib
    return _gen


_tables = {}


def _normal_table_device(device) -> torch.Tensor:
    """The generator's float32 normal-quantile table on `device` (one copy per device)."""
    dev = torch.device(device)
    if dev.index is None:
        dev = torch.device(dev.type, torch.cuda.current_device())
    if dev not in _tables:
        _tables[dev] = torch.from_numpy(I.normal_table()).to(dev)
    return _tables[dev]


def gen_mx_matrix_device(codes: torch.Tensor, scales: torch.Tensor, rows: int, k: int, seed: int,
                         stream: int, sigma: float) -> None:
    table = _normal_table_device(codes.device)
    rc = _genlib().mxmoe_gen_mx_matrix(codes.data_ptr(), scales.data_ptr(), rows, k, seed, stream,
                                       table.data_ptr(), float(sigma),
                                       torch.cuda.current_stream().cuda_stream)
    if rc != 0:
        raise RuntimeError(f"mxmoe_gen_mx_matrix failed ({rc})")


def gen_experts_device(cfg: I.LayerConfig, kind: str, count: int, layer: int = 0,
                       device="cuda") -> Tuple[torch.Tensor, ...]:
    """Stacked (gu_codes, gu_scales, dn_codes, dn_scales) of `count` experts."""
    d, f = cfg.d_model, cfg.d_ff
    guc = torch.empty((count, 2 * f, d // 2), dtype=torch.uint8, device=device)
    gus = torch.empty((count, 2 * f, d // 32), dtype=torch.uint8, device=device)
    dnc = torch.empty((count, d, f // 2), dtype=torch.uint8, device=device)
    dns = torch.empty((count, d, f // 32), dtype=torch.uint8, device=device)
    sg = I.weight_sigma(d)
    for i in range(count):
        slot = I.expert_slot(kind, i)
        gen_mx_matrix_device(guc[i], gus[i], 2 * f, d, cfg.seed, I.stream_id(I.KIND_GU_CODES, slot, layer), sg)
        gen_mx_matrix_device(dnc[i], dns[i], d, f, cfg.seed, I.stream_id(I.KIND_DN_CODES, slot, layer), sg)
    return guc, gus, dnc, dns


def bf16_tensor(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def packed_experts_device(cfg: I.LayerConfig, kind: str, count: int, layer: int = 0,
                          device="cuda") -> Tuple[torch.Tensor, ...]:
    """(gu_codes, gu_scales, dn_codes, dn_scales) of `count` experts in the
    packed tile order moe_forward reads, one flat row per expert.  Each expert
    is drawn in canonical form into a scratch buffer and packed on the device."""
    d, f = cfg.d_model, cfg.d_ff
    gsb, dsb = M.moe_packed_scale_bytes(2 * f, d), M.moe_packed_scale_bytes(d, f)
    out = (torch.empty((count, f * d), dtype=torch.uint8, device=device),
           torch.empty((count, gsb), dtype=torch.uint8, device=device),
           torch.empty((count, d * f // 2), dtype=torch.uint8, device=device),
           torch.empty((count, dsb), dtype=torch.uint8, device=device))
    tgc = torch.empty((2 * f, d // 2), dtype=torch.uint8, device=device)
    tgs = torch.empty((2 * f, d // 32), dtype=torch.uint8, device=device)
    tdc = torch.empty((d, f // 2), dtype=torch.uint8, device=device)
    tds = torch.empty((d, f // 32), dtype=torch.uint8, device=device)
    sg = I.weight_sigma(d)
    st = torch.cuda.current_stream().cuda_stream
    for i in range(count):
        slot = I.expert_slot(kind, i)
        gen_mx_matrix_device(tgc, tgs, 2 * f, d, cfg.seed, I.stream_id(I.KIND_GU_CODES, slot, layer), sg)
        gen_mx_matrix_device(tdc, tds, d, f, cfg.seed, I.stream_id(I.KIND_DN_CODES, slot, layer), sg)
        M.moe_pack_mx4(tgc.data_ptr(), tgs.data_ptr(), 1, 2 * f, d, 1, out[0][i].data_ptr(),
                       out[1][i].data_ptr(), st)
        M.moe_pack_mx4(tdc.data_ptr(), tds.data_ptr(), 1, d, f, 0, out[2][i].data_ptr(),
                       out[3][i].data_ptr(), st)
    return out


def device_weights(cfg: I.LayerConfig, layer: int = 0, device="cuda") -> DeviceWeights:
    """The layer's weights on the GPU, expert matrices packed for moe_forward."""
    guc, gus, dnc, dns = packed_experts_device(cfg, "routed", cfg.num_experts, layer, device)
    if cfg.num_shared:
        sguc, sgus, sdnc, sdns = packed_experts_device(cfg, "shared", cfg.num_shared, layer, device)
    else:
        sguc = sgus = sdnc = sdns = None
    wr = torch.from_numpy(I.gen_router_w(cfg, layer)).to(device)
    b = I.gen_router_b(cfg)
    br = torch.from_numpy(b).to(device) if b is not None else None
    return DeviceWeights(guc, gus, dnc, dns, sguc, sgus, sdnc, sdns, wr, br)


def device_weights_canonical(cfg: I.LayerConfig, layer: int = 0, device="cuda") -> DeviceWeights:
    """The same weights as device_weights, expert matrices in canonical form."""
    guc, gus, dnc, dns = gen_experts_device(cfg, "routed", cfg.num_experts, layer, device)
    if cfg.num_shared:
        sguc, sgus, sdnc, sdns = gen_experts_device(cfg, "shared", cfg.num_shared, layer, device)
    else:
        sguc = sgus = sdnc = sdns = None
    wr = torch.from_numpy(I.gen_router_w(cfg, layer)).to(device)
    b = I.gen_router_b(cfg)
    br = torch.from_numpy(b).to(device) if b is not None else None
    return DeviceWeights(guc, gus, dnc, dns, sguc, sgus, sdnc, sdns, wr, br, M.MOE_WEIGHTS_CANONICAL)


def device_x(cfg: I.LayerConfig, tokens: Optional[int] = None, layer: int = 0,
             device="cuda") -> torch.Tensor:
    return bf16_tensor(I.gen_x(cfg, tokens, layer), device)
