"""Torch-facing convenience wrapper: device buffers from PyTorch, every step of
the layer in the HIP library (through :mod:`.mxmoe`)."""

from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional

import torch

from . import mxmoe as M


@dataclass
class DeviceWeights:
    """MXFP4 expert weights (packed tile order, one flat row per expert, or
    canonical [E, N, K/2] codes and [E, N, K/32] scales, as ``layout`` says)
    and router parameters resident on one GPU."""
    gu_codes: torch.Tensor    # uint8 [E, d_ff*d]
    gu_scales: torch.Tensor   # uint8 [E, moe_packed_scale_bytes(2 d_ff, d)]
    dn_codes: torch.Tensor    # uint8 [E, d*d_ff/2]
    dn_scales: torch.Tensor   # uint8 [E, moe_packed_scale_bytes(d, d_ff)]
    sgu_codes: Optional[torch.Tensor]
    sgu_scales: Optional[torch.Tensor]
    sdn_codes: Optional[torch.Tensor]
    sdn_scales: Optional[torch.Tensor]
    router_w: torch.Tensor    # float32 [E, d]
    router_b: Optional[torch.Tensor]
    layout: int = M.MOE_WEIGHTS_PACKED

    def abi(self) -> M.MoeWeights:
        p = lambda t: (t.data_ptr() if t is not None else None)
        return M.MoeWeights(p(self.gu_codes), p(self.gu_scales), p(self.dn_codes),
                            p(self.dn_scales), p(self.sgu_codes), p(self.sgu_scales),
                            p(self.sdn_codes), p(self.sdn_scales), p(self.router_w),
                            p(self.router_b), self.layout)


class MoeLayer:
    """One MoE layer on the current CUDA/HIP device."""

    def __init__(self, d_model: int, d_ff: int, num_experts: int, top_k: int, num_shared: int,
                 max_tokens: int, weights: DeviceWeights, flags: int = 0):
        self.shape = dict(d_model=d_model, d_ff=d_ff, num_experts=num_experts, top_k=top_k,
                          num_shared=num_shared, max_tokens=max_tokens, flags=flags)
        self.plan = M.moe_plan(d_model, d_ff, num_experts, top_k, num_shared, max_tokens, flags)
        self.weights = weights
        self._wabi = weights.abi()
        self._ws: Optional[torch.Tensor] = None

    def __del__(self):
        try:
            M.moe_plan_destroy(self.plan)
        except Exception:
            pass

    def workspace_bytes(self, num_tokens: int) -> int:
        return M.moe_workspace_bytes(self.plan, num_tokens)

    def workspace(self, num_tokens: int, device=None) -> torch.Tensor:
        need = self.workspace_bytes(num_tokens)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 256), dtype=torch.uint8,
                                   device=device or self.weights.router_w.device)
        return self._ws

    def forward(self, x: torch.Tensor, y: Optional[torch.Tensor] = None,
                taps: Optional[Dict[str, torch.Tensor]] = None,
                workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
        """x: bfloat16 [T, d] on the device -> y bfloat16 [T, d]."""
        assert x.dtype == torch.bfloat16 and x.is_contiguous() and x.dim() == 2
        t = x.shape[0]
        if y is None:
            y = torch.empty_like(x)
        ws = workspace if workspace is not None else self.workspace(t, x.device)
        tp = None
        if taps:
            tp = M.MoeTaps(**{k: v.data_ptr() for k, v in taps.items()})
        M.moe_forward(self.plan, self._wabi, x.data_ptr(), t, y.data_ptr(), ws.data_ptr(),
                      ws.numel(), tp, torch.cuda.current_stream().cuda_stream)
        return y


def quantize_act(src: torch.Tensor):
    """MXFP8 codes and scales of a 2-D bf16/fp32 tensor along its last axis."""
    assert src.dim() == 2 and src.stride(1) == 1
    rows, cols = src.shape
    codes = torch.empty((rows, cols), dtype=torch.uint8, device=src.device)
    scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=src.device)
    dt = M.MOE_SRC_FP32 if src.dtype == torch.float32 else M.MOE_SRC_BF16
    assert src.dtype in (torch.float32, torch.bfloat16)
    M.moe_quantize_act(src.data_ptr(), dt, rows, cols, src.stride(0), codes.data_ptr(),
                       scales.data_ptr(), torch.cuda.current_stream().cuda_stream)
    return codes, scales
