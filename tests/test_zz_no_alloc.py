"""moe_forward_noalloc (the entry point for callers that cannot allocate)
against moe_forward, through the C ABI: the same bytes out, on two calls in
a row, the second with fewer tokens than the first (the scratch array keeps
the first call's contents)."""

import numpy as np
import pytest
import torch

from mxfp4_expert_grouped_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mxfp4_expert_grouped_amd import mxmoe
    mxmoe.load_library()
    torch.cuda.set_device(0)
    return mxmoe


def _taps(cfg, T, a16=False):
    k, S, d, f = cfg.top_k, cfg.num_shared, cfg.d_model, cfg.d_ff
    R = T * k + S * T
    h = (dict(h_bf16=torch.empty((R, f), dtype=torch.int16, device="cuda")) if a16
         else dict(h_codes=torch.empty((R, f), dtype=torch.uint8, device="cuda")))
    return dict(topk_ids=torch.empty((T, k), dtype=torch.int32, device="cuda"),
                y_routed=torch.empty((T, d), dtype=torch.float32, device="cuda"), **h)


def _both(M, layer, x, cfg, a16=False):
    T = x.shape[0]
    st = torch.cuda.current_stream().cuda_stream
    y_ref = torch.empty_like(x)
    t_ref = _taps(cfg, T, a16)
    layer.forward(x, y=y_ref, taps=t_ref)
    y = torch.full_like(x, float("nan"))
    t = _taps(cfg, T, a16)
    M.moe_forward_noalloc(layer.plan, layer._wabi, x.data_ptr(), T, y.data_ptr(),
                          M.MoeTaps(**{n: v.data_ptr() for n, v in t.items()}), st)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
    for n in t:
        assert torch.equal(t[n], t_ref[n]), n


@pytest.mark.parametrize("name,T1,T2,a16", [
    ("small", 40, 7, False), ("decode_full", 256, 1, False),
    # 75 then 37.5 rows per expert: the 256-row prefill kernels both times
    ("prefill", 600, 300, False),
    # A16W4: prefill kernels, then the weight-streaming ones
    ("a16w4_prefill_then_decode", 600, 40, True),
])
def test_noalloc_matches_forward_on_two_calls(lib, name, T1, T2, a16):
    from mxfp4_expert_grouped_amd import inputs_gpu as IG
    from mxfp4_expert_grouped_amd.layer import MoeLayer
    cfg = (I.CONFIGS["decode256"] if name == "decode_full"
           else I.LayerConfig("noalloc", T1, 256, 16, 2, 128, 2, seed=90))
    W = IG.device_weights(cfg)
    layer = MoeLayer(cfg.d_model, cfg.d_ff, cfg.num_experts, cfg.top_k, cfg.num_shared, T1, W,
                     flags=lib.MOE_FLAG_A16W4 if a16 else 0)
    x1 = IG.device_x(cfg, tokens=T1, layer=1)
    x2 = IG.device_x(cfg, tokens=T2, layer=2)
    print(f"noalloc case {name}: T={T1} then T={T2}", flush=True)
    _both(lib, layer, x1, cfg, a16)
    _both(lib, layer, x2, cfg, a16)
    del layer, W
    torch.cuda.empty_cache()
