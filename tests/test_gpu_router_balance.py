"""GPU parity of the router-bias balancing step (moe_router_bias_update)
through the C ABI: bit-exact against the oracle's step on the loads of a real
forward, and repeated forward + step rounds evening out a Zipf-skewed load."""

import numpy as np
import pytest
import torch

from mxfp4_expert_grouped_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mxfp4_expert_grouped_amd import mxmoe
    mxmoe.load_library()
    torch.cuda.set_device(0)
    yield


import parity as P  # noqa: E402


def _round(layer, M, x, offs, b_dev, rate):
    layer.forward(x, taps={"expert_offsets": offs})
    M.moe_router_bias_update(layer.plan, offs.data_ptr(), x.shape[0], rate, b_dev.data_ptr(),
                             torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return np.diff(offs.cpu().numpy())


@pytest.mark.parametrize("T", [5, 300, 1500])
def test_bias_step_matches_oracle_and_evens_the_load(T):
    from mxfp4_expert_grouped_amd import mxmoe as M
    from mxfp4_expert_grouped_amd.layer import MoeLayer
    from oracle import moe as OM
    cfg = I.LayerConfig("bal", T, 256, 64, 4, 128, 1, zipf_bias=True, seed=80 + T)
    W = P.IG.device_weights(cfg)
    b = I.gen_router_b(cfg)
    b_dev = torch.from_numpy(b.copy()).cuda()
    W.router_b = b_dev
    layer = MoeLayer(cfg.d_model, cfg.d_ff, cfg.num_experts, cfg.top_k, cfg.num_shared, T, W)
    x = P.IG.device_x(cfg)
    offs = torch.empty(cfg.num_experts + 1, dtype=torch.int32, device="cuda")
    rate = 0.2
    b_host = b.copy()
    first = None
    P.log(f"router balance: T={T} E={cfg.num_experts} k={cfg.top_k}")
    for it in range(25):
        counts = _round(layer, M, x, offs, b_dev, rate)
        first = counts if first is None else first
        b_host = OM.router_bias_update(b_host, counts, T, cfg.top_k, rate)
        assert np.array_equal(b_dev.cpu().numpy().view(np.uint32), b_host.view(np.uint32)), f"round {it}"
    layer.forward(x, taps={"expert_offsets": offs})
    torch.cuda.synchronize()
    last = np.diff(offs.cpu().numpy())
    P.log(f"T={T}: max load {first.max()} -> {last.max()}, std {first.std():.1f} -> {last.std():.1f}")
    if T >= 300:
        assert last.max() < first.max() and last.std() < 0.6 * first.std()
