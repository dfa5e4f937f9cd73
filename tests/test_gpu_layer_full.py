"""GPU parity of the full-size layer (d=7168, 896 experts, top-16, d_ff=2048,
2 shared) at each benchmark workload, in the launch configuration the
benchmark times.

The whole layer runs on the GPU for every token; the oracle recomputes routing,
permutation and x quantisation for every token and the expert outputs for a
sample of tokens (each token's output depends only on its own row).
"""

import numpy as np
import pytest
import torch

from mxfp4_expert_grouped_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def big():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mxfp4_expert_grouped_amd import mxmoe
    mxmoe.load_library()
    import parity as P
    cfg = I.CONFIGS["decode1"]
    P.log("generating the 896-expert layer on the GPU")
    W = P.IG.device_weights(cfg)
    torch.cuda.synchronize()
    ref = I.ExpertWeights(cfg)  # numpy twin, generated lazily per expert
    yield P, W, ref
    del W
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,sample", [
    ("decode1", [0]),
    ("decode256", [3, 200]),
    ("prefill8k", [17, 8000]),
    ("prefill32k_skew", [0, 31000]),
])
def test_full_layer(big, name, sample):
    P, W, ref = big
    cfg = I.CONFIGS[name]
    b = I.gen_router_b(cfg)
    W.router_b = torch.from_numpy(b).cuda() if b is not None else None
    x_bits = I.gen_x(cfg)
    x = P.IG.bf16_tensor(x_bits)
    P.log(f"{name}: GPU forward T={cfg.tokens}")
    g = P.run_gpu(cfg, W, x, skip=("gu_acc",))
    # every token: routing ids valid, weights sum to one, outputs finite
    assert np.all(np.abs(g["topk_w"].sum(1) - 1) < 1e-5)
    y = P.bf16_bits_to_f64(g["y"])
    assert np.all(np.isfinite(y))
    res, differ = P.compare_layer(cfg, x_bits, I.gen_router_w(cfg), b, ref, g, tokens=sample)
    # the x bytes of every token, not only the sampled ones
    from oracle import moe as OM, mx as OX
    step = max(1, cfg.tokens // 512)
    rows = np.arange(0, cfg.tokens, step)
    xc, xs = OX.mx_quantize(OM.bf16_to_f64(x_bits[rows]), "e4m3")
    assert np.array_equal(g["x_codes"][rows], xc) and np.array_equal(g["x_scales"][rows], xs)
    if name == "prefill32k_skew":
        counts = np.diff(g["expert_offsets"])
        P.log(f"skew: max rows/expert {counts.max()}, experts touched {(counts > 0).sum()}, "
              f">2000 rows: {(counts > 2000).sum()}")
        assert counts.max() > 2000 and (counts == 0).sum() > 0
    W.router_b = None
