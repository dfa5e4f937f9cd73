"""GPU parity of the A16W4 variant (bf16 activations, MXFP4 weights) through
the C ABI against the oracle's A16W4 layer: the gate/up accumulators bit for
bit in the exact-arithmetic regime (the bf16 MFMA on weights expanded from
FP4 in registers), the whole layer with the parity rules on the streaming
kernels' shapes (K split and whole items, ragged token counts, top-20, five
shared experts, the Zipf bias) and on the 256-row prefill tiles (ragged
last tiles, several tiles per expert, a d_model that ends on half a column
block); the full-size workloads are in the full-layer tests."""

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


EXACT = [
    ("ksplit", 40, 256, 128, 8, 2, None),
    ("ksplit_k1024", 40, 1024, 512, 8, 2, None),
    ("ksplit_wide_scales", 40, 256, 128, 8, 2, (122, 132)),
    ("whole_items", 2048, 256, 512, 1024, 8, (122, 132)),
    # d_model 512: enough down items for the two-group (wide) ones
    ("whole_items_wide_down", 2048, 512, 512, 1024, 8, (122, 132)),
    # 32 tokens: routing launch with the shared items, then two-group routed
    # gate_up items
    ("phases_wide_items", 32, 512, 2048, 256, 16, None),
    # at most four tokens: four-row activation slots, seven-slot ring
    ("four_row_slots", 3, 256, 128, 8, 2, None),
    ("four_row_slots_wide_scales", 4, 256, 128, 8, 3, (122, 132)),
    # from 24 rows per expert on average: 256-row tiles on the bf16 MFMA
    ("prefill_tiles", 300, 256, 128, 8, 2, None),
    ("prefill_tiles_wide_scales", 300, 256, 256, 8, 2, (122, 132)),
    ("prefill_k1024", 200, 1024, 512, 4, 2, None),
    # 600 rows per shared expert (tiles of 256, 256, 88); d_model 384: the
    # last down column block is half a block
    ("prefill_d384_shared_tiles", 600, 384, 256, 8, 2, None),
]


@pytest.mark.parametrize("name,T,d,f,E,k,scales", EXACT, ids=[c[0] for c in EXACT])
def test_a16w4_gate_up_accumulators_exact(name, T, d, f, E, k, scales):
    """x integer-valued in [-16, 16] (exact in bf16), weights with bounded
    scale bytes: every product is exact and every partial sum below 2^24 of
    the products' granularity (asserted), so the bf16-MFMA accumulators must
    equal the float64 sums bit for bit."""
    cfg = I.LayerConfig("a16_" + name, T, d, E, k, f, 1, seed=22)
    bits = P.integer_x(cfg, 6)
    x = P.IG.bf16_tensor(bits)
    if scales is None:
        W = P.IG.device_weights(cfg)
        ref = I.ExpertWeights(cfg)
    else:
        W, ref = P.weights_with_scale_range(cfg, 78, *scales)
    P.log(f"A16W4 exact case {name}: T={T} d={d} d_ff={f} E={E} k={k} scale bytes {scales}")
    g = P.run_gpu(cfg, W, x, a16=True)
    tokens = None if T <= 64 else sorted(set(range(0, T, max(1, T // 48))) | {T - 1})
    if scales is not None:
        # the accumulators only: with scale bytes up to 2^5 the integer rows
        # reach |g| ~ 1e4, where silu(g) leaves the fp32 range (exp(-g)
        # overflows for g < -88.7) and h is ~1e-38 or ~1e8 -- values the layer
        # never sees; the layer comparison runs on the standard weights
        from oracle import moe as OM
        res = OM.forward(bits, I.gen_router_w(cfg), None, ref, num_experts=E, top_k=k, num_shared=1,
                         d_ff=f, tokens=tokens, topk_ids=g["topk_ids"], intermediates=True,
                         activations="bf16")
        assert np.array_equal(g["topk_ids"], OM.topk_select(res.logits, k)[0])
    else:
        res, differ = P.compare_layer(cfg, bits, I.gen_router_w(cfg), None, ref, g, tokens=tokens,
                                      activations="bf16")
        assert not differ
    # the lowest scale byte of the experts the compared rows use
    lo = scales[0] if scales is not None else ref.min_scale_byte()
    q = 0.5 * 2.0 ** (lo - 127)
    acc = g["gu_acc"]
    nmis = nrows = 0
    for r, mid in list(res.mid_rows.items()) + [(T * k + t, m) for (s, t), m in res.mid_shared.items()]:
        assert np.all(mid["gu_abs"] < 2.0 ** 24 * q), "case outside the exact regime"
        nmis += int(np.sum(acc[r].astype(np.float64) != mid["gu"]))
        nrows += 1
    P.log(f"{name}: {nrows} rows of gate/up accumulators, {nmis} differ from the exact values")
    assert nrows > 0 and nmis == 0


def _case(cfg, bias=None, tokens=None):
    x_bits = I.gen_x(cfg)
    W = P.IG.device_weights(cfg)
    b = I.gen_router_b(cfg) if bias is None else np.asarray(bias, np.float32)
    if b is not None:
        W.router_b = torch.from_numpy(b).cuda()
    P.log(f"A16W4 case {cfg}")
    g = P.run_gpu(cfg, W, P.IG.bf16_tensor(x_bits), a16=True)
    return P.compare_layer(cfg, x_bits, I.gen_router_w(cfg), b, I.ExpertWeights(cfg), g, tokens,
                           activations="bf16")


def test_a16w4_tiny():
    _case(I.CONFIGS["tiny"])


@pytest.mark.parametrize("T", [1, 3, 4, 5, 13, 64, 100])
def test_a16w4_ragged(T):
    _case(I.LayerConfig("a16_ragged", T, 256, 16, 2, 128, 1, seed=100 + T))


def test_a16w4_top_20_and_five_shared():
    _case(I.LayerConfig("a16_k20", 3, 256, 48, 20, 128, 1, seed=120))
    _case(I.LayerConfig("a16_s5", 5, 256, 16, 2, 128, 5, seed=121))


def test_a16w4_zipf_bias():
    _case(I.LayerConfig("a16_skew", 300, 512, 64, 4, 256, 2, zipf_bias=True, seed=122),
          tokens=list(range(0, 300, 7)) + [299])


@pytest.mark.parametrize("cfg", [
    I.LayerConfig("a16_prefill", 700, 512, 16, 2, 256, 1, seed=130),
    I.LayerConfig("a16_prefill_d384", 400, 384, 8, 2, 256, 2, seed=131),
    I.LayerConfig("a16_prefill_k1024", 260, 1024, 8, 3, 512, 1, seed=132),
], ids=["d512", "d384_two_shared", "d1024"])
def test_a16w4_prefill(cfg):
    _case(cfg)


def test_a16w4_prefill_zipf_bias():
    # 128 rows per expert on average, skewed: one to many tiles per expert
    _case(I.LayerConfig("a16_skew_prefill", 2048, 512, 64, 4, 256, 2, zipf_bias=True, seed=133),
          tokens=list(range(0, 2048, 23)) + [2047])


def test_a16w4_differs_from_a8w4_and_is_deterministic():
    cfg = I.LayerConfig("a16_det", 40, 512, 16, 2, 256, 2, seed=123)
    x = P.IG.device_x(cfg)
    W = P.IG.device_weights(cfg)
    a = P.run_gpu(cfg, W, x, taps=False, a16=True, workspace_fill=0)["y"]
    b = P.run_gpu(cfg, W, x, taps=False, a16=True, workspace_fill=0xFF)["y"]
    c = P.run_gpu(cfg, W, x, taps=False)["y"]
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    ya, yc = a.float(), c.float()
    assert (ya - yc).norm() > 1e-4 * ya.norm()
