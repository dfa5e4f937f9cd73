"""Canonical (unpacked) MXFP4 weights through the C ABI: moe_forward and
moe_latent_tail read them when the layout tag says MOE_WEIGHTS_CANONICAL, and
every kernel path must then give bit for bit what it gives on the same
matrices packed by moe_pack_mx4 -- the same operands reach the same MFMAs in
the same order; only the copies' addresses and the scale bytes' selection
differ.  The paths: the few-token two-launch gate_up, K-split and
whole-item decode GEMMs (one- and two-group down items), the prefill GEMM
with per-step and grouped scales and a half-used last output block, the
A16W4 variant, and the tail's split-K GEMV, 256-row and K-sliced
projections.  The layer's parity against the oracle itself is covered by the
other GPU tests (on packed weights)."""

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

CASES = [
    # name, T, d, d_ff, E, k, S, a16
    ("few_tokens_phases", 8, 256, 128, 16, 2, 1, False),
    ("stream_ksplit", 40, 256, 128, 8, 2, 1, False),
    ("stream_whole_items_wide_down", 2048, 512, 512, 1024, 8, 1, False),
    ("phases_whole_items", 32, 512, 2048, 256, 16, 1, False),
    ("prefill_step_scales", 300, 256, 128, 8, 2, 1, False),
    ("prefill_grouped_scales", 300, 1024, 512, 8, 2, 2, False),
    ("prefill_d384", 300, 384, 128, 8, 2, 1, False),
    ("a16w4_few_tokens", 8, 256, 128, 16, 2, 1, True),
    ("a16w4_four_tokens", 4, 256, 128, 16, 2, 1, True),
    ("a16w4_stream", 200, 512, 256, 64, 4, 1, True),
    ("a16w4_whole_items_wide_down", 2048, 512, 512, 1024, 8, 1, True),
    ("a16w4_phases_wide_items", 32, 512, 2048, 256, 16, 1, True),
    ("a16w4_prefill", 300, 1024, 512, 8, 2, 2, True),
    ("a16w4_prefill_d384", 300, 384, 128, 8, 2, 1, True),
]


def _taps(cfg, T, a16):
    t = P.alloc_taps(cfg, T, a16=a16)
    return t


@pytest.mark.parametrize("name,T,d,f,E,k,S,a16", CASES, ids=[c[0] for c in CASES])
def test_canonical_weights_match_packed_bit_for_bit(name, T, d, f, E, k, S, a16):
    from mxfp4_expert_grouped_amd import mxmoe as M
    cfg = I.LayerConfig(name, T, d, E, k, f, S, seed=31)
    P.log(f"canonical case {name}: T={T} d={d} d_ff={f} E={E} k={k} S={S} a16={a16}")
    x = P.IG.device_x(cfg)
    Wp = P.IG.device_weights(cfg)
    Wc = P.IG.device_weights_canonical(cfg)
    assert Wc.layout == M.MOE_WEIGHTS_CANONICAL
    gp = P.run_gpu(cfg, Wp, x, a16=a16)
    gc = P.run_gpu(cfg, Wc, x, a16=a16)
    yp = gp.y.view(torch.int16).cpu().numpy()
    yc = gc.y.view(torch.int16).cpu().numpy()
    assert np.array_equal(yp, yc), f"{name}: y differs in {(yp != yc).sum()} of {yp.size}"
    for tap in gp.taps:
        a, b = gp[tap], gc[tap]
        assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8)), f"{name}: tap {tap} differs"


@pytest.mark.parametrize("T,l,H", [(5, 1024, 256), (40, 512, 384), (300, 2048, 256), (256, 1024, 512)])
def test_tail_canonical_matches_packed(T, l, H):
    import test_gpu_tail as TT
    P.log(f"tail canonical case T={T} latent={l} hidden={H}")
    z, s, gamma = I.gen_tail_inputs(T, l, H, seed=T + 3)
    up_c, up_s = I.gen_up_matrix(H, l, seed=T + 3)
    yp = TT.run_tail(z, s, gamma, 1e-6, up_c, up_s, H)[0]
    yc = TT.run_tail(z, s, gamma, 1e-6, up_c, up_s, H, canonical=True)[0]
    a, b = yp.view(torch.int16).cpu().numpy(), yc.view(torch.int16).cpu().numpy()
    assert np.array_equal(a, b), f"tail T={T}: y differs in {(a != b).sum()} of {a.size}"
