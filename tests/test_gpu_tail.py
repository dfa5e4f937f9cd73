"""GPU parity of the LatentMoE tail y = MXFP8(RMSNorm(z)) W_up^T + s through
the C ABI (moe_latent_tail), against the oracle's latent_tail: the small
widths reach the weight-streaming projection (fewer than 24 rows) and the
256-row one (per-step and grouped activation scales); the full width 7168
at decode and prefill sizes, the last on sampled rows; s absent; and the
tail chained behind the layer's own routed and shared sums."""

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


def _pack(codes, scales, rows, k):
    from mxfp4_expert_grouped_amd import mxmoe as M
    sb = M.moe_packed_scale_bytes(rows, k)
    cp = torch.empty(rows * k // 2, dtype=torch.uint8, device="cuda")
    sp = torch.empty(sb, dtype=torch.uint8, device="cuda")
    tc, ts = torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda()
    M.moe_pack_mx4(tc.data_ptr(), ts.data_ptr(), 1, rows, k, 0, cp.data_ptr(), sp.data_ptr(),
                   torch.cuda.current_stream().cuda_stream)
    return cp, sp


def run_tail(z, s, gamma, eps, up_c, up_s, hidden, canonical=False):
    from mxfp4_expert_grouped_amd import mxmoe as M
    T, l = z.shape
    if canonical:
        cp, sp = torch.from_numpy(up_c).cuda(), torch.from_numpy(up_s).cuda()
    else:
        cp, sp = _pack(up_c, up_s, hidden, l)
    g = torch.from_numpy(gamma).cuda()
    zt = torch.from_numpy(np.ascontiguousarray(z)).cuda()
    st = torch.from_numpy(np.ascontiguousarray(s)).cuda() if s is not None else None
    y = torch.empty((T, hidden), dtype=torch.bfloat16, device="cuda")
    inv = torch.empty(T, dtype=torch.float32, device="cuda")
    codes = torch.empty((T, l), dtype=torch.uint8, device="cuda")
    scales = torch.empty((T, l // 32), dtype=torch.uint8, device="cuda")
    nb = M.moe_latent_tail_workspace_bytes(T, l, hidden)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda")
    ws.fill_(0xA5)
    W = M.MoeTailWeights(cp.data_ptr(), sp.data_ptr(), g.data_ptr(),
                         M.MOE_WEIGHTS_CANONICAL if canonical else M.MOE_WEIGHTS_PACKED)
    taps = M.MoeTailTaps(inv.data_ptr(), codes.data_ptr(), scales.data_ptr())
    M.moe_latent_tail(T, l, hidden, eps, W, zt.data_ptr(), st.data_ptr() if st is not None else None,
                      y.data_ptr(), ws.data_ptr(), nb, taps, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return y, inv.cpu().numpy(), codes.cpu().numpy(), scales.cpu().numpy()


@pytest.mark.parametrize("T,l,H,with_s", [
    (1, 256, 256, True), (5, 256, 512, True), (13, 384, 256, False),
    (40, 1024, 256, True), (300, 384, 512, True), (300, 512, 768, False),
    (100, 2048, 512, False),  # four K slices, no shared output
    (300, 2048, 256, True),   # four K slices over a full and a partial tile
    (60, 512, 384, True), (3, 256, 384, True),  # hidden an odd multiple of 128
    (1, 7168, 7168, True), (256, 7168, 7168, True), (8192, 7168, 7168, True),
])
def test_tail_matches_oracle(T, l, H, with_s):
    P.log(f"tail case T={T} latent={l} hidden={H} s={'yes' if with_s else 'no'}")
    z, s, gamma = I.gen_tail_inputs(T, l, H, seed=T + l)
    up_c, up_s = I.gen_up_matrix(H, l, seed=T + l)
    if not with_s:
        s = None
    y, inv, codes, scales = run_tail(z, s, gamma, 1e-6, up_c, up_s, H)
    rows = None if T <= 300 else sorted(set(range(0, T, T // 48)) | {T - 1, 255, 256})
    P.compare_tail(z, s, gamma, 1e-6, up_c, up_s, y, inv, codes, scales, rows)


def test_tail_zero_rows_with_eps():
    # an all-zero z row: 1/rms = 1/sqrt(eps), n = 0, y = s exactly (bf16 of s)
    T, l, H = 3, 256, 256
    z, s, gamma = I.gen_tail_inputs(T, l, H, seed=3)
    z[1] = 0
    up_c, up_s = I.gen_up_matrix(H, l, seed=3)
    y, inv, codes, scales = run_tail(z, s, gamma, 1e-6, up_c, up_s, H)
    assert np.all(codes[1] & 0x7F == 0) and np.all(scales[1] == 0)
    from oracle import moe as OM
    assert np.array_equal(y[1].view(torch.int16).cpu().numpy().view(np.uint16), OM.f64_to_bf16(s[1]))
    P.compare_tail(z, s, gamma, 1e-6, up_c, up_s, y, inv, codes, scales)


def test_tail_chained_behind_the_layer():
    # the layer's fp32 routed and shared sums feed the tail (latent = hidden =
    # the experts' width), straight from moe_forward's taps; against the
    # oracle's chain (its own float64 sums rounded to fp32).  The tail
    # re-quantises the normalised sums to MXFP8, so the layer's own error
    # (relative ~1e-3 on the routed sum) flips about 16 x 1e-3 of those codes,
    # each by one E4M3 step (~1/16 of the element): about 0.8 % relative L2
    # on the projection, which is what the chain must stay within (2e-2);
    # the tail itself, on identical inputs, is held to 5e-3 above
    from oracle import moe as OM
    cfg = I.LayerConfig("chain", 24, 512, 16, 2, 256, 2, seed=70)
    x_bits = I.gen_x(cfg)
    W = P.IG.device_weights(cfg)
    g = P.run_gpu(cfg, W, P.IG.bf16_tensor(x_bits), skip=("gu_acc",))
    res = OM.forward(x_bits, I.gen_router_w(cfg), None, I.ExpertWeights(cfg), num_experts=16,
                     top_k=2, num_shared=2, d_ff=256)
    _, _, gamma = I.gen_tail_inputs(1, 512, 512, seed=71)
    up_c, up_s = I.gen_up_matrix(512, 512, seed=71)
    y, inv, codes, scales = run_tail(g["y_routed"], g["y_shared"], gamma, 1e-6, up_c, up_s, 512)
    y_o = OM.latent_tail(res.y_routed.astype(np.float32), gamma, 1e-6, up_c, up_s,
                         res.y_shared.astype(np.float32))
    yg = P.bf16_bits_to_f64(y)
    rel = np.linalg.norm(yg - y_o) / np.linalg.norm(y_o)
    P.log(f"chained tail y: rel_l2={rel:.3e}")
    assert rel <= 2e-2 and np.all(np.isfinite(yg))
