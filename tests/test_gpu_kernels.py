"""GPU parity at small and medium sizes, through the C ABI, against the oracle.

Covers: the GPU twin of the input generator, the MXFP8 quantiser (bit-exact,
bf16 and fp32 sources, adversarial blocks), the scaled-MFMA operand layout in
the exact-arithmetic regime (bit-exact gate/up accumulators), the tiny layer
with every tap, ragged token counts on both permutation paths and both tile
heights, a single expert receiving every token, k=1 without shared experts,
determinism and indifference to workspace contents.
"""

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
    mxmoe.load_library()  # raises if the HIP library is missing: no fallback
    torch.cuda.set_device(0)
    yield


import parity as P  # noqa: E402  (after the marker; imports torch-side helpers)


# ---------------------------------------------------------------------------
# input generator twin
# ---------------------------------------------------------------------------

def test_gpu_generator_matches_numpy_tiny_all_experts():
    cfg = I.CONFIGS["tiny"]
    ref = I.ExpertWeights(cfg)
    Wr = P.IG.gen_experts_device(cfg, "routed", cfg.num_experts)
    Ws = P.IG.gen_experts_device(cfg, "shared", cfg.num_shared)
    for e in range(cfg.num_experts):
        for got, want in zip((t[e] for t in Wr), ref("routed", e)):
            assert np.array_equal(got.cpu().numpy(), want)
    for got, want in zip((t[0] for t in Ws), ref("shared", 0)):
        assert np.array_equal(got.cpu().numpy(), want)


def _pack_reference(codes, scales, rows, k, interleave):
    """The packed tile order, written out with plain loops over its definition."""
    nsteps = k // 128
    cp = np.zeros((rows // 64, nsteps, 4, 64, 16), np.uint8)
    sp = np.zeros((rows // 64, nsteps, 64, 4), np.uint8)

    def row(G, j, r):
        if interleave:
            return (j // 2) * (rows // 2) + 32 * G + 16 * (j % 2) + r
        return 64 * G + 16 * j + r

    for G in range(rows // 64):
        for s in range(nsteps):
            for lane in range(64):
                g, r = lane // 16, lane % 16
                for j in range(4):
                    cp[G, s, j, lane] = codes[row(G, j, r), 64 * s + 16 * g: 64 * s + 16 * g + 16]
                    sp[G, s, lane, j] = scales[row(G, j, r), 4 * s + g]
    return cp.reshape(-1), sp.reshape(-1)


@pytest.mark.parametrize("rows,k,interleave", [(64, 128, 0), (64, 256, 1), (128, 640, 0), (192, 2048, 1),
                                               (64, 7168, 1)])
def test_pack_mx4_layout(rows, k, interleave):
    from mxfp4_expert_grouped_amd import mxmoe as M
    rng = np.random.default_rng(rows + k)
    mats = 3
    codes = rng.integers(0, 256, size=(mats, rows, k // 2), dtype=np.uint8)
    scales = rng.integers(0, 255, size=(mats, rows, k // 32), dtype=np.uint8)
    sb = M.moe_packed_scale_bytes(rows, k)
    assert sb == rows * k // 32
    cp = torch.empty(mats * rows * k // 2, dtype=torch.uint8, device="cuda")
    spk = torch.empty(mats * sb, dtype=torch.uint8, device="cuda")
    M.moe_pack_mx4(None, None, 0, rows, k, interleave, None, None)  # zero matrices: no-op
    tc, ts = torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda()
    M.moe_pack_mx4(tc.data_ptr(), ts.data_ptr(), mats, rows, k, interleave, cp.data_ptr(), spk.data_ptr(),
                   torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    cpn, spn = cp.cpu().numpy(), spk.cpu().numpy()
    for m in range(mats):
        rc, rs = _pack_reference(codes[m], scales[m], rows, k, interleave)
        assert np.array_equal(cpn[m * rows * k // 2:(m + 1) * rows * k // 2], rc)
        assert np.array_equal(spn[m * sb:(m + 1) * sb], rs)


def test_gpu_generator_matches_numpy_full_shape_sample():
    cfg = I.CONFIGS["decode1"]
    guc, gus, dnc, dns = P.IG.gen_experts_device(cfg, "routed", 1)
    sg = I.weight_sigma(cfg.d_model)
    c, s = I.gen_mx_matrix(cfg.seed, I.stream_id(I.KIND_GU_CODES, 0), 2 * cfg.d_ff, cfg.d_model, sg,
                           row0=1000, nrows=64)
    assert np.array_equal(guc[0, 1000:1064].cpu().numpy(), c)
    assert np.array_equal(gus[0, 1000:1064].cpu().numpy(), s)
    c, s = I.gen_mx_matrix(cfg.seed, I.stream_id(I.KIND_DN_CODES, 0), cfg.d_model, cfg.d_ff, sg,
                           row0=7100, nrows=68)
    assert np.array_equal(dnc[0, 7100:].cpu().numpy(), c)
    assert np.array_equal(dns[0, 7100:].cpu().numpy(), s)


# ---------------------------------------------------------------------------
# MXFP8 quantiser
# ---------------------------------------------------------------------------

def _adversarial_rows(rng, cols):
    rows = []
    rows.append(rng.standard_normal(cols))
    rows.append(rng.standard_normal(cols) * 1e-30)
    rows.append(rng.standard_normal(cols) * 3e4)
    rows.append(np.zeros(cols))
    r = rng.standard_normal(cols)
    r[::32] = 1.9 * 8  # saturating block maxima
    rows.append(r)
    # exact E4M3 midpoints at scale 1 (amax forced to 256 -> e = 0)
    mids = (OXgrid[:-1] + OXgrid[1:]) / 2
    r = np.resize(np.concatenate([mids, -mids]), cols)
    r[::32] = 256.0
    rows.append(r)
    r = np.full(cols, -0.0)
    rows.append(r)
    r = rng.standard_normal(cols) * 2.0 ** -130  # fp32 subnormals
    rows.append(r)
    r = rng.standard_normal(cols)
    r[5::32] = 2.0 ** -140  # tiny element in a normal block
    rows.append(r)
    return np.array(rows)


from oracle import mx as OX  # noqa: E402

OXgrid = OX.decode_e4m3(np.arange(0, 0x7F))


@pytest.mark.parametrize("src", ["fp32", "bf16"])
def test_quantize_act_bit_exact(src):
    from mxfp4_expert_grouped_amd.layer import quantize_act
    rng = np.random.default_rng(11)
    cols = 7168
    v = np.concatenate([_adversarial_rows(rng, cols), rng.standard_normal((55, cols)) * 5])
    v32 = v.astype(np.float32)
    if src == "bf16":
        bits = I.f32_to_bf16_bits(v32)
        t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
        ref_in = P.OM.bf16_to_f64(bits)
    else:
        t = torch.from_numpy(v32).cuda()
        ref_in = v32.astype(np.float64)
    codes, scales = quantize_act(t)
    torch.cuda.synchronize()
    rc, rs = OX.mx_quantize(ref_in, "e4m3")
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def test_quantize_act_strided_and_ragged_rows():
    from mxfp4_expert_grouped_amd import mxmoe as M
    rng = np.random.default_rng(12)
    full = rng.standard_normal((37, 160)).astype(np.float32)
    t = torch.from_numpy(full).cuda()
    view = t[:, :96]  # ld = 160 elements, cols = 96
    codes = torch.empty((37, 96), dtype=torch.uint8, device="cuda")
    scales = torch.empty((37, 3), dtype=torch.uint8, device="cuda")
    M.moe_quantize_act(view.data_ptr(), M.MOE_SRC_FP32, 37, 96, 160, codes.data_ptr(),
                       scales.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    rc, rs = OX.mx_quantize(full[:, :96].astype(np.float64), "e4m3")
    assert np.array_equal(codes.cpu().numpy(), rc) and np.array_equal(scales.cpu().numpy(), rs)


# ---------------------------------------------------------------------------
# exact-arithmetic regime: gate/up accumulators bit-exact
# ---------------------------------------------------------------------------

# (name, tokens, d, d_ff, experts, top_k, scale bytes or None for the standard
# recipe).  The kernel each case reaches: 40 tokens of 8 experts -> 10 rows
# per expert, 8-row tiles, the K-split streaming gate_up; 300 tokens -> 75 per
# expert, 256-row tiles, the prefill GEMM (per-step activation scales at
# d = 256, scales grouped per four K steps at d = 1024); 2048 tokens of 1024
# experts at top-8 -> 16 rows per expert but enough items for the streaming
# gate_up without the K split and the two-group down items.
EXACT_CASES = [
    ("stream_ksplit", 40, 256, 128, 8, 2, None),
    ("stream_ksplit_k1024", 40, 1024, 512, 8, 2, None),
    ("stream_ksplit_wide_scales", 40, 256, 128, 8, 2, (122, 132)),
    ("prefill_step_scales", 300, 256, 128, 8, 2, (122, 132)),
    ("prefill_grouped_scales", 300, 1024, 512, 8, 2, (124, 130)),
    # d_model 512: 26,624 down items, enough for the two-group (wide) items
    ("stream_whole_items_wide_down", 2048, 512, 512, 1024, 8, (122, 132)),
    # 32 tokens: the routing launch runs the shared experts' items and the
    # routed gate_up launch has enough items (20,736) for whole items per wave
    ("stream_phases_whole_items", 32, 512, 2048, 256, 16, None),
    # prefill tiles of at most 64 rows (six-slot ring), of 161-256 rows
    # (three slots) next to a short remainder tile, per-step and grouped scales
    ("prefill_rows64_step_scales", 128, 256, 128, 8, 2, (122, 132)),
    ("prefill_rows64_grouped_scales", 128, 1024, 512, 8, 2, (124, 130)),
    ("prefill_rows256_grouped_scales", 1200, 1024, 512, 8, 2, (124, 130)),
    # d_model an odd multiple of 128: half of the last output block
    ("stream_d384", 40, 384, 128, 8, 2, (122, 132)),
    ("prefill_d384", 300, 384, 128, 8, 2, (122, 132)),
    ("prefill_d640_grouped", 300, 640, 512, 8, 2, (124, 130)),
]


@pytest.mark.parametrize("name,T,d,f,E,k,scales", EXACT_CASES, ids=[c[0] for c in EXACT_CASES])
def test_gate_up_accumulators_exact(name, T, d, f, E, k, scales):
    """x integer-valued in [-16, 16]: every MXFP8 element is exact, and with
    the weights' scale bytes in a bounded range every product is a multiple
    of q = 0.5 * 2^(lowest scale - 127) and every partial sum stays below
    2^24 q (asserted from the oracle's term magnitudes), so fp32 accumulation
    in any order is exact and the GPU's gate/up values must equal the float64
    ones bit for bit: any lane, K-step or scale-byte layout error shows.  The
    whole layer is then compared with the full parity rules on a sample."""
    cfg = I.LayerConfig(name, T, d, E, k, f, 1, seed=21)
    bits = P.integer_x(cfg, 5)
    x = P.IG.bf16_tensor(bits)
    if scales is None:
        W = P.IG.device_weights(cfg)
        ref = I.ExpertWeights(cfg)
    else:
        W, ref = P.weights_with_scale_range(cfg, 77, *scales)
    P.log(f"exact case {name}: T={T} d={d} d_ff={f} E={E} k={k} scale bytes {scales}")
    g = P.run_gpu(cfg, W, x)
    tokens = None if T <= 64 else sorted(set(range(0, T, max(1, T // 48))) | {T - 1})
    wr = I.gen_router_w(cfg)
    res, differ = P.compare_layer(cfg, bits, wr, None, ref, g, tokens=tokens)
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


# ---------------------------------------------------------------------------
# whole layer at small sizes
# ---------------------------------------------------------------------------

def _layer_case(cfg, bias=None, tokens=None):
    x_bits = I.gen_x(cfg)
    x = P.IG.bf16_tensor(x_bits)
    W = P.IG.device_weights(cfg)
    b = I.gen_router_b(cfg) if bias is None else np.asarray(bias, np.float32)
    if b is not None:
        W.router_b = torch.from_numpy(b).cuda()
    P.log(f"case {cfg}")
    g = P.run_gpu(cfg, W, x)
    return P.compare_layer(cfg, x_bits, I.gen_router_w(cfg), b, I.ExpertWeights(cfg), g, tokens)


def test_tiny_layer_all_taps():
    cfg = I.CONFIGS["tiny"]
    res, differ = _layer_case(cfg)
    assert not differ


@pytest.mark.parametrize("T", [1, 3, 4, 5, 13, 64, 65, 200, 256, 1100, 1500])
def test_ragged_token_counts(T):
    # 256 and above use 64-row tiles (>= 24 rows per expert on average);
    # above 1024 tokens the multi-kernel permutation path runs
    cfg = I.LayerConfig("ragged", T, 256, 16, 2, 128, 1, seed=T)
    tokens = None if T <= 256 else list(range(0, T, max(1, T // 40)))
    _layer_case(cfg, tokens=tokens)


def test_prefill_tiles_over_many_groups():
    # 256-row tiles (about 130 rows per expert): 63 routed tiles + 8 shared
    # ones = 71 tiles, i.e. 18 groups of up to four tiles dealt to the eight
    # XCDs, the last group partial; two column blocks in both GEMMs
    cfg = I.LayerConfig("groups", 2048, 512, 63, 4, 256, 1, seed=41)
    _layer_case(cfg, tokens=list(range(0, 2048, 37)) + [2047])


def test_router_many_token_and_expert_tiles():
    # the MFMA router without a K split over 157 token tiles (the last
    # ragged) x 8 expert tiles of 1024 experts: logits of every token within
    # 1e-4 of the oracle, routing bit-exact up to near-ties, the layer on a
    # token sample
    cfg = I.LayerConfig("router_tiles", 20000, 256, 1024, 8, 128, 1, seed=71)
    _layer_case(cfg, tokens=list(range(0, 20000, 499)) + [255, 256, 19999])


@pytest.mark.parametrize("T", [5, 300])
def test_more_than_two_shared_experts(T):
    # the combine reads up to eight shared rows per token once S > 2; both
    # the permuted-row (decode) and the (token, slot) (prefill) o layouts
    cfg = I.LayerConfig("shared5", T, 256, 16, 2, 128, 5, seed=50 + T)
    _layer_case(cfg, tokens=None if T <= 64 else list(range(0, T, 7)) + [T - 1])


@pytest.mark.parametrize("T", [3, 300])
def test_top_k_above_16(T):
    # 20 of 48 experts: top-k keeps more than 16 candidates and the combine
    # sums its slots in two passes of 16
    cfg = I.LayerConfig("k20", T, 256, 48, 20, 128, 1, seed=60 + T)
    _layer_case(cfg, tokens=None if T <= 64 else list(range(0, T, 7)) + [T - 1])


def test_medium_layer_k4_two_shared():
    cfg = I.LayerConfig("mid", 96, 1024, 32, 4, 512, 2, seed=7)
    _layer_case(cfg)


def test_all_tokens_to_one_expert_k1_no_shared():
    cfg = I.LayerConfig("hot", 300, 256, 16, 1, 128, 0, seed=8)
    bias = np.zeros(16, np.float32)
    bias[5] = 50.0
    res, _ = _layer_case(cfg, bias=bias)
    assert np.all(res.topk_ids == 5)


def test_zipf_bias_small():
    cfg = I.LayerConfig("skew", 400, 512, 64, 4, 256, 2, zipf_bias=True, seed=9)
    _layer_case(cfg)


def test_zero_tokens_is_noop():
    from mxfp4_expert_grouped_amd.layer import MoeLayer
    cfg = I.CONFIGS["tiny"]
    W = P.IG.device_weights(cfg)
    layer = MoeLayer(256, 128, 16, 2, 1, 8, W)
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device="cuda")
    y = layer.forward(x)
    torch.cuda.synchronize()
    assert y.shape == (0, 256)


def test_deterministic_and_workspace_independent():
    cfg = I.LayerConfig("det", 200, 1024, 32, 4, 512, 2, seed=10)
    x = P.IG.device_x(cfg)
    W = P.IG.device_weights(cfg)
    a = P.run_gpu(cfg, W, x, taps=False, workspace_fill=0)["y"]
    b = P.run_gpu(cfg, W, x, taps=False, workspace_fill=0xFF)["y"]
    c = P.run_gpu(cfg, W, x, taps=True, workspace_fill=0x5A)["y"]
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))


@pytest.mark.parametrize("T,a16", [(1, False), (40, False), (300, False), (3, True), (300, True)],
                         ids=["T1", "T40", "T300_prefill", "T3_a16w4", "T300_prefill_a16w4"])
def test_graph_replay_matches_eager(T, a16):
    # a captured forward (T = 1: few-token router with the fused x
    # quantisation and the one-workgroup top-k/permutation; T = 40: MFMA
    # router, top-k launch, permutation launch; T = 300: 37.5 rows per expert,
    # the 256-row prefill kernels; the A16W4 variant at a few tokens and at
    # prefill size) replays several times, with eager forwards of other
    # inputs in between, and every replay equals the eager result bit for bit
    from mxfp4_expert_grouped_amd import mxmoe as M
    from mxfp4_expert_grouped_amd.layer import MoeLayer
    cfg = I.LayerConfig("graph", T, 256, 16, 2, 128, 2, seed=20 + T + (7 if a16 else 0))
    W = P.IG.device_weights(cfg)
    layer = MoeLayer(cfg.d_model, cfg.d_ff, cfg.num_experts, cfg.top_k, cfg.num_shared, T, W,
                     flags=M.MOE_FLAG_A16W4 if a16 else 0)
    xs = [P.IG.device_x(cfg, layer=i) for i in range(2)]
    ws = torch.empty(layer.workspace_bytes(T), dtype=torch.uint8, device="cuda")
    refs = [layer.forward(x, workspace=ws).clone() for x in xs]
    torch.cuda.synchronize()
    assert not torch.equal(refs[0].view(torch.int16), refs[1].view(torch.int16))
    x_static = xs[0].clone()
    y_static = torch.empty_like(x_static)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.forward(x_static, y=y_static, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(x_static, y=y_static, workspace=ws)
    y_eager = torch.empty_like(x_static)
    for i in range(4):
        x_static.copy_(xs[i % 2])
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_static.view(torch.int16), refs[i % 2].view(torch.int16)), f"replay {i}"
        layer.forward(xs[(i + 1) % 2], y=y_eager, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(y_eager.view(torch.int16), refs[(i + 1) % 2].view(torch.int16)), f"eager {i}"


def test_forward_on_a_non_default_caller_stream():
    # every launch of the forward goes to the caller's stream
    cfg = I.LayerConfig("stream", 3, 256, 16, 2, 128, 2, seed=31)
    W = P.IG.device_weights(cfg)
    x = P.IG.device_x(cfg)
    ref = P.run_gpu(cfg, W, x, taps=False)["y"]
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        got = P.run_gpu(cfg, W, x, taps=False)["y"]
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
