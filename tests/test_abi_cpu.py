"""The C-ABI library on the host (no GPU needed): it loads, exports every
function the header declares, and rejects bad arguments with the documented
status before touching a device."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxmoe.h")


@pytest.fixture(scope="module")
def M():
    from mxfp4_expert_grouped_amd import mxmoe
    if not os.path.exists(mxmoe.LIB_PATH):
        from mxfp4_expert_grouped_amd import build
        build.build()
    mxmoe.load_library()
    return mxmoe


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(moe_[a-z_0-9]+)\s*\(", text, re.M)))


def test_library_exports_every_header_function(M):
    fns = header_functions()
    assert set(fns) == set(M.EXPORTED), fns
    lib = ctypes.CDLL(M.LIB_PATH)
    for name in fns:
        assert hasattr(lib, name), name


def test_input_generator_library_exports():
    from mxfp4_expert_grouped_amd import inputs_gpu
    if not os.path.exists(inputs_gpu.GEN_LIB_PATH):
        from mxfp4_expert_grouped_amd import build
        build.build()
    lib = ctypes.CDLL(inputs_gpu.GEN_LIB_PATH)
    assert hasattr(lib, "mxmoe_gen_mx_matrix")


def test_status_strings(M):
    lib = M.load_library()
    for s in range(5):
        assert lib.moe_status_string(s)
    assert lib.moe_status_string(99) == b"unknown status"


@pytest.mark.parametrize("kw,status", [
    (dict(d_model=7168, d_ff=2048, num_experts=896, top_k=16, num_shared=2, max_tokens=32768), 0),
    (dict(d_model=256, d_ff=128, num_experts=16, top_k=2, num_shared=1, max_tokens=8), 0),
    (dict(d_model=200, d_ff=128, num_experts=16, top_k=2, num_shared=1, max_tokens=8), 2),
    (dict(d_model=384, d_ff=128, num_experts=16, top_k=2, num_shared=1, max_tokens=8), 0),
    (dict(d_model=320, d_ff=128, num_experts=16, top_k=2, num_shared=1, max_tokens=8), 2),
    (dict(d_model=256, d_ff=96, num_experts=16, top_k=2, num_shared=1, max_tokens=8), 2),
    (dict(d_model=256, d_ff=128, num_experts=1025, top_k=2, num_shared=1, max_tokens=8), 2),
    (dict(d_model=256, d_ff=128, num_experts=16, top_k=17, num_shared=1, max_tokens=8), 2),
    (dict(d_model=256, d_ff=128, num_experts=64, top_k=33, num_shared=1, max_tokens=8), 2),
    (dict(d_model=256, d_ff=128, num_experts=16, top_k=0, num_shared=1, max_tokens=8), 1),
    (dict(d_model=256, d_ff=128, num_experts=16, top_k=2, num_shared=-1, max_tokens=8), 1),
    (dict(d_model=256, d_ff=128, num_experts=16, top_k=2, num_shared=9, max_tokens=8), 2),
    (dict(d_model=256, d_ff=128, num_experts=16, top_k=2, num_shared=1, max_tokens=0), 1),
    (dict(d_model=256, d_ff=128, num_experts=16, top_k=2, num_shared=1, max_tokens=8, flags=1), 0),
    (dict(d_model=256, d_ff=128, num_experts=16, top_k=2, num_shared=1, max_tokens=8, flags=2), 1),
    (dict(d_model=256, d_ff=128, num_experts=16, top_k=2, num_shared=1, max_tokens=8, flags=3), 1),
])
def test_plan_validation(M, kw, status):
    if status == 0:
        p = M.moe_plan(**kw)
        assert p.value
        M.moe_plan_destroy(p)
    else:
        with pytest.raises(M.MoeError) as ei:
            M.moe_plan(**kw)
        assert ei.value.status == status
        assert ei.value.detail


def test_workspace_bytes(M):
    p = M.moe_plan(7168, 2048, 896, 16, 2, 32768)
    try:
        assert M.moe_workspace_bytes(p, 0) == 0
        w1 = M.moe_workspace_bytes(p, 1)
        w256 = M.moe_workspace_bytes(p, 256)
        w32k = M.moe_workspace_bytes(p, 32768)
        assert 0 < w1 < w256 < w32k
        # at least the bf16 expert outputs at prefill: (T*k + S*T) rows of d values
        assert w32k >= 32768 * 18 * 7168 * 2
        with pytest.raises(M.MoeError) as ei:
            M.moe_workspace_bytes(p, 32769)
        assert ei.value.status == M.MOE_ERR_INVALID_ARG
    finally:
        M.moe_plan_destroy(p)


def test_forward_argument_errors_before_any_device_call(M):
    p = M.moe_plan(256, 128, 16, 2, 1, 8)
    fake = 1 << 20  # never dereferenced: every call below fails validation first
    W = M.MoeWeights(fake, fake, fake, fake, fake, fake, fake, fake, fake, None, M.MOE_WEIGHTS_PACKED)
    ws = M.moe_workspace_bytes(p, 8)
    try:
        # T == 0 is a no-op even with null buffers
        M.moe_forward(p, W, None, 0, None, None, 0)
        cases = [
            (dict(num_tokens=9), M.MOE_ERR_INVALID_ARG),
            (dict(num_tokens=-1), M.MOE_ERR_INVALID_ARG),
            (dict(x=0), M.MOE_ERR_INVALID_ARG),
            (dict(workspace=0), M.MOE_ERR_WORKSPACE),
            (dict(workspace_bytes=ws - 1), M.MOE_ERR_WORKSPACE),
            (dict(workspace=fake + 16), M.MOE_ERR_WORKSPACE),
            (dict(x=fake + 2), M.MOE_ERR_INVALID_ARG),
        ]
        for over, status in cases:
            args = dict(x=fake, num_tokens=8, y=fake, workspace=fake, workspace_bytes=ws)
            args.update(over)
            with pytest.raises(M.MoeError) as ei:
                M.moe_forward(p, W, args["x"] or None, args["num_tokens"], args["y"],
                              args["workspace"] or None, args["workspace_bytes"])
            assert ei.value.status == status, (over, ei.value)
        # missing shared weights
        W2 = M.MoeWeights(fake, fake, fake, fake, None, None, None, None, fake, None, M.MOE_WEIGHTS_PACKED)
        with pytest.raises(M.MoeError) as ei:
            M.moe_forward(p, W2, fake, 8, fake, fake, ws)
        assert ei.value.status == M.MOE_ERR_INVALID_ARG
    finally:
        M.moe_plan_destroy(p)


def test_forward_rejects_untagged_weights(M):
    # moe_forward reads packed or canonical expert matrices as the layout tag
    # says: any other tag (a zero-initialised struct among them) fails
    # before anything is enqueued, whatever else is valid
    p = M.moe_plan(256, 128, 16, 2, 1, 8)
    fake = 1 << 20
    ws = M.moe_workspace_bytes(p, 8)
    try:
        for tag in (0, M.MOE_WEIGHTS_PACKED + 1, M.MOE_WEIGHTS_CANONICAL + 1, 1):
            W = M.MoeWeights(fake, fake, fake, fake, fake, fake, fake, fake, fake, None, tag)
            with pytest.raises(M.MoeError) as ei:
                M.moe_forward(p, W, fake, 8, fake, fake, ws)
            assert ei.value.status == M.MOE_ERR_INVALID_ARG
            assert "MOE_WEIGHTS_PACKED" in ei.value.detail
        # the default of the binding's struct (zero) is no tag
        W = M.MoeWeights(fake, fake, fake, fake, fake, fake, fake, fake, fake, None)
        with pytest.raises(M.MoeError) as ei:
            M.moe_forward(p, W, fake, 8, fake, fake, ws)
        assert ei.value.status == M.MOE_ERR_INVALID_ARG
    finally:
        M.moe_plan_destroy(p)


def test_forward_rejects_misaligned_scale_taps(M):
    # x_scales and h_scales taps are read back by the prefill GEMM in
    # 16-byte pieces: a 4-byte-aligned tap is refused
    p = M.moe_plan(256, 128, 16, 2, 1, 8)
    fake = 1 << 20
    ws = M.moe_workspace_bytes(p, 8)
    W = M.MoeWeights(fake, fake, fake, fake, fake, fake, fake, fake, fake, None, M.MOE_WEIGHTS_PACKED)
    try:
        for name in ("x_scales", "h_scales", "y_routed", "y_shared", "x_codes", "h_codes"):
            taps = M.MoeTaps(**{name: fake + 4})
            with pytest.raises(M.MoeError) as ei:
                M.moe_forward(p, W, fake, 8, fake, fake, ws, taps)
            assert ei.value.status == M.MOE_ERR_INVALID_ARG, name
            assert "tap" in ei.value.detail
    finally:
        M.moe_plan_destroy(p)


def test_quantize_argument_errors(M):
    fake = 1 << 20
    M.moe_quantize_act(None, M.MOE_SRC_BF16, 0, 64, 64, None, None)  # empty: no-op
    for args, status in [
        ((fake, 7, 4, 64, 64, fake, fake), M.MOE_ERR_INVALID_ARG),
        ((fake, M.MOE_SRC_BF16, 4, 48, 48, fake, fake), M.MOE_ERR_UNSUPPORTED),
        ((fake, M.MOE_SRC_BF16, 4, 64, 32, fake, fake), M.MOE_ERR_INVALID_ARG),
        ((None, M.MOE_SRC_BF16, 4, 64, 64, fake, fake), M.MOE_ERR_INVALID_ARG),
        ((fake + 4, M.MOE_SRC_FP32, 4, 64, 64, fake, fake), M.MOE_ERR_UNSUPPORTED),
    ]:
        with pytest.raises(M.MoeError) as ei:
            M.moe_quantize_act(*args)
        assert ei.value.status == status


def test_no_device_reports_device_error(M):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    p = M.moe_plan(256, 128, 16, 2, 1, 8)
    fake = 1 << 20
    W = M.MoeWeights(fake, fake, fake, fake, fake, fake, fake, fake, fake, None, M.MOE_WEIGHTS_PACKED)
    try:
        with pytest.raises(M.MoeError) as ei:
            M.moe_forward(p, W, fake, 8, fake, fake, M.moe_workspace_bytes(p, 8))
        assert ei.value.status == M.MOE_ERR_DEVICE
    finally:
        M.moe_plan_destroy(p)


def test_pack_sizes_and_argument_errors(M):
    assert M.moe_packed_scale_bytes(4096, 7168) == 4096 * 224
    assert M.moe_packed_scale_bytes(7168, 2048) == 7168 * 64
    assert M.moe_packed_scale_bytes(256, 256) == 256 * 8
    assert M.moe_packed_scale_bytes(0, 128) == 0
    assert M.moe_packed_scale_bytes(32, 256) == 0   # rows not a multiple of 64
    assert M.moe_packed_scale_bytes(64, 192) == 0   # k not a multiple of 128
    fake = 1 << 20
    M.moe_pack_mx4(None, None, 0, 64, 256, 0, None, None)  # nothing to pack
    for args, status in [
        ((fake, fake, 1, 24, 256, 0, fake, fake), M.MOE_ERR_UNSUPPORTED),
        ((fake, fake, 1, 32, 256, 0, fake, fake), M.MOE_ERR_UNSUPPORTED),
        ((fake, fake, 1, 64, 192, 0, fake, fake), M.MOE_ERR_UNSUPPORTED),
        ((fake, fake, -1, 64, 256, 0, fake, fake), M.MOE_ERR_INVALID_ARG),
        ((fake, fake, 1, 64, 256, 2, fake, fake), M.MOE_ERR_INVALID_ARG),
        ((None, fake, 1, 64, 256, 1, fake, fake), M.MOE_ERR_INVALID_ARG),
        ((fake + 8, fake, 1, 64, 256, 1, fake, fake), M.MOE_ERR_INVALID_ARG),
    ]:
        with pytest.raises(M.MoeError) as ei:
            M.moe_pack_mx4(*args)
        assert ei.value.status == status


def test_noalloc_forward_rejects_token_counts_above_its_scratch(M):
    # checked on the host before any device call: 300 tokens of the full layer
    # need more than the fixed scratch array; 0 tokens is a no-op
    p = M.moe_plan(7168, 2048, 896, 16, 2, 1024)
    fake = 1 << 20
    W = M.MoeWeights(fake, fake, fake, fake, fake, fake, fake, fake, fake, None, M.MOE_WEIGHTS_PACKED)
    try:
        assert M.moe_workspace_bytes(p, 256) <= M.NOALLOC_SCRATCH_BYTES < M.moe_workspace_bytes(p, 300)
        M.moe_forward_noalloc(p, W, None, 0, None)
        with pytest.raises(M.MoeError) as ei:
            M.moe_forward_noalloc(p, W, fake, 300, fake)
        assert ei.value.status == M.MOE_ERR_WORKSPACE and "scratch" in ei.value.detail
        with pytest.raises(M.MoeError) as ei:
            M.moe_forward_noalloc(p, M.MoeWeights(), fake, 8, fake)
        assert ei.value.status == M.MOE_ERR_INVALID_ARG
    finally:
        M.moe_plan_destroy(p)


def test_latent_tail_host_checks(M):
    fake = 1 << 20
    W = M.MoeTailWeights(fake, fake, fake, M.MOE_WEIGHTS_PACKED)
    assert M.moe_latent_tail_workspace_bytes(0, 7168, 7168) == 0
    w1 = M.moe_latent_tail_workspace_bytes(1, 7168, 7168)
    w8k = M.moe_latent_tail_workspace_bytes(8192, 7168, 7168)
    assert 0 < w1 < w8k and w8k >= 8192 * 7168 * 2
    # T == 0 is a no-op with null buffers
    M.moe_latent_tail(0, 256, 256, 1e-6, W, None, None, None, None, 0)
    ws = M.moe_latent_tail_workspace_bytes(4, 256, 256)
    for args, status in [
        ((4, 200, 256, 1e-6, W, fake, fake, fake, fake, ws), M.MOE_ERR_UNSUPPORTED),   # latent % 128
        ((4, 256, 192, 1e-6, W, fake, fake, fake, fake, ws), M.MOE_ERR_UNSUPPORTED),   # hidden % 128
        ((4, 256, 256, -1.0, W, fake, fake, fake, fake, ws), M.MOE_ERR_INVALID_ARG),   # eps < 0
        ((4, 256, 256, float("nan"), W, fake, fake, fake, fake, ws), M.MOE_ERR_INVALID_ARG),
        ((4, 256, 256, 1e-6, M.MoeTailWeights(fake, fake, fake, 0), fake, fake, fake, fake, ws),
         M.MOE_ERR_INVALID_ARG),                                                       # not tagged packed
        ((4, 256, 256, 1e-6, W, None, fake, fake, fake, ws), M.MOE_ERR_INVALID_ARG),   # z NULL
        ((4, 256, 256, 1e-6, W, fake + 4, fake, fake, fake, ws), M.MOE_ERR_INVALID_ARG),  # z misaligned
        ((4, 256, 256, 1e-6, W, fake, fake, fake, fake, ws - 1), M.MOE_ERR_WORKSPACE),
        ((4, 256, 256, 1e-6, W, fake, fake, fake, fake + 16, ws), M.MOE_ERR_WORKSPACE),
        ((-1, 256, 256, 1e-6, W, fake, fake, fake, fake, ws), M.MOE_ERR_INVALID_ARG),
    ]:
        with pytest.raises(M.MoeError) as ei:
            M.moe_latent_tail(*args)
        assert ei.value.status == status, (args, ei.value)


def test_a16w4_host_checks(M):
    # bf16 activations: no MXFP8 taps, at decode and prefill sizes; h through
    # its own bf16 tap
    fake = 1 << 20
    W = M.MoeWeights(fake, fake, fake, fake, fake, fake, fake, fake, fake, None, M.MOE_WEIGHTS_PACKED)
    p = M.moe_plan(256, 128, 16, 2, 1, 1024, M.MOE_FLAG_A16W4)
    p8 = M.moe_plan(256, 128, 16, 2, 1, 1024)
    try:
        ws = M.moe_workspace_bytes(p, 1024)
        # 8 tokens: the streaming kernels; 192 x 2 / 16 = 24 rows per expert:
        # the 256-row tiles
        for T in (8, 192):
            for name in ("x_codes", "x_scales", "h_codes", "h_scales"):
                with pytest.raises(M.MoeError) as ei:
                    M.moe_forward(p, W, fake, T, fake, fake, ws, M.MoeTaps(**{name: fake}))
                assert ei.value.status == M.MOE_ERR_INVALID_ARG and "A16W4" in ei.value.detail
        with pytest.raises(M.MoeError) as ei:
            M.moe_forward(p8, W, fake, 8, fake, fake, M.moe_workspace_bytes(p8, 8), M.MoeTaps(h_bf16=fake))
        assert ei.value.status == M.MOE_ERR_INVALID_ARG
        # h in bf16 takes twice the bytes of MXFP8 codes, no scales
        assert M.moe_workspace_bytes(p, 8) > M.moe_workspace_bytes(p8, 8)
    finally:
        M.moe_plan_destroy(p)
        M.moe_plan_destroy(p8)


def test_router_bias_update_host_checks(M):
    p = M.moe_plan(256, 128, 16, 2, 1, 8)
    fake = 1 << 20
    try:
        M.moe_router_bias_update(p, None, 0, 0.1, None)  # no tokens: nothing to do
        for args, status in [((p, fake, 9, 0.1, fake), M.MOE_ERR_INVALID_ARG),
                             ((p, fake, 4, -0.1, fake), M.MOE_ERR_INVALID_ARG),
                             ((p, fake, 4, float("inf"), fake), M.MOE_ERR_INVALID_ARG),
                             ((p, None, 4, 0.1, fake), M.MOE_ERR_INVALID_ARG),
                             ((p, fake, 4, 0.1, fake + 2), M.MOE_ERR_INVALID_ARG),
                             ((None, fake, 4, 0.1, fake), M.MOE_ERR_INVALID_ARG)]:
            with pytest.raises(M.MoeError) as ei:
                M.moe_router_bias_update(*args)
            assert ei.value.status == status
    finally:
        M.moe_plan_destroy(p)
