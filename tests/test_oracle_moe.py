"""Pins for the oracle's router, permutation, expert MLP and combine (CPU only).

* top-k against a brute-force search over every k-subset;
* routing weights against torch's softmax of log-sigmoid (a different route
  to sigmoid(l)/sum sigmoid(l));
* the permutation against a plain loop over experts and tokens, plus its
  invariants;
* the sparse layer against a dense all-experts masked computation;
* E=1, k=1, no shared expert against a textbook SwiGLU MLP in torch float64
  with torch's float8 cast doing the MXFP8 element rounding of h.
"""

import itertools

import numpy as np
import pytest
import torch

from mxfp4_expert_grouped_amd import inputs as I
from oracle import moe, mx


def test_topk_matches_subset_brute_force_tiny():
    cfg = I.CONFIGS["tiny"]
    x = I.gen_x(cfg)
    logits = moe.router_logits(x, I.gen_router_w(cfg), I.gen_router_b(cfg))
    ids, gap = moe.topk_select(logits, cfg.top_k)
    for t in range(cfg.tokens):
        best = max(itertools.combinations(range(cfg.num_experts), cfg.top_k),
                   key=lambda s: (sum(logits[t, list(s)]), [-i for i in s]))
        assert tuple(ids[t]) == best
        srt = np.sort(logits[t])[::-1]
        assert gap[t] == srt[cfg.top_k - 1] - srt[cfg.top_k]


def test_topk_ties_go_to_lower_index():
    l = np.array([[2.0, 1.0, 1.0, 0.0, 1.0], [0.5, 0.5, 0.5, 0.5, 0.5]])
    ids, gap = moe.topk_select(l, 2)
    assert ids.tolist() == [[0, 1], [0, 1]]
    assert gap.tolist() == [0.0, 0.0]
    # brute force: among max-sum subsets, the lexicographically smallest
    for t in range(2):
        subs = list(itertools.combinations(range(5), 2))
        m = max(sum(l[t, list(s)]) for s in subs)
        assert tuple(ids[t]) == min(s for s in subs if sum(l[t, list(s)]) == m)


def test_topk_random_against_full_sort():
    rng = np.random.default_rng(7)
    l = rng.standard_normal((50, 896))
    ids, _ = moe.topk_select(l, 16)
    for t in range(50):
        assert set(ids[t]) == set(np.argsort(-l[t], kind="stable")[:16])
        assert np.all(np.diff(ids[t]) > 0)


def test_routing_weights_library_and_invariants():
    rng = np.random.default_rng(8)
    l = rng.standard_normal((20, 64)) * 2
    ids, _ = moe.topk_select(l, 16)
    w = moe.routing_weights(l, ids)
    sel = torch.from_numpy(np.take_along_axis(l, ids.astype(np.int64), 1))
    ref = torch.softmax(torch.nn.functional.logsigmoid(sel), dim=1).numpy()
    assert np.allclose(w, ref, rtol=1e-13, atol=0)
    assert np.all(np.abs(w.sum(1) - 1) <= 1e-12) and np.all(w > 0)
    # equal logits -> equal weights 1/k
    assert np.allclose(moe.routing_weights(np.zeros((1, 8)), np.arange(4)[None]), 0.25)


def test_router_logits_exact_products():
    # small integers: the float64 sum is exact, so it must equal an integer matmul
    rng = np.random.default_rng(9)
    xi = rng.integers(-4, 5, size=(3, 64))
    wi = rng.integers(-4, 5, size=(5, 64))
    x_bits = I.f32_to_bf16_bits(xi.astype(np.float32))
    l = moe.router_logits(x_bits, wi.astype(np.float32), np.arange(5, dtype=np.float32))
    assert np.array_equal(l, (xi @ wi.T + np.arange(5)).astype(np.float64))


def test_permute_against_loop_and_invariants():
    rng = np.random.default_rng(10)
    t_count, e_count, k = 37, 11, 3
    ids = np.stack([np.sort(rng.choice(e_count, k, replace=False)) for _ in range(t_count)])
    counts, offsets, row_src, token_row = moe.permute(ids, e_count)
    order = []
    for e in range(e_count):
        for t in range(t_count):
            for j in range(k):
                if ids[t, j] == e:
                    order.append(t * k + j)
    assert row_src.tolist() == order
    assert counts.sum() == t_count * k and offsets[0] == 0 and offsets[-1] == t_count * k
    assert np.all(np.diff(offsets) == counts)
    assert sorted(row_src.tolist()) == list(range(t_count * k))
    for t in range(t_count):
        for j in range(k):
            r = token_row[t, j]
            assert row_src[r] == t * k + j
            assert offsets[ids[t, j]] <= r < offsets[ids[t, j] + 1]


def test_sparse_equals_dense_tiny():
    cfg = I.CONFIGS["tiny"]
    x, wr, b = I.gen_x(cfg), I.gen_router_w(cfg), I.gen_router_b(cfg)
    W = I.ExpertWeights(cfg)
    kw = dict(num_experts=cfg.num_experts, top_k=cfg.top_k, num_shared=cfg.num_shared, d_ff=cfg.d_ff)
    res = moe.forward(x, wr, b, W, **kw)
    dense = moe.forward_dense(x, wr, b, W, **kw)
    rel = np.linalg.norm(res.y - dense) / np.linalg.norm(dense)
    assert rel <= 1e-12
    assert np.linalg.norm(res.y_routed) > 0 and np.linalg.norm(res.y_shared) > 0


def test_sparse_equals_dense_with_bias_and_subset():
    cfg = I.LayerConfig("t2", 12, 128, 24, 4, 64, 2, zipf_bias=True, seed=3)
    x, wr, b = I.gen_x(cfg), I.gen_router_w(cfg), I.gen_router_b(cfg)
    W = I.ExpertWeights(cfg)
    kw = dict(num_experts=cfg.num_experts, top_k=cfg.top_k, num_shared=cfg.num_shared, d_ff=cfg.d_ff)
    dense = moe.forward_dense(x, wr, b, W, **kw)
    sub = moe.forward(x, wr, b, W, tokens=[5, 2, 11], **kw)
    assert sub.tokens.tolist() == [2, 5, 11]
    assert np.allclose(sub.y, dense[[2, 5, 11]], rtol=1e-12, atol=1e-14 * np.abs(dense).max())


def _torch_mx8_roundtrip(h: torch.Tensor) -> torch.Tensor:
    """Independent MXFP8 fake-quant of h along its last axis with torch ops."""
    blocks = h.reshape(h.shape[0], -1, 32)
    amax = blocks.abs().amax(dim=2, keepdim=True)
    _, ex = torch.frexp(amax)
    e = torch.clamp(ex.to(torch.int64) - 1 - 8, -127, 127).to(torch.float64)
    scale = torch.pow(2.0, e)
    q = (blocks / scale).clamp(-448, 448).to(torch.float32).to(torch.float8_e4m3fn).to(torch.float64)
    return (q * scale).reshape(h.shape)


def test_single_expert_is_textbook_swiglu_mlp():
    cfg = I.LayerConfig("one", 4, 128, 1, 1, 64, 0, seed=5)
    x, wr = I.gen_x(cfg), I.gen_router_w(cfg)
    W = I.ExpertWeights(cfg)
    res = moe.forward(x, wr, None, W, num_experts=1, top_k=1, num_shared=0, d_ff=cfg.d_ff)
    assert np.all(res.topk_w == 1.0)
    guc, gus, dnc, dns = W("routed", 0)
    xt = torch.from_numpy(moe.bf16_to_f64(x))
    a = _torch_mx8_roundtrip(xt)
    wgu = torch.from_numpy(mx.mx_decode(guc, gus, "e2m1"))
    wdn = torch.from_numpy(mx.mx_decode(dnc, dns, "e2m1"))
    g = a @ wgu[:64].T
    u = a @ wgu[64:].T
    h = torch.nn.functional.silu(g) * u
    y = _torch_mx8_roundtrip(h) @ wdn.T
    assert np.allclose(res.y, y.numpy(), rtol=1e-12, atol=1e-13 * float(y.abs().max()))


def test_layer_outputs_nontrivial_tiny():
    cfg = I.CONFIGS["tiny"]
    res = moe.forward(I.gen_x(cfg), I.gen_router_w(cfg), None, I.ExpertWeights(cfg),
                      num_experts=16, top_k=2, num_shared=1, d_ff=128)
    assert len(set(res.topk_ids.reshape(-1).tolist())) >= 6  # several experts touched
    assert np.all(np.isfinite(res.y)) and res.y.std() > 0
    assert len(res.h_rows) == 16 and len(res.h_shared) == 8


def test_given_routing_equals_dense_masked_sum():
    # the layer evaluated for a routing it did not choose itself (what the
    # parity tests do for near-tie tokens): every token's output must be the
    # dense sum over all experts with weights that are zero off the given
    # set and sigmoid-renormalised on it (weights here through torch's softmax
    # of log-sigmoid, expert outputs without any permutation)
    cfg = I.LayerConfig("given", 10, 128, 12, 3, 64, 1, seed=13)
    x, wr = I.gen_x(cfg), I.gen_router_w(cfg)
    W = I.ExpertWeights(cfg)
    rng = np.random.default_rng(14)
    given = np.stack([np.sort(rng.choice(cfg.num_experts, cfg.top_k, replace=False))
                      for _ in range(cfg.tokens)]).astype(np.int32)
    own, _ = moe.topk_select(moe.router_logits(x, wr), cfg.top_k)
    assert not np.array_equal(given, own)
    res = moe.forward(x, wr, None, W, num_experts=12, top_k=3, num_shared=1, d_ff=64,
                      topk_ids=given)
    assert np.array_equal(res.topk_ids, given)
    logits = moe.router_logits(x, wr)
    sel = torch.from_numpy(np.take_along_axis(logits, given.astype(np.int64), 1))
    wts = torch.softmax(torch.nn.functional.logsigmoid(sel), dim=1).numpy()
    dense_w = np.zeros((cfg.tokens, cfg.num_experts))
    np.put_along_axis(dense_w, given.astype(np.int64), wts, axis=1)
    xc, xs = mx.mx_quantize(moe.bf16_to_f64(x), "e4m3")
    y_r = np.zeros((cfg.tokens, cfg.d_model))
    for e in range(cfg.num_experts):
        y_r += dense_w[:, e:e + 1] * moe.expert_mlp(xc, xs, *W("routed", e), d_ff=64)[2]
    y_s = moe.expert_mlp(xc, xs, *W("shared", 0), d_ff=64)[2]
    assert np.allclose(res.y_routed, y_r, rtol=1e-12, atol=1e-14 * np.abs(y_r).max())
    assert np.allclose(res.y_shared, y_s, rtol=0, atol=0)
    # its permutation is the one of the given ids
    c, o, rs, tr = moe.permute(given, cfg.num_experts)
    assert np.array_equal(res.row_src, rs) and np.array_equal(res.token_row, tr)


def test_intermediates_exact_on_integer_operands():
    # integer-valued MXFP8 rows and weight codes whose values are integers
    # (E2M1 codes 2, 4, 5, 6, 7 with scale 2^0 are 1, 2, 3, 4, 6): [g|u] must
    # be the exact integer matmul, h = silu(g) u from torch, and with all
    # operands non-negative the term magnitudes equal the sums themselves
    rng = np.random.default_rng(15)
    d, f, n = 64, 32, 5
    xi = rng.integers(0, 9, size=(n, d)).astype(np.float64)
    xi[:, ::32] = 16.0  # every block's amax is 16: scale 2^-4, codes exact
    a_codes, a_scales = mx.mx_quantize(xi, "e4m3")
    assert np.array_equal(mx.mx_decode(a_codes, a_scales, "e4m3"), xi)
    value_code = {1: 2, 2: 4, 3: 5, 4: 6, 6: 7}
    wg = rng.choice([1, 2, 3, 4, 6], size=(2 * f, d))
    wd = rng.choice([1, 2, 3, 4, 6], size=(d, f))
    enc = np.vectorize(value_code.get)
    guc, gus = mx.pack_fp4(enc(wg).astype(np.uint8)), np.full((2 * f, d // 32), 127, np.uint8)
    dnc, dns = mx.pack_fp4(enc(wd).astype(np.uint8)), np.full((d, f // 32), 127, np.uint8)
    mid = {}
    hc, hs, o = moe.expert_mlp(a_codes, a_scales, guc, gus, dnc, dns, d_ff=f, intermediates=mid)
    want = xi.astype(np.int64) @ wg.T.astype(np.int64)
    assert np.array_equal(mid["gu"], want.astype(np.float64))
    assert np.array_equal(mid["gu_abs"], mid["gu"])
    g, u = torch.from_numpy(want[:, :f].astype(np.float64)), torch.from_numpy(want[:, f:].astype(np.float64))
    assert np.allclose(mid["h"], (torch.nn.functional.silu(g) * u).numpy(), rtol=1e-15, atol=0)
    assert np.all(mid["h"] >= 0)
    assert np.allclose(mid["o_abs"], o, rtol=1e-15, atol=0)
    # a row with mixed signs: the magnitudes bound the sums
    mid2 = {}
    moe.expert_mlp(a_codes, a_scales, guc | 0x88, gus, dnc, dns, d_ff=f, intermediates=mid2)
    assert np.array_equal(mid2["gu"], -mid["gu"]) and np.array_equal(mid2["gu_abs"], mid["gu_abs"])


def test_forward_intermediates_match_rows():
    cfg = I.CONFIGS["tiny"]
    x, wr = I.gen_x(cfg), I.gen_router_w(cfg)
    W = I.ExpertWeights(cfg)
    res = moe.forward(x, wr, None, W, num_experts=16, top_k=2, num_shared=1, d_ff=128,
                      intermediates=True)
    assert set(res.mid_rows) == set(res.h_rows) and set(res.mid_shared) == set(res.h_shared)
    for r, m in res.mid_rows.items():
        assert np.all(m["gu_abs"] >= np.abs(m["gu"]))
        hc, hs = mx.mx_quantize(m["h"][None], "e4m3")
        assert np.array_equal(hc[0], res.h_rows[r][0]) and np.array_equal(hs[0], res.h_rows[r][1])
    t = 3
    y_r = sum(res.topk_w[t, j] * res.mid_rows[int(res.token_row[t, j])]["o"] for j in range(2))
    assert np.allclose(y_r, res.y_routed[t], rtol=1e-13, atol=0)
    assert np.allclose(res.mid_shared[(0, t)]["o"], res.y_shared[t], rtol=0, atol=0)


# ---------------------------------------------------------------------------
# LatentMoE tail
# ---------------------------------------------------------------------------

def test_rms_norm_matches_torch():
    rng = np.random.default_rng(30)
    z = rng.standard_normal((9, 256)) * rng.uniform(0.01, 50, size=(9, 1))
    gamma = 1 + 0.1 * rng.standard_normal(256)
    for eps in (0.0, 1e-6, 1e-2):
        ref = torch.nn.functional.rms_norm(torch.from_numpy(z), (256,), torch.from_numpy(gamma), eps)
        assert np.allclose(moe.rms_norm(z, gamma, eps), ref.numpy(), rtol=1e-14, atol=0)


def test_rms_norm_properties():
    rng = np.random.default_rng(31)
    z = rng.standard_normal((4, 128))
    one = np.ones(128)
    n = moe.rms_norm(z, one, 0.0)
    assert np.allclose(np.mean(n * n, axis=1), 1.0, rtol=1e-14)       # unit mean square
    assert np.allclose(moe.rms_norm(37.5 * z, one, 0.0), n, rtol=1e-14)  # scale invariant
    assert np.allclose(moe.rms_norm(n, one, 0.0), n, rtol=1e-14)        # idempotent
    g = rng.uniform(0.5, 2, 128)
    assert np.allclose(moe.rms_norm(z, g, 0.0), n * g, rtol=1e-14)       # gain per column
    assert np.all(moe.rms_norm(np.zeros((1, 128)), one, 1e-6) == 0)     # zero row with eps


def test_latent_tail_exact_on_integer_operands():
    # rows whose RMSNorm is integer-valued (z = c * v with v in {-1, 1}, so
    # mean(v^2) = 1 and n = v), integer weights with scale 2^0: the projection
    # is the exact integer matmul, plus s
    rng = np.random.default_rng(32)
    T, l, H = 3, 64, 96
    v = rng.choice([-1.0, 1.0], size=(T, l))
    z = v * np.array([[0.5], [3.0], [1e3]])
    value_code = {1: 2, 2: 4, 3: 5, 4: 6, 6: 7}
    wi = rng.choice([1, 2, 3, 4, 6], size=(H, l)) * rng.choice([-1, 1], size=(H, l))
    codes = np.vectorize(lambda q: value_code[abs(q)] | (8 if q < 0 else 0))(wi).astype(np.uint8)
    up_c, up_s = mx.pack_fp4(codes), np.full((H, l // 32), 127, np.uint8)
    s = rng.integers(-5, 6, size=(T, H)).astype(np.float64)
    mid = {}
    y = moe.latent_tail(z, np.ones(l), 0.0, up_c, up_s, s, intermediates=mid)
    assert np.array_equal(mid["n"], v)
    want = v.astype(np.int64) @ wi.T.astype(np.int64) + s.astype(np.int64)
    assert np.array_equal(y, want.astype(np.float64))
    assert np.array_equal(mid["y_abs"], np.abs(v) @ np.abs(wi).T.astype(np.float64))
    assert np.array_equal(moe.latent_tail(z, np.ones(l), 0.0, up_c, up_s), want - s)


def test_latent_tail_is_norm_quantise_project_add():
    # the composition against torch: rms_norm, torch's float8 cast for the
    # MXFP8 elements, matmul with the decoded weights, add
    cfg = I.LayerConfig("tail", 5, 256, 1, 1, 128, 0, seed=33)
    rng = np.random.default_rng(34)
    z = (rng.standard_normal((5, 256)) * 0.3).astype(np.float32)
    s = rng.standard_normal((5, 256)).astype(np.float32)
    gamma = (1 + 0.05 * rng.standard_normal(256)).astype(np.float32)
    up_c, up_s = I.gen_mx_matrix(33, I.stream_id(7, 0), 256, 256, I.weight_sigma(256))
    y = moe.latent_tail(z, gamma, 1e-6, up_c, up_s, s)
    n = torch.nn.functional.rms_norm(torch.from_numpy(z.astype(np.float64)), (256,),
                                     torch.from_numpy(gamma.astype(np.float64)), 1e-6)
    a = _torch_mx8_roundtrip(n)
    w = torch.from_numpy(mx.mx_decode(up_c, up_s, "e2m1"))
    ref = a @ w.T + torch.from_numpy(s.astype(np.float64))
    assert np.allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12 * float(ref.abs().max()))


# ---------------------------------------------------------------------------
# A16W4 variant (bf16 activations, MXFP4 weights)
# ---------------------------------------------------------------------------

def test_a16w4_single_expert_is_textbook_swiglu_with_bf16_h():
    cfg = I.LayerConfig("one16", 4, 128, 1, 1, 64, 0, seed=6)
    x, wr = I.gen_x(cfg), I.gen_router_w(cfg)
    W = I.ExpertWeights(cfg)
    res = moe.forward(x, wr, None, W, num_experts=1, top_k=1, num_shared=0, d_ff=cfg.d_ff,
                      activations="bf16")
    guc, gus, dnc, dns = W("routed", 0)
    xt = torch.from_numpy(moe.bf16_to_f64(x))
    wgu = torch.from_numpy(mx.mx_decode(guc, gus, "e2m1"))
    wdn = torch.from_numpy(mx.mx_decode(dnc, dns, "e2m1"))
    h = torch.nn.functional.silu(xt @ wgu[:64].T) * (xt @ wgu[64:].T)
    hb = h.to(torch.bfloat16)
    y = hb.to(torch.float64) @ wdn.T
    assert np.allclose(res.y, y.numpy(), rtol=1e-12, atol=1e-13 * float(y.abs().max()))
    assert np.array_equal(res.h_rows[0][0], hb[0].view(torch.int16).numpy().view(np.uint16))
    assert res.h_rows[0][1] is None and res.x_scales.shape == (4, 0)


def test_a16w4_sparse_equals_dense():
    cfg = I.LayerConfig("t16", 12, 128, 24, 4, 64, 2, zipf_bias=True, seed=7)
    x, wr, b = I.gen_x(cfg), I.gen_router_w(cfg), I.gen_router_b(cfg)
    W = I.ExpertWeights(cfg)
    kw = dict(num_experts=24, top_k=4, num_shared=2, d_ff=64, activations="bf16")
    dense = moe.forward_dense(x, wr, b, W, **kw)
    sparse = moe.forward(x, wr, b, W, **kw)
    assert np.allclose(sparse.y, dense, rtol=1e-12, atol=1e-14 * np.abs(dense).max())
    # and it differs from the MXFP8-activation layer by more than rounding noise
    a8 = moe.forward(x, wr, b, W, num_experts=24, top_k=4, num_shared=2, d_ff=64)
    assert np.linalg.norm(a8.y - sparse.y) > 1e-4 * np.linalg.norm(sparse.y)


def test_a16w4_intermediates_exact_on_integer_operands():
    rng = np.random.default_rng(16)
    d, f, n = 64, 32, 4
    xi = rng.integers(-16, 17, size=(n, d)).astype(np.float32)
    bits = I.f32_to_bf16_bits(xi)
    value_code = {1: 2, 2: 4, 3: 5, 4: 6, 6: 7}
    wg = rng.choice([1, 2, 3, 4, 6], size=(2 * f, d)) * rng.choice([-1, 1], size=(2 * f, d))
    enc = np.vectorize(lambda q: value_code[abs(q)] | (8 if q < 0 else 0))
    guc, gus = mx.pack_fp4(enc(wg).astype(np.uint8)), np.full((2 * f, d // 32), 127, np.uint8)
    dnc = mx.pack_fp4(enc(rng.choice([1, 2], size=(d, f))).astype(np.uint8))
    dns = np.full((d, f // 32), 127, np.uint8)
    mid = {}
    hb, o = moe.expert_mlp_a16(bits, guc, gus, dnc, dns, d_ff=f, intermediates=mid)
    assert np.array_equal(mid["gu"], (xi.astype(np.int64) @ wg.T.astype(np.int64)).astype(np.float64))
    assert np.array_equal(hb, moe.f64_to_bf16(mid["h"]))


# ---------------------------------------------------------------------------
# router bias balancing step
# ---------------------------------------------------------------------------

def test_router_bias_update_by_hand():
    # 4 experts, 6 tokens, top-2: mean load 3
    b = np.array([0.5, -1.0, 0.0, 2.0], np.float32)
    counts = np.array([5, 3, 1, 3])
    out = moe.router_bias_update(b, counts, 6, 2, 0.25)
    assert out.dtype == np.float32
    assert out.tolist() == [0.25, -1.0, 0.25, 2.0]
    # the addition is the fp32 one: 1 + 2^-30 stays 1
    out = moe.router_bias_update(np.ones(2, np.float32), [0, 4], 2, 1, 2.0 ** -30)
    assert out.tolist() == [1.0, 1.0]


def test_router_bias_updates_even_out_a_skewed_load():
    # repeated steps on the Zipf-skewed router of a small layer: the most
    # loaded expert's share falls and the spread of the loads shrinks
    cfg = I.LayerConfig("bal", 512, 128, 32, 4, 64, 0, zipf_bias=True, seed=17)
    x, wr, b = I.gen_x(cfg), I.gen_router_w(cfg), I.gen_router_b(cfg)
    def loads(bias):
        ids, _ = moe.topk_select(moe.router_logits(x, wr, bias), cfg.top_k)
        return np.bincount(ids.reshape(-1), minlength=cfg.num_experts)
    c0 = loads(b)
    for _ in range(40):
        b = moe.router_bias_update(b, loads(b), cfg.tokens, cfg.top_k, 0.2)
    c1 = loads(b)
    mean = cfg.tokens * cfg.top_k / cfg.num_experts
    assert c1.max() < 0.5 * c0.max() and np.std(c1) < 0.5 * np.std(c0)
    assert abs(c1.max() - mean) < abs(c0.max() - mean)
