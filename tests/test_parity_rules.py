"""CPU checks of the layer comparison rules in parity.py.

A stand-in for a GPU result is built from the oracle's own outputs for a small
layer, then one mistake is planted in it: the comparison must accept exactly
what its contract allows and reject the rest.  No GPU is used.
"""

import numpy as np
import pytest
import torch

from mxfp4_expert_grouped_amd import inputs as I
from oracle import moe as OM
from oracle import mx as OX

import parity as P  # noqa: E402


CFG = I.LayerConfig("rules", 64, 256, 16, 2, 128, 1, seed=5)


def _oracle_as_gpu(cfg):
    x = I.gen_x(cfg)
    wr = I.gen_router_w(cfg)
    W = I.ExpertWeights(cfg)
    res = OM.forward(x, wr, None, W, num_experts=cfg.num_experts, top_k=cfg.top_k,
                     num_shared=cfg.num_shared, d_ff=cfg.d_ff)
    T, k, S, f = cfg.tokens, cfg.top_k, cfg.num_shared, cfg.d_ff
    h_codes = np.zeros((T * k + S * T, f), np.uint8)
    h_scales = np.zeros((T * k + S * T, f // 32), np.uint8)
    for r in range(T * k):
        h_codes[r], h_scales[r] = res.h_rows[r]
    for s in range(S):
        for t in range(T):
            h_codes[T * k + s * T + t], h_scales[T * k + s * T + t] = res.h_shared[(s, t)]
    g = {
        "logits": res.logits.astype(np.float32), "topk_ids": res.topk_ids.astype(np.int32),
        "topk_w": res.topk_w.astype(np.float32), "expert_offsets": res.offsets.copy(),
        "row_src": res.row_src.copy(), "token_row": res.token_row.copy(),
        "x_codes": res.x_codes.copy(), "x_scales": res.x_scales.copy(),
        "h_codes": h_codes, "h_scales": h_scales,
        "y_routed": res.y_routed.copy(), "y_shared": res.y_shared.copy(),
    }
    return x, wr, W, res, g


def _set_y(g):
    bits = OM.f64_to_bf16(g["y_routed"] + g["y_shared"])
    g["y"] = torch.from_numpy(bits.view(np.int16).copy())


def _plant_shared_flip(cfg, res, W, g, move_code):
    """Move the largest shared-expert h element of token 0 by one E4M3 step
    (toward zero: a block's largest element sits near the top of the range)
    and shift y_shared by that step times its W_dn column.
    With move_code False the h byte keeps the oracle's value: the same output
    error then has no differing byte to account for it."""
    t, s = 0, 0
    r = cfg.tokens * cfg.top_k + s * cfg.tokens + t
    hc, hs = res.h_shared[(s, t)]
    vals = OX.decode_e4m3(np.arange(256))
    col = int(np.argmax(np.abs(vals[hc])))
    c = int(hc[col])
    assert (c & 0x7F) >= 1
    c2 = c - 1                              # one step toward zero, same sign
    dh = (vals[c2] - vals[c]) * OX.decode_e8m0(hs[col // 32])
    wcol = P._dn_columns(W("shared", s)[2], W("shared", s)[3], np.array([col]))[:, 0]
    if move_code:
        g["h_codes"][r, col] = c2
    g["y_shared"][t] += dh * wcol
    _set_y(g)
    rms = np.sqrt(np.mean(res.y_shared ** 2))
    return np.max(np.abs(dh * wcol)) / rms


def test_oracle_against_itself_passes():
    x, wr, W, res, g = _oracle_as_gpu(CFG)
    _set_y(g)
    P.compare_layer(CFG, x, wr, None, W, g)


def test_output_effect_of_a_flipped_h_byte_is_allowed():
    x, wr, W, res, g = _oracle_as_gpu(CFG)
    effect = _plant_shared_flip(CFG, res, W, g, move_code=True)
    assert effect > P.MAX_ERR_RMS, "the planted step must exceed the plain elementwise bar"
    P.compare_layer(CFG, x, wr, None, W, g)


def test_same_output_error_without_a_flipped_byte_is_rejected():
    x, wr, W, res, g = _oracle_as_gpu(CFG)
    effect = _plant_shared_flip(CFG, res, W, g, move_code=False)
    assert effect > P.MAX_ERR_RMS
    with pytest.raises(AssertionError, match="max error"):
        P.compare_layer(CFG, x, wr, None, W, g)
