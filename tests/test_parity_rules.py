"""CPU checks of the layer comparison rules in parity.py.

A stand-in for a GPU result is built from the oracle's own outputs for a small
layer (its gate/up accumulators rounded to fp32, as the GPU writes them), then
one mistake or one legitimate difference is planted in it: the comparison
must accept exactly what its contract allows and reject the rest.  No GPU is
used.
"""

import numpy as np
import pytest
import torch

from mxfp4_expert_grouped_amd import inputs as I
from oracle import moe as OM
from oracle import mx as OX

import parity as P  # noqa: E402


CFG = I.LayerConfig("rules", 64, 256, 16, 2, 128, 1, seed=5)


def _oracle_as_gpu(cfg, bias=None, ids=None):
    x = I.gen_x(cfg)
    wr = I.gen_router_w(cfg)
    W = I.ExpertWeights(cfg)
    res = OM.forward(x, wr, bias, W, num_experts=cfg.num_experts, top_k=cfg.top_k,
                     num_shared=cfg.num_shared, d_ff=cfg.d_ff, topk_ids=ids, intermediates=True)
    T, k, S, f = cfg.tokens, cfg.top_k, cfg.num_shared, cfg.d_ff
    R = T * k + S * T
    h_codes = np.zeros((R, f), np.uint8)
    h_scales = np.zeros((R, f // 32), np.uint8)
    gu_acc = np.zeros((R, 2 * f), np.float32)
    for r in range(T * k):
        h_codes[r], h_scales[r] = res.h_rows[r]
        gu_acc[r] = res.mid_rows[r]["gu"]
    for s in range(S):
        for t in range(T):
            r = T * k + s * T + t
            h_codes[r], h_scales[r] = res.h_shared[(s, t)]
            gu_acc[r] = res.mid_shared[(s, t)]["gu"]
    taps = {
        "logits": res.logits.astype(np.float32), "topk_ids": res.topk_ids.astype(np.int32),
        "topk_w": res.topk_w.astype(np.float32), "expert_offsets": res.offsets.copy(),
        "row_src": res.row_src.copy(), "token_row": res.token_row.copy(),
        "x_codes": res.x_codes.copy(), "x_scales": res.x_scales.copy(),
        "h_codes": h_codes, "h_scales": h_scales, "gu_acc": gu_acc,
        "y_routed": res.y_routed.copy(), "y_shared": res.y_shared.copy(),
    }
    g = P.Run(taps, None)
    _set_y(g)
    return x, wr, W, res, g


def _set_y(g):
    bits = OM.f64_to_bf16(g.taps["y_routed"] + g.taps["y_shared"])
    g.y = torch.from_numpy(bits.view(np.int16).copy())


def _shared_row(cfg, t, s=0):
    return cfg.tokens * cfg.top_k + s * cfg.tokens + t


def _shift_outputs(cfg, W, g, t, s, col, dh):
    wcol = P._dn_columns(W("shared", s)[2], W("shared", s)[3], np.array([col]))[:, 0]
    g.taps["y_shared"][t] += dh * wcol
    _set_y(g)
    return wcol


def _vals():
    return OX.decode_e4m3(np.arange(256))


def _largest_shared_element(res, t=0, s=0):
    hc, hs = res.h_shared[(s, t)]
    vals = _vals()
    col = int(np.argmax(np.abs(vals[hc])))
    return col, hc, hs


def test_oracle_against_itself_passes():
    x, wr, W, res, g = _oracle_as_gpu(CFG)
    P.compare_layer(CFG, x, wr, None, W, g)


def _plant_genuine_flip(cfg, res, W, g):
    """Move one shared-expert up accumulator (within the accumulator bound) just
    across the rounding midpoint of its h element, give that element the code
    of the new value and the outputs its exact effect -- what a GPU whose fp32
    sum landed on the other side of a boundary produces."""
    f = cfg.d_ff
    vals = _vals()
    best = None
    for t in range(cfg.tokens):
        mid = res.mid_shared[(0, t)]
        hc, hs = res.h_shared[(0, t)]
        h, gu, gu_abs = mid["h"], mid["gu"], mid["gu_abs"]
        blocks = np.abs(h).reshape(-1, 32)
        for c in range(f):
            if np.abs(h[c]) >= blocks[c // 32].max() or h[c] == 0:
                continue  # keep the block maximum, so the scale byte stays
            e = float(hs[c // 32]) - 127
            q = h[c] / 2 ** e
            v = vals[hc[c]]
            # neighbour on the far side of q from its code value
            others = np.abs(vals[:0x7F])
            up = others[others > abs(v)].min() if abs(v) < 448 else None
            if up is None:
                continue
            m = np.sign(q) * (abs(v) + up) / 2
            need = (m * (1 + 1e-6) - q) * 2 ** e  # h change that crosses the midpoint
            silu_g = OM.silu(gu[c])
            du = need / silu_g
            ratio = abs(du) / gu_abs[f + c]
            if best is None or ratio < best[0]:
                best = (ratio, t, c, du)
    ratio, t, c, du = best
    assert ratio < 0.2 * P.EPS_ACC, "no element close enough to a midpoint for a legitimate flip"
    r = _shared_row(cfg, t)
    acc = g.taps["gu_acc"]
    acc[r, f + c] = np.float32(res.mid_shared[(0, t)]["gu"][f + c] + du)
    h_new = OM.silu(acc[r, :f].astype(np.float64)) * acc[r, f:].astype(np.float64)
    qc, qs = OX.mx_quantize(h_new[None], "e4m3")
    hc, hs = res.h_shared[(0, t)]
    assert np.array_equal(qs[0], hs), "the planted change must keep the scale bytes"
    diff = np.nonzero(qc[0] != hc)[0]
    assert c in diff
    old = OX.mx_decode(hc[None], hs[None], "e4m3")[0]
    new = OX.mx_decode(qc, qs, "e4m3")[0]
    g.taps["h_codes"][r] = qc[0]
    for col in diff:
        _shift_outputs(cfg, W, g, t, 0, int(col), new[col] - old[col])
    return t, c


def test_genuine_one_step_flip_is_accepted():
    x, wr, W, res, g = _oracle_as_gpu(CFG)
    _plant_genuine_flip(CFG, res, W, g)
    P.compare_layer(CFG, x, wr, None, W, g)


def test_flip_the_accumulators_do_not_explain_is_rejected():
    # one E4M3 step on a byte whose accumulators say otherwise, outputs moved
    # consistently: the byte is not the quantisation of the GPU's own sums
    x, wr, W, res, g = _oracle_as_gpu(CFG)
    col, hc, hs = _largest_shared_element(res)
    r = _shared_row(CFG, 0)
    c = int(hc[col])
    g.taps["h_codes"][r, col] = c - 1
    dh = (_vals()[c - 1] - _vals()[c]) * OX.decode_e8m0(hs[col // 32])
    _shift_outputs(CFG, W, g, 0, 0, col, dh)
    with pytest.raises(AssertionError, match="not at a rounding midpoint|not the quantisation"):
        P.compare_layer(CFG, x, wr, None, W, g)


@pytest.mark.parametrize("with_acc", [True, False])
def test_two_step_flip_is_rejected(with_acc):
    x, wr, W, res, g = _oracle_as_gpu(CFG)
    if not with_acc:
        del g.taps["gu_acc"]
    col, hc, hs = _largest_shared_element(res)
    r = _shared_row(CFG, 0)
    c = int(hc[col])
    g.taps["h_codes"][r, col] = c - 2
    dh = (_vals()[c - 2] - _vals()[c]) * OX.decode_e8m0(hs[col // 32])
    _shift_outputs(CFG, W, g, 0, 0, col, dh)
    with pytest.raises(AssertionError, match="more than one E4M3 step|not the quantisation"):
        P.compare_layer(CFG, x, wr, None, W, g)


def test_accumulator_outside_the_bound_is_rejected():
    x, wr, W, res, g = _oracle_as_gpu(CFG)
    r = 5
    mid = res.mid_rows[r]
    c = int(np.argmax(mid["gu_abs"]))
    g.taps["gu_acc"][r, c] = np.float32(mid["gu"][c] + 3 * P.EPS_ACC * mid["gu_abs"][c])
    with pytest.raises(AssertionError, match="accumulators off"):
        P.compare_layer(CFG, x, wr, None, W, g)


def test_same_output_error_without_a_flipped_byte_is_rejected():
    x, wr, W, res, g = _oracle_as_gpu(CFG)
    rms = np.sqrt(np.mean(res.y_shared ** 2))
    # the token whose largest shared-expert h element, moved one E4M3 step,
    # moves an output the most
    best = None
    for t in range(CFG.tokens):
        col, hc, hs = _largest_shared_element(res, t)
        c = int(hc[col])
        dh = (_vals()[c - 1] - _vals()[c]) * OX.decode_e8m0(hs[col // 32])
        wcol = P._dn_columns(W("shared", 0)[2], W("shared", 0)[3], np.array([col]))[:, 0]
        m = float(np.max(np.abs(dh * wcol)))
        if best is None or m > best[0]:
            best = (m, t, col, dh)
    m, t, col, dh = best
    _shift_outputs(CFG, W, g, t, 0, col, dh)
    assert m / rms > P.MAX_ERR_RMS, "must exceed the plain elementwise bar"
    with pytest.raises(AssertionError, match="max error|relative L2 error"):
        P.compare_layer(CFG, x, wr, None, W, g)


def test_small_error_inside_the_contract_but_above_the_arithmetic_bound_is_rejected():
    # 1e-3 * rms on one element passes the 5e-2 * rms contract bar but not the
    # per-element bound from the arithmetic (bf16 rounding + accumulation)
    x, wr, W, res, g = _oracle_as_gpu(CFG)
    rms = np.sqrt(np.mean(res.y_routed ** 2))
    t, c = 7, 100
    g.taps["y_routed"][t, c] += 1e-3 * rms + 0.01 * abs(res.y_routed[t, c])
    _set_y(g)
    with pytest.raises(AssertionError, match="arithmetic bound"):
        P.compare_layer(CFG, x, wr, None, W, g)


def _near_tie_case():
    """A token whose 2nd and 3rd logits are 5e-7 apart (through the bias):
    an fp32 evaluation may pick either expert.  Returns the inputs, the
    oracle's own selection and the swapped one."""
    x, wr = I.gen_x(CFG), I.gen_router_w(CFG)
    l = OM.router_logits(x, wr)
    t = 3
    order = np.argsort(-l[t], kind="stable")
    e_in, e_out = int(order[1]), int(order[2])
    b = np.zeros(CFG.num_experts, np.float32)
    b[e_out] = np.float32(l[t, e_in] - l[t, e_out] - 5e-7)
    l2 = OM.router_logits(x, wr, b)
    own, gap = OM.topk_select(l2, CFG.top_k)
    assert gap[t] < P.TAU and e_in in own[t] and e_out not in own[t]
    swapped = own.copy()
    swapped[t] = np.sort([e_out if e == e_in else e for e in own[t]])
    return b, t, own, swapped


def test_near_tie_token_is_compared_with_the_oracle_on_the_gpu_routing():
    b, t, own, swapped = _near_tie_case()
    x, wr, W, res, g = _oracle_as_gpu(CFG, bias=b, ids=swapped)
    res2, differ = P.compare_layer(CFG, x, wr, b, W, g)
    assert differ == {t}
    assert t in res2.tokens.tolist()


def test_error_on_a_near_tie_token_is_caught():
    b, t, own, swapped = _near_tie_case()
    x, wr, W, res, g = _oracle_as_gpu(CFG, bias=b, ids=swapped)
    rms = np.sqrt(np.mean(res.y_routed ** 2))
    g.taps["y_routed"][t] += 0.1 * rms
    _set_y(g)
    with pytest.raises(AssertionError, match="y_routed"):
        P.compare_layer(CFG, x, wr, b, W, g)


def test_swap_that_is_not_a_near_tie_is_rejected():
    x, wr, W, res, g = _oracle_as_gpu(CFG)
    ids = g.taps["topk_ids"]
    t = 10
    gap = OM.topk_select(res.logits, CFG.top_k)[1]
    if gap[t] < P.TAU:
        t = 11
    other = [e for e in range(CFG.num_experts) if e not in ids[t]][0]
    ids[t] = np.sort([ids[t][0], other])
    with pytest.raises(AssertionError, match="routing differs|near-tie"):
        P.compare_layer(CFG, x, wr, None, W, g)


def test_multi_step_move_of_a_cancelling_accumulator_is_accepted():
    # an up accumulator far smaller than its terms (heavy cancellation): an
    # error well inside the accumulator bound moves its h element by two or
    # more E4M3 steps; bytes that are the quantisation of the moved sums, with
    # the outputs moved by their exact effect, are legitimate
    cfg = CFG
    x, wr, W, res, g = _oracle_as_gpu(cfg)
    f = cfg.d_ff
    vals = _vals()
    best = None
    for t in range(cfg.tokens):
        mid = res.mid_shared[(0, t)]
        cond = mid["gu_abs"][f:] / np.maximum(np.abs(mid["gu"][f:]), 1e-300)
        hb = np.abs(mid["h"]).reshape(-1, 32).max(axis=1)
        for c in np.argsort(-cond)[:8]:
            if abs(mid["h"][c]) < hb[c // 32] / 2 and mid["h"][c] != 0:
                if best is None or cond[c] > best[0]:
                    best = (cond[c], t, int(c))
    cond, t, c = best
    mid = res.mid_shared[(0, t)]
    r = _shared_row(cfg, t)
    acc = g.taps["gu_acc"]
    du = 0.5 * P.EPS_ACC * mid["gu_abs"][f + c] * np.sign(mid["gu"][f + c])
    acc[r, f + c] = np.float32(mid["gu"][f + c] + du)
    h_new = OM.silu(acc[r, :f].astype(np.float64)) * acc[r, f:].astype(np.float64)
    qc, qs = OX.mx_quantize(h_new[None], "e4m3")
    hc, hs = res.h_shared[(0, t)]
    assert np.array_equal(qs[0], hs)
    steps = abs(P._grid_index(vals[qc[0][c:c + 1]]) - P._grid_index(vals[hc[c:c + 1]]))[0]
    assert steps >= 2, f"the planted move is {steps} step(s) (condition {cond:.3g})"
    old = OX.mx_decode(hc[None], hs[None], "e4m3")[0]
    new = OX.mx_decode(qc, qs, "e4m3")[0]
    g.taps["h_codes"][r] = qc[0]
    for col in np.nonzero(qc[0] != hc)[0]:
        _shift_outputs(cfg, W, g, t, 0, int(col), new[col] - old[col])
    P.compare_layer(cfg, x, wr, None, W, g)
