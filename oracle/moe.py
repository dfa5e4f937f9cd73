"""The sparse MoE layer, step by step, in float64 (oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Structure from the pages ("Kimi K3 Tech Intro", section 4.3 "MXFP4 MoE +
SiTU"): input token -> router (top-16) -> routed experts + shared expert(s);
16 of 896 routed experts per token ("Kimi K3 Tech Intro", section 1 table;
"K3部署推理引擎指南", Stable LatentMoE paragraph) and 2 shared experts
("Kimi K3本地部署指南", section 1 spec table); MXFP4 expert weights with MXFP8
activations ("Kimi K3 ... MoE推理系统工程分析").  The pages leave the router's
score function, the activation (SiTU is named, not defined) and the combine
rule open; the readings taken are:

* logits l = x W_r^T + b (x bf16, W_r and b fp32), selection on l, ties to the
  lower expert index, ids reported in ascending order;
* weights w = sigmoid(l) / sum of sigmoid(l) over the selected experts;
* expert MLP: [g | u] = A W_gu^T, h = silu(g) * u (SwiGLU standing in for SiTU),
  h re-quantised to MXFP8 along d_ff, o = h W_dn^T; A is x quantised to MXFP8;
* y = sum_j w[t, j] o_j + sum_s o_s (shared experts unweighted).

Everything runs in float64 on exactly decoded MX values.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Dict, Optional, Sequence, Tuple

import numpy as np

from . import mx


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 (exact: bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16(v) -> np.ndarray:
    """float64 -> bf16 bit patterns, round-to-nearest-even on the bf16 grid.

    Done in exact arithmetic: split |v| into binary exponent and a 53-bit
    significand, keep 8 significant bits with ties to even.  Finite inputs only.
    """
    v = np.asarray(v, dtype=np.float64)
    assert np.all(np.isfinite(v))
    out = np.zeros(v.shape, dtype=np.uint16)
    a = np.abs(v)
    nz = a > 0
    m, ex = np.frexp(a)  # a = m * 2**ex, m in [0.5, 1)
    # bf16 normal: 8 significant bits; below 2**-126 the grid step is 2**-133
    step_exp = np.maximum(ex - 8, -133)
    q = a / np.exp2(step_exp)  # exact (power-of-two scaling)
    r = np.floor(q)
    frac = q - r
    r = r + ((frac > 0.5) | ((frac == 0.5) & (np.fmod(r, 2) == 1)))
    val = r * np.exp2(step_exp)  # the rounded magnitude, exact
    f32 = val.astype(np.float32)  # exactly representable -> exact cast
    bits = (f32.view(np.uint32) >> 16).astype(np.uint16)
    out[nz] = bits[nz]
    out = out | np.where(np.signbit(v), 0x8000, 0).astype(np.uint16)
    return out


# --------------------------------------------------------------------------
# Router
# --------------------------------------------------------------------------


def router_logits(x_bf16, w_r, b=None) -> np.ndarray:
    """l[t, e] = sum_i x[t, i] * W_r[e, i] + b[e], float64.

    Products of a bf16 and an fp32 value are exact in float64, so the only
    rounding is the float64 summation.
    """
    x = bf16_to_f64(x_bf16)
    w = np.asarray(w_r, dtype=np.float32).astype(np.float64)
    l = x @ w.T
    if b is not None:
        l = l + np.asarray(b, dtype=np.float32).astype(np.float64)[None, :]
    return l


def topk_select(logits, k: int):
    """Per row: the k experts with the largest logits (ties -> lower index).

    Returns (ids ascending [T, k] int32, gap [T]) where gap is the difference
    between the k-th and (k+1)-th largest logits (inf when k == E): tokens whose
    gap is tiny are the ones where a different but equally valid set may come
    out of a lower-precision computation.
    """
    l = np.asarray(logits, dtype=np.float64)
    t_count, e_count = l.shape
    idx = np.broadcast_to(np.arange(e_count), l.shape)
    # per row: primary key logit descending, then expert index ascending
    order = np.lexsort((idx, -l), axis=-1)
    ids = np.sort(order[:, :k], axis=1).astype(np.int32)
    gap = np.full(t_count, np.inf)
    if k < e_count:
        rows = np.arange(t_count)
        gap = l[rows, order[:, k - 1]] - l[rows, order[:, k]]
    return ids, gap


def sigmoid(v):
    v = np.asarray(v, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-v))


def routing_weights(logits, ids) -> np.ndarray:
    """w[t, j] = sigmoid(l[t, ids[t, j]]) / sum_j' sigmoid(l[t, ids[t, j']])."""
    sel = np.take_along_axis(np.asarray(logits, np.float64), np.asarray(ids, np.int64), axis=1)
    s = sigmoid(sel)
    return s / s.sum(axis=1, keepdims=True)


def router_bias_update(b, counts, num_tokens: int, top_k: int, rate: float) -> np.ndarray:
    """One balancing step of the router bias from the loads of a batch.

    "Kimi K3 Tech Intro" (section 1 table, section 4.3) names "quantile
    balancing" for the router without defining it; the router bias is the
    layer's only balancing hook.  The step taken here: an expert loaded above
    the mean load T*k/E has its bias lowered by `rate`, one below it raised
    by `rate`, one exactly at it kept (b_e + rate * sign(mean - c_e)).  The
    bias is an fp32 tensor, so the update is one fp32 addition per expert:
    computed here in float32 exactly as defined, rate rounded to fp32 first.
    """
    b = np.asarray(b, dtype=np.float32)
    c = np.asarray(counts, dtype=np.float64)
    mean = num_tokens * top_k / b.size
    step = np.sign(mean - c).astype(np.float32) * np.float32(rate)
    return (b + step).astype(np.float32)


# --------------------------------------------------------------------------
# Permutation
# --------------------------------------------------------------------------


def permute(ids, num_experts: int):
    """Expert-contiguous order of the (token, slot) pairs.

    Pairs are sorted by (expert ascending, token ascending); pair p = t*k + j.
    Returns counts [E], offsets [E+1], row_src [T*k] (pair index of each
    permuted row) and token_row [T, k] (permuted row of each pair).
    """
    ids = np.asarray(ids, dtype=np.int64)
    t_count, k = ids.shape
    pair_expert = ids.reshape(-1)
    pair_token = np.repeat(np.arange(t_count), k)
    key = pair_expert * t_count + pair_token
    row_src = np.argsort(key, kind="stable").astype(np.int32)
    counts = np.bincount(pair_expert, minlength=num_experts).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    token_row = np.empty(t_count * k, dtype=np.int32)
    token_row[row_src] = np.arange(t_count * k, dtype=np.int32)
    return counts, offsets, row_src, token_row.reshape(t_count, k)


# --------------------------------------------------------------------------
# Experts
# --------------------------------------------------------------------------


def silu(g):
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):  # exp(-g) = inf for g < -709: the quotient is then -0
        return g / (1.0 + np.exp(-g))


def expert_mlp(a_codes, a_scales, gu_codes, gu_scales, dn_codes, dn_scales, d_ff: int,
               intermediates: Optional[dict] = None):
    """One expert on a set of MXFP8 rows.

    A = decoded MXFP8 rows [n, d]; [g | u] = A W_gu^T with W_gu [2 d_ff, d]
    (rows [0, d_ff) gate, [d_ff, 2 d_ff) up); h = silu(g) * u; h quantised to
    MXFP8 along d_ff; o = dec(h_q) W_dn^T with W_dn [d, d_ff].
    Returns (h_codes [n, d_ff], h_scales [n, d_ff/32], o [n, d] float64).

    With a dict ``intermediates`` it also receives the float64 values the
    definition passes through: "gu" ([g | u], [n, 2 d_ff]), "h" (before its
    quantisation, [n, d_ff]), and the magnitudes of the terms of each dot
    product, "gu_abs" = |A| |W_gu|^T and "o_abs" = |dec(h_q)| |W_dn|^T (the
    scale of the rounding error any finite-precision evaluation of those sums
    can make).
    """
    a = mx.mx_decode(a_codes, a_scales, "e4m3")
    wgu = mx.mx_decode(gu_codes, gu_scales, "e2m1")
    gu = a @ wgu.T
    if intermediates is not None:
        intermediates["gu"] = gu
        intermediates["gu_abs"] = np.abs(a) @ np.abs(wgu).T
    del wgu
    g, u = gu[:, :d_ff], gu[:, d_ff:]
    h = silu(g) * u
    h_codes, h_scales = mx.mx_quantize(h, "e4m3")
    hq = mx.mx_decode(h_codes, h_scales, "e4m3")
    wdn = mx.mx_decode(dn_codes, dn_scales, "e2m1")
    o = hq @ wdn.T
    if intermediates is not None:
        intermediates["h"] = h
        intermediates["o_abs"] = np.abs(hq) @ np.abs(wdn).T
    return h_codes, h_scales, o


def expert_mlp_a16(a_bf16, gu_codes, gu_scales, dn_codes, dn_scales, d_ff: int,
                   intermediates: Optional[dict] = None):
    """One expert with bf16 activations and MXFP4 weights (the A16W4 variant
    of "Kimi K3 Tech Intro", sections 4.3 and 10): A = the bf16 rows as they
    are; [g | u] = A W_gu^T; h = silu(g) * u rounded to bf16 (round to
    nearest even), the 16-bit activation between the two projections;
    o = h W_dn^T.  Returns (h bf16 bit patterns [n, d_ff], o [n, d] float64).
    ``intermediates`` as for expert_mlp ("gu", "gu_abs", "h" before its
    rounding, "o_abs")."""
    a = bf16_to_f64(a_bf16)
    wgu = mx.mx_decode(gu_codes, gu_scales, "e2m1")
    gu = a @ wgu.T
    if intermediates is not None:
        intermediates["gu"] = gu
        intermediates["gu_abs"] = np.abs(a) @ np.abs(wgu).T
    del wgu
    h = silu(gu[:, :d_ff]) * gu[:, d_ff:]
    h_bits = f64_to_bf16(h)
    hq = bf16_to_f64(h_bits)
    wdn = mx.mx_decode(dn_codes, dn_scales, "e2m1")
    o = hq @ wdn.T
    if intermediates is not None:
        intermediates["h"] = h
        intermediates["o_abs"] = np.abs(hq) @ np.abs(wdn).T
    return h_bits, o


def _expert_job(job):
    """One expert on its rows: job = (weights, kind, index, a_codes, a_scales,
    d_ff, intermediates, activations) -> (h_codes, h_scales, o, mid); with
    bf16 activations a_codes are the rows' bf16 bits, h_codes h's bf16 bits
    and h_scales None."""
    weights, kind, index, a_codes, a_scales, d_ff, intermediates, activations = job
    mid = {} if intermediates else None
    if activations == "bf16":
        h_c, o = expert_mlp_a16(a_codes, *weights(kind, index), d_ff=d_ff, intermediates=mid)
        return h_c, None, o, mid
    h_c, h_s, o = expert_mlp(a_codes, a_scales, *weights(kind, index), d_ff=d_ff, intermediates=mid)
    return h_c, h_s, o, mid


# --------------------------------------------------------------------------
# Whole layer
# --------------------------------------------------------------------------

# weights(kind, index) -> (gu_codes, gu_scales, dn_codes, dn_scales) of routed
# expert `index` (kind "routed") or shared expert `index` (kind "shared")
WeightSource = Callable[[str, int], Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]]


@dataclass
class LayerResult:
    logits: np.ndarray
    gap: np.ndarray
    topk_ids: np.ndarray
    topk_w: np.ndarray
    counts: np.ndarray
    offsets: np.ndarray
    row_src: np.ndarray
    token_row: np.ndarray
    tokens: np.ndarray  # tokens whose activations and outputs below were computed
    x_codes: np.ndarray  # [len(tokens), d]
    x_scales: np.ndarray
    y_routed: np.ndarray  # [len(tokens), d] float64
    y_shared: np.ndarray
    y: np.ndarray
    # h in permuted-row order for the computed tokens: {row: (codes, scales)}
    h_rows: Dict[int, Tuple[np.ndarray, np.ndarray]] = field(default_factory=dict)
    # shared-expert h for the computed tokens: {(s, t): (codes, scales)}
    h_shared: Dict[Tuple[int, int], Tuple[np.ndarray, np.ndarray]] = field(default_factory=dict)
    # with intermediates=True: per routed row / per (s, t) the float64 values
    # of expert_mlp's intermediates dict ("gu", "gu_abs", "h", "o_abs", and
    # "o", the row's down-projection output), one row each
    mid_rows: Dict[int, Dict[str, np.ndarray]] = field(default_factory=dict)
    mid_shared: Dict[Tuple[int, int], Dict[str, np.ndarray]] = field(default_factory=dict)


def forward(x_bf16, w_r, b, weights: WeightSource, *, num_experts: int, top_k: int,
            num_shared: int, d_ff: int, tokens: Optional[Sequence[int]] = None,
            topk_ids=None, intermediates: bool = False, logits=None,
            expert_map=map, activations: str = "mxfp8") -> LayerResult:
    """Full layer.  Routing, permutation and the MXFP8 quantisation of x are
    computed for every token; expert outputs only for ``tokens`` (all when
    None).  Each token's output depends only on its own row, so a subset gives
    exactly the rows the full computation would.  Experts are visited one at a
    time so the decoded float64 weights of only one expert are live.

    ``topk_ids`` ([T, top_k] expert ids, ascending per row), when given,
    replaces the selection: the layer is evaluated for that routing (weights
    sigmoid(l)/sum sigmoid(l) over those experts, their permutation, their
    experts), as for a token whose k-th and (k+1)-th logits are so close that
    another evaluation of the logits may legitimately pick the other expert.
    ``gap`` is still the one of the layer's own selection.  ``logits``, when
    given, must be this function's own router_logits(x_bf16, w_r, b) from an
    earlier call (it saves recomputing them for another subset of tokens).
    ``expert_map(fn, jobs)`` evaluates the independent per-expert jobs (the
    builtin map: one after another here; a process pool's map runs them side
    by side); results are used in job order.
    ``activations``: "mxfp8" (the layer: MXFP8 x and h) or "bf16" (the A16W4
    variant: x as given, h rounded to bf16; expert_mlp_a16).  With "bf16",
    x_codes holds the computed tokens' bf16 bits, x_scales has no columns,
    and h_rows / h_shared hold (h bf16 bits, None).
    """
    assert activations in ("mxfp8", "bf16")
    x_bf16 = np.asarray(x_bf16, dtype=np.uint16)
    t_count, d = x_bf16.shape
    if logits is None:
        logits = router_logits(x_bf16, w_r, b)
    ids, gap = topk_select(logits, top_k)
    if topk_ids is not None:
        given = np.asarray(topk_ids, dtype=np.int64)
        assert given.shape == ids.shape
        assert np.all((given >= 0) & (given < num_experts))
        assert np.all(np.diff(given, axis=1) > 0), "ids must be distinct and ascending per row"
        ids = given.astype(np.int32)
    w = routing_weights(logits, ids)
    counts, offsets, row_src, token_row = permute(ids, num_experts)

    toks = np.arange(t_count) if tokens is None else np.asarray(sorted(set(int(t) for t in tokens)))
    pos = {int(t): i for i, t in enumerate(toks)}
    # MXFP8 activations of the computed tokens (row i <-> token toks[i])
    if activations == "bf16":
        x_codes, x_scales = x_bf16[toks].copy(), np.zeros((len(toks), 0), np.uint8)
    else:
        x_codes, x_scales = mx.mx_quantize(bf16_to_f64(x_bf16[toks]), "e4m3")
    y_routed = np.zeros((len(toks), d))
    y_shared = np.zeros((len(toks), d))
    res_h: Dict[int, Tuple[np.ndarray, np.ndarray]] = {}
    res_hs: Dict[Tuple[int, int], Tuple[np.ndarray, np.ndarray]] = {}
    res_mid: Dict[int, Dict[str, np.ndarray]] = {}
    res_mids: Dict[Tuple[int, int], Dict[str, np.ndarray]] = {}

    # one job per expert with rows among the computed tokens: the routed
    # experts in order, then the shared experts on every computed token
    want = np.zeros(t_count, dtype=bool)
    want[toks] = True
    jobs, placement = [], []
    for e in range(num_experts):
        rows = np.arange(offsets[e], offsets[e + 1])
        rows = rows[want[row_src[rows] // top_k]]
        if rows.size == 0:
            continue
        pairs = row_src[rows]
        xi = np.array([pos[int(t)] for t in pairs // top_k])
        jobs.append((weights, "routed", e, x_codes[xi], x_scales[xi], d_ff, intermediates, activations))
        placement.append(("routed", e, rows, pairs // top_k, pairs % top_k))
    for s in range(num_shared):
        jobs.append((weights, "shared", s, x_codes, x_scales, d_ff, intermediates, activations))
        placement.append(("shared", s, None, toks, None))
    # expert_map only decides where the jobs run (default: here, in order);
    # the results are summed below in job order either way
    for (kind, e, rows, tk, jj), (h_c, h_s, o, mid) in zip(placement, expert_map(_expert_job, jobs)):
        if kind == "routed":
            for i in range(rows.size):
                res_h[int(rows[i])] = (h_c[i], None if h_s is None else h_s[i])
                y_routed[pos[int(tk[i])]] += w[tk[i], jj[i]] * o[i]
                if intermediates:
                    res_mid[int(rows[i])] = dict({k: v[i] for k, v in mid.items()}, o=o[i])
        else:
            for i, t in enumerate(toks):
                res_hs[(e, int(t))] = (h_c[i], None if h_s is None else h_s[i])
                if intermediates:
                    res_mids[(e, int(t))] = dict({k: v[i] for k, v in mid.items()}, o=o[i])
            y_shared += o
    return LayerResult(logits=logits, gap=gap, topk_ids=ids, topk_w=w, counts=counts,
                       offsets=offsets, row_src=row_src, token_row=token_row,
                       x_codes=x_codes, x_scales=x_scales, tokens=toks,
                       y_routed=y_routed, y_shared=y_shared, y=y_routed + y_shared,
                       h_rows=res_h, h_shared=res_hs, mid_rows=res_mid, mid_shared=res_mids)


def forward_dense(x_bf16, w_r, b, weights: WeightSource, *, num_experts: int, top_k: int,
                  num_shared: int, d_ff: int, activations: str = "mxfp8") -> np.ndarray:
    """The same layer computed densely: every expert on every token, scaled by a
    full [T, E] weight matrix that is zero for unselected experts.  Used only to
    pin :func:`forward` (sparse gather/scatter) against a computation that has
    no permutation at all.
    """
    x_bf16 = np.asarray(x_bf16, dtype=np.uint16)
    t_count, d = x_bf16.shape
    logits = router_logits(x_bf16, w_r, b)
    ids, _ = topk_select(logits, top_k)
    w = routing_weights(logits, ids)
    dense_w = np.zeros((t_count, num_experts))
    np.put_along_axis(dense_w, ids.astype(np.int64), w, axis=1)
    x_codes, x_scales = mx.mx_quantize(bf16_to_f64(x_bf16), "e4m3")

    def run(kind, idx):
        if activations == "bf16":
            return expert_mlp_a16(x_bf16, *weights(kind, idx), d_ff=d_ff)[1]
        return expert_mlp(x_codes, x_scales, *weights(kind, idx), d_ff=d_ff)[2]

    y = np.zeros((t_count, d))
    for e in range(num_experts):
        y += dense_w[:, e:e + 1] * run("routed", e)
    for s in range(num_shared):
        y += run("shared", s)
    return y


# --------------------------------------------------------------------------
# LatentMoE tail ("Kimi K3 Tech Intro", section 4.3: after the routed and
# shared experts come the latent up-projection, RMSNorm and an element-wise
# add; section 4.4: the routed output goes through RMSNorm and the up
# projection, the shared output is added to it directly)
# --------------------------------------------------------------------------


def rms_norm(z, gamma, eps: float) -> np.ndarray:
    """Each row z / sqrt(mean(z^2) + eps), times the per-column gain gamma (float64)."""
    z = np.asarray(z, dtype=np.float64)
    ms = np.mean(z * z, axis=1, keepdims=True)
    return z / np.sqrt(ms + eps) * np.asarray(gamma, dtype=np.float64)[None, :]


def latent_tail(z, gamma, eps: float, up_codes, up_scales, s=None,
                intermediates: Optional[dict] = None) -> np.ndarray:
    """y = MXFP8(RMSNorm(z)) W_up^T + s for the routed experts' weighted sum z
    [T, l] (float32 values), the gain gamma [l], the up projection W_up
    [H, l] in MXFP4 (codes [H, l/2], scales [H, l/32]) and the shared
    experts' output s [T, H] (None: zero).  The normalised rows enter the
    projection as MXFP8 (32-element blocks along l), like every activation
    of the layer.  Returns y [T, H] in float64 (the layer rounds it to bf16).
    With a dict `intermediates`: "n" (the normalised rows, float64), "a_codes",
    "a_scales" (their MXFP8 bytes), "y_abs" (|A| |W_up|^T, the magnitude of
    the dot products' terms).
    """
    n = rms_norm(z, gamma, eps)
    a_codes, a_scales = mx.mx_quantize(n, "e4m3")
    a = mx.mx_decode(a_codes, a_scales, "e4m3")
    w = mx.mx_decode(up_codes, up_scales, "e2m1")
    y = a @ w.T
    if s is not None:
        y = y + np.asarray(s, dtype=np.float64)
    if intermediates is not None:
        intermediates.update(n=n, a_codes=a_codes, a_scales=a_scales, y_abs=np.abs(a) @ np.abs(w).T)
    return y
