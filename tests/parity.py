"""Shared helpers for the GPU parity tests: run the HIP layer through the C ABI
with every tap attached, run the oracle on the same seeded inputs, and compare
them with the stated rules.

Bars (from the layer's contract):
* routing ids, permutation, and MXFP8 bytes of x: bit-exact, except tokens
  whose oracle gap between the k-th and (k+1)-th logit is below TAU: there a
  different set is accepted if every swapped expert's logit lies within TAU of
  the k-th logit (fp32 accumulation over d=7168 gives ~1e-5 logit error);
* y_routed, y_shared and y, each: relative L2 error <= 5e-3 and, per
  element, |err| <= 5e-2 * rms(reference) + the exact effect of the h bytes
  that differ (their change times their W_dn column, times the routing
  weight for routed rows);
* h bytes: a small fraction may differ by one rounding step (the GPU's fp32 h
  and the oracle's fp64 h can fall on either side of a rounding boundary).
"""

from __future__ import annotations

import sys
import time
from typing import Dict, Optional, Sequence

import numpy as np
import torch

from mxfp4_expert_grouped_amd import inputs as I
from mxfp4_expert_grouped_amd import inputs_gpu as IG
from mxfp4_expert_grouped_amd.layer import DeviceWeights, MoeLayer
from oracle import moe as OM
from oracle import mx as OX

TAU = 1e-4
REL_L2 = 5e-3
MAX_ERR_RMS = 5e-2


def log(msg: str) -> None:
    print(f"[parity {time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def bf16_bits_to_f64(t: torch.Tensor) -> np.ndarray:
    return OM.bf16_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))


def alloc_taps(cfg: I.LayerConfig, T: int, device="cuda", skip=()) -> Dict[str, torch.Tensor]:
    E, k, S, d, f = cfg.num_experts, cfg.top_k, cfg.num_shared, cfg.d_model, cfg.d_ff
    R = T * k + S * T
    z = lambda shape, dt: torch.empty(shape, dtype=dt, device=device)
    taps = dict(
        logits=z((T, E), torch.float32), topk_ids=z((T, k), torch.int32),
        topk_w=z((T, k), torch.float32), expert_offsets=z((E + 1,), torch.int32),
        row_src=z((T * k,), torch.int32), token_row=z((T, k), torch.int32),
        x_codes=z((T, d), torch.uint8), x_scales=z((T, d // 32), torch.uint8),
        h_codes=z((R, f), torch.uint8), h_scales=z((R, f // 32), torch.uint8),
        gu_acc=z((R, 2 * f), torch.float32), y_routed=z((T, d), torch.float32),
        y_shared=z((T, d), torch.float32))
    return {n: t for n, t in taps.items() if n not in skip}


def run_gpu(cfg: I.LayerConfig, W: DeviceWeights, x: torch.Tensor, taps: bool = True,
            workspace_fill: Optional[int] = None, skip=()):
    T = x.shape[0]
    layer = MoeLayer(cfg.d_model, cfg.d_ff, cfg.num_experts, cfg.top_k, cfg.num_shared,
                     max(T, 1), W)
    tp = alloc_taps(cfg, T, skip=skip) if taps and T > 0 else None
    ws = torch.empty(max(layer.workspace_bytes(T), 256), dtype=torch.uint8, device=x.device)
    if workspace_fill is not None:
        ws.fill_(workspace_fill)
    y = torch.zeros_like(x)
    layer.forward(x, y=y, taps=tp, workspace=ws)
    torch.cuda.synchronize()
    out = {k: v.cpu().numpy() for k, v in (tp or {}).items()}
    out["y"] = y
    return out


def device_inputs(cfg: I.LayerConfig, W: Optional[DeviceWeights] = None, bias=None):
    """x and device weights for a config (weights generated on the GPU)."""
    if W is None:
        W = IG.device_weights(cfg)
    if bias is not None:
        W.router_b = torch.from_numpy(np.asarray(bias, np.float32)).cuda()
    return IG.device_x(cfg), W


def check_routing(cfg, res: OM.LayerResult, g: Dict[str, np.ndarray]):
    """Returns the set of tokens whose GPU expert set differs (each one checked
    to be an accepted near-tie)."""
    ids_g = g["topk_ids"]
    T, k = ids_g.shape
    assert np.all(np.diff(ids_g, axis=1) > 0), "GPU ids not strictly ascending"
    assert ids_g.min() >= 0 and ids_g.max() < cfg.num_experts
    differ = np.where(np.any(ids_g != res.topk_ids, axis=1))[0]
    for t in differ:
        assert res.gap[t] < TAU, f"token {t}: routing differs with gap {res.gap[t]}"
        lk = np.sort(res.logits[t])[::-1][k - 1]
        swapped = set(ids_g[t]).symmetric_difference(set(res.topk_ids[t]))
        for e in swapped:
            assert abs(res.logits[t, e] - lk) < TAU, f"token {t}: expert {e} is not a near-tie"
    log(f"routing: {len(differ)} near-tie tokens of {T} differ (accepted)")
    return set(int(t) for t in differ)


def check_permutation(cfg, res: OM.LayerResult, g, differ):
    T, k = g["topk_ids"].shape
    ids = g["topk_ids"].astype(np.int64)
    if not differ:
        assert np.array_equal(g["expert_offsets"], res.offsets)
        assert np.array_equal(g["row_src"], res.row_src)
        assert np.array_equal(g["token_row"], res.token_row)
        return
    # routing differs on near-tie tokens: check the properties that determine
    # the permutation of the GPU's own routing uniquely
    counts = np.bincount(ids.reshape(-1), minlength=cfg.num_experts)
    assert np.array_equal(g["expert_offsets"], np.concatenate([[0], np.cumsum(counts)]))
    rs = g["row_src"].astype(np.int64)
    assert np.array_equal(np.sort(rs), np.arange(T * k))
    pe = ids.reshape(-1)[rs]
    pt = rs // k
    key = pe * T + pt
    assert np.all(np.diff(key) > 0), "rows not ordered by (expert, token)"
    tr = g["token_row"].reshape(-1)
    assert np.array_equal(rs[tr], np.arange(T * k))


def rel_err(got: np.ndarray, ref: np.ndarray):
    diff = got - ref
    rel = np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300)
    rms = np.sqrt(np.mean(ref ** 2))
    return rel, np.abs(diff).max() / max(rms, 1e-300)


def check_outputs(name: str, got: np.ndarray, ref: np.ndarray, allow: Optional[np.ndarray] = None):
    """Relative L2 over everything, and elementwise |got - ref| <=
    MAX_ERR_RMS * rms(ref) + allow, where `allow` (same shape, default 0) is
    the exact effect of the h bytes that differ from the oracle's: a code on
    the other side of a rounding boundary moves the output by that element's
    change times its W_dn column, which for one FP8 step of a large element
    is a sizeable fraction of rms(ref)."""
    rel, mx = rel_err(got, ref)
    if allow is not None:
        rms = max(np.sqrt(np.mean(ref ** 2)), 1e-300)
        mx = float(np.max((np.abs(got - ref) - allow) / rms))
        log(f"{name}: rel_l2={rel:.3e} (max_err - h flip effect)/rms={mx:.3e} "
            f"(largest flip effect {np.max(allow) / rms:.3e} rms)")
    else:
        log(f"{name}: rel_l2={rel:.3e} max_err/rms={mx:.3e}")
    assert rel <= REL_L2, f"{name}: relative L2 error {rel}"
    assert mx <= MAX_ERR_RMS, f"{name}: max error {mx} x rms"
    return rel, mx


def _dn_columns(dn_codes: np.ndarray, dn_scales: np.ndarray, cols: np.ndarray) -> np.ndarray:
    """Decoded columns `cols` of an MXFP4 W_dn [d, d_ff] (canonical layout:
    element 2i in the low nibble of byte i, one scale per 32 along d_ff)."""
    nib = (dn_codes[:, cols // 2] >> (4 * (cols % 2))[None, :]) & 0xF
    return OX.decode_e2m1(nib) * OX.decode_e8m0(dn_scales[:, cols // 32])


def compare_layer(cfg: I.LayerConfig, x_bits: np.ndarray, wr, b, weights, g,
                  tokens: Optional[Sequence[int]] = None):
    """Full comparison of a GPU run `g` (taps) against the oracle."""
    T = x_bits.shape[0]
    t0 = time.time()
    res = OM.forward(x_bits, wr, b, weights, num_experts=cfg.num_experts, top_k=cfg.top_k,
                     num_shared=cfg.num_shared, d_ff=cfg.d_ff, tokens=tokens)
    log(f"oracle forward ({len(res.tokens)} tokens) {time.time() - t0:.1f}s")
    # logits (fp32 accumulation vs fp64)
    lerr = np.abs(g["logits"].astype(np.float64) - res.logits).max()
    log(f"logits max abs err {lerr:.3e}")
    assert lerr < 1e-4
    differ = check_routing(cfg, res, g)
    check_permutation(cfg, res, g, differ)
    same = np.array([t for t in range(T) if t not in differ])
    # w = sigmoid(l)/sum sigmoid(l): d(log w_j)/d l_i = (1 - s_j) delta_ij - w_i (1 - s_i),
    # so a logit error dl moves w_j by at most w_j * 2 * max|dl| (first order),
    # plus fp32 rounding of the sigmoid and the normalisation
    dl = np.abs(g["logits"].astype(np.float64) - res.logits).max(axis=1)[same, None]
    wref = res.topk_w[same]
    werr = np.abs(g["topk_w"][same] - wref)
    bound = wref * (2.0 * dl + 1e-6) + 1e-8
    log(f"topk_w max abs err {werr.max():.3e} (max err/bound {np.max(werr / bound):.2f})")
    assert np.all(werr <= bound)
    # MXFP8 bytes of x: bit-exact
    toks = res.tokens
    assert np.array_equal(g["x_codes"][toks], res.x_codes)
    assert np.array_equal(g["x_scales"][toks], res.x_scales)
    # h bytes of the computed tokens
    ok = np.array([t for t in toks if t not in differ])
    nbytes = nflip = 0
    sflip = 0
    hdiff = []
    pos = {int(t): i for i, t in enumerate(toks)}
    d = res.y.shape[1]
    # exact effect of the differing h bytes on y_routed and y_shared
    allow_r = np.zeros((len(toks), d))
    allow_s = np.zeros((len(toks), d))

    def flip_effect(gh, oh, dn):
        cols = np.nonzero(gh != oh)[0]
        if cols.size == 0:
            return 0.0
        return np.abs(_dn_columns(dn[2], dn[3], cols)) @ np.abs(gh[cols] - oh[cols])

    for t in ok:
        for j in range(cfg.top_k):
            r = int(g["token_row"][t, j])
            rr = int(res.token_row[t, j])
            hc, hs = res.h_rows[rr]
            nbytes += hc.size
            nflip += int(np.sum(g["h_codes"][r] != hc))
            sflip += int(np.sum(g["h_scales"][r] != hs))
            gh = OX.mx_decode(g["h_codes"][r:r + 1], g["h_scales"][r:r + 1], "e4m3")
            oh = OX.mx_decode(hc[None], hs[None], "e4m3")
            hdiff.append((gh, oh))
            if not np.array_equal(gh, oh):
                e = int(res.topk_ids[t, j])
                allow_r[pos[int(t)]] += res.topk_w[t, j] * flip_effect(gh[0], oh[0], weights("routed", e))
        for s in range(cfg.num_shared):
            r = T * cfg.top_k + s * T + int(t)
            hc, hs = res.h_shared[(s, int(t))]
            nbytes += hc.size
            nflip += int(np.sum(g["h_codes"][r] != hc))
            sflip += int(np.sum(g["h_scales"][r] != hs))
            gh = OX.mx_decode(g["h_codes"][r:r + 1], g["h_scales"][r:r + 1], "e4m3")[0]
            oh = OX.mx_decode(hc[None], hs[None], "e4m3")[0]
            if not np.array_equal(gh, oh):
                allow_s[pos[int(t)]] += flip_effect(gh, oh, weights("shared", s))
    rate = nflip / max(nbytes, 1)
    log(f"h codes differing: {nflip}/{nbytes} ({rate:.2e}); scale bytes differing {sflip}")
    assert rate <= 5e-3
    if hdiff:
        a = np.concatenate([u for u, _ in hdiff]); b_ = np.concatenate([v for _, v in hdiff])
        hrel = np.linalg.norm(a - b_) / np.linalg.norm(b_)
        log(f"routed h decoded rel_l2 {hrel:.2e}")
        assert hrel < 1e-2
    # outputs on the tokens routed identically
    sel = [pos[int(t)] for t in ok]
    if sel:
        check_outputs("y_routed", g["y_routed"][ok].astype(np.float64), res.y_routed[sel], allow_r[sel])
        check_outputs("y_shared", g["y_shared"][ok].astype(np.float64), res.y_shared[sel], allow_s[sel])
        y_gpu = bf16_bits_to_f64(g["y"])[ok]
        check_outputs("y", y_gpu, res.y[sel], allow_r[sel] + allow_s[sel])
    return res, differ
