"""Shared helpers for the GPU parity tests: run the HIP layer through the C ABI
with every tap attached, run the oracle on the same seeded inputs, and compare
them with the stated rules.

Bars (from the layer's contract):

* routing ids: bit-exact, except tokens whose oracle gap between the k-th and
  (k+1)-th logit is below TAU, where a different set is accepted if every
  swapped expert's logit lies within TAU of the k-th logit (fp32 accumulation
  over d = 7168 gives ~1e-5 logit error);
* everything after the routing is compared against the oracle re-run with
  the GPU's accepted routing, for every computed token (near-ties included):
  the permutation and the MXFP8 bytes of x bit for bit;
* h: the GPU's fp32 gate/up accumulators must lie within EPS_ACC times the
  sum of the magnitudes of their terms of the oracle's float64 values; every
  GPU h byte must be the MXFP8 quantisation of silu(g)*u rebuilt from those
  same GPU accumulators (a byte may take the neighbouring code only where
  that value sits within H_SLACK of a rounding midpoint or power-of-two block
  boundary: the GPU evaluates silu in fp32); a byte that differs from the
  oracle's must then be one step away on the E4M3 grid with the rounding
  midpoint between the two values (a scale byte one step away with the block
  maxima on either side of the power of two);
* y_routed, y_shared and y, each: relative L2 error <= 5e-3 and, per
  element, |err| <= 5e-2 * rms(reference) + the exact effect of the h bytes
  that differ (their change times their W_dn column, times the routing
  weight for routed rows); and a tighter per-element bound from the
  arithmetic: bf16 rounding of every o row, EPS_MFMA_WIDE times the term
  magnitudes of the down projection, the routing-weight error, plus the h
  effect.
"""

from __future__ import annotations

import os
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
# |gu_gpu - gu_oracle| <= EPS_ACC * sum_i |a_i w_i|.  The scaled MFMA
# accumulates 128 exact products per instruction into an fp32 sum, and
# K/128 <= 56 of those sums add below 56 * 2^-24 = 3.3e-6 of the term
# magnitudes.  Over every GPU parity case the largest ratio seen for the
# gate/up accumulators is 5.4e-6 (K = 256 .. 1024; 6e-7 at K = 7168); the
# bound keeps about 4x of margin over that.
EPS_ACC = 2e-5
# The same for sums whose activation codes span the whole E4M3 range within
# a block (h after SwiGLU, the tail's normalised rows): a probe with operands
# over the whole E4M3 range and scale exponents +-7 found the MFMA result up
# to 1.2e-4 of the term magnitudes from the exact sum (the instruction does
# not keep every product's low bits when their magnitudes differ widely);
# the bound on the down projection's outputs keeps 2x of that.
EPS_MFMA_WIDE = 2.5e-4
# GPU h (silu in fp32 with the hardware exponential) against silu(g)*u in
# float64 from the same fp32 g, u: a few fp32 ulps, times |g| through exp.
H_SLACK = 1e-5
# differing h code bytes (each one verified to be a genuine one-step flip)
FLIP_RATE_CAP = 2e-3
BF16_HALF_ULP = 2.0 ** -8

E4M3_GRID = np.unique(np.abs(OX.decode_e4m3(np.arange(0, 0x7F))))  # 0 .. 448, ascending
E4M3_VALS = OX.decode_e4m3(np.arange(256))


def log(msg: str) -> None:
    print(f"[parity {time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def bf16_bits_to_f64(t) -> np.ndarray:
    if isinstance(t, np.ndarray):
        return OM.bf16_to_f64(t.view(np.uint16))
    return OM.bf16_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))


class Run:
    """Outputs of one GPU forward: taps stay where they are (device tensors,
    or numpy arrays for a stand-in built on the CPU); whole taps come to the
    host on first use, big ones can be fetched row by row."""

    def __init__(self, taps: Dict[str, object], y):
        self.taps = dict(taps)
        self.y = y
        self._host: Dict[str, np.ndarray] = {}

    def __contains__(self, name):
        return name in self.taps

    def __getitem__(self, name):
        if name == "y":
            return self.y
        if name not in self._host:
            t = self.taps[name]
            self._host[name] = t if isinstance(t, np.ndarray) else t.cpu().numpy()
        return self._host[name]

    def rows(self, name, idx) -> np.ndarray:
        idx = np.asarray(idx, dtype=np.int64)
        t = self.taps[name]
        if isinstance(t, np.ndarray):
            out = t[idx]
        elif name in self._host:
            out = self._host[name][idx]
        else:
            out = t.index_select(0, torch.from_numpy(idx).to(t.device)).cpu().numpy()
        return out.view(np.uint16) if name == "h_bf16" else out


def alloc_taps(cfg: I.LayerConfig, T: int, device="cuda", skip=(), a16: bool = False) -> Dict[str, torch.Tensor]:
    E, k, S, d, f = cfg.num_experts, cfg.top_k, cfg.num_shared, cfg.d_model, cfg.d_ff
    R = T * k + S * T
    z = lambda shape, dt: torch.empty(shape, dtype=dt, device=device)
    taps = dict(
        logits=z((T, E), torch.float32), topk_ids=z((T, k), torch.int32),
        topk_w=z((T, k), torch.float32), expert_offsets=z((E + 1,), torch.int32),
        row_src=z((T * k,), torch.int32), token_row=z((T, k), torch.int32),
        gu_acc=z((R, 2 * f), torch.float32), y_routed=z((T, d), torch.float32),
        y_shared=z((T, d), torch.float32))
    if a16:
        taps["h_bf16"] = z((R, f), torch.int16)
    else:
        taps.update(x_codes=z((T, d), torch.uint8), x_scales=z((T, d // 32), torch.uint8),
                    h_codes=z((R, f), torch.uint8), h_scales=z((R, f // 32), torch.uint8))
    return {n: t for n, t in taps.items() if n not in skip}


def run_gpu(cfg: I.LayerConfig, W: DeviceWeights, x: torch.Tensor, taps: bool = True,
            workspace_fill: Optional[int] = None, skip=(), a16: bool = False) -> Run:
    from mxfp4_expert_grouped_amd import mxmoe as M
    T = x.shape[0]
    layer = MoeLayer(cfg.d_model, cfg.d_ff, cfg.num_experts, cfg.top_k, cfg.num_shared,
                     max(T, 1), W, flags=M.MOE_FLAG_A16W4 if a16 else 0)
    tp = alloc_taps(cfg, T, skip=skip, a16=a16) if taps and T > 0 else None
    ws = torch.empty(max(layer.workspace_bytes(T), 256), dtype=torch.uint8, device=x.device)
    if workspace_fill is not None:
        ws.fill_(workspace_fill)
    y = torch.zeros_like(x)
    layer.forward(x, y=y, taps=tp, workspace=ws)
    torch.cuda.synchronize()
    return Run(tp or {}, y)


# ---------------------------------------------------------------------------
# inputs outside the standard recipe
# ---------------------------------------------------------------------------

def pack_device(codes: np.ndarray, scales: np.ndarray, rows: int, k: int, interleave: int):
    """Canonical MXFP4 matrices [n, rows, k/2] / [n, rows, k/32] (numpy) ->
    packed device tensors [n, ...] through moe_pack_mx4."""
    from mxfp4_expert_grouped_amd import mxmoe as M
    n = codes.shape[0]
    sb = M.moe_packed_scale_bytes(rows, k)
    cp = torch.empty((n, rows * k // 2), dtype=torch.uint8, device="cuda")
    sp = torch.empty((n, sb), dtype=torch.uint8, device="cuda")
    tc, ts = torch.from_numpy(np.ascontiguousarray(codes)).cuda(), torch.from_numpy(np.ascontiguousarray(scales)).cuda()
    M.moe_pack_mx4(tc.data_ptr(), ts.data_ptr(), n, rows, k, interleave, cp.data_ptr(), sp.data_ptr(),
                   torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return cp, sp


def weights_with_scale_range(cfg, seed: int, lo: int, hi: int):
    """Expert weights whose E2M1 codes are uniform random bytes and whose E8M0
    scale bytes are uniform in [lo, hi] (a spread the standard recipe never
    produces), as device weights and as the oracle's weight source."""
    from mxfp4_expert_grouped_amd.layer import DeviceWeights
    rng = np.random.default_rng(seed)
    d, f = cfg.d_model, cfg.d_ff

    def mats(n, rows, k):
        return (rng.integers(0, 256, size=(n, rows, k // 2), dtype=np.uint8),
                rng.integers(lo, hi + 1, size=(n, rows, k // 32), dtype=np.uint8))

    E, S = cfg.num_experts, cfg.num_shared
    gu, dn = mats(E, 2 * f, d), mats(E, d, f)
    sgu, sdn = mats(S, 2 * f, d), mats(S, d, f)
    src = lambda kind, i: ((gu[0][i], gu[1][i], dn[0][i], dn[1][i]) if kind == "routed"
                           else (sgu[0][i], sgu[1][i], sdn[0][i], sdn[1][i]))
    g_ = pack_device(*gu, 2 * f, d, 1)
    d_ = pack_device(*dn, d, f, 0)
    sg = pack_device(*sgu, 2 * f, d, 1) if S else (None, None)
    sd = pack_device(*sdn, d, f, 0) if S else (None, None)
    wr = torch.from_numpy(I.gen_router_w(cfg)).cuda()
    return DeviceWeights(g_[0], g_[1], d_[0], d_[1], sg[0], sg[1], sd[0], sd[1], wr, None), src


def integer_x(cfg, seed):
    rng = np.random.default_rng(seed)
    xi = rng.integers(-16, 17, size=(cfg.tokens, cfg.d_model)).astype(np.float32)
    return I.f32_to_bf16_bits(xi)


# ---------------------------------------------------------------------------
# routing
# ---------------------------------------------------------------------------

def check_routing(cfg, logits: np.ndarray, own_ids: np.ndarray, gap: np.ndarray,
                  ids_g: np.ndarray):
    """The GPU's expert sets against the oracle's own selection.  Returns the
    tokens whose sets differ (each one checked to be an accepted near-tie)."""
    T, k = ids_g.shape
    assert np.all(np.diff(ids_g, axis=1) > 0), "GPU ids not strictly ascending"
    assert ids_g.min() >= 0 and ids_g.max() < cfg.num_experts
    differ = np.where(np.any(ids_g != own_ids, axis=1))[0]
    for t in differ:
        assert gap[t] < TAU, f"token {t}: routing differs with gap {gap[t]}"
        lk = np.sort(logits[t])[::-1][k - 1]
        swapped = set(ids_g[t]).symmetric_difference(set(own_ids[t]))
        for e in swapped:
            assert abs(logits[t, e] - lk) < TAU, f"token {t}: expert {e} is not a near-tie"
    log(f"routing: {len(differ)} near-tie tokens of {T} differ (accepted; compared below "
        f"against the oracle with the GPU's routing)")
    return set(int(t) for t in differ)


_POOL = None


def _process_map(workers: int):
    """map() over a pool of fresh CPU-only Python processes (spawned: they
    import numpy and the oracle, never torch or the GPU), one numpy/BLAS
    thread each, started once per test session."""
    global _POOL
    if _POOL is None:
        import multiprocessing as mp
        from concurrent.futures import ProcessPoolExecutor
        env = {"OMP_NUM_THREADS": "1", "OPENBLAS_NUM_THREADS": "1", "MKL_NUM_THREADS": "1",
               "MXMOE_GEN_THREADS": "1"}
        saved = {k: os.environ.get(k) for k in env}
        os.environ.update(env)
        try:
            _POOL = ProcessPoolExecutor(workers, mp_context=mp.get_context("spawn"))
            list(_POOL.map(abs, range(workers)))  # start the workers with this environment
            import atexit
            atexit.register(_POOL.shutdown)
        finally:
            for k, v in saved.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v
    return lambda fn, jobs: _POOL.map(fn, jobs)


def oracle_workers() -> int:
    """CPU processes for the oracle's expert jobs (the machine's CPU share is 16)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_forward(cfg, x_bits, wr, b, weights, tokens, ids, logits, workers: int = 1,
                   activations: str = "mxfp8"):
    """The oracle layer for the given routing.  With workers > 1 its
    per-expert jobs run in that many CPU processes; `weights` must then be
    picklable (an ExpertWeights without cache)."""
    kw = dict(num_experts=cfg.num_experts, top_k=cfg.top_k, num_shared=cfg.num_shared,
              d_ff=cfg.d_ff, topk_ids=ids, intermediates=True, logits=logits, activations=activations)
    if workers > 1:
        kw["expert_map"] = _process_map(workers)
    return OM.forward(x_bits, wr, b, weights, tokens=tokens, **kw)


# ---------------------------------------------------------------------------
# h bytes
# ---------------------------------------------------------------------------

def _grid_index(v: np.ndarray) -> np.ndarray:
    """Position of E4M3 values on the signed value grid (-448 .. 0 .. 448;
    +0 and -0 are one point)."""
    pos = np.searchsorted(E4M3_GRID, np.abs(v))
    assert np.all(E4M3_GRID[pos] == np.abs(v)), "not an E4M3 value"
    return np.where(v < 0, -pos, pos)


def check_quantised(codes: np.ndarray, scales: np.ndarray, h: np.ndarray, slack: float):
    """codes/scales (one row) must be the MXFP8 quantisation of h, except that
    a scale byte may be the other one where the block maximum lies within
    `slack` of the power of two between them, and a code the neighbouring
    one where h / 2^e lies within `slack` of the rounding midpoint."""
    qc, qs = OX.mx_quantize(h[None], "e4m3")
    qc, qs = qc[0], qs[0].astype(np.int64)
    gs = scales.astype(np.int64)
    blocks = h.reshape(-1, 32)
    amax = np.abs(blocks).max(axis=1)
    for blk in np.nonzero(gs != qs)[0]:
        e_hi = max(gs[blk], qs[blk]) - 127
        assert abs(int(gs[blk]) - int(qs[blk])) == 1, f"h scale block {blk}: {gs[blk]} vs {qs[blk]}"
        edge = 2.0 ** (e_hi + 8)
        assert abs(amax[blk] - edge) <= slack * edge, \
            f"h scale block {blk}: amax {amax[blk]!r} is not at the boundary {edge!r}"
    # codes against h at the GPU's own scale
    q = blocks / np.exp2(gs - 127.0)[:, None]
    want = OX.round_to_grid(q, "e4m3").reshape(-1)
    q = q.reshape(-1)
    bad = np.nonzero(codes != want)[0]
    if bad.size:
        vg, vw = E4M3_VALS[codes[bad]], E4M3_VALS[want[bad]]
        step = np.abs(_grid_index(vg) - _grid_index(vw))
        assert np.all((step == 1) | (vg == vw)), f"h codes {bad[step > 1][:4]} are not the quantisation"
        mid = (vg + vw) / 2
        tol = slack * np.maximum(np.abs(q[bad]), np.abs(mid))
        assert np.all(np.abs(q[bad] - mid) <= tol), \
            f"h codes {bad[:4]}: value not at a rounding midpoint ({q[bad][:4]} vs {mid[:4]})"


def compare_h_row(gc, gs, gacc, oc, os_, mid, d_ff: int, stats: dict) -> np.ndarray:
    """One permuted row.  gc/gs: GPU h bytes; gacc: GPU fp32 [g | u]
    accumulators (None when not tapped); oc/os_: oracle bytes; mid: oracle
    intermediates.  Returns dh = decoded GPU h - decoded oracle h, whose
    effect on the outputs the output checks allow."""
    stats["bytes"] = stats.get("bytes", 0) + gc.size
    stats["blocks"] = stats.get("blocks", 0) + gs.size
    h_o = mid["h"]
    q_o = None
    if gacc is not None:
        gacc = gacc.astype(np.float64)
        err = np.abs(gacc - mid["gu"])
        ratio = float(np.max(err / np.maximum(mid["gu_abs"], 1e-300)))
        stats["acc_ratio"] = max(stats.get("acc_ratio", 0.0), ratio)
        assert np.all(err <= EPS_ACC * mid["gu_abs"]), \
            f"gate/up accumulators off by {ratio:.3e} of their term magnitudes"
        h_g = OM.silu(gacc[:d_ff]) * gacc[d_ff:]
        check_quantised(gc, gs, h_g, H_SLACK)
    else:
        h_g = None
    gsi, osi = gs.astype(np.int64), os_.astype(np.int64)
    sdiff = np.nonzero(gsi != osi)[0]
    stats["scale_flips"] = stats.get("scale_flips", 0) + int(sdiff.size)
    for blk in sdiff:
        assert abs(gsi[blk] - osi[blk]) == 1, f"h scale byte {blk}: {gsi[blk]} vs oracle {osi[blk]}"
        if h_g is not None:
            edge = 2.0 ** (max(gsi[blk], osi[blk]) - 127 + 8)
            ao = np.abs(h_o[32 * blk:32 * blk + 32]).max()
            ag = np.abs(h_g[32 * blk:32 * blk + 32]).max()
            lo, hi = min(ao, ag), max(ao, ag)
            assert lo <= edge * (1 + H_SLACK) and hi >= edge * (1 - H_SLACK), \
                f"h scale byte {blk}: block maxima {ao!r}, {ag!r} do not straddle {edge!r}"
    same_scale = np.repeat(gsi == osi, 32)
    cdiff = np.nonzero((gc != oc) & same_scale)[0]
    stats["code_flips"] = stats.get("code_flips", 0) + int(cdiff.size)
    if cdiff.size:
        vg, vo = E4M3_VALS[gc[cdiff]], E4M3_VALS[oc[cdiff]]
        step = np.abs(_grid_index(vg) - _grid_index(vo))
        if h_g is None:
            # nothing to explain a larger move: one step at most
            assert np.all(step <= 1), f"h bytes {cdiff[step > 1][:4]} differ by more than one E4M3 step"
        else:
            # the GPU byte is the quantisation of its own accumulators (checked
            # above) and those are within the bound of the exact sums, so the
            # byte sits across the rounding boundaries between the two values;
            # more than one step happens where an accumulator is much smaller
            # than its terms (cancellation), where the bounded error is a large
            # part of the value -- recorded here
            sc = np.exp2(gsi[cdiff // 32] - 127.0)
            qo, qg = h_o[cdiff] / sc, h_g[cdiff] / sc
            m = (vg + vo) / 2
            sl = H_SLACK * np.maximum(np.abs(qo), np.abs(qg))
            ok = (np.minimum(qo, qg) - sl <= m) & (m <= np.maximum(qo, qg) + sl)
            assert np.all(ok | (vg == vo)), \
                f"h bytes {cdiff[~ok][:4]}: the rounding midpoint is not between the two values"
            multi = cdiff[step > 1]
            stats["multi_step"] = stats.get("multi_step", 0) + int(multi.size)
            for c in multi:
                col = c if c < d_ff else c - d_ff
                cond = max(mid["gu_abs"][col] / max(abs(mid["gu"][col]), 1e-300),
                           mid["gu_abs"][d_ff + col] / max(abs(mid["gu"][d_ff + col]), 1e-300))
                stats["multi_step_min_cond"] = min(stats.get("multi_step_min_cond", np.inf), cond)
    dec = lambda c, s: OX.mx_decode(c[None], s[None], "e4m3")[0]
    return dec(gc, gs) - dec(oc, os_)


def _dn_columns(dn_codes: np.ndarray, dn_scales: np.ndarray, cols: np.ndarray) -> np.ndarray:
    """Decoded columns `cols` of an MXFP4 W_dn [d, d_ff] (canonical layout:
    element 2i in the low nibble of byte i, one scale per 32 along d_ff)."""
    nib = (dn_codes[:, cols // 2] >> (4 * (cols % 2))[None, :]) & 0xF
    return OX.decode_e2m1(nib) * OX.decode_e8m0(dn_scales[:, cols // 32])


def _flip_effect(dh: np.ndarray, weights, kind: str, index: int) -> np.ndarray:
    """|W_dn[:, cols]| @ |dh[cols]| over the columns where dh != 0; only those
    columns' blocks are drawn when the weight source can draw blocks."""
    cols = np.nonzero(dh)[0]
    if cols.size == 0:
        return 0.0
    if hasattr(weights, "dn_blocks"):
        kb = np.unique(cols // 32)
        c, sc = weights.dn_blocks(kind, index, kb)     # [d, n, 16], [d, n]
        pos = np.searchsorted(kb, cols // 32)
        within = cols % 32
        nib = (c[:, pos, within // 2] >> (4 * (within % 2))[None, :]) & 0xF
        w = OX.decode_e2m1(nib) * OX.decode_e8m0(sc[:, pos])
    else:
        dn = weights(kind, index)
        w = _dn_columns(dn[2], dn[3], cols)
    return np.abs(w) @ np.abs(dh[cols])


# ---------------------------------------------------------------------------
# outputs
# ---------------------------------------------------------------------------

def rel_err(got: np.ndarray, ref: np.ndarray):
    diff = got - ref
    rel = np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300)
    rms = np.sqrt(np.mean(ref ** 2))
    return rel, np.abs(diff).max() / max(rms, 1e-300)


def check_outputs(name: str, got: np.ndarray, ref: np.ndarray, allow: Optional[np.ndarray] = None,
                  tight: Optional[np.ndarray] = None):
    """Relative L2 over everything, and elementwise |got - ref| <=
    MAX_ERR_RMS * rms(ref) + allow, where `allow` (same shape, default 0) is
    the exact effect of the h bytes that differ from the oracle's: a code on
    the other side of a rounding boundary moves the output by that element's
    change times its W_dn column, which for one FP8 step of a large element
    is a sizeable fraction of rms(ref).  With `tight` (a per-element bound
    from the arithmetic, h effect included) also |got - ref| <= tight."""
    rel, mx = rel_err(got, ref)
    rms = max(np.sqrt(np.mean(ref ** 2)), 1e-300)
    if allow is not None:
        mx = float(np.max((np.abs(got - ref) - allow) / rms))
        log(f"{name}: rel_l2={rel:.3e} (max_err - h flip effect)/rms={mx:.3e} "
            f"(largest flip effect {np.max(allow) / rms:.3e} rms)")
    else:
        log(f"{name}: rel_l2={rel:.3e} max_err/rms={mx:.3e}")
    assert rel <= REL_L2, f"{name}: relative L2 error {rel}"
    assert mx <= MAX_ERR_RMS, f"{name}: max error {mx} x rms"
    if tight is not None:
        r = float(np.max(np.abs(got - ref) / np.maximum(tight, 1e-300)))
        log(f"{name}: max |err| / arithmetic bound = {r:.3f}")
        assert np.all(np.abs(got - ref) <= tight), f"{name}: error above the arithmetic bound ({r:.3f}x)"
    return rel, mx


def compare_h_row_bf16(gb, gacc, ob, mid, d_ff: int, stats: dict) -> np.ndarray:
    """One permuted row of the A16W4 variant, whose h is bf16: gb / ob the
    GPU's and the oracle's h bits.  The GPU bits must be the bf16 rounding of
    silu(g)*u rebuilt from the GPU's own accumulators (the neighbouring bf16
    value only within H_SLACK of the rounding midpoint), those accumulators
    within EPS_ACC of the oracle's term magnitudes.  Returns dh (decoded GPU h
    minus decoded oracle h)."""
    stats["bytes"] = stats.get("bytes", 0) + gb.size
    vg, vo = OM.bf16_to_f64(gb), OM.bf16_to_f64(ob)
    if gacc is not None:
        gacc = gacc.astype(np.float64)
        err = np.abs(gacc - mid["gu"])
        ratio = float(np.max(err / np.maximum(mid["gu_abs"], 1e-300)))
        stats["acc_ratio"] = max(stats.get("acc_ratio", 0.0), ratio)
        assert np.all(err <= EPS_ACC * mid["gu_abs"]), \
            f"gate/up accumulators off by {ratio:.3e} of their term magnitudes"
        # the rounding decision in the kernel's precision: silu(g) * u from the
        # GPU's fp32 sums evaluated in fp32 as the kernel does (an fp32
        # exp(-g) overflows for g < -88.7, giving -0 where float64 still has a
        # value near 1e-38; last-ulp differences of exp stay within H_SLACK)
        g32, u32 = gacc[:d_ff].astype(np.float32), gacc[d_ff:].astype(np.float32)
        with np.errstate(over="ignore"):
            h_g = ((g32 / (np.float32(1) + np.exp(-g32))) * u32).astype(np.float64)
        want = OM.f64_to_bf16(h_g)
        bad = np.nonzero(gb != want)[0]
        if bad.size:
            vw = OM.bf16_to_f64(want[bad])
            m = (vg[bad] + vw) / 2
            # neighbours: no bf16 value strictly between them (their bit
            # patterns differ by one in the same sign, or both are zeros)
            adj = (np.abs(gb[bad].astype(np.int64) - want[bad].astype(np.int64)) == 1) | (vg[bad] == vw)
            assert np.all(adj), f"h bits {bad[~adj][:4]} are not the bf16 rounding of the GPU's sums"
            assert np.all(np.abs(h_g[bad] - m) <= H_SLACK * np.abs(h_g[bad])), \
                f"h bits {bad[:4]}: value not at a bf16 rounding midpoint"
    else:
        d = np.abs(gb.astype(np.int64) - ob.astype(np.int64))
        assert np.all((d <= 1) | (vg == vo)), "h bits differ by more than one bf16 step"
    stats["code_flips"] = stats.get("code_flips", 0) + int(np.sum(gb != ob))
    return vg - vo


def compare_layer(cfg: I.LayerConfig, x_bits: np.ndarray, wr, b, weights, g: Run,
                  tokens: Optional[Sequence[int]] = None, workers: int = 1,
                  activations: str = "mxfp8"):
    """Full comparison of a GPU run `g` (taps) against the oracle.
    activations="bf16": the A16W4 variant (bf16 x and h; h through the
    h_bf16 tap)."""
    a16 = activations == "bf16"
    T = x_bits.shape[0]
    k, S, f = cfg.top_k, cfg.num_shared, cfg.d_ff
    t0 = time.time()
    logits = OM.router_logits(x_bits, wr, b)
    own_ids, gap = OM.topk_select(logits, k)
    lerr = np.abs(g["logits"].astype(np.float64) - logits).max()
    log(f"logits max abs err {lerr:.3e} ({time.time() - t0:.1f}s)")
    assert lerr < 1e-4
    ids_g = g["topk_ids"].astype(np.int32)
    differ = check_routing(cfg, logits, own_ids, gap, ids_g)
    # the oracle layer for the GPU's (accepted) routing
    t0 = time.time()
    res = oracle_forward(cfg, x_bits, wr, b, weights, tokens, ids_g, logits, workers, activations)
    log(f"oracle forward with the GPU routing ({len(res.tokens)} tokens, "
        f"{sum(1 for t in res.tokens if int(t) in differ)} of them near-ties) {time.time() - t0:.1f}s")
    assert len(res.tokens) >= 1
    # permutation of that routing: bit-exact
    assert np.array_equal(g["expert_offsets"], res.offsets)
    assert np.array_equal(g["row_src"], res.row_src)
    assert np.array_equal(g["token_row"], res.token_row)
    # routing weights: w = sigmoid(l)/sum sigmoid(l), d(log w_j)/d l_i =
    # (1 - s_j) delta_ij - w_i (1 - s_i), so a logit error dl moves w_j by at
    # most w_j * 2 * max|dl| (first order), plus fp32 rounding of the sigmoid
    # and the normalisation
    dl = np.abs(g["logits"].astype(np.float64) - logits).max(axis=1)[:, None]
    wref = res.topk_w
    wg = g["topk_w"].astype(np.float64)
    werr = np.abs(wg - wref)
    bound = wref * (2.0 * dl + 1e-6) + 1e-8
    log(f"topk_w max abs err {werr.max():.3e} (max err/bound {np.max(werr / bound):.2f})")
    assert np.all(werr <= bound)
    # MXFP8 bytes of x: bit-exact
    toks = res.tokens
    if a16:
        assert "x_codes" not in g and "h_codes" not in g
    else:
        assert np.array_equal(g.rows("x_codes", toks), res.x_codes)
        assert np.array_equal(g.rows("x_scales", toks), res.x_scales)
    # h rows of the computed tokens, in one gather per tap
    nt, d = len(toks), res.y.shape[1]
    rows_r = np.array([int(res.token_row[t, j]) for t in toks for j in range(k)], np.int64)
    rows_s = np.array([T * k + s * T + int(t) for t in toks for s in range(S)], np.int64)
    rows = np.concatenate([rows_r, rows_s]).astype(np.int64)
    if a16:
        hc, hs = g.rows("h_bf16", rows), None
    else:
        hc, hs = g.rows("h_codes", rows), g.rows("h_scales", rows)

    def h_row(q, oc, os_, mid):
        if a16:
            dh = compare_h_row_bf16(hc[q], None if acc is None else acc[q], oc, mid, f, stats)
            return dh, OM.bf16_to_f64(oc)
        dh = compare_h_row(hc[q], hs[q], None if acc is None else acc[q], oc, os_, mid, f, stats)
        return dh, OX.mx_decode(oc[None], os_[None], "e4m3")[0]

    acc = g.rows("gu_acc", rows) if "gu_acc" in g else None
    stats: dict = {}
    allow_r, allow_s = np.zeros((nt, d)), np.zeros((nt, d))
    tight_r, tight_s = np.zeros((nt, d)), np.zeros((nt, d))
    dn_abs_r, dn_abs_s = np.zeros((nt, d)), np.zeros((nt, d))
    hdiff = []
    for i, t in enumerate(toks):
        t = int(t)
        for j in range(k):
            q = i * k + j
            r = int(rows_r[q])
            oc, os_ = res.h_rows[r]
            mid = res.mid_rows[r]
            dh, hov = h_row(q, oc, os_, mid)
            hdiff.append((dh, hov))
            e = int(ids_g[t, j])
            w = max(float(wref[t, j]), float(wg[t, j]))
            eff = _flip_effect(dh, weights, "routed", e)
            allow_r[i] += w * eff
            o = mid["o"]
            tight_r[i] += (w * (BF16_HALF_ULP * (np.abs(o) + eff) + EPS_MFMA_WIDE * mid["o_abs"] + eff)
                           + werr[t, j] * np.abs(o) + 2.0 ** -20 * w * np.abs(o))
            dn_abs_r[i] += w * mid["o_abs"]
        for s in range(S):
            q = len(rows_r) + i * S + s
            oc, os_ = res.h_shared[(s, t)]
            mid = res.mid_shared[(s, t)]
            dh, _ = h_row(q, oc, os_, mid)
            eff = _flip_effect(dh, weights, "shared", s)
            allow_s[i] += eff
            o = mid["o"]
            tight_s[i] += (BF16_HALF_ULP * (np.abs(o) + eff) + EPS_MFMA_WIDE * mid["o_abs"] + eff
                           + 2.0 ** -20 * np.abs(o))
            dn_abs_s[i] += mid["o_abs"]
    rate = stats.get("code_flips", 0) / max(stats.get("bytes", 1), 1)
    log(f"h: {stats.get('code_flips', 0)}/{stats.get('bytes', 0)} code bytes differ ({rate:.2e}), "
        f"{stats.get('scale_flips', 0)}/{stats.get('blocks', 0)} scale bytes, every one across a "
        f"rounding boundary ({stats.get('multi_step', 0)} by more than one step, all at "
        f"accumulators >= {stats.get('multi_step_min_cond', float('nan')):.3g} times smaller than "
        f"their term magnitudes); accumulators within {stats.get('acc_ratio', float('nan')):.2e} of "
        f"their term magnitudes (bound {EPS_ACC:g})")
    assert stats.get("code_flips", 0) <= max(4, FLIP_RATE_CAP * stats.get("bytes", 0))
    if hdiff:
        a = np.concatenate([u for u, _ in hdiff])
        b_ = np.concatenate([v for _, v in hdiff])
        hrel = np.linalg.norm(a) / max(np.linalg.norm(b_), 1e-300)
        log(f"routed h decoded rel_l2 {hrel:.2e}")
        assert hrel < 1e-2
    # outputs of every computed token (near-ties included)
    yr = g.rows("y_routed", toks).astype(np.float64)
    ys = g.rows("y_shared", toks).astype(np.float64)
    # what the arithmetic bound leaves to the down projection's accumulation,
    # as a fraction of its term magnitudes (recorded: EPS_MFMA_WIDE bounds it)
    for name, got, ref, tb, ab in (("y_routed", yr, res.y_routed, tight_r, dn_abs_r),
                                   ("y_shared", ys, res.y_shared, tight_s, dn_abs_s)):
        if np.any(ab > 0):
            rest = np.abs(got - ref) - (tb - EPS_MFMA_WIDE * ab)
            log(f"{name}: down-projection accumulation error <= "
                f"{np.max(np.maximum(rest, 0) / np.maximum(ab, 1e-300)):.2e} of its term magnitudes")
    check_outputs("y_routed", yr, res.y_routed, allow_r, tight_r)
    if S:
        check_outputs("y_shared", ys, res.y_shared, allow_s, tight_s)
    else:
        assert np.all(ys == 0)
    y_gpu = bf16_bits_to_f64(g["y"])[toks]
    tight_y = ((tight_r + tight_s) * (1 + 2.0 ** -7) + BF16_HALF_ULP * np.abs(res.y)
               + 2.0 ** -20 * (np.abs(res.y_routed) + np.abs(res.y_shared)))
    check_outputs("y", y_gpu, res.y, allow_r + allow_s, tight_y)
    return res, differ


# ---------------------------------------------------------------------------
# LatentMoE tail
# ---------------------------------------------------------------------------

def compare_tail(z, s, gamma, eps, up_c, up_s, y_gpu, inv_g, codes_g, scales_g,
                 rows: Optional[Sequence[int]] = None):
    """The tail y = MXFP8(RMSNorm(z)) W_up^T + s on the GPU against the oracle,
    on `rows` (all when None).  inv_g, codes_g, scales_g: the GPU's taps
    (fp32 1/rms per row, MXFP8 bytes of the normalised rows), y_gpu bf16 bits.

    * 1/rms: within the rounding of an fp32 sum of squares of `latent` terms
      (a serial part of latent/256 terms per thread plus a tree) and of the
      square root and division, relative;
    * the MXFP8 bytes must be the quantisation of z * inv_g * gamma rebuilt in
      float64 from the GPU's own 1/rms (a neighbouring code only within
      H_SLACK of a rounding midpoint: the GPU multiplies in fp32); where they
      differ from the oracle's, the difference comes from the bounded 1/rms
      difference, and its exact effect on y is allowed;
    * y: relative L2 <= 5e-3 and |err| <= 5e-2 rms + that effect (the
      contract), and per element the arithmetic bound: EPS_MFMA_WIDE times the term
      magnitudes, bf16 rounding of the projection (when s is added after it)
      and of y, plus the effect of the differing bytes."""
    T, l = z.shape
    rows = np.arange(T) if rows is None else np.asarray(sorted(set(int(r) for r in rows)))
    zr = z[rows].astype(np.float64)
    sr = None if s is None else s[rows].astype(np.float64)
    mid = {}
    y_o = OM.latent_tail(zr, gamma, eps, up_c, up_s, sr, intermediates=mid)
    inv_o = 1.0 / np.sqrt(np.mean(zr * zr, axis=1) + eps)
    ig = inv_g[rows].astype(np.float64)
    rel = np.abs(ig - inv_o) / inv_o
    inv_bound = (l / 256 + 16) * 2.0 ** -24
    log(f"tail: 1/rms max rel err {rel.max():.2e} (bound {inv_bound:.2e})")
    assert np.all(rel <= inv_bound)
    w = OX.mx_decode(up_c, up_s, "e2m1")
    stats: dict = {}
    allow = np.zeros_like(y_o)
    for i, r in enumerate(rows):
        n_g = zr[i] * ig[i] * gamma.astype(np.float64)
        check_quantised(codes_g[r], scales_g[r], n_g, H_SLACK)
        gc, gs = codes_g[r], scales_g[r]
        oc, os_ = mid["a_codes"][i], mid["a_scales"][i]
        stats["bytes"] = stats.get("bytes", 0) + gc.size
        stats["flips"] = stats.get("flips", 0) + int(np.sum(gc != oc))
        stats["scale_flips"] = stats.get("scale_flips", 0) + int(np.sum(gs != os_))
        da = OX.mx_decode(gc[None], gs[None], "e4m3")[0] - OX.mx_decode(oc[None], os_[None], "e4m3")[0]
        nz = np.nonzero(da)[0]
        if nz.size:
            allow[i] = np.abs(w[:, nz]) @ np.abs(da[nz])
    log(f"tail: {stats['flips']}/{stats['bytes']} MXFP8 codes and {stats['scale_flips']} scale bytes "
        f"differ from the oracle's (each the quantisation of the GPU's own 1/rms)")
    assert stats["flips"] <= max(4, FLIP_RATE_CAP * stats["bytes"])
    y_g = bf16_bits_to_f64(y_gpu)[rows]
    proj = y_o if sr is None else y_o - sr
    rest = np.abs(bf16_bits_to_f64(y_gpu)[rows] - y_o) - (allow + BF16_HALF_ULP * (np.abs(y_o) + allow)
                                                          + (0.0 if sr is None else BF16_HALF_ULP * (np.abs(y_o - sr) + allow)))
    log(f"tail: projection accumulation error <= "
        f"{np.max(np.maximum(rest, 0) / np.maximum(mid['y_abs'], 1e-300)):.2e} of its term magnitudes")
    tight = (EPS_MFMA_WIDE * mid["y_abs"] + allow + BF16_HALF_ULP * (np.abs(y_o) + allow)
             + (0.0 if sr is None else BF16_HALF_ULP * (np.abs(proj) + allow)) + 2.0 ** -20 * np.abs(y_o))
    check_outputs("tail y", y_g, y_o, allow, tight)
    return y_o
