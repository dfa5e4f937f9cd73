#!/usr/bin/env python3
"""Benchmark of the MXFP4/MXFP8 sparse MoE layer on one MI355X.

One step = one whole forward of the layer (router, top-k, MXFP8 quantisation,
permutation, gate_up + SwiGLU + re-quantisation, down, combine) over one batch
of synthetic tokens, inputs already resident in HBM.

Default workload: the largest one, prefill of 32768 tokens with the Zipf-skewed
router bias (d=7168, 896 experts, top-16, d_ff=2048, 2 shared).  `--config`
selects the others (tiny, decode1, decode256, prefill8k).  Decode steps use
different token batches and rotate over several independently generated
copies of the layer's weights, so no step finds its experts in the 256 MB
last-level cache (as in a real decode step, where the other layers' weights
pass through in between).

Prints ONE JSON line.  Also reports the dominant kernel's achieved bandwidth
(or MFMA rate) against the MI355X peak, timed with HIP events inside the timed
region, and the CPU oracle's throughput on a bounded sample.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "MoE-layer tokens/s + HBM GB/s (decode) / MXFP4 TFLOPS (prefill) vs peak"
HBM_PEAK_GBS = 8000.0
FP8_MFMA_PEAK_TFLOPS = 5000.0   # dense FP8 (the rate of FP8 x FP4 operand pairs)
FP4_MFMA_PEAK_TFLOPS = 10100.0  # dense MXFP4 x MXFP4
BF16_MFMA_PEAK_TFLOPS = 2500.0  # dense bf16 (the A16W4 prefill kernel's MFMA)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--config", default="prefill32k_skew",
                    choices=["tiny", "decode1", "decode256", "prefill8k", "prefill32k_skew"])
    ap.add_argument("--layers", type=int, default=None,
                    help="independent weight copies rotated per step")
    ap.add_argument("--batches", type=int, default=None, help="distinct token batches per layer")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true", help="replay the forward as a HIP graph")
    ap.add_argument("--breakdown", action="store_true", help="also time every stage (untimed pass)")
    ap.add_argument("--canonical", action="store_true",
                    help="expert weights in the canonical layout instead of the packed one")
    ap.add_argument("--a16w4", action="store_true",
                    help="the A16W4 variant (bf16 activations, MXFP4 weights)")
    ap.add_argument("--tail", action="store_true",
                    help="also time the LatentMoE tail (moe_latent_tail) on the same token count, "
                         "latent = hidden = d_model, and report it as 'latent_tail'")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after timing, copy this many MiB device-to-device once (a plain copy "
                         "kernel of known size, to calibrate hardware byte counters)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the layer fits one "
                                   "MI355X and nothing here shards it; --gpus must be 1"}))
        sys.exit(2)

    import torch
    from mxfp4_expert_grouped_amd import inputs as I
    from mxfp4_expert_grouped_amd import inputs_gpu as IG
    from mxfp4_expert_grouped_amd import mxmoe as M
    from mxfp4_expert_grouped_amd.layer import MoeLayer

    M.load_library()
    torch.cuda.set_device(0)
    cfg = I.CONFIGS[args.config]
    decode = cfg.tokens <= 256
    flags = M.MOE_FLAG_A16W4 if args.a16w4 else 0
    steps = args.steps or (200 if decode else 10)
    warmup = args.warmup if args.warmup is not None else (20 if decode else 2)
    nlayers = args.layers or (4 if decode else 1)
    nbatch = args.batches or (8 if cfg.tokens <= 256 else 1)
    T = cfg.tokens

    # ---- inputs resident in HBM ------------------------------------------------
    t0 = time.time()
    layers, xs = [], []
    for li in range(nlayers):
        W = (IG.device_weights_canonical if args.canonical else IG.device_weights)(cfg, layer=li)
        layers.append(MoeLayer(cfg.d_model, cfg.d_ff, cfg.num_experts, cfg.top_k, cfg.num_shared, T, W,
                               flags=flags))
        xs.append([IG.device_x(cfg, layer=1000 * li + bi) for bi in range(nbatch)])
    ws = torch.empty(layers[0].workspace_bytes(T), dtype=torch.uint8, device="cuda")
    ys = torch.empty((T, cfg.d_model), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    # realised routing of every (layer, batch): touched experts -> algorithmic bytes
    gu_bytes = I.matrix_bytes(2 * cfg.d_ff, cfg.d_model)
    dn_bytes = I.matrix_bytes(cfg.d_model, cfg.d_ff)
    touched = {}
    offs = torch.empty(cfg.num_experts + 1, dtype=torch.int32, device="cuda")
    for li, L in enumerate(layers):
        for bi, x in enumerate(xs[li]):
            L.forward(x, y=ys, taps={"expert_offsets": offs}, workspace=ws)
            counts = np.diff(offs.cpu().numpy())
            touched[(li, bi)] = (int((counts > 0).sum()), counts)
    R = T * cfg.top_k + cfg.num_shared * T
    if args.a16w4:
        act_in = T * cfg.d_model * 2                            # bf16 x rows
        h_bytes = R * cfg.d_ff * 2                              # bf16 h rows
    else:
        act_in = T * (cfg.d_model + cfg.d_model // 32)          # MXFP8 x rows
        h_bytes = R * (cfg.d_ff + cfg.d_ff // 32)               # MXFP8 h rows
    router_bytes = cfg.num_experts * cfg.d_model * 4
    xy_bytes = 2 * T * cfg.d_model * 2

    def step_bytes(key):
        n = touched[key][0] + cfg.num_shared
        return n * (gu_bytes + dn_bytes) + router_bytes + xy_bytes

    # For a few tokens the library runs the shared experts' gate_up inside the
    # routing launch (next to the top-k), so the gate_up launch then streams
    # the routed experts alone (the library's rule: T <= 32 with the one-pass
    # router, 8-row tiles, shared experts present).
    phase_split = decode and T <= 32 and T * (cfg.d_model // 32) <= 32 * cfg.num_experts and cfg.num_shared > 0

    def gate_up_bytes(key):
        if phase_split:
            return touched[key][0] * gu_bytes + act_in + h_bytes * cfg.top_k // (cfg.top_k + cfg.num_shared)
        n = touched[key][0] + cfg.num_shared
        return n * gu_bytes + act_in + h_bytes

    sched = [(s % nlayers, (s // nlayers) % nbatch) for s in range(steps)]

    def run(s):
        li, bi = sched[s % len(sched)] if s >= 0 else (0, 0)
        layers[li].forward(xs[li][bi], y=ys, workspace=ws)

    graphs = None
    if args.graph:
        graphs = {}
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            for key in set(sched):
                layers[key[0]].forward(xs[key[0]][key[1]], y=ys, workspace=ws)
        torch.cuda.current_stream().wait_stream(st)
        for key in set(sched):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                layers[key[0]].forward(xs[key[0]][key[1]], y=ys, workspace=ws)
            graphs[key] = g

        def run(s):  # noqa: F811
            graphs[sched[s % len(sched)]].replay()

    # ---- warmup, then the timed region (no per-stage events inside it: a timed
    # HIP event between two kernels costs several microseconds of idle GPU) ---------
    for s in range(warmup):
        run(s)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record()
    for s in range(steps):
        run(s)
    ev1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - w0) * 1e3
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = wall_ms / steps

    # ---- the same steps again, one event pair per step (torch's current stream,
    # where every launch of the forward goes): per-step median and spread.  A
    # separate pass, because an event between two steps idles the GPU for a few
    # microseconds, which the timed region above must not include -------------------
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
    for s in range(steps):
        step_ev[s][0].record()
        run(s)
        step_ev[s][1].record()
    torch.cuda.synchronize()
    per_step = np.array([a.elapsed_time(b) for a, b in step_ev])
    p10, p50, p90 = (float(np.percentile(per_step, q)) for q in (10, 50, 90))

    # ---- the same steps again with HIP events around the gate_up launch (on the
    # stream it runs on) for the dominant kernel's average duration ------------------
    gu_ms = None
    if not args.graph:
        for L in layers:
            M.moe_profile_begin(L.plan, ["gate_up"], steps)
        for s in range(steps):
            run(s)
        torch.cuda.synchronize()
        tot, calls = 0.0, 0
        for L in layers:
            stage_ms, n = M.moe_profile_end(L.plan)
            tot += stage_ms["gate_up"]
            calls += n
        gu_ms = tot / max(calls, 1)

    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    stage_avg = None
    if args.breakdown:
        for L in layers:
            M.moe_profile_begin(L.plan, list(M.STAGES), max(1, steps // nlayers + 1))
        for s in range(min(steps, 8 * nlayers)):
            run(s)
        torch.cuda.synchronize()
        acc = {k: 0.0 for k in M.STAGES}
        calls = 0
        for L in layers:
            sm, n = M.moe_profile_end(L.plan)
            calls += n
            for k in acc:
                acc[k] += sm[k]
        stage_avg = {k: round(v / max(calls, 1), 5) for k, v in acc.items()}

    # ---- derived figures ------------------------------------------------------------------
    # counter traffic is kept per kernel variant: activation type and weight layout
    traffic_key = cfg.name + ("_a16w4" if args.a16w4 else "") + ("_canonical" if args.canonical else "")
    mean_step_bytes = float(np.mean([step_bytes(k) for k in sched]))
    mean_gu_bytes = float(np.mean([gate_up_bytes(k) for k in sched]))
    flops = 2.0 * R * 3 * cfg.d_model * cfg.d_ff
    tokens_per_s = T / (ms_per_step / 1e3)
    layer_gbs = mean_step_bytes / (ms_per_step / 1e3) / 1e9
    layer_tflops = flops / (ms_per_step / 1e3) / 1e12
    if decode:
        kern_ms = gu_ms if gu_ms else ms_per_step
        achieved = mean_gu_bytes / (kern_ms / 1e3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": profiled_traffic(traffic_key),
                    "kernel": ("gate_up grouped GEMM, routed experts (k_gemm_stream, 8-row tiles; the shared "
                               "experts' gate_up runs in the routing launch)" if phase_split
                               else "gate_up grouped GEMM (k_gemm_stream, 8-row tiles)"),
                    "kernel_ms": round(kern_ms, 5),
                    "algorithmic_bytes_per_launch": int(mean_gu_bytes)}
    elif args.a16w4:
        # bf16 activations: the weights are expanded to bf16 in registers and
        # the contraction runs on the bf16 MFMA, whose dense rate is its peak
        kern_ms = gu_ms if gu_ms else ms_per_step
        gu_flops = 2.0 * R * cfg.d_model * 2 * cfg.d_ff
        achieved = gu_flops / (kern_ms / 1e3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_MFMA_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / BF16_MFMA_PEAK_TFLOPS, 4),
                    "traffic": profiled_traffic(traffic_key),
                    "kernel": "gate_up grouped GEMM (k_gemm_pf16, 256-row tiles, bf16 MFMA)",
                    "kernel_ms": round(kern_ms, 5), "algorithmic_flops_per_launch": gu_flops}
    else:
        kern_ms = gu_ms if gu_ms else ms_per_step
        gu_flops = 2.0 * R * cfg.d_model * 2 * cfg.d_ff
        achieved = gu_flops / (kern_ms / 1e3) / 1e12
        # MXFP8 x MXFP4 operands issue at the dense FP8 rate on gfx950, so that
        # is the contraction's own peak; the fraction of the dense MXFP4 peak
        # (the rate FP4 x FP4 operands would reach) is reported beside it
        roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": FP8_MFMA_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / FP8_MFMA_PEAK_TFLOPS, 4),
                    "peak_mxfp4": FP4_MFMA_PEAK_TFLOPS,
                    "frac_of_mxfp4_peak": round(achieved / FP4_MFMA_PEAK_TFLOPS, 4),
                    "traffic": profiled_traffic(traffic_key),
                    "kernel": "gate_up grouped GEMM (k_gemm_pf, 256-row tiles)",
                    "kernel_ms": round(kern_ms, 5), "algorithmic_flops_per_launch": gu_flops}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, a16w4=args.a16w4)

    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16 x mxfp4 (A16W4), fp32 accumulate" if args.a16w4
                  else "mxfp8 x mxfp4, fp32 accumulate"),
        "data": "synthetic (seeded; random-init MXFP4 weights)",
        "config": {"workload": f"{cfg.name}: T={T}, d_model={cfg.d_model}, experts={cfg.num_experts}, "
                               f"top_k={cfg.top_k}, d_ff={cfg.d_ff}, shared={cfg.num_shared}"
                               + (", Zipf(1.1) router bias" if cfg.zipf_bias else ""),
                   "tokens_per_step": T, "weight_copies_rotated": nlayers,
                   "token_batches": nbatch, "hip_graph": bool(args.graph),
                   "variant": "A16W4" if args.a16w4 else "A8W4",
                   "weights": "canonical" if args.canonical else "packed"},
        "layer_hbm_gbps": round(layer_gbs, 1),
        "layer_hbm_frac": round(layer_gbs / HBM_PEAK_GBS, 4),
        "layer_tflops": round(layer_tflops, 2),
        "algorithmic_bytes_per_step": int(mean_step_bytes),
        "gpu_event_ms_per_step": round(gpu_ms / steps, 5),
        "step_ms_p10": round(p10, 5), "step_ms_p50": round(p50, 5), "step_ms_p90": round(p90, 5),
        "layer_tflops_p50": round(flops / (p50 / 1e3) / 1e12, 2),
        "layer_frac_of_fp8_rate": round(layer_tflops / FP8_MFMA_PEAK_TFLOPS, 4),
        "layer_frac_of_mxfp4_peak": round(layer_tflops / FP4_MFMA_PEAK_TFLOPS, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "setup_s": round(setup_s, 1),
    }
    if stage_avg:
        out["stage_ms"] = stage_avg
    if args.tail:
        out["latent_tail"] = bench_tail(cfg, steps, warmup)
    print(json.dumps(out), flush=True)


def bench_tail(cfg, steps: int, warmup: int):
    """The LatentMoE tail y = MXFP8(RMSNorm(z)) W_up^T + s on the workload's
    token count at latent = hidden = d_model, inputs resident in HBM; HIP
    events around the timed calls on torch's current stream (the stream every
    launch of the call goes to)."""
    import torch
    from mxfp4_expert_grouped_amd import inputs as I
    from mxfp4_expert_grouped_amd import mxmoe as M
    T, l = cfg.tokens, cfg.d_model
    H = l
    z, s, gamma = I.gen_tail_inputs(T, l, H, seed=1)
    up_c, up_s = I.gen_up_matrix(H, l, seed=1)
    tc, ts = torch.from_numpy(up_c).cuda(), torch.from_numpy(up_s).cuda()
    cp = torch.empty(H * l // 2, dtype=torch.uint8, device="cuda")
    sp = torch.empty(M.moe_packed_scale_bytes(H, l), dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    M.moe_pack_mx4(tc.data_ptr(), ts.data_ptr(), 1, H, l, 0, cp.data_ptr(), sp.data_ptr(), st)
    zt, stt, gt = (torch.from_numpy(a).cuda() for a in (z, s, gamma))
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    nb = M.moe_latent_tail_workspace_bytes(T, l, H)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda")
    W = M.MoeTailWeights(cp.data_ptr(), sp.data_ptr(), gt.data_ptr(), M.MOE_WEIGHTS_PACKED)

    def call():
        M.moe_latent_tail(T, l, H, 1e-6, W, zt.data_ptr(), stt.data_ptr(), y.data_ptr(), ws.data_ptr(),
                          nb, None, st)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = T * l * 4 + T * H * 4 + T * H * 2 + H * l // 2 + H * l // 32 + l * 4
    flops = 2.0 * T * l * H
    t_hbm, t_mfma = nbytes / (HBM_PEAK_GBS * 1e9), flops / (FP8_MFMA_PEAK_TFLOPS * 1e12)
    bound = "hbm" if t_hbm >= t_mfma else "mfma"
    achieved = nbytes / (ms / 1e3) / 1e9 if bound == "hbm" else flops / (ms / 1e3) / 1e12
    peak = HBM_PEAK_GBS if bound == "hbm" else FP8_MFMA_PEAK_TFLOPS
    return {"tokens": T, "latent": l, "hidden": H, "ms_per_call": round(ms, 5),
            "tokens_per_s": round(T / (ms / 1e3), 1), "algorithmic_bytes": int(nbytes),
            "algorithmic_flops": flops,
            "roofline": {"bound": bound, "achieved": round(achieved, 1), "peak": peak,
                         "unit": "GB/s" if bound == "hbm" else "TFLOP/s",
                         "frac": round(achieved / peak, 4),
                         "frac_of_bound_time": round(max(t_hbm, t_mfma) * 1e3 / ms, 4)}}


def profiled_traffic(workload: str):
    """HBM bytes per launch of the dominant kernel from the committed hardware-
    counter summary, if one exists for this workload and kernel variant (e.g.
    "decode256_a16w4") and the kernel sources are unchanged since it was taken
    (else None)."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, "profiles", f"gate_up_{workload}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in ("kernels_gemm.hip", "mx_device.h", "internal.h", "topk_device.h"):
        h.update(open(os.path.join(root, "mxfp4_expert_grouped_amd", "csrc", f), "rb").read())
    if fields.get("source_sha256") != h.hexdigest():
        return None
    return int(fields["traffic_bytes_per_launch"])


def cpu_baseline(cfg, a16w4: bool = False):
    """The oracle, untuned, on the host cores for a bounded sample of the
    workload: the whole step at the tiny and decode1 workloads, else the first
    tokens of the batch (rows are independent).  The decode of the touched
    experts' MXFP4 weights to float64 is also timed alone (the oracle's own
    decode routine on the same matrices), so the record splits the step into
    weight decode and the rest (fp64 GEMMs, routing, quantisation)."""
    from mxfp4_expert_grouped_amd import inputs as I
    from oracle import moe as OM
    from oracle import mx as OX
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    wr, b = I.gen_router_w(cfg, 0), I.gen_router_b(cfg)
    W = I.ExpertWeights(cfg)
    if cfg.tokens <= 16:
        ntok = cfg.tokens if cfg.tokens <= 8 else 1
    else:
        # about 10 s of oracle work: the first tokens until they touch 80
        # experts (at most 32; about 0.12 s of float64 work per expert)
        x32 = I.gen_x(cfg, layer=0)[:32]
        ids32 = OM.topk_select(OM.router_logits(x32, wr, b), cfg.top_k)[0]
        ntok, seen = len(ids32), set()
        for t in range(len(ids32)):
            seen.update(ids32[t].tolist())
            if len(seen) >= 80:
                ntok = t + 1
                break
    x = I.gen_x(cfg, layer=0)[:ntok]
    ids = OM.topk_select(OM.router_logits(x, wr, b), cfg.top_k)[0]
    touched = sorted(set(ids.reshape(-1).tolist()))
    mats = [W("routed", e) for e in touched] + [W("shared", s) for s in range(cfg.num_shared)]
    runs = 5 if cfg.name == "tiny" else 1
    total = decode = float("inf")
    for _ in range(runs):  # best of `runs`; input generation stays outside the timing
        t0 = time.perf_counter()
        OM.forward(x, wr, b, W, num_experts=cfg.num_experts, top_k=cfg.top_k,
                   num_shared=cfg.num_shared, d_ff=cfg.d_ff, activations="bf16" if a16w4 else "mxfp8")
        total = min(total, time.perf_counter() - t0)
        t0 = time.perf_counter()
        for gc, gs, dc, ds in mats:
            OX.mx_decode(gc, gs, "e2m1")
            OX.mx_decode(dc, ds, "e2m1")
        decode = min(decode, time.perf_counter() - t0)
    return {"value": round(ntok / total, 4), "unit": "tokens/s",
            "cores": int(max(blas_threads, 1)), "kind": "oracle",
            "sample": f"{ntok} token(s) of the {cfg.name} workload (layer copy 0, batch 0): "
                      + ("routing, bf16 activations (A16W4), " if a16w4 else "routing, MXFP8 quantisation, ")
                      + f"{len(touched)} routed + {cfg.num_shared} shared experts in float64; {total:.2f} s"
                      + (f" (best of {runs})" if runs > 1 else ""),
            "seconds": round(total, 4), "weight_decode_s": round(decode, 4),
            "compute_s": round(max(total - decode, 0.0), 4),
            "host_cpus": len(os.sched_getaffinity(0))}


if __name__ == "__main__":
    main()
