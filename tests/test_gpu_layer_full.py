"""GPU parity of the full-size layer (d=7168, 896 experts, top-16, d_ff=2048,
2 shared) at each benchmark workload, in the launch configuration the
benchmark times.

The whole layer runs on the GPU for every token; the oracle recomputes routing,
permutation and x quantisation for every token and the expert outputs for a
sample of tokens (each token's output depends only on its own row).  The
sample is chosen by where the tokens' rows sit in the grouped GEMMs' tiles:
the first, middle and last rows of the hottest experts' tiles (both row
halves of a prefill tile, the first row of a second tile, the ragged last
tile), rows of a median expert and of the least loaded experts, tokens at the
shared experts' tile boundaries, then evenly spaced tokens up to the sample
size.  The oracle's per-expert work runs in CPU processes.
"""

import numpy as np
import pytest
import torch

from mxfp4_expert_grouped_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def big():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mxfp4_expert_grouped_amd import mxmoe
    mxmoe.load_library()
    import parity as P
    cfg = I.CONFIGS["decode1"]
    P.log("generating the 896-expert layer on the GPU")
    W = P.IG.device_weights(cfg)
    torch.cuda.synchronize()
    ref = I.ExpertWeights(cfg, cache=False)  # numpy twin, regenerated per expert in the oracle's processes
    yield P, W, ref
    del W
    torch.cuda.empty_cache()


def pick_tokens(cfg, offsets: np.ndarray, row_src: np.ndarray, n: int):
    """Tokens whose rows sit at chosen tile positions (see the module doc)."""
    T, k = cfg.tokens, cfg.top_k
    if n >= T:
        return list(range(T))
    bm = 256 if (T * k) // cfg.num_experts >= 24 else 8
    counts = np.diff(offsets)
    order = np.argsort(-counts, kind="stable")
    picks = []

    def add_rows(e, positions):
        c = int(counts[e])
        for p in positions:
            if 0 <= p < c:
                picks.append(int(row_src[offsets[e] + p]) // k)

    for e in order[:3]:                                     # hottest experts
        c = int(counts[e])
        first = min(bm, c)
        nb = (first + 31) // 32                              # 32-row blocks of the first tile
        half = 32 * ((nb + 1) // 2)                          # row-half boundary of a prefill tile
        last0 = (c - 1) // bm * bm                           # first row of the last tile
        add_rows(e, [0, first // 2, first - 1, half - 1, half, bm, last0, (last0 + c - 1) // 2, c - 1])
    touched = [e for e in order if counts[e] > 0]
    med = touched[len(touched) // 2]                         # a median-load expert
    add_rows(med, [0, int(counts[med]) // 2, int(counts[med]) - 1])
    for e in touched[::-1][:6]:                              # least loaded experts: all their rows (few)
        add_rows(e, range(min(int(counts[e]), 2)))
    for t in (0, T - 1, bm - 1, bm, T // 2, T // 2 + bm - 1):  # shared-expert tile boundaries
        if 0 <= t < T:
            picks.append(t)
    picks = sorted(set(picks))
    fill = np.linspace(0, T - 1, n).astype(int).tolist()
    for t in fill:
        if len(picks) >= n:
            break
        if t not in picks:
            picks.append(t)
    return sorted(set(picks))


@pytest.mark.parametrize("name,nsample,a16", [
    ("decode1", 1, False),
    ("decode256", 12, False),
    ("prefill8k", 32, False),
    ("prefill32k_skew", 32, False),
    ("decode1", 1, True),
    ("decode256", 12, True),
    ("prefill8k", 32, True),
], ids=["decode1", "decode256", "prefill8k", "prefill32k_skew", "decode1_a16w4", "decode256_a16w4",
        "prefill8k_a16w4"])
def test_full_layer(big, name, nsample, a16):
    P, W, ref = big
    cfg = I.CONFIGS[name]
    b = I.gen_router_b(cfg)
    W.router_b = torch.from_numpy(b).cuda() if b is not None else None
    x_bits = I.gen_x(cfg)
    x = P.IG.bf16_tensor(x_bits)
    P.log(f"{name}: GPU forward T={cfg.tokens} (all taps{', A16W4' if a16 else ''})")
    g = P.run_gpu(cfg, W, x, a16=a16)
    # every token: routing weights sum to one, outputs finite
    assert np.all(np.abs(g["topk_w"].sum(1) - 1) < 1e-5)
    y = P.bf16_bits_to_f64(g["y"])
    assert np.all(np.isfinite(y))
    sample = pick_tokens(cfg, g["expert_offsets"], g["row_src"], nsample)
    P.log(f"{name}: sampled tokens {sample}")
    assert len(sample) >= nsample
    res, differ = P.compare_layer(cfg, x_bits, I.gen_router_w(cfg), b, ref, g, tokens=sample,
                                  workers=P.oracle_workers(), activations="bf16" if a16 else "mxfp8")
    assert len(res.tokens) == len(sample)
    if a16:
        W.router_b = None
        return
    # the x bytes of every 1/512th token, not only the sampled ones
    from oracle import moe as OM, mx as OX
    step = max(1, cfg.tokens // 512)
    rows = np.arange(0, cfg.tokens, step)
    xc, xs = OX.mx_quantize(OM.bf16_to_f64(x_bits[rows]), "e4m3")
    assert np.array_equal(g.rows("x_codes", rows), xc) and np.array_equal(g.rows("x_scales", rows), xs)
    if name == "prefill32k_skew":
        counts = np.diff(g["expert_offsets"])
        P.log(f"skew: max rows/expert {counts.max()}, experts touched {(counts > 0).sum()}, "
              f">2000 rows: {(counts > 2000).sum()}")
        assert counts.max() > 2000 and (counts == 0).sum() > 0
    W.router_b = None
