"""The seeded input generator (CPU only): Philox against numpy's library
implementation, determinism, per-expert regeneration, and the stated recipe
(normal samples, OCP MX quantisation) checked against its definition."""

import math

import numpy as np

from mxfp4_expert_grouped_amd import inputs as I


def test_philox4x64_matches_numpy_library():
    for key, ctr in [((5, 0), 7), ((0, 0), 0), ((0xDEADBEEF, 12345), 2 ** 40 + 3),
                     ((2 ** 64 - 1, 2 ** 63 + 5), 2 ** 62)]:
        g = np.random.Philox(key=key[0] + (key[1] << 64), counter=ctr)
        ref = g.random_raw(12)
        # numpy advances the counter before each block
        mine = I.philox4x64_10(key, np.arange(ctr + 1, ctr + 4, dtype=np.uint64)).reshape(-1)
        assert np.array_equal(ref, mine)


def test_philox_counter_words():
    g = np.random.Philox(key=9, counter=(2 ** 64 - 1) + (3 << 64))
    ref = g.random_raw(4)  # counter wraps word 0 and carries into word 1
    mine = I.philox4x64_10((9, 0), np.array([0], dtype=np.uint64), c1=4).reshape(-1)
    assert np.array_equal(ref, mine)


def test_weights_regenerate_by_rows_and_are_deterministic():
    cfg = I.CONFIGS["tiny"]
    a = I.gen_expert(cfg, "routed", 3)
    b = I.gen_expert(cfg, "routed", 3)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    c, s = I.gen_mx_matrix(cfg.seed, I.stream_id(I.KIND_GU_CODES, 3), 2 * cfg.d_ff, cfg.d_model,
                           I.weight_sigma(cfg.d_model), row0=37, nrows=50)
    assert np.array_equal(c, a[0][37:87]) and np.array_equal(s, a[1][37:87])
    other = I.gen_expert(cfg, "routed", 4)
    assert not np.array_equal(a[0], other[0])
    sh = I.gen_expert(cfg, "shared", 3)
    assert not np.array_equal(a[0], sh[0])


def test_normal_table_is_the_normal_quantile():
    t = I.normal_table()
    assert t.dtype == np.float32 and t.size == 65536
    assert np.all(np.diff(t) > 0) and np.array_equal(t, -t[::-1])
    # Phi(t[u]) = (u + 1/2) / 65536, through the error function
    for u in (0, 1, 100, 20000, 32767, 40000, 65535):
        p = 0.5 * (1.0 + math.erf(float(t[u]) / math.sqrt(2.0)))
        want = (u + 0.5) / 65536
        assert abs(min(p, 1 - p) - min(want, 1 - want)) < 1e-5 * min(want, 1 - want)


def _e2m1_nearest(a):
    """Nearest E2M1 magnitude to a >= 0 by exhaustive search, ties to the even
    code (mantissa bit 0), saturating at 6: the OCP definition, element by element."""
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    if a >= 6.0:
        return 7
    best = min(range(8), key=lambda c: (abs(grid[c] - a), c & 1))
    return best


def test_weights_are_normal_samples_quantised_to_mxfp4():
    """The literal recipe: N(0, 1/sqrt(d)) samples, each block quantised with
    E8M0 scale 2^(floor(log2 amax) - 2) and E2M1 elements rounded to nearest
    (ties to even), checked element by element in float64 for a sample of
    blocks."""
    d = 7168
    sigma = I.weight_sigma(d)
    blocks = np.arange(0, 4096 * 7, 7, dtype=np.uint64)
    x = I.normal_blocks(0, 99, blocks, sigma)
    assert abs(x.mean()) < 0.01 * sigma and abs(x.std() / sigma - 1) < 0.01
    kurt = ((x / x.std()) ** 4).mean()
    assert abs(kurt - 3) < 0.1
    packed, scales = I.quantize_blocks_mx4(x)
    codes = np.stack([packed & 15, packed >> 4], axis=2).reshape(-1, 32)
    for i in range(0, blocks.size, 97):
        xb = x[i].astype(np.float64)
        amax = np.abs(xb).max()
        e = math.floor(math.log2(amax)) - 2
        assert scales[i] == e + 127
        for j in range(32):
            want = _e2m1_nearest(abs(xb[j]) / 2.0 ** e) | (8 if xb[j] < 0 else 0)
            assert codes[i, j] == want, (i, j, xb[j], e)
    # every block's largest element lands on 4 or 6 times its scale
    assert np.all((codes & 7).max(axis=1) >= 6)


def test_mxfp4_quantiser_ties_zero_and_saturation():
    # |x| / 2^e at every E2M1 midpoint (amax forced to 4 * 2^e, e = 0)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)
    blk = np.zeros((2, 32), dtype=np.float32)
    blk[0, :7] = mids
    blk[0, 7:14] = -mids
    blk[0, 31] = 4.0
    packed, scales = I.quantize_blocks_mx4(blk)
    codes = np.stack([packed & 15, packed >> 4], axis=2).reshape(-1, 32)
    assert scales[0] == 127 and scales[1] == 0
    assert codes[0, :7].tolist() == [0, 2, 2, 4, 4, 6, 6]
    assert codes[0, 7:14].tolist() == [8, 10, 10, 12, 12, 14, 14]
    assert codes[0, 31] == 6 and np.all(codes[1] == 0)
    # 7.99 * 2^e saturates to 6, scale from its exponent
    blk = np.full((1, 32), 0.001, dtype=np.float32)
    blk[0, 0] = 7.99
    packed, scales = I.quantize_blocks_mx4(blk)
    assert scales[0] == 127 and (packed[0, 0] & 15) == 7


def test_dense_inputs():
    cfg = I.CONFIGS["tiny"]
    x = I.gen_x(cfg)
    assert x.shape == (8, 256) and x.dtype == np.uint16
    xf = (x.astype(np.uint32) << 16).view(np.float32)
    assert abs(xf.std() - 1) < 0.1
    w = I.gen_router_w(cfg)
    assert w.dtype == np.float32 and abs(w.std() - 0.02) < 0.002
    assert I.gen_router_b(cfg) is None
    b = I.gen_router_b(I.CONFIGS["prefill32k_skew"])
    assert b.shape == (896,) and b.dtype == np.float32
    h = sum(r ** -1.1 for r in range(1, 897))
    assert abs(b[0] - 1.5 * np.log(1 / h)) < 1e-5
    assert abs(b[895] - 1.5 * np.log(896 ** -1.1 / h)) < 1e-5
    assert np.all(np.diff(b) < 0)


def test_dn_blocks_are_the_matrix_blocks():
    cfg = I.LayerConfig("blk", 3, 256, 4, 2, 128, 1, seed=4)
    full = I.gen_expert(cfg, "routed", 2)
    for cache in (False, True):
        W = I.ExpertWeights(cfg, cache=cache)
        if cache:
            W("routed", 2)
        c, s = W.dn_blocks("routed", 2, [0, 3])
        assert np.array_equal(c, full[2].reshape(256, -1, 16)[:, [0, 3]])
        assert np.array_equal(s, full[3][:, [0, 3]])
    sh = I.gen_expert(cfg, "shared", 0)
    c, s = I.ExpertWeights(cfg, cache=False).dn_blocks("shared", 0, [1])
    assert np.array_equal(c[:, 0], sh[2].reshape(256, -1, 16)[:, 1]) and np.array_equal(s[:, 0], sh[3][:, 1])
