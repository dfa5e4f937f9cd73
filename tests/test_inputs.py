"""The seeded input generator (CPU only): Philox against numpy's library
implementation, determinism, per-expert regeneration, and the recipe's stated
distributions."""

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
    eb = I.scale_exponent_base(cfg.d_model)
    c, s = I.gen_mx_matrix(cfg.seed, I.stream_id(I.KIND_GU_CODES, 3), I.stream_id(I.KIND_GU_SCALES, 3),
                           2 * cfg.d_ff, cfg.d_model, eb, row0=37, nrows=50)
    assert np.array_equal(c, a[0][37:87]) and np.array_equal(s, a[1][37:87])
    other = I.gen_expert(cfg, "routed", 4)
    assert not np.array_equal(a[0], other[0])
    sh = I.gen_expert(cfg, "shared", 3)
    assert not np.array_equal(a[0], sh[0])


def test_weight_recipe_distribution():
    cfg = I.CONFIGS["decode1"]
    eb = I.scale_exponent_base(cfg.d_model)
    assert eb == -8 and I.scale_exponent_base(256) == -5
    c, s = I.gen_mx_matrix(0, 99, 100, 256, 7168, eb)
    nib = np.concatenate([c & 15, c >> 4]).reshape(-1)
    freq = np.bincount(nib & 7, minlength=8) / nib.size
    assert np.allclose(freq, np.array(I.MAG_SLOTS) / 128, atol=0.003)
    assert abs((nib >> 3).mean() - 0.5) < 0.003
    sv, sc = np.unique(s, return_counts=True)
    assert sv.tolist() == [127 + eb, 128 + eb]
    assert abs(sc[1] / s.size - 0.25) < 0.01


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
