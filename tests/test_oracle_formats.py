"""Pins for the oracle's MX encodings and quantiser (CPU only).

Each test checks the oracle against something other than its own formula:
the value table printed in the OCP MX v1.0 specification, torch's float8
dtypes (a library decode/cast), brute-force nearest-code search, and algebraic
properties that a dropped term or a wrong index would break.
"""

import itertools
import math

import numpy as np
import pytest
import torch

from oracle import mx
from oracle.moe import bf16_to_f64, f64_to_bf16

# ---------------------------------------------------------------------------
# Decode tables
# ---------------------------------------------------------------------------


def test_e2m1_table_exhaustive():
    # the 16 E2M1 values as listed in the OCP MX spec's FP4 table
    listed = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    want = listed + [-v for v in listed]
    got = mx.decode_e2m1(np.arange(16))
    assert np.array_equal(got, np.array(want))
    assert np.signbit(got[8])  # code 8 is -0


def test_e4m3_decode_matches_torch_all_256():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = mx.decode_e4m3(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    # landmarks: max finite, min normal, min subnormal
    assert got[0x7E] == 448.0 and got[0x08] == 2.0 ** -6 and got[0x01] == 2.0 ** -9


def test_e8m0_decode_matches_torch_all_256():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = mx.decode_e8m0(np.arange(256))
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])
    assert got[127] == 1.0 and got[0] == 2.0 ** -127


def test_fp4_pack_roundtrip_and_nibble_order():
    rng = np.random.default_rng(0)
    c = rng.integers(0, 16, size=(5, 64)).astype(np.uint8)
    p = mx.pack_fp4(c)
    assert p.shape == (5, 32)
    assert np.array_equal(mx.unpack_fp4(p), c)
    # element 0 in the low nibble, element 1 in the high nibble
    assert mx.pack_fp4(np.array([[0x3, 0xA]], np.uint8))[0, 0] == 0xA3


# ---------------------------------------------------------------------------
# Quantiser
# ---------------------------------------------------------------------------


def brute_force_code(q: float, fmt: str) -> int:
    """Nearest finite code by exhaustive search; ties -> even code; sign kept."""
    if fmt == "e4m3":
        allc = [c for c in range(128) if c != 0x7F]
        vals = mx.decode_e4m3(np.array(allc))
        signbit = 0x80
    else:
        allc = list(range(8))
        vals = mx.decode_e2m1(np.array(allc))
        signbit = 8
    a = abs(q)
    if a >= vals.max():
        best = allc[int(np.argmax(vals))]
    else:
        dist = np.abs(vals - a)
        m = dist.min()
        cands = [c for c, dd in zip(allc, dist) if dd == m]
        best = [c for c in cands if c % 2 == 0][0] if len(cands) > 1 else cands[0]
    return best | (signbit if math.copysign(1.0, q) < 0 else 0)


def brute_force_exponent(amax: float, emax: int) -> int:
    if amax == 0:
        return -127
    n = 0
    while 2.0 ** n > amax:
        n -= 1
    while 2.0 ** (n + 1) <= amax:
        n += 1
    return max(-127, min(127, n - emax))


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_quantiser_matches_brute_force(fmt):
    rng = np.random.default_rng(1)
    emax = 8 if fmt == "e4m3" else 2
    rows = []
    for scale in (1e-30, 1e-3, 0.37, 1.0, 7.5, 3e5):
        rows.append(rng.standard_normal(64) * scale)
    rows.append(np.concatenate([rng.standard_normal(31) * 1e-6, [5.0]]).tolist() + [0.0] * 32)
    rows.append([0.0] * 64)
    rows.append([-0.0] * 32 + [1e-40] + [0.0] * 31)
    v = np.array(rows, dtype=np.float64)
    codes, scales = mx.mx_quantize(v, fmt)
    if fmt == "e2m1":
        codes = mx.unpack_fp4(codes)
    for r in range(v.shape[0]):
        for b in range(2):
            blk = v[r, 32 * b:32 * b + 32]
            e = brute_force_exponent(float(np.max(np.abs(blk))), emax)
            assert scales[r, b] == e + 127
            for i in range(32):
                want = brute_force_code(float(blk[i]) / 2.0 ** e, fmt)
                assert codes[r, 32 * b + i] == want, (r, b, i, blk[i], e)


def test_e4m3_rounding_matches_torch_cast_in_range():
    # torch's float32 -> float8_e4m3fn cast is round-to-nearest-even; it returns
    # NaN above the finite range, so compare only |q| <= 448
    rng = np.random.default_rng(2)
    q = np.concatenate([
        rng.uniform(-448, 448, 20000),
        rng.uniform(-1, 1, 20000) * 2.0 ** -5,
        # exact midpoints between neighbouring codes (ties)
        (mx.decode_e4m3(np.arange(0, 0x7E)) + mx.decode_e4m3(np.arange(1, 0x7F))) / 2,
        -(mx.decode_e4m3(np.arange(0, 0x7E)) + mx.decode_e4m3(np.arange(1, 0x7F))) / 2,
    ])
    q = q.astype(np.float32).astype(np.float64)  # representable in fp32 for torch
    ref = torch.from_numpy(q.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = mx.round_to_grid(q, "e4m3")
    assert np.array_equal(got, ref)


def test_e4m3_saturates_instead_of_nan():
    got = mx.round_to_grid(np.array([448.0, 460.0, 464.0, 470.0, 511.9, -500.0]), "e4m3")
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE]


def test_e4m3_ties_and_signed_zero():
    # 1.0625 is halfway between 1.0 (0x38) and 1.125 (0x39): even -> 1.0;
    # 1.1875 halfway between 1.125 and 1.25 (0x3A): even -> 1.25
    got = mx.round_to_grid(np.array([1.0625, 1.1875, -1e-6, 2.0 ** -10, 3 * 2.0 ** -10]), "e4m3")
    assert list(got) == [0x38, 0x3A, 0x80, 0x00, 0x02]


def test_block_scale_rule_saturates_top_element():
    # amax = 1.9 * 2**3: e = 3 - 8 = -5, 1.9*8/2**-5 = 486.4 -> saturates to 448
    v = np.zeros((1, 32))
    v[0, 0] = 1.9 * 8
    codes, scales = mx.mx_quantize(v, "e4m3")
    assert scales[0, 0] == 127 - 5 and codes[0, 0] == 0x7E
    # FP4: amax = 7 -> e = 2 - 2 = 0, 7 saturates to 6
    v[0, 0] = 7.0
    codes, scales = mx.mx_quantize(v, "e2m1")
    assert scales[0, 0] == 127 and (codes[0, 0] & 0xF) == 0x7


def test_quantiser_power_of_two_equivariance():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((4, 96))
    c0, s0 = mx.mx_quantize(v, "e4m3")
    for j in (-20, -1, 1, 7, 40):
        c1, s1 = mx.mx_quantize(v * 2.0 ** j, "e4m3")
        assert np.array_equal(c0, c1)
        assert np.array_equal(s1.astype(int), s0.astype(int) + j)


def test_quantiser_idempotent_on_grid_and_sign_symmetric():
    rng = np.random.default_rng(4)
    v = rng.standard_normal((6, 64)) * 3
    c, s = mx.mx_quantize(v, "e4m3")
    dq = mx.mx_decode(c, s, "e4m3")
    c2, s2 = mx.mx_quantize(dq, "e4m3")
    assert np.array_equal(c, c2) and np.array_equal(s, s2)
    cn, sn = mx.mx_quantize(-v, "e4m3")
    assert np.array_equal(cn, c ^ 0x80) and np.array_equal(sn, s)
    # relative error bound of RNE with 3 mantissa bits: 2**-4, for elements in
    # the normal, non-saturating range of the element grid
    q = np.abs(v) / np.exp2(s.astype(float) - 127).repeat(32, axis=1)
    normal = (q >= 2.0 ** -6) & (q <= 448.0)
    rel = np.abs(dq - v)[normal] / np.abs(v)[normal]
    assert normal.sum() > 300 and rel.max() <= 2.0 ** -4 + 1e-12
    # a saturated element loses at most its excess over 448 (amax < 512)
    sat = q > 448.0
    assert np.all(np.abs(dq)[sat] == 448.0 * np.exp2(s.astype(float) - 127).repeat(32, axis=1)[sat])


def test_quantiser_monotone():
    v = np.sort(np.random.default_rng(5).uniform(-3, 3, 32))[None, :]
    c, s = mx.mx_quantize(v, "e4m3")
    d = mx.mx_decode(c, s, "e4m3")[0]
    assert np.all(np.diff(d) >= 0)


def test_quantiser_rejects_non_finite():
    with pytest.raises(ValueError):
        mx.mx_quantize(np.array([[np.inf] + [0.0] * 31]), "e4m3")


# ---------------------------------------------------------------------------
# bf16 helpers
# ---------------------------------------------------------------------------


def test_bf16_roundtrip_matches_torch():
    rng = np.random.default_rng(6)
    v = np.concatenate([rng.standard_normal(5000) * 10.0 ** rng.integers(-30, 30, 5000),
                        [0.0, -0.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1e-40, -3e-39]])
    v32 = v.astype(np.float32)
    ref = torch.from_numpy(v32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = f64_to_bf16(v32.astype(np.float64))
    assert np.array_equal(got, ref)
    back = torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(bf16_to_f64(ref), back)


def test_bf16_ties_to_even():
    # 1 + 2**-8 is halfway between 1 and 1 + 2**-7: even -> 1.0 (0x3F80)
    got = f64_to_bf16(np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8)]))
    assert list(got) == [0x3F80, 0x3F82, 0xBF80]


def test_all_e4m3_codes_roundtrip():
    for c in itertools.chain(range(0, 0x7F), range(0x80, 0xFF)):
        v = mx.decode_e4m3(np.array([c]))[0]
        assert mx.round_to_grid(np.array([v]), "e4m3")[0] == c
