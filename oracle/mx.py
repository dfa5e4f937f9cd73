"""MX element / scale encodings and the MX block quantiser (oracle, float64).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

The pages name the formats only ("MXFP4 weights", "MXFP8 activations":
"Kimi K3 ... MoE推理系统工程分析"; "Kimi K3本地部署指南", section 1 spec table).
Their bit layouts are the public OCP Microscaling v1.0 ones:

* E2M1 (FP4): 1 sign, 2 exponent (bias 1), 1 mantissa bit; no inf/NaN;
  magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
* E4M3 (FP8, "fn" variant): 1 sign, 4 exponent (bias 7), 3 mantissa bits;
  exponent field 0 is subnormal; S.1111.111 is NaN; largest finite 448.
* E8M0 (block scale): an unsigned biased exponent, value 2**(k-127); 0xFF NaN.

An MX block is 32 consecutive elements along a GEMM's reduction axis sharing
one E8M0 scale.  FP4 codes are packed two per byte, element 2i in the low
nibble of byte i.
"""

from __future__ import annotations

import numpy as np

BLOCK = 32

# --------------------------------------------------------------------------
# Element decodes, written from the bit-field definitions.
# --------------------------------------------------------------------------


def decode_e2m1(code) -> np.ndarray:
    """Value of E2M1 codes (uint8 in [0, 16)), exact in float64."""
    c = np.asarray(code).astype(np.int64)
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    # exponent field 0: subnormal m * 2**(1 - bias) * 2**-1 = m * 0.5
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e - 1.0))
    return np.where(s == 1, -mag, mag).astype(np.float64)


def decode_e4m3(code) -> np.ndarray:
    """Value of E4M3 ("fn") codes (uint8), exact in float64; NaN for 0x7F/0xFF."""
    c = np.asarray(code).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag).astype(np.float64)


def decode_e8m0(code) -> np.ndarray:
    """Value 2**(k-127) of E8M0 scale bytes, float64; NaN for 0xFF."""
    k = np.asarray(code).astype(np.int64)
    return np.where(k == 255, np.nan, np.exp2(k - 127.0))


def unpack_fp4(packed) -> np.ndarray:
    """[..., K/2] packed bytes -> [..., K] E2M1 codes (low nibble = even index)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def pack_fp4(codes) -> np.ndarray:
    """[..., K] E2M1 codes -> [..., K/2] packed bytes (low nibble = even index)."""
    c = np.asarray(codes, dtype=np.uint8)
    assert c.shape[-1] % 2 == 0
    return (c[..., 0::2] & 0x0F) | ((c[..., 1::2] & 0x0F) << 4)


def mx_decode(codes, scales, fmt: str) -> np.ndarray:
    """Decode an MX matrix to float64.

    codes: [rows, K] uint8 element codes for "e4m3"; [rows, K/2] packed bytes
    for "e2m1".  scales: [rows, K/32] E8M0 bytes.  Each block of 32 elements
    along K is multiplied by its own scale (exact: a power of two).
    """
    # decode through the format's value table (same values as the bit-field
    # decoders, looked up per code for speed on large matrices)
    if fmt == "e2m1":
        vals = decode_e2m1(np.arange(16))[unpack_fp4(codes)]
    elif fmt == "e4m3":
        vals = decode_e4m3(np.arange(256))[np.asarray(codes, dtype=np.uint8)]
    else:
        raise ValueError(fmt)
    rows, k = vals.shape
    sc = decode_e8m0(scales)
    assert sc.shape == (rows, k // BLOCK), (sc.shape, vals.shape)
    return (vals.reshape(rows, k // BLOCK, BLOCK) * sc[:, :, None]).reshape(rows, k)


# --------------------------------------------------------------------------
# Quantiser: OCP MX rule, round-to-nearest-even on the element grid.
# --------------------------------------------------------------------------

# largest exponent of the element format (floor(log2(max finite)))
_EMAX = {"e2m1": 2, "e4m3": 8}


def _positive_grid(fmt: str):
    """Non-negative finite values of the element format, ascending, with codes."""
    if fmt == "e2m1":
        codes = np.arange(0, 8, dtype=np.int64)
        vals = decode_e2m1(codes)
    elif fmt == "e4m3":
        codes = np.arange(0, 0x7F, dtype=np.int64)  # 0x7F is NaN
        vals = decode_e4m3(codes)
    else:
        raise ValueError(fmt)
    assert np.all(np.diff(vals) > 0)
    return vals, codes


def round_to_grid(q, fmt: str) -> np.ndarray:
    """Element codes of float64 values q (already divided by the block scale).

    Nearest grid value; a tie goes to the code with an even mantissa (the even
    code, since codes are consecutive along the grid); magnitudes beyond the
    largest finite value saturate to it.  The sign bit is kept even when the
    magnitude rounds to zero (IEEE-style signed zero).
    """
    q = np.asarray(q, dtype=np.float64)
    if not np.all(np.isfinite(q)):
        raise ValueError("MX quantiser input must be finite")
    vals, codes = _positive_grid(fmt)
    a = np.abs(q)
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, len(vals) - 1)
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    d_lo = a - vals[lo]
    d_hi = vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (codes[hi] % 2 == 0))
    # beyond the top of the grid: hi == lo == last -> saturate
    idx = np.where(pick_hi, hi, lo)
    idx = np.where(a >= vals[-1], len(vals) - 1, idx)
    mag_code = codes[idx]
    sign_bit = 8 if fmt == "e2m1" else 0x80
    return (mag_code + np.where(np.signbit(q), sign_bit, 0)).astype(np.uint8)


def block_exponent(amax, fmt: str) -> np.ndarray:
    """Shared exponent of a block: clamp(floor(log2(amax)) - emax, -127, 127).

    amax == 0 gives -127 (scale byte 0x00).  floor(log2) is taken exactly from
    the binary exponent (frexp), not from a floating-point log.
    """
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(amax)  # amax = m * 2**ex, m in [0.5, 1)
    flog2 = ex.astype(np.int64) - 1
    e = np.clip(flog2 - _EMAX[fmt], -127, 127)
    return np.where(amax == 0, -127, e).astype(np.int64)


def mx_quantize(v, fmt: str):
    """MX-quantise a [rows, K] float matrix along K in blocks of 32.

    Returns (codes, scales): codes [rows, K] uint8 (E4M3) or [rows, K/2] packed
    uint8 (E2M1); scales [rows, K/32] E8M0 bytes (= e + 127).
    Per block: e from :func:`block_exponent`; elements v / 2**e rounded by
    :func:`round_to_grid` (dividing by a power of two is exact in float64 here).
    """
    v = np.asarray(v, dtype=np.float64)
    rows, k = v.shape
    assert k % BLOCK == 0
    blocks = v.reshape(rows, k // BLOCK, BLOCK)
    amax = np.max(np.abs(blocks), axis=2)
    e = block_exponent(amax, fmt)
    q = blocks / np.exp2(e.astype(np.float64))[:, :, None]
    codes = round_to_grid(q, fmt).reshape(rows, k)
    scales = (e + 127).astype(np.uint8)
    if fmt == "e2m1":
        codes = pack_fp4(codes)
    return codes, scales
