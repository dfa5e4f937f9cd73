"""Seeded synthetic inputs for the MoE layer (shared by the tests, the oracle
checks and the benchmark).

This module holds none of the layer's arithmetic: it only draws inputs.  It is
the one piece of code both the oracle and the HIP path are fed from.

Workloads (shapes and distributions follow the stated configurations; the
pages give no layer shapes, so d_model=7168 / d_ff=2048 are assumed):

* ``tiny``            T=8,     d=256,  E=16,  top-2,  d_ff=128,  1 shared
* ``decode1``         T=1,     d=7168, E=896, top-16, d_ff=2048, 2 shared
* ``decode256``       T=256,   same layer
* ``prefill8k``       T=8192,  same layer
* ``prefill32k_skew`` T=32768, same layer + Zipf(s=1.1) router bias

Recipes
-------
x      : N(0, 1) drawn in float32 (numpy PCG64, seed sequence [seed, 1]),
         rounded to bf16 with round-to-nearest-even.
W_r    : N(0, 0.02) float32 (seed sequence [seed, 2]).
bias   : zero, or for the skewed workload b_e = fp32(1.5 * ln p_e) with
         p_e = (e+1)^-1.1 / sum_r r^-1.1 (expert 0 hottest).
experts: N(0, 1/sqrt(d)) quantised to MXFP4, from a counter-based generator
         (Philox4x64-10, Salmon et al., SC'11) so that any expert can be
         regenerated alone and the GPU can generate the 21 GB layer itself
         bit-identically.  Block b (32 consecutive elements of a row) takes the
         64 bytes of counters 2b and 2b+1: 32 little-endian 16-bit uniforms u,
         each mapped through the inverse normal CDF at (u + 1/2) / 65536 (a
         float32 table of 65536 entries) and multiplied in float32 by
         sigma = float32(1/sqrt(d)).  The block is then quantised as the OCP MX
         format defines: E8M0 scale 2^e with e = floor(log2(amax)) - 2 (E2M1's
         largest exponent), elements x / 2^e rounded to the nearest E2M1 value
         (ties to the even code, saturating at 6).  The LatentMoE tail's W_up
         takes sigma from its own reduction width.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np

# ---------------------------------------------------------------------------
# Workload configurations
# ---------------------------------------------------------------------------


@dataclass(frozen=True)
class LayerConfig:
    name: str
    tokens: int
    d_model: int
    num_experts: int
    top_k: int
    d_ff: int
    num_shared: int
    zipf_bias: bool = False
    seed: int = 0


CONFIGS = {
    "tiny": LayerConfig("tiny", 8, 256, 16, 2, 128, 1),
    "decode1": LayerConfig("decode1", 1, 7168, 896, 16, 2048, 2),
    "decode256": LayerConfig("decode256", 256, 7168, 896, 16, 2048, 2),
    "prefill8k": LayerConfig("prefill8k", 8192, 7168, 896, 16, 2048, 2),
    "prefill32k_skew": LayerConfig("prefill32k_skew", 32768, 7168, 896, 16, 2048, 2, zipf_bias=True),
}

# ---------------------------------------------------------------------------
# Dense inputs
# ---------------------------------------------------------------------------


def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round-to-nearest-even (finite inputs)."""
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32)
    r = (u + (np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1)))) >> 16
    return r.astype(np.uint16)


def gen_x(cfg: LayerConfig, tokens: Optional[int] = None, layer: int = 0) -> np.ndarray:
    """Activations [T, d] as bf16 bit patterns (uint16)."""
    t = cfg.tokens if tokens is None else tokens
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, 1, layer])))
    return f32_to_bf16_bits(rng.standard_normal((t, cfg.d_model), dtype=np.float32))


def gen_router_w(cfg: LayerConfig, layer: int = 0) -> np.ndarray:
    """Router weight [E, d] float32, N(0, 0.02)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, 2, layer])))
    return rng.standard_normal((cfg.num_experts, cfg.d_model), dtype=np.float32) * np.float32(0.02)


def gen_router_b(cfg: LayerConfig) -> Optional[np.ndarray]:
    """Router bias [E] float32, or None (zero bias)."""
    if not cfg.zipf_bias:
        return None
    ranks = np.arange(1, cfg.num_experts + 1, dtype=np.float64)
    pmf = ranks ** -1.1
    pmf /= pmf.sum()
    return (1.5 * np.log(pmf)).astype(np.float32)


# ---------------------------------------------------------------------------
# Philox4x64-10 (Salmon, Moraes, Dror, Shaw: "Parallel random numbers: as easy
# as 1, 2, 3", SC'11).  Counter-based: output = f(key, counter).
# ---------------------------------------------------------------------------

PHILOX_M0 = 0xD2E7470EE14C6C93
PHILOX_M1 = 0xCA5A826395121157
PHILOX_W0 = 0x9E3779B97F4A7C15
PHILOX_W1 = 0xBB67AE8584CAA73B
_MASK32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def _mulhilo64(a_const: int, b: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """(hi, lo) 64-bit halves of the 128-bit product a_const * b (uint64 arrays)."""
    a_lo = np.uint64(a_const & 0xFFFFFFFF)
    a_hi = np.uint64(a_const >> 32)
    b_lo = b & _MASK32
    b_hi = b >> _S32
    p0 = a_lo * b_lo
    p1 = a_lo * b_hi
    p2 = a_hi * b_lo
    p3 = a_hi * b_hi
    mid = (p0 >> _S32) + (p1 & _MASK32) + (p2 & _MASK32)
    hi = p3 + (p1 >> _S32) + (p2 >> _S32) + (mid >> _S32)
    lo = b * np.uint64(a_const)  # wraps modulo 2**64
    return hi, lo


def philox4x64_10(key: Tuple[int, int], c0: np.ndarray, c1=0, c2=0, c3=0) -> np.ndarray:
    """Philox4x64 with 10 rounds.  c0: uint64 array of counters (word 0); the
    other counter words are scalars.  Returns [n, 4] uint64."""
    with np.errstate(over="ignore"):
        c0 = np.asarray(c0, dtype=np.uint64)
        x0 = c0.copy()
        x1 = np.full_like(c0, np.uint64(c1))
        x2 = np.full_like(c0, np.uint64(c2))
        x3 = np.full_like(c0, np.uint64(c3))
        k0, k1 = int(key[0]) & 0xFFFFFFFFFFFFFFFF, int(key[1]) & 0xFFFFFFFFFFFFFFFF
        for r in range(10):
            if r:
                k0 = (k0 + PHILOX_W0) & 0xFFFFFFFFFFFFFFFF
                k1 = (k1 + PHILOX_W1) & 0xFFFFFFFFFFFFFFFF
            hi0, lo0 = _mulhilo64(PHILOX_M0, x0)
            hi1, lo1 = _mulhilo64(PHILOX_M1, x2)
            x0, x1, x2, x3 = hi1 ^ x1 ^ np.uint64(k0), lo1, hi0 ^ x3 ^ np.uint64(k1), lo0
    return np.stack([x0, x1, x2, x3], axis=-1)


def philox_bytes(key: Tuple[int, int], first: int, count: int, c1: int = 0) -> np.ndarray:
    """32 bytes per counter value, for counters first..first+count-1:
    [count, 32] uint8, byte j of a call = byte j%8 (little-endian) of word j/8."""
    ctr = np.arange(first, first + count, dtype=np.uint64)
    words = philox4x64_10(key, ctr, c1)
    return words.astype("<u8").view(np.uint8).reshape(count, 32)


# ---------------------------------------------------------------------------
# MXFP4 weights: N(0, sigma) samples quantised block by block
# ---------------------------------------------------------------------------

KIND_GU_CODES, KIND_DN_CODES = 1, 3
KIND_UP_CODES = 5  # LatentMoE tail up projection
SHARED_BASE = 0x10000

_NORMAL_TABLE = None


def normal_table() -> np.ndarray:
    """float32 [65536]: the standard normal quantile at (u + 1/2) / 65536."""
    global _NORMAL_TABLE
    if _NORMAL_TABLE is None:
        from scipy.special import ndtri
        _NORMAL_TABLE = ndtri((np.arange(65536, dtype=np.float64) + 0.5) / 65536.0).astype(np.float32)
    return _NORMAL_TABLE


def weight_sigma(width: int) -> np.float32:
    """float32(1 / sqrt(width)): the standard deviation of the weights of a
    matrix whose rows are `width` long."""
    return np.float32(1.0 / np.sqrt(float(width)))


def stream_id(kind: int, expert_slot: int, layer: int = 0) -> int:
    return (layer << 48) | (kind << 32) | expert_slot


def expert_slot(kind: str, index: int) -> int:
    return index if kind == "routed" else SHARED_BASE + index


# E2M1 rounding boundaries of |x| / 2^e, each with the side a tie goes to:
# values at a boundary round to the code with the even mantissa (0, 1.0, 2.0,
# 4.0), so a code is reached above 0.25, 1.25, 2.5 and 5 but from 0.75, 1.75
# and 3.5 on
_E2M1_ABOVE = np.array([0.25, 1.25, 2.5, 5.0], dtype=np.float32)
_E2M1_FROM = np.array([0.75, 1.75, 3.5], dtype=np.float32)


def quantize_blocks_mx4(x: np.ndarray):
    """OCP MX quantisation of float32 blocks [n, 32] to (packed E2M1 codes
    [n, 16] uint8, element 2i in the low nibble of byte i; E8M0 scale bytes
    [n] uint8)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=1)
    ebits = ((amax.view(np.uint32) >> 23) & 0xFF).astype(np.int64)   # biased exponent of amax
    zero = amax == 0
    # floor(log2 amax) - 2, kept where 2^-e is a normal float32 (blocks of
    # normal, finite values well inside the float32 range stay unclamped)
    e = np.where(zero, -127, np.clip(ebits - 127 - 2, -126, 125))
    # 2^-e as float32 (exact); all-zero blocks use 1
    inv = np.where(zero, np.uint32(127 << 23), ((127 - e) << 23).astype(np.uint32)).astype(np.uint32).view(np.float32)
    a = np.abs(x) * inv[:, None]
    mag = np.zeros(x.shape, dtype=np.uint8)
    for t in _E2M1_ABOVE:
        mag += (a > t).astype(np.uint8)
    for t in _E2M1_FROM:
        mag += (a >= t).astype(np.uint8)
    codes = mag | ((x < 0).astype(np.uint8) << 3)
    packed = codes[:, 0::2] | (codes[:, 1::2] << 4)
    scales = (e + 127).astype(np.uint8)
    return packed, scales


def normal_blocks(seed: int, stream: int, blocks: np.ndarray, sigma: np.float32) -> np.ndarray:
    """float32 [n, 32]: the N(0, sigma) samples of blocks `blocks` (counters
    2b and 2b+1 of each block b)."""
    blocks = np.asarray(blocks, dtype=np.uint64)
    ctr = np.stack([2 * blocks, 2 * blocks + np.uint64(1)], axis=1).reshape(-1)
    words = philox4x64_10((seed, stream), ctr).astype("<u8")                # [2n, 4]
    u = words.view(np.uint16).reshape(blocks.size, 32)                      # 64 bytes -> 32 uniforms
    return normal_table()[u] * np.float32(sigma)


def gen_mx_matrix(seed: int, stream: int, rows: int, k: int, sigma: np.float32,
                  row0: int = 0, nrows: Optional[int] = None):
    """Rows [row0, row0+nrows) of one MXFP4 matrix [rows, k] drawn from
    N(0, sigma): (packed codes [n, k/2] uint8, scales [n, k/32] uint8)."""
    n = rows - row0 if nrows is None else nrows
    nb = k // 32
    b0 = row0 * nb
    nblk = n * nb
    packed = np.empty((nblk, 16), dtype=np.uint8)
    scales = np.empty(nblk, dtype=np.uint8)

    # chunked over threads (numpy releases the GIL inside its array operations)
    def fill(lo: int, hi: int) -> None:
        x = normal_blocks(seed, stream, np.arange(b0 + lo, b0 + hi, dtype=np.uint64), sigma)
        packed[lo:hi], scales[lo:hi] = quantize_blocks_mx4(x)

    step = 1 << 14
    spans = [(lo, min(lo + step, nblk)) for lo in range(0, nblk, step)]
    threads = min(len(spans), os.cpu_count() or 1, 16, int(os.environ.get("MXMOE_GEN_THREADS", "16")))
    if threads > 1:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(lambda sp: fill(*sp), spans))
    else:
        for sp in spans:
            fill(*sp)
    return packed.reshape(n, k // 2), scales.reshape(n, nb)


def gen_mx_matrix_kblocks(seed: int, stream: int, rows: int, k: int, sigma: np.float32, kblocks):
    """The same matrix as gen_mx_matrix, only the 32-wide K blocks `kblocks`
    of every row: (packed codes [rows, len(kblocks), 16], scales [rows,
    len(kblocks)]), drawn from the same counters."""
    kb = np.asarray(kblocks, dtype=np.int64)
    nb = k // 32
    blk = (np.arange(rows, dtype=np.int64)[:, None] * nb + kb[None, :]).reshape(-1)
    packed, scales = quantize_blocks_mx4(normal_blocks(seed, stream, blk.astype(np.uint64), sigma))
    return packed.reshape(rows, kb.size, 16), scales.reshape(rows, kb.size)


def gen_expert(cfg: LayerConfig, kind: str, index: int, layer: int = 0):
    """(gu_codes [2 d_ff, d/2], gu_scales [2 d_ff, d/32],
        dn_codes [d, d_ff/2],   dn_scales [d, d_ff/32]) of one expert."""
    slot = expert_slot(kind, index)
    sg = weight_sigma(cfg.d_model)
    guc, gus = gen_mx_matrix(cfg.seed, stream_id(KIND_GU_CODES, slot, layer), 2 * cfg.d_ff, cfg.d_model, sg)
    dnc, dns = gen_mx_matrix(cfg.seed, stream_id(KIND_DN_CODES, slot, layer), cfg.d_model, cfg.d_ff, sg)
    return guc, gus, dnc, dns


class ExpertWeights:
    """Lazily generated, cached per-expert weights: callable as weights(kind, i)."""

    def __init__(self, cfg: LayerConfig, layer: int = 0, cache: bool = True):
        self.cfg, self.layer, self.cache = cfg, layer, cache
        self._c = {}

    def __call__(self, kind: str, index: int):
        key = (kind, index)
        if key in self._c:
            return self._c[key]
        w = gen_expert(self.cfg, kind, index, self.layer)
        if self.cache:
            self._c[key] = w
        return w

    def min_scale_byte(self) -> Optional[int]:
        """The smallest E8M0 scale byte among the experts drawn so far (None if none)."""
        if not self._c:
            return None
        return int(min(min(int(w[1].min()), int(w[3].min())) for w in self._c.values()))

    def dn_blocks(self, kind: str, index: int, kblocks):
        """Blocks `kblocks` (32 columns each) of every row of W_dn [d, d_ff]:
        (packed codes [d, n, 16], scales [d, n]), without drawing the rest."""
        key = (kind, index)
        kb = np.asarray(kblocks, dtype=np.int64)
        if key in self._c:
            dnc, dns = self._c[key][2], self._c[key][3]
            return (dnc.reshape(dnc.shape[0], -1, 16)[:, kb], dns[:, kb])
        slot = expert_slot(kind, index)
        return gen_mx_matrix_kblocks(self.cfg.seed, stream_id(KIND_DN_CODES, slot, self.layer),
                                     self.cfg.d_model, self.cfg.d_ff, weight_sigma(self.cfg.d_model), kb)

    def stacked(self):
        """All routed and shared experts stacked (small configs only)."""
        e, s = self.cfg.num_experts, self.cfg.num_shared
        r = [self("routed", i) for i in range(e)]
        sh = [self("shared", i) for i in range(s)]
        stack = lambda lst, j: np.stack([w[j] for w in lst]) if lst else None
        return ([stack(r, j) for j in range(4)], [stack(sh, j) for j in range(4)])


def matrix_bytes(rows: int, k: int) -> int:
    return rows * k // 2 + rows * k // 32



# ---------------------------------------------------------------------------
# LatentMoE tail inputs
# ---------------------------------------------------------------------------


def gen_up_matrix(hidden: int, latent: int, seed: int = 0, layer: int = 0):
    """W_up [hidden, latent] in canonical MXFP4 (codes [hidden, latent/2],
    scales [hidden, latent/32]): N(0, 1/sqrt(latent)) quantised to MXFP4 by
    the experts' recipe."""
    return gen_mx_matrix(seed, stream_id(KIND_UP_CODES, 0, layer), hidden, latent, weight_sigma(latent))


def gen_tail_inputs(tokens: int, latent: int, hidden: int, seed: int = 0, layer: int = 0):
    """(z [T, latent], s [T, hidden], gamma [latent]) float32: z ~ N(0, 0.5^2)
    (the routed experts' weighted sum), s ~ N(0, 1) (the shared experts'
    output), gamma ~ 1 + N(0, 0.1^2) (the RMSNorm gain)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 3, layer])))
    z = rng.standard_normal((tokens, latent), dtype=np.float32) * np.float32(0.5)
    s = rng.standard_normal((tokens, hidden), dtype=np.float32)
    gamma = np.float32(1) + rng.standard_normal(latent, dtype=np.float32) * np.float32(0.1)
    return z, s, gamma
