"""NF4 storage format in plain numpy: the codebook, blockwise absmax quantisation, nibble packing,
double quantisation of the block scales, and the two-level dequantisation to bf16.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the benchmark's CPU baseline,
never by the HIP path. Sources are the pages' statement of the method, cited per function as
"page title, section".
"""
from __future__ import annotations

from fractions import Fraction
from statistics import NormalDist

import numpy as np

BLOCK = 64          # NF4 blocksize ("QLoRA, explained", Blockwise absmax quantisation)
DQ_GROUP = 256      # scales per second-level constant ("QLoRA, explained", Double quantisation)
NF4_ZERO_INDEX = 7  # index of the exact zero in the ascending codebook


def codebook() -> np.ndarray:
    """The 16 NF4 codes as float32, ascending (index 0 is -1, index 7 is 0, index 15 is +1).

    "QLoRA, explained", NormalFloat 4 (NF4): the codes sit at standard-normal quantiles (k = 4), the
    negative and positive halves are built separately so that an exact zero exists (the halves hold 8
    and 9 codes, zero being in both), and the set is renormalised into [-1, 1]. The page's formula
    and printed table did not survive; the reading taken here, which reproduces every code the
    worked example prints, is:

    * delta = the mean of the two extreme probability levels 1 - 1/30 and 1 - 1/32, i.e. 929/960
      (the "average of adjacent quantiles" at the tail);
    * positive half: Phi^-1(p) at 8 probabilities evenly spaced from delta towards 1/2
      (9 points from delta to 1/2 inclusive, the last one, 1/2, dropped);
    * negative half: -Phi^-1(p) at 7 probabilities spaced the same way (8 points, last dropped);
    * add 0, divide everything by Phi^-1(delta), sort ascending.

    The quantiles are evaluated in float64 with ``statistics.NormalDist`` and rounded once to float32.
    """
    delta = (Fraction(29, 30) + Fraction(31, 32)) / 2
    half = Fraction(1, 2)
    nd = NormalDist()
    pos = [nd.inv_cdf(float(delta - i * (delta - half) / 8)) for i in range(8)]
    neg = [-nd.inv_cdf(float(delta - i * (delta - half) / 7)) for i in range(7)]
    top = nd.inv_cdf(float(delta))
    vals = sorted([v / top for v in pos + neg] + [0.0])
    return np.array(vals, dtype=np.float64).astype(np.float32)


def quantize_blocks(w, blocksize: int = BLOCK, codes: np.ndarray | None = None):
    """Blockwise absmax quantisation to the nearest code.

    "QLoRA, explained", Blockwise absmax quantisation, and The algorithm, step by step:
    flatten W row-major, cut it into blocks of ``blocksize`` consecutive values, store per block the
    scale c = max |w| and per value the index of the code nearest to w / c.

    The decision is exact: w / c is nearer q[i+1] than q[i] exactly when w / c > (q[i] + q[i+1]) / 2,
    i.e. when w > c * m_i with m_i the midpoint. Each m_i is a float64 sum of two float32 codes
    (exact) halved (exact), and c * m_i multiplies a 24-bit by a <= 26-bit significand, which float64
    holds exactly; so ``w > c * m_i`` below is the exact comparison. A value exactly on a midpoint
    goes to the lower index. An all-zero block (c = 0) has no quotient; every value then takes the
    exact-zero code, the reading of the page's remark that the zero code serves padding and
    zero-valued weights.

    Returns (idx uint8 [nblocks, blocksize], absmax float32 [nblocks]).
    """
    if codes is None:
        codes = codebook()
    codes = np.asarray(codes, dtype=np.float32)
    w = np.asarray(w, dtype=np.float32).reshape(-1)
    if w.size % blocksize:
        raise ValueError("numel must be a multiple of the blocksize")
    blocks = w.reshape(-1, blocksize)
    absmax = np.abs(blocks).max(axis=1)                      # exact in float32
    q = codes.astype(np.float64)
    mids = (q[:-1] + q[1:]) / 2.0
    b64 = blocks.astype(np.float64)
    c64 = absmax.astype(np.float64)[:, None]
    idx = np.zeros(blocks.shape, dtype=np.uint8)
    for m in mids:
        idx += (b64 > c64 * m)
    zero_index = int(np.flatnonzero(codes == 0.0)[0])
    idx[absmax == 0] = zero_index
    return idx, absmax


def pack_nibbles(idx) -> np.ndarray:
    """Two 4-bit indices per byte ("QLoRA, explained", Minimal implementation: indices are packed
    two per byte). Reading: byte j holds element 2j in its high nibble and element 2j+1 in its low
    nibble."""
    idx = np.asarray(idx, dtype=np.uint8).reshape(-1)
    if idx.size % 2:
        raise ValueError("odd number of indices")
    return ((idx[0::2] << 4) | idx[1::2]).astype(np.uint8)


def unpack_nibbles(packed, numel: int | None = None) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8).reshape(-1)
    out = np.empty(packed.size * 2, dtype=np.uint8)
    out[0::2] = packed >> 4
    out[1::2] = packed & 0x0F
    return out if numel is None else out[:numel]


def quantize(w):
    """NF4 quantisation of a float32 weight with blocksize 64.

    Returns (packed uint8 [numel/2], absmax float32 [numel/64]); the first-level scales are exact
    float32 block maxima, before double quantisation.
    """
    idx, absmax = quantize_blocks(w, BLOCK)
    return pack_nibbles(idx), absmax


def e4m3_value(code: int) -> Fraction:
    """Value of an 8-bit float code in the OCP E4M3 layout (1 sign, 4 exponent bits with bias 7,
    3 mantissa bits; exponent field 0 is subnormal: m * 2^-9). Codes 0x7F/0xFF are NaN.

    "QLoRA, explained", Double quantisation, says only "8-bit floats"; E4M3 is the reading taken.
    """
    code = int(code) & 0xFF
    if code & 0x7F == 0x7F:
        raise ValueError("NaN code")
    sign = -1 if code & 0x80 else 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0:
        v = Fraction(m, 512)
    else:
        v = Fraction(8 + m, 8) * Fraction(2) ** (e - 7)
    return sign * v


def e4m3_unit_values() -> np.ndarray:
    """The E4M3 values in [0, 1] as float64, ascending; the array index equals the code (0x00..0x38)."""
    return np.array([float(e4m3_value(c)) for c in range(0x39)], dtype=np.float64)


def double_quant(absmax, group: int = DQ_GROUP):
    """Double quantisation of the first-level scales.

    "QLoRA, explained", Double quantisation, and The algorithm, step by step: the fp32
    block scales go through a second quantisation, to an 8-bit float format, in groups of 256
    scales, each group also storing a single fp32 constant. Readings taken where the page is
    silent:

    * the second-level constant of a group is its largest scale, c2 = max c1 (all scales are >= 0),
      so every ratio c1 / c2 lies in [0, 1]; the last group may hold fewer than 256 scales;
    * the 8-bit float is OCP E4M3 and the code is the E4M3 value nearest to the exact ratio c1 / c2,
      ties going to the even code; a group whose constant is 0 stores code 0.

    Exactness: a decision boundary is a midpoint between neighbouring E4M3 values (at most 5
    significant bits), so c2 * mid is exact in float64 and ``c1 > c2 * mid`` is the exact test.

    Returns (codes uint8 [nblocks], c2 float32 [ceil(nblocks / group)]).
    """
    c1 = np.asarray(absmax, dtype=np.float32).reshape(-1)
    nb = c1.size
    ng = -(-nb // group)
    padded = np.zeros(ng * group, dtype=np.float32)
    padded[:nb] = c1
    c2 = padded.reshape(ng, group).max(axis=1).astype(np.float32)
    vals = e4m3_unit_values()
    mids = (vals[:-1] + vals[1:]) / 2.0
    c1d = c1.astype(np.float64)
    c2d = np.repeat(c2.astype(np.float64), group)[:nb]
    code = np.zeros(nb, dtype=np.int64)
    for m in mids:
        code += (c1d > c2d * m)
    inside = code < mids.size
    tie = np.zeros(nb, dtype=bool)
    tie[inside] = c1d[inside] == c2d[inside] * mids[code[inside]]
    code[tie & (code % 2 == 1)] += 1
    code[c2d == 0] = 0
    return code.astype(np.uint8), c2


def dequant_scales(codes, c2, group: int = DQ_GROUP) -> np.ndarray:
    """First dequantisation level: c1' = fl32(e4m3(code) * c2), one float32 product per block.

    "QLoRA, explained", The forward pass and gradients: dDQ's first level turns each 8-bit scale code
    back into a float with its group's fp32 constant."""
    codes = np.asarray(codes, dtype=np.uint8).reshape(-1)
    vals = e4m3_unit_values().astype(np.float32)            # <= 4 significant bits: exact
    c2 = np.asarray(c2, dtype=np.float32).reshape(-1)
    c2b = np.repeat(c2, group)[: codes.size]
    return (vals[codes] * c2b).astype(np.float32)           # one IEEE float32 multiply, RNE


def bf16_bits_from_f32(x) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even) by integer arithmetic on the bits.
    Finite inputs only."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite value")
    u = x.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def f32_from_bf16_bits(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def dequant(packed, codes, c2, numel: int) -> np.ndarray:
    """Two-level dequantisation to bf16; returns uint16 bit patterns [numel].

    "QLoRA, explained", The forward pass and gradients: the block scales are recovered from their
    8-bit codes and group constants first; those scales then turn the NF4 indices into a bf16 weight. Rounding order (the
    reading taken): c1' = fl32(e4m3 * c2), w32 = fl32(q[idx] * c1'), bf16 = RNE(w32).
    """
    idx = unpack_nibbles(packed, numel).reshape(-1, BLOCK)
    c1p = dequant_scales(codes, c2)
    q = codebook()
    w32 = (q[idx] * c1p[:, None]).astype(np.float32)
    return bf16_bits_from_f32(w32).reshape(-1)


def quantize_with(w, codes, blocksize: int):
    """Blockwise absmax quantisation with any ascending codebook and blocksize, packed two indices
    per byte: the format the toy run compares ("QLoRA, explained", A toy run; the blocksize
    discussion). Returns (packed uint8 [numel/2], absmax float32 [numel/blocksize])."""
    idx, absmax = quantize_blocks(w, blocksize, codes)
    return pack_nibbles(idx), absmax


def dequant_blocks(packed, scales, codes, blocksize: int, numel: int) -> np.ndarray:
    """bf16(fl32(q[idx] * s_b)) with one fp32 scale s_b per block of ``blocksize`` values; returns
    uint16 bit patterns [numel]. The scale is the fp32 absmax itself when the scales are not double
    quantised ("QLoRA, explained", Double quantisation: the baseline that stores fp32 scales), or
    c1' = fl32(e4m3 * c2) from ``dequant_scales`` when they are."""
    codes = np.asarray(codes, dtype=np.float32)
    idx = unpack_nibbles(packed, numel).reshape(-1, blocksize)
    if idx.max(initial=0) >= codes.size:
        raise ValueError("index outside the codebook")
    s = np.asarray(scales, dtype=np.float32).reshape(-1)
    w32 = (codes[idx] * s[:, None]).astype(np.float32)      # one IEEE float32 multiply, RNE
    return bf16_bits_from_f32(w32).reshape(-1)


def storage_bits(blocksize: int = BLOCK, double_quantised: bool = True, group: int = DQ_GROUP) -> float:
    """Bits per parameter: 4-bit index + scale storage ("QLoRA, explained", Double quantisation and
    the toy run's blocksize discussion): fp32 scales cost 32/B; with double quantisation 8/B plus
    32/(B * group)."""
    if double_quantised:
        return 4 + 8 / blocksize + 32 / (blocksize * group)
    return 4 + 32 / blocksize
