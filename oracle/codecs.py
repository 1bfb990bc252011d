"""Storage codecs for packed compressed-KV rows (test infrastructure only).

The cache keeps the rotary dimensions in BF16 and the remaining dimensions in
FP8 ([P4] "The attention stack, and why it is two mechanisms"; [P5] "Two ways
to shrink attention, interleaved").  The pages say only "FP8"; the reading
taken here is the OCP 8-bit E4M3 format ("E4M3FN": exponent bias 7, no
infinities, the single NaN pattern S.1111.111, largest finite 448), with
round-to-nearest-even and saturation to +-448, and no scale factor.

Everything is written from the format definitions:
  e4m3: value = (-1)^s * 2^(e-7) * (1 + f/8)   for e in 1..15 (except NaN)
        value = (-1)^s * 2^-6    * (f/8)       for e == 0
  bf16: the upper 16 bits of an IEEE binary32, i.e. 8 exponent bits (bias
        127) and 7 fraction bits.

The MXFP4 indexer (a next-row variant; [P5] "Two ways to shrink attention,
interleaved": the indexer's attention runs in FP4) reads OCP MX FP4 data:
blocks of 32 E2M1 elements sharing one E8M0 scale,
  e2m1: value = (-1)^s * 2^(e-1) * (1 + m/2)   for e in 1..3
        value = (-1)^s * (m/2)                 for e == 0   (4 bits: s e e m)
  e8m0: scale = 2^(x-127) for x in 0..254 (x = 255 is NaN).
Two E2M1 codes share a byte, the lower-indexed element in the low nibble.

Packed row layout (D dims, last R rotary): bytes [0, D-R) hold E4M3 codes of
dims 0..D-R-1; bytes [D-R, D+R) hold little-endian bf16 of dims D-R..D-1.
"""

import numpy as np

E4M3_MAX = 448.0
_E4M3_NAN = 0x7F


def e4m3_decode(codes):
    """uint8 E4M3FN codes -> float64 values (exact)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = (c >> 7) & 1
    e = (c >> 3) & 0xF
    f = c & 0x7
    normal = np.ldexp(1.0 + f / 8.0, e - 7)
    sub = np.ldexp(f / 8.0, -6)
    v = np.where(e == 0, sub, normal)
    v = np.where((e == 15) & (f == 7), np.nan, v)
    return np.where(sign == 1, -v, v)


# Table of the 127 non-negative finite codes (0x00..0x7E) and their values,
# ascending in both code and value.
_POS_CODES = np.arange(0x7F, dtype=np.uint8)
_POS_VALUES = e4m3_decode(_POS_CODES)


def _round_to_grid(a, emin, mbits):
    """Round non-negative float64 `a` to nearest-even on a binary grid with
    `mbits` fraction bits and minimum normal exponent `emin` (subnormals below
    it share the quantum 2^(emin-mbits)).  Returns float64."""
    a = np.asarray(a, dtype=np.float64)
    _, ex = np.frexp(a)               # a = frac * 2^ex, frac in [0.5, 1)
    e = np.maximum(ex - 1, emin)      # floor(log2 a), clamped to the subnormal range
    q = np.ldexp(1.0, e - mbits)      # quantum of that binade
    return np.rint(a / q) * q         # np.rint rounds half to even


def e4m3_encode(x):
    """float64 -> uint8 E4M3FN codes, round-to-nearest-even, saturating."""
    x = np.asarray(x, dtype=np.float64)
    nan = np.isnan(x)
    sign = np.signbit(x)
    a = np.minimum(np.abs(np.where(nan, 0.0, x)), E4M3_MAX)
    r = np.minimum(_round_to_grid(a, -6, 3), E4M3_MAX)
    idx = np.searchsorted(_POS_VALUES, r)
    assert np.all(_POS_VALUES[idx] == r), "rounded value not on the E4M3 grid"
    code = idx.astype(np.uint8) | np.where(sign, 0x80, 0).astype(np.uint8)
    return np.where(nan, np.uint8(_E4M3_NAN), code).astype(np.uint8)


def e2m1_decode(nibbles):
    """4-bit E2M1 codes (ints 0..15) -> float64 values (exact)."""
    c = np.asarray(nibbles).astype(np.int64)
    sign = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    v = np.where(e == 0, m / 2.0, np.ldexp(1.0 + m / 2.0, e - 1))
    return np.where(sign == 1, -v, v)


def e8m0_decode(x):
    """uint8 E8M0 scale codes -> float64 2^(x-127) (NaN for 255)."""
    x = np.asarray(x, dtype=np.uint8).astype(np.int64)
    return np.where(x == 255, np.nan, np.ldexp(1.0, x - 127))


def mxfp4_decode(packed, scales):
    """MXFP4 rows -> float64 [..., d]: packed uint8 [..., d/2] (element 2i in
    the low nibble of byte i) and E8M0 scales uint8 [..., d/32], one per
    block of 32 consecutive elements."""
    p = np.asarray(packed, dtype=np.uint8)
    lo, hi = p & 0xF, p >> 4
    nib = np.stack([lo, hi], axis=-1).reshape(*p.shape[:-1], 2 * p.shape[-1])
    v = e2m1_decode(nib)
    s = e8m0_decode(scales)
    return v * np.repeat(s, 32, axis=-1)


def bf16_decode(bits):
    """uint16 bf16 bit patterns -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_encode(x):
    """float64 -> uint16 bf16 bits, round-to-nearest-even from the exact
    float64 value (no intermediate float32 rounding).  Finite inputs only."""
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x)
    a = np.abs(x)
    r = _round_to_grid(a, -126, 7)
    r = np.where(sign, -r, r)
    # r is exactly representable in bf16, hence in float32.
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def pack_rows(vals, R):
    """float64 [..., D] -> uint8 [..., D+R] packed rows (E4M3 | bf16 rotary)."""
    vals = np.asarray(vals, dtype=np.float64)
    D = vals.shape[-1]
    lo = e4m3_encode(vals[..., : D - R])
    hi = bf16_encode(vals[..., D - R:]).astype("<u2").view(np.uint8)
    hi = hi.reshape(vals.shape[:-1] + (2 * R,))
    return np.concatenate([lo, hi], axis=-1)


def unpack_rows(rows, D, R):
    """uint8 [..., D+R] packed rows -> float64 [..., D]."""
    rows = np.asarray(rows, dtype=np.uint8)
    assert rows.shape[-1] == D + R
    lo = e4m3_decode(rows[..., : D - R])
    hi_bytes = np.ascontiguousarray(rows[..., D - R:])
    hi = bf16_decode(hi_bytes.view("<u2"))
    return np.concatenate([lo, hi], axis=-1)
