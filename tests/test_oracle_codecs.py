"""Pins for the oracle's E4M3FN / bf16 codecs: torch's own casts (a library
routine), the OCP format's published constants, ties-to-even at every
midpoint, saturation, and round trips."""

import numpy as np
import pytest
import torch

from oracle import codecs


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = codecs.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2                      # 0x7F and 0xFF only
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zeros
    assert np.signbit(ours[0x80]) and not np.signbit(ours[0x00])


def test_e4m3_published_constants():
    dec = codecs.e4m3_decode
    assert dec(0x7E) == 448.0                  # largest finite
    assert dec(0x08) == 2.0 ** -6              # smallest normal
    assert dec(0x01) == 2.0 ** -9              # smallest subnormal
    assert dec(0x38) == 1.0                    # exponent field 7 = bias
    assert dec(0xB8) == -1.0


def test_e4m3_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    back = codecs.e4m3_encode(codecs.e4m3_decode(codes))
    assert np.array_equal(back, codes)


def test_e4m3_midpoints_round_to_even():
    vals = codecs.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2          # exact in float64
    enc = codecs.e4m3_encode(mids)
    lo = np.arange(0x7E)
    expect = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(enc.astype(int), expect)
    assert np.array_equal(codecs.e4m3_encode(-mids).astype(int), expect | 0x80)
    # a hair above / below a midpoint goes to the nearer code
    assert np.array_equal(codecs.e4m3_encode(np.nextafter(mids, np.inf)),
                          (lo + 1).astype(np.uint8))
    assert np.array_equal(codecs.e4m3_encode(np.nextafter(mids, -np.inf)),
                          lo.astype(np.uint8))


def test_e4m3_saturates():
    enc = codecs.e4m3_encode(np.array([448.0, 463.9, 464.0, 1e4, -1e9, np.inf]))
    assert list(enc) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x7E]
    assert codecs.e4m3_encode(np.array([np.nan]))[0] == 0x7F


def test_e4m3_encode_matches_torch_in_range():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(200_000) * s
                        for s in (1e-3, 0.05, 1.0, 30.0, 200.0)])
    x = x[np.abs(x) < 440].astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codecs.e4m3_encode(x.astype(np.float64)), ref)


def test_bf16_decode_and_encode_match_torch():
    g = np.random.default_rng(1)
    bits = g.integers(0, 1 << 16, 100_000).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]     # finite only
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(codecs.bf16_decode(bits), ref)
    x = (g.standard_normal(1_000_000) * np.exp(g.uniform(-20, 20, 1_000_000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(codecs.bf16_encode(x.astype(np.float64)), ref)


def test_bf16_midpoints_and_direct_rounding():
    # 1 + 2^-8 is the midpoint of 1 and 1 + 2^-7: ties to even -> 1.0
    assert codecs.bf16_encode(np.array([1.0 + 2.0 ** -8]))[0] == 0x3F80
    # 1 + 3*2^-8 is the midpoint of 1+2^-7 (odd) and 1+2^-6: -> 1+2^-6
    assert codecs.bf16_encode(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 0x3F82
    # just above the first midpoint by less than a float32 ulp: rounding from
    # the exact float64 value must go up (a float32 detour would tie to even)
    assert codecs.bf16_encode(np.array([1.0 + 2.0 ** -8 + 2.0 ** -40]))[0] == 0x3F81


@pytest.mark.parametrize("D,R", [(128, 64), (512, 64)])
def test_pack_unpack_roundtrip(D, R):
    g = np.random.default_rng(2)
    v = g.standard_normal((7, D))
    rows = codecs.pack_rows(v, R)
    assert rows.shape == (7, D + R) and rows.dtype == np.uint8
    back = codecs.unpack_rows(rows, D, R)
    assert np.array_equal(codecs.pack_rows(back, R), rows)
    # FP8 part within half an E4M3 quantum, bf16 part within half a bf16 ulp
    q8 = np.ldexp(1.0, np.maximum(np.frexp(np.abs(v[:, :D - R]))[1] - 1, -6) - 3)
    assert np.all(np.abs(back[:, :D - R] - v[:, :D - R]) <= q8 / 2)
    qb = np.ldexp(1.0, np.frexp(np.abs(v[:, D - R:]))[1] - 1 - 7)
    assert np.all(np.abs(back[:, D - R:] - v[:, D - R:]) <= qb / 2)
    # layout: bf16 little-endian after the D-R fp8 bytes
    lo_byte, hi_byte = rows[0, D - R], rows[0, D - R + 1]
    assert (int(hi_byte) << 8 | int(lo_byte)) == codecs.bf16_encode(v[0, D - R])


# ---------------------------------------------------------------- MXFP4 --
# The OCP Microscaling (MX) v1.0 element table for FP4 E2M1 (magnitudes of
# codes 0..7; bit 3 is the sign) and the E8M0 scale (2^(x-127), 255 = NaN).
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_decode_matches_the_element_table():
    v = codecs.e2m1_decode(np.arange(16))
    assert v[:8].tolist() == E2M1_TABLE
    assert v[8:].tolist() == [-x for x in E2M1_TABLE]
    assert np.signbit(v[8])          # code 8 is -0


def test_e8m0_decode():
    v = codecs.e8m0_decode(np.array([0, 1, 126, 127, 128, 254, 255], dtype=np.uint8))
    assert v[:6].tolist() == [2.0 ** -127, 2.0 ** -126, 0.5, 1.0, 2.0, 2.0 ** 127]
    assert np.isnan(v[6])


def test_mxfp4_decode_nibble_order_and_block_scales():
    # 64 elements: bytes 0..31; element 2i is the low nibble of byte i.
    # Block 0 (elements 0..31) scaled by 2^1, block 1 (32..63) by 2^-2.
    packed = np.zeros(32, dtype=np.uint8)
    packed[0] = 0x72      # elements 0, 1 = 1.0, 6.0
    packed[15] = 0xA3     # elements 30, 31 = 1.5, -1.0
    packed[16] = 0x0D     # elements 32, 33 = -3.0, 0.0
    got = codecs.mxfp4_decode(packed, np.array([128, 125], dtype=np.uint8))
    want = np.zeros(64)
    want[0], want[1], want[30], want[31] = 2.0, 12.0, 3.0, -2.0
    want[32] = -0.75
    assert np.array_equal(got, want)
