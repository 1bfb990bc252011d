"""Test helpers: byte conversions between torch tensors and the oracle's
numpy inputs, and the comparison rules the parity tests use."""

import numpy as np
import torch

from oracle import codecs


def bf16_to_f64(t):
    """bf16 torch tensor (any device) -> float64 numpy via the oracle decoder."""
    bits = t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    return codecs.bf16_decode(bits)


def rows_to_f64(t, D, R):
    """Packed uint8 rows (any device) -> float64 numpy via the oracle decoder."""
    return codecs.unpack_rows(t.detach().cpu().numpy(), D, R)


def err_stats(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    d = got - want
    max_abs = float(np.max(np.abs(d))) if d.size else 0.0
    denom = float(np.linalg.norm(want))
    rel_l2 = float(np.linalg.norm(d) / denom) if denom > 0 else float(np.linalg.norm(d))
    return max_abs, rel_l2


# Attention tolerance for bf16/fp8 inputs with fp32 accumulation.
MAX_ABS = 2e-2
REL_L2 = 5e-3


def bf16_half_spacing(x):
    """Half the bf16 spacing at magnitude |x|: the largest error of rounding
    an exact value of that size to a bf16 output."""
    a = float(np.max(np.abs(x))) if np.size(x) else 0.0
    if a == 0.0:
        return 0.0
    return 2.0 ** (np.floor(np.log2(a)) - 8)


def assert_attn_close(got, want, what=""):
    """Attention outputs: rel-L2 <= 5e-3 and max-abs <= 2e-2 + half the bf16
    spacing at the largest |out| of the case.

    The output is bf16, so even the exact result rounded to an output is off
    by up to half a spacing; the second term grants exactly that and leaves
    the 2e-2 to the arithmetic.  At the workloads' 1/sqrt(D) logit scale
    |out| stays below 0.5 and the term is at most 1e-3.  With 4x sharper
    logits a few rows dominate, |out| reaches 4-5 (spacing 2^-5), and the
    term is 1.6e-2: measured max-abs 1.5e-2 on 2 queries and 2.0e-2 on 256
    queries (an element whose exact value lies within the kernel's ~1e-3
    relative logit-path error of a rounding midpoint lands on the far
    neighbour), against a float64 model of the kernel's roundings (two-term
    E4M3 q~, bf16 rotary q~, two-term E4M3 probabilities, bf16 output; the
    16-bit split partials add about 2^-15 of a head's largest partial) that
    gives 1.3-1.5e-2 per query."""
    max_abs, rel_l2 = err_stats(got, want)
    bar_abs = MAX_ABS + bf16_half_spacing(want)
    assert max_abs <= bar_abs and rel_l2 <= REL_L2, \
        f"{what}: max_abs {max_abs:.3e} (<= {bar_abs:.3e}), rel_l2 {rel_l2:.3e} (<= {REL_L2})"
    return max_abs, rel_l2


def quantum_e4m3(v):
    a = np.abs(v)
    e = np.maximum(np.frexp(a)[1] - 1, -6)
    return np.ldexp(1.0, e - 3)


def quantum_bf16(v):
    a = np.abs(v)
    e = np.maximum(np.frexp(a)[1] - 1, -126)
    return np.ldexp(1.0, e - 7)


def assert_rows_within_one_ulp(gpu_rows, exact_f64, D, R, min_identical=0.999):
    """Every stored value within one unit in the last place of the exact
    float64 value, and most bytes identical to the oracle's own rounding.

    The kernel computes in fp32, so a rotated value that nearly cancels
    (x0 cos - x1 sin ~ 0) carries an absolute fp32 error of order 2^-24
    times its O(1) operands, which can exceed one bf16 ulp of the tiny
    result: the bf16 bound adds 2^-16 absolute (rows are RMS-normalised)."""
    g = codecs.unpack_rows(gpu_rows, D, R)
    lo_q = quantum_e4m3(exact_f64[..., : D - R])
    hi_q = quantum_bf16(exact_f64[..., D - R:]) + 2.0 ** -16
    assert np.all(np.abs(g[..., : D - R] - exact_f64[..., : D - R]) <= lo_q), "fp8 > 1 ulp"
    assert np.all(np.abs(g[..., D - R:] - exact_f64[..., D - R:]) <= hi_q), "bf16 > 1 ulp"
    want = codecs.pack_rows(exact_f64, R)
    same = np.mean(gpu_rows == want)
    assert same >= min_identical, f"only {same:.5f} of bytes identical"
    return same
