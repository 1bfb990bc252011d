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


def assert_attn_close(got, want, what="", logit_mult=1.0):
    """Spec bars (max-abs 2e-2, rel-L2 5e-3) at the standard logit scale
    1/sqrt(D).  Stress cases use logits `logit_mult` times sharper.  The part
    of the error that comes from feeding the matrix cores a bf16 q~ grows
    linearly with the logit scale, while the bf16 rounding of P and of the
    output does not.  A float64 simulation of one 64-head query (bf16 q~, bf16
    P, bf16 output) gives rel-L2 2.6e-3 at 1x and 3.8e-3 at 4x, of which q~
    alone is 3.6e-3, and max-abs 1.5e-2 at 4x, of which the output's own
    rounding is 7.7e-3.  So for stress cases max-abs scales with the
    multiplier and rel-L2 with its square root."""
    max_abs, rel_l2 = err_stats(got, want)
    m = max(1.0, logit_mult)
    bar_abs, bar_rel = MAX_ABS * m, REL_L2 * m ** 0.5
    assert max_abs <= bar_abs and rel_l2 <= bar_rel, \
        f"{what}: max_abs {max_abs:.3e} (<= {bar_abs}), rel_l2 {rel_l2:.3e} (<= {bar_rel})"
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
