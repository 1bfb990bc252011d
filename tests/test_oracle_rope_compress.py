"""Pins for the oracle's RoPE, RMSNorm and sequence compression.

RoPE is checked against the complex-number form of a rotary embedding, the
inverse and relative-position properties; RMSNorm against torch's rms_norm;
pooling against an independent weight-matrix formulation (brute force over
every (entry, token) pair), sum-to-one, shift invariance, closed forms and
the pages' counting examples."""

import json
import os

import numpy as np
import pytest
import torch

from oracle import compress as oc
from oracle import rope as orope

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def complex_rope(x, pos, R, base):
    """Independent statement: pair (x0, x1) -> (x0 + i x1) * exp(i pos theta)."""
    D = x.shape[-1]
    theta = float(base) ** (-np.arange(0, R, 2, dtype=np.float64) / R)
    z = x[..., D - R::2] + 1j * x[..., D - R + 1::2]
    z = z * np.exp(1j * np.asarray(pos, np.float64)[..., None] * theta)
    y = np.array(x, dtype=np.float64)
    y[..., D - R::2] = z.real
    y[..., D - R + 1::2] = z.imag
    return y


@pytest.mark.parametrize("pos", [0, 1, 7, 4095, 1 << 20, -(1 << 20) - 3])
def test_rope_matches_complex_form(pos):
    g = np.random.default_rng(pos & 0xFFFF)
    x = g.standard_normal((3, 128))
    np.testing.assert_allclose(orope.rope(x, pos, 64, 10000.0),
                               complex_rope(x, pos, 64, 10000.0), atol=1e-12)


def test_rope_fixed_values_and_untouched_dims():
    x = np.zeros(128)
    x[64] = 1.0                      # first rotary pair, theta_0 = 1
    y = orope.rope(x, 1, 64, 10000.0)
    assert y[64] == pytest.approx(np.cos(1.0)) and y[65] == pytest.approx(np.sin(1.0))
    x = np.random.default_rng(3).standard_normal(128)
    y = orope.rope(x, 12345, 64, 10000.0)
    assert np.array_equal(y[:64], x[:64])
    # pair norms preserved
    np.testing.assert_allclose(np.hypot(y[64::2], y[65::2]), np.hypot(x[64::2], x[65::2]))
    # last pair frequency: 10000^(-62/64)
    assert orope.inv_freq(64, 10000.0)[-1] == pytest.approx(10000.0 ** (-62 / 64), rel=1e-15)


def test_rope_inverse_and_relative():
    g = np.random.default_rng(4)
    x, y = g.standard_normal((2, 512))
    for a, b in [(0, 5), (1 << 20, (1 << 20) - 1000), (77, 77)]:
        back = orope.rope(orope.rope(x, a, 64, 1e4), -a, 64, 1e4)
        np.testing.assert_allclose(back, x, atol=1e-12)
        lhs = orope.rope(x, a, 64, 1e4) @ orope.rope(y, b, 64, 1e4)
        rhs = x @ orope.rope(y, b - a, 64, 1e4)
        assert lhs == pytest.approx(rhs, abs=1e-9)


def test_rmsnorm_matches_torch_and_scale_invariance():
    g = np.random.default_rng(5)
    x = g.standard_normal((4, 512)) * 3
    gamma = 1 + 0.1 * g.standard_normal(512)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (512,),
                                       torch.from_numpy(gamma), eps=1e-6).numpy()
    np.testing.assert_allclose(oc.rmsnorm(x, gamma, 1e-6), ref, rtol=1e-12)
    np.testing.assert_allclose(oc.rmsnorm(7.5 * x, gamma, 0.0),
                               oc.rmsnorm(x, gamma, 0.0), rtol=1e-12)


def _pool_bruteforce(c, s, bias, m):
    """Weight matrix A[j, t] over all (entry, token) pairs, rows normalised."""
    T = c.shape[0]
    N = T // m
    A = np.zeros((N, T))
    for j in range(N):
        for t in range(T):
            off = t - (j - 1) * m
            if 0 <= off < 2 * m:
                A[j, t] = np.exp(s[t] + bias[off])
        A[j] /= A[j].sum()
    return A, A @ c


@pytest.mark.parametrize("T,m,D", [(32, 4, 128), (24, 3, 64), (32, 8, 128), (9, 1, 64)])
def test_pool_matches_bruteforce(T, m, D):
    g = np.random.default_rng(T * 10 + m)
    c = g.standard_normal((T, D))
    s = g.standard_normal(T)
    bias = 0.1 * g.standard_normal(2 * m)
    gamma = 1 + 0.1 * g.standard_normal(D)
    A, pooled = _pool_bruteforce(c, s, bias, m)
    js, e = oc.compress_pool(c, s, 0, m, bias, gamma, 1e-6, 64, 1e4)
    assert list(js) == list(range(T // m))
    ref = np.stack([complex_rope(torch.nn.functional.rms_norm(
        torch.from_numpy(pooled[j]), (D,), torch.from_numpy(gamma), eps=1e-6).numpy(),
        j * m, 64, 1e4) for j in range(T // m)])
    np.testing.assert_allclose(e, ref, rtol=1e-11, atol=1e-12)
    # each row of A is a 2m-wide window ending at the group's last token
    for j in range(T // m):
        nz = np.nonzero(A[j])[0]
        assert nz[-1] == (j + 1) * m - 1 and nz[0] == max(0, (j - 1) * m)


@pytest.mark.parametrize("m", [4, 128])
def test_weights_sum_to_one_and_shift_invariant(m):
    g = np.random.default_rng(m)
    T = 4 * m
    s = g.standard_normal(T)
    bias = 0.1 * g.standard_normal(2 * m)
    for j in range(T // m):
        pos, a = oc.pool_weights(s, bias, j, m)
        assert a.sum() == pytest.approx(1.0, abs=1e-14)
        assert len(pos) == (m if j == 0 else 2 * m)
        _, a2 = oc.pool_weights(s + 3.7, bias, j, m)
        np.testing.assert_allclose(a, a2, rtol=1e-12)


def test_closed_form_group_mean_and_single_token():
    g = np.random.default_rng(9)
    m, D, T = 4, 128, 16
    c = g.standard_normal((T, D))
    s = np.zeros(T)
    bias = np.concatenate([np.full(m, -np.inf), np.zeros(m)])
    gamma = np.ones(D)
    js, e = oc.compress_pool(c, s, 0, m, bias, gamma, 1e-6, 64, 1e4)
    for j in js:
        mean = c[j * m:(j + 1) * m].mean(axis=0)
        np.testing.assert_allclose(e[j], orope.rope(oc.rmsnorm(mean, gamma, 1e-6), j * m, 64, 1e4),
                                   rtol=1e-12)
    # m = 1 with bias (-inf, 0): entry j is token j's own window row
    js, e = oc.compress_pool(c, g.standard_normal(T), 0, 1, np.array([-np.inf, 0.0]),
                             gamma, 1e-6, 64, 1e4)
    np.testing.assert_allclose(e, oc.compress_pack(c, 0, gamma, 1e-6, 64, 1e4), rtol=1e-12)


def test_streaming_equals_batch():
    g = np.random.default_rng(11)
    m, D, T = 4, 64, 40
    c = g.standard_normal((T, D))
    s = g.standard_normal(T)
    bias = g.standard_normal(2 * m) * 0.1
    gamma = np.ones(D)
    _, batch = oc.compress_pool(c, s, 0, m, bias, gamma, 1e-6, 32, 1e4)
    for j in range(T // m):
        lo = (j - 1) * m
        rows = c[max(lo, 0):(j + 1) * m]
        js, e = oc.compress_pool(rows, s[max(lo, 0):(j + 1) * m], max(lo, 0), m,
                                 bias, gamma, 1e-6, 32, 1e4, j0=j, n=1)
        assert list(js) == [j]
        np.testing.assert_array_equal(e[0], batch[j])


def test_entries_written_ranges():
    assert oc.entries_written(0, 4096, 4) == (0, 1024)
    assert oc.entries_written(-4, 8, 4) == (0, 1)          # decode, entry 0
    P = 1 << 20
    assert oc.entries_written(P - 4, 4100, 4) == (P // 4, P // 4 + 1024)
    assert oc.entries_written(P - 128, 4224, 128) == (P // 128, P // 128 + 32)
    assert oc.entries_written(8, 4, 4) == (3, 3)           # window incomplete


def test_page_counting_examples():
    with open(os.path.join(GOLDEN, "entry_counts.json")) as f:
        gold = json.load(f)
    for case in gold["cases"]:
        want = case.get("entries_floor", case["entries"])
        assert oc.entry_count(case["tokens"], case["m"]) == want, case["source"]
        # the page's own figure is within rounding of the count
        assert abs(case["tokens"] / case["m"] - case["entries"]) < 1
    ws = gold["window_share"]
    assert round(100 * ws["window"] / ws["tokens"], 3) == ws["percent"]


def test_index_key_pooling_weights_are_the_entry_weights():
    # pooling a constant key stream gives the constant (weights sum to 1);
    # a one-hot stream at position p gives entry j's weight of p, read from
    # the pinned pool_weights; adding a constant to every score changes
    # nothing
    from oracle import compress as occ
    g = np.random.default_rng(3)
    m, L, dI = 4, 24, 8
    s = g.normal(size=L)
    bias = g.normal(0, 0.3, size=2 * m)
    js = np.arange(0, L // m)
    const = np.tile(g.normal(size=dI), (L, 1))
    assert np.allclose(occ.pool_index_keys(const, s, 0, m, bias, js), const[: len(js)], atol=1e-13)

    class _S:
        def __getitem__(self, q):
            return s[q]

    for p in (0, 5, 11):
        onehot = np.zeros((L, dI))
        onehot[p, 0] = 1.0
        got = occ.pool_index_keys(onehot, s, 0, m, bias, js)[:, 0]
        for r, j in enumerate(js):
            pos, alpha = occ.pool_weights(_S(), bias, j, m)
            want = alpha[list(pos).index(p)] if p in pos else 0.0
            assert abs(got[r] - want) < 1e-15
    kI = g.normal(size=(L, dI))
    assert np.allclose(occ.pool_index_keys(kI, s + 3.0, 0, m, bias, js),
                       occ.pool_index_keys(kI, s, 0, m, bias, js), atol=1e-13)
