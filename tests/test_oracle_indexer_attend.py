"""Pins for the oracle's indexer, top-k and attention.

Indexer: exact integer arithmetic against pure-Python loops.  Top-k: the
rank definition checked pair by pair (brute force), ties to the lower index,
"below the budget nothing is dropped".  Attention: torch's
scaled_dot_product_attention in float64 with an explicit sink column (a
library routine), sink sums, a closed form with identical rows, CSA with k
covering every entry equals dense/HCA, relative-position (shift) invariance
and permutation invariance."""

import numpy as np
import pytest
import torch

from oracle import attend as oa
from oracle import compress as oc
from oracle import indexer as oi

from test_oracle_rope_compress import complex_rope


# ---------------------------------------------------------------- indexer --

def test_index_scores_integer_bruteforce():
    g = np.random.default_rng(0)
    HI, dI, N = 4, 32, 50
    q = g.integers(-3, 4, (HI, dI))
    w = g.integers(-3, 4, HI)
    k = g.integers(-3, 4, (N, dI))
    got = oi.index_scores(q, w, k, N)
    for j in range(N):
        total = 0
        for h in range(HI):
            dot = 0
            for d in range(dI):
                dot += int(q[h, d]) * int(k[j, d])
            total += int(w[h]) * max(dot, 0)
        assert got[j] == total
    # only the first V entries are scored
    assert oi.index_scores(q, w, k, 17).shape == (17,)


# E4M3FN codes of a few exact values (sign bit 0x80; 1.0 = exponent 7, bias 7)
_E4M3 = {0.0: 0x00, 0.5: 0x30, 1.0: 0x38, 1.5: 0x3C, 2.0: 0x40, 3.0: 0x44}


def _code(v):
    return _E4M3[abs(v)] | (0x80 if v < 0 else 0)


def test_index_scores_fp8_hand_example():
    # q = q_scale * q8 = [[2, 4], [-0.5, 0.25]];  k = k_scale * k8 =
    # [[1, -1], [2.25, 1.125], [2, 8]];  w = [1, -2]:
    # j=0: dots -2, -0.75 -> 0;  j=1: 9, -0.84375 -> 9;  j=2: 36, 1 -> 36 - 2 = 34
    q8 = np.array([[_code(1.0), _code(2.0)], [_code(-1.0), _code(0.5)]], dtype=np.uint8)
    k8 = np.array([[_code(1.0), _code(-1.0)], [_code(3.0), _code(1.5)],
                   [_code(0.5), _code(2.0)]], dtype=np.uint8)
    got = oi.index_scores_fp8(q8, np.array([2.0, 0.5]), np.array([1.0, -2.0]), k8,
                              np.array([1.0, 0.75, 4.0]), 3)
    assert got.tolist() == [0.0, 9.0, 34.0]


def test_index_scores_fp8_integer_codes_equal_integer_scores():
    # unit scales and integer codes reduce to the integer indexer above
    g = np.random.default_rng(3)
    HI, dI, N = 4, 64, 40
    q = g.integers(-3, 4, (HI, dI))
    k = g.integers(-3, 4, (N, dI))
    w = g.integers(-3, 4, HI).astype(np.float64)
    enc = np.vectorize(lambda v: _code(float(v)))
    got = oi.index_scores_fp8(enc(q).astype(np.uint8), np.ones(HI), w,
                              enc(k).astype(np.uint8), np.ones(N), N)
    assert np.array_equal(got, oi.index_scores(q, w, k, N))


def test_index_scores_fp8_scales_are_per_row():
    g = np.random.default_rng(4)
    HI, dI, N = 3, 64, 20
    q8 = g.integers(0, 0x7F, (HI, dI)).astype(np.uint8) | (g.integers(0, 2, (HI, dI)) * 0x80).astype(np.uint8)
    k8 = g.integers(0, 0x7F, (N, dI)).astype(np.uint8) | (g.integers(0, 2, (N, dI)) * 0x80).astype(np.uint8)
    qs, ks, w = g.uniform(0.5, 2, HI), g.uniform(0.5, 2, N), g.normal(size=HI)
    base = oi.index_scores_fp8(q8, qs, w, k8, ks, N)
    # a key's scale multiplies its score (positive homogeneity of ReLU)
    ks2 = ks.copy()
    ks2[5] *= 4.0
    s2 = oi.index_scores_fp8(q8, qs, w, k8, ks2, N)
    assert np.isclose(s2[5], 4.0 * base[5], rtol=1e-12)
    assert np.array_equal(np.delete(s2, 5), np.delete(base, 5))
    # a query head's scale acts like a factor on that head's weight
    qs2, w2 = qs.copy(), w.copy()
    qs2[1] *= 8.0
    w2[1] *= 8.0
    assert np.allclose(oi.index_scores_fp8(q8, qs2, w, k8, ks, N),
                       oi.index_scores_fp8(q8, qs, w2, k8, ks, N), rtol=1e-12, atol=0)


# E2M1 codes of exact values (bit 3 is the sign)
_E2M1 = {0.0: 0x0, 0.5: 0x1, 1.0: 0x2, 1.5: 0x3, 2.0: 0x4, 3.0: 0x5, 4.0: 0x6, 6.0: 0x7}


def _pack_e2m1(vals):
    c = np.array([_E2M1[abs(v)] | (8 if v < 0 else 0) for v in np.ravel(vals)], dtype=np.uint8)
    c = c.reshape(*np.shape(vals))
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def test_index_scores_mxfp4_hand_example():
    # d_I = 32 (one block).  q head 0 = 2^1 * [1, 2, 0...], head 1 = 2^0 * [-1, 0.5, 0...];
    # keys (scale 2^-1): k0 = 0.5 * [3, 1, 0...] = [1.5, 0.5], k1 = 0.5 * [-4, 6] = [-2, 3]
    # w = [1, 2]:  j=0: dots 2*1.5 + 4*0.5 = 5, -1.5 + 0.25 -> 0  => 5
    #             j=1: -4 + 12 = 8, 2 + 1.5 = 3.5 => 8 + 7 = 15
    q = np.zeros((2, 32)); q[0, :2] = [1.0, 2.0]; q[1, :2] = [-1.0, 0.5]
    k = np.zeros((2, 32)); k[0, :2] = [3.0, 1.0]; k[1, :2] = [-4.0, 6.0]
    got = oi.index_scores_mxfp4(_pack_e2m1(q), np.array([[128], [127]], dtype=np.uint8),
                                np.array([1.0, 2.0]), _pack_e2m1(k),
                                np.array([[126], [126]], dtype=np.uint8), 2)
    assert got.tolist() == [5.0, 15.0]


def test_index_scores_mxfp4_integer_codes_equal_integer_scores():
    g = np.random.default_rng(5)
    HI, dI, N = 4, 64, 30
    vals = np.array([0.0, 1.0, -1.0, 2.0, -2.0, 3.0, -3.0, 4.0, -4.0, 6.0, -6.0])
    q = g.choice(vals, (HI, dI))
    k = g.choice(vals, (N, dI))
    w = g.integers(-3, 4, HI).astype(np.float64)
    got = oi.index_scores_mxfp4(_pack_e2m1(q), np.full((HI, 2), 127, np.uint8), w,
                                _pack_e2m1(k), np.full((N, 2), 127, np.uint8), N)
    assert np.array_equal(got, oi.index_scores(q, w, k, N))


def test_visible_entries():
    assert oi.visible_entries(4095, 1024, 4) == 1024
    assert oi.visible_entries(4094, 1024, 4) == 1023
    assert oi.visible_entries(2, 1024, 4) == 0
    assert oi.visible_entries((1 << 20) + 4095, 263168, 4) == 263168
    assert oi.visible_entries((1 << 20) + 126, 8224, 128) == 8192


def _topk_by_rank(scores, k):
    """Brute force: j is kept iff fewer than k entries beat it, where i beats
    j when s_i > s_j, or s_i == s_j and i < j."""
    V = len(scores)
    keep = []
    for j in range(V):
        beats = sum(1 for i in range(V)
                    if scores[i] > scores[j] or (scores[i] == scores[j] and i < j))
        if beats < k:
            keep.append(j)
    return keep


@pytest.mark.parametrize("V,k,spread", [(300, 64, 3), (300, 64, 1000), (40, 64, 2),
                                        (64, 64, 1), (1, 4, 0), (129, 128, 0)])
def test_topk_matches_rank_definition(V, k, spread):
    g = np.random.default_rng(V + k + spread)
    s = g.integers(-spread, spread + 1, V).astype(np.float64)
    got = oi.topk_select(s, k)
    want = _topk_by_rank(list(s), k)
    assert list(got[: len(want)]) == want
    assert np.all(got[len(want):] == -1)
    if V <= k:                         # below the budget nothing is dropped
        assert list(got[:V]) == list(range(V))


def test_topk_ties_go_to_lower_index():
    s = np.zeros(10)
    s[7] = 1.0
    assert list(oi.topk_select(s, 3)) == [0, 1, 7]


# --------------------------------------------------------------- attention --

def _setup(H=4, D=128, R=64, n=20, seed=0):
    g = np.random.default_rng(seed)
    return (g.standard_normal((H, D)), 1 + 0.1 * g.standard_normal(D),
            g.standard_normal((n, D)), g.standard_normal(H))


def _sdpa_with_sink(qt, rows, sink, scale):
    """torch SDPA (float64, CPU) over rows plus one zero key/value whose
    additive mask is the sink logit."""
    H, D = qt.shape
    keys = np.concatenate([rows, np.zeros((1, D))])
    mask = np.zeros((H, 1, keys.shape[0]))
    mask[:, 0, -1] = sink
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qt)[:, None, :], torch.from_numpy(keys)[None].expand(H, -1, -1),
        torch.from_numpy(keys)[None].expand(H, -1, -1), attn_mask=torch.from_numpy(mask),
        scale=scale)
    return out[:, 0, :].numpy()


@pytest.mark.parametrize("t", [0, 5, 4095, (1 << 20) - 1])
def test_attend_rows_matches_sdpa_with_sink(t):
    q, gq, rows, sink = _setup(seed=t & 0xFF)
    D = q.shape[1]
    scale = D ** -0.5
    out, p, lse = oa.attend_rows(q, gq, t, rows, sink, scale, 1e-6, 64, 1e4)
    qn = torch.nn.functional.rms_norm(torch.from_numpy(q), (D,), torch.from_numpy(gq),
                                      eps=1e-6).numpy()
    qt = complex_rope(qn, t, 64, 1e4)
    o = _sdpa_with_sink(qt, rows, sink, scale)
    np.testing.assert_allclose(out, complex_rope(o, -t, 64, 1e4), rtol=1e-10, atol=1e-12)
    # lse: log of the full denominator, sink included
    logits = scale * qt @ rows.T
    want = np.log(np.exp(sink) + np.exp(logits).sum(-1))
    np.testing.assert_allclose(lse, want, rtol=1e-12)


def test_sink_sums():
    q, gq, rows, sink = _setup(seed=3)
    _, p, lse = oa.attend_rows(q, gq, 9, rows, np.full(4, -np.inf), 0.1, 1e-6, 64, 1e4)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=1e-13)
    _, p, lse = oa.attend_rows(q, gq, 9, rows, sink, 0.1, 1e-6, 64, 1e4)
    assert np.all(p.sum(-1) < 1.0)
    np.testing.assert_allclose(p.sum(-1), 1.0 - np.exp(sink - lse), rtol=1e-12)
    # no rows at all: weight all on the sink, zero output
    out, p, lse = oa.attend_rows(q, gq, 9, rows[:0], sink, 0.1, 1e-6, 64, 1e4)
    assert np.all(out == 0) and np.allclose(lse, sink)


def test_closed_form_identical_rows():
    g = np.random.default_rng(5)
    H, D, n = 3, 128, 37
    u = g.standard_normal(D)
    u[64:] = 0.0                        # zero rotary dims
    rows = np.tile(u, (n, 1))
    q = g.standard_normal((H, D))
    sink = g.standard_normal(H)
    scale = 0.3
    out, _, _ = oa.attend_rows(q, np.ones(D), 123, rows, sink, scale, 1e-6, 64, 1e4)
    qt = oc.rmsnorm(q, np.ones(D), 1e-6)    # RoPE leaves q . u unchanged here
    a = scale * (qt @ u)
    S = n * np.exp(a) / (n * np.exp(a) + np.exp(sink))
    np.testing.assert_allclose(out, S[:, None] * u[None, :], rtol=1e-12, atol=1e-15)


def _cache(T, m, D, R, seed):
    """Float64 entries and window rows built by the oracle's compressor."""
    g = np.random.default_rng(seed)
    c = g.standard_normal((T, D))
    s = g.standard_normal(T)
    bias = 0.1 * g.standard_normal(2 * m)
    gamma = np.ones(D)
    _, ent = oc.compress_pool(c, s, 0, m, bias, gamma, 1e-6, R, 1e4)
    return c, s, bias, gamma, ent


def test_csa_with_full_k_equals_hca_and_dense():
    T, m, D, R, H, W = 256, 4, 128, 64, 4, 16
    c, s, bias, gamma, ent = _cache(T, m, D, R, 1)
    g = np.random.default_rng(2)
    q = g.standard_normal((1, H, D))
    sink = g.standard_normal(H)
    t = T - 1
    N = ent.shape[0]
    win = oc.compress_pack(c[t - W + 1:t + 1], t - W + 1, gamma, 1e-6, R, 1e4)
    topk = np.arange(N, dtype=np.int32)[None]
    a, la = oa.attend_csa(q, ent, topk, win, np.ones(D), sink, t, W, D ** -0.5, 1e-6, R, 1e4)
    b, lb = oa.attend_hca(q, ent, N, m, win, np.ones(D), sink, t, W, D ** -0.5, 1e-6, R, 1e4)
    np.testing.assert_allclose(a, b, rtol=1e-12)
    np.testing.assert_allclose(la, lb, rtol=1e-12)
    # a permuted top-k list (with -1 holes) gives the same output
    perm = np.random.default_rng(3).permutation(N).astype(np.int32)
    padded = np.concatenate([perm, np.full(7, -1, np.int32)])[None]
    c2, _ = oa.attend_csa(q, ent, padded, win, np.ones(D), sink, t, W, D ** -0.5, 1e-6, R, 1e4)
    np.testing.assert_allclose(c2, a, rtol=1e-12)
    # W = 0 (no window): dense SDPA over every entry
    d, _ = oa.attend_hca(q, ent, N, m, win[:0], np.ones(D), sink, t, 0, D ** -0.5, 1e-6, R, 1e4)
    qt = complex_rope(oc.rmsnorm(q[0], np.ones(D), 1e-6), t, R, 1e4)
    o = _sdpa_with_sink(qt, ent, sink, D ** -0.5)
    np.testing.assert_allclose(d[0], complex_rope(o, -t, R, 1e4), rtol=1e-10, atol=1e-13)


def test_relative_positions_shift_invariance():
    """Shifting every position by a multiple of m leaves the output unchanged:
    the output's inverse rotation removes the absolute position."""
    T, m, D, R, H, W = 128, 4, 128, 64, 3, 8
    g = np.random.default_rng(7)
    c = g.standard_normal((T, D))
    s = g.standard_normal(T)
    bias = 0.1 * g.standard_normal(2 * m)
    q = g.standard_normal((1, H, D))
    sink = g.standard_normal(H)
    outs = []
    for shift in (0, 4 * 1000, 4 * 262144):
        # the same T tokens at positions shift..shift+T-1; entries whose whole
        # 2m window lies in the block (the first one would need older tokens)
        js, ent = oc.compress_pool(c, s, shift, m, bias, np.ones(D), 1e-6, R, 1e4,
                                   j0=shift // m + 1, n=T // m - 1)
        assert js[0] == shift // m + 1
        t = shift + T - 1
        win = oc.compress_pack(c[T - W:], t - W + 1, np.ones(D), 1e-6, R, 1e4)
        topk = np.arange(len(js), dtype=np.int32)[None]   # rows of `ent`
        out, lse = oa.attend_csa(q, ent, topk, win, np.ones(D), sink, t, W, D ** -0.5,
                                 1e-6, R, 1e4)
        outs.append((out, lse))
    for out, lse in outs[1:]:
        np.testing.assert_allclose(out, outs[0][0], rtol=1e-8, atol=1e-9)
        np.testing.assert_allclose(lse, outs[0][1], rtol=1e-12)


def test_window_rows_at_sequence_start():
    D, W = 8, 4
    win = np.arange(2 + W - 1)[:, None] * np.ones(D)   # buffer rows for q_pos0=1, Tq=2
    r0 = oa.window_rows(win, 1, 1, W)                   # t = 1 sees positions 0..1
    assert r0.shape[0] == 2 and r0[0, 0] == 2 and r0[-1, 0] == 3
    r1 = oa.window_rows(win, 2, 1, W)                   # t = 2 sees positions 0..2
    assert r1.shape[0] == 3 and r1[-1, 0] == 4
