"""GPU parity of the MXFP4 lightning indexer (v4attn_index_score_mxfp4,
v4attn_index_topk_mxfp4) against the float64 oracle on the same seeded bytes.

Bars: top-k index sets and their scores bit-exact on integer-valued E2M1
codes (0, +-1, +-2, +-3, +-4, +-6) with unit scales; on random codes and
scales every visible score within 5e-4 of the absolute sum
A = sum_h |w_h| sum_d |q_hd k_jd| of the dequantised rows (the same
derivation as the FP8 indexer: the matrix core's own summation of one
k-step's 64 products, measured up to ~2^-12 of the largest product, plus
(64 + 1) * 2^-24 A of fp32 steps after it); top-k sets may differ from the
oracle's only among near-ties within that bar."""

import numpy as np
import pytest
import torch

from long_context_sparse_csa_amd import synth
from oracle import codecs
from oracle import indexer as oi

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = 5e-4   # of the absolute sum A (module docstring)

# E2M1 codes of the integers the format holds exactly
_INT_CODES = {0: 0x0, 1: 0x2, 2: 0x4, 3: 0x5, 4: 0x6, 6: 0x7}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from long_context_sparse_csa_amd import ops
    ops.lib()   # raises if the HIP library is missing
    yield


def ops():
    from long_context_sparse_csa_amd import ops as o
    return o


def log(msg):
    print(msg, flush=True)


def _random_inputs(B, Tq, HI, dI, Ncap, seed):
    q4, qs = synth.mxfp4_codes((B, Tq, HI), dI, seed, "q4", DEV)
    k4, ks = synth.mxfp4_codes((B, Ncap), dI, seed, "k4", DEV)
    w = synth.normal((B, Tq, HI), seed, "w", DEV)
    return q4, qs, w, k4, ks


def _integer_codes(shape, d, seed, name):
    vals = synth.integers((*shape, d), 0, 10, seed, name, DEV).to(torch.int64)
    # index 0..10 -> 0, +-1, +-2, +-3, +-4, +-6
    table = torch.tensor([0x0, 0x2, 0xA, 0x4, 0xC, 0x5, 0xD, 0x6, 0xE, 0x7, 0xF], device=DEV)
    c = table[vals]
    return (c[..., 0::2] | (c[..., 1::2] << 4)).to(torch.uint8)


def _integer_inputs(B, Tq, HI, dI, Ncap, seed):
    q4 = _integer_codes((B, Tq, HI), dI, seed, "q4")
    k4 = _integer_codes((B, Ncap), dI, seed, "k4")
    w = synth.integers((B, Tq, HI), -3, 3, seed, "w", DEV)
    qs = torch.full((B, Tq, HI, dI // 32), 127, dtype=torch.uint8, device=DEV)
    ks = torch.full((B, Ncap, dI // 32), 127, dtype=torch.uint8, device=DEV)
    return q4, qs, w, k4, ks


def _abs_bound(q4, qs, w, k4, ks, V):
    qa = np.abs(codecs.mxfp4_decode(q4, qs))
    ka = np.abs(codecs.mxfp4_decode(k4[:V], ks[:V]))
    return (ka @ qa.T) @ np.abs(w)


def _np(*ts):
    return [t.cpu().numpy() if t.dtype == torch.uint8 else t.cpu().double().numpy() for t in ts]


SCORE_CASES = [
    # B, Tq, HI, dI, Ncap, n_entries, q_pos0, m
    (2, 1, 64, 128, 5000, 4999, 19999, 4),    # decode kernel, ragged last chunk
    (1, 3, 20, 64, 3001, 3001, 12000, 4),     # decode kernel, dI = 64, 20 heads, causal rows
    (1, 24, 64, 128, 6000, 6000, 23950, 4),   # query block kernel, causal edge
    (2, 9, 40, 128, 3000, 2990, 11950, 4),    # query block kernel, ragged query block, 40 heads
    (1, 1, 64, 128, 100, 90, 4, 4),           # V_t = 1
]


@pytest.mark.parametrize("case", SCORE_CASES)
def test_index_score_mxfp4_matches_oracle(case):
    B, Tq, HI, dI, Ncap, n_ent, q_pos0, m = case
    log(f"index_score_mxfp4 {case}")
    q4, qs, w, k4, ks = _random_inputs(B, Tq, HI, dI, Ncap, sum(case) % 991)
    sc = ops().index_score_mxfp4(q4, qs, w, k4, ks, n_entries=n_ent, q_pos0=q_pos0, m=m)
    torch.cuda.synchronize()
    got = sc.cpu().numpy()
    q4n, qsn, wn, k4n, ksn = _np(q4, qs, w, k4, ks)
    for b in range(B):
        for r in range(Tq):
            V = oi.visible_entries(q_pos0 + r, n_ent, m)
            want = oi.index_scores_mxfp4(q4n[b, r], qsn[b, r], wn[b, r], k4n[b], ksn[b], V)
            bound = _abs_bound(q4n[b, r], qsn[b, r], wn[b, r], k4n[b], ksn[b], V)
            err = np.abs(got[b * Tq + r, :V].astype(np.float64) - want)
            assert np.all(err <= TOL * bound + 1e-30), (b, r, float((err / np.maximum(bound, 1e-300)).max()))


INT_CASES = [
    # B, Tq, HI, dI, Ncap, n_entries, q_pos0, m, k
    (2, 1, 64, 128, 40000, 40000, 159999, 4, 1024),   # decode kernel, three parts + merge
    (1, 2, 16, 64, 5000, 5000, 19990, 4, 256),        # decode kernel, dI = 64
    (1, 40, 64, 128, 6000, 6000, 23900, 4, 256),      # query block kernel, causal edge
    (2, 16, 40, 128, 20000, 20000, 79990, 4, 1024),   # query block kernel, 40 heads
]


@pytest.mark.parametrize("case", INT_CASES)
def test_index_topk_mxfp4_bit_exact_on_integer_codes(case):
    B, Tq, HI, dI, Ncap, n_ent, q_pos0, m, k = case
    log(f"index_topk_mxfp4 int {case}")
    q4, qs, w, k4, ks = _integer_inputs(B, Tq, HI, dI, Ncap, sum(case) % 1000)
    topk, ts = ops().index_topk_mxfp4(q4, qs, w, k4, ks, n_entries=n_ent, q_pos0=q_pos0, m=m,
                                      k=k, want_scores=True)
    torch.cuda.synchronize()
    got, got_s = topk.cpu().numpy(), ts.cpu().numpy()
    q4n, qsn, wn, k4n, ksn = _np(q4, qs, w, k4, ks)
    for b in range(B):
        want, scores = oi.index_topk_mxfp4(q4n[b], qsn[b], wn[b], k4n[b], ksn[b], n_ent,
                                           q_pos0 + np.arange(Tq), m, k)
        np.testing.assert_array_equal(got[b], want)
        for r in range(Tq):
            sel = want[r][want[r] >= 0]
            np.testing.assert_array_equal(got_s[b, r, : len(sel)], scores[r][sel])
            assert np.all(np.isneginf(got_s[b, r, len(sel):]))


@pytest.mark.parametrize("Tq", [2, 24])
def test_index_topk_mxfp4_quantized_rows_near_tie_tolerant(Tq):
    B, HI, dI, N, k = 2, 64, 128, 20000, 1024
    log(f"index_topk_mxfp4 quantized rows Tq={Tq}")
    q4, qs = synth.mxfp4_rows((B, Tq, HI, dI), 7, "q4", DEV)
    k4, ks = synth.mxfp4_rows((B, N, dI), 7, "k4", DEV)
    w = synth.normal((B, Tq, HI), 7, "w", DEV)
    q_pos0 = 4 * N - 2
    topk, ts = ops().index_topk_mxfp4(q4, qs, w, k4, ks, n_entries=N, q_pos0=q_pos0, m=4, k=k,
                                      want_scores=True)
    torch.cuda.synchronize()
    got, got_s = topk.cpu().numpy(), ts.cpu().numpy()
    q4n, qsn, wn, k4n, ksn = _np(q4, qs, w, k4, ks)
    for b in range(B):
        for r in range(Tq):
            V = oi.visible_entries(q_pos0 + r, N, 4)
            sc = oi.index_scores_mxfp4(q4n[b, r], qsn[b, r], wn[b, r], k4n[b], ksn[b], V)
            bound = _abs_bound(q4n[b, r], qsn[b, r], wn[b, r], k4n[b], ksn[b], V)
            want = oi.topk_select(sc, k)
            g = got[b, r]
            assert np.all(np.diff(g[g >= 0]) > 0), "not ascending"
            tau = np.sort(sc)[::-1][k - 1]
            tol = 2 * TOL * bound.max()
            only_gpu = np.setdiff1d(g, want)
            only_orc = np.setdiff1d(want, g)
            assert np.all(sc[only_gpu] >= tau - tol)
            assert np.all(sc[only_orc] <= tau + tol)
            assert np.all(np.abs(got_s[b, r].astype(np.float64) - sc[g]) <= TOL * bound[g] + 1e-30)


def test_index_score_mxfp4_decode_shape_sampled():
    """The 1M-context decode shape (8 sequences x 262,144 entries, 64 heads x
    128 dims), in the launch configuration the benchmark times; sampled rows
    and entries against the oracle."""
    B, HI, dI, N = 8, 64, 128, 262144
    q_pos0 = 4 * N - 1
    log("index_score_mxfp4 decode 8 x 262144")
    q4, qs = synth.mxfp4_rows((B, 1, HI, dI), 5, "q4", DEV)
    k4, ks = synth.mxfp4_rows((B, N, dI), 5, "k4", DEV)
    w = synth.normal((B, 1, HI), 5, "w", DEV)
    sc = ops().index_score_mxfp4(q4, qs, w, k4, ks, n_entries=N, q_pos0=q_pos0, m=4)
    torch.cuda.synchronize()
    g = np.random.default_rng(9)
    for b in (0, 5):
        idx = torch.from_numpy(np.sort(np.concatenate([g.choice(N, 4000, replace=False),
                                                       [0, N - 1]]))).to(DEV)
        k4n, ksn = k4[b, idx].cpu().numpy(), ks[b, idx].cpu().numpy()
        q4n, qsn, wn = q4[b, 0].cpu().numpy(), qs[b, 0].cpu().numpy(), w[b, 0].cpu().double().numpy()
        want = oi.index_scores_mxfp4(q4n, qsn, wn, k4n, ksn, len(idx))
        bound = _abs_bound(q4n, qsn, wn, k4n, ksn, len(idx))
        got = sc[b, idx].cpu().double().numpy()
        assert np.all(np.abs(got - want) <= TOL * bound + 1e-30)
