"""GPU parity of the FP8 lightning indexer (v4attn_index_score_fp8,
v4attn_index_topk_fp8) against the float64 oracle on the same seeded bytes.

Bars: top-k index sets and their scores bit-exact on integer-valued codes
with unit scales (every product and partial sum is a small integer); on
random codes and scales every visible score within 5e-4 of the absolute sum
A = sum_h |w_h| sq_h sk_j sum_d |q8_hd k8_jd|.  The matrix core does not add
the 64 E4M3 products of one k-step in round-to-nearest fp32: on uniformly
random codes its sum is off by up to 2.9e-4 (median 4e-5) of the largest
product, and the largest product is at most that head's share of A; the
fp32 steps after it add (64 + 2) * 2^-24 A.  Hence 2^-11 A ~ 5e-4 A.  Top-k
sets may differ from the oracle's only among near-ties within the same bar.
"""

import numpy as np
import pytest
import torch

from long_context_sparse_csa_amd import synth
from oracle import codecs
from oracle import indexer as oi

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = 5e-4   # of the absolute sum A (module docstring)


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
    q8 = synth.e4m3_codes((B, Tq, HI, dI), seed, "q8", DEV)
    k8 = synth.e4m3_codes((B, Ncap, dI), seed, "k8", DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    qs = torch.rand((B, Tq, HI), generator=g, device=DEV) * 1.5 + 0.25
    ks = torch.rand((B, Ncap), generator=g, device=DEV) * 1.5 + 0.25
    w = synth.normal((B, Tq, HI), seed, "w", DEV)
    return q8, qs, w, k8, ks


def _integer_inputs(B, Tq, HI, dI, Ncap, seed):
    # integers in [-3, 3] are exact E4M3 values; unit scales
    q8 = synth.integers((B, Tq, HI, dI), -3, 3, seed, "q8", DEV).to(torch.float8_e4m3fn).view(torch.uint8)
    k8 = synth.integers((B, Ncap, dI), -3, 3, seed, "k8", DEV).to(torch.float8_e4m3fn).view(torch.uint8)
    w = synth.integers((B, Tq, HI), -3, 3, seed, "w", DEV)
    return q8, torch.ones((B, Tq, HI), device=DEV), w, k8, torch.ones((B, Ncap), device=DEV)


def _abs_bound(q8, qs, w, k8, ks, V):
    qa = np.abs(codecs.e4m3_decode(q8)) * qs[:, None]
    ka = np.abs(codecs.e4m3_decode(k8[:V])) * ks[:V, None]
    return (ka @ qa.T) @ np.abs(w)


SCORE_CASES = [
    # B, Tq, HI, dI, Ncap, n_entries, q_pos0, m
    (2, 1, 64, 128, 5000, 4999, 19999, 4),    # decode kernel, ragged last chunk
    (1, 3, 20, 64, 3001, 3001, 12000, 4),     # decode kernel, dI = 64, 20 heads, causal rows
    (1, 24, 64, 128, 6000, 6000, 23950, 4),   # query block kernel, causal edge
    (2, 9, 40, 128, 3000, 2990, 11950, 4),    # query block kernel, ragged query block, 40 heads
    (1, 1, 64, 128, 100, 90, 4, 4),           # V_t = 1
]


@pytest.mark.parametrize("case", SCORE_CASES)
def test_index_score_fp8_matches_oracle(case):
    B, Tq, HI, dI, Ncap, n_ent, q_pos0, m = case
    log(f"index_score_fp8 {case}")
    q8, qs, w, k8, ks = _random_inputs(B, Tq, HI, dI, Ncap, sum(case) % 997)
    sc = ops().index_score_fp8(q8, qs, w, k8, ks, n_entries=n_ent, q_pos0=q_pos0, m=m)
    torch.cuda.synchronize()
    got = sc.cpu().numpy()
    q8n, qsn, wn = q8.cpu().numpy(), qs.cpu().double().numpy(), w.cpu().double().numpy()
    k8n, ksn = k8.cpu().numpy(), ks.cpu().double().numpy()
    for b in range(B):
        for r in range(Tq):
            V = oi.visible_entries(q_pos0 + r, n_ent, m)
            want = oi.index_scores_fp8(q8n[b, r], qsn[b, r], wn[b, r], k8n[b], ksn[b], V)
            bound = _abs_bound(q8n[b, r], qsn[b, r], wn[b, r], k8n[b], ksn[b], V)
            err = np.abs(got[b * Tq + r, :V].astype(np.float64) - want)
            assert np.all(err <= TOL * bound + 1e-30), (b, r, float((err / bound).max()))


INT_CASES = [
    # B, Tq, HI, dI, Ncap, n_entries, q_pos0, m, k
    (2, 1, 64, 128, 40000, 40000, 159999, 4, 1024),   # decode kernel, three parts + merge
    (1, 2, 16, 64, 5000, 5000, 19990, 4, 256),        # decode kernel, dI = 64
    (1, 40, 64, 128, 6000, 6000, 23900, 4, 256),      # query block kernel, causal edge
    (2, 16, 40, 128, 20000, 20000, 79990, 4, 1024),   # query block kernel, 40 heads
]


@pytest.mark.parametrize("case", INT_CASES)
def test_index_topk_fp8_bit_exact_on_integer_codes(case):
    B, Tq, HI, dI, Ncap, n_ent, q_pos0, m, k = case
    log(f"index_topk_fp8 int {case}")
    q8, qs, w, k8, ks = _integer_inputs(B, Tq, HI, dI, Ncap, sum(case) % 1000)
    topk, ts = ops().index_topk_fp8(q8, qs, w, k8, ks, n_entries=n_ent, q_pos0=q_pos0, m=m, k=k,
                                    want_scores=True)
    torch.cuda.synchronize()
    got, got_s = topk.cpu().numpy(), ts.cpu().numpy()
    q8n, qsn, wn = q8.cpu().numpy(), qs.cpu().double().numpy(), w.cpu().double().numpy()
    k8n, ksn = k8.cpu().numpy(), ks.cpu().double().numpy()
    for b in range(B):
        want, scores = oi.index_topk_fp8(q8n[b], qsn[b], wn[b], k8n[b], ksn[b], n_ent,
                                         q_pos0 + np.arange(Tq), m, k)
        np.testing.assert_array_equal(got[b], want)
        for r in range(Tq):
            sel = want[r][want[r] >= 0]
            np.testing.assert_array_equal(got_s[b, r, : len(sel)], scores[r][sel])
            assert np.all(np.isneginf(got_s[b, r, len(sel):]))


@pytest.mark.parametrize("Tq", [2, 24])
def test_index_topk_fp8_quantized_rows_near_tie_tolerant(Tq):
    B, HI, dI, N, k = 2, 64, 128, 20000, 1024
    log(f"index_topk_fp8 quantized rows Tq={Tq}")
    q8, qs = synth.e4m3_rows((B, Tq, HI, dI), 7, "q8", DEV)
    k8, ks = synth.e4m3_rows((B, N, dI), 7, "k8", DEV)
    w = synth.normal((B, Tq, HI), 7, "w", DEV)
    q_pos0 = 4 * N - 2
    topk, ts = ops().index_topk_fp8(q8, qs, w, k8, ks, n_entries=N, q_pos0=q_pos0, m=4, k=k,
                                    want_scores=True)
    torch.cuda.synchronize()
    got, got_s = topk.cpu().numpy(), ts.cpu().numpy()
    q8n, qsn, wn = q8.cpu().numpy(), qs.cpu().double().numpy(), w.cpu().double().numpy()
    k8n, ksn = k8.cpu().numpy(), ks.cpu().double().numpy()
    for b in range(B):
        for r in range(Tq):
            V = oi.visible_entries(q_pos0 + r, N, 4)
            sc = oi.index_scores_fp8(q8n[b, r], qsn[b, r], wn[b, r], k8n[b], ksn[b], V)
            bound = _abs_bound(q8n[b, r], qsn[b, r], wn[b, r], k8n[b], ksn[b], V)
            want = oi.topk_select(sc, k)
            g = got[b, r]
            assert np.all(np.diff(g[g >= 0]) > 0), "not ascending"
            tau = np.sort(sc)[::-1][k - 1]
            tol = 2 * TOL * bound.max()
            only_gpu = np.setdiff1d(g, want)
            only_orc = np.setdiff1d(want, g)
            assert np.all(sc[only_gpu] >= tau - tol)
            assert np.all(sc[only_orc] <= tau + tol)
            assert len(only_gpu) <= 0.01 * k
            assert np.all(np.abs(got_s[b, r].astype(np.float64) - sc[g]) <= TOL * bound[g] + 1e-30)


def test_index_score_fp8_decode_shape_sampled():
    """The 1M-context decode shape (8 sequences x 262,144 entries, 64 heads x
    128 dims), in the launch configuration the benchmark times; sampled rows
    and entries against the oracle."""
    B, HI, dI, N = 8, 64, 128, 262144
    q_pos0 = 4 * N - 1
    log("index_score_fp8 decode 8 x 262144")
    q8, qs = synth.e4m3_rows((B, 1, HI, dI), 5, "q8", DEV)
    k8, ks = synth.e4m3_rows((B, N, dI), 5, "k8", DEV)
    w = synth.normal((B, 1, HI), 5, "w", DEV)
    sc = ops().index_score_fp8(q8, qs, w, k8, ks, n_entries=N, q_pos0=q_pos0, m=4)
    torch.cuda.synchronize()
    g = np.random.default_rng(9)
    for b in (0, 5):
        idx = np.sort(np.concatenate([g.choice(N, 4000, replace=False), [0, N - 1]]))
        k8n = k8[b, torch.from_numpy(idx).to(DEV)].cpu().numpy()
        ksn = ks[b, torch.from_numpy(idx).to(DEV)].cpu().double().numpy()
        q8n, qsn, wn = q8[b, 0].cpu().numpy(), qs[b, 0].cpu().double().numpy(), w[b, 0].cpu().double().numpy()
        want = oi.index_scores_fp8(q8n, qsn, wn, k8n, ksn, len(idx))
        bound = _abs_bound(q8n, qsn, wn, k8n, ksn, len(idx))
        got = sc[b, torch.from_numpy(idx).to(DEV)].cpu().double().numpy()
        assert np.all(np.abs(got - want) <= TOL * bound + 1e-30)
