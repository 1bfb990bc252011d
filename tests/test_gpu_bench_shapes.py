"""GPU parity at the shapes and launch configurations the benchmark times,
on sampled outputs the float64 oracle computes one by one.

  * HCA decode at a 1M-token context: 32 sequences x 8,192 entries + the
    128-row window at t = 2^20 - 1 (8 key-range splits of 9 tiles each, the
    in-split online softmax and the split merge);
  * the 4096-token prefill chunk on a 2^20-token context: HCA attention over
    ~8.2K entries (one split of ~66 tiles per query) and CSA attention over
    1,024 selected of ~263K entries (one split of 9 tiles per query);
  * the bf16 lightning indexer at the 1M decode shape (8 x 262,144 entries)
    and its top-k;
  * the prefill indexer + top-k at 4096 queries x ~263K entries, whose fp32
    score buffer passes 2^32 bytes (rows beyond it are sampled);
  * the ragged HCA decode batch (32 sequences of 256 to 8,192 visible
    entries, each with its own split count).

Bars as everywhere: attention rel-L2 <= 5e-3 and max-abs <= 2e-2 plus half
the bf16 spacing at the case's largest |out| (helpers.assert_attn_close) per
sampled query; scores within fp32 rounding of the float64 sum; top-k sets
equal to the oracle's up to near-ties at the threshold."""

import numpy as np
import pytest
import torch

from long_context_sparse_csa_amd import synth
from long_context_sparse_csa_amd.configs import CSA_1M, HCA_1M, PREFILL_1M
from oracle import attend as oa
from oracle import indexer as oi

from helpers import assert_attn_close, bf16_to_f64, rows_to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from long_context_sparse_csa_amd import ops
    ops.lib()
    yield


def ops():
    from long_context_sparse_csa_amd import ops as o
    return o


def log(msg):
    print(msg, flush=True)


def _attend_one(q_bh, rows, gamma, sink, t, scale, D):
    out, _, lse = oa.attend_rows(q_bh, gamma, t, rows, sink, scale, 1e-6, 64, 1e4)
    return out, lse


# ------------------------------------------------------------ HCA decode 1M --

@pytest.mark.parametrize("scale_mult", [1.0, 4.0])
def test_hca_decode_1m_sampled(scale_mult):
    """32 x 8,192 entries at t = 2^20 - 1: every split runs several tiles."""
    h = HCA_1M
    B, H, D, R, W, m = h.B, h.H, h.D, h.R, h.W, h.m
    N, t = h.T // m, h.T - 1
    log(f"hca decode 1M B={B} N={N} scale x{scale_mult}")
    ent = synth.packed_rows((B, N), D, R, h.seed, "entries", DEV)
    win = synth.packed_rows((B, W), D, R, h.seed, "win", DEV)
    q = synth.normal((B, 1, H, D), h.seed, "q", DEV, dtype=torch.bfloat16)
    gq = synth.normal((D,), h.seed, "gamma_q", DEV, mean=1.0, std=0.1)
    sink = synth.normal((H,), h.seed, "sink", DEV)
    scale = scale_mult * D ** -0.5
    ws_bytes = ops().hca_attend_workspace_bytes(B, 1, H, D, N, m, t, W)
    assert ws_bytes > 0, "the benchmarked launch splits every query's rows"
    out, lse = ops().hca_attend(q, ent, win, gq, sink, n_entries=N, m=m, q_pos0=t, W=W,
                                scale=scale, want_lse=True)
    torch.cuda.synchronize()
    gqn, sk = gq.cpu().double().numpy(), sink.cpu().double().numpy()
    for b in (0, 13, 31):
        rows = np.concatenate([rows_to_f64(ent[b], D, R), rows_to_f64(win[b], D, R)])
        o, l = _attend_one(bf16_to_f64(q[b, 0]), rows, gqn, sk, t, scale, D)
        ma, rl = assert_attn_close(bf16_to_f64(out[b, 0]), o, f"hca 1M b={b}")
        log(f"  b={b} max_abs {ma:.2e} rel_l2 {rl:.2e}")
        np.testing.assert_allclose(lse[b, 0].cpu().numpy(), l, rtol=2e-3, atol=2e-3)


# ------------------------------------------------------- prefill attention --

def _prefill_attn_inputs():
    p = PREFILL_1M
    P, Tq, H, D, R, W = p.T, p.Tq, p.H, p.D, p.R, p.W
    q = synth.normal((1, Tq, H, D), p.seed, "q", DEV, dtype=torch.bfloat16)
    win = synth.packed_rows((1, Tq + W - 1), D, R, p.seed, "win", DEV)
    gq = synth.normal((D,), p.seed, "gamma_q", DEV, mean=1.0, std=0.1)
    sink = synth.normal((H,), p.seed, "sink", DEV)
    return p, q, win, gq, sink


SAMPLE_Q = (0, 1, 127, 128, 2047, 2048, 4094, 4095)


def test_hca_prefill_4096_on_1m_sampled():
    """4096 queries at positions 2^20 .. 2^20 + 4095 over ~8.2K causal HCA
    entries (V_t grows every 128 queries) plus the causal window."""
    p, q, win, gq, sink = _prefill_attn_inputs()
    P, Tq, H, D, R, W, mh = p.T, p.Tq, p.H, p.D, p.R, p.W, p.extra["m_hca"]
    Nh = P // mh + Tq // mh
    log(f"hca prefill Tq={Tq} N={Nh}")
    ent = synth.packed_rows((1, Nh), D, R, p.seed, "entries_h", DEV)
    out, lse = ops().hca_attend(q, ent, win, gq, sink, n_entries=Nh, m=mh, q_pos0=P, W=W,
                                want_lse=True)
    torch.cuda.synchronize()
    en, wn = rows_to_f64(ent[0], D, R), rows_to_f64(win[0], D, R)
    gqn, sk = gq.cpu().double().numpy(), sink.cpu().double().numpy()
    for r in SAMPLE_Q:
        t = P + r
        V = min(Nh, (t + 1) // mh)
        rows = np.concatenate([en[:V], oa.window_rows(wn, t, P, W)])
        o, l = _attend_one(bf16_to_f64(q[0, r]), rows, gqn, sk, t, p.scale, D)
        ma, rl = assert_attn_close(bf16_to_f64(out[0, r]), o, f"hca prefill r={r}")
        log(f"  r={r} V={V} max_abs {ma:.2e} rel_l2 {rl:.2e}")
        np.testing.assert_allclose(lse[0, r].cpu().numpy(), l, rtol=2e-3, atol=2e-3)


def _spread_topk(Tq, k, vis, seed):
    """Sorted distinct entries per query, one drawn from each of k equal
    ranges of its visible entries (a stand-in selection over the whole row)."""
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    step = (vis // k)[:, None]                                   # [Tq, 1]
    off = (torch.rand((Tq, k), generator=g, device=DEV) * step).long()
    sel = torch.arange(k, device=DEV)[None] * step + off
    return sel.to(torch.int32)[None].contiguous()


def test_csa_prefill_4096_on_1m_sampled():
    """4096 queries, each over 1,024 entries spread across its ~263K visible
    ones plus the causal window (9 tiles in one split per query)."""
    p, q, win, gq, sink = _prefill_attn_inputs()
    P, Tq, H, D, R, W, k, m = p.T, p.Tq, p.H, p.D, p.R, p.W, p.k, p.m
    Nc = P // m + Tq // m
    log(f"csa prefill Tq={Tq} N={Nc}")
    ent = synth.packed_rows((1, Nc), D, R, p.seed, "entries", DEV, chunk_rows=1 << 18)
    vis = torch.clamp((P + torch.arange(Tq, device=DEV) + 1) // m, max=Nc)
    topk = _spread_topk(Tq, k, vis, 17)
    out, lse = ops().csa_attend(q, ent, topk, win, gq, sink, q_pos0=P, W=W, want_lse=True)
    torch.cuda.synchronize()
    tk = topk[0].cpu().numpy()
    wn = rows_to_f64(win[0], D, R)
    gqn, sk = gq.cpu().double().numpy(), sink.cpu().double().numpy()
    for r in SAMPLE_Q:
        t = P + r
        sel = torch.from_numpy(tk[r].astype(np.int64)).to(DEV)
        rows = np.concatenate([rows_to_f64(ent[0, sel], D, R), oa.window_rows(wn, t, P, W)])
        o, l = _attend_one(bf16_to_f64(q[0, r]), rows, gqn, sk, t, p.scale, D)
        ma, rl = assert_attn_close(bf16_to_f64(out[0, r]), o, f"csa prefill r={r}")
        log(f"  r={r} max_abs {ma:.2e} rel_l2 {rl:.2e}")
        np.testing.assert_allclose(lse[0, r].cpu().numpy(), l, rtol=2e-3, atol=2e-3)


# -------------------------------------------------------------- indexer ---

def _score_bound(q, w, k):
    """sum_h |w_h| sum_d |q_hd k_d| per entry: the scale of fp32 rounding."""
    return np.abs(k) @ np.abs(q).T @ np.abs(w)


def _check_topk_near_ties(got, sc, k, bound):
    want = oi.topk_select(sc, k)
    assert np.all(np.diff(got[got >= 0]) > 0), "not ascending"
    tau = np.sort(sc)[::-1][k - 1]
    tol = 1e-5 * bound.max()
    only_gpu = np.setdiff1d(got, want)
    only_orc = np.setdiff1d(want, got)
    assert np.all(sc[only_gpu] >= tau - tol), "a GPU-only entry is below the threshold"
    assert np.all(sc[only_orc] <= tau + tol), "an oracle-only entry is above the threshold"
    assert len(only_gpu) <= 0.01 * k
    return len(only_gpu)


def test_index_score_bf16_decode_1m_sampled():
    """8 sequences x 262,144 entries, 64 heads x 128 dims (the launch the
    benchmark times); every score of two sampled sequences, and their top-k."""
    c = CSA_1M
    B, HI, dI, N, k = c.B, c.HI, c.dI, c.T // c.m, c.k
    t = c.T - 1
    log(f"index_score bf16 decode B={B} N={N}")
    q = synth.normal((B, 1, HI, dI), c.seed, "qI", DEV, dtype=torch.bfloat16)
    w = synth.normal((B, 1, HI), c.seed, "w", DEV)
    kk = synth.normal((B, N, dI), c.seed, "kI", DEV, dtype=torch.bfloat16)
    sc = ops().index_score(q, w, kk, n_entries=N, q_pos0=t, m=c.m)
    topk, ts = ops().index_topk(q, w, kk, n_entries=N, q_pos0=t, m=c.m, k=k, want_scores=True)
    torch.cuda.synchronize()
    for b in (0, 7):
        qn, wn, kn = bf16_to_f64(q[b, 0]), w[b, 0].cpu().double().numpy(), bf16_to_f64(kk[b])
        want = oi.index_scores(qn, wn, kn, N)
        bound = _score_bound(qn, wn, kn)
        got = sc[b, :N].cpu().double().numpy()
        # fp32 products of bf16 values are exact; 128-term dot products and
        # the 64-head sum add at most ~(128 + 64) 2^-24 of the bound
        assert np.all(np.abs(got - want) <= 2.0 ** -12 * bound), "score beyond fp32 rounding"
        g = topk[b, 0].cpu().numpy()
        n_diff = _check_topk_near_ties(g, want, k, bound)
        log(f"  b={b}: {n_diff} near-tie swaps")
        np.testing.assert_array_equal(ts[b, 0].cpu().numpy(), sc[b, g.astype(np.int64)].cpu().numpy())


def test_prefill_index_topk_4096_on_1m_sampled_past_4gib():
    """4096 queries x ~263K entries: the fp32 score workspace is larger than
    2^32 bytes; sampled rows on both sides of that offset."""
    p = PREFILL_1M
    P, Tq, HI, dI, k, m = p.T, p.Tq, p.HI, p.dI, p.k, p.m
    Nc = P // m + Tq // m
    log(f"prefill index_topk Tq={Tq} N={Nc}")
    stride = ops().score_stride(Tq, Nc, P, m)
    assert Tq * stride * 4 > (1 << 32), "the score buffer should pass 4 GiB"
    q = synth.normal((1, Tq, HI, dI), p.seed, "qI", DEV, dtype=torch.bfloat16)
    w = synth.normal((1, Tq, HI), p.seed, "w", DEV)
    kk = synth.normal((1, Nc, dI), p.seed, "kI", DEV, dtype=torch.bfloat16)
    topk, ts = ops().index_topk(q, w, kk, n_entries=Nc, q_pos0=P, m=m, k=k, want_scores=True)
    torch.cuda.synchronize()
    kn = bf16_to_f64(kk[0])
    first_past = -(-(1 << 32) // (stride * 4))
    rows = sorted({0, 2048, first_past - 1, first_past, 4090, Tq - 1})
    for r in rows:
        t = P + r
        V = oi.visible_entries(t, Nc, m)
        qn, wn = bf16_to_f64(q[0, r]), w[0, r].cpu().double().numpy()
        sc = oi.index_scores(qn, wn, kn, V)
        bound = _score_bound(qn, wn, kn[:V])
        g = topk[0, r].cpu().numpy()
        n_diff = _check_topk_near_ties(g, sc, k, bound)
        got_s = ts[0, r].cpu().double().numpy()
        assert np.all(np.abs(got_s - sc[g]) <= 2.0 ** -12 * bound[g]), f"row {r}: scores"
        log(f"  r={r} V={V} byte offset {r * stride * 4}: {n_diff} near-tie swaps")


def test_hca_ragged_decode_sampled():
    """The ragged decode batch the benchmark times: 32 sequences at positions
    (b + 1) 2^15 - 1 (256 to 8,192 visible entries), each with its own split
    count; sampled sequences against the oracle."""
    h = HCA_1M
    B, H, D, R, W, m = h.B, h.H, h.D, h.R, h.W, h.m
    N = h.T // m
    pos = [(b + 1) * (1 << 15) - 1 for b in range(B)]
    log(f"hca ragged decode B={B}")
    ent = synth.packed_rows((B, N), D, R, h.seed, "entries", DEV)
    win = synth.packed_rows((B, W), D, R, h.seed, "win", DEV)
    q = synth.normal((B, 1, H, D), h.seed, "q", DEV, dtype=torch.bfloat16)
    gq = synth.normal((D,), h.seed, "gamma_q", DEV, mean=1.0, std=0.1)
    sink = synth.normal((H,), h.seed, "sink", DEV)
    out, lse = ops().hca_attend(q, ent, win, gq, sink, n_entries=N, m=m, W=W, seq_pos=pos,
                                want_lse=True)
    torch.cuda.synchronize()
    gqn, sk = gq.cpu().double().numpy(), sink.cpu().double().numpy()
    for b in (0, 1, 15, 31):
        t = pos[b]
        V = min(N, (t + 1) // m)
        rows = np.concatenate([rows_to_f64(ent[b, :V], D, R), rows_to_f64(win[b], D, R)])
        o, l = _attend_one(bf16_to_f64(q[b, 0]), rows, gqn, sk, t, h.scale, D)
        ma, rl = assert_attn_close(bf16_to_f64(out[b, 0]), o, f"hca ragged b={b}")
        log(f"  b={b} V={V} max_abs {ma:.2e} rel_l2 {rl:.2e}")
        np.testing.assert_allclose(lse[b, 0].cpu().numpy(), l, rtol=2e-3, atol=2e-3)
