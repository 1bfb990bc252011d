"""GPU parity of the attention backward (v4attn_csa_attend_backward,
v4attn_hca_attend_backward) against the float64 oracle's chain rule
(oracle/backward.py), on the same seeded bytes.

The GPU takes the forward's stored outputs (bf16 out, fp32 lse) and enters
bf16 operands into the matrix cores: q~, do = RoPE_t(dout), every row (exact
in bf16), and per row and head p and scale dl (each rounded once, 2^-9
relative).  D_h = dout . out uses the bf16 out (2^-9 relative).  Every
product in a gradient therefore carries at most two roundings of 2^-9 on
top of fp32 accumulation, so each gradient tensor is within
rel-L2 <= 4 * 2^-9 ~ 7.8e-3 of the exact one (the roundings are
independent; the bar allows the sum of four), and element-wise within
3e-2 of the tensor's largest magnitude (a single element can collect the
rounding of a probability that dominates its row).

d_sink_h = -sum_q p_sink D_h is the exception: D_h = dout . out is a signed
sum, so the bf16 rounding of out bounds its error by 2^-9 sum_d |dout out|,
not by 2^-9 |D_h|.  Its bar is element-wise:
|d d_sink_h| <= 2^-8 (sum_q p_sink sum_d |dout_qhd out_qhd| + |d_sink_h|)."""

import re

import numpy as np
import pytest
import torch

from long_context_sparse_csa_amd import synth
from oracle import attend as oa
from oracle import backward as ob

from helpers import bf16_to_f64, rows_to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"
R, EPS, BASE = 64, 1e-6, 1e4
REL_L2 = 4 * 2.0 ** -9
MAX_REL = 3e-2


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


def _close(got, want, what):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    scale = np.abs(want).max()
    err = np.abs(got - want)
    rel = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300)
    log(f"  {what}: rel-L2 {rel:.2e}, max-abs/max {err.max() / max(scale, 1e-300):.2e}")
    assert rel <= REL_L2, (what, rel)
    assert np.all(err <= MAX_REL * scale + 1e-30), (what, float(err.max() / scale))


def _inputs(B, Tq, H, D, Ncap, W, seed):
    q = synth.normal((B, Tq, H, D), seed, "q", DEV, dtype=torch.bfloat16)
    ent = synth.packed_rows((B, Ncap), D, R, seed, "entries", DEV)
    win = synth.packed_rows((B, Tq + W - 1), D, R, seed, "win", DEV)
    gq = synth.normal((D,), seed, "gamma_q", DEV, mean=1.0, std=0.1)
    sink = synth.normal((H,), seed, "sink", DEV)
    dout = synth.normal((B, Tq, H, D), seed, "dout", DEV, dtype=torch.bfloat16)
    return q, ent, win, gq, sink, dout


def _reference(q, ent, win, gq, sink, dout, rows_of, q_pos0, W, scale, D):
    """Oracle gradients, row gradients added per (sequence, row)."""
    B, Tq, H, _ = q.shape
    qn, doutn = bf16_to_f64(q), bf16_to_f64(dout)
    en, wn = rows_to_f64(ent, D, R), rows_to_f64(win, D, R)
    gqn, sk = gq.cpu().double().numpy(), sink.cpu().double().numpy()
    dq = np.zeros((B, Tq, H, D))
    d_ent = np.zeros(en.shape)
    d_win = np.zeros(wn.shape)
    d_sink = np.zeros(H)
    d_gamma = np.zeros(D)
    sink_abs = np.zeros(H)   # sum_q p_sink sum_d |dout out|: the d_sink bar
    for b in range(B):
        for r in range(Tq):
            t = q_pos0 + r
            ent_idx, win_rows = rows_of(b, r, t)
            rows = np.concatenate([en[b][ent_idx], wn[b][win_rows]])
            g_q, g_rows, g_sink, g_gamma = ob.attend_rows_backward(
                qn[b, r], gqn, t, rows, sk, scale, EPS, R, BASE, doutn[b, r])
            dq[b, r] = g_q
            np.add.at(d_ent[b], ent_idx, g_rows[: len(ent_idx)])
            np.add.at(d_win[b], win_rows, g_rows[len(ent_idx):])
            d_sink += g_sink
            d_gamma += g_gamma
            o, _, lse = oa.attend_rows(qn[b, r], gqn, t, rows, sk, scale, EPS, R, BASE)
            sink_abs += np.exp(sk - lse) * np.sum(np.abs(doutn[b, r] * o), axis=1)
    return (dq, d_ent, d_win, d_sink, d_gamma), sink_abs


def _win_rows(t, q_pos0, W):
    base = q_pos0 - (W - 1)
    lo = max(0, t - W + 1)
    return np.arange(lo - base, t + 1 - base)


def _check(got, ref, what):
    want, sink_abs = ref
    names = ("dq", "d_entries", "d_win", "d_sink", "d_gamma_q")
    for n, g, w in zip(names, got, want):
        if n == "d_sink":
            err = np.abs(g.cpu().double().numpy() - w)
            bar = 2.0 ** -8 * (sink_abs + np.abs(w))
            log(f"  {what} d_sink: error <= {float((err / bar).max()):.2f} of the bar")
            assert np.all(err <= bar), (what, float((err / bar).max()))
        else:
            _close(g.cpu().numpy(), w, f"{what} {n}")


CSA_CASES = [
    # B, Tq, H, D, Ncap, k, W, q_pos0, n_valid
    (2, 3, 64, 512, 300, 64, 16, 1000, 60),    # rows shared across queries, -1 padding
    (1, 4, 40, 256, 200, 48, 8, 500, None),    # 40 heads, D = 256
    (2, 1, 64, 512, 4096, 1024, 128, (1 << 20) - 1, None),   # decode shape
    (1, 2, 8, 128, 100, 32, 0, 50, None),      # no window, D = 128
]


@pytest.mark.parametrize("case", CSA_CASES)
def test_csa_attend_backward_matches_oracle(case):
    B, Tq, H, D, Ncap, k, W, q_pos0, nv = case
    log(f"csa backward {case}")
    q, ent, win, gq, sink, dout = _inputs(B, Tq, H, D, Ncap, W, sum(case[:7]) % 991)
    g = torch.Generator().manual_seed(5)
    topk = torch.full((B, Tq, k), -1, dtype=torch.int32)
    for b in range(B):
        for r in range(Tq):
            n = k if nv is None else nv
            topk[b, r, :n] = torch.randperm(Ncap, generator=g)[:n].sort().values.to(torch.int32)
    topk = topk.to(DEV)
    scale = D ** -0.5
    out, lse = ops().csa_attend(q, ent, topk, win, gq, sink, q_pos0=q_pos0, W=W, scale=scale,
                                want_lse=True)
    got = ops().csa_attend_backward(q, ent, topk, win, gq, sink, out, lse, dout, q_pos0=q_pos0,
                                    W=W, scale=scale)
    torch.cuda.synchronize()
    tk = topk.cpu().numpy()

    def rows_of(b, r, t):
        sel = tk[b, r]
        return sel[sel >= 0], (_win_rows(t, q_pos0, W) if W > 0 else np.zeros(0, np.int64))

    want = _reference(q, ent, win, gq, sink, dout, rows_of, q_pos0, W, scale, D)
    _check(got, want, f"csa {case}")


HCA_CASES = [
    # B, Tq, H, D, n_entries, m, W, q_pos0
    (1, 5, 64, 512, 40, 4, 8, 160 - 3),        # causal: V_t changes in the block
    (2, 2, 16, 128, 300, 128, 16, 300 * 128 + 5),
    (2, 1, 64, 512, 1024, 128, 128, (1 << 17) - 1),   # dense decode rows, shared by nothing
]


@pytest.mark.parametrize("case", HCA_CASES)
def test_hca_attend_backward_matches_oracle(case):
    B, Tq, H, D, n_ent, m, W, q_pos0 = case
    log(f"hca backward {case}")
    q, ent, win, gq, sink, dout = _inputs(B, Tq, H, D, n_ent, W, sum(case[:7]) % 983)
    scale = D ** -0.5
    out, lse = ops().hca_attend(q, ent, win, gq, sink, n_entries=n_ent, m=m, q_pos0=q_pos0, W=W,
                                scale=scale, want_lse=True)
    got = ops().hca_attend_backward(q, ent, win, gq, sink, out, lse, dout, n_entries=n_ent, m=m,
                                    q_pos0=q_pos0, W=W, scale=scale)
    torch.cuda.synchronize()

    def rows_of(b, r, t):
        V = min(n_ent, (t + 1) // m)
        return np.arange(V), _win_rows(t, q_pos0, W)

    want = _reference(q, ent, win, gq, sink, dout, rows_of, q_pos0, W, scale, D)
    _check(got, want, f"hca {case}")


def _min_workspace(call):
    """The smallest workspace a call accepts (the per-chunk buffers alone),
    as the V4ATTN_EWORKSPACE error of a call with 16 bytes reports it."""
    with pytest.raises(ops().V4AttnError) as err:
        call(16)
    m = re.search(r"need (\d+)", str(err.value))
    assert err.value.status == -3 and m, str(err.value)
    return int(m.group(1))


def test_csa_backward_row_gradient_paths_match_oracle():
    """The row gradients grouped in one group (the queried workspace), in
    several groups (a byte less: 128 + 32 queries), and added with atomics
    (the per-chunk buffers alone: the smallest workspace accepted), on 160
    queries whose window rows and top-k entries are shared."""
    B, Tq, H, D, Ncap, k, W, q_pos0 = 2, 80, 8, 128, 300, 48, 16, 700
    q, ent, win, gq, sink, dout = _inputs(B, Tq, H, D, Ncap, W, 17)
    g = torch.Generator().manual_seed(9)
    topk = torch.stack([torch.stack([torch.randperm(120, generator=g)[:k].sort().values
                                     for _ in range(Tq)]) for _ in range(B)]).to(torch.int32)
    topk = topk.to(DEV)
    scale = D ** -0.5
    out, lse = ops().csa_attend(q, ent, topk, win, gq, sink, q_pos0=q_pos0, W=W, scale=scale,
                                want_lse=True)
    full = ops().lib().v4attn_csa_attend_backward_workspace(B, Tq, H, D, k, W, Ncap)
    tk = topk.cpu().numpy()

    def rows_of(b, r, t):
        return tk[b, r], _win_rows(t, q_pos0, W)

    want = _reference(q, ent, win, gq, sink, dout, rows_of, q_pos0, W, scale, D)

    def call(nbytes):
        return ops().csa_attend_backward(q, ent, topk, win, gq, sink, out, lse, dout,
                                         q_pos0=q_pos0, W=W, scale=scale, workspace_bytes=nbytes)

    least = _min_workspace(call)
    assert least < full - 1
    for nbytes, what in ((full, "one group"), (full - 1, "two groups"), (least, "atomics")):
        log(f"csa backward row gradients: {what}, workspace {nbytes} of {full} bytes")
        got = call(nbytes)
        torch.cuda.synchronize()
        _check(got, want, f"csa rows {what}")


def _misaligned_zeros(shape):
    """Zeros whose first element sits 4 bytes past a 16-byte boundary."""
    n = int(np.prod(shape))
    return torch.zeros(n + 1, dtype=torch.float32, device=DEV)[1:].view(shape)


def test_backward_misaligned_row_gradients_take_the_atomic_path():
    """Row and key gradients not 16-byte aligned cannot take the grouped
    sum's vector adds: the calls fall back to atomics and still match the
    oracle."""
    B, Tq, H, D, Ncap, k, W, q_pos0 = 1, 6, 16, 128, 100, 24, 8, 300
    q, ent, win, gq, sink, dout = _inputs(B, Tq, H, D, Ncap, W, 31)
    g = torch.Generator().manual_seed(3)
    topk = torch.stack([torch.randperm(40, generator=g)[:k].sort().values
                        for _ in range(Tq)])[None].to(torch.int32).to(DEV)
    scale = D ** -0.5
    out, lse = ops().csa_attend(q, ent, topk, win, gq, sink, q_pos0=q_pos0, W=W, scale=scale,
                                want_lse=True)
    grads = {"d_entries": _misaligned_zeros((B, Ncap, D)),
             "d_win": _misaligned_zeros((B, Tq + W - 1, D))}
    assert grads["d_entries"].data_ptr() % 16 == 4
    got = ops().csa_attend_backward(q, ent, topk, win, gq, sink, out, lse, dout, q_pos0=q_pos0,
                                    W=W, scale=scale, grads=grads)
    torch.cuda.synchronize()
    tk = topk.cpu().numpy()

    def rows_of(b, r, t):
        return tk[b, r], _win_rows(t, q_pos0, W)

    _check(got, _reference(q, ent, win, gq, sink, dout, rows_of, q_pos0, W, scale, D),
           "csa misaligned rows")
    inp = _kl_inputs(1, 5, 8, 64, 90, 64, 40, 41)
    dk = _misaligned_zeros((1, 90, 64))
    got = ops().index_kl_backward(*inp, dk=dk)
    torch.cuda.synchronize()
    _kl_check(got, _kl_reference(*inp))


def test_backward_adds_into_given_gradients():
    """Row, sink and gamma gradients are added to what the buffers hold."""
    B, Tq, H, D, Ncap, k, W, q_pos0 = 1, 2, 16, 128, 64, 16, 4, 100
    q, ent, win, gq, sink, dout = _inputs(B, Tq, H, D, Ncap, W, 3)
    topk = torch.arange(k, dtype=torch.int32, device=DEV).expand(B, Tq, k).contiguous()
    out, lse = ops().csa_attend(q, ent, topk, win, gq, sink, q_pos0=q_pos0, W=W, want_lse=True)
    a = ops().csa_attend_backward(q, ent, topk, win, gq, sink, out, lse, dout, q_pos0=q_pos0, W=W)
    grads = {n: t.clone() for n, t in zip(("dq", "d_entries", "d_win", "d_sink", "d_gamma_q"), a)}
    b = ops().csa_attend_backward(q, ent, topk, win, gq, sink, out, lse, dout, q_pos0=q_pos0, W=W,
                                  grads=grads)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0])                        # dq is written, not added
    for x, y in zip(a[1:], b[1:]):
        assert torch.allclose(y, 2 * x, rtol=1e-5, atol=1e-6)


# ------------------------------------------------------- compressor backward --
# Every input is exact in fp32 (bf16 latents); the kernel works in fp32, so
# each gradient is the float64 one up to fp32 rounding of sums of at most
# D + 2m terms: rel-L2 and max-abs (of the tensor's largest) within 1e-4.

POOL_BWD_CASES = [
    # B, L, D, m, pos0
    (2, 40, 512, 4, 0),        # entry 0 (half window) included
    (1, 4 * 128, 256, 128, 128),
    (2, 96, 128, 16, 32),      # rows start mid-sequence
]


@pytest.mark.parametrize("case", POOL_BWD_CASES)
def test_compress_backward_matches_oracle(case):
    from oracle import compress as oc
    B, L, D, m, pos0 = case
    log(f"compress backward {case}")
    seed = sum(case) % 977
    raw = synth.normal((B, L, D), seed, "raw", DEV, dtype=torch.bfloat16)
    sc = synth.normal((B, L), seed, "score", DEV)
    bias = synth.normal((2 * m,), seed, "bias", DEV, std=0.3)
    gam = synth.normal((D,), seed, "gamma", DEV, mean=1.0, std=0.1)
    j_lo, j_hi = oc.entries_written(pos0, L, m)
    js = np.arange(j_lo, j_hi)
    de = synth.normal((B, len(js), D), seed, "de", DEV)
    got = ops().compress_backward(raw, sc, bias, gam, de, raw_pos0=pos0, m=m, entry0=int(j_lo))
    torch.cuda.synchronize()
    rn, sn = bf16_to_f64(raw), sc.cpu().double().numpy()
    bn, gn, den = bias.cpu().double().numpy(), gam.cpu().double().numpy(), de.cpu().double().numpy()
    d_raw, d_sc = np.zeros((B, L, D)), np.zeros((B, L))
    d_b, d_g = np.zeros(2 * m), np.zeros(D)
    for b in range(B):
        dc, ds, db, dg = ob.compress_pool_backward(rn[b], sn[b], pos0, m, bn, gn, EPS, R, BASE, js,
                                                   den[b])
        d_raw[b], d_sc[b] = dc, ds
        d_b += db
        d_g += dg
    for n, g_, w_ in zip(("d_raw", "d_score", "d_bias", "d_gamma"), got, (d_raw, d_sc, d_b, d_g)):
        g_ = g_.cpu().double().numpy()
        rel = np.linalg.norm(g_ - w_) / np.linalg.norm(w_)
        mx = np.abs(g_ - w_).max() / np.abs(w_).max()
        log(f"  {n}: rel-L2 {rel:.2e}, max-abs/max {mx:.2e}")
        assert rel <= 1e-4 and mx <= 1e-4, n


# ------------------------------------------------------ indexer KL backward --
# q^I.k^I is exact up to fp32 summation (bf16 inputs), so the scores, Q, the
# loss and dw are fp32-accurate (rel 1e-4 allows sums over 4096 entries);
# ds w [q.k > 0] enters the dq and dk products rounded to bf16 (2^-9), so
# dq and dk are within rel-L2 4 * 2^-9 and 3e-2 of their largest element.

KL_CASES = [
    # B, Tq, HI, dI, Ncap, ns, n_valid
    (2, 3, 64, 128, 3000, 1024, 1000),   # -1 padded sets, keys shared across queries
    (1, 4, 40, 64, 500, 256, None),
    (2, 2, 4, 32, 200, 64, 50),          # the tiny indexer shape
]


def _kl_inputs(B, Tq, HI, dI, Ncap, ns, nv, seed):
    qi = synth.normal((B, Tq, HI, dI), seed, "qI", DEV, dtype=torch.bfloat16)
    wi = synth.normal((B, Tq, HI), seed, "w", DEV)
    ki = synth.normal((B, Ncap, dI), seed, "kI", DEV, dtype=torch.bfloat16)
    g = torch.Generator().manual_seed(seed)
    sel = torch.full((B, Tq, ns), -1, dtype=torch.int32)
    for b in range(B):
        for r in range(Tq):
            n = ns if nv is None else nv
            sel[b, r, :n] = torch.randperm(Ncap, generator=g)[:n].sort().values.to(torch.int32)
    tgt = torch.rand((B, Tq, ns), generator=g)
    tgt[tgt < 0.1] = 0.0
    return qi, wi, ki, sel.to(DEV), tgt.to(DEV)


def _kl_reference(qi, wi, ki, sel, tgt):
    B, Tq, HI, dI = qi.shape
    qn, kn = bf16_to_f64(qi), bf16_to_f64(ki)
    wn, seln, tn = wi.cpu().double().numpy(), sel.cpu().numpy(), tgt.cpu().double().numpy()
    r_loss, r_dq, r_dw = np.zeros((B, Tq)), np.zeros((B, Tq, HI, dI)), np.zeros((B, Tq, HI))
    r_dk = np.zeros((B, ki.shape[1], dI))
    for b in range(B):
        for r in range(Tq):
            v = seln[b, r] >= 0
            idx = seln[b, r][v]
            P = tn[b, r][v] / tn[b, r][v].sum()
            l_, dq_, dw_, dk_ = ob.indexer_kl(qn[b, r], wn[b, r], kn[b][idx], P)
            r_loss[b, r], r_dq[b, r], r_dw[b, r] = l_, dq_, dw_
            np.add.at(r_dk[b], idx, dk_)
    return r_loss, r_dq, r_dw, r_dk


def _kl_check(got, want):
    loss, dq, dw, dk = got
    r_loss, r_dq, r_dw, r_dk = want
    np.testing.assert_allclose(loss.cpu().double().numpy(), r_loss, rtol=1e-4, atol=1e-6)
    for n, g_, w_, tol in (("dw", dw, r_dw, 1e-4), ("dq", dq, r_dq, REL_L2), ("dk", dk, r_dk, REL_L2)):
        g_ = g_.cpu().double().numpy()
        rel = np.linalg.norm(g_ - w_) / np.linalg.norm(w_)
        mx = np.abs(g_ - w_).max() / np.abs(w_).max()
        log(f"  {n}: rel-L2 {rel:.2e}, max-abs/max {mx:.2e}")
        assert rel <= tol and mx <= max(tol, MAX_REL if n != "dw" else 1e-4), n


@pytest.mark.parametrize("case", KL_CASES)
def test_index_kl_backward_matches_oracle(case):
    B, Tq, HI, dI, Ncap, ns, nv = case
    log(f"indexer KL backward {case}")
    inp = _kl_inputs(B, Tq, HI, dI, Ncap, ns, nv, sum(case[:6]) % 953)
    got = ops().index_kl_backward(*inp)
    torch.cuda.synchronize()
    _kl_check(got, _kl_reference(*inp))


def test_index_kl_backward_key_gradient_paths_match_oracle():
    """dk grouped in one group (the queried workspace), in several (a byte
    less: 256 + 44 queries), and added with atomics (the per-chunk buffers
    alone), on 300 queries whose sets share keys."""
    B, Tq, HI, dI, Ncap, ns = 1, 300, 4, 32, 200, 64
    inp = _kl_inputs(B, Tq, HI, dI, Ncap, ns, 60, 23)
    want = _kl_reference(*inp)
    full = ops().lib().v4attn_index_kl_backward_workspace(B, Tq, dI, ns, Ncap)
    least = _min_workspace(lambda n: ops().index_kl_backward(*inp, workspace_bytes=n))
    assert least < full - 1
    for nbytes, what in ((full, "one group"), (full - 1, "two groups"), (least, "atomics")):
        log(f"indexer KL backward dk: {what}, workspace {nbytes} of {full} bytes")
        got = ops().index_kl_backward(*inp, workspace_bytes=nbytes)
        torch.cuda.synchronize()
        _kl_check(got, want)


def test_attention_backward_p_sel_is_the_kl_target():
    """p_sel of the CSA backward = sum over heads of the attention
    probabilities of the top-k slots (bf16 q~ in the logits: rel-L2 4 * 2^-9)."""
    B, Tq, H, D, Ncap, k, W, q_pos0 = 2, 2, 64, 512, 2000, 256, 128, 9000
    q, ent, win, gq, sink, dout = _inputs(B, Tq, H, D, Ncap, W, 77)
    g = torch.Generator().manual_seed(7)
    topk = torch.stack([torch.stack([torch.randperm(Ncap, generator=g)[:k].sort().values
                                     for _ in range(Tq)]) for _ in range(B)]).to(torch.int32)
    topk[0, 0, -10:] = -1
    topk = topk.to(DEV)
    out, lse = ops().csa_attend(q, ent, topk, win, gq, sink, q_pos0=q_pos0, W=W, want_lse=True)
    p_sel = torch.empty((B, Tq, k), dtype=torch.float32, device=DEV)
    ops().csa_attend_backward(q, ent, topk, win, gq, sink, out, lse, dout, q_pos0=q_pos0, W=W,
                              p_sel=p_sel)
    torch.cuda.synchronize()
    qn, en, wn = bf16_to_f64(q), rows_to_f64(ent, D, R), rows_to_f64(win, D, R)
    tk = topk.cpu().numpy()
    for b in range(B):
        for r in range(Tq):
            t = q_pos0 + r
            sel = tk[b, r]
            rows = np.concatenate([en[b][sel[sel >= 0]], wn[b][_win_rows(t, q_pos0, W)]])
            _, p, _ = oa.attend_rows(qn[b, r], gq.cpu().double().numpy(), t, rows,
                                     sink.cpu().double().numpy(), D ** -0.5, EPS, R, BASE)
            want = np.zeros(k)
            want[sel >= 0] = p[:, : int((sel >= 0).sum())].sum(axis=0)
            got = p_sel[b, r].cpu().double().numpy()
            assert np.all(got[sel < 0] == 0)
            assert np.linalg.norm(got - want) <= REL_L2 * np.linalg.norm(want)
