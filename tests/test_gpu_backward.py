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
