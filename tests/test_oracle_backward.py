"""Pins for the oracle's gradients (oracle/backward.py).

Each gradient is checked against central finite differences of the already
pinned forward functions (a different computation: it never uses the chain
rule), plus invariants a dropped term, a wrong sign or a transposed operand
breaks: softmax shift invariance (the logit and sink gradients sum to zero),
the pooling weights' shift invariance (token-score gradients of a window sum
to zero), a lone row with no sink (only the value path), KL(P || P) = 0 with
zero gradients, and the ReLU mask."""

import numpy as np

from oracle import attend as oa
from oracle import backward as ob
from oracle import compress as oc

R, BASE, EPS = 8, 1e4, 1e-6


def _fd(f, x, h=1e-6):
    """Central differences of scalar f over every element of x (in place)."""
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = x[i]
        x[i] = old + h
        fp = f()
        x[i] = old - h
        fm = f()
        x[i] = old
        g[i] = (fp - fm) / (2 * h)
    return g


def _attn_case(seed, H=3, D=24, n=5):
    g = np.random.default_rng(seed)
    return dict(q=g.normal(size=(H, D)), rows=g.normal(size=(n, D)), sink=g.normal(size=H),
                gamma=g.normal(1.0, 0.2, size=D), dout=g.normal(size=(H, D)), t=37,
                scale=0.3)


def test_attention_gradients_match_finite_differences():
    c = _attn_case(1)

    def loss():
        out = oa.attend_rows(c["q"], c["gamma"], c["t"], c["rows"], c["sink"], c["scale"], EPS, R,
                             BASE)[0]
        return float(np.sum(out * c["dout"]))

    dq, drows, dsink, dgamma = ob.attend_rows_backward(c["q"], c["gamma"], c["t"], c["rows"],
                                                       c["sink"], c["scale"], EPS, R, BASE,
                                                       c["dout"])
    for name, got in (("q", dq), ("rows", drows), ("sink", dsink), ("gamma", dgamma)):
        want = _fd(loss, c[name])
        assert np.allclose(got, want, rtol=1e-6, atol=1e-8), name


def test_attention_logit_and_sink_gradients_sum_to_zero():
    # adding one constant to every logit and to the sink changes nothing
    c = _attn_case(2)
    qn = oc.rmsnorm(c["q"], c["gamma"], EPS)
    dq, drows, dsink, _ = ob.attend_rows_backward(c["q"], c["gamma"], c["t"], c["rows"],
                                                  c["sink"], c["scale"], EPS, R, BASE, c["dout"])
    # d loss / d logits, recovered from the key path: drows - value path
    from oracle.rope import rope
    out, p, _ = oa.attend_rows(c["q"], c["gamma"], c["t"], c["rows"], c["sink"], c["scale"], EPS,
                               R, BASE)
    do = rope(c["dout"], c["t"], R, BASE)
    dp = do @ c["rows"].T
    dl = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
    assert np.allclose(dl.sum(axis=1) + dsink, 0.0, atol=1e-12)
    assert np.allclose(qn.shape, dq.shape)


def test_lone_row_without_sink_passes_dout_to_the_value():
    c = _attn_case(3, n=1)
    dq, drows, dsink, dgamma = ob.attend_rows_backward(c["q"], c["gamma"], c["t"], c["rows"],
                                                       np.full(3, -np.inf), c["scale"], EPS, R,
                                                       BASE, c["dout"])
    from oracle.rope import rope
    assert np.allclose(dq, 0.0) and np.allclose(dgamma, 0.0) and np.allclose(dsink, 0.0)
    assert np.allclose(drows[0], rope(c["dout"], c["t"], R, BASE).sum(axis=0))


def _pool_case(seed, m=4, L=20, D=16):
    g = np.random.default_rng(seed)
    return dict(c=g.normal(size=(L, D)), s=g.normal(size=L), bias=g.normal(0, 0.3, size=2 * m),
                gamma=g.normal(1.0, 0.2, size=D), m=m, pos0=0)


def test_compress_gradients_match_finite_differences():
    k = _pool_case(4)
    js, e = oc.compress_pool(k["c"], k["s"], k["pos0"], k["m"], k["bias"], k["gamma"], EPS, R, BASE)
    de = np.random.default_rng(5).normal(size=e.shape)

    def loss():
        return float(np.sum(oc.compress_pool(k["c"], k["s"], k["pos0"], k["m"], k["bias"],
                                             k["gamma"], EPS, R, BASE)[1] * de))

    dc, ds, dbias, dgamma = ob.compress_pool_backward(k["c"], k["s"], k["pos0"], k["m"], k["bias"],
                                                      k["gamma"], EPS, R, BASE, js, de)
    for name, got in (("c", dc), ("s", ds), ("bias", dbias), ("gamma", dgamma)):
        want = _fd(loss, k[name])
        assert np.allclose(got, want, rtol=1e-6, atol=1e-8), name


def test_compress_score_gradients_of_one_window_sum_to_zero():
    # one entry: adding a constant to the scores of its window changes nothing
    k = _pool_case(6, L=8)
    de = np.random.default_rng(7).normal(size=(1, 16))
    _, ds, dbias, _ = ob.compress_pool_backward(k["c"], k["s"], 0, 4, k["bias"], k["gamma"], EPS,
                                                R, BASE, np.array([1]), de)
    assert abs(ds.sum()) < 1e-12 and abs(dbias.sum()) < 1e-12


def _kl_case(seed, H=4, d=8, n=7):
    g = np.random.default_rng(seed)
    P = g.random(n)
    P[2] = 0.0
    return dict(q=g.normal(size=(H, d)), w=g.normal(size=H), k=g.normal(size=(n, d)),
                P=P / P.sum())


def test_indexer_kl_gradients_match_finite_differences():
    c = _kl_case(8)
    loss, dq, dw, dk = ob.indexer_kl(c["q"], c["w"], c["k"], c["P"])
    f = lambda: ob.indexer_kl(c["q"], c["w"], c["k"], c["P"])[0]
    for name, got in (("q", dq), ("w", dw), ("k", dk)):
        assert np.allclose(got, _fd(f, c[name]), rtol=1e-6, atol=1e-8), name
    # the definition written out once more at these inputs: KL >= 0
    assert loss >= 0.0


def test_indexer_kl_is_zero_when_the_indexer_matches_the_target():
    c = _kl_case(9)
    act = np.maximum(c["q"] @ c["k"].T, 0.0)
    P = np.exp(c["w"] @ act)
    P /= P.sum()
    loss, dq, dw, dk = ob.indexer_kl(c["q"], c["w"], c["k"], P)
    assert abs(loss) < 1e-12
    assert np.allclose(dq, 0, atol=1e-12) and np.allclose(dw, 0, atol=1e-12) \
        and np.allclose(dk, 0, atol=1e-12)


def test_indexer_kl_heads_with_negative_dots_get_no_key_gradient():
    c = _kl_case(10, H=1)
    c["k"] = -np.abs(c["k"]) * np.sign(c["q"][0])[None, :]   # every q.k < 0
    _, dq, dw, dk = ob.indexer_kl(c["q"], c["w"], c["k"], c["P"])
    assert np.all(dq == 0) and np.all(dw == 0) and np.all(dk == 0)


def test_kl_target_renormalises_over_the_set():
    p = np.array([[0.1, 0.2, 0.0], [0.3, 0.1, 0.1]])
    assert np.allclose(ob.kl_target(p), np.array([0.4, 0.3, 0.1]) / 0.8)
