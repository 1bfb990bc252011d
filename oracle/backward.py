"""Gradients of the attention step (test infrastructure only).

What the pages fix: the attention step is trained end to end, except the
top-k choice, which is a hard selection with no gradient; DSA trains its
lightning indexer with a KL-divergence loss that pulls the indexer's scores
toward the main attention's distribution, with the indexer's input detached
so that loss never reaches the main model, first over every entry (dense
warm-up), then over the selected ones ("DeepSeek-V4, explained", step 7).
NSA trains its selector through the compressed branch instead (same step).

Each function is the chain rule of the forward definition in this package,
written out in float64, step by step in the forward's order reversed.

Readings:
  * attention: gradients of attend_rows' output with respect to the raw
    query q, every attended row x (a row is both key and value, so it gets
    both contributions), the sink logit z_h (its value is zero) and gamma_q;
    the top-k set and the window are fixed;
  * compressor: gradients of compress_pool's float64 entries (after RoPE,
    before quantisation: the caller's gradient is taken with respect to the
    stored values, the rounding passed straight through) with respect to the
    raw latents c, the token scores s, the positional biases b and gamma;
  * indexer loss over one query's entry set S (the selected entries, or every
    visible one): target P_j = sum_h p_hj / sum_{j' in S} sum_h p_hj', the
    main attention's probabilities of the entries summed over heads and
    renormalised over S (window rows and sink left out); indexer distribution
    Q = softmax over S of the indexer scores; loss KL(P || Q) =
    sum_j P_j (log P_j - log Q_j) (P_j = 0 terms are zero).  P is a constant
    (the detach); gradients go to q^I, w and k^I.
"""

import numpy as np

from .compress import pool_weights, rmsnorm, window_positions
from .rope import rope


def rmsnorm_backward(x, gamma, eps, dy):
    """y = gamma x / r with r = sqrt(mean(x^2) + eps) over the last axis.
    Returns (dx, dgamma) for the upstream gradient dy (dgamma summed over
    the leading axes)."""
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    gamma = np.asarray(gamma, dtype=np.float64)
    D = x.shape[-1]
    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    g = dy * gamma
    # dr/dx = x / (D r)
    dx = g / r - x * np.sum(g * x, axis=-1, keepdims=True) / (D * r ** 3)
    dgamma = np.sum((dy * x / r).reshape(-1, D), axis=0)
    return dx, dgamma


def attend_rows_backward(q, gamma_q, t, rows, sink, scale, eps, R, base, dout):
    """Backward of attend_rows for one query token.

    q [H, D] raw query; rows [n, D]; sink [H]; dout [H, D] the gradient of
    the output.  Returns (dq [H, D], drows [n, D], dsink [H], dgamma [D])."""
    q = np.asarray(q, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.float64).reshape(-1, q.shape[-1])
    z = np.asarray(sink, dtype=np.float64)[:, None]
    dout = np.asarray(dout, dtype=np.float64)
    # forward
    qn = rmsnorm(q, gamma_q, eps)
    qt = rope(qn, t, R, base)
    logits = scale * (qt @ rows.T)                                   # [H, n]
    mx = np.maximum(np.max(logits, axis=-1, keepdims=True), z) if rows.shape[0] else z.copy()
    mx = np.where(np.isfinite(mx), mx, 0.0)
    den = np.exp(z - mx) + np.sum(np.exp(logits - mx), axis=-1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        p = np.where(den > 0, np.exp(logits - mx) / np.where(den > 0, den, 1.0), 0.0)
        pz = np.where(den > 0, np.exp(z - mx) / np.where(den > 0, den, 1.0), 0.0)   # sink weight
    # out = RoPE_{-t}(o): the rotation is orthogonal, so do = RoPE_t(dout)
    do = rope(dout, t, R, base)
    dp = do @ rows.T                                                 # [H, n]
    Dh = np.sum(p * dp, axis=-1, keepdims=True)                      # = do . o
    dl = p * (dp - Dh)                                               # through the softmax
    dsink = (pz * (0.0 - Dh))[:, 0]                                  # the sink's value is zero
    drows = scale * (dl.T @ qt) + p.T @ do                           # key and value paths
    dqt = scale * (dl @ rows)
    dqn = rope(dqt, -t, R, base)                                     # RoPE_t transposed
    dq, dgamma = rmsnorm_backward(q, gamma_q, eps, dqn)
    return dq, drows, dsink, dgamma


def compress_pool_backward(c, s, pos0, m, bias, gamma, eps, R, base, js, de):
    """Backward of compress_pool for entries js of one sequence.

    c [L, D] raw latents at positions pos0..; s [L]; de [len(js), D] the
    gradient of the float64 entries.  Returns (dc [L, D], ds [L],
    dbias [2m], dgamma [D])."""
    c = np.asarray(c, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    L, D = c.shape
    dc = np.zeros_like(c)
    ds = np.zeros(L)
    dbias = np.zeros(2 * m)
    dgamma = np.zeros(D)

    class _ByPos:
        def __getitem__(self, p):
            return s[p - pos0]

    for r, j in enumerate(js):
        pos, alpha = pool_weights(_ByPos(), bias, j, m)
        _, lo = window_positions(j, m)
        x = c[pos - pos0]                                    # [n, D]
        pooled = alpha @ x
        dy = rope(np.asarray(de[r], dtype=np.float64), -j * m, R, base)   # RoPE at j m, transposed
        dpooled, dg = rmsnorm_backward(pooled, gamma, eps, dy)
        dgamma += dg
        dc[pos - pos0] += alpha[:, None] * dpooled[None, :]
        dalpha = x @ dpooled                                 # [n]
        dlogit = alpha * (dalpha - np.sum(alpha * dalpha))   # through the window softmax
        ds[pos - pos0] += dlogit
        dbias[pos - lo] += dlogit
    return dc, ds, dbias, dgamma


def kl_target(p_rows):
    """P over an entry set from the main attention's probabilities p_rows
    [H, n] of those entries (heads summed, renormalised over the set)."""
    a = np.asarray(p_rows, dtype=np.float64).sum(axis=0)
    tot = a.sum()
    return a / tot if tot > 0 else a


def indexer_kl(q_idx, w, k_rows, P):
    """KL(P || softmax(scores)) over one query's entry set and its gradients.

    q_idx [H_I, d_I]; w [H_I]; k_rows [n, d_I] the set's indexer keys;
    P [n] the target.  Returns (loss, dq [H_I, d_I], dw [H_I], dk [n, d_I])."""
    q_idx = np.asarray(q_idx, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    k_rows = np.asarray(k_rows, dtype=np.float64)
    P = np.asarray(P, dtype=np.float64)
    a = q_idx @ k_rows.T                                     # [H_I, n]
    act = np.maximum(a, 0.0)
    sc = w @ act                                             # [n]
    mx = sc.max()
    lq = sc - mx - np.log(np.sum(np.exp(sc - mx)))           # log Q
    Q = np.exp(lq)
    with np.errstate(divide="ignore", invalid="ignore"):
        loss = float(np.sum(np.where(P > 0, P * (np.log(np.where(P > 0, P, 1.0)) - lq), 0.0)))
    dsc = Q * P.sum() - P                                    # d loss / d scores
    dw = act @ dsc
    g = (a > 0) * w[:, None] * dsc[None, :]                  # [H_I, n]
    dq = g @ k_rows
    dk = g.T @ q_idx
    return loss, dq, dw, dk
