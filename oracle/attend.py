"""Shared-KV multi-query core attention with window and sink (test
infrastructure only).

What the pages fix:
  * ordinary softmax attention runs over the selected positions only ([P1]
    step 5); S_t is the kept positions plus any always-kept window, and keys
    and values are reconstructed from the cached latents ([P1] glossary);
  * CSA attends to the top-k compressed entries; HCA attends densely to every
    compressed entry ([P5] "Two ways to shrink attention, interleaved"; [P3]
    "A coarse overview alongside local detail");
  * both keep a 128-token uncompressed sliding-window branch, a learnable
    per-head attention sink that lets the weights sum to less than one, and a
    shared-KV multi-query layout ([P4] "The attention stack, and why it is two
    mechanisms"; [P2] "Compressing the past");
  * queries get an extra RMSNorm, RoPE acts on the last 64 dims, a compressed
    entry is both key and value, and RoPE at position -i is applied to the
    output so it carries relative positions ([P5] same section).

Readings:
  * q~ = RoPE_t(RMSNorm_gamma_q(q)); logits l = scale * q~ . x for every row x
    in the selected entries and the window rows at positions
    max(0, t-W+1) .. t (the query's own token included);
  * the window and the selected entries share ONE softmax together with the
    sink: p_x = e^{l_x} / (e^{z_h} + sum_y e^{l_y}); the sink logit z_h is not
    multiplied by `scale` and carries a zero value;
  * o = sum_x p_x x (values are the stored rows, rotary dims included);
    out = RoPE_{-t}(o) on the last R dims;
  * lse = log(e^{z_h} + sum_y e^{l_y});
  * rows a window token and a compressed entry both cover are not
    de-duplicated.
"""

import numpy as np

from .compress import rmsnorm
from .rope import rope


def attend_rows(q, gamma_q, t, rows, sink, scale, eps, R, base):
    """One query token over an explicit row set.

    q: [H, D] raw query; rows: [n, D] float64 (keys == values); sink: [H].
    Returns (out [H, D], p [H, n], lse [H])."""
    q = np.asarray(q, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.float64).reshape(-1, q.shape[-1])
    z = np.asarray(sink, dtype=np.float64)[:, None]            # [H, 1]
    qt = rope(rmsnorm(q, gamma_q, eps), t, R, base)
    logits = scale * (qt @ rows.T)                              # [H, n]
    if rows.shape[0]:
        mx = np.maximum(np.max(logits, axis=-1, keepdims=True), z)
    else:
        mx = z.copy()
    mx = np.where(np.isfinite(mx), mx, 0.0)
    e = np.exp(logits - mx)
    den = np.exp(z - mx) + np.sum(e, axis=-1, keepdims=True)
    with np.errstate(invalid="ignore", divide="ignore"):
        p = np.where(den > 0, e / np.where(den > 0, den, 1.0), 0.0)
        lse = (mx + np.log(den))[:, 0]
    o = p @ rows
    return rope(o, -t, R, base), p, lse


def window_rows(win, t, q_pos0, W):
    """Rows of the window buffer a query at position t uses.

    win: [Tq+W-1, D]; buffer row r holds position q_pos0-(W-1)+r.  The query
    sees positions max(0, t-W+1)..t."""
    base_pos = q_pos0 - (W - 1)
    lo = max(0, t - W + 1)
    return win[lo - base_pos: t + 1 - base_pos]


def attend_csa(q, entries, topk, win, gamma_q, sink, q_pos0, W, scale, eps,
               R, base):
    """CSA core attention for one sequence.

    q: [Tq, H, D]; entries: [>= max index + 1, D] float64; topk: [Tq, k]
    (entries with index -1 are skipped); win: [Tq+W-1, D].
    Returns (out [Tq, H, D], lse [Tq, H])."""
    Tq, H, D = q.shape
    out = np.zeros((Tq, H, D))
    lse = np.zeros((Tq, H))
    for r in range(Tq):
        t = q_pos0 + r
        sel = topk[r][topk[r] >= 0]
        rows = np.concatenate([entries[sel], window_rows(win, t, q_pos0, W)])
        out[r], _, lse[r] = attend_rows(q[r], gamma_q, t, rows, sink, scale,
                                        eps, R, base)
    return out, lse


def attend_hca(q, entries, n_entries, m, win, gamma_q, sink, q_pos0, W, scale,
               eps, R, base):
    """HCA core attention for one sequence: every visible entry
    j < min(n_entries, floor((t+1)/m)) plus the window."""
    Tq, H, D = q.shape
    out = np.zeros((Tq, H, D))
    lse = np.zeros((Tq, H))
    for r in range(Tq):
        t = q_pos0 + r
        V = min(n_entries, (t + 1) // m)
        rows = np.concatenate([entries[:V], window_rows(win, t, q_pos0, W)])
        out[r], _, lse[r] = attend_rows(q[r], gamma_q, t, rows, sink, scale,
                                        eps, R, base)
    return out, lse
