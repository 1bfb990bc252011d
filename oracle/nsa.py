"""NSA-style compress-select-window attention with learned gates (test
infrastructure only).

What the pages fix ([P1] "DeepSeek-V4, explained", steps 2-6 of how one
query's layer works, on Native Sparse Attention, V4's ancestor): the cached
sequence is cut into blocks of consecutive tokens, the unit of selection; the
block scores come from attention over compressed block representations, so
the coarse view doubles as the selector; the k highest-scoring blocks are
kept and attended at full fidelity; a sliding window of the most recent
tokens is always kept; the compressed, selected and window outputs are mixed
with learned gates.

Readings (the page gives no formulas):
  * compressed branch: attention of q~ over the visible compressed entries
    j < V_t = min(n_entries, floor((t+1)/m)) of the a1 compressor, with no
    window and no sink;
  * selection block j is the group of m tokens [j m, (j+1) m) that entry j
    completes; its score is the compressed branch's attention probability of
    entry j summed over the heads (all heads share one KV);
  * selected branch: attention over the full-fidelity rows of the tokens of
    the top-n blocks (the top-k rule of the indexer: score descending, index
    ascending), no window, no sink;
  * window branch: attention over the window rows max(0, t-W+1)..t, no sink;
  * out = sum_b g_b * out_b per query and head, gates g in the input; every
    branch output is already rotated by -t, so the sum is too.
"""

import numpy as np

from .attend import attend_rows, window_rows
from .indexer import topk_select, visible_entries


def nsa_attend(q, entries, n_entries, m, tokens, win, gamma_q, gates, q_pos0, W, n_sel,
               scale, eps, R, base):
    """One sequence.  q [Tq, H, D]; entries [>= n_entries, D] and tokens
    [>= q_pos0 + Tq, D] (row i = position i) float64; win [Tq+W-1, D];
    gates [Tq, H, 3] (compressed, selected, window).

    Returns (out [Tq, H, D], blocks int32 [Tq, n_sel] ascending and -1
    padded, list of block-score vectors, list of the branch outputs)."""
    Tq, H, D = q.shape
    no_sink = np.full(H, -np.inf)
    out = np.zeros((Tq, H, D))
    blocks = np.full((Tq, n_sel), -1, dtype=np.int32)
    scores, branches = [], []
    for r in range(Tq):
        t = q_pos0 + r
        V = visible_entries(t, n_entries, m)
        o_cmp, p_cmp, _ = attend_rows(q[r], gamma_q, t, entries[:V], no_sink, scale, eps, R, base)
        sc = p_cmp.sum(axis=0)                       # [V]
        blk = topk_select(sc, n_sel)
        sel = blk[blk >= 0]
        tok = (sel[:, None] * m + np.arange(m)[None, :]).ravel()
        o_slc = attend_rows(q[r], gamma_q, t, tokens[tok], no_sink, scale, eps, R, base)[0]
        o_win = attend_rows(q[r], gamma_q, t, window_rows(win, t, q_pos0, W), no_sink, scale,
                            eps, R, base)[0]
        g = np.asarray(gates[r], dtype=np.float64)
        out[r] = g[:, 0:1] * o_cmp + g[:, 1:2] * o_slc + g[:, 2:3] * o_win
        blocks[r] = blk
        scores.append(sc)
        branches.append((o_cmp, o_slc, o_win))
    return out, blocks, scores, branches
