"""Lightning indexer scores and top-k selection (test infrastructure only).

What the pages fix: a lightweight scorer ("a few small heads", [P1] step 3 of
the eight-step list) rates each compressed entry against the current query
([P5] "Two ways to shrink attention, interleaved"), and a top-k selector keeps
the k best for core attention, k = 1024 in V4-Pro ([P5] same section; [P1]
step 4; [P4] "The attention stack, and why it is two mechanisms").

Readings (the pages print no formula for the score):
  * score_{t,j} = sum_h w_{t,h} * ReLU(q^I_{t,h} . k^I_j): per-query indexer
    heads q^I, per-query head weights w, and ONE indexer key per compressed
    entry shared by all heads; no extra scale (it folds into w);
  * query at position t sees entries j < V_t = min(n_entries, floor((t+1)/m))
    (entry j exists once token (j+1)m-1 is cached);
  * FP8 indexer ([P1] step 3: the indexer's few heads run in FP8; [P5] same
    section: the indexer's attention runs at reduced precision): queries and
    keys are OCP E4M3FN codes with one positive scale per row (per query
    head, per key); the score is the score above of the dequantised rows;
  * MXFP4 indexer ([P5] same section: the indexer's attention runs in FP4):
    queries and keys in the OCP MX FP4 format (E2M1 elements, one E8M0 scale
    per 32 consecutive dims); again the score of the dequantised rows;
  * top-k order is (score descending, index ascending): ties go to the lower
    entry index.  The first min(k, V_t) entries in that order form the set;
    it is returned in ascending index order, padded with -1 to length k.
    Below the budget nothing is dropped ([P1] intro: when V_t <= k every
    visible entry is kept).
"""

import numpy as np

from .codecs import e4m3_decode, mxfp4_decode


def visible_entries(t, n_entries, m):
    """V_t = min(n_entries, floor((t+1)/m)) for query position t."""
    return int(min(n_entries, (t + 1) // m))


def index_scores(q_idx, w, k_idx, V):
    """Scores of one query against entries 0..V-1, float64 [V].

    q_idx: [H_I, d_I]; w: [H_I]; k_idx: [>=V, d_I]."""
    q = np.asarray(q_idx, dtype=np.float64)
    k = np.asarray(k_idx[:V], dtype=np.float64)
    logits = k @ q.T                                  # [V, H_I]
    return np.maximum(logits, 0.0) @ np.asarray(w, dtype=np.float64)


def topk_select(scores, k):
    """Indices of the min(k, len(scores)) best entries under (score desc,
    index asc), ascending, padded with -1 to length k.  int32 [k]."""
    scores = np.asarray(scores, dtype=np.float64)
    V = scores.shape[0]
    order = np.lexsort((np.arange(V), -scores))     # primary key: -score
    sel = np.sort(order[: min(k, V)])
    out = np.full(k, -1, dtype=np.int32)
    out[: sel.shape[0]] = sel
    return out


def index_topk(q_idx, w, k_idx, n_entries, q_pos, m, k):
    """Per-query scores and top-k for a block of queries of one sequence.

    q_idx: [Tq, H_I, d_I]; w: [Tq, H_I]; k_idx: [>= n_entries, d_I];
    q_pos: [Tq] positions.  Returns (topk int32 [Tq, k], list of score
    vectors, one float64 [V_t] per query)."""
    Tq = q_idx.shape[0]
    topk = np.full((Tq, k), -1, dtype=np.int32)
    scores = []
    for r in range(Tq):
        V = visible_entries(int(q_pos[r]), n_entries, m)
        sc = index_scores(q_idx[r], w[r], k_idx, V)
        topk[r] = topk_select(sc, k)
        scores.append(sc)
    return topk, scores


def index_scores_fp8(q8, q_scale, w, k8, k_scale, V):
    """FP8 indexer scores of one query against entries 0..V-1, float64 [V].

    q8: uint8 E4M3 codes [H_I, d_I]; q_scale: [H_I]; w: [H_I];
    k8: uint8 E4M3 codes [>=V, d_I]; k_scale: [>=V].  Query head h is
    q_scale[h] * decode(q8[h]) and key j is k_scale[j] * decode(k8[j])."""
    q = e4m3_decode(np.asarray(q8)) * np.asarray(q_scale, dtype=np.float64)[:, None]
    k = e4m3_decode(np.asarray(k8[:V])) * np.asarray(k_scale[:V], dtype=np.float64)[:, None]
    return index_scores(q, w, k, V)


def index_topk_fp8(q8, q_scale, w, k8, k_scale, n_entries, q_pos, m, k):
    """index_topk for the FP8 indexer: q8 [Tq, H_I, d_I], q_scale and w
    [Tq, H_I], k8 [>= n_entries, d_I], k_scale [>= n_entries]."""
    Tq = q8.shape[0]
    topk = np.full((Tq, k), -1, dtype=np.int32)
    scores = []
    for r in range(Tq):
        V = visible_entries(int(q_pos[r]), n_entries, m)
        sc = index_scores_fp8(q8[r], q_scale[r], w[r], k8, k_scale, V)
        topk[r] = topk_select(sc, k)
        scores.append(sc)
    return topk, scores


def index_scores_mxfp4(q4, q_sc, w, k4, k_sc, V):
    """MXFP4 indexer scores of one query against entries 0..V-1, float64 [V].

    q4: uint8 [H_I, d_I/2] packed E2M1; q_sc: uint8 [H_I, d_I/32] E8M0;
    w: [H_I]; k4: uint8 [>=V, d_I/2]; k_sc: uint8 [>=V, d_I/32]."""
    q = mxfp4_decode(q4, q_sc)
    k = mxfp4_decode(k4[:V], k_sc[:V])
    return index_scores(q, w, k, V)


def index_topk_mxfp4(q4, q_sc, w, k4, k_sc, n_entries, q_pos, m, k):
    """index_topk for the MXFP4 indexer: q4 [Tq, H_I, d_I/2], q_sc
    [Tq, H_I, d_I/32], w [Tq, H_I], k4 [>= n_entries, d_I/2], k_sc
    [>= n_entries, d_I/32]."""
    Tq = q4.shape[0]
    topk = np.full((Tq, k), -1, dtype=np.int32)
    scores = []
    for r in range(Tq):
        V = visible_entries(int(q_pos[r]), n_entries, m)
        sc = index_scores_mxfp4(q4[r], q_sc[r], w[r], k4, k_sc, V)
        topk[r] = topk_select(sc, k)
        scores.append(sc)
    return topk, scores
