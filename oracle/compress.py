"""Sequence compression of the KV stream (test infrastructure only).

What the pages fix ([P5] "Two ways to shrink attention, interleaved"; [P4]
"The attention stack, and why it is two mechanisms"; [P2] "Compressing the
past"): every m consecutive tokens' KV entries are pooled into one entry with
learned per-token compression weights and positional biases, with deliberate
overlap -- each entry draws on 2m source tokens while the sequence still
shrinks by a factor m.  CSA uses m = 4, HCA m' = 128.  Compressed entries get
an extra RMSNorm, RoPE acts on their last 64 dims, and they are stored with
BF16 rotary dims and FP8 for the rest.

Readings (the pages are silent on these):
  * window of entry j is the token positions [(j-1)m, (j+1)m): the group that
    entry j completes plus the previous group -- causal, and it gives
    floor(T/m) entries for T cached tokens;
  * entry 0 has no previous group: the missing positions are dropped and the
    softmax renormalises over the m real tokens;
  * weights alpha_{j,t} = softmax over the window of (s_t + b_{t-(j-1)m}):
    one scalar score s_t per token (shared by all channels) and a positional
    bias vector b of length 2m;
  * order of operations: pool -> RMSNorm (over all D dims, with gain gamma and
    epsilon eps) -> RoPE at position j*m on the last R dims -> quantise;
  * window (uncompressed) rows are the per-token latents with the same
    RMSNorm and RoPE at their own position ("PACK" below);
  * indexer keys of the compressed entries: the per-token indexer-key stream
    pooled by the same compressor, i.e. with entry j's own window weights
    alpha_{j,t}; no RMSNorm and no RoPE (the indexer's score uses the keys
    as they are), stored as bf16 ("pool_index_keys" below).
"""

import numpy as np

from .rope import rope


def rmsnorm(x, gamma, eps):
    """gamma * x / sqrt(mean(x^2) + eps), over the last axis, float64."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return np.asarray(gamma, dtype=np.float64) * x / np.sqrt(ms + eps)


def entry_count(T, m):
    """Entries that exist once positions 0..T-1 are cached: completed groups."""
    return T // m


def window_positions(j, m):
    """Token positions entry j pools over (negative ones do not exist)."""
    lo = (j - 1) * m
    return np.arange(max(lo, 0), (j + 1) * m), lo


def pool_weights(scores, bias, j, m):
    """alpha_{j,t} for the existing tokens of entry j's window.

    `scores` maps position -> s_t (indexable by absolute position);
    `bias` has length 2m and is indexed by the offset t - (j-1)m."""
    pos, lo = window_positions(j, m)
    logits = np.asarray([scores[p] for p in pos], dtype=np.float64) \
        + np.asarray(bias, dtype=np.float64)[pos - lo]
    mx = np.max(logits)
    w = np.exp(logits - mx)
    return pos, w / np.sum(w)


def entries_written(pos0, L, m):
    """Entries j whose whole (existing) window lies in raw positions
    [pos0, pos0+L) and whose last token is among them: range(j_lo, j_hi)."""
    j_hi = (pos0 + L) // m if pos0 + L >= 0 else 0
    if pos0 <= 0:
        j_lo = 0
    else:
        j_lo = -(-pos0 // m) + 1          # smallest j with (j-1)m >= pos0
    return j_lo, max(j_lo, j_hi)


def compress_pool(c, s, pos0, m, bias, gamma, eps, R, base, j0=None, n=None):
    """Pool raw latents of one sequence into compressed entries.

    c: [L, D] raw latents for positions pos0..pos0+L-1; s: [L] token scores.
    Entries j0..j0+n-1 are produced (default: every entry the rows allow);
    each one's existing window must lie inside the rows.
    Returns (js, e): the entry indices and their float64 values [n, D] after
    pooling, RMSNorm and RoPE at position j*m (not quantised)."""
    c = np.asarray(c, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    L, D = c.shape
    j_lo, j_hi = entries_written(pos0, L, m)
    if j0 is not None:
        assert j_lo <= j0 and j0 + n <= j_hi, "window rows not all present"
        j_lo, j_hi = j0, j0 + n
    js = np.arange(j_lo, j_hi)
    out = np.zeros((len(js), D))

    class _ByPos:
        def __getitem__(self, p):
            return s[p - pos0]

    for r, j in enumerate(js):
        pos, alpha = pool_weights(_ByPos(), bias, j, m)
        pooled = alpha @ c[pos - pos0]
        out[r] = rope(rmsnorm(pooled, gamma, eps), j * m, R, base)
    return js, out


def compress_pack(c, pos0, gamma, eps, R, base):
    """Window rows: each raw latent normalised and rotated at its own
    position (no pooling).  c: [L, D] -> float64 [L, D]."""
    c = np.asarray(c, dtype=np.float64)
    pos = pos0 + np.arange(c.shape[0])
    return rope(rmsnorm(c, gamma, eps), pos, R, base)


def pool_index_keys(kI, s, pos0, m, bias, js):
    """Indexer keys of entries js: sum_t alpha_{j,t} kI_t over entry j's
    window, with the weights of the entry itself (pool_weights).

    kI: [L, d_I] per-token indexer keys for positions pos0..; s: [L].
    Returns float64 [len(js), d_I] (not rounded)."""
    kI = np.asarray(kI, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)

    class _ByPos:
        def __getitem__(self, p):
            return s[p - pos0]

    out = np.zeros((len(js), kI.shape[1]))
    for r, j in enumerate(js):
        pos, alpha = pool_weights(_ByPos(), bias, j, m)
        out[r] = alpha @ kI[pos - pos0]
    return out
