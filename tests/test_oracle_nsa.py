"""Pins for the oracle's NSA-style variant (compressed, selected and window
branches mixed by gates).

The branches are the already-pinned attention over explicit row sets; these
tests pin what the variant adds: which rows each branch sees, the block
scores and their selection, and the gated sum.  Each pin fails for a
plausible mistake: a block mapped to the wrong tokens, scores not summed over
heads, a sink left in, ties broken upwards, gates swapped."""

import numpy as np
import torch

from oracle import attend as oa
from oracle import nsa

R, BASE, EPS = 16, 1e4, 1e-6


def _case(seed, Tq=3, H=4, D=64, m=4, n_entries=30, W=8):
    g = np.random.default_rng(seed)
    q_pos0 = n_entries * m - Tq + 1           # the last query completes the last entry
    T = q_pos0 + Tq
    q = g.normal(size=(Tq, H, D))
    entries = g.normal(size=(n_entries, D))
    tokens = g.normal(size=(T, D))
    win = tokens[q_pos0 - (W - 1): q_pos0 + Tq]
    gamma = g.normal(1.0, 0.1, size=D)
    gates = g.uniform(size=(Tq, H, 3))
    return dict(q=q, entries=entries, n_entries=n_entries, m=m, tokens=tokens, win=win,
                gamma_q=gamma, gates=gates, q_pos0=q_pos0, W=W), H, D


def _run(c, n_sel, scale=0.125):
    return nsa.nsa_attend(c["q"], c["entries"], c["n_entries"], c["m"], c["tokens"], c["win"],
                          c["gamma_q"], c["gates"], c["q_pos0"], c["W"], n_sel, scale, EPS, R,
                          BASE)


def test_block_scores_sum_to_heads_and_follow_the_compressed_branch():
    c, H, D = _case(1)
    _, blocks, scores, _ = _run(c, 5)
    for r, sc in enumerate(scores):
        assert np.isclose(sc.sum(), H, rtol=1e-12)    # no sink: every head's weights sum to 1
        # the compressed branch on its own: dense attention over the visible entries
        t = c["q_pos0"] + r
        V = min(c["n_entries"], (t + 1) // c["m"])
        _, p, _ = oa.attend_rows(c["q"][r], c["gamma_q"], t, c["entries"][:V],
                                 np.full(H, -np.inf), 0.125, EPS, R, BASE)
        assert np.allclose(sc, p.sum(axis=0), rtol=1e-12, atol=0)
        # the selection is the rank definition: no unselected block beats a selected one
        sel = blocks[r][blocks[r] >= 0]
        rest = np.setdiff1d(np.arange(V), sel)
        assert len(sel) == 5 and np.all(np.diff(sel) > 0)
        assert sc[sel].min() >= sc[rest].max()


def test_every_block_selected_is_dense_attention_over_the_covered_tokens():
    c, H, D = _case(2)
    V = c["n_entries"]
    _, blocks, _, br = _run(c, V + 3)
    r = c["q"].shape[0] - 1                      # the query that sees every entry
    t = c["q_pos0"] + r
    assert (t + 1) // c["m"] == V
    assert list(blocks[r][:V]) == list(range(V)) and np.all(blocks[r][V:] == -1)
    dense = oa.attend_rows(c["q"][r], c["gamma_q"], t, c["tokens"][: V * c["m"]],
                           np.full(H, -np.inf), 0.125, EPS, R, BASE)[0]
    assert np.allclose(br[r][1], dense, rtol=1e-12, atol=1e-12)


def test_selected_branch_reads_the_tokens_of_its_blocks():
    # Make the entries of blocks 3 and 7 dominant: they must be selected, and
    # the selected branch must equal attention over tokens 12..15 and 28..31.
    c, H, D = _case(3)
    c["entries"][3] *= 0.0
    c["entries"][7] *= 0.0
    qt_dir = np.ones(D)
    c["entries"][3] += 50 * qt_dir
    c["entries"][7] += 50 * qt_dir
    c["q"][:] = np.abs(c["q"]) + 1.0
    c["gamma_q"][:] = 1.0
    _, blocks, _, br = _run(c, 2, scale=0.05)
    r = 0
    t = c["q_pos0"]
    assert list(blocks[r]) == [3, 7]
    rows = np.concatenate([c["tokens"][12:16], c["tokens"][28:32]])
    want = oa.attend_rows(c["q"][r], c["gamma_q"], t, rows, np.full(H, -np.inf), 0.05, EPS,
                          R, BASE)[0]
    assert np.allclose(br[r][1], want, rtol=1e-12, atol=1e-12)


def test_equal_scores_select_the_lowest_blocks():
    c, H, D = _case(4)
    c["entries"][:] = c["entries"][0]              # identical entries: equal scores
    _, blocks, scores, _ = _run(c, 4)
    for r, sc in enumerate(scores):
        assert np.allclose(sc, sc[0], rtol=1e-12)
        assert list(blocks[r]) == [0, 1, 2, 3]


def test_gates_mix_the_three_branches_linearly():
    c, H, D = _case(5)
    out, _, _, br = _run(c, 3)
    for r in range(c["q"].shape[0]):
        g = c["gates"][r]
        want = g[:, 0:1] * br[r][0] + g[:, 1:2] * br[r][1] + g[:, 2:3] * br[r][2]
        assert np.allclose(out[r], want, rtol=1e-13, atol=1e-13)
    c2 = dict(c)
    c2["gates"] = np.zeros_like(c["gates"])
    c2["gates"][..., 2] = 1.0
    out2, _, _, _ = _run(c2, 3)
    t0 = c["q_pos0"]
    win = oa.attend_rows(c["q"][0], c["gamma_q"], t0, oa.window_rows(c["win"], t0, t0, c["W"]),
                         np.full(H, -np.inf), 0.125, EPS, R, BASE)[0]
    assert np.allclose(out2[0], win, rtol=1e-12, atol=1e-12)


def test_window_branch_matches_sdpa_without_sink():
    # an independent library routine: torch's SDPA in float64 over the window rows
    from oracle.compress import rmsnorm
    from oracle.rope import rope
    c, H, D = _case(6)
    out, _, _, br = _run(c, 2)
    r, t = 1, c["q_pos0"] + 1
    rows = oa.window_rows(c["win"], t, c["q_pos0"], c["W"])
    qt = rope(rmsnorm(c["q"][r], c["gamma_q"], EPS), t, R, BASE)
    o = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qt)[None, :, None, :], torch.from_numpy(rows)[None, None].expand(1, H, -1, -1),
        torch.from_numpy(rows)[None, None].expand(1, H, -1, -1), scale=0.125)[0, :, 0].numpy()
    assert np.allclose(br[r][2], rope(o, -t, R, BASE), rtol=1e-10, atol=1e-12)
