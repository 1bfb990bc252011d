"""The decode step's other schedules (HCA attention on a second stream, the
one bench.py times; HIP-graph replays) give exactly the outputs of the
calls launched one by one.

The step's kernels are deterministic and its writes (window row, pooled
entry) are idempotent, so every run must reproduce the eager outputs bit for
bit.  Graphs are replayed several times with eager work and synchronisation
in between, each replay checked.
"""

import pytest
import torch

from long_context_sparse_csa_amd import decode
from long_context_sparse_csa_amd.configs import CSA_1M, HCA_1M

pytestmark = pytest.mark.gpu


def _snap(st):
    torch.cuda.synchronize()
    return [st.topk.clone(), st.out_c.clone(), st.out_h.clone()]


def _same(a, b):
    return all(torch.equal(x, y) for x, y in zip(a, b))


def test_decode_step_graph_replays_match_eager():
    dev = "cuda:0"
    c = CSA_1M.with_(B=2, T=1 << 17)   # 32768 entries: the multi-part top-k path
    h = HCA_1M.with_(B=3, T=1 << 16)
    inp = decode.build_inputs(c, h, dev, rotate=2)
    st = decode.DecodeStep(inp, c, h, dev)
    ref = []
    for r in range(2):
        st.run_eager(r)
        ref.append(_snap(st))
    assert not torch.equal(ref[0][2], ref[1][2]), "the two HCA caches should differ"
    for r in range(2):
        st.run_overlapped(r)
        assert _same(_snap(st), ref[r]), f"overlapped schedule, cache {r}"
    for i in range(4):   # concurrent schedule, back to back without syncs in between
        st.run_concurrent(i % 2)
        st.run_concurrent((i + 1) % 2)
        assert _same(_snap(st), ref[(i + 1) % 2]), f"concurrent schedule, round {i}"
    graphs = [st.capture(r) for r in range(2)]
    for i in range(6):
        r = i % 2
        graphs[r].replay()
        assert _same(_snap(st), ref[r]), f"replay {i} (cache {r})"
        # eager work between replays
        st.run_eager(1 - r)
        assert _same(_snap(st), ref[1 - r]), f"eager run after replay {i}"
        torch.zeros(1 << 20, device=dev).sum().item()
