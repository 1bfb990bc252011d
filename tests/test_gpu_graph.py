"""The decode step as a unit: one CSA layer and one HCA layer.

  * Against the float64 oracle: from the raw latents and token keys of the
    new token, the step writes the window row, the completed entry and its
    pooled indexer key; the indexer and top-k then see that entry; the
    attention reads the new rows.  The rows the step writes are poisoned
    beforehand, so a kernel that read them before the compress step wrote
    them would see the poison.
  * The schedule bench.py times (HCA attention on a second stream) and HIP
    graph replays of it reproduce the one-stream launches bit for bit; the
    rows the step writes are poisoned before every run, and graphs are
    replayed several times with eager work and synchronisation in between.
"""

import numpy as np
import pytest
import torch

from long_context_sparse_csa_amd import decode
from long_context_sparse_csa_amd.configs import CSA_1M, HCA_1M
from oracle import attend as oa
from oracle import codecs
from oracle import compress as oc
from oracle import indexer as oi

from helpers import assert_attn_close, assert_rows_within_one_ulp, bf16_to_f64, quantum_bf16

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from long_context_sparse_csa_amd import ops
    ops.lib()
    yield


def log(msg):
    print(msg, flush=True)


def _snap(st):
    torch.cuda.synchronize()
    return [st.topk.clone(), st.out_c.clone(), st.out_h.clone(),
            st.inp["csa"]["k_idx"][:, -1].clone(), st.inp["csa"]["entries"][:, -1].clone()]


def _same(a, b):
    return all(torch.equal(x, y) for x, y in zip(a, b))


def _poison(st, rot):
    """Overwrite every row the step writes (CSA and HCA window rows, the
    completed entries, the completed entry's indexer key)."""
    a, b = st.inp["csa"], st.inp["hca"]
    a["entries"][:, -1].fill_(0x55)
    a["win"][:, -1].fill_(0x55)
    a["k_idx"][:, -1].fill_(-3.0)
    b["entries"][rot][:, -1].fill_(0x55)
    b["win"][:, -1].fill_(0x55)


def _small():
    c = CSA_1M.with_(B=2, T=1 << 17)   # 32768 entries: the multi-part top-k path
    h = HCA_1M.with_(B=3, T=1 << 16)
    return c, h


def test_decode_step_matches_oracle():
    c, h = _small()
    log(f"decode step: CSA B={c.B} T={c.T}, HCA B={h.B} T={h.T}")
    inp = decode.build_inputs(c, h, DEV, rotate=1)
    st = decode.DecodeStep(inp, c, h, DEV)
    _poison(st, 0)
    st.run_concurrent(0)
    torch.cuda.synchronize()
    R, eps, base = c.R, c.eps, c.rope_base
    for lay, w in (("csa", c), ("hca", h)):
        d = inp[lay]
        ent = d["entries"] if lay == "csa" else d["entries"][0]
        t, N, m = d["t"], d["N"], w.m
        raw = bf16_to_f64(d["raw"])
        sc, bias = d["score"].cpu().double().numpy(), d["bias"].cpu().double().numpy()
        gm = d["gamma"].cpu().double().numpy()
        for b in range(w.B):
            # the new token's window row and the entry it completes
            e = oc.compress_pack(raw[b, -1:], t, gm, eps, R, base)
            assert_rows_within_one_ulp(d["win"][b, -1:].cpu().numpy(), e, w.D, R)
            js, e = oc.compress_pool(raw[b], sc[b], t + 1 - 2 * m, m, bias, gm, eps, R, base,
                                     j0=N - 1, n=1)
            assert_rows_within_one_ulp(ent[b, -1:].cpu().numpy(), e, w.D, R)
    a = inp["csa"]
    kraw = bf16_to_f64(a["raw_idx"])
    for b in range(c.B):
        want = oc.pool_index_keys(kraw[b], a["score"][b].cpu().double().numpy(),
                                  a["t"] + 1 - 2 * c.m, c.m, a["bias"].cpu().double().numpy(),
                                  [a["N"] - 1])[0]
        got = bf16_to_f64(a["k_idx"][b, -1])
        assert np.all(np.abs(got - want) <= quantum_bf16(want) + 1e-30), "pooled indexer key"
    # indexer + top-k over the keys as the step left them (the new one included)
    t, N = a["t"], a["N"]
    kn = bf16_to_f64(a["k_idx"])
    for b in range(c.B):
        qn, wn = bf16_to_f64(a["q_idx"][b, 0]), a["w_idx"][b, 0].cpu().double().numpy()
        sc = oi.index_scores(qn, wn, kn[b], oi.visible_entries(t, N, c.m))
        want = oi.topk_select(sc, c.k)
        g = st.topk[b, 0].cpu().numpy()
        tau = np.sort(sc)[::-1][c.k - 1]
        tol = 1e-5 * (np.abs(kn[b]) @ np.abs(qn).T @ np.abs(wn)).max()
        assert np.all(sc[np.setdiff1d(g, want)] >= tau - tol)
        assert np.all(sc[np.setdiff1d(want, g)] <= tau + tol)
        assert (N - 1 in g) == (N - 1 in want) or abs(sc[N - 1] - tau) <= tol
    # attention over the rows as the step left them
    for lay, w, out in (("csa", c, st.out_c), ("hca", h, st.out_h)):
        d = inp[lay]
        ent = d["entries"] if lay == "csa" else d["entries"][0]
        t = d["t"]
        for b in range(w.B):
            if lay == "csa":
                sel = st.topk[b, 0].long()
                rows = ent[b, sel[sel >= 0]]
            else:
                rows = ent[b, : min(d["N"], (t + 1) // w.m)]
            rows = codecs.unpack_rows(torch.cat([rows, d["win"][b]]).cpu().numpy(), w.D, R)
            o, _, _ = oa.attend_rows(bf16_to_f64(d["q"][b, 0]), d["gamma"].cpu().double().numpy(),
                                     t, rows, d["sink"].cpu().double().numpy(), w.scale, eps, R,
                                     base)
            ma, rl = assert_attn_close(bf16_to_f64(out[b, 0]), o, f"{lay} b={b}")
            log(f"  {lay} b={b} max_abs {ma:.2e} rel_l2 {rl:.2e}")


def test_decode_step_schedules_and_graph_replays_match_eager():
    c, h = _small()
    inp = decode.build_inputs(c, h, DEV, rotate=2)
    st = decode.DecodeStep(inp, c, h, DEV)
    ref = []
    for r in range(2):
        _poison(st, r)
        st.run_eager(r)
        ref.append(_snap(st))
    assert not torch.equal(ref[0][2], ref[1][2]), "the two HCA caches should differ"
    for i in range(4):   # concurrent schedule, back to back without syncs in between
        _poison(st, i % 2)
        st.run_concurrent(i % 2)
        _poison(st, (i + 1) % 2)
        st.run_concurrent((i + 1) % 2)
        assert _same(_snap(st), ref[(i + 1) % 2]), f"concurrent schedule, round {i}"
    graphs = [st.capture(r) for r in range(2)]
    for i in range(6):
        r = i % 2
        _poison(st, r)
        graphs[r].replay()
        assert _same(_snap(st), ref[r]), f"replay {i} (cache {r})"
        # eager work between replays
        _poison(st, 1 - r)
        st.run_eager(1 - r)
        assert _same(_snap(st), ref[1 - r]), f"eager run after replay {i}"
        torch.zeros(1 << 20, device=DEV).sum().item()


def test_layer_stack_graph_replays_match_eager():
    """Four alternating layers (CSA, HCA, CSA, HCA, each pair with its own
    caches) on one stream, captured as one HIP graph: every replay equals the
    eager launches bit for bit, with the written rows poisoned before each run
    and eager work and synchronisation between replays."""
    c, h = _small()
    sts = []
    for i in range(2):
        ci = c.with_(seed=c.seed + 1000 * (i + 1))
        hi = h.with_(seed=h.seed + 1000 * (i + 1))
        sts.append(decode.DecodeStep(decode.build_inputs(ci, hi, DEV, rotate=1), ci, hi, DEV))
    launches = decode.stack_launches(sts)
    names = [n for n, _ in launches]
    assert names[:6] == ["L0_csa_compress", "L0_index_score", "L0_topk_select",
                         "L0_csa_attend", "L1_hca_compress", "L1_hca_attend"]
    assert len(names) == 12

    def run_eager():
        for st in sts:
            _poison(st, 0)
        for _, fn in launches:
            fn()
        return [x for st in sts for x in _snap(st)]

    ref = run_eager()
    assert not torch.equal(ref[1], ref[6]), "the two CSA layers should differ"
    g = decode.capture_launches(launches)
    for i in range(4):
        for st in sts:
            _poison(st, 0)
        g.replay()
        got = [x for st in sts for x in _snap(st)]
        assert _same(got, ref), f"stack replay {i}"
        assert _same(run_eager(), ref), f"eager stack after replay {i}"
        torch.zeros(1 << 20, device=DEV).sum().item()
