"""Host-side checks of the C ABI (no GPU needed): the library loads and
exports every function include/v4attn.h declares, workspace queries are pure
host arithmetic, and invalid arguments return the documented status before
any device call.  Every call below fails validation, so nothing is launched
even on a machine with a GPU; the fake pointers are never dereferenced."""

import ctypes

import pytest

from long_context_sparse_csa_amd import LIB_PATH
import os

pytestmark = pytest.mark.skipif(not os.path.exists(LIB_PATH),
                                reason="libv4attn.so not built (python -m long_context_sparse_csa_amd.build)")


def L():
    from long_context_sparse_csa_amd import ops
    return ops.lib()


def ops():
    from long_context_sparse_csa_amd import ops as o
    return o


FAKE = ctypes.c_void_p(0x100000)     # aligned, never dereferenced
MISALIGNED = ctypes.c_void_p(0x100008)


def test_exports_every_header_function():
    names = ops().header_functions()
    assert "v4attn_compress" in names and "v4attn_hca_attend" in names
    assert len(names) == 29
    for n in names:
        assert hasattr(L(), n), n
    assert L().v4attn_version() == 1
    assert L().v4attn_status_string(-3) == b"workspace missing or too small"


def _compress(**kw):
    a = dict(raw=FAKE, tok_score=FAKE, pos_bias=FAKE, gamma=FAKE, B=1, L=16, D=512, R=64,
             raw_pos0=0, mode=0, m=4, entry0=0, n_out=4, eps=1e-6, base=1e4, out=FAKE,
             out_rows=4, stream=None)
    a.update(kw)
    return L().v4attn_compress(a["raw"], a["tok_score"], a["pos_bias"], a["gamma"], a["B"],
                               a["L"], a["D"], a["R"], a["raw_pos0"], a["mode"], a["m"],
                               a["entry0"], a["n_out"], a["eps"], a["base"], a["out"],
                               a["out_rows"], a.get("ri"), a.get("dI", 0), a.get("ko"),
                               a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(raw=None), -1),
    (dict(D=100), -2),
    (dict(R=32), -2),
    (dict(mode=7), -1),
    (dict(m=0), -2),
    (dict(m=300), -2),
    (dict(n_out=5), -1),                  # n_out > out_rows
    (dict(n_out=4, out_rows=4, L=15), -1),  # last window needs position 15
    (dict(raw_pos0=1), -1),               # entry 0 needs position 0
    (dict(entry0=-1), -1),
    (dict(tok_score=None), -1),
    (dict(raw=MISALIGNED), -1),
    (dict(eps=-1.0), -1),
    (dict(mode=1, n_out=17, out_rows=20), -1),   # PACK beyond L
    (dict(ri=FAKE, dI=128, ko=None), -1),        # pooled indexer keys need an output
    (dict(ri=FAKE, dI=96, ko=FAKE), -1),         # dI not built
])
def test_compress_rejects(kw, status):
    assert _compress(**kw) == status
    assert L().v4attn_last_error() != b""


def _positions(*p):
    return ctypes.cast((ctypes.c_int64 * len(p))(*p), ctypes.c_void_p)


def _step(**kw):
    a = dict(raw=FAKE, s=FAKE, b=FAKE, g=FAKE, B=2, L=8, D=512, R=64, raw_pos0=100, m=4, t=107,
             ent=FAKE, ent_rows=27, win=FAKE, win_rows=128, win_row=127, sp=None)
    a.update(kw)
    return L().v4attn_compress_step(a["raw"], a["s"], a["b"], a["g"], a["B"], a["L"], a["D"],
                                    a["R"], a["raw_pos0"], a["m"], a["t"], a["sp"], 1e-6, 1e4,
                                    a["ent"],
                                    a["ent_rows"], a["win"], a["win_rows"], a["win_row"],
                                    a.get("ri"), a.get("dI", 0), a.get("ko"), None)


@pytest.mark.parametrize("kw,status", [
    (dict(raw=None), -1),
    (dict(win=None), -1),
    (dict(t=108), -1),                 # t outside the raw rows [100, 108)
    (dict(t=99), -1),
    (dict(raw_pos0=101, L=7), -1),     # entry 26's window starts at 100 < raw_pos0
    (dict(ent_rows=26), -1),           # entry 26 needs 27 rows
    (dict(ent=None), -1),              # an entry completes at t = 107
    (dict(win_row=128), -1),
    (dict(m=0), -2),
    (dict(D=384), -2),
    # per-sequence positions: t must be the largest; each sequence's entry checked
    (dict(sp=_positions(107, 99), t=106), -1),
    (dict(sp=_positions(107, -1)), -1),
    (dict(sp=_positions(107, 103), ent_rows=26), -1),   # sequence 0 completes entry 26
    (dict(sp=_positions(107, 103), L=7), -1),           # window of entry 26 needs 8 rows
])
def test_compress_step_rejects(kw, status):
    assert _step(**kw) == status


def test_compress_step_pack_only_needs_no_entry_buffers():
    # t = 106 completes no group: scores, biases and entries may be null.  A
    # bad win_row is rejected on the host before any launch.
    assert _step(t=106, s=None, b=None, ent=None, win_row=-1) == -1


def _index(**kw):
    a = dict(q=FAKE, w=FAKE, k=FAKE, B=2, Tq=1, HI=64, dI=128, Ncap=1000, n=1000, q_pos0=3999,
             m=4, k_=64, topk=FAKE, ts=None, ws=FAKE, ws_bytes=0)
    a.update(kw)
    return L().v4attn_index_topk(a["q"], a["w"], a["k"], a["B"], a["Tq"], a["HI"], a["dI"],
                                 a["Ncap"], a["n"], a["q_pos0"], a.get("sp"), a["m"], a["k_"],
                                 a["topk"],
                                 a["ts"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1),
    (dict(HI=65), -2),
    (dict(dI=96), -2),
    (dict(n=1001), -1),
    (dict(k_=5000), -2),
    (dict(m=0), -2),
    (dict(q_pos0=-1), -1),
    (dict(ws_bytes=10), -3),
    (dict(ws=None, ws_bytes=1 << 40), -3),
])
def test_index_topk_rejects(kw, status):
    assert _index(**kw) == status


def _index_fp8(**kw):
    a = dict(q=FAKE, qs=FAKE, w=FAKE, k=FAKE, ks=FAKE, B=2, Tq=1, HI=64, dI=128, Ncap=1000,
             n=1000, q_pos0=3999, m=4, k_=64, topk=FAKE, ts=None, ws=FAKE, ws_bytes=0)
    a.update(kw)
    return L().v4attn_index_topk_fp8(a["q"], a["qs"], a["w"], a["k"], a["ks"], a["B"], a["Tq"],
                                     a["HI"], a["dI"], a["Ncap"], a["n"], a["q_pos0"], a["m"],
                                     a["k_"], a["topk"], a["ts"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1),
    (dict(qs=None), -1),
    (dict(ks=None), -1),
    (dict(k=MISALIGNED), -1),
    (dict(HI=65), -2),
    (dict(dI=32), -2),
    (dict(n=1001), -1),
    (dict(k_=5000), -2),
    (dict(ws_bytes=10), -3),
])
def test_index_topk_fp8_rejects(kw, status):
    assert _index_fp8(**kw) == status


def test_index_score_fp8_rejects_short_stride():
    # 1000 visible entries need a score row of at least 1000
    st = L().v4attn_index_score_fp8(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 128, 1000, 1000,
                                    3999, 4, FAKE, 999, None)
    assert st == -1


def _index_mxfp4(**kw):
    a = dict(q=FAKE, qs=FAKE, w=FAKE, k=FAKE, ks=FAKE, B=2, Tq=1, HI=64, dI=128, Ncap=1000,
             n=1000, q_pos0=3999, m=4, k_=64, topk=FAKE, ts=None, ws=FAKE, ws_bytes=0)
    a.update(kw)
    return L().v4attn_index_topk_mxfp4(a["q"], a["qs"], a["w"], a["k"], a["ks"], a["B"], a["Tq"],
                                       a["HI"], a["dI"], a["Ncap"], a["n"], a["q_pos0"], a["m"],
                                       a["k_"], a["topk"], a["ts"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1),
    (dict(qs=None), -1),
    (dict(ks=None), -1),
    (dict(k=MISALIGNED), -1),
    (dict(ks=ctypes.c_void_p(0x100002)), -1),   # 4 scale bytes per key: 4-byte aligned
    (dict(HI=65), -2),
    (dict(dI=32), -2),
    (dict(n=1001), -1),
    (dict(ws_bytes=10), -3),
])
def test_index_topk_mxfp4_rejects(kw, status):
    assert _index_mxfp4(**kw) == status


def test_workspace_sizes_are_host_arithmetic():
    # 1M-token decode: 8 queries x 262144 fp32 scores plus two candidate buffers
    n = L().v4attn_index_topk_workspace(8, 1, 262144, (1 << 20) - 1, 4, 1024)
    assert n >= 8 * 262144 * 4
    assert L().v4attn_index_topk_workspace(-1, 1, 10, 0, 4, 1) == 0
    # many queries need no split partials
    assert L().v4attn_csa_attend_workspace(4096, 1, 64, 512, 1024, 128) == 0
    assert L().v4attn_hca_attend_workspace(32, 1, 64, 512, 8192, 128, (1 << 20) - 1, 128) > 0


def test_backward_workspaces_hold_the_grouped_gradients():
    """The backward workspace queries include the dense per-slot gradients
    and the sort buffers of one group (all queries, under 12 GiB), so they
    grow with the number of queries and destination rows; past 32-bit slot
    or destination ids the grouped path is off and the query returns the
    per-chunk part alone."""
    csa = L().v4attn_csa_attend_backward_workspace
    # 4096 queries x (1024 + 128) rows x 512 dims, 3 bytes a value = 7.25 GB of dense dX
    dense = 4096 * 1152 * 512 * 3
    n = csa(1, 4096, 64, 512, 1024, 128, 262144)
    assert dense < n < (12 << 30) + (2 << 30)
    assert csa(1, 64, 64, 512, 1024, 128, 262144) < n          # one chunk
    assert csa(1, 4096, 64, 512, 1024, 128, 1 << 20) > n       # more destinations
    base = csa(1, 4096, 64, 512, 1024, 128, 1 << 31)          # ids past 2^31: atomics
    assert base < dense < n
    assert csa(1, 4096, 64, 512, 1024, 128, -1) == 0
    hca = L().v4attn_hca_attend_backward_workspace
    assert hca(2, 8, 64, 512, 300, 128, 300 * 128 + 5, 16, 300) > 0
    kl = L().v4attn_index_kl_backward_workspace
    n = kl(1, 4096, 128, 1024, 262144)                         # 1.6 GB of dense dk, 3 bytes a value
    assert 4096 * 1024 * 128 * 3 < n
    assert kl(1, 4096, 128, 1024, 1 << 31) < 4096 * 1024 * 128 * 3
    assert kl(1, 4096, 128, 1024, -1) == 0


def _csa(**kw):
    a = dict(q=FAKE, e=FAKE, t=FAKE, w=FAKE, g=FAKE, s=FAKE, B=1, Tq=1, H=64, D=512, R=64,
             Ncap=100, k=64, W=128, q_pos0=500, scale=0.04, eps=1e-6, base=1e4, out=FAKE,
             lse=None, ws=FAKE, ws_bytes=0)
    a.update(kw)
    return L().v4attn_csa_attend(a["q"], a["e"], a["t"], a["w"], a["g"], a["s"], a["B"], a["Tq"],
                                 a["H"], a["D"], a["R"], a["Ncap"], a["k"], a["W"], a["q_pos0"],
                                 a.get("sp"), a["scale"], a["eps"], a["base"], a["out"], a["lse"],
                                 a["ws"],
                                 a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1),
    (dict(t=None), -1),
    (dict(H=0), -2),
    (dict(H=65), -2),
    (dict(D=384), -2),
    (dict(k=0), -2),
    (dict(W=5000), -2),
    (dict(W=16, w=None), -1),
    (dict(scale=float("nan")), -1),
    (dict(out=MISALIGNED), -1),
    (dict(q_pos0=-5), -1),
    (dict(sp=_positions(500, 501), B=2), -1),  # q_pos0 is not the largest position
    (dict(sp=_positions(*range(65)), B=65, q_pos0=64), -2),   # more sequences than built
])
def test_csa_attend_rejects(kw, status):
    assert _csa(**kw) == status


def test_hca_attend_rejects():
    f = L().v4attn_hca_attend
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 512, 64, 10, 11, 128, 128, 5000, None, 0.04,
            1e-6, 1e4, FAKE, None, FAKE, 0, None]
    assert f(*args) == -1          # n_entries > Ncap
    args[11] = 10
    args[12] = 0
    assert f(*args) == -2          # m = 0
    args[12] = 128
    args[22] = 0
    # 32 sequences at 1M need split partials: workspace too small
    args[5], args[10], args[11], args[14] = 32, 8192, 8192, (1 << 20) - 1
    assert f(*args) == -3


def test_hca_attend_noalloc_rejects_before_any_device_call():
    f = L().v4attn_hca_attend_noalloc
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 512, 64, 10, 11, 128, 128, 5000, None, 0.04,
            1e-6, 1e4, FAKE, None, None]
    assert f(*args) == -1          # n_entries > Ncap
    args[11] = 10
    args[12] = 0
    assert f(*args) == -2          # m = 0
    args[12] = 128
    # 255 queries over 328 rows: two splits of partials, 33.5 MB > the 24 MiB scratch
    args[5], args[10], args[11], args[14] = 255, 200, 200, 200 * 128 + 5
    assert f(*args) == -3
    assert b"scratch" in L().v4attn_last_error()


def _nsa(**kw):
    a = dict(q=FAKE, e=FAKE, tok=FAKE, w=FAKE, g=FAKE, gates=FAKE, B=1, Tq=1, H=64, D=512, R=64,
             Ncap=100, n_entries=100, m=4, Ntok=400, W=128, n_sel=16, q_pos0=500, scale=0.04,
             eps=1e-6, base=1e4, out=FAKE, blocks=None, bscore=None, ws=FAKE, ws_bytes=1 << 40)
    a.update(kw)
    return L().v4attn_nsa_attend(a["q"], a["e"], a["tok"], a["w"], a["g"], a["gates"], a["B"],
                                 a["Tq"], a["H"], a["D"], a["R"], a["Ncap"], a["n_entries"],
                                 a["m"], a["Ntok"], a["W"], a["n_sel"], a["q_pos0"], a["scale"],
                                 a["eps"], a["base"], a["out"], a["blocks"], a["bscore"], a["ws"],
                                 a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(gates=None), -1),
    (dict(tok=None), -1),
    (dict(tok=MISALIGNED), -1),
    (dict(n_entries=101), -1),            # more entries than the cache holds
    (dict(m=0), -2),
    (dict(n_sel=0), -2),
    (dict(n_sel=2048, m=4), -2),          # n_sel m > 4096 token slots
    (dict(Ntok=399), -1),                 # the last visible block's tokens are missing
    (dict(H=65), -2),
    (dict(ws_bytes=16), -3),
    (dict(ws=MISALIGNED), -1),
])
def test_nsa_attend_rejects(kw, status):
    assert _nsa(**kw) == status


def test_nsa_workspace_holds_the_compressed_logits():
    # 8 queries x 64 heads x 8192 visible entries (1M context, m = 128) of fp32 logits
    n = L().v4attn_nsa_attend_workspace(8, 1, 64, 512, 8192, 128, (1 << 20) - 1, 128, 16)
    assert n >= 8 * 64 * 8192 * 4
    assert L().v4attn_nsa_attend_workspace(8, 1, 64, 512, 8192, 128, 0, 128, 0) == 0
