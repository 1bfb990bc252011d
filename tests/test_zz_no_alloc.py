"""v4attn_hca_attend_noalloc (the HCA attention with its split partials in
the library's fixed device scratch) against v4attn_hca_attend (the same call
with a caller workspace), through the C ABI: identical outputs and lse on
two calls in a row, the second with a smaller input, and the first call also
against the float64 oracle on sampled sequences."""

import numpy as np
import pytest
import torch

from long_context_sparse_csa_amd import synth
from oracle import attend as oa

from helpers import assert_attn_close, bf16_to_f64, rows_to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from long_context_sparse_csa_amd import ops
    ops.lib()
    yield


def ops():
    from long_context_sparse_csa_amd import ops as o
    return o


def _inputs(B, H, D, N, W, seed):
    R = 64
    q = synth.normal((B, 1, H, D), seed, "q", DEV, dtype=torch.bfloat16)
    ent = synth.packed_rows((B, max(N, 1)), D, R, seed, "entries", DEV)
    win = synth.packed_rows((B, W), D, R, seed, "win", DEV)
    gq = synth.normal((D,), seed, "gamma_q", DEV, mean=1.0, std=0.1)
    sink = synth.normal((H,), seed, "sink", DEV)
    return q, ent, win, gq, sink


# (B, H, D, n_entries, m, t): the 1M-context decode launch (8 splits of 9
# tiles), then a smaller one (4 splits) that leaves the first call's
# partials behind it in the scratch
CALLS = [(32, 64, 512, 8192, 128, (1 << 20) - 1), (4, 64, 512, 500, 128, 500 * 128 + 7)]


def test_noalloc_matches_workspace_call_twice():
    W = 128
    for i, (B, H, D, N, m, t) in enumerate(CALLS):
        print(f"noalloc call {i}: B={B} N={N} t={t}", flush=True)
        q, ent, win, gq, sink = _inputs(B, H, D, N, W, 40 + i)
        assert ops().hca_attend_workspace_bytes(B, 1, H, D, N, m, t, W) > 0, "splits expected"
        out = torch.empty_like(q)
        lse = torch.empty((B, 1, H), dtype=torch.float32, device=DEV)
        ops().hca_attend_noalloc(q, ent, win, gq, sink, n_entries=N, m=m, q_pos0=t, W=W,
                                 out=out, lse=lse)
        ref, ref_lse = ops().hca_attend(q, ent, win, gq, sink, n_entries=N, m=m, q_pos0=t, W=W,
                                        want_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"call {i}: output differs from the workspace call"
        assert torch.equal(lse, ref_lse), f"call {i}: lse differs from the workspace call"
        for b in (0, B - 1):
            rows = np.concatenate([rows_to_f64(ent[b, :N], D, 64), rows_to_f64(win[b], D, 64)])
            o, _, _ = oa.attend_rows(bf16_to_f64(q[b, 0]), gq.cpu().double().numpy(), t, rows,
                                     sink.cpu().double().numpy(), D ** -0.5, 1e-6, 64, 1e4)
            assert_attn_close(bf16_to_f64(out[b, 0]), o, f"noalloc call {i} b={b}")


def test_noalloc_rejects_partials_beyond_the_scratch():
    """255 queries over 328 rows need two splits of partials (33.5 MB), more
    than the 24 MiB scratch: an error, nothing launched."""
    B, H, D, N, m, t, W = 255, 64, 512, 200, 128, 200 * 128 + 5, 128
    q, ent, win, gq, sink = _inputs(B, H, D, N, W, 7)
    need = ops().hca_attend_workspace_bytes(B, 1, H, D, N, m, t, W)
    assert need > ops().lib().v4attn_hca_attend_workspace(32, 1, H, D, N, m, t, W)
    assert need > (24 << 20)
    with pytest.raises(ops().V4AttnError) as ei:
        ops().hca_attend_noalloc(q, ent, win, gq, sink, n_entries=N, m=m, q_pos0=t, W=W)
    assert ei.value.status == ops().V4ATTN_EWORKSPACE
