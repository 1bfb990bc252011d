"""Thin ctypes binding over libv4attn.so (include/v4attn.h).

Argument marshalling only: shape/dtype checks, pointer and stream extraction,
output and workspace allocation through torch.  Every step of the method runs
in the library's HIP kernels; there is no fallback.  If the library is
missing this module raises on first use.
"""

import ctypes
import os
import re

import torch

from . import LIB_PATH, PACKAGE_DIR

V4ATTN_OK = 0
V4ATTN_EINVAL = -1
V4ATTN_EUNSUPPORTED = -2
V4ATTN_EWORKSPACE = -3
V4ATTN_EHIP = -4
POOL = 0
PACK = 1

HEADER = os.path.join(os.path.dirname(PACKAGE_DIR), "include", "v4attn.h")

_c = ctypes
_P = _c.c_void_p
_I = _c.c_int
_L = _c.c_int64
_F = _c.c_float
_Z = _c.c_size_t

_SIGS = {
    "v4attn_version": (_I, []),
    "v4attn_status_string": (_c.c_char_p, [_I]),
    "v4attn_last_error": (_c.c_char_p, []),
    "v4attn_compress": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _L, _I, _I, _L, _I, _F, _F, _P, _L,
                             _P, _I, _P, _P]),
    "v4attn_compress_step": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _L, _I, _L, _P, _F, _F, _P, _L,
                                  _P, _L, _L, _P, _I, _P, _P]),
    "v4attn_compress_steps": (_I, [_P, _I, _P]),
    "v4attn_index_topk_workspace": (_Z, [_I, _I, _L, _L, _I, _I]),
    "v4attn_index_topk": (_I, [_P, _P, _P, _I, _I, _I, _I, _L, _L, _L, _P, _I, _I, _P, _P, _P, _Z,
                               _P]),
    "v4attn_index_score": (_I, [_P, _P, _P, _I, _I, _I, _I, _L, _L, _L, _P, _I, _P, _L, _P]),
    "v4attn_index_score_fp8": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _L, _L, _L, _I, _P, _L,
                                    _P]),
    "v4attn_index_topk_fp8": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _L, _L, _L, _I, _I, _P,
                                   _P, _P, _Z, _P]),
    "v4attn_index_score_mxfp4": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _L, _L, _L, _I, _P,
                                      _L, _P]),
    "v4attn_index_topk_mxfp4": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _L, _L, _L, _I, _I, _P,
                                     _P, _P, _Z, _P]),
    "v4attn_topk_select_workspace": (_Z, [_I, _I, _L, _L, _I, _I]),
    "v4attn_topk_select": (_I, [_P, _L, _I, _I, _L, _L, _P, _I, _I, _P, _P, _P, _Z, _P]),
    "v4attn_csa_attend_workspace": (_Z, [_I, _I, _I, _I, _I, _I]),
    "v4attn_csa_attend": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _L, _I, _I, _L, _P,
                               _F, _F, _F, _P, _P, _P, _Z, _P]),
    "v4attn_hca_attend_workspace": (_Z, [_I, _I, _I, _I, _L, _I, _L, _I]),
    "v4attn_hca_attend": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _L, _L, _I, _I, _L, _P,
                               _F, _F, _F, _P, _P, _P, _Z, _P]),
    "v4attn_hca_attend_noalloc": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _L, _L, _I, _I, _L,
                                       _P, _F, _F, _F, _P, _P, _P]),
    "v4attn_csa_attend_backward_workspace": (_Z, [_I, _I, _I, _I, _I, _I, _L]),
    "v4attn_csa_attend_backward": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _L, _I, _I,
                                        _L, _F, _F, _F, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                        _Z, _P]),
    "v4attn_compress_backward": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _L, _I, _L, _I, _F, _F, _P,
                                      _P, _P, _P, _P, _P]),
    "v4attn_index_kl_backward_workspace": (_Z, [_I, _I, _I, _I, _L]),
    "v4attn_index_kl_backward": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _L, _I, _P, _P, _P, _P,
                                      _P, _Z, _P]),
    "v4attn_hca_attend_backward_workspace": (_Z, [_I, _I, _I, _I, _L, _I, _L, _I, _L]),
    "v4attn_hca_attend_backward": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _L, _L, _I, _I,
                                        _L, _F, _F, _F, _P, _P, _P, _P, _P, _P, _P, _P, _P, _Z,
                                        _P]),
    "v4attn_nsa_attend_workspace": (_Z, [_I, _I, _I, _I, _L, _I, _L, _I, _I]),
    "v4attn_nsa_attend": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _L, _L, _I, _L, _I,
                               _I, _L, _F, _F, _F, _P, _P, _P, _P, _Z, _P]),
}

class CompressStepDesc(_c.Structure):
    """v4attn_compress_step_desc: one layer's decode-step arguments."""
    _fields_ = [("raw", _c.c_void_p), ("tok_score", _c.c_void_p), ("pos_bias", _c.c_void_p),
                ("gamma", _c.c_void_p), ("B", _c.c_int), ("L", _c.c_int), ("D", _c.c_int),
                ("R", _c.c_int), ("raw_pos0", _c.c_int64), ("m", _c.c_int), ("t", _c.c_int64),
                ("seq_pos", _c.c_void_p), ("eps", _c.c_float), ("rope_base", _c.c_float),
                ("entries", _c.c_void_p), ("ent_rows", _c.c_int64), ("win", _c.c_void_p),
                ("win_rows", _c.c_int64), ("win_row", _c.c_int64), ("raw_idx", _c.c_void_p),
                ("dI", _c.c_int), ("k_idx", _c.c_void_p)]


_lib = None


class V4AttnError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"v4attn status {status}: {msg}")
        self.status = status


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m long_context_sparse_csa_amd.build` (no CPU fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def header_functions():
    """Names of the functions include/v4attn.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(v4attn_\w+)\s*\(", text)))


def check(status):
    if status != V4ATTN_OK:
        msg = lib().v4attn_last_error().decode()
        raise V4AttnError(status, msg)


def _ptr(t):
    return None if t is None else _c.c_void_p(t.data_ptr())


def _stream(t):
    return _c.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(t, name, dtype, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


_ARRAY_TYPES = {}


def _int64_array(n):
    """The ctypes type int64[n], made once per n: a new array type per call
    is a class object with reference cycles, and cyclic garbage sets off the
    interpreter's full garbage collections (tens of milliseconds each, inside
    whatever loop is launching)."""
    t = _ARRAY_TYPES.get(n)
    if t is None:
        t = _ARRAY_TYPES[n] = _c.c_int64 * n
    return t


def _desc_array(n):
    """CompressStepDesc[n], made once per n (see _int64_array)."""
    key = ("desc", n)
    t = _ARRAY_TYPES.get(key)
    if t is None:
        t = _ARRAY_TYPES[key] = CompressStepDesc * n
    return t


def _seq_pos(seq_pos, B, q_pos0):
    """Per-sequence positions as a host int64 array (kept alive by the
    caller for the call) and the q_pos0 the library expects with it (their
    largest)."""
    if seq_pos is None:
        if q_pos0 is None:
            raise ValueError("q_pos0 (or seq_pos) is required")
        return None, None, int(q_pos0)
    sp = [int(x) for x in seq_pos]
    if len(sp) != B:
        raise ValueError(f"seq_pos has {len(sp)} positions for {B} sequences")
    arr = _int64_array(max(B, 1))(*sp)
    # the address, not ctypes.cast (which ties the two objects in a reference
    # cycle); the caller keeps arr alive for the call
    return arr, _c.c_void_p(_c.addressof(arr)), max(sp) if sp else int(q_pos0 or 0)


def _workspace(nbytes, device, ws):
    if nbytes == 0:
        return ws
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return ws


# ------------------------------------------------------------------ compress --

def _row_ptr(out, row0, row_bytes):
    if row0 < 0 or row0 > out.shape[1]:
        raise ValueError("out_row0 out of range")
    return _c.c_void_p(out.data_ptr() + row0 * row_bytes)


def _kidx_args(raw_idx, k_idx, B, L, row0):
    """(raw_idx ptr, dI, k_idx row pointer) for the pooled indexer keys."""
    if raw_idx is None:
        return None, 0, None
    _need(raw_idx, "raw_idx", torch.bfloat16, 3)
    _need(k_idx, "k_idx", torch.bfloat16, 3)
    dI = raw_idx.shape[2]
    if tuple(raw_idx.shape[:2]) != (B, L) or k_idx.shape[0] != B or k_idx.shape[2] != dI:
        raise ValueError("shape mismatch")
    return _ptr(raw_idx), dI, _c.c_void_p(k_idx.data_ptr() + row0 * dI * 2)


def compress_pool(raw, tok_score, pos_bias, gamma, out, *, raw_pos0, m, entry0, n_out,
                  out_row0=0, eps=1e-6, rope_base=10000.0, R=64, raw_idx=None, k_idx=None):
    """Pool 2m-token windows of raw bf16 latents [B, L, D] into packed entries
    entry0..entry0+n_out-1, written to out[b, out_row0 + i] (uint8 [B, rows, D+R]).
    With raw_idx (bf16 [B, L, dI], the tokens' indexer keys) the entries'
    indexer keys, pooled with the same weights, go to k_idx[b, out_row0 + i]."""
    _need(raw, "raw", torch.bfloat16, 3)
    _need(tok_score, "tok_score", torch.float32, 2)
    _need(pos_bias, "pos_bias", torch.float32, 1)
    _need(gamma, "gamma", torch.float32, 1)
    _need(out, "out", torch.uint8, 3)
    B, L, D = raw.shape
    if tuple(tok_score.shape) != (B, L) or pos_bias.numel() != 2 * m or gamma.numel() != D \
            or out.shape[0] != B or out.shape[2] != D + R or out_row0 + n_out > out.shape[1]:
        raise ValueError("shape mismatch")
    ri, dI, kp = _kidx_args(raw_idx, k_idx, B, L, out_row0)
    if raw_idx is not None and k_idx.shape[1] != out.shape[1]:
        raise ValueError("k_idx must have out's rows")
    check(lib().v4attn_compress(_ptr(raw), _ptr(tok_score), _ptr(pos_bias), _ptr(gamma), B, L, D,
                                R, int(raw_pos0), POOL, int(m), int(entry0), int(n_out),
                                float(eps), float(rope_base), _row_ptr(out, out_row0, D + R),
                                out.shape[1], ri, dI, kp, _stream(raw)))
    return out


def compress_step(raw, tok_score, pos_bias, gamma, entries, win, *, m, win_row, raw_pos0=None,
                  t=None, seq_pos=None, eps=1e-6, rope_base=10000.0, R=64, raw_idx=None,
                  k_idx=None):
    """One decode step of the compressor in one launch: the window row of the
    token at position t -> win[b, win_row], and, when (t+1) % m == 0, the
    entry j = (t+1)/m - 1 it completes -> entries[b, j].  With seq_pos (one
    position per sequence) each sequence's raw rows are the L positions
    ending at its own token.  With raw_idx (bf16 [B, L, dI]) a completed
    entry's pooled indexer key goes to k_idx[b, j] (bf16 [B, rows, dI])."""
    _need(raw, "raw", torch.bfloat16, 3)
    _need(tok_score, "tok_score", torch.float32, 2)
    _need(pos_bias, "pos_bias", torch.float32, 1)
    _need(gamma, "gamma", torch.float32, 1)
    _need(entries, "entries", torch.uint8, 3)
    _need(win, "win", torch.uint8, 3)
    B, L, D = raw.shape
    if tuple(tok_score.shape) != (B, L) or pos_bias.numel() != 2 * m or gamma.numel() != D \
            or entries.shape[0] != B or entries.shape[2] != D + R or win.shape[0] != B \
            or win.shape[2] != D + R:
        raise ValueError("shape mismatch")
    arr, sp, t = _seq_pos(seq_pos, B, t)
    raw_pos0 = t - L + 1 if raw_pos0 is None else raw_pos0
    ri, dI, kp = _kidx_args(raw_idx, k_idx, B, L, 0)
    if raw_idx is not None and k_idx.shape[1] != entries.shape[1]:
        raise ValueError("k_idx must have the entries' rows")
    check(lib().v4attn_compress_step(_ptr(raw), _ptr(tok_score), _ptr(pos_bias), _ptr(gamma), B, L,
                                     D, R, int(raw_pos0), int(m), int(t), sp, float(eps),
                                     float(rope_base), _ptr(entries), entries.shape[1], _ptr(win),
                                     win.shape[1], int(win_row), ri, dI, kp, _stream(raw)))
    return entries, win


def compress_steps(layers):
    """compress_step for several layers (each a dict of compress_step's
    arguments; same D) in one launch."""
    descs = _desc_array(len(layers))()
    keep = []
    for z, kw in enumerate(layers):
        kw = dict(kw)
        raw, ts, pb, gm = kw.pop("raw"), kw.pop("tok_score"), kw.pop("pos_bias"), kw.pop("gamma")
        ent, win = kw.pop("entries"), kw.pop("win")
        m, win_row = kw.pop("m"), kw.pop("win_row")
        R = kw.pop("R", 64)
        B, L, D = raw.shape
        arr, sp, t = _seq_pos(kw.pop("seq_pos", None), B, kw.pop("t", None))
        raw_pos0 = kw.pop("raw_pos0", None)
        raw_pos0 = t - L + 1 if raw_pos0 is None else raw_pos0
        raw_idx, k_idx = kw.pop("raw_idx", None), kw.pop("k_idx", None)
        eps, base = kw.pop("eps", 1e-6), kw.pop("rope_base", 10000.0)
        if kw:
            raise ValueError(f"unknown arguments {sorted(kw)}")
        ri, dI, kp = _kidx_args(raw_idx, k_idx, B, L, 0)
        keep.append(arr)
        d = descs[z]
        d.raw, d.tok_score, d.pos_bias, d.gamma = (raw.data_ptr(), ts.data_ptr(), pb.data_ptr(),
                                                   gm.data_ptr())
        d.B, d.L, d.D, d.R = B, L, D, R
        d.raw_pos0, d.m, d.t, d.seq_pos = int(raw_pos0), int(m), int(t), sp
        d.eps, d.rope_base = float(eps), float(base)
        d.entries, d.ent_rows, d.win, d.win_rows = (ent.data_ptr(), ent.shape[1], win.data_ptr(),
                                                    win.shape[1])
        d.win_row, d.raw_idx, d.dI, d.k_idx = int(win_row), ri, dI, kp
    check(lib().v4attn_compress_steps(_c.c_void_p(_c.addressof(descs)), len(layers),
                                      _stream(layers[0]["raw"])))


def compress_pack(raw, gamma, out, *, raw_pos0, n_out=None, out_row0=0, eps=1e-6,
                  rope_base=10000.0, R=64):
    """Pack raw rows 0..n_out-1 (positions raw_pos0..) as window rows, written
    to out[b, out_row0 + i]."""
    _need(raw, "raw", torch.bfloat16, 3)
    _need(gamma, "gamma", torch.float32, 1)
    _need(out, "out", torch.uint8, 3)
    B, L, D = raw.shape
    n_out = L if n_out is None else n_out
    if gamma.numel() != D or out.shape[0] != B or out.shape[2] != D + R \
            or out_row0 + n_out > out.shape[1]:
        raise ValueError("shape mismatch")
    check(lib().v4attn_compress(_ptr(raw), None, None, _ptr(gamma), B, L, D, R, int(raw_pos0),
                                PACK, 1, 0, int(n_out), float(eps), float(rope_base),
                                _row_ptr(out, out_row0, D + R), out.shape[1], None, 0, None,
                                _stream(raw)))
    return out


# ----------------------------------------------------------------- index/topk --

def index_topk_workspace_bytes(B, Tq, n_entries, q_pos0, m, k):
    return lib().v4attn_index_topk_workspace(B, Tq, n_entries, q_pos0, m, k)


def index_topk(q_idx, w_idx, k_idx, *, n_entries, m, k, q_pos0=None, seq_pos=None, topk=None,
               topk_score=None, want_scores=False, workspace=None):
    """Top-k entry indices per query (int32 [B, Tq, k], ascending, -1 padded)."""
    _need(q_idx, "q_idx", torch.bfloat16, 4)
    _need(w_idx, "w_idx", torch.float32, 3)
    _need(k_idx, "k_idx", torch.bfloat16, 3)
    B, Tq, HI, dI = q_idx.shape
    Ncap = k_idx.shape[1]
    if tuple(w_idx.shape) != (B, Tq, HI) or k_idx.shape[0] != B or k_idx.shape[2] != dI:
        raise ValueError("shape mismatch")
    dev = q_idx.device
    if topk is None:
        topk = torch.empty((B, Tq, k), dtype=torch.int32, device=dev)
    _need(topk, "topk", torch.int32, 3)
    if want_scores and topk_score is None:
        topk_score = torch.empty((B, Tq, k), dtype=torch.float32, device=dev)
    arr, sp, q_pos0 = _seq_pos(seq_pos, B, q_pos0)
    nbytes = index_topk_workspace_bytes(B, Tq, n_entries, q_pos0, m, k)
    workspace = _workspace(nbytes, dev, workspace)
    check(lib().v4attn_index_topk(_ptr(q_idx), _ptr(w_idx), _ptr(k_idx), B, Tq, HI, dI, Ncap,
                                  int(n_entries), int(q_pos0), sp, int(m), int(k), _ptr(topk),
                                  _ptr(topk_score), _ptr(workspace), nbytes, _stream(q_idx)))
    return topk, topk_score


def score_stride(Tq, n_entries, q_pos0, m):
    """Smallest score row length index_score accepts (rounded up to 64)."""
    v = min(n_entries, (q_pos0 + Tq) // m) if Tq > 0 else 0
    return (v + 63) // 64 * 64


def index_score(q_idx, w_idx, k_idx, *, n_entries, m, q_pos0=None, seq_pos=None, scores=None):
    """Indexer scores f32 [B*Tq, stride]; row b*Tq+r is valid for j < V_t."""
    _need(q_idx, "q_idx", torch.bfloat16, 4)
    _need(w_idx, "w_idx", torch.float32, 3)
    _need(k_idx, "k_idx", torch.bfloat16, 3)
    B, Tq, HI, dI = q_idx.shape
    if tuple(w_idx.shape) != (B, Tq, HI) or k_idx.shape[0] != B or k_idx.shape[2] != dI:
        raise ValueError("shape mismatch")
    arr, sp, q_pos0 = _seq_pos(seq_pos, B, q_pos0)
    if scores is None:
        scores = torch.empty((B * Tq, max(score_stride(Tq, n_entries, q_pos0, m), 1)),
                             dtype=torch.float32, device=q_idx.device)
    _need(scores, "scores", torch.float32, 2)
    check(lib().v4attn_index_score(_ptr(q_idx), _ptr(w_idx), _ptr(k_idx), B, Tq, HI, dI,
                                   k_idx.shape[1], int(n_entries), int(q_pos0), sp, int(m),
                                   _ptr(scores), scores.shape[1], _stream(q_idx)))
    return scores


def _fp8_inputs(q8, q_scale, w_idx, k8, k_scale):
    _need(q8, "q8", torch.uint8, 4)
    _need(q_scale, "q_scale", torch.float32, 3)
    _need(w_idx, "w_idx", torch.float32, 3)
    _need(k8, "k8", torch.uint8, 3)
    _need(k_scale, "k_scale", torch.float32, 2)
    B, Tq, HI, dI = q8.shape
    if tuple(q_scale.shape) != (B, Tq, HI) or tuple(w_idx.shape) != (B, Tq, HI) \
            or k8.shape[0] != B or k8.shape[2] != dI or tuple(k_scale.shape) != tuple(k8.shape[:2]):
        raise ValueError("shape mismatch")
    return B, Tq, HI, dI, k8.shape[1]


def index_score_fp8(q8, q_scale, w_idx, k8, k_scale, *, n_entries, q_pos0, m, scores=None):
    """FP8 indexer scores f32 [B*Tq, stride] from E4M3 codes (uint8) and
    per-row fp32 scales; row b*Tq+r is valid for j < V_t."""
    B, Tq, HI, dI, Ncap = _fp8_inputs(q8, q_scale, w_idx, k8, k_scale)
    if scores is None:
        scores = torch.empty((B * Tq, max(score_stride(Tq, n_entries, q_pos0, m), 1)),
                             dtype=torch.float32, device=q8.device)
    _need(scores, "scores", torch.float32, 2)
    check(lib().v4attn_index_score_fp8(_ptr(q8), _ptr(q_scale), _ptr(w_idx), _ptr(k8),
                                       _ptr(k_scale), B, Tq, HI, dI, Ncap, int(n_entries),
                                       int(q_pos0), int(m), _ptr(scores), scores.shape[1],
                                       _stream(q8)))
    return scores


def index_topk_fp8(q8, q_scale, w_idx, k8, k_scale, *, n_entries, q_pos0, m, k, topk=None,
                   topk_score=None, want_scores=False, workspace=None):
    """Top-k entry indices per query from the FP8 indexer (int32 [B, Tq, k])."""
    B, Tq, HI, dI, Ncap = _fp8_inputs(q8, q_scale, w_idx, k8, k_scale)
    dev = q8.device
    if topk is None:
        topk = torch.empty((B, Tq, k), dtype=torch.int32, device=dev)
    _need(topk, "topk", torch.int32, 3)
    if want_scores and topk_score is None:
        topk_score = torch.empty((B, Tq, k), dtype=torch.float32, device=dev)
    nbytes = index_topk_workspace_bytes(B, Tq, n_entries, q_pos0, m, k)
    workspace = _workspace(nbytes, dev, workspace)
    check(lib().v4attn_index_topk_fp8(_ptr(q8), _ptr(q_scale), _ptr(w_idx), _ptr(k8),
                                      _ptr(k_scale), B, Tq, HI, dI, Ncap, int(n_entries),
                                      int(q_pos0), int(m), int(k), _ptr(topk), _ptr(topk_score),
                                      _ptr(workspace), nbytes, _stream(q8)))
    return topk, topk_score


def _mxfp4_inputs(q4, q_sc, w_idx, k4, k_sc):
    _need(q4, "q4", torch.uint8, 4)
    _need(q_sc, "q_sc", torch.uint8, 4)
    _need(w_idx, "w_idx", torch.float32, 3)
    _need(k4, "k4", torch.uint8, 3)
    _need(k_sc, "k_sc", torch.uint8, 3)
    B, Tq, HI, half = q4.shape
    dI = 2 * half
    if tuple(q_sc.shape) != (B, Tq, HI, dI // 32) or tuple(w_idx.shape) != (B, Tq, HI) \
            or k4.shape[0] != B or k4.shape[2] != half \
            or tuple(k_sc.shape) != (B, k4.shape[1], dI // 32):
        raise ValueError("shape mismatch")
    return B, Tq, HI, dI, k4.shape[1]


def index_score_mxfp4(q4, q_sc, w_idx, k4, k_sc, *, n_entries, q_pos0, m, scores=None):
    """MXFP4 indexer scores f32 [B*Tq, stride] from packed E2M1 codes (uint8,
    two per byte) and E8M0 block scales (uint8, one per 32 dims)."""
    B, Tq, HI, dI, Ncap = _mxfp4_inputs(q4, q_sc, w_idx, k4, k_sc)
    if scores is None:
        scores = torch.empty((B * Tq, max(score_stride(Tq, n_entries, q_pos0, m), 1)),
                             dtype=torch.float32, device=q4.device)
    _need(scores, "scores", torch.float32, 2)
    check(lib().v4attn_index_score_mxfp4(_ptr(q4), _ptr(q_sc), _ptr(w_idx), _ptr(k4), _ptr(k_sc),
                                         B, Tq, HI, dI, Ncap, int(n_entries), int(q_pos0), int(m),
                                         _ptr(scores), scores.shape[1], _stream(q4)))
    return scores


def index_topk_mxfp4(q4, q_sc, w_idx, k4, k_sc, *, n_entries, q_pos0, m, k, topk=None,
                     topk_score=None, want_scores=False, workspace=None):
    """Top-k entry indices per query from the MXFP4 indexer (int32 [B, Tq, k])."""
    B, Tq, HI, dI, Ncap = _mxfp4_inputs(q4, q_sc, w_idx, k4, k_sc)
    dev = q4.device
    if topk is None:
        topk = torch.empty((B, Tq, k), dtype=torch.int32, device=dev)
    _need(topk, "topk", torch.int32, 3)
    if want_scores and topk_score is None:
        topk_score = torch.empty((B, Tq, k), dtype=torch.float32, device=dev)
    nbytes = index_topk_workspace_bytes(B, Tq, n_entries, q_pos0, m, k)
    workspace = _workspace(nbytes, dev, workspace)
    check(lib().v4attn_index_topk_mxfp4(_ptr(q4), _ptr(q_sc), _ptr(w_idx), _ptr(k4), _ptr(k_sc),
                                        B, Tq, HI, dI, Ncap, int(n_entries), int(q_pos0), int(m),
                                        int(k), _ptr(topk), _ptr(topk_score), _ptr(workspace),
                                        nbytes, _stream(q4)))
    return topk, topk_score


def topk_select_workspace_bytes(B, Tq, n_entries, q_pos0, m, k):
    return lib().v4attn_topk_select_workspace(B, Tq, n_entries, q_pos0, m, k)


def topk_select(scores, *, B, Tq, n_entries, m, k, q_pos0=None, seq_pos=None, topk=None,
                topk_score=None, want_scores=False, workspace=None):
    """Top-k selection from an index_score buffer."""
    _need(scores, "scores", torch.float32, 2)
    dev = scores.device
    if topk is None:
        topk = torch.empty((B, Tq, k), dtype=torch.int32, device=dev)
    _need(topk, "topk", torch.int32, 3)
    if want_scores and topk_score is None:
        topk_score = torch.empty((B, Tq, k), dtype=torch.float32, device=dev)
    arr, sp, q_pos0 = _seq_pos(seq_pos, B, q_pos0)
    nbytes = topk_select_workspace_bytes(B, Tq, n_entries, q_pos0, m, k)
    workspace = _workspace(nbytes, dev, workspace)
    check(lib().v4attn_topk_select(_ptr(scores), scores.shape[1], B, Tq, int(n_entries),
                                   int(q_pos0), sp, int(m), int(k), _ptr(topk), _ptr(topk_score),
                                   _ptr(workspace), nbytes, _stream(scores)))
    return topk, topk_score


# ------------------------------------------------------------------- attention --

def _attend_io(q, out, lse, want_lse):
    B, Tq, H, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, 4)
    if want_lse and lse is None:
        lse = torch.empty((B, Tq, H), dtype=torch.float32, device=q.device)
    return out, lse


def csa_attend_workspace_bytes(B, Tq, H, D, k, W):
    return lib().v4attn_csa_attend_workspace(B, Tq, H, D, k, W)


def hca_attend_workspace_bytes(B, Tq, H, D, n_entries, m, q_pos0, W):
    return lib().v4attn_hca_attend_workspace(B, Tq, H, D, n_entries, m, q_pos0, W)


def csa_attend(q, entries, topk, win, gamma_q, sink, *, W, q_pos0=None, seq_pos=None,
               scale=None, eps=1e-6, rope_base=10000.0, R=64, out=None, lse=None,
               want_lse=False, workspace=None):
    """Sparse shared-KV attention over the top-k entries plus the window."""
    _need(q, "q", torch.bfloat16, 4)
    _need(entries, "entries", torch.uint8, 3)
    _need(topk, "topk", torch.int32, 3)
    _need(win, "win", torch.uint8, 3)
    _need(gamma_q, "gamma_q", torch.float32, 1)
    _need(sink, "sink", torch.float32, 1)
    B, Tq, H, D = q.shape
    k = topk.shape[2]
    if entries.shape[0] != B or entries.shape[2] != D + R or tuple(topk.shape[:2]) != (B, Tq) \
            or tuple(win.shape) != (B, Tq + W - 1, D + R) or gamma_q.numel() != D \
            or sink.numel() != H:
        raise ValueError("shape mismatch")
    scale = D ** -0.5 if scale is None else scale
    out, lse = _attend_io(q, out, lse, want_lse)
    arr, sp, q_pos0 = _seq_pos(seq_pos, B, q_pos0)
    nbytes = csa_attend_workspace_bytes(B, Tq, H, D, k, W)
    workspace = _workspace(nbytes, q.device, workspace)
    check(lib().v4attn_csa_attend(_ptr(q), _ptr(entries), _ptr(topk), _ptr(win), _ptr(gamma_q),
                                  _ptr(sink), B, Tq, H, D, R, entries.shape[1], k, int(W),
                                  int(q_pos0), sp, float(scale), float(eps), float(rope_base),
                                  _ptr(out), _ptr(lse), _ptr(workspace), nbytes, _stream(q)))
    return out, lse


def hca_attend(q, entries, win, gamma_q, sink, *, n_entries, m, W, q_pos0=None, seq_pos=None,
               scale=None, eps=1e-6, rope_base=10000.0, R=64, out=None, lse=None,
               want_lse=False, workspace=None):
    """Dense shared-KV attention over every visible entry plus the window."""
    _need(q, "q", torch.bfloat16, 4)
    _need(entries, "entries", torch.uint8, 3)
    _need(win, "win", torch.uint8, 3)
    _need(gamma_q, "gamma_q", torch.float32, 1)
    _need(sink, "sink", torch.float32, 1)
    B, Tq, H, D = q.shape
    if entries.shape[0] != B or entries.shape[2] != D + R \
            or tuple(win.shape) != (B, Tq + W - 1, D + R) or gamma_q.numel() != D \
            or sink.numel() != H:
        raise ValueError("shape mismatch")
    scale = D ** -0.5 if scale is None else scale
    out, lse = _attend_io(q, out, lse, want_lse)
    arr, sp, q_pos0 = _seq_pos(seq_pos, B, q_pos0)
    nbytes = hca_attend_workspace_bytes(B, Tq, H, D, n_entries, m, q_pos0, W)
    workspace = _workspace(nbytes, q.device, workspace)
    check(lib().v4attn_hca_attend(_ptr(q), _ptr(entries), _ptr(win), _ptr(gamma_q), _ptr(sink), B,
                                  Tq, H, D, R, entries.shape[1], int(n_entries), int(m), int(W),
                                  int(q_pos0), sp, float(scale), float(eps), float(rope_base),
                                  _ptr(out), _ptr(lse), _ptr(workspace), nbytes, _stream(q)))
    return out, lse


def hca_attend_noalloc(q, entries, win, gamma_q, sink, *, n_entries, m, W, q_pos0=None,
                       seq_pos=None, scale=None, eps=1e-6, rope_base=10000.0, R=64, out=None,
                       lse=None, want_lse=False):
    """hca_attend with the split partials in the library's fixed device
    scratch (no workspace; out and lse must be given to allocate nothing)."""
    _need(q, "q", torch.bfloat16, 4)
    _need(entries, "entries", torch.uint8, 3)
    _need(win, "win", torch.uint8, 3)
    _need(gamma_q, "gamma_q", torch.float32, 1)
    _need(sink, "sink", torch.float32, 1)
    B, Tq, H, D = q.shape
    if entries.shape[0] != B or entries.shape[2] != D + R \
            or tuple(win.shape) != (B, Tq + W - 1, D + R) or gamma_q.numel() != D \
            or sink.numel() != H:
        raise ValueError("shape mismatch")
    scale = D ** -0.5 if scale is None else scale
    out, lse = _attend_io(q, out, lse, want_lse)
    arr, sp, q_pos0 = _seq_pos(seq_pos, B, q_pos0)
    check(lib().v4attn_hca_attend_noalloc(_ptr(q), _ptr(entries), _ptr(win), _ptr(gamma_q),
                                          _ptr(sink), B, Tq, H, D, R, entries.shape[1],
                                          int(n_entries), int(m), int(W), int(q_pos0), sp,
                                          float(scale), float(eps), float(rope_base), _ptr(out),
                                          _ptr(lse), _stream(q)))
    return out, lse


def nsa_attend_workspace_bytes(B, Tq, H, D, n_entries, m, q_pos0, W, n_sel):
    return lib().v4attn_nsa_attend_workspace(B, Tq, H, D, n_entries, m, q_pos0, W, n_sel)


def nsa_attend(q, entries, tokens, win, gamma_q, gates, *, n_entries, m, q_pos0, W, n_sel,
               scale=None, eps=1e-6, rope_base=10000.0, R=64, out=None, want_blocks=False,
               workspace=None):
    """NSA-style variant: compressed, selected-block and window branches mixed
    by per-head gates.  Returns (out, blocks, block_score); the last two are
    None unless want_blocks."""
    _need(q, "q", torch.bfloat16, 4)
    _need(entries, "entries", torch.uint8, 3)
    _need(tokens, "tokens", torch.uint8, 3)
    _need(win, "win", torch.uint8, 3)
    _need(gamma_q, "gamma_q", torch.float32, 1)
    _need(gates, "gates", torch.float32, 4)
    B, Tq, H, D = q.shape
    if entries.shape[0] != B or entries.shape[2] != D + R or tokens.shape[0] != B \
            or tokens.shape[2] != D + R or tuple(win.shape) != (B, Tq + W - 1, D + R) \
            or gamma_q.numel() != D or tuple(gates.shape) != (B, Tq, H, 3):
        raise ValueError("shape mismatch")
    scale = D ** -0.5 if scale is None else scale
    out, _ = _attend_io(q, out, None, False)
    blocks = block_score = None
    if want_blocks:
        blocks = torch.empty((B, Tq, n_sel), dtype=torch.int32, device=q.device)
        block_score = torch.empty((B, Tq, n_sel), dtype=torch.float32, device=q.device)
    nbytes = nsa_attend_workspace_bytes(B, Tq, H, D, n_entries, m, q_pos0, W, n_sel)
    workspace = _workspace(nbytes, q.device, workspace)
    check(lib().v4attn_nsa_attend(_ptr(q), _ptr(entries), _ptr(tokens), _ptr(win), _ptr(gamma_q),
                                  _ptr(gates), B, Tq, H, D, R, entries.shape[1], int(n_entries),
                                  int(m), tokens.shape[1], int(W), int(n_sel), int(q_pos0),
                                  float(scale), float(eps), float(rope_base), _ptr(out),
                                  _ptr(blocks), _ptr(block_score), _ptr(workspace), nbytes,
                                  _stream(q)))
    return out, blocks, block_score


def _bwd_outputs(q, entries, win, H, D, grads):
    """Gradient buffers: dq written, the rest zeroed here unless given."""
    B, Tq = q.shape[:2]
    dev = q.device
    g = dict(grads or {})
    dq = g.get("dq")
    if dq is None:
        dq = torch.empty((B, Tq, H, D), dtype=torch.float32, device=dev)
    d_ent = g.get("d_entries")
    if d_ent is None:
        d_ent = torch.zeros((B, entries.shape[1], D), dtype=torch.float32, device=dev)
    d_win = g.get("d_win")
    if d_win is None:
        d_win = torch.zeros((B, win.shape[1], D), dtype=torch.float32, device=dev)
    d_sink = g.get("d_sink")
    if d_sink is None:
        d_sink = torch.zeros(H, dtype=torch.float32, device=dev)
    d_gamma = g.get("d_gamma_q")
    if d_gamma is None:
        d_gamma = torch.zeros(D, dtype=torch.float32, device=dev)
    for t, n in ((dq, "dq"), (d_ent, "d_entries"), (d_win, "d_win"), (d_sink, "d_sink"),
                 (d_gamma, "d_gamma_q")):
        _need(t, n, torch.float32)
    return dq, d_ent, d_win, d_sink, d_gamma


def csa_attend_backward(q, entries, topk, win, gamma_q, sink, out, lse, dout, *, q_pos0, W,
                        scale=None, eps=1e-6, rope_base=10000.0, R=64, grads=None,
                        p_sel=None, workspace=None, workspace_bytes=None):
    """Gradients of csa_attend.  Returns (dq, d_entries, d_win, d_sink,
    d_gamma_q); the last four are added into `grads` entries if given.
    p_sel (f32 [B, Tq, k], optional) receives sum_h p of every top-k slot.
    workspace_bytes below the queried size (down to the per-chunk buffers)
    makes the library add the row gradients with atomics instead of
    grouping them."""
    _need(dout, "dout", torch.bfloat16, 4)
    _need(out, "out", torch.bfloat16, 4)
    _need(lse, "lse", torch.float32, 3)
    B, Tq, H, D = q.shape
    k = topk.shape[2]
    scale = D ** -0.5 if scale is None else scale
    dq, d_ent, d_win, d_sink, d_gamma = _bwd_outputs(q, entries, win, H, D, grads)
    nbytes = lib().v4attn_csa_attend_backward_workspace(B, Tq, H, D, k, W, entries.shape[1])
    nbytes = nbytes if workspace_bytes is None else int(workspace_bytes)
    workspace = _workspace(nbytes, q.device, workspace)
    check(lib().v4attn_csa_attend_backward(
        _ptr(q), _ptr(entries), _ptr(topk), _ptr(win), _ptr(gamma_q), _ptr(sink), B, Tq, H, D, R,
        entries.shape[1], k, int(W), int(q_pos0), float(scale), float(eps), float(rope_base),
        _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(d_ent), _ptr(d_win), _ptr(d_sink),
        _ptr(d_gamma), _ptr(p_sel), _ptr(workspace), nbytes, _stream(q)))
    return dq, d_ent, d_win, d_sink, d_gamma


def hca_attend_backward(q, entries, win, gamma_q, sink, out, lse, dout, *, n_entries, m, q_pos0,
                        W, scale=None, eps=1e-6, rope_base=10000.0, R=64, grads=None,
                        workspace=None, workspace_bytes=None):
    """Gradients of hca_attend (see csa_attend_backward)."""
    _need(dout, "dout", torch.bfloat16, 4)
    _need(out, "out", torch.bfloat16, 4)
    _need(lse, "lse", torch.float32, 3)
    B, Tq, H, D = q.shape
    scale = D ** -0.5 if scale is None else scale
    dq, d_ent, d_win, d_sink, d_gamma = _bwd_outputs(q, entries, win, H, D, grads)
    nbytes = lib().v4attn_hca_attend_backward_workspace(B, Tq, H, D, n_entries, m, q_pos0, W,
                                                        entries.shape[1])
    nbytes = nbytes if workspace_bytes is None else int(workspace_bytes)
    workspace = _workspace(nbytes, q.device, workspace)
    check(lib().v4attn_hca_attend_backward(
        _ptr(q), _ptr(entries), _ptr(win), _ptr(gamma_q), _ptr(sink), B, Tq, H, D, R,
        entries.shape[1], int(n_entries), int(m), int(W), int(q_pos0), float(scale), float(eps),
        float(rope_base), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(d_ent), _ptr(d_win),
        _ptr(d_sink), _ptr(d_gamma), _ptr(workspace), nbytes, _stream(q)))
    return dq, d_ent, d_win, d_sink, d_gamma


def compress_backward(raw, tok_score, pos_bias, gamma, d_entries, *, raw_pos0, m, entry0,
                      eps=1e-6, rope_base=10000.0, R=64, grads=None):
    """Gradients of compress_pool for entries entry0 .. entry0 + n_out - 1
    (n_out = d_entries.shape[1]).  Returns (d_raw, d_score, d_bias, d_gamma),
    added into `grads` entries if given, else into fresh zeros."""
    _need(raw, "raw", torch.bfloat16, 3)
    _need(d_entries, "d_entries", torch.float32, 3)
    B, L, D = raw.shape
    n_out = d_entries.shape[1]
    g = dict(grads or {})
    dev = raw.device

    def buf(name, shape):
        t = g.get(name)
        if t is None:
            t = torch.zeros(shape, dtype=torch.float32, device=dev)
        _need(t, name, torch.float32)
        return t
    d_raw = buf("d_raw", (B, L, D))
    d_score = buf("d_score", (B, L))
    d_bias = buf("d_bias", (2 * m,))
    d_gamma = buf("d_gamma", (D,))
    check(lib().v4attn_compress_backward(
        _ptr(raw), _ptr(tok_score), _ptr(pos_bias), _ptr(gamma), B, L, D, R, int(raw_pos0), int(m),
        int(entry0), n_out, float(eps), float(rope_base), _ptr(d_entries), _ptr(d_raw),
        _ptr(d_score), _ptr(d_bias), _ptr(d_gamma), _stream(raw)))
    return d_raw, d_score, d_bias, d_gamma


def index_kl_backward(q_idx, w_idx, k_idx, sel, target, *, dk=None, workspace=None,
                      workspace_bytes=None):
    """Indexer KL loss over the entry set `sel` (int32 [B, Tq, ns]) with target
    weights (f32 [B, Tq, ns]).  Returns (loss [B, Tq], dq_idx, dw_idx, dk_idx);
    dk_idx is added into `dk` if given.  workspace_bytes below the queried
    size (down to the per-chunk buffers) makes the library add the dk rows
    with atomics instead of grouping them."""
    _need(q_idx, "q_idx", torch.bfloat16, 4)
    _need(k_idx, "k_idx", torch.bfloat16, 3)
    _need(sel, "sel", torch.int32, 3)
    _need(target, "target", torch.float32, 3)
    B, Tq, HI, dI = q_idx.shape
    ns = sel.shape[2]
    dev = q_idx.device
    loss = torch.empty((B, Tq), dtype=torch.float32, device=dev)
    dq = torch.empty((B, Tq, HI, dI), dtype=torch.float32, device=dev)
    dw = torch.empty((B, Tq, HI), dtype=torch.float32, device=dev)
    if dk is None:
        dk = torch.zeros((B, k_idx.shape[1], dI), dtype=torch.float32, device=dev)
    nbytes = lib().v4attn_index_kl_backward_workspace(B, Tq, dI, ns, k_idx.shape[1])
    nbytes = nbytes if workspace_bytes is None else int(workspace_bytes)
    workspace = _workspace(nbytes, dev, workspace)
    check(lib().v4attn_index_kl_backward(
        _ptr(q_idx), _ptr(w_idx), _ptr(k_idx), _ptr(sel), _ptr(target), B, Tq, HI, dI,
        k_idx.shape[1], ns, _ptr(loss), _ptr(dq), _ptr(dw), _ptr(dk), _ptr(workspace), nbytes,
        _stream(q_idx)))
    return loss, dq, dw, dk
