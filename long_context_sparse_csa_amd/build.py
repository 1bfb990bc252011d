"""Build libv4attn.so in-tree with hipcc for gfx950.

    python -m long_context_sparse_csa_amd.build [--verbose]

Every call recompiles (a build check must see the current sources).  The
result is long_context_sparse_csa_amd/libv4attn.so.
"""

import concurrent.futures
import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
OUT = os.path.join(PKG, "libv4attn.so")

SOURCES = ["api.cpp", "compress.hip", "indexer.hip", "indexer_fp8.hip", "indexer_mxfp4.hip", "topk.hip", "attend.hip", "nsa.hip", "backward.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # the packed fp32 VALU forms are kept out of generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose=False):
    objs = []
    with tempfile.TemporaryDirectory(prefix="v4attn_build_") as tmp:
        cmds = []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
            if src.endswith(".cpp"):
                cmd.insert(1, "-xhip")
            cmds.append(cmd)
            objs.append(obj)
        # one hipcc per source, compiled side by side (at most 16 at once)
        jobs = max(1, min(len(cmds), os.cpu_count() or 1, 16))
        with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
            for f in [ex.submit(_run, c, verbose) for c in cmds]:
                f.result()
        tmp_out = OUT + ".tmp"
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp_out], verbose)
        os.replace(tmp_out, OUT)
    return OUT


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in p.stderr.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
