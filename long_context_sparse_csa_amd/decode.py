"""One decode step of a CSA layer and an HCA layer, as a runnable unit.

Per decode token and sequence, a layer
  * CSA (compression m, top-k k, window W): packs the new token's window row
    and pools the compressed entry the token completes (one fused compress
    step), scores every visible entry with the lightning indexer, selects the
    top-k, and attends over them plus the window;
  * HCA (compression m'): the compress step, then attention over every entry
    plus the window.
`run_concurrent` issues both layers' compress steps in one launch, then
the CSA layer's indexer, top-k and attention on the launching stream and the
HCA layer's attention on a second stream beside them (every kernel that
reads an entry, an indexer key or a window row runs after the compress step
that writes it).  `capture` records that schedule in a HIP graph.
`stack_launches` lists the calls of a dependent stack of alternating CSA and
HCA layers (each layer's calls after the previous layer's, one stream) and
`capture_launches` records such a list in one HIP graph.

Inputs are seeded synthetic tensors shaped like the workloads in configs.py
(the random-number recipe is in synth.py).  The HCA caches can rotate over
several copies, one per graph, so successive steps do not hit the Infinity
Cache.
"""

import torch

from . import ops, synth


def build_inputs(c, h, dev, rotate=1):
    """Inputs of the decode step for CSA workload c and HCA workload h."""
    inp = {"csa": {}, "hca": {}}
    d = inp["csa"]
    N = c.T // c.m
    d["N"], d["t"] = N, c.T - 1
    d["entries"] = synth.packed_rows((c.B, N), c.D, c.R, c.seed, "entries", dev,
                                     chunk_rows=1 << 18)
    d["k_idx"] = synth.normal((c.B, N, c.dI), c.seed, "kI", dev, dtype=torch.bfloat16)
    d["q_idx"] = synth.normal((c.B, 1, c.HI, c.dI), c.seed, "qI", dev, dtype=torch.bfloat16)
    d["w_idx"] = synth.normal((c.B, 1, c.HI), c.seed, "w", dev)
    d["q"] = synth.normal((c.B, 1, c.H, c.D), c.seed, "q", dev, dtype=torch.bfloat16)
    d["win"] = synth.packed_rows((c.B, c.W), c.D, c.R, c.seed, "win", dev)
    d["raw"] = synth.normal((c.B, 2 * c.m, c.D), c.seed, "raw", dev, dtype=torch.bfloat16)
    # the tokens' indexer keys: the compressor pools them into k_idx
    d["raw_idx"] = synth.normal((c.B, 2 * c.m, c.dI), c.seed, "rawI", dev, dtype=torch.bfloat16)
    d["score"] = synth.normal((c.B, 2 * c.m), c.seed, "score", dev)
    d["bias"] = synth.normal((2 * c.m,), c.seed, "bias", dev, std=0.1)
    d["sink"] = synth.normal((c.H,), c.seed, "sink", dev)
    d["gamma"] = torch.ones(c.D, device=dev)
    d = inp["hca"]
    N = h.T // h.m
    d["N"], d["t"] = N, h.T - 1
    d["entries"] = [synth.packed_rows((h.B, N), h.D, h.R, h.seed + 100 * i, "entries", dev)
                    for i in range(rotate)]
    d["q"] = synth.normal((h.B, 1, h.H, h.D), h.seed, "q", dev, dtype=torch.bfloat16)
    d["win"] = synth.packed_rows((h.B, h.W), h.D, h.R, h.seed, "win", dev)
    d["raw"] = synth.normal((h.B, 2 * h.m, h.D), h.seed, "raw", dev, dtype=torch.bfloat16)
    d["score"] = synth.normal((h.B, 2 * h.m), h.seed, "score", dev)
    d["bias"] = synth.normal((2 * h.m,), h.seed, "bias", dev, std=0.1)
    d["sink"] = synth.normal((h.H,), h.seed, "sink", dev)
    d["gamma"] = torch.ones(h.D, device=dev)
    return inp


_SIDE = {}


def side_stream(dev):
    """One second stream per device (default priority), shared by every
    DecodeStep: a new stream per step object would take a hardware queue of
    its own the first time it is used."""
    d = torch.device(dev)
    key = d.index if d.index is not None else torch.cuda.current_device()
    if key not in _SIDE:
        _SIDE[key] = torch.cuda.Stream(device=d)
    return _SIDE[key]


class DecodeStep:
    """The library calls of one decode step over fixed buffers."""

    # both layers' compress steps go out in one launch ("compress"); the
    # per-layer calls remain available as "csa_compress" / "hca_compress"
    NAMES = ("compress", "index_score", "topk_select", "csa_attend", "hca_attend")

    def __init__(self, inp, c, h, dev, csa_pos=None, hca_pos=None):
        """csa_pos / hca_pos: optional per-sequence positions of the new
        tokens (a ragged batch); by default every sequence is at T - 1."""
        self.inp, self.c, self.h = inp, c, h
        self.csa_pos, self.hca_pos = csa_pos, hca_pos
        a, b = inp["csa"], inp["hca"]
        Nc, Nh, tc, th = a["N"], b["N"], a["t"], b["t"]
        if csa_pos is not None:
            tc = max(csa_pos)
        if hca_pos is not None:
            th = max(hca_pos)
        self.scores = torch.empty((c.B, ops.score_stride(1, Nc, tc, c.m)), dtype=torch.float32,
                                  device=dev)
        self.topk = torch.empty((c.B, 1, c.k), dtype=torch.int32, device=dev)
        self.tk_ws = torch.empty(max(ops.topk_select_workspace_bytes(c.B, 1, Nc, tc, c.m, c.k), 16),
                                 dtype=torch.uint8, device=dev)
        self.out_c = torch.empty_like(a["q"])
        self.out_h = torch.empty_like(b["q"])
        self.csa_ws = torch.empty(max(ops.csa_attend_workspace_bytes(c.B, 1, c.H, c.D, c.k, c.W), 16),
                                  dtype=torch.uint8, device=dev)
        self.hca_ws = torch.empty(max(ops.hca_attend_workspace_bytes(h.B, 1, h.H, h.D, Nh, h.m, th,
                                                                     h.W), 16),
                                  dtype=torch.uint8, device=dev)
        a["raw_last"] = a["raw"][:, -1:].contiguous()   # the new token's raw latent
        b["raw_last"] = b["raw"][:, -1:].contiguous()
        self.side = side_stream(dev)
        self._calls = {}
        self.ev = [torch.cuda.Event() for _ in range(4)]

    def calls(self, rot=0):
        """name -> zero-argument launch, HCA cache copy `rot`."""
        c, h = self.c, self.h
        a, b = self.inp["csa"], self.inp["hca"]
        Nc, Nh, tc, th = a["N"], b["N"], a["t"], b["t"]
        cp, hp = self.csa_pos, self.hca_pos
        if cp is not None:
            tc = max(cp)
        if hp is not None:
            th = max(hp)
        ent_h = b["entries"][rot % len(b["entries"])]
        csa_step = dict(raw=a["raw"], tok_score=a["score"], pos_bias=a["bias"], gamma=a["gamma"],
                        entries=a["entries"], win=a["win"], raw_pos0=tc + 1 - 2 * c.m, m=c.m, t=tc,
                        seq_pos=cp, win_row=c.W - 1, raw_idx=a["raw_idx"], k_idx=a["k_idx"])
        hca_step = dict(raw=b["raw"], tok_score=b["score"], pos_bias=b["bias"], gamma=b["gamma"],
                        entries=ent_h, win=b["win"], raw_pos0=th + 1 - 2 * h.m, m=h.m, t=th,
                        seq_pos=hp, win_row=h.W - 1)
        return {
            "compress": lambda: ops.compress_steps([csa_step, hca_step]),
            "csa_compress": lambda: ops.compress_step(a["raw"], a["score"], a["bias"], a["gamma"],
                                                      a["entries"], a["win"],
                                                      raw_pos0=tc + 1 - 2 * c.m, m=c.m, t=tc,
                                                      seq_pos=cp, win_row=c.W - 1,
                                                      raw_idx=a["raw_idx"], k_idx=a["k_idx"]),
            "index_score": lambda: ops.index_score(a["q_idx"], a["w_idx"], a["k_idx"], n_entries=Nc,
                                                   q_pos0=tc, seq_pos=cp, m=c.m,
                                                   scores=self.scores),
            "topk_select": lambda: ops.topk_select(self.scores, B=c.B, Tq=1, n_entries=Nc,
                                                   q_pos0=tc, seq_pos=cp, m=c.m, k=c.k,
                                                   topk=self.topk,
                                                   workspace=self.tk_ws),
            "csa_attend": lambda: ops.csa_attend(a["q"], a["entries"], self.topk, a["win"],
                                                 a["gamma"], a["sink"], q_pos0=tc, seq_pos=cp,
                                                 W=c.W,
                                                 out=self.out_c, workspace=self.csa_ws),
            "hca_compress": lambda: ops.compress_step(b["raw"], b["score"], b["bias"], b["gamma"],
                                                      ent_h, b["win"], raw_pos0=th + 1 - 2 * h.m,
                                                      m=h.m, t=th, seq_pos=hp, win_row=h.W - 1),
            "hca_attend": lambda: ops.hca_attend(b["q"], ent_h, b["win"], b["gamma"], b["sink"],
                                                 n_entries=Nh, m=h.m, q_pos0=th, seq_pos=hp,
                                                 W=h.W,
                                                 out=self.out_h, workspace=self.hca_ws),
        }

    def run_eager(self, rot=0):
        """The calls in order on the current stream."""
        f = self.calls(rot)
        for n in self.NAMES:
            f[n]()

    def run_concurrent(self, rot=0):
        """The step with the HCA layer's attention on a second stream beside
        the CSA layer's indexer, top-k and attention: the HCA attention is
        bound by its matrix-core issue, the indexer by HBM, so they overlap.
        The current stream waits for both before it goes on."""
        if rot not in self._calls:      # built once per cache copy (host time per step)
            self._calls[rot] = self.calls(rot)
        f = self._calls[rot]
        main, side, ev = torch.cuda.current_stream(), self.side, self.ev
        f["compress"]()
        ev[2].record(main)
        f["index_score"]()
        side.wait_event(ev[2])
        with torch.cuda.stream(side):
            f["hca_attend"]()
            ev[3].record(side)
        f["topk_select"]()
        f["csa_attend"]()
        main.wait_event(ev[3])

    def capture(self, rot=0):
        """A HIP graph of run_concurrent(rot) (run it eagerly once first, so
        that nothing is allocated during the capture)."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run_concurrent(rot)
        return g


# the calls of one layer, in order (the per-layer compress steps)
CSA_LAYER = ("csa_compress", "index_score", "topk_select", "csa_attend")
HCA_LAYER = ("hca_compress", "hca_attend")


def stack_launches(steps, rot=0):
    """(name, fn) launches of a stack of alternating layers: for each
    DecodeStep in `steps`, its CSA layer's calls and then its HCA layer's
    (layers 2i and 2i + 1), all on the current stream, so every layer runs
    after the one before it as in a model."""
    out = []
    for i, st in enumerate(steps):
        f = st.calls(rot)
        out += [(f"L{2 * i}_{n}", f[n]) for n in CSA_LAYER]
        out += [(f"L{2 * i + 1}_{n}", f[n]) for n in HCA_LAYER]
    return out


def capture_launches(launches):
    """A HIP graph of the launches in order on one stream.  Run them eagerly
    once before capturing, so that nothing is allocated during the capture;
    the library itself allocates nothing and records no memset."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _, fn in launches:
            fn()
    return g
