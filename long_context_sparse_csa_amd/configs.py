"""The workloads the library is tested and measured on.

Shapes follow the pages' V4-Pro setting: CSA compression m = 4 with top-k
1024, HCA compression m' = 128, a 128-token window, RoPE on the last 64 of a
512-wide shared latent ("DeepSeek-V4: Making a Million Tokens Affordable",
section "Two ways to shrink attention, interleaved"), at a million-token
context ("Decoding DeepSeek-V4", section "Compressing the past").
"""

from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "csa_decode", "hca_decode" or "prefill"
    B: int               # sequences in the batch
    Tq: int              # query tokens per sequence
    T: int               # tokens cached before the query block (decode: incl. the query)
    H: int = 64          # query heads sharing one KV head
    D: int = 512         # latent / head dim
    R: int = 64          # rotary dims (the last R)
    m: int = 4           # compression ratio
    HI: int = 64         # indexer heads
    dI: int = 128        # indexer head dim
    k: int = 1024        # top-k
    W: int = 128         # uncompressed window
    rope_base: float = 10000.0
    eps: float = 1e-6
    seed: int = 0
    int_indexer: bool = False   # integer-valued indexer inputs in [-3, 3]
    extra: dict = field(default_factory=dict, compare=False)

    @property
    def row(self):
        """Packed row bytes: (D-R) E4M3 + R bf16."""
        return self.D + self.R

    @property
    def scale(self):
        return self.D ** -0.5

    @property
    def n_entries(self):
        """Compressed entries after the cached context (completed groups)."""
        return self.T // self.m

    @property
    def q_pos0(self):
        """Position of the first query token."""
        return self.T - 1 if self.kind != "prefill" else self.T

    def with_(self, **kw):
        return replace(self, **kw)


TINY_CSA = Workload("tiny_csa_decode", "csa_decode", B=1, Tq=1, T=4096, H=8,
                    D=128, R=64, m=4, HI=4, dI=32, k=64, W=128, seed=1,
                    int_indexer=True)
CSA_128K = Workload("csa_decode_128k", "csa_decode", B=16, Tq=1, T=131072,
                    m=4, seed=2)
HCA_1M = Workload("hca_decode_1m", "hca_decode", B=32, Tq=1, T=1 << 20,
                  m=128, seed=3)
CSA_1M = Workload("csa_decode_1m", "csa_decode", B=8, Tq=1, T=1 << 20, m=4,
                  seed=4)
PREFILL_1M = Workload("prefill_4096_on_1m", "prefill", B=1, Tq=4096,
                      T=1 << 20, m=4, seed=5, extra={"m_hca": 128})

# The NSA-style variant ("DeepSeek-V4, explained", the numbered steps of how a
# compress-then-select layer handles one query): 64-token blocks, one
# compressed entry each, 16 blocks selected, the same 128-token window.
NSA_1M = Workload("nsa_decode_1m", "nsa_decode", B=8, Tq=1, T=1 << 20, m=64,
                  seed=6, extra={"n_sel": 16})

ALL = [TINY_CSA, CSA_128K, HCA_1M, CSA_1M, PREFILL_1M, NSA_1M]
BY_NAME = {w.name: w for w in ALL}
