"""Workload shapes for the MSA forward path.

The five named workloads are: a tiny fp32 case the oracle checks in full, and
bf16 cases at 8K, 2x32K, 128K (with long-range stripes) and 1M tokens (with the
KL-alignment forward). Block size Bk = 128 and k = 16 are the method's defaults
(MiniMax Sparse Attention (MSA) article on 7minutos.es, section "¿Qué es MSA?").
"""
from dataclasses import dataclass, field, asdict


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    kv_heads: int
    group_size: int
    head_dim: int
    index_dim: int
    block_size: int = 128
    topk: int = 16
    dtype: str = "bf16"            # "bf16" or "f32": dtype of every input tensor
    seed: int = 0
    stripe_frac: float = 0.0       # fraction of key blocks that get a k_idx bias
    stripe_bias: float = 0.0
    index_absmax: int = 4          # index inputs are integers in [-index_absmax, index_absmax]
    with_kl: bool = False
    sampled_rows: int = 0          # 0 = check every query position

    @property
    def q_heads(self) -> int:
        return self.kv_heads * self.group_size

    @property
    def nblocks(self) -> int:
        return -(-self.seqlen // self.block_size)

    def dims(self) -> dict:
        return {k: v for k, v in asdict(self).items()
                if k in ("batch", "seqlen", "kv_heads", "group_size", "head_dim",
                         "index_dim", "block_size", "topk", "dtype")}

    def with_(self, **kw) -> "Workload":
        d = asdict(self)
        d.update(kw)
        return Workload(**d)


CONFIGS = {
    "tiny": Workload("tiny", 1, 1024, 1, 4, 64, 64, topk=4, dtype="f32"),
    "n8k": Workload("n8k", 1, 8192, 8, 8, 128, 128),
    "n32k": Workload("n32k", 2, 32768, 8, 8, 128, 128, sampled_rows=4096),
    "n128k": Workload("n128k", 1, 131072, 8, 8, 128, 128, stripe_frac=0.01,
                      stripe_bias=3.0, sampled_rows=4096),
    "n1m": Workload("n1m", 1, 1048576, 4, 8, 128, 128, with_kl=True, sampled_rows=4096),
}


def get_workload(name: str) -> Workload:
    return CONFIGS[name]


# Decode batches: ``batch`` sequences, a cache of ``seqlen`` tokens each (the
# capacity; the cached lengths are drawn uniformly on [1, seqlen]), one new
# query per sequence, the model sizes of the 128K workload.
DECODE_CONFIGS = {
    "decode_n8k_b8": Workload("decode_n8k_b8", 8, 8192, 8, 8, 128, 128),
    "decode_n128k_b64": Workload("decode_n128k_b64", 64, 131072, 8, 8, 128, 128, stripe_frac=0.01,
                                 stripe_bias=3.0),
}
