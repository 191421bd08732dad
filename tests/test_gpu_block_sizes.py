"""Block sizes other than the default 128 (MSA article on 7minutos.es, "¿Qué
es MSA?": 128 is the default block size): the selection with Bk = 64 and
Bk = 256 against the float64 oracle, which takes Bk as a parameter, on every
row; integer-valued index inputs keep every score exact, so block indices
must match bit for bit, ties included."""
import numpy as np
import pytest
import torch

import block_sparse_gqa_index_amd as msa
from oracle import msa_oracle as O
from synth import Workload, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def log(msg):
    print(f"[bk] {msg}", flush=True)


def inputs(w, on_gpu_rng=False):
    x = make_inputs(w, device=DEV if on_gpu_rng else "cpu")
    return {k: (v.to(DEV) if k != "stripes" else v) for k, v in x.items()}


SELECTION = [
    # tiny-scale (fp32, the 2-wave kernel) and 8K-scale (bf16, the pipelined kernel) shapes per block size
    Workload("tiny_bk64", 1, 1024, 1, 4, 64, 64, block_size=64, topk=4, dtype="f32"),
    Workload("tiny_bk256", 1, 1024, 1, 4, 64, 64, block_size=256, topk=4, dtype="f32"),
    Workload("n8k_bk64", 1, 8192, 8, 8, 128, 128, block_size=64, topk=16),
    Workload("n8k_bk256", 1, 8192, 8, 8, 128, 128, block_size=256, topk=16),
    # ragged ends, both kernels, k = 1 and 32, ties, stripes
    Workload("ragged_bk64_hkv4", 2, 1000, 4, 1, 64, 128, block_size=64, topk=8),
    Workload("ragged_bk64_last_half", 1, 1400, 4, 1, 64, 64, block_size=64, topk=6),
    Workload("ragged_bk256_hkv3", 1, 1777, 3, 1, 64, 128, block_size=256, topk=5),
    Workload("bk64_k32_ties", 1, 3000, 8, 1, 64, 128, block_size=64, topk=32, index_absmax=1),
    Workload("bk256_k32_ties", 1, 5000, 4, 1, 64, 128, block_size=256, topk=32, index_absmax=1),
    Workload("bk64_k1", 1, 700, 2, 1, 64, 64, block_size=64, topk=1),
    Workload("bk256_short", 3, 200, 4, 1, 64, 128, block_size=256, topk=4),
    Workload("bk64_stripes_f32", 1, 2600, 2, 1, 64, 64, block_size=64, topk=7, dtype="f32",
             stripe_frac=0.1, stripe_bias=3.0),
]


@pytest.mark.parametrize("w", SELECTION, ids=[w.name for w in SELECTION])
def test_selection_block_sizes(w):
    log(f"{w.name}: B={w.batch} N={w.seqlen} Hkv={w.kv_heads} Di={w.index_dim} Bk={w.block_size} k={w.topk} "
        f"{w.dtype}")
    x = inputs(w)
    bi = msa.index_topk(x["q_idx"], x["k_idx"], w.topk, block_size=w.block_size)
    torch.cuda.synchronize()
    want = O.index_topk(x["q_idx"].cpu(), x["k_idx"].cpu(), w.block_size, w.topk)
    got = bi.cpu().numpy()
    bad = np.argwhere((got != want).any(axis=3))
    assert len(bad) == 0, (f"{len(bad)} rows differ, first (b, g, i) = {bad[0].tolist()}: "
                           f"got {got[tuple(bad[0])].tolist()} want {want[tuple(bad[0])].tolist()}")
    bad_rows = msa.check_block_idx(bi, block_size=w.block_size)
    torch.cuda.synchronize()
    assert int(bad_rows.item()) == 0
    log(f"  block_idx bit-exact on every row; layout check passes")
