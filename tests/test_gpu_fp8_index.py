"""Parity of the fp8 (OCP e4m3) block selection with the oracle.

The index inputs are the seeded integer-valued workloads in [-7, 7], which e4m3
holds exactly, so every index score is an exact integer on both sides and the
block indices must match the float64 oracle bit for bit, ties included. The
same values in bf16 give the same selection, which is checked as well.
"""
import numpy as np
import pytest
import torch

import block_sparse_gqa_index_amd as msa
from oracle import msa_oracle as O
from synth import CONFIGS, Workload, make_inputs, sample_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
FP8 = torch.float8_e4m3fn


def log(msg):
    print(f"[fp8] {msg}", flush=True)


def check(w: Workload, positions=None, on_gpu_rng=False):
    log(f"{w.name}: B={w.batch} N={w.seqlen} Hkv={w.kv_heads} Di={w.index_dim} k={w.topk}")
    dev = DEV if on_gpu_rng else "cpu"
    x = make_inputs(w, device=dev, kinds=("q_idx", "k_idx"))
    qi, ki = x["q_idx"].to(DEV), x["k_idx"].to(DEV)
    qi8, ki8 = qi.to(FP8), ki.to(FP8)
    assert torch.equal(qi8.float(), qi.float()) and torch.equal(ki8.float(), ki.float())
    bi8 = msa.index_topk(qi8, ki8, w.topk)
    bi = msa.index_topk(qi, ki, w.topk)
    torch.cuda.synchronize()
    assert torch.equal(bi8, bi)

    if positions is None:
        positions = np.array([(b, i) for b in range(w.batch) for i in range(w.seqlen)],
                             dtype=np.int64).reshape(-1, 2)
    b = torch.as_tensor(positions[:, 0], device=DEV)
    i = torch.as_tensor(positions[:, 1], device=DEV)
    qi_rows = qi8[b, i].cpu()
    want = O.map_positions(
        lambda c, qr: O.index_topk_rows(None, ki8.cpu(), c, w.block_size, w.topk, q_rows=qr),
        positions, (qi_rows,), workers=1, chunk=1024)
    got = bi8[b, :, i].cpu().numpy()
    bad = np.nonzero((got != want).any(axis=2))
    assert len(bad[0]) == 0, (f"fp8 block_idx mismatch at {len(bad[0])} (row, group) pairs, first "
                              f"pos={positions[bad[0][0]]} got={got[bad[0][0], bad[1][0]]} "
                              f"want={want[bad[0][0], bad[1][0]]}")
    log(f"  fp8 block_idx bit-exact on {len(positions)} positions")


SHAPES = [
    # the 8-wave pipelined kernel (Hkv % 4 == 0)
    Workload("pipe_di128", 1, 2048, 4, 1, 64, 128, topk=8),
    Workload("pipe_ragged_b2_di64", 2, 1500, 4, 1, 64, 64, topk=6),
    Workload("pipe_k32", 1, 3000, 8, 1, 64, 128, topk=32),
    Workload("pipe_ties", 1, 2048, 4, 1, 64, 128, topk=8, index_absmax=1),
    Workload("pipe_stripes", 1, 4100, 8, 1, 64, 128, stripe_frac=0.05, stripe_bias=3.0),
    # the 2- and 4-wave kernel (other Hkv)
    Workload("gen_hkv2_di64", 2, 1000, 2, 1, 64, 64, topk=3),
    Workload("gen_hkv3_di128", 1, 777, 3, 1, 64, 128, topk=8),
    Workload("gen_k1", 1, 600, 1, 1, 64, 64, topk=1),
    Workload("gen_ties", 1, 1300, 2, 1, 64, 128, topk=8, index_absmax=1),
    Workload("short", 3, 100, 4, 1, 64, 128, topk=16),
]


@pytest.mark.parametrize("w", SHAPES, ids=[w.name for w in SHAPES])
def test_fp8_selection_every_row(w):
    check(w)


def test_fp8_selection_n128k_sampled_rows():
    w = CONFIGS["n128k"]
    check(w, positions=sample_rows(w), on_gpu_rng=True)
