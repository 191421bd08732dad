"""Parity of the fp4 (OCP e2m1, two values per byte) block selection with the
oracle.

The fp4 matrix cores multiply e2m1 values exactly and accumulate in fp32; every
product is a multiple of 1/4 below 37 in magnitude, so every index score is
exact (|score| < 2^13 for Di <= 128) and the selection must match the float64
oracle on the decoded values bit for bit, ties included, whatever the inputs.
The seeded integer index inputs in [-4, 4] are held exactly by e2m1, so on
them the fp4 selection must also equal the bf16 one; the 128K workload's
stripes (+3, values up to 7) are rounded to e2m1 first (5 -> 4, 7 -> 6), so
there the oracle runs on the rounded values.
"""
import numpy as np
import pytest
import torch

import block_sparse_gqa_index_amd as msa
from oracle import msa_oracle as O
from synth import CONFIGS, Workload, make_inputs, sample_rows, to_fp4_e2m1

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
FP4 = torch.float4_e2m1fn_x2


def log(msg):
    print(f"[fp4] {msg}", flush=True)


def rows_of(t, b, i):
    """t[b, i] of a packed fp4 tensor (gathered through its bytes), on the host."""
    return t.view(torch.uint8)[b, i].cpu().view(FP4)


def check(w: Workload, positions=None, on_gpu_rng=False, same_as_bf16=True):
    log(f"{w.name}: B={w.batch} N={w.seqlen} Hkv={w.kv_heads} Di={w.index_dim} k={w.topk}")
    dev = DEV if on_gpu_rng else "cpu"
    x = make_inputs(w, device=dev, kinds=("q_idx", "k_idx"))
    qi, ki = x["q_idx"].to(DEV), x["k_idx"].to(DEV)
    qi4, ki4 = to_fp4_e2m1(qi), to_fp4_e2m1(ki)
    bi4 = msa.index_topk(qi4, ki4, w.topk)
    torch.cuda.synchronize()
    if same_as_bf16:
        bi = msa.index_topk(qi, ki, w.topk)
        torch.cuda.synchronize()
        assert torch.equal(bi4, bi), "fp4 selection differs from the bf16 one on exactly representable inputs"
        del bi
    if positions is None:
        positions = np.array([(b, i) for b in range(w.batch) for i in range(w.seqlen)],
                             dtype=np.int64).reshape(-1, 2)
    b = torch.as_tensor(positions[:, 0], device=DEV)
    i = torch.as_tensor(positions[:, 1], device=DEV)
    qi_rows = rows_of(qi4, b, i)
    kih = O.fp4_e2m1_values(ki4.view(torch.uint8).cpu().numpy())   # decoded once
    want = O.map_positions(
        lambda c, qr: O.index_topk_rows(None, kih, c, w.block_size, w.topk, q_rows=qr),
        positions, (O.fp4_e2m1_values(qi_rows.view(torch.uint8).numpy()),), workers=1, chunk=1024)
    got = bi4[b, :, i].cpu().numpy()
    bad = np.nonzero((got != want).any(axis=2))
    assert len(bad[0]) == 0, (f"fp4 block_idx mismatch at {len(bad[0])} (row, group) pairs, first "
                              f"pos={positions[bad[0][0]]} got={got[bad[0][0], bad[1][0]]} "
                              f"want={want[bad[0][0], bad[1][0]]}")
    log(f"  fp4 block_idx bit-exact on {len(positions)} positions")


SHAPES = [
    # the 8-wave pipelined kernel (Hkv % 4 == 0, Di = 128)
    Workload("pipe_di128", 1, 2048, 4, 1, 64, 128, topk=8),
    Workload("pipe_ragged_b2", 2, 1500, 4, 1, 64, 128, topk=6),
    Workload("pipe_k32", 1, 3000, 8, 1, 64, 128, topk=32),
    Workload("pipe_ties", 1, 2048, 4, 1, 64, 128, topk=8, index_absmax=1),
    Workload("pipe_stripes", 1, 4100, 8, 1, 64, 128, stripe_frac=0.05, stripe_bias=3.0),
    # the 2- and 4-wave kernel (other Hkv, and Di = 64: 32-byte rows)
    Workload("gen_hkv4_di64", 1, 1800, 4, 1, 64, 64, topk=8),
    Workload("gen_hkv2_di64_b2", 2, 1000, 2, 1, 64, 64, topk=3),
    Workload("gen_hkv3_di128", 1, 777, 3, 1, 64, 128, topk=8),
    Workload("gen_k1", 1, 600, 1, 1, 64, 64, topk=1),
    Workload("gen_ties", 1, 1300, 2, 1, 64, 128, topk=8, index_absmax=1),
    Workload("short", 3, 100, 4, 1, 64, 128, topk=16),
]


@pytest.mark.parametrize("w", SHAPES, ids=[w.name for w in SHAPES])
def test_fp4_selection_every_row(w):
    check(w, same_as_bf16=w.stripe_frac == 0)


def test_fp4_general_values_every_row():
    """Inputs spread over every e2m1 code (not only integers): the scores are
    multiples of 1/4, still exact, and the selection still the oracle's."""
    w = Workload("fp4_codes", 1, 2500, 4, 1, 64, 128, topk=8)
    g = torch.Generator().manual_seed(11)
    qi = torch.randn((1, w.seqlen, w.kv_heads, w.index_dim), generator=g) * 2.5
    ki = torch.randn((1, w.seqlen, w.index_dim), generator=g) * 2.5
    qi4, ki4 = to_fp4_e2m1(qi).to(DEV), to_fp4_e2m1(ki).to(DEV)
    bi4 = msa.index_topk(qi4, ki4, w.topk)
    torch.cuda.synchronize()
    want = O.index_topk(qi4.cpu(), ki4.cpu(), w.block_size, w.topk)
    assert np.array_equal(bi4.cpu().numpy(), want)


@pytest.mark.parametrize("name", ["n8k", "n32k", "n1m"])
def test_fp4_selection_named_workloads(name):
    """Integer index inputs in [-4, 4]: exact in e2m1, so the selection equals
    the bf16 one everywhere and the oracle's on sampled rows (every row at 8K)."""
    w = CONFIGS[name]
    check(w, positions=None if name == "n8k" else sample_rows(w, n=4096 if name == "n32k" else 512),
          on_gpu_rng=True)


def test_fp4_selection_n128k_sampled_rows():
    w = CONFIGS["n128k"]
    check(w, positions=sample_rows(w), on_gpu_rng=True, same_as_bf16=False)
