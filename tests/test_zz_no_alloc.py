"""The no-allocation decode entry point (msa_decode_noalloc, through the C
ABI) against msa_decode on the same inputs: the same kernels on the library's
fixed scratch array instead of a workspace, so every output must be bitwise
msa_decode's. Two calls in a row on one GPU, the second with a smaller batch
(the scratch array keeps the first call's contents), then the first batch
again, and a multi-query step; the largest problem that fits the array is run
as well."""
import numpy as np
import pytest
import torch

import block_sparse_gqa_index_amd as msa
from synth import Workload, make_decode_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def log(msg):
    print(f"[noalloc] {msg}", flush=True)


def _inputs(w, lengths=None, R=1, seed=0, device="cpu"):
    x = make_decode_inputs(w, device=device, lengths=lengths, seed=seed)
    d = {k: v.to(DEV) for k, v in x.items() if k != "stripes"}
    if R > 1:   # R new queries per sequence: [B, R, ...] query tensors drawn from their own generator
        g = torch.Generator().manual_seed(seed + 77)
        d["q_idx"] = torch.randint(-4, 5, (w.batch, R, w.kv_heads, w.index_dim), generator=g).to(
            d["k_idx"].dtype).to(DEV)
        d["q"] = torch.randn((w.batch, R, w.q_heads, w.head_dim), generator=g).to(d["k"].dtype).to(DEV)
    return d


def _both(w, d):
    want = msa.decode(d["q_idx"], d["k_idx"], d["q"], d["k"], d["v"], d["seqlens"], w.topk)
    got = msa.decode_noalloc(d["q_idx"], d["k_idx"], d["q"], d["k"], d["v"], d["seqlens"], w.topk)
    torch.cuda.synchronize()
    for name, a, b in zip(("block_idx", "o", "lse"), got, want):
        assert torch.equal(a, b), f"{w.name}: {name} differs from msa_decode"
    log(f"{w.name}: B={w.batch} C={w.seqlen} bitwise msa_decode's")
    return got


def test_noalloc_decode_matches_decode_twice_smaller_second():
    big = Workload("noalloc_big", 16, 8192, 8, 8, 128, 128, topk=16)
    small = Workload("noalloc_small", 3, 1500, 8, 8, 128, 128, topk=16)
    d_big = _inputs(big)
    first = _both(big, d_big)
    d_small = _inputs(small, lengths=[1500, 129, 1], seed=5)
    _both(small, d_small)
    again = msa.decode_noalloc(d_big["q_idx"], d_big["k_idx"], d_big["q"], d_big["k"], d_big["v"], d_big["seqlens"],
                               big.topk)
    torch.cuda.synchronize()
    for a, b in zip(again, first):
        assert torch.equal(a, b)


def test_noalloc_decode_other_shapes():
    for w, R in ((Workload("noalloc_g4_d64_fp32", 5, 3000, 2, 4, 64, 64, topk=6, dtype="f32"), 1),
                 (Workload("noalloc_multi_query", 4, 4096, 4, 8, 128, 128, topk=8), 3)):
        _both(w, _inputs(w, R=R, seed=9))


def test_noalloc_decode_largest_fitting_batch():
    """The largest batch of 2K-token caches (Hkv 8, G 8, D 128, k 16) whose
    decode workspace fits the 64 MiB array; one more sequence is refused."""
    def need(B):
        dims = msa.make_dims(B, 2048, 8, 8, 128, 128, 16, torch.bfloat16)
        return msa.decode_workspace_bytes(dims, msa.MSA_OP_DECODE, 1)
    B = 1
    while need(B + 1) <= msa.NOALLOC_SCRATCH_BYTES:
        B += 1
    w = Workload("noalloc_max", B, 2048, 8, 8, 128, 128, topk=16)
    log(f"largest batch that fits: {B} sequences ({need(B)} bytes)")
    _both(w, _inputs(w, seed=3, device=DEV))
    w1 = w.with_(name="noalloc_over", batch=B + 1)
    d = _inputs(w1, seed=4, device=DEV)
    with pytest.raises(msa.MsaError) as e:
        msa.decode_noalloc(d["q_idx"], d["k_idx"], d["q"], d["k"], d["v"], d["seqlens"], w1.topk)
    assert e.value.status == 7
