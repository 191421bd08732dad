"""Parity of the dense causal attention (the warm-up's full attention) through
the C ABI with the CPU oracle: O within max-abs 1e-2 and LSE within abs 1e-3
of the float64 oracle given every visible block (pinned against torch's causal
SDPA). Small shapes on every row, the 32K and 128K shapes on seeded sampled
rows plus the block-edge rows."""
import sys
import time

import numpy as np
import pytest
import torch

import block_sparse_gqa_index_amd as msa
from oracle import msa_oracle as O
from synth import Workload, make_inputs, sample_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
O_TOL, LSE_TOL = 1e-2, 1e-3


def log(msg):
    print(f"[dense] {msg}", flush=True)
    sys.stdout.flush()


def _check(w, x, o, lse, pos):
    b = torch.as_tensor(pos[:, 0], device=x["q"].device)
    i = torch.as_tensor(pos[:, 1], device=x["q"].device)
    q_rows = x["q"][b, i].cpu()
    kh, vh = x["k"].cpu(), x["v"].cpu()
    rows = O.dense_block_idx_rows(pos, w.kv_heads, w.block_size)
    want_o, want_l = O.map_positions(
        lambda c, br, qr: O.attention_rows(None, kh, vh, br, c, w.block_size, q_rows=qr),
        pos, (rows, q_rows), workers=16)
    got_o = o[b, i].float().cpu().numpy()
    got_l = lse.permute(0, 2, 1)[b, i].cpu().numpy()
    eo = float(np.abs(got_o - want_o).max())
    el = float(np.abs(got_l - want_l).max())
    log(f"  {w.name}: {len(pos)} rows, max|dO|={eo:.2e} max|dLSE|={el:.2e}")
    assert eo <= O_TOL and el <= LSE_TOL, (eo, el)


@pytest.mark.parametrize("w", [
    Workload("dense_f32", 2, 1000, 2, 4, 64, 64, dtype="f32"),
    Workload("dense_f32_d128", 1, 700, 1, 2, 128, 64, dtype="f32"),
    Workload("dense_bf16", 1, 3000, 2, 8, 128, 128),
    Workload("dense_g1", 2, 1100, 3, 1, 128, 128),
    Workload("dense_g32", 1, 600, 1, 32, 64, 64),
    Workload("dense_one_block", 1, 128, 2, 4, 128, 128),
    Workload("dense_ragged", 1, 129, 2, 16, 64, 64),
    Workload("dense_one_token", 3, 1, 2, 2, 64, 64),
])
def test_dense_small(w):
    log(f"{w.name}: B={w.batch} N={w.seqlen} Hkv={w.kv_heads} G={w.group_size} D={w.head_dim} {w.dtype}")
    x = {k: (v.to(DEV) if k != "stripes" else v) for k, v in make_inputs(w, device="cpu").items()}
    o, lse = msa.dense_attn_fwd(x["q"], x["k"], x["v"])
    torch.cuda.synchronize()
    pos = np.array([(b, i) for b in range(w.batch) for i in range(w.seqlen)], dtype=np.int64)
    _check(w, x, o, lse, pos)
    o2, lse2 = msa.dense_attn_fwd(x["q"], x["k"], x["v"])
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def test_dense_equals_sparse_with_every_block():
    """k >= blocks: the sparse path keeps every block, so both entry points
    compute the same attention (to within rounding)."""
    w = Workload("dense_vs_sparse", 1, 4096, 2, 8, 128, 128, topk=32)
    x = make_inputs(w, device=DEV)
    bi = msa.index_topk(x["q_idx"], x["k_idx"], w.topk)
    o_s, lse_s = msa.sparse_attn_fwd(x["q"], x["k"], x["v"], bi)
    o_d, lse_d = msa.dense_attn_fwd(x["q"], x["k"], x["v"])
    torch.cuda.synchronize()
    assert float((o_s.float() - o_d.float()).abs().max()) <= 1e-2
    assert float((lse_s - lse_d).abs().max()) <= 1e-4


@pytest.mark.parametrize("name,B,N,rows", [("dense_n32k", 2, 32768, 256), ("dense_n128k", 1, 131072, 128)])
def test_dense_large_sampled(name, B, N, rows):
    w = Workload(name, B, N, 8, 8, 128, 128)
    log(f"{name}: drawing inputs on the device")
    x = make_inputs(w, device=DEV, kinds=("q", "k", "v"))
    t0 = time.time()
    o, lse = msa.dense_attn_fwd(x["q"], x["k"], x["v"])
    torch.cuda.synchronize()
    log(f"  dense forward done ({time.time() - t0:.2f}s)")
    pos = sample_rows(w, n=rows, seed=1)
    _check(w, x, o, lse, pos)
