"""Parity of the warm-up's dense paths through the C ABI with the CPU oracle:
the dense causal attention (O within max-abs 1e-2, LSE within abs 1e-3 of the
float64 oracle given every visible block, which is pinned against torch's
causal SDPA) and the dense KL loss (rows within 1e-3 + 1e-3|KL|, kl_sum within
relative 1e-3, the forward KL's bars). Small shapes on every row, the 32K and
128K shapes on seeded sampled rows plus the block-edge rows."""
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


def _check_kl(w, x, kl, kl_sum, pos, full_sum=False):
    b = torch.as_tensor(pos[:, 0], device=x["q"].device)
    i = torch.as_tensor(pos[:, 1], device=x["q"].device)
    kh, kih = x["k"].cpu(), x["k_idx"].cpu()
    rows = O.dense_block_idx_rows(pos, w.kv_heads, w.block_size)
    want = O.map_positions(
        lambda c, br, qr, qir: O.kl_rows(None, kh, None, kih, br, c, w.block_size, q_rows=qr, qi_rows=qir),
        pos, (rows, x["q"][b, i].cpu(), x["q_idx"][b, i].cpu()), workers=16)          # [M, Hkv]
    got = kl.permute(0, 2, 1)[b, i].cpu().numpy()
    err = np.abs(got - want)
    tol = 1e-3 + 1e-3 * np.abs(want)          # per row, as the sparse KL's bar
    worst = float((err / tol).max())
    log(f"  {w.name}: dense KL on {len(pos)} rows, max|dKL|={float(err.max()):.2e}, "
        f"worst error / per-row tolerance = {worst:.3f}")
    assert worst <= 1.0
    if full_sum:
        assert abs(float(kl_sum.item()) - float(want.sum())) <= 1e-3 * abs(float(want.sum())) + 1e-3


@pytest.mark.parametrize("w", [
    Workload("dkl_f32", 2, 700, 2, 4, 64, 64, dtype="f32"),
    Workload("dkl_bf16", 1, 1500, 2, 8, 128, 128),
    Workload("dkl_g1_mixed_dims", 1, 900, 3, 1, 128, 64),
    Workload("dkl_g32", 1, 300, 1, 32, 64, 128),
    Workload("dkl_ragged", 1, 129, 2, 2, 64, 64),
])
def test_dense_kl_small(w):
    log(f"{w.name}: B={w.batch} N={w.seqlen} Hkv={w.kv_heads} G={w.group_size} D={w.head_dim} Di={w.index_dim}")
    x = {k: (v.to(DEV) if k != "stripes" else v) for k, v in make_inputs(w, device="cpu").items()}
    _, lse = msa.dense_attn_fwd(x["q"], x["k"], x["v"])
    kl, kl_sum = msa.dense_kl_align_fwd(x["q"], x["k"], x["q_idx"], x["k_idx"], lse)
    torch.cuda.synchronize()
    pos = np.array([(b, i) for b in range(w.batch) for i in range(w.seqlen)], dtype=np.int64)
    _check_kl(w, x, kl, kl_sum, pos, full_sum=True)


def test_dense_kl_equals_sparse_kl_with_every_block():
    w = Workload("dkl_vs_sparse", 1, 4096, 2, 8, 128, 128, topk=32)
    x = make_inputs(w, device=DEV)
    bi = msa.index_topk(x["q_idx"], x["k_idx"], w.topk)
    _, lse_s = msa.sparse_attn_fwd(x["q"], x["k"], x["v"], bi)
    kl_s, sum_s = msa.kl_align_fwd(x["q"], x["k"], x["q_idx"], x["k_idx"], bi, lse_s)
    _, lse_d = msa.dense_attn_fwd(x["q"], x["k"], x["v"])
    kl_d, sum_d = msa.dense_kl_align_fwd(x["q"], x["k"], x["q_idx"], x["k_idx"], lse_d)
    torch.cuda.synchronize()
    assert float((kl_s - kl_d).abs().max()) <= 1e-3 + 1e-3 * float(kl_s.abs().max())
    assert abs(float(sum_s.item()) - float(sum_d.item())) <= 1e-3 * abs(float(sum_s.item()))


def test_dense_kl_n32k_sampled():
    w = Workload("dkl_n32k", 1, 32768, 8, 8, 128, 128)
    x = make_inputs(w, device=DEV, kinds=("q_idx", "k_idx", "q", "k", "v"))
    _, lse = msa.dense_attn_fwd(x["q"], x["k"], x["v"])
    kl, kl_sum = msa.dense_kl_align_fwd(x["q"], x["k"], x["q_idx"], x["k_idx"], lse)
    torch.cuda.synchronize()
    _check_kl(w, x, kl, kl_sum, sample_rows(w, n=128, seed=1))


def test_dense_kl_n128k_sampled():
    """The dense KL at the 128K shapes the benchmark times (B 1, N 131072,
    Hkv 8, G 8, D = Di = 128), on seeded sampled rows plus the sequence's
    last row."""
    w = Workload("dkl_n128k", 1, 131072, 8, 8, 128, 128)
    log(f"{w.name}: drawing inputs on the device")
    x = make_inputs(w, device=DEV, kinds=("q_idx", "k_idx", "q", "k", "v"))
    _, lse = msa.dense_attn_fwd(x["q"], x["k"], x["v"])
    kl, kl_sum = msa.dense_kl_align_fwd(x["q"], x["k"], x["q_idx"], x["k_idx"], lse)
    torch.cuda.synchronize()
    pos = np.concatenate([sample_rows(w, n=96, seed=1), np.array([[0, w.seqlen - 1]])])
    _check_kl(w, x, kl, kl_sum, pos)
