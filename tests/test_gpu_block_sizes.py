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


WORKERS = 16
O_TOL, LSE_TOL = 1e-2, 1e-3

ATTENTION = [
    Workload("tiny_bk64", 1, 1024, 1, 4, 64, 64, block_size=64, topk=4, dtype="f32"),
    Workload("tiny_bk256", 1, 1024, 1, 4, 64, 64, block_size=256, topk=4, dtype="f32"),
    Workload("n8k_bk64", 1, 8192, 8, 8, 128, 128, block_size=64, topk=16),
    Workload("n8k_bk256", 1, 8192, 8, 8, 128, 128, block_size=256, topk=16),
    Workload("ragged_bk64_b2", 2, 1000, 2, 2, 128, 64, block_size=64, topk=6),
    Workload("ragged_bk64_ties", 1, 1400, 2, 8, 64, 128, block_size=64, topk=9, index_absmax=1),
    Workload("ragged_bk256_hkv3", 1, 1777, 3, 1, 64, 128, block_size=256, topk=5),
    Workload("bk64_k32_g32", 1, 1500, 1, 32, 64, 64, block_size=64, topk=32),
    Workload("bk64_k1", 1, 700, 2, 4, 128, 64, block_size=64, topk=1),
    Workload("bk256_short_b2", 2, 200, 2, 8, 128, 128, block_size=256, topk=4),
    Workload("bk256_k1", 1, 900, 2, 4, 64, 64, block_size=256, topk=1),
    Workload("bk256_stripes", 1, 4000, 2, 8, 128, 128, block_size=256, topk=16, stripe_frac=0.1, stripe_bias=3.0),
]


def _rows(t_bn, pos):
    b = torch.as_tensor(pos[:, 0], device=t_bn.device)
    i = torch.as_tensor(pos[:, 1], device=t_bn.device)
    return t_bn[b, i].cpu()


def _rows_bhn(t, pos):
    b = torch.as_tensor(pos[:, 0], device=t.device)
    i = torch.as_tensor(pos[:, 1], device=t.device)
    return t[b, :, i].cpu().numpy()


@pytest.mark.parametrize("w", ATTENTION, ids=[w.name for w in ATTENTION])
def test_attention_and_kl_block_sizes(w):
    """Every row: block ids bit-exact, O within 1e-2, LSE within 1e-3, KL rows
    within 1e-3 + 1e-3 |KL| and kl_sum within relative 1e-3 of the oracle at
    this block size; the attention also on the oracle's ids (same bits), and
    msa_forward equal to the separate calls."""
    Bk = w.block_size
    log(f"{w.name}: B={w.batch} N={w.seqlen} Hkv={w.kv_heads} G={w.group_size} D={w.head_dim} Di={w.index_dim} "
        f"Bk={Bk} k={w.topk} {w.dtype}")
    x = inputs(w)
    bi = msa.index_topk(x["q_idx"], x["k_idx"], w.topk, block_size=Bk)
    o, lse = msa.sparse_attn_fwd(x["q"], x["k"], x["v"], bi, block_size=Bk)
    ilse = torch.empty((w.batch, w.kv_heads, w.seqlen), dtype=torch.float32, device=DEV)
    kl, kl_sum = msa.kl_align_fwd(x["q"], x["k"], x["q_idx"], x["k_idx"], bi, lse, block_size=Bk, index_lse=ilse)
    torch.cuda.synchronize()
    pos = np.array([(b, i) for b in range(w.batch) for i in range(w.seqlen)], dtype=np.int64)
    kh, vh, kih = x["k"].cpu(), x["v"].cpu(), x["k_idx"].cpu()
    want_bi = O.index_topk(x["q_idx"].cpu(), kih, Bk, w.topk)
    assert np.array_equal(bi.cpu().numpy(), want_bi)
    rows = want_bi.transpose(0, 2, 1, 3).reshape(-1, w.kv_heads, w.topk)
    q_rows, qi_rows = _rows(x["q"], pos), _rows(x["q_idx"], pos)
    want_o, want_lse = O.map_positions(
        lambda c, br, qr: O.attention_rows(None, kh, vh, br, c, Bk, q_rows=qr), pos, (rows, q_rows),
        workers=WORKERS)
    err_o = float(np.abs(_rows(o, pos).float().numpy() - want_o).max())
    err_l = float(np.abs(_rows_bhn(lse, pos) - want_lse).max())
    log(f"  attention: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}")
    assert err_o <= O_TOL and err_l <= LSE_TOL
    want_kl = O.map_positions(
        lambda c, br, qr, qir: O.kl_rows(None, kh, None, kih, br, c, Bk, q_rows=qr, qi_rows=qir),
        pos, (rows, q_rows, qi_rows), workers=WORKERS)
    got_kl = _rows_bhn(kl, pos)
    worst = float((np.abs(got_kl - want_kl) / (1e-3 + 1e-3 * np.abs(want_kl))).max())
    total = float(want_kl.sum())
    log(f"  KL: worst error / per-row tolerance {worst:.3f}; kl_sum {float(kl_sum.item()):.6g} vs {total:.6g}")
    assert worst <= 1.0
    assert abs(float(kl_sum.item()) - total) <= 1e-3 * abs(total) + 1e-3

    # the attention on the oracle's ids gives the same bits; msa_forward equals the separate calls
    o2, lse2 = msa.sparse_attn_fwd(x["q"], x["k"], x["v"], torch.as_tensor(want_bi).to(DEV), block_size=Bk)
    bi_f, o_f, lse_f = msa.forward(x["q_idx"], x["k_idx"], x["q"], x["k"], x["v"], w.topk, block_size=Bk)
    torch.cuda.synchronize()
    assert torch.equal(o2, o) and torch.equal(lse2, lse)
    assert torch.equal(bi_f, bi) and torch.equal(o_f, o) and torch.equal(lse_f, lse)
