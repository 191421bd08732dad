"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Block indices must match bit for bit; O within max-abs 1e-2 and LSE within abs
1e-3 of the float64 oracle; KL rows within 1e-3 + 1e-3*|KL| and kl_sum within
relative 1e-3. Small shapes are compared on every row; the named workloads at
full size are compared on seeded sampled rows plus the block-edge rows.
"""
import os
import sys
import time

import numpy as np
import pytest
import torch

import block_sparse_gqa_index_amd as msa
from oracle import msa_oracle as O
from synth import CONFIGS, Workload, make_inputs, sample_rows, uniform_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
WORKERS = max(1, min(16, os.cpu_count() or 1))
O_TOL, LSE_TOL = 1e-2, 1e-3


def log(msg):
    print(f"[parity] {msg}", flush=True)
    sys.stdout.flush()


def inputs_for(w: Workload, on_gpu_rng: bool):
    """Small workloads are drawn on the host (CPU generator) and copied; large
    ones are drawn on the device. Either way both sides read the same bits."""
    if on_gpu_rng:
        return make_inputs(w, device=DEV)
    x = make_inputs(w, device="cpu")
    return {k: (v.to(DEV) if k != "stripes" else v) for k, v in x.items()}


def host(t):
    return t.detach().cpu()


def all_positions(w):
    return np.array([(b, i) for b in range(w.batch) for i in range(w.seqlen)], dtype=np.int64).reshape(-1, 2)


def rows_of(t_bhn, pos):
    """[B, H, N, ...] device tensor -> host rows [M, H, ...] at positions."""
    b = torch.as_tensor(pos[:, 0], device=t_bhn.device)
    i = torch.as_tensor(pos[:, 1], device=t_bhn.device)
    return t_bhn[b, :, i].cpu().numpy()


def rows_bn(t_bn, pos):
    b = torch.as_tensor(pos[:, 0], device=t_bn.device)
    i = torch.as_tensor(pos[:, 1], device=t_bn.device)
    return t_bn[b, i].cpu()


def run_and_check(w: Workload, positions=None, on_gpu_rng=False, check_kl=False):
    """Run the HIP path on workload w and compare with the oracle at positions
    (all positions if None). When every row is checked, the attention is also
    run on the oracle's block indices, so its parity does not rest on the
    selection. Returns the GPU outputs."""
    log(f"{w.name}: B={w.batch} N={w.seqlen} Hkv={w.kv_heads} G={w.group_size} D={w.head_dim} "
        f"Di={w.index_dim} k={w.topk} {w.dtype}")
    x = inputs_for(w, on_gpu_rng)
    pos = all_positions(w) if positions is None else positions
    t0 = time.time()
    bi = msa.index_topk(x["q_idx"], x["k_idx"], w.topk)
    torch.cuda.synchronize()
    log(f"  index_topk done ({time.time() - t0:.2f}s)")

    kh, vh, kih = host(x["k"]), host(x["v"]), host(x["k_idx"])
    qi_rows = rows_bn(x["q_idx"], pos)
    q_rows = rows_bn(x["q"], pos)
    want_bi = O.map_positions(
        lambda c, qr: O.index_topk_rows(None, kih, c, w.block_size, w.topk, q_rows=qr),
        pos, (qi_rows,), workers=1, chunk=1024)
    got_bi = rows_of(bi, pos)
    bad = np.nonzero((got_bi != want_bi).any(axis=2))
    assert len(bad[0]) == 0, (f"block_idx mismatch at {len(bad[0])} (row, group) pairs, first "
                              f"pos={pos[bad[0][0]]} g={bad[1][0]} got={got_bi[bad[0][0], bad[1][0]]} "
                              f"want={want_bi[bad[0][0], bad[1][0]]}")
    log(f"  block_idx bit-exact on {len(pos)} positions")

    if positions is None:
        oracle_bi = torch.as_tensor(want_bi.reshape(w.batch, w.seqlen, w.kv_heads, w.topk)
                                    .transpose(0, 2, 1, 3).copy()).to(DEV)
        o2, lse2 = msa.sparse_attn_fwd(x["q"], x["k"], x["v"], oracle_bi)
    o, lse = msa.sparse_attn_fwd(x["q"], x["k"], x["v"], bi)
    torch.cuda.synchronize()
    if positions is None:
        assert torch.equal(o, o2) and torch.equal(lse, lse2)
    want_o, want_lse = O.map_positions(
        lambda c, br, qr: O.attention_rows(None, kh, vh, br, c, w.block_size, q_rows=qr),
        pos, (want_bi, q_rows), workers=WORKERS)
    got_o = rows_bn(o, pos).float().numpy()
    got_lse = rows_of(lse, pos)
    err_o = np.abs(got_o - want_o).max()
    err_l = np.abs(got_lse - want_lse).max()
    log(f"  attention: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e} max|O|={np.abs(want_o).max():.2f}")
    assert err_o <= O_TOL and err_l <= LSE_TOL

    # The one-call forward and the staged attention (what bench.py times)
    # give the same bits as the two separate calls checked above.
    bi_f, o_f, lse_f = msa.forward(x["q_idx"], x["k_idx"], x["q"], x["k"], x["v"], w.topk)
    torch.cuda.synchronize()
    assert torch.equal(bi_f, bi) and torch.equal(o_f, o) and torch.equal(lse_f, lse)
    dims = msa.make_dims(w.batch, w.seqlen, w.kv_heads, w.group_size, w.head_dim, w.index_dim, w.topk,
                         x["q"].dtype)
    ws = torch.empty(max(1, msa.workspace_bytes(dims, msa.MSA_OP_ATTN)), dtype=torch.uint8, device=x["q"].device)
    o_s, lse_s = torch.empty_like(o), torch.empty_like(lse)
    for stage in (msa.STAGE_PREPARE, msa.STAGE_NONLOCAL, msa.STAGE_COMBINE):
        msa.sparse_attn_fwd(x["q"], x["k"], x["v"], bi, o=o_s, lse=lse_s, workspace=ws, stages=stage)
    torch.cuda.synchronize()
    assert torch.equal(o_s, o) and torch.equal(lse_s, lse)
    log("  msa_forward and the staged attention bitwise equal to the separate calls")

    if check_kl:
        kl, kl_sum = msa.kl_align_fwd(x["q"], x["k"], x["q_idx"], x["k_idx"], bi, lse)
        torch.cuda.synchronize()
        want_kl = O.map_positions(
            lambda c, br, qr, qir: O.kl_rows(None, kh, None, kih, br, c, w.block_size,
                                             q_rows=qr, qi_rows=qir),
            pos, (want_bi, q_rows, qi_rows), workers=WORKERS)
        got_kl = rows_of(kl, pos)
        err = np.abs(got_kl - want_kl)
        bound = 1e-3 + 1e-3 * np.abs(want_kl)
        log(f"  KL rows: max err {err.max():.3e}, max rel {(err / np.maximum(np.abs(want_kl), 1e-9)).max():.3e}")
        assert (err <= bound).all()
        if positions is None:
            ref_sum = want_kl.sum()
            log(f"  kl_sum {kl_sum.item():.6e} vs {ref_sum:.6e}")
            assert abs(kl_sum.item() - ref_sum) <= 1e-3 * abs(ref_sum) + 1e-3
        else:
            # kl_sum is the fixed-order sum of the GPU rows
            assert abs(kl_sum.item() - kl.double().sum().item()) <= 1e-4 * abs(kl.double().sum().item()) + 1e-3
            # and, independently of the GPU rows, agrees with the oracle's estimate
            # of the total from the uniformly drawn positions (B*N times their mean
            # row total over the groups) within five standard errors of that mean
            flat = pos[:, 0] * w.seqlen + pos[:, 1]
            per_pos = np.asarray(want_kl, dtype=np.float64).reshape(len(pos), -1).sum(axis=1)
            t = per_pos[np.isin(flat, uniform_rows(w))]
            total = w.batch * w.seqlen
            est = total * t.mean()
            se = total * t.std(ddof=1) / np.sqrt(len(t))
            log(f"  kl_sum {kl_sum.item():.6e} vs oracle estimate {est:.6e} +- {se:.2e} ({len(t)} uniform rows)")
            assert abs(kl_sum.item() - est) <= 5 * se
    return x, bi, o, lse


SMALL = [
    Workload("b8_g8", 1, 1024, 8, 8, 128, 128, topk=4),
    Workload("ragged_b2", 2, 1000, 2, 4, 64, 64, topk=3),
    Workload("hkv3_f32", 1, 777, 3, 2, 64, 128, topk=8, dtype="f32"),
    Workload("k1", 1, 600, 1, 16, 128, 64, topk=1),
    Workload("k32_g32", 1, 5000, 2, 32, 64, 64, topk=32),
    Workload("short", 3, 100, 4, 1, 128, 128, topk=16),
    Workload("ties", 1, 2048, 4, 8, 128, 128, topk=8, index_absmax=1),
    Workload("warmup_dense", 1, 520, 2, 4, 128, 64, topk=8),
    Workload("f32_d128_g8", 1, 700, 2, 8, 128, 64, topk=5, dtype="f32"),
    # the 8-wave pipelined selection kernel (bf16, Hkv % 4 == 0): ragged N, B > 1, Di 64, k = 32
    Workload("pipe_ragged_b2_di64", 2, 1500, 4, 2, 64, 64, topk=6),
    Workload("pipe_k32_g1", 1, 3000, 8, 1, 64, 128, topk=32),
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_small_shapes_every_row(w):
    run_and_check(w, check_kl=True)


def test_tiny_workload_every_row():
    run_and_check(CONFIGS["tiny"], check_kl=True)


def test_n8k_workload_every_row():
    run_and_check(CONFIGS["n8k"], on_gpu_rng=True)


def test_n32k_workload_sampled_rows():
    w = CONFIGS["n32k"]
    run_and_check(w, positions=sample_rows(w), on_gpu_rng=True)


def test_n128k_workload_sampled_rows():
    w = CONFIGS["n128k"]
    run_and_check(w, positions=sample_rows(w), on_gpu_rng=True)


def test_n1m_workload_sampled_rows_with_kl():
    w = CONFIGS["n1m"]
    run_and_check(w, positions=sample_rows(w), on_gpu_rng=True, check_kl=True)


def test_deterministic_rerun():
    w = CONFIGS["n8k"].with_(seqlen=4096)
    x = inputs_for(w, True)
    outs = []
    for _ in range(2):
        bi = msa.index_topk(x["q_idx"], x["k_idx"], w.topk)
        o, lse = msa.sparse_attn_fwd(x["q"], x["k"], x["v"], bi)
        kl, s = msa.kl_align_fwd(x["q"], x["k"], x["q_idx"], x["k_idx"], bi, lse)
        outs.append([t.clone() for t in (bi, o, lse, kl, s)])
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_block_idx_layout_check():
    w = SMALL[0]
    x = inputs_for(w, on_gpu_rng=False)
    bi = msa.index_topk(x["q_idx"], x["k_idx"], w.topk)
    assert int(msa.check_block_idx(bi).item()) == 0
    bad = bi.clone()
    bad[0, 0, 500, 0] = bad[0, 0, 500, 1]          # repeated id
    bad[0, 1, 700, w.topk - 1] = 0                 # local block not last
    bad[0, 2, 5, 1] = 3                            # padding that is not -1
    bad[0, 3, 900, 0] = -1                         # hole among the kept blocks
    torch.cuda.synchronize()
    assert int(msa.check_block_idx(bad).item()) == 4
    # the oracle's selection follows the layout too
    kih = host(x["k_idx"])
    pos = all_positions(w)[::97]
    want = O.index_topk_rows(host(x["q_idx"]), kih, pos, w.block_size, w.topk)
    got = rows_of(bi, pos)
    assert np.array_equal(got, want)


def test_empty_problems():
    for B, N in ((0, 256), (1, 0)):
        q_idx = torch.zeros((B, N, 2, 64), dtype=torch.bfloat16, device=DEV)
        k_idx = torch.zeros((B, N, 64), dtype=torch.bfloat16, device=DEV)
        bi = msa.index_topk(q_idx, k_idx, 4)
        q = torch.zeros((B, N, 8, 64), dtype=torch.bfloat16, device=DEV)
        kv = torch.zeros((B, N, 2, 64), dtype=torch.bfloat16, device=DEV)
        o, lse = msa.sparse_attn_fwd(q, kv, kv, bi)
        kl, s = msa.kl_align_fwd(q, kv, q_idx, k_idx, bi, lse)
        torch.cuda.synchronize()
        assert s.item() == 0.0 and o.numel() == 0


def test_single_token_row_is_its_value():
    w = Workload("one", 1, 1, 1, 4, 128, 64, topk=4)
    x, bi, o, lse = run_and_check(w)
    assert bi[0, 0, 0].tolist() == [0, -1, -1, -1]
    assert torch.equal(o[0, 0].float(), x["v"][0, 0, 0].float().expand(4, -1))
    z = (x["q"][0, 0].float() @ x["k"][0, 0, 0].float()) / 128 ** 0.5
    assert torch.allclose(lse[0, :, 0], z, atol=1e-3)
