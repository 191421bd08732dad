"""Parity of the KL-term backward (index-branch gradients dq_idx, dk_idx; HIP,
through the C ABI) with the float64 oracle, for seeded per-row loss weights.

Tolerance, as for the main-branch backward: the kernels round dU to bf16 as a
matrix-core operand (twice: dU and dU/G), the dq_idx partials and the outputs,
each within 2^-9 of a value bounded by the tensor's largest entry, and sum in
fp32: every element within 2^-6 of the tensor's largest magnitude, relative
Frobenius error within 2^-7. The 128K workload compares dq_idx on sampled rows
and checks the dk_idx sum rule: over all keys dk_idx sums to 0, within the
first-order bound 2^-8 sum_rows w c |q_idx| (sum_t |s_t - p_t| <= 2 per row)
plus the output rounding 2^-9 sum_t |dk_idx_t|.
"""
import os
import sys
import time

import numpy as np
import pytest
import torch

import block_sparse_gqa_index_amd as msa
from oracle import msa_oracle as O
from synth import CONFIGS, Workload, make_inputs, make_row_weights, sample_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
WORKERS = max(1, min(16, os.cpu_count() or 1))
ELEM_TOL = 2.0 ** -6
FRO_TOL = 2.0 ** -7


def log(msg):
    print(f"[klbwd] {msg}", flush=True)
    sys.stdout.flush()


def run_gpu(w, on_gpu_rng):
    dev = DEV if on_gpu_rng else "cpu"
    x = {k: (v.to(DEV) if k != "stripes" else v) for k, v in make_inputs(w, device=dev).items()}
    wr = make_row_weights(w, device=dev).to(DEV)
    bi = msa.index_topk(x["q_idx"], x["k_idx"], w.topk)
    o, lse = msa.sparse_attn_fwd(x["q"], x["k"], x["v"], bi)
    ilse = torch.empty((w.batch, w.kv_heads, w.seqlen), dtype=torch.float32, device=DEV)
    kl_rows, kl_sum = msa.kl_align_fwd(x["q"], x["k"], x["q_idx"], x["k_idx"], bi, lse, index_lse=ilse)
    t0 = time.time()
    dqi, dki = msa.kl_align_bwd(x["q"], x["k"], x["q_idx"], x["k_idx"], bi, lse, ilse, dkl_rows=wr)
    torch.cuda.synchronize()
    log(f"  backward done ({time.time() - t0:.2f}s)")
    return x, wr, bi, lse, ilse, dqi, dki


def compare(name, got, want):
    got = got.float().cpu().numpy().astype(np.float64)
    scale = np.abs(want).max()
    err = np.abs(got - want).max()
    fro = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300)
    log(f"  {name}: max|err| {err:.3e} = {err / max(scale, 1e-300):.2e} of max|{name}| {scale:.3e}, "
        f"relative Frobenius {fro:.2e}")
    assert err <= ELEM_TOL * scale and fro <= FRO_TOL, name


_JOB = None


def _group_job(job):
    bg, rows = job
    q, k, qi, ki, bi, wr, w = _JOB
    b, g = divmod(bg, w.kv_heads)
    G = w.group_size
    hs = slice(g * G, (g + 1) * G)
    return O.kl_backward(q[b:b + 1, :, hs], k[b:b + 1, :, g:g + 1], qi[b:b + 1, :, g:g + 1], ki[b:b + 1],
                         bi[b:b + 1, g:g + 1], w.block_size, dkl_rows=wr[b:b + 1, g:g + 1],
                         scale=1 / np.sqrt(w.head_dim), index_scale=1 / np.sqrt(w.index_dim), row_range=rows)


def row_chunks(N, parts):
    """Contiguous row ranges covering [0, N): the oracle's results over them add up."""
    step = -(-N // parts)
    return [(i, min(N, i + step)) for i in range(0, N, step)]


def _one_thread():
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)


def oracle_by_group(host, wr, bi, w):
    """The oracle's KL backward, one (batch, group) sub-problem per worker: the
    same computation with Hkv = 1, whose dk_idx contributions add up over the
    groups. Numpy only in the children (one thread each)."""
    import multiprocessing as mp
    global _JOB
    _JOB = tuple(t.float().numpy() for t in (host["q"], host["k"], host["q_idx"], host["k_idx"])) + \
        (bi, wr.numpy(), w)
    n = w.batch * w.kv_heads
    chunks = max(1, WORKERS // n) if w.seqlen >= 16384 else 1
    jobs = [(bg, rows) for bg in range(n) for rows in row_chunks(w.seqlen, chunks)]
    if len(jobs) == 1 or WORKERS == 1:
        parts = [_group_job(j) for j in jobs]
    else:
        with mp.get_context("fork").Pool(min(WORKERS, len(jobs)), initializer=_one_thread) as pool:
            parts = pool.map(_group_job, jobs)
    dqi = np.zeros((w.batch, w.seqlen, w.kv_heads, w.index_dim))
    dki = np.zeros((w.batch, w.seqlen, w.index_dim))
    for (bg, _), (a, c) in zip(jobs, parts):
        b, g = divmod(bg, w.kv_heads)
        dqi[b, :, g] += a[0, :, 0]
        dki[b] += c[0]
    return dqi, dki


def check_every_element(w, on_gpu_rng=False):
    log(f"{w.name}: B={w.batch} N={w.seqlen} Hkv={w.kv_heads} G={w.group_size} D={w.head_dim} "
        f"Di={w.index_dim} k={w.topk}")
    x, wr, bi, lse, ilse, dqi, dki = run_gpu(w, on_gpu_rng)
    host = {k: v.cpu() for k, v in x.items() if k != "stripes"}
    want_bi = O.index_topk(host["q_idx"], host["k_idx"], w.block_size, w.topk)
    assert np.array_equal(bi.cpu().numpy(), want_bi)
    t0 = time.time()
    wq, wk = oracle_by_group(host, wr.cpu(), want_bi, w)
    log(f"  oracle KL backward ({time.time() - t0:.1f}s)")
    compare("dq_idx", dqi, wq)
    compare("dk_idx", dki, wk)


SMALL = [
    Workload("g8_di128", 1, 1500, 2, 8, 128, 128, topk=4),
    Workload("g1_d64_di64_ragged_b2", 2, 1000, 2, 1, 64, 64, topk=3),
    Workload("g2_hkv3_di64", 1, 777, 3, 2, 128, 64, topk=5),
    Workload("g4_k16", 1, 2100, 1, 4, 64, 128, topk=16),
    Workload("g16", 1, 600, 2, 16, 128, 64, topk=2),
    Workload("g32_dense", 1, 1200, 1, 32, 64, 64, topk=32),
    Workload("k1_local_only", 1, 700, 2, 4, 128, 64, topk=1),
    Workload("short", 2, 100, 2, 4, 128, 128, topk=4),
    Workload("stripes", 1, 3000, 2, 8, 128, 128, topk=6, stripe_frac=0.1, stripe_bias=3.0),
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_kl_backward_every_element(w):
    check_every_element(w)


def test_kl_backward_n8k_every_element():
    check_every_element(CONFIGS["n8k"], on_gpu_rng=True)


def test_kl_backward_two_windows_every_element():
    """Two windows of the inverted selection (N = 65,836): dk_idx of a key
    block sums the items of both windows over every group."""
    check_every_element(Workload("two_windows", 1, 65536 + 300, 2, 8, 128, 128, topk=8), on_gpu_rng=True)


def test_kl_backward_n128k_sampled_rows_and_sum_rule():
    w = CONFIGS["n128k"]
    log(f"{w.name}: B={w.batch} N={w.seqlen} Hkv={w.kv_heads} G={w.group_size} D={w.head_dim} k={w.topk}")
    x, wr, bi, lse, ilse, dqi, dki = run_gpu(w, on_gpu_rng=True)
    dqi2, dki2 = msa.kl_align_bwd(x["q"], x["k"], x["q_idx"], x["k_idx"], bi, lse, ilse, dkl_rows=wr)
    torch.cuda.synchronize()
    assert torch.equal(dqi, dqi2) and torch.equal(dki, dki2)
    log("  rerun bitwise equal")

    pos = sample_rows(w)
    b = torch.as_tensor(pos[:, 0], device=DEV)
    i = torch.as_tensor(pos[:, 1], device=DEV)
    kh, kih = x["k"].cpu(), x["k_idx"].cpu()
    q_rows, qi_rows = x["q"][b, i].cpu(), x["q_idx"][b, i].cpu()
    w_rows = wr[b, :, i].cpu().numpy()
    want_bi = O.map_positions(
        lambda c, qr: O.index_topk_rows(None, kih, c, w.block_size, w.topk, q_rows=qr),
        pos, (qi_rows,), workers=1, chunk=1024)
    assert np.array_equal(bi[b, :, i].cpu().numpy(), want_bi)
    want = O.map_positions(
        lambda c, br, qr, qir, wrr: O.kl_dq_idx_rows(None, kh, kih, br, c, w.block_size, w_rows=wrr,
                                                      q_rows=qr, qi_rows=qir),
        pos, (want_bi, q_rows, qi_rows, w_rows), workers=WORKERS)
    compare("dq_idx (sampled rows)", dqi[b, i], want)

    c = 1.0 / np.sqrt(w.index_dim)
    dk = dki.double()
    lhs = dk.sum(dim=(0, 1))
    bound = 2.0 ** -8 * c * (wr.double().permute(0, 2, 1)[..., None] * x["q_idx"].double().abs()).sum(dim=(0, 1, 2)) \
        + 2.0 ** -9 * dk.abs().sum(dim=(0, 1))
    worst = (lhs.abs() / bound).max().item()
    log(f"  dk_idx sum rule: error / bound = {worst:.3e}")
    assert worst <= 1.0
