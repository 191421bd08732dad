"""Parity of the main-branch backward (HIP, through the C ABI) with the float64
oracle, for the loss <dO, O> with a seeded dO.

Tolerance: the kernels round four quantities to bf16 on the way (P and dS as
matrix-core operands, the per-slot dQ partials, the outputs), each within a
relative 2^-9 of a value bounded by the tensor's largest entry, and sum in
fp32; so every element must lie within 2^-6 (twice 4 x 2^-9) of the tensor's
largest magnitude, and the relative Frobenius error within 2^-7. Small shapes
compare dQ, dK and dV element by element; the 128K workload compares dQ on
sampled rows and checks the dV sum rule (the dV of all keys of a group sums to
the group's dO rows) within its first-order rounding bound, and that a rerun
gives the same bits.
"""
import os
import sys
import time

import numpy as np
import pytest
import torch

import block_sparse_gqa_index_amd as msa
from oracle import msa_oracle as O
from synth import CONFIGS, Workload, make_grad_output, make_inputs, sample_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
WORKERS = max(1, min(16, os.cpu_count() or 1))
ELEM_TOL = 2.0 ** -6
FRO_TOL = 2.0 ** -7


def log(msg):
    print(f"[bwd] {msg}", flush=True)
    sys.stdout.flush()


def run_gpu(w, on_gpu_rng):
    dev = DEV if on_gpu_rng else "cpu"
    x = {k: (v.to(DEV) if k != "stripes" else v) for k, v in make_inputs(w, device=dev).items()}
    dout = make_grad_output(w, device=dev).to(DEV)
    bi = msa.index_topk(x["q_idx"], x["k_idx"], w.topk)
    o, lse = msa.sparse_attn_fwd(x["q"], x["k"], x["v"], bi)
    t0 = time.time()
    dq, dk, dv = msa.sparse_attn_bwd(x["q"], x["k"], x["v"], bi, o, lse, dout)
    torch.cuda.synchronize()
    log(f"  backward done ({time.time() - t0:.2f}s)")
    return x, dout, bi, o, lse, dq, dk, dv


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
    q, k, v, dout, bi, w = _JOB
    b, g = divmod(bg, w.kv_heads)
    G = w.group_size
    hs = slice(g * G, (g + 1) * G)
    return O.attention_backward(q[b:b + 1, :, hs], k[b:b + 1, :, g:g + 1], v[b:b + 1, :, g:g + 1],
                                dout[b:b + 1, :, hs], bi[b:b + 1, g:g + 1], w.block_size, row_range=rows)


def row_chunks(N, parts):
    """Contiguous row ranges covering [0, N): the oracle's results over them add up."""
    step = -(-N // parts)
    return [(i, min(N, i + step)) for i in range(0, N, step)]


def _one_thread():
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)


def oracle_backward_by_group(host, dout, bi, w):
    """The oracle's backward, one (batch, group) sub-problem per worker: each
    is the same computation with Hkv = 1 (groups do not interact). Tensors
    become numpy arrays before the fork: the children run numpy only, one
    thread each (a forked child that enters torch's OpenMP pool can block)."""
    import multiprocessing as mp
    global _JOB
    _JOB = tuple(t.float().numpy() for t in (host["q"], host["k"], host["v"], dout)) + (bi, w)
    n = w.batch * w.kv_heads
    # long sequences: every (batch, group) split into row ranges as well
    chunks = max(1, WORKERS // n) if w.seqlen >= 16384 else 1
    jobs = [(bg, rows) for bg in range(n) for rows in row_chunks(w.seqlen, chunks)]
    if len(jobs) == 1 or WORKERS == 1:
        parts = [_group_job(j) for j in jobs]
    else:
        with mp.get_context("fork").Pool(min(WORKERS, len(jobs)), initializer=_one_thread) as pool:
            parts = pool.map(_group_job, jobs)
    B, N, G, D = w.batch, w.seqlen, w.group_size, w.head_dim
    dq = np.zeros((B, N, w.q_heads, D))
    dk = np.zeros((B, N, w.kv_heads, D))
    dv = np.zeros((B, N, w.kv_heads, D))
    for (bg, _), (a, c, e) in zip(jobs, parts):
        b, g = divmod(bg, w.kv_heads)
        dq[b, :, g * G:(g + 1) * G] += a[0]
        dk[b, :, g] += c[0, :, 0]
        dv[b, :, g] += e[0, :, 0]
    return dq, dk, dv


def check_every_element(w, on_gpu_rng=False):
    log(f"{w.name}: B={w.batch} N={w.seqlen} Hkv={w.kv_heads} G={w.group_size} D={w.head_dim} k={w.topk}")
    x, dout, bi, o, lse, dq, dk, dv = run_gpu(w, on_gpu_rng)
    host = {k: v.cpu() for k, v in x.items() if k != "stripes"}
    want_bi = O.index_topk(host["q_idx"], host["k_idx"], w.block_size, w.topk)
    assert np.array_equal(bi.cpu().numpy(), want_bi)
    t0 = time.time()
    wq, wk, wv = oracle_backward_by_group(host, dout.cpu(), want_bi, w)
    log(f"  oracle backward ({time.time() - t0:.1f}s)")
    compare("dQ", dq, wq)
    compare("dK", dk, wk)
    compare("dV", dv, wv)
    return dq, dk, dv


SMALL = [
    Workload("g8_d128", 1, 1500, 2, 8, 128, 64, topk=4),
    Workload("g1_d64_ragged_b2", 2, 1000, 2, 1, 64, 64, topk=3),
    Workload("g2_hkv3", 1, 777, 3, 2, 128, 64, topk=5),
    Workload("g4_k16", 1, 2100, 1, 4, 64, 64, topk=16),
    Workload("g16", 1, 600, 1, 16, 128, 64, topk=2),
    Workload("g32_dense", 1, 1200, 1, 32, 64, 64, topk=32),     # k >= blocks: dense causal
    Workload("k1_local_only", 1, 700, 2, 4, 128, 64, topk=1),
    Workload("short", 2, 100, 2, 4, 128, 64, topk=4),           # one partial block
    Workload("stripes", 1, 3000, 2, 8, 128, 64, topk=6, stripe_frac=0.1, stripe_bias=3.0),
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_backward_every_element(w):
    check_every_element(w)


def test_backward_n8k_every_element():
    check_every_element(CONFIGS["n8k"], on_gpu_rng=True)


# Query positions past 65,536 fall in a second window of the inverted
# selection, so a key block's dK/dV sums the items of both windows (and the
# block's own causal rows); the last block is partial.
TWO_WINDOWS = Workload("two_windows", 1, 65536 + 300, 2, 8, 128, 128, topk=8)


def test_backward_two_windows_every_element():
    check_every_element(TWO_WINDOWS, on_gpu_rng=True)


def test_backward_n128k_sampled_rows_and_sum_rule():
    w = CONFIGS["n128k"]
    log(f"{w.name}: B={w.batch} N={w.seqlen} Hkv={w.kv_heads} G={w.group_size} D={w.head_dim} k={w.topk}")
    x, dout, bi, o, lse, dq, dk, dv = run_gpu(w, on_gpu_rng=True)
    # rerun: the same bits
    dq2, dk2, dv2 = msa.sparse_attn_bwd(x["q"], x["k"], x["v"], bi, o, lse, dout)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)
    log("  rerun bitwise equal")

    pos = sample_rows(w)
    b = torch.as_tensor(pos[:, 0], device=DEV)
    i = torch.as_tensor(pos[:, 1], device=DEV)
    kh, vh, kih = x["k"].cpu(), x["v"].cpu(), x["k_idx"].cpu()
    qi_rows, q_rows, do_rows = x["q_idx"][b, i].cpu(), x["q"][b, i].cpu(), dout[b, i].cpu()
    want_bi = O.map_positions(
        lambda c, qr: O.index_topk_rows(None, kih, c, w.block_size, w.topk, q_rows=qr),
        pos, (qi_rows,), workers=1, chunk=1024)
    assert np.array_equal(bi[b, :, i].cpu().numpy(), want_bi)
    want_dq = O.map_positions(
        lambda c, br, qr, dr: O.attention_dq_rows(None, kh, vh, None, br, c, w.block_size, q_rows=qr, do_rows=dr),
        pos, (want_bi, q_rows, do_rows), workers=WORKERS)
    compare("dQ (sampled rows)", dq[b, i], want_dq)

    # sum rule per group, with its first-order rounding bound: the probability
    # roundings perturb each row's total weight by <= 2^-8 |dO| (operand and
    # accumulation), the output rounding each dV_t by <= 2^-9 |dV_t|
    G = w.group_size
    dvf = dv.double()
    dof = dout.double()
    for g in range(w.kv_heads):
        lhs = dvf[:, :, g].sum(dim=(0, 1))
        rhs = dof[:, :, g * G:(g + 1) * G].sum(dim=(0, 1, 2))
        bound = 2.0 ** -8 * dof[:, :, g * G:(g + 1) * G].abs().sum(dim=(0, 1, 2)) + \
            2.0 ** -9 * dvf[:, :, g].abs().sum(dim=(0, 1))
        worst = ((lhs - rhs).abs() / bound).max().item()
        log(f"  group {g}: sum-rule error / bound = {worst:.3f}")
        assert worst <= 1.0


def test_backward_deterministic_small():
    w = SMALL[-1]
    x, dout, bi, o, lse, dq, dk, dv = run_gpu(w, on_gpu_rng=False)
    outs = [msa.sparse_attn_bwd(x["q"], x["k"], x["v"], bi, o, lse, dout) for _ in range(2)]
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    assert torch.equal(outs[0][0], dq)
