"""Parity of the fused backward of both branches (msa_fused_bwd: dQ, dK, dV of
the main branch for <dO, O> and dq_idx, dk_idx of the KL term for seeded row
weights, from one pass) with the float64 oracle, through the C ABI.

Tolerance as for the separate backward kernels (four bf16 roundings on the way,
each within 2^-9 of a value bounded by the tensor's largest entry, fp32 sums):
every element within 2^-6 of the tensor's largest magnitude and the relative
Frobenius error within 2^-7. Small shapes and two 64K-position windows are
compared element by element for all five gradients, and the small shapes also
with the separate backward kernels' gradients (within 2^-7 of their largest
magnitude); at a million tokens dQ and dq_idx are compared on seeded sampled
rows, with the dV and dk_idx sum rules over every key.
"""
import os
import sys
import time

import numpy as np
import pytest
import torch

import block_sparse_gqa_index_amd as msa
from oracle import msa_oracle as O
from synth import CONFIGS, Workload, make_grad_output, make_inputs, make_row_weights, sample_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
WORKERS = max(1, min(16, os.cpu_count() or 1))
ELEM_TOL = 2.0 ** -6
FRO_TOL = 2.0 ** -7


def log(msg):
    print(f"[fused] {msg}", flush=True)
    sys.stdout.flush()


def run_gpu(w, on_gpu_rng):
    dev = DEV if on_gpu_rng else "cpu"
    x = {k: (v.to(DEV) if k != "stripes" else v) for k, v in make_inputs(w, device=dev).items()}
    dout = make_grad_output(w, device=dev).to(DEV)
    wr = make_row_weights(w, device=dev).to(DEV)
    bi = msa.index_topk(x["q_idx"], x["k_idx"], w.topk)
    o, lse = msa.sparse_attn_fwd(x["q"], x["k"], x["v"], bi)
    ilse = torch.empty((w.batch, w.kv_heads, w.seqlen), dtype=torch.float32, device=DEV)
    msa.kl_align_fwd(x["q"], x["k"], x["q_idx"], x["k_idx"], bi, lse, index_lse=ilse)
    t0 = time.time()
    grads = msa.fused_bwd(x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], bi, o, lse, ilse, dout, dkl_rows=wr)
    torch.cuda.synchronize()
    log(f"  fused backward done ({time.time() - t0:.2f}s)")
    return x, dout, wr, bi, o, lse, ilse, grads


def compare(name, got, want):
    got = got.float().cpu().numpy().astype(np.float64)
    scale = np.abs(want).max()
    err = np.abs(got - want).max()
    fro = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300)
    log(f"  {name}: max|err| {err:.3e} = {err / max(scale, 1e-300):.2e} of max|{name}| {scale:.3e}, "
        f"relative Frobenius {fro:.2e}")
    assert err <= ELEM_TOL * scale and fro <= FRO_TOL, name


_JOB = None


def _job(job):
    kind, bg, rows = job
    q, k, v, qi, ki, dout, bi, wr, w = _JOB
    b, g = divmod(bg, w.kv_heads)
    G = w.group_size
    hs = slice(g * G, (g + 1) * G)
    if kind == "main":
        return O.attention_backward(q[b:b + 1, :, hs], k[b:b + 1, :, g:g + 1], v[b:b + 1, :, g:g + 1],
                                    dout[b:b + 1, :, hs], bi[b:b + 1, g:g + 1], w.block_size, row_range=rows)
    return O.kl_backward(q[b:b + 1, :, hs], k[b:b + 1, :, g:g + 1], qi[b:b + 1, :, g:g + 1], ki[b:b + 1],
                         bi[b:b + 1, g:g + 1], w.block_size, dkl_rows=wr[b:b + 1, g:g + 1], row_range=rows)


def _one_thread():
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)


def oracle_grads(host, dout, wr, bi, w):
    """Both oracle backwards, one (branch, batch, group, row range) job per
    worker; the results of row ranges covering [0, N) add up."""
    import multiprocessing as mp
    global _JOB
    _JOB = tuple(t.float().numpy() for t in (host["q"], host["k"], host["v"], host["q_idx"], host["k_idx"], dout)) + \
        (bi, wr.numpy(), w)
    n = w.batch * w.kv_heads
    chunks = max(1, WORKERS // n) if w.seqlen >= 16384 else 1
    step = -(-w.seqlen // chunks)
    ranges = [(i, min(w.seqlen, i + step)) for i in range(0, w.seqlen, step)]
    jobs = [(kind, bg, r) for kind in ("main", "kl") for bg in range(n) for r in ranges]
    with mp.get_context("fork").Pool(min(WORKERS, len(jobs)), initializer=_one_thread) as pool:
        parts = pool.map(_job, jobs)
    B, N, G, D, Di = w.batch, w.seqlen, w.group_size, w.head_dim, w.index_dim
    dq = np.zeros((B, N, w.q_heads, D))
    dk = np.zeros((B, N, w.kv_heads, D))
    dv = np.zeros((B, N, w.kv_heads, D))
    dqi = np.zeros((B, N, w.kv_heads, Di))
    dki = np.zeros((B, N, Di))
    for (kind, bg, _), res in zip(jobs, parts):
        b, g = divmod(bg, w.kv_heads)
        if kind == "main":
            a, c, e = res
            dq[b, :, g * G:(g + 1) * G] += a[0]
            dk[b, :, g] += c[0, :, 0]
            dv[b, :, g] += e[0, :, 0]
        else:
            a, c = res
            dqi[b, :, g] += a[0, :, 0]
            dki[b] += c[0]
    return dq, dk, dv, dqi, dki


def check_every_element(w, on_gpu_rng=False):
    log(f"{w.name}: B={w.batch} N={w.seqlen} Hkv={w.kv_heads} G={w.group_size} D={w.head_dim} Di={w.index_dim} "
        f"k={w.topk}")
    x, dout, wr, bi, o, lse, ilse, grads = run_gpu(w, on_gpu_rng)
    host = {k: v.cpu() for k, v in x.items() if k != "stripes"}
    want_bi = O.index_topk(host["q_idx"], host["k_idx"], w.block_size, w.topk)
    assert np.array_equal(bi.cpu().numpy(), want_bi)
    t0 = time.time()
    want = oracle_grads(host, dout.cpu(), wr.cpu(), want_bi, w)
    log(f"  oracle backwards ({time.time() - t0:.1f}s)")
    for name, got, ref in zip(("dQ", "dK", "dV", "dq_idx", "dk_idx"), grads, want):
        compare(name, got, ref)
    return x, dout, wr, bi, o, lse, ilse, grads


SMALL = [
    Workload("g8_d128_di128", 1, 1500, 2, 8, 128, 128, topk=4),
    Workload("g1_d64_di64_ragged_b2", 2, 1000, 2, 1, 64, 64, topk=3),
    Workload("g2_hkv3_d128_di64", 1, 777, 3, 2, 128, 64, topk=5),
    Workload("g4_d64_di128_k16", 1, 2100, 1, 4, 64, 128, topk=16),
    Workload("g16", 1, 600, 2, 16, 128, 64, topk=2),
    Workload("g32_dense", 1, 1200, 1, 32, 64, 64, topk=32),
    Workload("k1_local_only", 1, 700, 2, 4, 128, 64, topk=1),
    Workload("short", 2, 100, 2, 4, 128, 128, topk=4),
    Workload("stripes", 1, 3000, 2, 8, 128, 128, topk=6, stripe_frac=0.1, stripe_bias=3.0),
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_fused_backward_every_element(w):
    x, dout, wr, bi, o, lse, ilse, grads = check_every_element(w)
    # the separate kernels' gradients: the same products, summed in a different
    # association at most (dQ's key slices), so within a few bf16 roundings
    dq, dk, dv = msa.sparse_attn_bwd(x["q"], x["k"], x["v"], bi, o, lse, dout)
    dqi, dki = msa.kl_align_bwd(x["q"], x["k"], x["q_idx"], x["k_idx"], bi, lse, ilse, dkl_rows=wr)
    torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV", "dq_idx", "dk_idx"), grads, (dq, dk, dv, dqi, dki)):
        diff = float((a.float() - b.float()).abs().max())
        assert diff <= 2.0 ** -7 * float(b.float().abs().max()), f"{name} differs from the separate kernels: {diff}"


def test_fused_backward_n8k_every_element():
    check_every_element(CONFIGS["n8k"], on_gpu_rng=True)


def test_fused_backward_two_windows_every_element():
    """N = 65,836: the second window's rows reach back into the first window's
    key blocks, whose dK, dV, dk_idx then sum over both windows."""
    check_every_element(Workload("two_windows", 1, 65536 + 300, 2, 8, 128, 128, topk=8), on_gpu_rng=True)


def test_fused_backward_deterministic():
    w = SMALL[-1]
    x, dout, wr, bi, o, lse, ilse, grads = run_gpu(w, on_gpu_rng=False)
    again = msa.fused_bwd(x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], bi, o, lse, ilse, dout, dkl_rows=wr)
    torch.cuda.synchronize()
    for a, b in zip(grads, again):
        assert torch.equal(a, b)


def test_fused_backward_n1m_sampled_rows_and_sum_rules():
    """The million-token workload (B 1, N 1,048,576, Hkv 4, G 8, D = Di = 128,
    k 16): dQ and dq_idx on 1024 seeded rows plus the block-edge rows against
    the oracle; every key's dV and dk_idx through their sum rules (per group,
    dV over all keys sums to the group's dO rows; dk_idx over all keys sums to
    0), within their first-order rounding bounds."""
    w = CONFIGS["n1m"]
    log(f"{w.name}: B={w.batch} N={w.seqlen} Hkv={w.kv_heads} G={w.group_size} D={w.head_dim} k={w.topk}")
    x, dout, wr, bi, o, lse, ilse, grads = run_gpu(w, on_gpu_rng=True)
    dq, dk, dv, dqi, dki = grads
    del o
    pos = sample_rows(w, n=1024)
    b = torch.as_tensor(pos[:, 0], device=DEV)
    i = torch.as_tensor(pos[:, 1], device=DEV)
    kh, vh, kih = x["k"].cpu(), x["v"].cpu(), x["k_idx"].cpu()
    q_rows, qi_rows, do_rows = x["q"][b, i].cpu(), x["q_idx"][b, i].cpu(), dout[b, i].cpu()
    got_bi = bi[b, :, i].cpu().numpy()
    want_bi = O.map_positions(
        lambda c, qr: O.index_topk_rows(None, kih, c, w.block_size, w.topk, q_rows=qr),
        pos, (qi_rows,), workers=1, chunk=1024)
    assert np.array_equal(got_bi, want_bi)
    want_dq = O.map_positions(
        lambda c, br, qr, dr: O.attention_dq_rows(None, kh, vh, None, br, c, w.block_size, q_rows=qr, do_rows=dr),
        pos, (want_bi, q_rows, do_rows), workers=WORKERS)
    compare("dQ (sampled rows)", dq[b, i], want_dq)
    w_rows = wr[b, :, i].cpu().numpy()
    want_dqi = O.map_positions(
        lambda c, br, qr, qir, wrr: O.kl_dq_idx_rows(None, kh, kih, br, c, w.block_size, w_rows=wrr, q_rows=qr,
                                                      qi_rows=qir),
        pos, (want_bi, q_rows, qi_rows, w_rows), workers=WORKERS)
    compare("dq_idx (sampled rows)", dqi[b, i], want_dqi)

    G = w.group_size
    for g in range(w.kv_heads):
        dvf = dv[:, :, g].double()
        dof = dout[:, :, g * G:(g + 1) * G].double()
        lhs = dvf.sum(dim=(0, 1))
        rhs = dof.sum(dim=(0, 1, 2))
        bound = 2.0 ** -8 * dof.abs().sum(dim=(0, 1, 2)) + 2.0 ** -9 * dvf.abs().sum(dim=(0, 1))
        del dvf, dof
        worst = ((lhs - rhs).abs() / bound).max().item()
        log(f"  dV sum rule, group {g}: error / bound = {worst:.3f}")
        assert worst <= 1.0
    c = 1.0 / np.sqrt(w.index_dim)
    dkf = dki.double()
    lhs = dkf.sum(dim=(0, 1))
    bound = 2.0 ** -8 * c * (wr.double().permute(0, 2, 1)[..., None] * x["q_idx"].double().abs()).sum(dim=(0, 1, 2)) \
        + 2.0 ** -9 * dkf.abs().sum(dim=(0, 1))
    worst = (lhs.abs() / bound).max().item()
    log(f"  dk_idx sum rule: error / bound = {worst:.3e}")
    assert worst <= 1.0
    for name, t in (("dK", dk), ("dV", dv), ("dq_idx", dqi), ("dk_idx", dki), ("dQ", dq)):
        assert bool(torch.isfinite(t.float()).all()), name
