"""Parity of the decode path (one new query per sequence against a cache)
through the C ABI with the CPU oracle.

Block indices bit-exact; O within max-abs 1e-2 and LSE within abs 1e-3 of the
float64 oracle (the forward's bars: the same selection and attention, for the
row n_b - 1). Invalid lengths must give ids -1, O = 0 and LSE = -inf. Small
batches are checked on every sequence; the 64-sequence 128K-capacity batch the
benchmark times is checked on a seeded subset of its sequences.
"""
import sys
import time

import numpy as np
import pytest
import torch

import block_sparse_gqa_index_amd as msa
from oracle import msa_oracle as O
from synth import DECODE_CONFIGS, Workload, make_decode_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
O_TOL, LSE_TOL = 1e-2, 1e-3


def log(msg):
    print(f"[decode] {msg}", flush=True)
    sys.stdout.flush()


def _dev(x):
    return {k: (v.to(DEV) if k != "stripes" else v) for k, v in x.items()}


def _check(w, x, bi, o, lse, seqs=None):
    """Compare GPU outputs with the oracle on the sequences `seqs` (all if None),
    each oracle call given only that sequence's cached prefix."""
    lens = x["seqlens"].cpu().numpy().astype(np.int64)
    C = w.seqlen
    seqs = range(w.batch) if seqs is None else seqs
    bi_h, o_h, lse_h = bi.cpu().numpy(), o.float().cpu().numpy(), lse.cpu().numpy()
    worst_o = worst_l = 0.0
    for b in seqs:
        n = int(lens[b])
        keep = max(1, min(n, C))
        sl = slice(b, b + 1)
        ki = x["k_idx"][sl, :keep].cpu()
        kc = x["k"][sl, :keep].cpu()
        vc = x["v"][sl, :keep].cpu()
        # Lengths outside [1, C] are judged against the full capacity.
        n_eff = np.array([n if 1 <= n <= C else (0 if n < 1 else keep + 1)])
        want_bi = O.decode_index_topk(x["q_idx"][sl].cpu(), ki, n_eff, w.block_size, w.topk)
        assert np.array_equal(bi_h[b], want_bi[0]), (b, n, bi_h[b], want_bi[0])
        want_o, want_l = O.decode_attention(x["q"][sl].cpu(), kc, vc, n_eff, want_bi, w.block_size)
        if not np.isfinite(want_l).all():
            assert (o_h[b] == 0).all() and np.isneginf(lse_h[b]).all(), b
            continue
        eo = float(np.abs(o_h[b] - want_o[0]).max())
        el = float(np.abs(lse_h[b] - want_l[0]).max())
        worst_o, worst_l = max(worst_o, eo), max(worst_l, el)
        assert eo <= O_TOL, (b, n, eo)
        assert el <= LSE_TOL, (b, n, el)
    log(f"  {w.name}: {len(list(seqs))} sequences, max|dO|={worst_o:.2e} max|dLSE|={worst_l:.2e}")


def _run(w, lengths):
    log(f"{w.name}: B={w.batch} C={w.seqlen} Hkv={w.kv_heads} G={w.group_size} D={w.head_dim} "
        f"Di={w.index_dim} k={w.topk} {w.dtype} lengths={list(lengths)[:12]}")
    x = _dev(make_decode_inputs(w, device="cpu", lengths=lengths))
    bi, o, lse = msa.decode(x["q_idx"], x["k_idx"], x["q"], x["k"], x["v"], x["seqlens"], w.topk)
    torch.cuda.synchronize()
    return x, bi, o, lse


EDGE = [1, 2, 127, 128, 129, 255, 256, 257, 640, 1000]


@pytest.mark.parametrize("w", [
    Workload("dec_f32", 10, 1000, 1, 4, 64, 64, topk=4, dtype="f32"),
    Workload("dec_bf16", 10, 1000, 2, 8, 128, 128, topk=3),
    Workload("dec_k1", 10, 1000, 2, 2, 64, 128, topk=1),
    Workload("dec_k32", 10, 5000, 3, 1, 128, 64, topk=32),
    Workload("dec_g32", 10, 2000, 2, 32, 64, 128, topk=5),
    Workload("dec_g16_f32", 10, 1500, 2, 16, 128, 128, topk=6, dtype="f32"),
    Workload("dec_hkv40", 10, 1300, 40, 1, 64, 64, topk=7),          # two chunks of 32 groups
    Workload("dec_ties", 10, 3000, 4, 4, 128, 128, topk=9, index_absmax=1),
])
def test_decode_small(w):
    lengths = [min(x, w.seqlen) for x in EDGE]
    lengths[-1] = w.seqlen
    x, bi, o, lse = _run(w, lengths)
    _check(w, x, bi, o, lse)


def test_decode_random_lengths_and_separate_calls():
    w = Workload("dec_rand", 24, 4096, 8, 8, 128, 128, topk=16)
    x = _dev(make_decode_inputs(w, device="cpu"))
    bi, o, lse = msa.decode(x["q_idx"], x["k_idx"], x["q"], x["k"], x["v"], x["seqlens"], w.topk)
    bi2 = msa.decode_index_topk(x["q_idx"], x["k_idx"], x["seqlens"], w.topk)
    o2, lse2 = msa.decode_attn(x["q"], x["k"], x["v"], x["seqlens"], bi2)
    bi3, o3, lse3 = msa.decode(x["q_idx"], x["k_idx"], x["q"], x["k"], x["v"], x["seqlens"], w.topk)
    torch.cuda.synchronize()
    assert torch.equal(bi, bi2) and torch.equal(o, o2) and torch.equal(lse, lse2)
    assert torch.equal(bi, bi3) and torch.equal(o, o3) and torch.equal(lse, lse3)   # reruns are bitwise equal
    _check(w, x, bi, o, lse)


def test_decode_invalid_lengths():
    w = Workload("dec_bad", 4, 600, 2, 4, 64, 64, topk=3)
    x, bi, o, lse = _run(w, [0, 601, -5, 600])
    bi_h = bi.cpu()
    assert (bi_h[:3] == -1).all()
    assert (o[:3].float() == 0).all() and torch.isneginf(lse[:3]).all()
    _check(w, x, bi, o, lse, seqs=[3])


def test_decode_matches_forward_row():
    """The decode selection of a sequence is the forward selection's row n_b - 1
    (both on the GPU, bit for bit)."""
    w = Workload("dec_fwd", 3, 2048, 4, 4, 128, 128, topk=5)
    lengths = [2048, 700, 129]
    x = _dev(make_decode_inputs(w, device="cpu", lengths=lengths))
    bi = msa.decode_index_topk(x["q_idx"], x["k_idx"], x["seqlens"], w.topk)
    q_idx_full = torch.zeros((w.batch, w.seqlen, w.kv_heads, w.index_dim), dtype=x["q_idx"].dtype, device=DEV)
    for b, n in enumerate(lengths):
        q_idx_full[b, n - 1] = x["q_idx"][b]
    bi_full = msa.index_topk(q_idx_full, x["k_idx"], w.topk)
    torch.cuda.synchronize()
    for b, n in enumerate(lengths):
        assert torch.equal(bi[b], bi_full[b, :, n - 1]), b


def test_decode_n128k_b64_sampled_sequences():
    """The benchmark's decode batch (64 sequences, 128K-token caches, lengths
    uniform on [1, 128K]) in its launch configuration; selection checked on 16
    seeded sequences (plus the longest and shortest), O and LSE on 8 of them."""
    w = DECODE_CONFIGS["decode_n128k_b64"]
    log(f"{w.name}: drawing inputs on the device")
    x = make_decode_inputs(w, device=DEV)
    t0 = time.time()
    bi, o, lse = msa.decode(x["q_idx"], x["k_idx"], x["q"], x["k"], x["v"], x["seqlens"], w.topk)
    torch.cuda.synchronize()
    log(f"  decode done ({time.time() - t0:.2f}s)")
    lens = x["seqlens"].cpu().numpy()
    rng = np.random.default_rng(1)
    pick = set(rng.choice(w.batch, size=16, replace=False).tolist())
    pick |= {int(lens.argmax()), int(lens.argmin())}
    pick = sorted(pick)
    bi_h = bi.cpu().numpy()
    for b in pick:
        n = int(lens[b])
        want = O.decode_index_topk(x["q_idx"][b:b + 1].cpu(), x["k_idx"][b:b + 1, :n].cpu(), np.array([n]),
                                   w.block_size, w.topk)
        assert np.array_equal(bi_h[b], want[0]), b
    log(f"  block indices exact on {len(pick)} sequences")
    _check(w, x, bi, o, lse, seqs=pick[:8])


def test_decode_fp8_index_cache():
    """An fp8 e4m3 index cache (integer index values are exact in it): the same
    selection as the bf16 cache and as the oracle, on a ragged batch and on the
    benchmark's 64 x 128K batch."""
    fp8 = torch.float8_e4m3fn
    w = Workload("dec_fp8", 12, 3000, 8, 8, 128, 128, topk=16)
    lengths = [min(x, w.seqlen) for x in EDGE] + [2999, 3000]
    x = _dev(make_decode_inputs(w, device="cpu", lengths=lengths))
    bi = msa.decode_index_topk(x["q_idx"], x["k_idx"], x["seqlens"], w.topk)
    bi8 = msa.decode_index_topk(x["q_idx"].to(fp8), x["k_idx"].to(fp8), x["seqlens"], w.topk)
    w64 = Workload("dec_fp8_di64", 5, 900, 3, 1, 64, 64, topk=4)
    y = _dev(make_decode_inputs(w64, device="cpu", lengths=[900, 1, 129, 256, 640]))
    bj = msa.decode_index_topk(y["q_idx"], y["k_idx"], y["seqlens"], w64.topk)
    bj8 = msa.decode_index_topk(y["q_idx"].to(fp8), y["k_idx"].to(fp8), y["seqlens"], w64.topk)
    torch.cuda.synchronize()
    assert torch.equal(bi, bi8) and torch.equal(bj, bj8)
    want = O.decode_index_topk(x["q_idx"].to(fp8).cpu(), x["k_idx"].to(fp8).cpu(), np.array(lengths),
                               w.block_size, w.topk)
    assert np.array_equal(bi8.cpu().numpy(), want)

    w = DECODE_CONFIGS["decode_n128k_b64"]
    x = make_decode_inputs(w, device=DEV)
    bi = msa.decode_index_topk(x["q_idx"], x["k_idx"], x["seqlens"], w.topk)
    bi8 = msa.decode_index_topk(x["q_idx"].to(fp8), x["k_idx"].to(fp8), x["seqlens"], w.topk)
    torch.cuda.synchronize()
    assert torch.equal(bi, bi8)


def _to_pages(x, w, spare=5, seed=7):
    """The caches of x as page pools [P, 128, ...] in a seeded random page
    order (plus `spare` pages of other values) and the block table [B, nb]."""
    B, C = w.batch, w.seqlen
    nb = -(-C // 128)
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    P = B * nb + spare
    perm = torch.randperm(P, generator=g)[: B * nb].to(torch.int32)
    table = perm.view(B, nb)
    pools = {}
    for name in ("k_idx", "k", "v"):
        t = x[name]
        pad = nb * 128 - C
        if pad:
            t = torch.cat([t, torch.zeros((B, pad) + tuple(t.shape[2:]), dtype=t.dtype, device=t.device)], dim=1)
        pool = torch.randn((P, 128) + tuple(t.shape[2:]), generator=g).to(t.dtype).to(t.device)
        pool[perm.long().to(t.device)] = t.reshape((B * nb, 128) + tuple(t.shape[2:]))
        pools[name] = pool
    return pools, table.to(x["k"].device), P


@pytest.mark.parametrize("w", [
    Workload("paged_bf16", 10, 1000, 2, 8, 128, 128, topk=3),
    Workload("paged_f32", 10, 1000, 1, 4, 64, 64, topk=4, dtype="f32"),
    Workload("paged_k16", 6, 4096, 8, 8, 128, 128, topk=16),
])
def test_decode_paged_equals_contiguous(w):
    """Paged caches (random page order) give bitwise the contiguous decode's
    results, which the oracle checks."""
    lengths = [min(x, w.seqlen) for x in EDGE][: w.batch]
    lengths[-1] = w.seqlen
    x, bi, o, lse = _run(w, lengths)
    pools, table, P = _to_pages(x, w)
    bip, op, lsep = msa.decode_paged(x["q_idx"], pools["k_idx"], x["q"], pools["k"], pools["v"], table, x["seqlens"],
                                     w.topk)
    bip2 = msa.decode_paged_index_topk(x["q_idx"], pools["k_idx"], table, x["seqlens"], w.topk)
    op2, lsep2 = msa.decode_paged_attn(x["q"], pools["k"], pools["v"], table, x["seqlens"], bip2)
    torch.cuda.synchronize()
    assert torch.equal(bip, bi) and torch.equal(op, o) and torch.equal(lsep, lse)
    assert torch.equal(bip2, bi) and torch.equal(op2, o) and torch.equal(lsep2, lse)
    _check(w, x, bip, op, lsep)


def test_decode_paged_fp8_index_and_bad_pages():
    fp8 = torch.float8_e4m3fn
    w = Workload("paged_fp8", 4, 3000, 4, 4, 128, 128, topk=8)
    x = _dev(make_decode_inputs(w, device="cpu", lengths=[3000, 2000, 700, 129]))
    pools, table, P = _to_pages(x, w)
    bi = msa.decode_index_topk(x["q_idx"], x["k_idx"], x["seqlens"], w.topk)
    bi8 = msa.decode_paged_index_topk(x["q_idx"].to(fp8), pools["k_idx"].to(fp8), table, x["seqlens"], w.topk)
    torch.cuda.synchronize()
    assert torch.equal(bi8, bi)
    # Page ids outside the pool: those blocks are never read; the other sequences are unchanged.
    bad = table.clone()
    bad[0, 3] = -1
    bad[0, 5] = P
    bip, op, lsep = msa.decode_paged(x["q_idx"], pools["k_idx"], x["q"], pools["k"], pools["v"], bad, x["seqlens"],
                                     w.topk)
    bic, oc, lsec = msa.decode(x["q_idx"], x["k_idx"], x["q"], x["k"], x["v"], x["seqlens"], w.topk)
    torch.cuda.synchronize()
    assert torch.equal(bip[1:], bic[1:]) and torch.equal(op[1:], oc[1:]) and torch.equal(lsep[1:], lsec[1:])
    # 23 competing blocks for k - 1 = 7 slots: the -inf blocks are never kept
    assert torch.isfinite(lsep[0]).all() and bool(((bip[0] != 3) & (bip[0] != 5)).all())


@pytest.mark.parametrize("R", [3, 4])
def test_decode_two_column_sets(R):
    """R * Hkv in (16, 32] (24 and 32 (query, group) columns): the block scores
    run two 16-column sets per wave. bf16 and fp8 index caches against the
    oracle, and paged caches with pages outside the pool."""
    fp8 = torch.float8_e4m3fn
    w = Workload(f"dec_cs2_r{R}", 4, 2000, 8, 2, 128, 128, topk=8)
    lengths = [2000, 129, 2, 1999]
    x = _dev(make_decode_inputs(w, device="cpu", lengths=lengths))
    qi, q = _multi_queries(w, R, seed=17)
    bi = msa.decode_index_topk(qi, x["k_idx"], x["seqlens"], w.topk)
    bi8 = msa.decode_index_topk(qi.to(fp8), x["k_idx"].to(fp8), x["seqlens"], w.topk)
    torch.cuda.synchronize()
    want = O.decode_index_topk(qi.cpu(), x["k_idx"].cpu(), np.array(lengths), w.block_size, w.topk)
    assert np.array_equal(bi.cpu().numpy(), want)
    want8 = O.decode_index_topk(qi.to(fp8).cpu(), x["k_idx"].to(fp8).cpu(), np.array(lengths), w.block_size, w.topk)
    assert np.array_equal(bi8.cpu().numpy(), want8)
    pools, table, P = _to_pages(x, w)
    bad = table.clone()
    bad[0, 3] = -1
    bad[0, 5] = P
    for ki, bref in ((pools["k_idx"], bi), (pools["k_idx"].to(fp8), bi8)):
        qq = qi if ki.dtype != fp8 else qi.to(fp8)
        bp = msa.decode_paged_index_topk(qq, ki, table, x["seqlens"], w.topk)
        bb = msa.decode_paged_index_topk(qq, ki, bad, x["seqlens"], w.topk)
        torch.cuda.synchronize()
        assert torch.equal(bp, bref) and torch.equal(bb[1:], bref[1:])
        assert bool(((bb[0] != 3) & (bb[0] != 5)).all())


def test_decode_1m_capacity():
    """Million-token caches (up to 8191 competing blocks: the top-k scans its
    scores in several chunks per lane), the 1M workload's model sizes."""
    w = Workload("dec_1m", 2, 1048576, 4, 8, 128, 128, topk=16)
    x = make_decode_inputs(w, device=DEV, lengths=[1048576, 700001])
    bi, o, lse = msa.decode(x["q_idx"], x["k_idx"], x["q"], x["k"], x["v"], x["seqlens"], w.topk)
    bi8 = msa.decode_index_topk(x["q_idx"].to(torch.float8_e4m3fn), x["k_idx"].to(torch.float8_e4m3fn),
                                x["seqlens"], w.topk)
    torch.cuda.synchronize()
    assert torch.equal(bi, bi8)
    _check(w, x, bi, o, lse)


def _multi_queries(w, R, seed=11):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    qi = torch.randint(-4, 5, (w.batch, R, w.kv_heads, w.index_dim), generator=g).to(dt)
    q = torch.randn((w.batch, R, w.q_heads, w.head_dim), generator=g).to(dt)
    return qi.to(DEV), q.to(DEV)


@pytest.mark.parametrize("R", [2, 4, 7])
def test_decode_multi_query(R):
    """R new tokens per sequence (row r at position n_b - R + r): block ids,
    O and LSE against the oracle; each row bitwise equal to a one-query decode
    of the prefix that ends at it; rows at negative positions empty."""
    w = Workload(f"dec_r{R}", 6, 3000, 4, 8, 128, 128, topk=8)
    lengths = [1, 3, 129, 1000, 2999, 3000]
    x = _dev(make_decode_inputs(w, device="cpu", lengths=lengths))
    qi, q = _multi_queries(w, R)
    bi, o, lse = msa.decode(qi, x["k_idx"], q, x["k"], x["v"], x["seqlens"], w.topk)
    torch.cuda.synchronize()
    assert tuple(bi.shape) == (6, 4, R, 8) and tuple(o.shape) == (6, R, 32, 128) and tuple(lse.shape) == (6, 32, R)
    lens = np.array(lengths)
    want_bi = O.decode_index_topk(qi.cpu(), x["k_idx"].cpu(), lens, w.block_size, w.topk)
    assert np.array_equal(bi.cpu().numpy(), want_bi)
    want_o, want_l = O.decode_attention(q.cpu(), x["k"].cpu(), x["v"].cpu(), lens, want_bi, w.block_size)
    got_o, got_l = o.float().cpu().numpy(), lse.cpu().numpy()
    fin = np.isfinite(want_l)
    assert np.array_equal(fin, np.isfinite(got_l))
    assert (got_o[~fin.any(axis=1)] == 0).all()
    # O is stored in bf16: where |O| >= 4 its spacing is 2^-5, so the rounding
    # alone (half a spacing, 0.0156) exceeds 1e-2; there the bar is that
    # rounding plus 2e-3 (rows with one or two tokens, as at positions 1-2, can
    # reach |O| >= 4).
    big = np.abs(want_o) >= 4.0
    err = np.abs(got_o - want_o)
    eo = float(err[~big].max())
    el = float(np.abs(got_l[fin] - want_l[fin]).max())
    log(f"  dec_r{R}: max|dO|={eo:.2e} (|O| < 4), {int(big.sum())} elements with |O| >= 4 "
        f"(max err {float(err[big].max()) if big.any() else 0.0:.2e}), max|dLSE|={el:.2e}")
    assert eo <= O_TOL and el <= LSE_TOL
    assert (err[big] <= 2.0 ** -6 + 2e-3).all()
    for r in range(R):
        n_r = torch.clamp(x["seqlens"] - R + r + 1, min=0).to(torch.int32)
        b1, o1, l1 = msa.decode(qi[:, r].contiguous(), x["k_idx"], q[:, r].contiguous(), x["k"], x["v"], n_r, w.topk)
        torch.cuda.synchronize()
        assert torch.equal(b1, bi[:, :, r]) and torch.equal(o1, o[:, r]) and torch.equal(l1, lse[:, :, r])
    pools, table, P = _to_pages(x, w)
    bp, op, lp = msa.decode_paged(qi, pools["k_idx"], q, pools["k"], pools["v"], table, x["seqlens"], w.topk)
    torch.cuda.synchronize()
    assert torch.equal(bp, bi) and torch.equal(op, o) and torch.equal(lp, lse)


@pytest.mark.parametrize("w,R", [
    (Workload("dec_r3_hkv40", 4, 1300, 40, 1, 64, 64, topk=7), 3),        # R * Hkv = 120: four column chunks
    (Workload("dec_r5_k32_g32", 3, 5000, 2, 32, 64, 128, topk=32), 5),    # k = 32, G = 32
    (Workload("dec_r2_f32", 4, 700, 1, 4, 64, 64, topk=4, dtype="f32"), 2),
])
def test_decode_multi_query_shapes(w, R):
    lengths = [w.seqlen, 129, 2, w.seqlen - 1][: w.batch]
    x = _dev(make_decode_inputs(w, device="cpu", lengths=lengths))
    qi, q = _multi_queries(w, R, seed=13)
    bi, o, lse = msa.decode(qi, x["k_idx"], q, x["k"], x["v"], x["seqlens"], w.topk)
    torch.cuda.synchronize()
    lens = np.array(lengths)
    want_bi = O.decode_index_topk(qi.cpu(), x["k_idx"].cpu(), lens, w.block_size, w.topk)
    assert np.array_equal(bi.cpu().numpy(), want_bi)
    want_o, want_l = O.decode_attention(q.cpu(), x["k"].cpu(), x["v"].cpu(), lens, want_bi, w.block_size)
    got_o, got_l = o.float().cpu().numpy(), lse.cpu().numpy()
    fin = np.isfinite(want_l)
    assert np.array_equal(fin, np.isfinite(got_l))
    err = np.abs(got_o - want_o)
    big = np.abs(want_o) >= 4.0
    assert float(err[~big].max()) <= O_TOL and (err[big] <= 2.0 ** -6 + 2e-3).all()
    assert float(np.abs(got_l[fin] - want_l[fin]).max()) <= LSE_TOL
