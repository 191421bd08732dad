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
