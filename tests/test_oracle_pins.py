"""Pins of the CPU oracle against facts that do not come from the oracle itself:
hand-worked values, brute force, closed forms, torch's dense attention and
scipy's relative entropy. CPU only."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import msa_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


def _golden():
    with open(os.path.join(HERE, "golden", "hand_worked.json")) as f:
        return json.load(f)


# ---------------------------------------------------------------- selection --

def test_hand_worked_selection():
    g = _golden()["selection"]
    Bk, k = g["block_size"], g["topk"]
    k_idx = np.asarray(g["k_idx"], dtype=np.float64)[None]          # [1, N, Di]
    N, Di = k_idx.shape[1:]
    for row in g["rows"]:
        q_idx = np.zeros((1, N, 1, Di))
        q_idx[0, row["i"], 0] = row["q_idx"]
        got = O.index_topk_rows(q_idx, k_idx, np.array([[0, row["i"]]]), Bk, k)
        assert got[0, 0].tolist() == row["expect"], row["why"]


def _brute_force_row(q_row, k_idx_b, i, Bk, k):
    """Token scores by explicit loops, block max by loops, and the kept set as the
    unique subset whose members all outrank every non-member under
    (score desc, id asc), found by enumerating every subset."""
    L = i // Bk
    m = []
    for j in range(L):
        best = None
        for t in range(j * Bk, (j + 1) * Bk):
            s = 0.0
            for d in range(len(q_row)):
                s += float(q_row[d]) * float(k_idx_b[t][d])
            best = s if best is None or s > best else best
        m.append(best)

    def outranks(a, b):
        return m[a] > m[b] or (m[a] == m[b] and a < b)

    size = min(k - 1, L)
    found = []
    for subset in itertools.combinations(range(L), size):
        rest = [j for j in range(L) if j not in subset]
        if all(outranks(a, b) for a in subset for b in rest):
            found.append(subset)
    assert len(found) == 1
    ids = sorted(list(found[0]) + [L])
    return ids + [-1] * (k - len(ids))


@pytest.mark.parametrize("seed,N,Bk,k,Di,Hkv", [
    (0, 32, 4, 4, 3, 2),     # many ties (values in -2..2, Di = 3)
    (1, 29, 4, 3, 2, 1),     # ragged tail: N % Bk != 0
    (2, 24, 3, 6, 4, 2),     # k - 1 >= candidates for most rows
    (3, 40, 5, 1, 3, 1),     # k = 1: only the local block
])
def test_selection_matches_brute_force(seed, N, Bk, k, Di, Hkv):
    rng = np.random.default_rng(seed)
    q_idx = rng.integers(-2, 3, size=(1, N, Hkv, Di)).astype(np.float64)
    k_idx = rng.integers(-2, 3, size=(1, N, Di)).astype(np.float64)
    got = O.index_topk(q_idx, k_idx, Bk, k)
    for g in range(Hkv):
        for i in range(N):
            want = _brute_force_row(q_idx[0, i, g], k_idx[0], i, Bk, k)
            assert got[0, g, i].tolist() == want, (g, i)


def test_fp8_inputs_are_decoded_exactly():
    """OCP fp8 e4m3 (no infinities, bias 7): 0x38 = 1, 0xB8 = -1, 0x7E = 448
    (largest finite: exponent 15, mantissa 6/8), 0x08 = 2^-6 (smallest normal),
    0x01 = 2^-9 (smallest subnormal), 0x54 = 12 (2^3 * 1.5), 0x7F = NaN."""
    bits = torch.tensor([0x38, 0xB8, 0x7E, 0x08, 0x01, 0x54, 0x7F], dtype=torch.uint8)
    got = O._arr(bits.view(torch.float8_e4m3fn)).astype(np.float64)
    want = [1.0, -1.0, 448.0, 2.0 ** -6, 2.0 ** -9, 12.0]
    assert got[:6].tolist() == want and np.isnan(got[6])
    # and the selection over fp8 tensors is the brute-force one
    rng = np.random.default_rng(5)
    N, Bk, k, Di = 30, 4, 4, 3
    q8 = torch.as_tensor(rng.integers(-7, 8, size=(1, N, 1, Di)), dtype=torch.float32).to(torch.float8_e4m3fn)
    k8 = torch.as_tensor(rng.integers(-7, 8, size=(1, N, Di)), dtype=torch.float32).to(torch.float8_e4m3fn)
    got = O.index_topk(q8, k8, Bk, k)
    qf, kf = q8.float().numpy(), k8.float().numpy()
    for i in range(N):
        assert got[0, 0, i].tolist() == _brute_force_row(qf[0, i, 0], kf[0], i, Bk, k), i


def test_fp4_inputs_are_decoded_exactly():
    """OCP MX fp4 e2m1 (bias 1, one mantissa bit), the format's value table:
    codes 0..7 are 0, 0.5, 1, 1.5, 2, 3, 4, 6 and codes 8..15 their negatives;
    two codes per byte, the first in the low nibble (byte 0x72 = [1, 6])."""
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
    packed = torch.tensor([(2 * c) | ((2 * c + 1) << 4) for c in range(8)], dtype=torch.uint8)
    got = O._arr(packed.view(torch.float4_e2m1fn_x2))
    assert got.dtype == np.float32 and got.tolist() == table
    assert O._arr(torch.tensor([0x72], dtype=torch.uint8).view(torch.float4_e2m1fn_x2)).tolist() == [1.0, 6.0]
    # the encoder used for test inputs holds the integers -4..4 and +-6 exactly
    from synth import to_fp4_e2m1
    ints = torch.tensor([[-6, -4, -3, -2, -1, 0, 1, 2, 3, 4, 6, 0]], dtype=torch.float32)
    assert O._arr(to_fp4_e2m1(ints)).tolist() == ints.tolist()
    # and the selection over fp4 tensors is the brute-force one on the decoded values
    rng = np.random.default_rng(6)
    N, Bk, k, Di = 30, 4, 4, 4
    q4 = to_fp4_e2m1(torch.as_tensor(rng.integers(-4, 5, size=(1, N, 1, Di)), dtype=torch.float32))
    k4 = to_fp4_e2m1(torch.as_tensor(rng.integers(-4, 5, size=(1, N, Di)), dtype=torch.float32))
    got = O.index_topk(q4, k4, Bk, k)
    qf, kf = O._arr(q4), O._arr(k4)
    for i in range(N):
        assert got[0, 0, i].tolist() == _brute_force_row(qf[0, i, 0], kf[0], i, Bk, k), i


def test_selection_invariants_tiny_workload():
    from synth import get_workload, make_inputs
    w = get_workload("tiny")
    x = make_inputs(w)
    bi = O.index_topk(x["q_idx"], x["k_idx"], w.block_size, w.topk)
    Bk, k = w.block_size, w.topk
    for i in range(w.seqlen):
        L = i // Bk
        row = bi[0, 0, i].tolist()
        valid = [j for j in row if j >= 0]
        assert len(valid) == min(k, L + 1)                       # count
        assert valid == sorted(set(valid))                       # distinct, ascending
        assert valid[-1] == L                                    # local block present, last
        assert all(0 <= j <= L for j in valid)
        assert row[len(valid):] == [-1] * (k - len(valid))       # padding
        assert len(O.token_set(row, i, Bk)) == O.token_count(i, Bk, k)


def test_exp_free_equivalence():
    """Ranking by softmax probabilities (max-pooled per block) keeps exactly the
    same blocks as ranking the raw scores: softmax preserves order."""
    rng = np.random.default_rng(7)
    Bk, k, N, Di, Hkv = 8, 4, 96, 6, 2
    q_idx = rng.integers(-4, 5, size=(1, N, Hkv, Di)).astype(np.float64)
    k_idx = rng.integers(-4, 5, size=(1, N, Di)).astype(np.float64)
    raw = O.index_topk(q_idx, k_idx, Bk, k)
    for g in range(Hkv):
        for i in range(N):
            L = i // Bk
            if L == 0:
                continue
            s = k_idx[0, :L * Bk] @ q_idx[0, i, g]
            logp = s - (s.max() + math.log(np.exp(s - s.max()).sum()))   # log-softmax
            mp = logp.reshape(L, Bk).max(axis=1)
            ids = O.select_blocks(mp, L, k)
            assert ids + [-1] * (k - len(ids)) == raw[0, g, i].tolist()


def test_batched_scores_match_single_row():
    rng = np.random.default_rng(11)
    Bk, k, N, Di, Hkv = 4, 3, 64, 5, 3
    q_idx = rng.integers(-4, 5, size=(2, N, Hkv, Di)).astype(np.float64)
    k_idx = rng.integers(-4, 5, size=(2, N, Di)).astype(np.float64)
    pos = np.array([(b, i) for b in range(2) for i in range(0, N, 3)])
    got = O.index_topk_rows(q_idx, k_idx, pos, Bk, k, key_chunk=8)
    for r, (b, i) in enumerate(pos):
        for g in range(Hkv):
            m = O.visible_block_scores(q_idx[b, i, g], k_idx[b], i, Bk)
            ids = O.select_blocks(m, i // Bk, k)
            assert got[r, g].tolist() == ids + [-1] * (k - len(ids))


# ---------------------------------------------------------------- attention --

def test_hand_worked_attention():
    g = _golden()["attention"]
    Bk = g["block_size"]
    kk = np.asarray(g["k"])[None, :, None, None]
    vv = np.asarray(g["v"])[None, :, None, None]
    N = kk.shape[1]
    for row in g["rows"]:
        q = np.zeros((1, N, 1, 1))
        q[0, row["i"], 0, 0] = g["q"]
        bi = np.array([[row["blocks"]]])
        o, lse = O.attention_rows(q, kk, vv, bi, np.array([[0, row["i"]]]), Bk, scale=g["scale"])
        assert o[0, 0, 0] == pytest.approx(row["o"], abs=1e-14), row["why"]
        assert lse[0, 0] == pytest.approx(row["lse_value"], abs=1e-14), row["why"]


def _rand_case(seed, B=1, N=96, Hkv=2, G=3, D=16, Di=8, Bk=8, k=4):
    rng = np.random.default_rng(seed)
    q_idx = rng.integers(-4, 5, size=(B, N, Hkv, Di)).astype(np.float64)
    k_idx = rng.integers(-4, 5, size=(B, N, Di)).astype(np.float64)
    q = rng.standard_normal((B, N, Hkv * G, D))
    kk = rng.standard_normal((B, N, Hkv, D))
    vv = rng.standard_normal((B, N, Hkv, D))
    return q_idx, k_idx, q, kk, vv


@pytest.mark.parametrize("N,Bk", [(96, 8), (90, 8), (7, 8)])
def test_warmup_reduces_to_dense_causal_gqa(N, Bk):
    """With k >= number of blocks every block is kept: the sparse output must
    equal dense causal GQA attention (the indexer warm-up of section 'Como se
    entrena MSA'), here torch's SDPA in float64."""
    Hkv, G, D = 2, 3, 16
    q_idx, k_idx, q, kk, vv = _rand_case(5, N=N, Hkv=Hkv, G=G, D=D, Bk=Bk)
    k = -(-N // Bk) + 2
    bi = O.index_topk(q_idx, k_idx, Bk, k)
    o, lse = O.sparse_attention(q, kk, vv, bi, Bk)
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)          # [B, Hq, N, D]
    kt = torch.from_numpy(kk).permute(0, 2, 1, 3)
    vt = torch.from_numpy(vv).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True,
                                                           enable_gqa=True)
    np.testing.assert_allclose(o, ref.permute(0, 2, 1, 3).numpy(), atol=1e-12, rtol=0)
    scores = (qt @ kt.repeat_interleave(G, dim=1).transpose(-1, -2)) / math.sqrt(D)
    mask = torch.ones(N, N, dtype=torch.bool).tril()
    ref_lse = torch.logsumexp(scores.masked_fill(~mask, float("-inf")), dim=-1)
    np.testing.assert_allclose(lse, ref_lse.numpy(), atol=1e-12, rtol=0)


def test_zero_query_gives_uniform_average():
    """Q = 0 makes every logit 0: LSE = ln|T_i| and O = mean of V over T_i, with
    T_i enumerated here by explicit loops over the kept blocks."""
    Bk, k = 8, 4
    q_idx, k_idx, q, kk, vv = _rand_case(9, N=100, Bk=Bk, k=k)
    q[:] = 0.0
    bi = O.index_topk(q_idx, k_idx, Bk, k)
    o, lse = O.sparse_attention(q, kk, vv, bi, Bk)
    G = q.shape[2] // kk.shape[2]
    for g in range(kk.shape[2]):
        for i in range(q.shape[1]):
            toks = []
            for j in bi[0, g, i]:
                if j >= 0:
                    for t in range(j * Bk, j * Bk + Bk):
                        if t <= i:
                            toks.append(t)
            assert len(toks) == O.token_count(i, Bk, k)
            mean_v = sum(vv[0, t, g] for t in toks) / len(toks)
            for h in range(g * G, (g + 1) * G):
                assert lse[0, h, i] == pytest.approx(math.log(len(toks)), abs=1e-12)
                np.testing.assert_allclose(o[0, i, h], mean_v, atol=1e-12)


def test_constant_values_give_constant_output():
    Bk, k = 8, 3
    q_idx, k_idx, q, kk, vv = _rand_case(13, N=64, Bk=Bk, k=k)
    vv[:] = 0.375
    bi = O.index_topk(q_idx, k_idx, Bk, k)
    o, _ = O.sparse_attention(q, kk, vv, bi, Bk)
    np.testing.assert_allclose(o, 0.375, atol=1e-13)


def test_scale_enters_logits():
    """An explicit scale equal to 1/sqrt(D) matches the default; doubling the
    scale equals doubling Q."""
    Bk, k = 8, 3
    q_idx, k_idx, q, kk, vv = _rand_case(17, N=48, Bk=Bk, k=k)
    bi = O.index_topk(q_idx, k_idx, Bk, k)
    D = q.shape[-1]
    o0, l0 = O.sparse_attention(q, kk, vv, bi, Bk)
    o1, l1 = O.sparse_attention(q, kk, vv, bi, Bk, scale=1 / math.sqrt(D))
    o2, l2 = O.sparse_attention(2 * q, kk, vv, bi, Bk)
    o3, l3 = O.sparse_attention(q, kk, vv, bi, Bk, scale=2 / math.sqrt(D))
    np.testing.assert_allclose(o0, o1, atol=1e-14)
    np.testing.assert_allclose(o2, o3, atol=1e-12)
    np.testing.assert_allclose(l2, l3, atol=1e-12)


# ----------------------------------------------------------------------- KL --

def test_hand_worked_kl():
    g = _golden()["kl"]
    Bk, i = g["block_size"], g["i"]
    N = len(g["k"])
    H = len(g["q_heads"])
    q = np.zeros((1, N, H, 1))
    q[0, i, :, 0] = g["q_heads"]
    kk = np.asarray(g["k"])[None, :, None, None]
    q_idx = np.zeros((1, N, 1, 1))
    q_idx[0, i, 0, 0] = g["q_idx"]
    k_idx = np.asarray(g["k_idx"])[None, :, None]
    bi = np.array([[g["blocks"]]])
    kl = O.kl_rows(q, kk, q_idx, k_idx, bi, np.array([[0, i]]), Bk,
                   scale=g["scale"], index_scale=g["index_scale"])
    assert kl[0, 0] == pytest.approx(g["expect"], abs=1e-14), g["why"]


def test_kl_dense_matches_scipy_entropy():
    """Warm-up case (all blocks kept): teacher and student are dense causal
    softmaxes built with torch, the KL is scipy's relative entropy."""
    from scipy.stats import entropy
    Bk, N, Hkv, G, D, Di = 8, 40, 2, 3, 16, 8
    q_idx, k_idx, q, kk, vv = _rand_case(21, N=N, Hkv=Hkv, G=G, D=D, Di=Di, Bk=Bk)
    k = -(-N // Bk) + 1
    bi = O.index_topk(q_idx, k_idx, Bk, k)
    kl, total = O.kl_align(q, kk, q_idx, k_idx, bi, Bk, index_scale=0.25)
    mask = torch.ones(N, N, dtype=torch.bool).tril()
    for g in range(Hkv):
        qh = torch.from_numpy(q[0, :, g * G:(g + 1) * G]).permute(1, 0, 2)       # [G, N, D]
        s = (qh @ torch.from_numpy(kk[0, :, g]).T) / math.sqrt(D)
        teacher = torch.softmax(s.masked_fill(~mask, float("-inf")), dim=-1).mean(0)
        u = 0.25 * (torch.from_numpy(q_idx[0, :, g]) @ torch.from_numpy(k_idx[0]).T)
        student = torch.softmax(u.masked_fill(~mask, float("-inf")), dim=-1)
        for i in range(N):
            ref = entropy(teacher[i, :i + 1].numpy(), student[i, :i + 1].numpy())
            assert kl[0, g, i] == pytest.approx(ref, abs=1e-10)
    assert total == pytest.approx(kl.sum(), abs=1e-9)


def test_kl_nonnegative_and_identity_is_zero():
    Bk, N, D = 8, 64, 16
    q_idx, k_idx, q, kk, vv = _rand_case(23, N=N, Hkv=1, G=1, D=D, Di=D, Bk=Bk)
    bi = O.index_topk(q_idx, k_idx, Bk, 3)
    kl, _ = O.kl_align(q, kk, q_idx, k_idx, bi, Bk)
    assert (kl >= -1e-12).all()
    # identity: index branch = main branch (G = 1, same vectors, same scale)
    kl0, s0 = O.kl_align(q, kk, q, kk[:, :, 0, :], bi, Bk, scale=0.3, index_scale=0.3)
    np.testing.assert_allclose(kl0, 0.0, atol=1e-12)


def test_kl_teacher_of_identical_heads_is_that_head():
    Bk, N, D = 8, 48, 16
    q_idx, k_idx, q1, kk, vv = _rand_case(29, N=N, Hkv=1, G=1, D=D, Bk=Bk)
    bi = O.index_topk(q_idx, k_idx, Bk, 3)
    q4 = np.repeat(q1, 4, axis=2)
    a, _ = O.kl_align(q1, kk, q_idx, k_idx, bi, Bk)
    b, _ = O.kl_align(q4, kk, q_idx, k_idx, bi, Bk)
    np.testing.assert_allclose(a, b, atol=1e-12)


# --------------------------------------------------------------- mutations --

def test_planted_mistakes_are_caught(monkeypatch):
    """Each planted mistake in the oracle makes one of the pins above fail."""
    rng = np.random.default_rng(0)
    q_idx = rng.integers(-2, 3, size=(1, 32, 1, 3)).astype(np.float64)
    k_idx = rng.integers(-2, 3, size=(1, 32, 3)).astype(np.float64)

    def selection_ok():
        got = O.index_topk(q_idx, k_idx, 4, 4)
        return all(got[0, 0, i].tolist() == _brute_force_row(q_idx[0, i, 0], k_idx[0], i, 4, 4)
                   for i in range(32))

    assert selection_ok()
    real_select = O.select_blocks

    def wrong_tiebreak(m, L, k):   # higher id wins ties
        order = np.lexsort((-np.arange(L), -np.asarray(m)))
        return sorted([int(j) for j in order[:min(k - 1, L)]] + [L])

    monkeypatch.setattr(O, "select_blocks", wrong_tiebreak)
    assert not selection_ok()
    monkeypatch.setattr(O, "select_blocks", real_select)

    real_scores = O.visible_block_scores

    def mean_pool(q_row, k_b, i, Bk):   # mean instead of max pooling
        L = i // Bk
        return (np.asarray(k_b[:L * Bk]) @ q_row).reshape(L, Bk).mean(axis=1)

    monkeypatch.setattr(O, "visible_block_scores", mean_pool)
    monkeypatch.setattr(O, "index_topk_rows",
                        lambda qi, ki, pos, Bk, k: np.array(
                            [[O._pad(real_select(mean_pool(qi[b, i, g], ki[b], i, Bk), i // Bk, k), k)
                              for g in range(qi.shape[2])] for b, i in pos], dtype=np.int32))
    assert not selection_ok()


# ----------------------------------------------------------------- backward --

def _masked_dense_grads(q, kk, vv, do, bi, Bk, scale):
    """Gradients by torch autograd (float64) of dense attention whose logits are
    masked to each row's selected tokens: an independent derivation of the
    backward formulas."""
    B, N, Hq, D = q.shape
    Hkv = kk.shape[2]
    G = Hq // Hkv
    mask = torch.zeros(B, Hq, N, N, dtype=torch.bool)
    for b in range(B):
        for g in range(Hkv):
            for i in range(N):
                mask[b, g * G:(g + 1) * G, i, O.token_set(bi[b, g, i], i, Bk)] = True
    qt = torch.tensor(q).permute(0, 2, 1, 3).requires_grad_()
    kt = torch.tensor(kk).permute(0, 2, 1, 3).requires_grad_()
    vt = torch.tensor(vv).permute(0, 2, 1, 3).requires_grad_()
    ke = kt.repeat_interleave(G, dim=1)
    ve = vt.repeat_interleave(G, dim=1)
    logits = (scale * (qt @ ke.transpose(-1, -2))).masked_fill(~mask, float("-inf"))
    out = torch.softmax(logits, dim=-1) @ ve
    (out * torch.tensor(do).permute(0, 2, 1, 3)).sum().backward()
    return (qt.grad.permute(0, 2, 1, 3).numpy(), kt.grad.permute(0, 2, 1, 3).numpy(),
            vt.grad.permute(0, 2, 1, 3).numpy())


@pytest.mark.parametrize("seed,N,Bk,k,G", [(0, 64, 8, 3, 2), (1, 61, 8, 4, 1), (2, 40, 4, 16, 3)])
def test_backward_matches_autograd(seed, N, Bk, k, G):
    Hkv, D = 2, 8
    q_idx, k_idx, q, kk, vv = _rand_case(seed, N=N, Hkv=Hkv, G=G, D=D, Bk=Bk)
    do = np.random.default_rng(seed + 100).standard_normal(q.shape)
    bi = O.index_topk(q_idx, k_idx, Bk, k)
    scale = 0.3
    got = O.attention_backward(q, kk, vv, do, bi, Bk, scale)
    want = _masked_dense_grads(q, kk, vv, do, bi, Bk, scale)
    for a, b in zip(got, want):
        np.testing.assert_allclose(a, b, atol=1e-12, rtol=0)
    pos = np.array([(0, i) for i in range(0, N, 5)])
    rows = bi.transpose(0, 2, 1, 3)[0, pos[:, 1]]
    np.testing.assert_allclose(O.attention_dq_rows(q, kk, vv, do, rows, pos, Bk, scale), got[0][0, pos[:, 1]],
                               atol=1e-14, rtol=0)


def test_backward_finite_differences():
    """Directional derivative of <dO, O> (the pinned forward) by central
    differences equals <dQ, a> + <dK, b> + <dV, c>."""
    N, Bk, k, Hkv, G, D = 48, 8, 3, 2, 2, 8
    q_idx, k_idx, q, kk, vv = _rand_case(7, N=N, Hkv=Hkv, G=G, D=D, Bk=Bk)
    rng = np.random.default_rng(8)
    do = rng.standard_normal(q.shape)
    a, b, c = rng.standard_normal(q.shape), rng.standard_normal(kk.shape), rng.standard_normal(vv.shape)
    bi = O.index_topk(q_idx, k_idx, Bk, k)
    dq, dk, dv = O.attention_backward(q, kk, vv, do, bi, Bk)

    def f(t):
        o, _ = O.sparse_attention(q + t * a, kk + t * b, vv + t * c, bi, Bk)
        return float((o * do).sum())

    eps = 1e-5
    fd = (f(eps) - f(-eps)) / (2 * eps)
    an = float((dq * a).sum() + (dk * b).sum() + (dv * c).sum())
    assert abs(fd - an) <= 1e-7 * max(1.0, abs(an))


@pytest.mark.parametrize("N,Bk", [(64, 8), (50, 8)])
def test_backward_warmup_matches_sdpa(N, Bk):
    """k >= number of blocks: the gradients of dense causal GQA attention,
    here torch's SDPA backward in float64."""
    Hkv, G, D = 2, 2, 8
    q_idx, k_idx, q, kk, vv = _rand_case(9, N=N, Hkv=Hkv, G=G, D=D, Bk=Bk)
    do = np.random.default_rng(10).standard_normal(q.shape)
    bi = O.index_topk(q_idx, k_idx, Bk, -(-N // Bk) + 1)
    got = O.attention_backward(q, kk, vv, do, bi, Bk)
    qt = torch.tensor(q).permute(0, 2, 1, 3).requires_grad_()
    kt = torch.tensor(kk).permute(0, 2, 1, 3).requires_grad_()
    vt = torch.tensor(vv).permute(0, 2, 1, 3).requires_grad_()
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, enable_gqa=True)
    (out * torch.tensor(do).permute(0, 2, 1, 3)).sum().backward()
    for a, t in zip(got, (qt, kt, vt)):
        np.testing.assert_allclose(a, t.grad.permute(0, 2, 1, 3).numpy(), atol=1e-12, rtol=0)


def test_backward_invariants():
    """Per group: the dV of all keys sums to the sum of the group's dO rows
    (every row's probabilities sum to 1), and the dK of all keys sums to 0
    (every row's logit gradients sum to 0)."""
    N, Bk, k, Hkv, G, D = 80, 8, 4, 2, 3, 8
    q_idx, k_idx, q, kk, vv = _rand_case(11, N=N, Hkv=Hkv, G=G, D=D, Bk=Bk)
    do = np.random.default_rng(12).standard_normal(q.shape)
    bi = O.index_topk(q_idx, k_idx, Bk, k)
    _, dk, dv = O.attention_backward(q, kk, vv, do, bi, Bk)
    for g in range(Hkv):
        np.testing.assert_allclose(dv[0, :, g].sum(axis=0), do[0, :, g * G:(g + 1) * G].sum(axis=(0, 1)),
                                   atol=1e-10)
        np.testing.assert_allclose(dk[0, :, g].sum(axis=0), 0.0, atol=1e-10)


def test_backward_planted_mistakes_are_caught(monkeypatch):
    """A dropped softmax-Jacobian term, a transposed probability matrix or a
    missing scale in the row gradients each fails the autograd pin."""
    N, Bk, k, Hkv, G, D = 40, 8, 3, 1, 2, 8
    q_idx, k_idx, q, kk, vv = _rand_case(13, N=N, Hkv=Hkv, G=G, D=D, Bk=Bk)
    do = np.random.default_rng(14).standard_normal(q.shape)
    bi = O.index_topk(q_idx, k_idx, Bk, k)
    want = _masked_dense_grads(q, kk, vv, do, bi, Bk, 1 / math.sqrt(D))

    def ok():
        got = O.attention_backward(q, kk, vv, do, bi, Bk)
        return all(np.allclose(a, b, atol=1e-9) for a, b in zip(got, want))

    assert ok()
    real = O._row_backward

    def no_jacobian_term(qh, kt, vt, doh, scale):
        _, p = O._softmax_stats(scale * (qh @ kt.T))
        dz = p * (doh @ vt.T)
        return scale * (dz @ kt), scale * (dz.T @ qh), p.T @ doh

    def no_scale(qh, kt, vt, doh, scale):
        dq, dk, dv = real(qh, kt, vt, doh, scale)
        return dq / scale, dk / scale, dv

    def transposed_dv(qh, kt, vt, doh, scale):
        dq, dk, dv = real(qh, kt, vt, doh, scale)
        _, p = O._softmax_stats(scale * (qh @ kt.T))
        return dq, dk, (p.T[::-1] @ doh)

    for bad in (no_jacobian_term, no_scale, transposed_dv):
        monkeypatch.setattr(O, "_row_backward", bad)
        assert not ok(), bad.__name__
    monkeypatch.setattr(O, "_row_backward", real)


# -------------------------------------------------------------- KL backward --

def _kl_autograd(q, kk, q_idx, k_idx, bi, Bk, w, scale, iscale):
    """torch autograd (float64) of sum_rows w * KL over dense masked
    distributions, with the teacher detached."""
    B, N, Hq, D = q.shape
    Hkv = kk.shape[2]
    G = Hq // Hkv
    qi = torch.tensor(q_idx).requires_grad_()
    ki = torch.tensor(k_idx).requires_grad_()
    mask = torch.zeros(B, Hkv, N, N, dtype=torch.bool)
    for b in range(B):
        for g in range(Hkv):
            for i in range(N):
                mask[b, g, i, O.token_set(bi[b, g, i], i, Bk)] = True
    qt = torch.tensor(q).view(B, N, Hkv, G, D)
    kt = torch.tensor(kk)
    logits = scale * torch.einsum("bighd,btgd->bghit", qt, kt)
    logits = logits.masked_fill(~mask[:, :, None], float("-inf"))
    p = torch.softmax(logits, dim=-1).mean(dim=2).detach()          # [B, Hkv, N, N]
    u = iscale * torch.einsum("bigd,btd->bgit", qi, ki)
    log_s = torch.log_softmax(u.masked_fill(~mask, float("-inf")), dim=-1)
    terms = torch.where(mask & (p > 0), p * (torch.log(p) - log_s), torch.zeros((), dtype=torch.float64))
    loss = (torch.tensor(w) * terms.sum(dim=-1)).sum()
    loss.backward()
    return qi.grad.numpy(), ki.grad.numpy(), float(loss.detach())


@pytest.mark.parametrize("seed,N,Bk,k,G", [(0, 48, 8, 3, 2), (1, 45, 8, 4, 1), (2, 40, 4, 16, 4)])
def test_kl_backward_matches_autograd(seed, N, Bk, k, G):
    Hkv, D, Di = 2, 8, 4
    q_idx, k_idx, q, kk, vv = _rand_case(seed, N=N, Hkv=Hkv, G=G, D=D, Di=Di, Bk=Bk)
    q_idx, k_idx = q_idx / 2, k_idx / 2
    bi = O.index_topk(q_idx, k_idx, Bk, k)
    w = np.random.default_rng(seed + 50).uniform(0.5, 2.0, size=(1, Hkv, N))
    got = O.kl_backward(q, kk, q_idx, k_idx, bi, Bk, dkl_rows=w, scale=0.4, index_scale=0.3)
    gq, gk, loss = _kl_autograd(q, kk, q_idx, k_idx, bi, Bk, w, 0.4, 0.3)
    np.testing.assert_allclose(got[0], gq, atol=1e-12, rtol=0)
    np.testing.assert_allclose(got[1], gk, atol=1e-12, rtol=0)
    rows, _ = O.kl_align(q, kk, q_idx, k_idx, bi, Bk, scale=0.4, index_scale=0.3)
    assert abs(loss - float((w * rows).sum())) <= 1e-10 * max(1.0, abs(loss))


def test_kl_backward_finite_differences():
    """Directional derivative of kl_sum (the pinned forward) along (a, c) in
    (q_idx, k_idx) equals <dq_idx, a> + <dk_idx, c>; the selection is held
    fixed (it is an input of the loss)."""
    N, Bk, k, Hkv, G, D, Di = 40, 8, 3, 2, 2, 8, 4
    q_idx, k_idx, q, kk, vv = _rand_case(21, N=N, Hkv=Hkv, G=G, D=D, Di=Di, Bk=Bk)
    q_idx, k_idx = q_idx / 3, k_idx / 3
    bi = O.index_topk(q_idx, k_idx, Bk, k)
    rng = np.random.default_rng(22)
    a, c = rng.standard_normal(q_idx.shape), rng.standard_normal(k_idx.shape)
    dqi, dki = O.kl_backward(q, kk, q_idx, k_idx, bi, Bk)

    def f(t):
        return O.kl_align(q, kk, q_idx + t * a, k_idx + t * c, bi, Bk)[1]

    eps = 1e-5
    fd = (f(eps) - f(-eps)) / (2 * eps)
    an = float((dqi * a).sum() + (dki * c).sum())
    assert abs(fd - an) <= 1e-7 * max(1.0, abs(an))


def test_kl_backward_sum_rule_and_mistakes(monkeypatch):
    """The dk_idx of all keys sums to 0 (every row's logit gradients sum to 0);
    a sign flip, a missing index scale or a non-detached-teacher-shaped term
    fails the autograd pin."""
    N, Bk, k, Hkv, G, D, Di = 40, 8, 3, 2, 2, 8, 4
    q_idx, k_idx, q, kk, vv = _rand_case(23, N=N, Hkv=Hkv, G=G, D=D, Di=Di, Bk=Bk)
    q_idx, k_idx = q_idx / 2, k_idx / 2
    bi = O.index_topk(q_idx, k_idx, Bk, k)
    dqi, dki = O.kl_backward(q, kk, q_idx, k_idx, bi, Bk)
    np.testing.assert_allclose(dki.sum(axis=(0, 1)), 0.0, atol=1e-10)
    w = np.ones((1, Hkv, N))
    want = _kl_autograd(q, kk, q_idx, k_idx, bi, Bk, w, 1 / math.sqrt(D), 1 / math.sqrt(Di))[:2]

    def ok():
        got = O.kl_backward(q, kk, q_idx, k_idx, bi, Bk)
        return all(np.allclose(x, y, atol=1e-9) for x, y in zip(got, want))

    assert ok()
    real = O._kl_row_backward

    def flipped(qh, kt, qi, kit, scale, index_scale):
        a, c = real(qh, kt, qi, kit, scale, index_scale)
        return -a, -c

    def unscaled(qh, kt, qi, kit, scale, index_scale):
        a, c = real(qh, kt, qi, kit, scale, index_scale)
        return a / index_scale, c / index_scale

    def head0_teacher(qh, kt, qi, kit, scale, index_scale):   # first head instead of the group mean
        return real(qh[:1], kt, qi, kit, scale, index_scale)

    for bad in (flipped, unscaled, head0_teacher):
        monkeypatch.setattr(O, "_kl_row_backward", bad)
        assert not ok(), bad.__name__
    monkeypatch.setattr(O, "_kl_row_backward", real)


def test_kl_dq_idx_rows_is_the_full_backward_at_those_rows():
    N, Bk, k, Hkv, G, D, Di = 40, 8, 3, 2, 2, 8, 4
    q_idx, k_idx, q, kk, vv = _rand_case(24, N=N, Hkv=Hkv, G=G, D=D, Di=Di, Bk=Bk)
    bi = O.index_topk(q_idx, k_idx, Bk, k)
    w = np.random.default_rng(25).uniform(0.5, 2.0, size=(1, Hkv, N))
    full, _ = O.kl_backward(q, kk, q_idx, k_idx, bi, Bk, dkl_rows=w)
    pos = np.array([(0, i) for i in range(0, N, 3)])
    rows = bi.transpose(0, 2, 1, 3)[0, pos[:, 1]]
    got = O.kl_dq_idx_rows(q, kk, k_idx, rows, pos, Bk, w_rows=w[0][:, pos[:, 1]].T,
                           qi_rows=q_idx[0, pos[:, 1]])
    np.testing.assert_allclose(got, full[0, pos[:, 1]], atol=1e-14, rtol=0)


def test_dense_rows_are_causal_sdpa():
    """All visible blocks kept (the warm-up's full attention): the oracle's rows
    equal torch's causal GQA SDPA in float64, and the LSE the masked logsumexp."""
    rng = np.random.default_rng(11)
    B, N, Hkv, G, D, Bk = 2, 45, 2, 3, 8, 8
    q = rng.standard_normal((B, N, Hkv * G, D))
    k = rng.standard_normal((B, N, Hkv, D))
    v = rng.standard_normal((B, N, Hkv, D))
    pos = np.array([(b, i) for b in range(B) for i in range(N)])
    rows = O.dense_block_idx_rows(pos, Hkv, Bk)
    assert rows.shape == (B * N, Hkv, (N - 1) // Bk + 1)
    o, lse = O.attention_rows(q, k, v, rows, pos, Bk)
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    vt = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    want = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    z = (qt @ kt.transpose(-1, -2)) / math.sqrt(D)
    z = z.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), -math.inf)
    want_lse = torch.logsumexp(z, dim=-1)                                  # [B, Hq, N]
    np.testing.assert_allclose(o.reshape(B, N, Hkv * G, D), want.permute(0, 2, 1, 3).numpy(), atol=1e-12)
    np.testing.assert_allclose(lse.reshape(B, N, Hkv * G), want_lse.permute(0, 2, 1).numpy(), atol=1e-12)


def test_backward_row_ranges():
    """Keeping only the rows of a range in the backward is the gradient of the
    loss with dO zero on every other row (then those rows' dS and P^T dO
    vanish), checked against torch autograd; ranges covering [0, N) add up
    to the whole."""
    N, Bk, k, Hkv, G, D = 56, 8, 3, 2, 2, 8
    q_idx, k_idx, q, kk, vv = _rand_case(21, N=N, Hkv=Hkv, G=G, D=D, Bk=Bk)
    do = np.random.default_rng(22).standard_normal(q.shape)
    bi = O.index_topk(q_idx, k_idx, Bk, k)
    scale = 0.4
    parts = [O.attention_backward(q, kk, vv, do, bi, Bk, scale, row_range=r) for r in ((0, 19), (19, 40), (40, N))]
    masked = do.copy()
    masked[:, :19] = 0.0
    masked[:, 40:] = 0.0
    want = _masked_dense_grads(q, kk, vv, masked, bi, Bk, scale)
    for a, b in zip(parts[1], want):
        np.testing.assert_allclose(a, b, atol=1e-12, rtol=0)
    whole = O.attention_backward(q, kk, vv, do, bi, Bk, scale)
    for x in range(3):
        np.testing.assert_allclose(sum(p[x] for p in parts), whole[x], atol=1e-12, rtol=0)


def test_kl_backward_row_ranges():
    """The KL backward over a row range equals the whole backward with zero
    row weights elsewhere; ranges covering [0, N) add up to the whole."""
    N, Bk, k, Hkv, G, D = 56, 8, 3, 2, 2, 8
    q_idx, k_idx, q, kk, vv = _rand_case(23, N=N, Hkv=Hkv, G=G, D=D, Bk=Bk)
    bi = O.index_topk(q_idx, k_idx, Bk, k)
    w = np.random.default_rng(24).uniform(0.5, 1.5, size=(1, Hkv, N))
    a = O.kl_backward(q, kk, q_idx, k_idx, bi, Bk, dkl_rows=w, row_range=(10, 33))
    wm = np.zeros_like(w)
    wm[..., 10:33] = w[..., 10:33]
    b = O.kl_backward(q, kk, q_idx, k_idx, bi, Bk, dkl_rows=wm)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, atol=1e-13, rtol=0)
    rest = [O.kl_backward(q, kk, q_idx, k_idx, bi, Bk, dkl_rows=w, row_range=r) for r in ((0, 10), (33, N))]
    whole = O.kl_backward(q, kk, q_idx, k_idx, bi, Bk, dkl_rows=w)
    for x in range(2):
        np.testing.assert_allclose(a[x] + rest[0][x] + rest[1][x], whole[x], atol=1e-12, rtol=0)
