"""Plain CPU oracle of the MSA (MiniMax Sparse Attention) forward path, of the
backward over the cached block indices, and of decoding (one new query per
sequence against a cache).

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module. The product path (the HIP
library and its binding) never calls it and has no CPU fallback.

Everything here is the definition written out, in float64, one query row at a
time, with numpy matmuls as the only library step. It shares no code with the
HIP path.

Sources (web pages; cited by title and section):
  [P1] "Flash-MSA" kernel article on tech.kuratif.com (Indonesian), paragraphs
       on block-wise sparsity and on the proxy/main forward.
  [P2] "MiniMax Sparse Attention (MSA): una atención dispersa en bloques de dos
       ramas ..." on 7minutos.es, sections "¿Qué es MSA?", "Cómo funcionan las
       dos ramas", "Cómo se entrena MSA", "El codiseño del kernel".
  [P3] "Accelerating Million-Token Training with Sparse Attention Kernels"
       (DeepHorus blog).

Notation: B batch, N tokens (queries = keys), Hkv groups (= KV heads = index
query heads), G query heads per group, Hq = Hkv*G, D head dim, Di index dim,
Bk block size, k blocks kept per (query, group). For query position i the local
block is L = i // Bk; blocks j < L are fully visible and compete; the local
block is always kept.

Readings of points the pages leave open (each listed in the design notes):
  * index score = raw dot product q_idx . k_idx (no scale; a positive scale
    cannot change the selection);
  * ties in the block ranking go to the lower block id;
  * the kept ids are emitted in ascending order, padded with -1 to length k;
  * with fewer than k-1 competing blocks, all of them are kept;
  * token t is visible to query i iff t <= i;
  * query head h belongs to group h // G;
  * LSE is the natural-log log-sum-exp of the scaled logits;
  * KL is KL(teacher || student) summed over the row's selected tokens, with
    the teacher the group-mean of the G heads' main-branch probabilities and the
    student the softmax of index_scale * index score over the same tokens.
  * the backward differentiates the main-branch forward above for the loss
    <dO, O> (dO given); every key's gradient sums the contributions of all rows
    that selected its block;
  * the KL term's backward holds the teacher fixed (gradient stopped at the
    index branch input) and reaches q_idx and k_idx only;
  * decoding appends R >= 1 tokens per sequence: sequence b holds n_b cached
    tokens (positions 0 .. n_b - 1, the new ones last) and its r-th new query
    is the query of position n_b - R + r, so its selection and attention are
    exactly the forward's row there; cache slots at or past n_b are never
    read; a length outside [1, capacity] (or a negative position) gives an
    all -1 selection, O = 0 and LSE = -inf.

Parity: every function here is pinned by tests that do not re-use its code
(brute force, closed forms, torch's dense SDPA, scipy's entropy, invariants).
"""
import math

import numpy as np

__all__ = [
    "local_block", "visible_block_scores", "select_blocks", "index_topk_rows",
    "index_topk", "token_set", "token_count", "attention_rows", "sparse_attention",
    "kl_rows", "kl_align", "attention_backward", "attention_dq_rows", "kl_backward", "kl_dq_idx_rows",
    "map_positions", "decode_index_topk", "decode_attention", "dense_block_idx_rows", "fp4_e2m1_values",
]


def fp4_e2m1_values(packed):
    """Values of OCP MX fp4 e2m1 data stored two to a byte (element 2c in bits
    0-3 of byte c, element 2c+1 in bits 4-7), as float32 with the last axis
    doubled. Per the format: bit 3 is the sign, bits 2-1 the exponent E (bias
    1), bit 0 the mantissa M; E = 0 encodes the subnormals 0 and 0.5 (M / 2),
    E > 0 the normals 2^(E-1) (1 + M/2). [P2] "El codiseño del kernel": the
    open kernel runs in FP4 among other precisions."""
    b = np.asarray(packed, dtype=np.uint8)
    codes = np.stack([b & 0xF, b >> 4], axis=-1).reshape(b.shape[:-1] + (2 * b.shape[-1],))
    e = ((codes >> 1) & 3).astype(np.float64)
    m = (codes & 1).astype(np.float64)
    mag = np.where(e == 0, 0.5 * m, 2.0 ** (e - 1) * (1.0 + 0.5 * m))
    return np.where(codes & 8, -mag, mag).astype(np.float32)


def _arr(x):
    """Tensor or array -> numpy array without a copy where possible (bf16, fp16
    and fp8 tensors widen exactly to float32, packed fp4 tensors are decoded
    exactly to float32; everything is cast to float64 where it is used)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu")
            if x.dtype == getattr(torch, "float4_e2m1fn_x2", None):
                return fp4_e2m1_values(x.view(torch.uint8).numpy())
            if x.dtype.is_floating_point and x.element_size() < 4:
                x = x.float()   # bf16, fp16 and fp8 widen exactly to float32
            return x.numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x)


def local_block(i, Bk):
    """The block holding query i; [P2] "Cómo funcionan las dos ramas": the block
    that contains the query is always included."""
    return i // Bk


def visible_block_scores(q_idx_row, k_idx_b, i, Bk):
    """Max-pooled index scores of the competing blocks of query i.

    [P2] "Cómo funcionan las dos ramas": the index branch scores the visible key
    tokens with one index-query head per group against one shared index-key head,
    then max-pools the scores to the block level; [P1] paragraph on block-wise
    sparsity: blocks of 128 chosen by max-pooling the proxy scores.

    Only blocks j < L = i // Bk compete (fully visible, the local block is forced
    in). Returns a float64 array of length L with m_j = max_{t in block j}
    <q_idx_row, k_idx_b[t]>.
    """
    L = local_block(i, Bk)
    if L == 0:
        return np.zeros(0, dtype=np.float64)
    keys = np.asarray(_arr(k_idx_b)[: L * Bk], dtype=np.float64)   # [L*Bk, Di]
    s = keys @ np.asarray(_arr(q_idx_row), dtype=np.float64)       # one per token
    return s.reshape(L, Bk).max(axis=1)


def select_blocks(m, L, k):
    """Forced-local, exp-free top-k of one (query, group) row.

    [P2] "El codiseño del kernel": softmax keeps the order of the scores, so the
    ranking runs on the raw max-pooled scores; [P2] "Cómo funcionan las dos ramas":
    top-k per query and group, the local block always present; [P1] paragraph on
    the proxy forward: local scores are set to +inf so the window stays open.

    Ranking key: score descending, then block id ascending (lower id wins ties).
    Returns the kept ids as an ascending int list of length min(k, L + 1); the
    last entry is always L.
    """
    m = np.asarray(m, dtype=np.float64)
    assert m.shape == (L,)
    ids = np.arange(L)
    order = np.lexsort((ids, -m))               # primary: -m, secondary: id
    kept = [int(j) for j in order[: min(k - 1, L)]] + [L]
    return sorted(kept)


def _pad(ids, k):
    return list(ids) + [-1] * (k - len(ids))


def index_topk_rows(q_idx, k_idx, positions, Bk, k, key_chunk=16384, q_rows=None):
    """Block indices at the given (b, i) positions.

    q_idx [B, N, Hkv, Di], k_idx [B, N, Di]; positions int [M, 2]. Instead of
    q_idx, ``q_rows`` [M, Hkv, Di] may give just the rows at the positions.
    Returns int32 [M, Hkv, k] (ascending ids, -1 padded).

    Same definition as ``visible_block_scores`` + ``select_blocks`` per row; the
    scores of all requested rows of a batch entry are obtained from one matrix
    product per key chunk (a chunk holds whole blocks), then max-pooled per block.
    """
    ka = _arr(k_idx)
    positions = np.asarray(positions, dtype=np.int64).reshape(-1, 2)
    if q_rows is None:
        qa = _arr(q_idx)
        q_rows = qa[positions[:, 0], positions[:, 1]]
    q_rows = _arr(q_rows)
    Hkv, Di = q_rows.shape[1], q_rows.shape[2]
    out = np.full((len(positions), Hkv, k), -1, dtype=np.int32)
    key_chunk = max(Bk, key_chunk // Bk * Bk)
    for b in np.unique(positions[:, 0]):
        sel = np.nonzero(positions[:, 0] == b)[0]
        pos_i = positions[sel, 1]
        Lmax = int(pos_i.max()) // Bk
        qrows = np.asarray(q_rows[sel], dtype=np.float64).reshape(-1, Di)           # [P*Hkv, Di]
        m = np.empty((Lmax, qrows.shape[0]))
        for t0 in range(0, Lmax * Bk, key_chunk):
            t1 = min(Lmax * Bk, t0 + key_chunk)
            s = np.asarray(ka[b, t0:t1], dtype=np.float64) @ qrows.T       # [tokens, P*Hkv]
            m[t0 // Bk:t1 // Bk] = s.reshape((t1 - t0) // Bk, Bk, -1).max(axis=1)
        for p, (r, i) in enumerate(zip(sel, pos_i)):
            L = local_block(int(i), Bk)
            for g in range(Hkv):
                out[r, g] = _pad(select_blocks(m[:L, p * Hkv + g], L, k), k)
    return out


def index_topk(q_idx, k_idx, Bk, k):
    """Block indices for every position: int32 [B, Hkv, N, k]."""
    q_idx = _arr(q_idx)
    B, N, Hkv, _ = q_idx.shape
    pos = np.array([(b, i) for b in range(B) for i in range(N)], dtype=np.int64).reshape(-1, 2)
    rows = index_topk_rows(q_idx, k_idx, pos, Bk, k)     # [B*N, Hkv, k]
    return rows.reshape(B, N, Hkv, k).transpose(0, 2, 1, 3).copy()


def token_set(ids, i, Bk):
    """Causally visible tokens of the kept blocks of query i.

    [P2] "Cómo funcionan las dos ramas": the main branch gathers the causally
    visible tokens of the selected blocks. Block j contributes tokens
    j*Bk .. min((j+1)*Bk - 1, i). ``ids`` may contain -1 padding.
    """
    parts = []
    for j in ids:
        j = int(j)
        if j < 0:
            continue
        lo = j * Bk
        hi = min((j + 1) * Bk - 1, i)
        if hi >= lo:
            parts.append(np.arange(lo, hi + 1, dtype=np.int64))
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


def token_count(i, Bk, k):
    """Closed form of |T_i| for a well-formed selection: (min(k, L+1) - 1) full
    blocks plus the i mod Bk + 1 causal tokens of the local block ([P2] "¿Qué es
    MSA?": budget k*Bk tokens per query)."""
    L = i // Bk
    return (min(k, L + 1) - 1) * Bk + (i % Bk) + 1


def _softmax_stats(z):
    """Natural-log LSE and normalised probabilities of each row of z."""
    mx = z.max(axis=-1, keepdims=True)
    e = np.exp(z - mx)
    s = e.sum(axis=-1, keepdims=True)
    lse = (mx + np.log(s))[..., 0]
    return lse, e / s


def attention_rows(q, k, v, block_idx_rows, positions, Bk, scale=None, q_rows=None):
    """Main-branch output at the given (b, i) positions.

    [P2] "Cómo funcionan las dos ramas": exact scaled-dot-product softmax over
    the gathered tokens; each query head uses its own query and the block set of
    its group. [P1] paragraph on the forward: the output goes on and the LSE is
    kept for the backward.

    q [B,N,Hq,D] (or ``q_rows`` [M, Hq, D], the rows at the positions), k/v
    [B,N,Hkv,D], block_idx_rows int [M, Hkv, k] for the M positions. Returns (O [M, Hq, D], LSE [M, Hq]) in float64, where
    z_t = scale * <q, k_t>, LSE = ln sum_t exp z_t, O = sum_t exp(z_t - LSE) v_t.
    """
    kk = _arr(k)
    vv = _arr(v)
    positions = np.asarray(positions, dtype=np.int64).reshape(-1, 2)
    if q_rows is None:
        q_rows = _arr(q)[positions[:, 0], positions[:, 1]]
    q_rows = _arr(q_rows)
    Hq, D = q_rows.shape[1], q_rows.shape[2]
    Hkv = kk.shape[2]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(D) if scale is None or scale <= 0 else float(scale)
    M = len(positions)
    O = np.zeros((M, Hq, D))
    LSE = np.zeros((M, Hq))
    for b in np.unique(positions[:, 0]):
        rows = np.nonzero(positions[:, 0] == b)[0]
        for g in range(Hkv):
            kg = np.ascontiguousarray(kk[b, :, g], dtype=np.float64)        # [N, D]
            vg = np.ascontiguousarray(vv[b, :, g], dtype=np.float64)
            for r in rows:
                i = int(positions[r, 1])
                T = token_set(block_idx_rows[r, g], i, Bk)
                qh = np.asarray(q_rows[r, g * G:(g + 1) * G], dtype=np.float64)  # [G, D]
                z = scale * (qh @ kg[T].T)                                       # [G, |T|]
                lse, p = _softmax_stats(z)
                LSE[r, g * G:(g + 1) * G] = lse
                O[r, g * G:(g + 1) * G] = p @ vg[T]
    return O, LSE


def sparse_attention(q, k, v, block_idx, Bk, scale=None):
    """Full main-branch forward: O [B,N,Hq,D] and LSE [B,Hq,N] in float64."""
    q = _arr(q)
    B, N, Hq, D = q.shape
    pos = np.array([(b, i) for b in range(B) for i in range(N)], dtype=np.int64).reshape(-1, 2)
    bi = np.asarray(block_idx)
    rows = bi.transpose(0, 2, 1, 3).reshape(B * N, bi.shape[1], bi.shape[3])
    O, LSE = attention_rows(q, k, v, rows, pos, Bk, scale)
    return O.reshape(B, N, Hq, D), LSE.reshape(B, N, Hq).transpose(0, 2, 1).copy()


def _row_backward(qh, kt, vt, doh, scale):
    """Gradients of L = sum_h <dO_h, O_h> for one (position, group) row set.

    qh/doh [G, D] (the group's query heads and their output gradients), kt/vt
    [|T|, D] (keys and values of the row's selected tokens). Chain rule through
    O_h = sum_t P_ht v_t, P_h = softmax_t(z_h), z_ht = scale <q_h, k_t>:
      dV_t = sum_h P_ht dO_h,  dP_ht = <dO_h, v_t>,
      dz_ht = P_ht (dP_ht - sum_u P_hu dP_hu)   (softmax Jacobian),
      dQ_h = scale sum_t dz_ht k_t,  dK_t = scale sum_h dz_ht q_h.
    Returns (dQ [G, D], dK [|T|, D], dV [|T|, D])."""
    z = scale * (qh @ kt.T)                      # [G, |T|]
    _, p = _softmax_stats(z)
    dv = p.T @ doh
    dp = doh @ vt.T
    dz = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    return scale * (dz @ kt), scale * (dz.T @ qh), dv


def attention_backward(q, k, v, do, block_idx, Bk, scale=None, row_range=None):
    """Gradients of the main branch for every position: (dQ [B,N,Hq,D],
    dK [B,N,Hkv,D], dV [B,N,Hkv,D]) in float64, for the loss <dO, O>.

    [P1] paragraph on the backward: with the block indices cached by the
    forward, the backward runs over the same sparse blocks (linear in N). The
    function differentiated is the forward of ``attention_rows``; a key's
    gradient sums the contributions of every row that selected its block.
    ``row_range`` = (i0, i1) keeps only the rows i0 <= i < i1 in that sum (and
    in dQ): the results of disjoint ranges covering [0, N) add up to the whole.
    """
    qq, kk, vv, dd = _arr(q), _arr(k), _arr(v), _arr(do)
    B, N, Hq, D = qq.shape
    Hkv = kk.shape[2]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(D) if scale is None or scale <= 0 else float(scale)
    bi = np.asarray(block_idx)
    dQ = np.zeros((B, N, Hq, D))
    dK = np.zeros((B, N, Hkv, D))
    dV = np.zeros((B, N, Hkv, D))
    for b in range(B):
        for g in range(Hkv):
            hs = slice(g * G, (g + 1) * G)
            kg = np.asarray(kk[b, :, g], dtype=np.float64)
            vg = np.asarray(vv[b, :, g], dtype=np.float64)
            qg = np.asarray(qq[b, :, hs], dtype=np.float64)
            dg = np.asarray(dd[b, :, hs], dtype=np.float64)
            dKg = np.zeros((N, D))
            dVg = np.zeros((N, D))
            for i in range(*(row_range or (0, N))):
                T = token_set(bi[b, g, i], i, Bk)
                dq, dk, dv = _row_backward(qg[i], kg[T], vg[T], dg[i], scale)
                dQ[b, i, hs] = dq
                dKg[T] += dk          # T holds distinct tokens
                dVg[T] += dv
            dK[b, :, g] = dKg
            dV[b, :, g] = dVg
    return dQ, dK, dV


def attention_dq_rows(q, k, v, do, block_idx_rows, positions, Bk, scale=None, q_rows=None, do_rows=None):
    """dQ at the given (b, i) positions only ([M, Hq, D], float64): a row's dQ
    depends on its own selection alone, so large workloads are checked on
    sampled rows. Arguments as in ``attention_rows``; ``do_rows`` [M, Hq, D]
    may replace do by its rows at the positions."""
    kk, vv = _arr(k), _arr(v)
    positions = np.asarray(positions, dtype=np.int64).reshape(-1, 2)
    if q_rows is None:
        q_rows = _arr(q)[positions[:, 0], positions[:, 1]]
    if do_rows is None:
        do_rows = _arr(do)[positions[:, 0], positions[:, 1]]
    q_rows, do_rows = _arr(q_rows), _arr(do_rows)
    Hq, D = q_rows.shape[1], q_rows.shape[2]
    Hkv = kk.shape[2]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(D) if scale is None or scale <= 0 else float(scale)
    out = np.zeros((len(positions), Hq, D))
    for r, (b, i) in enumerate(positions):
        for g in range(Hkv):
            T = token_set(block_idx_rows[r, g], int(i), Bk)
            hs = slice(g * G, (g + 1) * G)
            out[r, hs] = _row_backward(np.asarray(q_rows[r, hs], dtype=np.float64),
                                       np.asarray(kk[b, T, g], dtype=np.float64),
                                       np.asarray(vv[b, T, g], dtype=np.float64),
                                       np.asarray(do_rows[r, hs], dtype=np.float64), scale)[0]
    return out


def kl_rows(q, k, q_idx, k_idx, block_idx_rows, positions, Bk, scale=None,
            index_scale=None, q_rows=None, qi_rows=None):
    """KL-alignment loss per (position, group) at the given positions.

    [P2] "Cómo se entrena MSA": a KL alignment loss matches the index branch's
    distribution to the main branch's attention pattern; the teacher is the main
    distribution averaged over the group, over the selected tokens. [P1]
    paragraph on the backward: computed without materialising the full
    distributions.

    Teacher p_t = mean_h softmax_t(scale <q_h, k_t>); student
    s_t = softmax_t(index_scale <q_idx, k_idx_t>); both over the row's selected
    tokens T_i. Returns float64 [M, Hkv] with sum_t p_t (ln p_t - ln s_t)
    (terms with p_t = 0 contribute 0). ``q_rows`` [M, Hq, D] / ``qi_rows``
    [M, Hkv, Di] may replace q / q_idx by their rows at the positions.
    """
    kk = _arr(k)
    ki = _arr(k_idx)
    positions = np.asarray(positions, dtype=np.int64).reshape(-1, 2)
    if q_rows is None:
        q_rows = _arr(q)[positions[:, 0], positions[:, 1]]
    if qi_rows is None:
        qi_rows = _arr(q_idx)[positions[:, 0], positions[:, 1]]
    q_rows, qi_rows = _arr(q_rows), _arr(qi_rows)
    Hq, D = q_rows.shape[1], q_rows.shape[2]
    Hkv, Di = kk.shape[2], qi_rows.shape[2]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(D) if scale is None or scale <= 0 else float(scale)
    index_scale = (1.0 / math.sqrt(Di) if index_scale is None or index_scale <= 0
                   else float(index_scale))
    out = np.zeros((len(positions), Hkv))
    for r, (b, i) in enumerate(positions):
        for g in range(Hkv):
            T = token_set(block_idx_rows[r, g], int(i), Bk)
            qh = np.asarray(q_rows[r, g * G:(g + 1) * G], dtype=np.float64)
            kt = np.asarray(kk[b, T, g], dtype=np.float64)
            z = scale * (qh @ kt.T)
            _, ph = _softmax_stats(z)
            p = ph.mean(axis=0)
            u = index_scale * (np.asarray(ki[b, T], dtype=np.float64)
                               @ np.asarray(qi_rows[r, g], dtype=np.float64))
            lse_u, _ = _softmax_stats(u[None, :])
            log_s = u - lse_u[0]
            nz = p > 0
            out[r, g] = float(np.sum(p[nz] * (np.log(p[nz]) - log_s[nz])))
    return out


def kl_align(q, k, q_idx, k_idx, block_idx, Bk, scale=None, index_scale=None):
    """Full KL forward: (kl_rows [B, Hkv, N], kl_sum) in float64; kl_sum is the
    plain sum over all rows."""
    q = _arr(q)
    B, N = q.shape[:2]
    pos = np.array([(b, i) for b in range(B) for i in range(N)], dtype=np.int64).reshape(-1, 2)
    bi = np.asarray(block_idx)
    rows = bi.transpose(0, 2, 1, 3).reshape(B * N, bi.shape[1], bi.shape[3])
    kl = kl_rows(q, k, q_idx, k_idx, rows, pos, Bk, scale, index_scale)
    kl = kl.reshape(B, N, -1).transpose(0, 2, 1).copy()
    return kl, float(kl.sum())


def _kl_row_backward(qh, kt, qi, kit, scale, index_scale):
    """Gradient of one row's KL term w.r.t. its student logits' inputs.

    qh [G, D] (the group's query heads), kt [|T|, D] (keys of the selected
    tokens), qi [Di] (the row's index query), kit [|T|, Di] (index keys).
    Teacher p = mean_h softmax_t(scale <q_h, k_t>) is held fixed (no gradient
    flows into the main branch); student s = softmax_t(index_scale <qi, kit_t>).
    KL = sum_t p_t (ln p_t - ln s_t) with ln s_t = index_scale u_t - LSE_u has
    dKL/du_t = index_scale (s_t sum_v p_v - p_t) = index_scale (s_t - p_t) for
    u_t = <qi, kit_t>, since the teacher sums to 1 over the same tokens.
    Returns (dKL/dqi [Di], dKL/dkit [|T|, Di])."""
    _, ph = _softmax_stats(scale * (qh @ kt.T))
    p = ph.mean(axis=0)
    _, sv = _softmax_stats(index_scale * (kit @ qi)[None, :])
    du = index_scale * (sv[0] - p)
    return du @ kit, np.outer(du, qi)


def kl_backward(q, k, q_idx, k_idx, block_idx, Bk, dkl_rows=None, scale=None, index_scale=None, row_range=None):
    """Gradients of L = sum over rows of dkl_rows[b, g, i] * KL_row (dkl_rows = 1
    everywhere: L = kl_sum) w.r.t. q_idx and k_idx: (dq_idx [B,N,Hkv,Di],
    dk_idx [B,N,Di]) in float64.

    [P2] "Cómo se entrena MSA": the KL alignment loss trains the index branch
    toward the main branch's attention pattern, and the gradient is stopped at
    the index branch's input, so the loss reaches the index projections only:
    the teacher (main-branch probabilities) is a constant here. [P1] paragraph
    on the backward: the proxy gradient comes from the cached block indices.
    k_idx is shared by the groups, so its gradient sums over every group's rows.
    ``row_range`` = (i0, i1) keeps only the rows i0 <= i < i1, as in
    ``attention_backward``.
    """
    qq, kk, qi, ki = _arr(q), _arr(k), _arr(q_idx), _arr(k_idx)
    B, N, Hq, D = qq.shape
    Hkv, Di = kk.shape[2], ki.shape[2]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(D) if scale is None or scale <= 0 else float(scale)
    index_scale = (1.0 / math.sqrt(Di) if index_scale is None or index_scale <= 0
                   else float(index_scale))
    bi = np.asarray(block_idx)
    w = np.ones((B, Hkv, N)) if dkl_rows is None else np.asarray(_arr(dkl_rows), dtype=np.float64)
    dqi = np.zeros((B, N, Hkv, Di))
    dki = np.zeros((B, N, Di))
    for b in range(B):
        kib = np.asarray(ki[b], dtype=np.float64)
        for g in range(Hkv):
            kg = np.asarray(kk[b, :, g], dtype=np.float64)
            qg = np.asarray(qq[b, :, g * G:(g + 1) * G], dtype=np.float64)
            qig = np.asarray(qi[b, :, g], dtype=np.float64)
            for i in range(*(row_range or (0, N))):
                T = token_set(bi[b, g, i], i, Bk)
                a, c = _kl_row_backward(qg[i], kg[T], qig[i], kib[T], scale, index_scale)
                dqi[b, i, g] = w[b, g, i] * a
                dki[b, T] += w[b, g, i] * c
    return dqi, dki


def kl_dq_idx_rows(q, k, k_idx, block_idx_rows, positions, Bk, w_rows=None, scale=None, index_scale=None,
                   q_rows=None, qi_rows=None):
    """dq_idx at the given (b, i) positions only ([M, Hkv, Di], float64): a
    row's dq_idx depends on its own selection alone. ``w_rows`` [M, Hkv] are the
    rows' loss weights (1 if None); ``q_rows`` [M, Hq, D] and ``qi_rows``
    [M, Hkv, Di] are the query and index-query rows at the positions."""
    kk, ki = _arr(k), _arr(k_idx)
    positions = np.asarray(positions, dtype=np.int64).reshape(-1, 2)
    if q_rows is None:
        q_rows = _arr(q)[positions[:, 0], positions[:, 1]]
    q_rows, qi_rows = _arr(q_rows), _arr(qi_rows)
    Hq, D = q_rows.shape[1], q_rows.shape[2]
    Hkv, Di = kk.shape[2], ki.shape[2]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(D) if scale is None or scale <= 0 else float(scale)
    index_scale = (1.0 / math.sqrt(Di) if index_scale is None or index_scale <= 0
                   else float(index_scale))
    out = np.zeros((len(positions), Hkv, Di))
    for r, (b, i) in enumerate(positions):
        for g in range(Hkv):
            T = token_set(block_idx_rows[r, g], int(i), Bk)
            a, _ = _kl_row_backward(np.asarray(q_rows[r, g * G:(g + 1) * G], dtype=np.float64),
                                    np.asarray(kk[b, T, g], dtype=np.float64),
                                    np.asarray(qi_rows[r, g], dtype=np.float64),
                                    np.asarray(ki[b, T], dtype=np.float64), scale, index_scale)
            out[r, g] = (1.0 if w_rows is None else float(w_rows[r, g])) * a
    return out


def dense_block_idx_rows(positions, Hkv, Bk):
    """Every causally visible block of each position, for the warm-up's full
    attention ([P2] "Cómo se entrena MSA": during the first iterations both
    branches attend to everything): int32 [M, Hkv, nb] with ids 0..L ascending,
    -1 padded, nb = the most blocks any of the positions sees. Passed to
    ``attention_rows`` this is dense causal attention."""
    positions = np.asarray(positions, dtype=np.int64).reshape(-1, 2)
    nb = int(positions[:, 1].max()) // Bk + 1 if len(positions) else 1
    out = np.full((len(positions), Hkv, nb), -1, dtype=np.int32)
    for r, (_, i) in enumerate(positions):
        out[r, :, : i // Bk + 1] = np.arange(i // Bk + 1, dtype=np.int32)
    return out


def _decode_positions(seqlens, capacity, R=1):
    """Query positions of a decode step: R new tokens per sequence, the r-th at
    position n_b - R + r. Returns (positions [M, 2] as (b, i), the (b, r) of
    each) for the rows that exist: n_b in [1, capacity] and i >= 0."""
    n = np.asarray(seqlens, dtype=np.int64).reshape(-1)
    rows = [(b, r, int(n[b]) - R + r) for b in range(len(n)) for r in range(R)
            if 1 <= n[b] <= capacity and int(n[b]) - R + r >= 0]
    pos = np.array([(b, i) for b, _, i in rows], dtype=np.int64).reshape(-1, 2)
    br = np.array([(b, r) for b, r, _ in rows], dtype=np.int64).reshape(-1, 2)
    return pos, br


def decode_index_topk(q_idx, k_idx, seqlens, Bk, k):
    """Block selection of the new queries of each sequence against a cache.

    [P2] "Cómo funcionan las dos ramas" and "El codiseño del kernel" (the same
    selection as the forward; only the query rows differ); [P3] (the block
    indices are all a sparse layer caches). k_idx [B, C, Di] is the index-key
    cache, seqlens [B] the cached lengths n_b (new tokens included). q_idx is
    [B, Hkv, Di] (one new token, position n_b - 1; returns int32 [B, Hkv, k])
    or [B, R, Hkv, Di] (R new tokens, the r-th at position n_b - R + r; returns
    [B, Hkv, R, k]). Rows of sequences with n_b outside [1, C], and rows at a
    negative position, are -1.
    """
    qi = _arr(q_idx)
    ka = _arr(k_idx)
    single = qi.ndim == 3
    if single:
        qi = qi[:, None]
    B, R, Hkv = qi.shape[0], qi.shape[1], qi.shape[2]
    out = np.full((B, Hkv, R, k), -1, dtype=np.int32)
    pos, br = _decode_positions(seqlens, ka.shape[1], R)
    if len(pos):
        rows = index_topk_rows(None, ka, pos, Bk, k, q_rows=qi[br[:, 0], br[:, 1]])   # [M, Hkv, k]
        out[br[:, 0], :, br[:, 1]] = rows
    return out[:, :, 0] if single else out


def decode_attention(q, k, v, seqlens, block_idx, Bk, scale=None):
    """Main-branch attention of the new queries of each sequence over their
    selected blocks of the cache ([P2] "Cómo funcionan las dos ramas", as for
    ``attention_rows`` at the queries' positions).

    k/v [B, C, Hkv, D] the caches, seqlens [B]. q [B, Hq, D] with block_idx
    [B, Hkv, k] (one new token) returns (O [B, Hq, D], LSE [B, Hq]); q
    [B, R, Hq, D] with block_idx [B, Hkv, R, k] returns (O [B, R, Hq, D], LSE
    [B, Hq, R]), float64. Rows that do not exist (see ``decode_index_topk``)
    get O = 0 and LSE = -inf.
    """
    qa = _arr(q)
    kk = _arr(k)
    bi = np.asarray(block_idx)
    single = qa.ndim == 3
    if single:
        qa, bi = qa[:, None], bi[:, :, None]
    B, R, Hq, D = qa.shape
    O = np.zeros((B, R, Hq, D))
    LSE = np.full((B, Hq, R), -np.inf)
    pos, br = _decode_positions(seqlens, kk.shape[1], R)
    if len(pos):
        o, lse = attention_rows(None, kk, v, bi[br[:, 0], :, br[:, 1]], pos, Bk, scale, q_rows=qa[br[:, 0], br[:, 1]])
        O[br[:, 0], br[:, 1]] = o
        LSE[br[:, 0], :, br[:, 1]] = lse
    return (O[:, 0], LSE[:, :, 0]) if single else (O, LSE)


def map_positions(fn, positions, row_arrays=(), workers=1, chunk=256):
    """Run a row-wise oracle function over position chunks in worker processes.

    ``fn(positions_chunk, *row_array_chunks)`` must return an array (or tuple of
    arrays) whose first axis follows the chunk's rows; ``row_arrays`` are split
    along their first axis like ``positions``. Rows are independent, so the
    result equals one call over all positions; this only spreads the rows over
    ``workers`` forked processes (the children run numpy only).
    """
    positions = np.asarray(positions, dtype=np.int64).reshape(-1, 2)
    spans = [(s, min(len(positions), s + chunk)) for s in range(0, len(positions), chunk)]
    jobs = [(positions[s:e],) + tuple(a[s:e] for a in row_arrays) for s, e in spans]
    if workers <= 1 or len(jobs) <= 1:
        parts = [fn(*j) for j in jobs]
    else:
        import multiprocessing as mp
        global _MAP_FN
        _MAP_FN = fn
        try:
            with mp.get_context("fork").Pool(workers, initializer=_single_thread_blas) as pool:
                parts = pool.map(_map_worker, jobs)
        finally:
            _MAP_FN = None
    if not parts:
        return None
    if isinstance(parts[0], tuple):
        return tuple(np.concatenate([p[t] for p in parts]) for t in range(len(parts[0])))
    return np.concatenate(parts)


_MAP_FN = None


def _single_thread_blas():
    """Workers each run one BLAS thread (the parallelism is across rows)."""
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:  # pragma: no cover
        pass


def _map_worker(job):
    return _MAP_FN(*job)
