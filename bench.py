"""Benchmark of the MSA forward hot path on one MI355X.

One step = the whole hot path on one batch of synthetic input already resident
in HBM: the selection (index scores, block max-pool, forced-local exp-free
top-k: msa_index_topk) and the block-sparse GQA attention with LSE (the three
stages of msa_sparse_attn_fwd_stages), back to back on one stream. HIP events
between the four calls time every kernel stage inside the timed steps.
Default workload: N = 128K tokens, Hkv = 8, G = 8, D = Di = 128, Bk = 128,
k = 16, bf16, with long-range stripes.

Prints one JSON line: tokens/s (value), TFLOP/s and the fraction of the bf16
MFMA peak for the step, a roofline entry for the dominant (longest) kernel and
for the other two main kernels, and the CPU oracle timed on a bounded sample of
the same workload.

    python bench.py [--steps K] [--warmup W] [--workload n128k] [--no-cpu-baseline]

With --decode the line is for one decode step instead (msa_decode_index_topk
then msa_decode_attn: one new token for each of 64 sequences with 128K-token
caches, lengths uniform on [1, 128K]); value = sequences (new tokens) per
second, roofline = HBM bytes the step must move per second.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import block_sparse_gqa_index_amd as msa  # noqa: E402
from synth import (CONFIGS, DECODE_CONFIGS, make_decode_inputs, make_grad_output, make_inputs,  # noqa: E402
                   make_row_weights, sample_rows, to_fp4_e2m1)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 (vector and MFMA)
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
PEAK_FP4_TFLOPS = 10100.0      # MI355X dense fp4 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
CSRC = os.path.join(ROOT, "block_sparse_gqa_index_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_n128k.json")
DECODE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_decode_n128k_b64.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def flops(w):
    """Algorithmic work: competing blocks only for the index GEMM; causally
    visible tokens of the kept blocks for the attention (QK^T and PV)."""
    B, N, Hkv, G, D, Di, Bk, k = (w.batch, w.seqlen, w.kv_heads, w.group_size, w.head_dim,
                                  w.index_dim, w.block_size, w.topk)
    nb_full = N // Bk
    f_idx = 2.0 * Di * B * Hkv * Bk * Bk * nb_full * (nb_full - 1) / 2
    i = np.arange(N, dtype=np.int64)
    L = i // Bk
    tokens = (np.minimum(k, L + 1) - 1) * Bk + (i % Bk) + 1
    f_main = 4.0 * D * B * Hkv * G * float(tokens.sum())
    return f_idx, f_main


def flops_split(w):
    """F_main split by kernel: the non-local kept blocks (every row's
    min(k, L+1) - 1 full blocks) and the local block ((i mod Bk) + 1 tokens)."""
    B, N, Hkv, G, D, Bk, k = w.batch, w.seqlen, w.kv_heads, w.group_size, w.head_dim, w.block_size, w.topk
    i = np.arange(N, dtype=np.int64)
    L = i // Bk
    per = 4.0 * D * B * Hkv * G
    return per * float(((np.minimum(k, L + 1) - 1) * Bk).sum()), per * float((i % Bk + 1).sum())


def compulsory_attention_bytes(w):
    """S4's compulsory HBM bytes: Q, K, V, block_idx read once, O and LSE written once."""
    es = 2 if w.dtype == "bf16" else 4
    B, N, Hkv, G, D, k = w.batch, w.seqlen, w.kv_heads, w.group_size, w.head_dim, w.topk
    return (2 * B * N * Hkv * G * D + 2 * B * N * Hkv * D) * es + B * Hkv * N * k * 4 + B * Hkv * G * N * 4


def kl_flops(w):
    """F_KL = (2·D·Hq + 2·Di·Hkv)·B·sum_i |T_i|: the main scores of the G heads and
    the index scores over every selected token."""
    B, N, Hkv, G, D, Di, Bk, k = (w.batch, w.seqlen, w.kv_heads, w.group_size, w.head_dim,
                                  w.index_dim, w.block_size, w.topk)
    i = np.arange(N, dtype=np.int64)
    L = i // Bk
    tokens = float(((np.minimum(k, L + 1) - 1) * Bk + (i % Bk) + 1).sum())
    return (2.0 * D * Hkv * G + 2.0 * Di * Hkv) * B * tokens


def kl_backward_flops(w):
    """F_KL_bwd = (2·D·Hq + 3 · 2·Di·Hkv)·B·sum_i |T_i|: the teacher scores of the
    G heads, and per (position, token) the student score, its dk_idx and its
    dq_idx products."""
    B, N, Hkv, G, D, Di, Bk, k = (w.batch, w.seqlen, w.kv_heads, w.group_size, w.head_dim,
                                  w.index_dim, w.block_size, w.topk)
    i = np.arange(N, dtype=np.int64)
    L = i // Bk
    tokens = float(((np.minimum(k, L + 1) - 1) * Bk + (i % Bk) + 1).sum())
    return (2.0 * D * Hkv * G + 6.0 * Di * Hkv) * B * tokens


def source_digest(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_entry(kernel, workload, path=TRAFFIC_FILE):
    """Measured HBM bytes per launch of `kernel` (FETCH_SIZE + WRITE_SIZE,
    calibrated against a copy of known size) from the committed counter
    summary, if it was taken on this workload and on the current source of the
    file that holds the kernel; else None."""
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("workload") != workload:
        return None
    e = t.get("kernels", {}).get(kernel)
    if not e or e.get("source_sha256_16") != source_digest(os.path.join(CSRC, e.get("source", "?"))):
        return None
    return e.get("bytes_per_launch")


def attention_bytes(w, block_idx):
    """Algorithmic HBM bytes of the two attention kernels for this selection.

    Non-local kernel, per kept non-local block of a (b, g, i) row: the row's G
    query vectors (gathered), its normalised partial output (G x D) and G LSEs,
    and its list entry; per distinct kept (b, g, j): K_j and V_j^T once.
    Local + combine kernel: every row's partials and LSEs back, Q, the local
    K/V block, O and LSE."""
    es = 2 if w.dtype == "bf16" else 4
    B, N, Hkv, G, D, Bk = w.batch, w.seqlen, w.kv_heads, w.group_size, w.head_dim, w.block_size
    L = (torch.arange(N, device=block_idx.device) // Bk).view(1, 1, N, 1)
    nl = (block_idx >= 0) & (block_idx < L)
    sel = int(nl.sum())
    nb = (N + Bk - 1) // Bk
    bg = torch.arange(B * Hkv, device=block_idx.device).view(B, Hkv, 1, 1).expand_as(block_idx)
    kv_blocks = int(torch.unique((bg * nb + block_idx.long())[nl]).numel())
    per_sel_nl = 2 * G * D * es + 4 * G + 4
    kvb = 2 * Bk * D * es
    nonlocal_b = sel * per_sel_nl + kv_blocks * kvb
    combine_b = (sel * (G * D * es + 4 * G) + 2 * B * N * Hkv * G * D * es + B * Hkv * G * N * 4
                 + B * Hkv * nb * kvb)
    return {"selections": sel, "kv_blocks": kv_blocks, "nonlocal": nonlocal_b, "combine": combine_b}


def cpu_baseline(w, x, seconds_target=15.0):
    """The oracle as it stands on a bounded sample of rows of this workload."""
    from oracle import msa_oracle as O
    workers = max(1, min(16, os.cpu_count() or 1))
    n = 64
    kih = x["k_idx"].cpu()
    kh, vh = x["k"].cpu(), x["v"].cpu()
    spent = 0.0
    rows = 0
    while True:
        pos = sample_rows(w, n=n, seed=2 + rows)
        b = torch.as_tensor(pos[:, 0], device=x["q"].device)
        i = torch.as_tensor(pos[:, 1], device=x["q"].device)
        qi_rows, q_rows = x["q_idx"][b, i].cpu(), x["q"][b, i].cpu()
        t0 = time.perf_counter()
        bi = O.index_topk_rows(None, kih, pos, w.block_size, w.topk, q_rows=qi_rows)
        O.map_positions(lambda c, br, qr: O.attention_rows(None, kh, vh, br, c, w.block_size, q_rows=qr),
                        pos, (bi, q_rows), workers=workers)
        spent += time.perf_counter() - t0
        rows += len(pos)
        if spent >= seconds_target * 0.5 or n >= 4096:
            break
        n *= 2
    return {"value": rows / spent, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "sample": f"{rows} query positions (all {w.kv_heads} groups, {w.q_heads} heads) drawn "
                      f"from the {w.name} workload; index selection + attention, float64 oracle; "
                      f"{spent:.1f} s"}


def decode_bytes(w, seqlens):
    """Algorithmic HBM bytes of one decode step, per stage.

    Selection: the competing blocks' index keys (L_b * Bk tokens of Di values
    for sequence b, L_b = (n_b - 1) // Bk), the new index queries, the lengths
    and the block ids written. Attention: the selected tokens' K and V
    (|T_b| = (min(k, L_b + 1) - 1) Bk + (n_b - 1) % Bk + 1 per group), the new
    queries, O, LSE and the block ids read."""
    es = 2 if w.dtype == "bf16" else 4
    Hkv, G, D, Di, Bk, k = w.kv_heads, w.group_size, w.head_dim, w.index_dim, w.block_size, w.topk
    n = np.asarray(seqlens, dtype=np.int64)
    i = n - 1
    L = i // Bk
    T = (np.minimum(k, L + 1) - 1) * Bk + (i % Bk) + 1
    B = len(n)
    sel = int((L * Bk).sum()) * Di * es + B * Hkv * Di * es + B * 4 + B * Hkv * k * 4
    att = int(T.sum()) * Hkv * 2 * D * es + 2 * B * Hkv * G * D * es + B * Hkv * G * 4 + B * Hkv * k * 4
    return {"selection": sel, "attention": att, "selected_tokens": int(T.sum()) * Hkv}


def decode_cpu_baseline(w, x, seconds_target=15.0):
    """The oracle's decode on a bounded sample of the batch's sequences."""
    from oracle import msa_oracle as O
    lens = x["seqlens"].cpu().numpy()
    order = np.random.default_rng(2).permutation(w.batch)
    spent, done = 0.0, 0
    for b in order:
        n = int(lens[b])
        sl = slice(int(b), int(b) + 1)
        qi, ki = x["q_idx"][sl].cpu(), x["k_idx"][sl, :n].cpu()
        q, kc, vc = x["q"][sl].cpu(), x["k"][sl, :n].cpu(), x["v"][sl, :n].cpu()
        t0 = time.perf_counter()
        bi = O.decode_index_topk(qi, ki, np.array([n]), w.block_size, w.topk)
        O.decode_attention(q, kc, vc, np.array([n]), bi, w.block_size)
        spent += time.perf_counter() - t0
        done += 1
        if spent >= seconds_target * 0.5:
            break
    try:
        from threadpoolctl import threadpool_info
        cores = max(i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas")
    except (ImportError, ValueError):
        cores = os.cpu_count()
    return {"value": done / spent, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} of the {w.batch} sequences of the {w.name} batch (one new token each: "
                      f"selection + attention, float64 oracle, numpy BLAS threads); {spent:.1f} s"}


def bench_decode(args, dev):
    w = DECODE_CONFIGS["decode_n128k_b64"]
    log(f"[bench] decode batch {w.name}: generating caches on {dev}")
    x = make_decode_inputs(w, device=dev)
    B, C, Hkv, G, D = w.batch, w.seqlen, w.kv_heads, w.group_size, w.head_dim
    dims = msa.make_dims(B, C, Hkv, G, D, w.index_dim, w.topk, x["q"].dtype)
    ws = torch.empty(max(1, msa.workspace_bytes(dims, msa.MSA_OP_DECODE)), dtype=torch.uint8, device=dev)
    bi = torch.empty((B, Hkv, w.topk), dtype=torch.int32, device=dev)
    o = torch.empty_like(x["q"])
    lse = torch.empty((B, Hkv * G), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(ev):
        ev[0].record(stream)
        msa.decode_index_topk(x["q_idx"], x["k_idx"], x["seqlens"], w.topk, block_idx=bi, workspace=ws)
        ev[1].record(stream)
        msa.decode_attn(x["q"], x["k"], x["v"], x["seqlens"], bi, o=o, lse=lse, workspace=ws)
        ev[2].record(stream)

    def events():
        return [torch.cuda.Event(enable_timing=True) for _ in range(3)]

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step(events())
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} decode steps")
    evs = [events() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for ev in evs:
        step(ev)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    stage_ms = {name: float(np.mean([ev[a].elapsed_time(ev[a + 1]) for ev in evs]))
                for a, name in enumerate(("selection", "attention"))}
    ref = (bi.clone(), o.clone(), lse.clone())
    msa.decode(x["q_idx"], x["k_idx"], x["q"], x["k"], x["v"], x["seqlens"], w.topk, block_idx=bi, o=o, lse=lse,
               workspace=ws)
    torch.cuda.synchronize()
    same = all(torch.equal(a, b) for a, b in zip(ref, (bi, o, lse)))
    nb = decode_bytes(w, x["seqlens"].cpu().numpy())
    kernels = {"selection": "decode_scores_kernel + decode_topk_kernel",
               "attention": "decode_attn_kernel + decode_combine_kernel"}

    def hbm(stage):
        a = nb[stage] / (stage_ms[stage] * 1e-3) / 1e9
        parts = [traffic_entry(k.strip(), w.name, DECODE_TRAFFIC_FILE) for k in kernels[stage].split("+")]
        return {"kernel": kernels[stage], "bound": "hbm", "achieved": a, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": a / PEAK_HBM_GBS, "traffic": None if None in parts else sum(parts),
                "algorithmic_bytes": nb[stage], "ms": stage_ms[stage]}

    rooflines = {s: hbm(s) for s in ("selection", "attention")}
    dominant = max(rooflines, key=lambda s: stage_ms[s])
    lens = x["seqlens"].cpu().numpy()
    out = {
        "metric": "MSA decode tokens/s (one new token per sequence; 64 sequences, 128K-token caches, k=16, Bk=128)",
        "value": B / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"{w.name}: B={B} sequences, cache capacity {C}, lengths uniform on [1, {C}] "
                               f"(mean {lens.mean():.0f}), Hkv={Hkv} G={G} D={D} Di={w.index_dim} "
                               f"Bk={w.block_size} k={w.topk} {w.dtype}",
                   "global_batch": B, "seq_len": C, "parallelism": "single GPU"},
        "stage_ms": stage_ms,
        "hbm_gbs": (nb["selection"] + nb["attention"]) / (ms_step * 1e-3) / 1e9,
        "decode_matches_stages": same,
        "roofline": rooflines[dominant],
        "rooflines": rooflines,
    }
    if args.decode_queries > 1:
        # R new tokens per sequence at once (positions n_b - R .. n_b - 1): one step.
        R = args.decode_queries
        g = torch.Generator(device=dev)
        g.manual_seed(w.seed + 4000)
        qiR = torch.randint(-4, 5, (B, R, Hkv, w.index_dim), generator=g, device=dev).to(x["q_idx"].dtype)
        qR = torch.randn((B, R, Hkv * G, D), generator=g, device=dev).to(x["q"].dtype)
        wsR = torch.empty(max(1, msa.decode_workspace_bytes(dims, msa.MSA_OP_DECODE, R)), dtype=torch.uint8,
                          device=dev)

        def rstep():
            msa.decode(qiR, x["k_idx"], qR, x["k"], x["v"], x["seqlens"], w.topk, workspace=wsR)
        for _ in range(args.warmup):
            rstep()
        evr = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for e in evr:
            e[0].record(stream)
            rstep()
            e[1].record(stream)
        torch.cuda.synchronize()
        msr = float(np.mean([e[0].elapsed_time(e[1]) for e in evr]))
        out["multi_query"] = {"queries_per_sequence": R, "ms": msr, "tokens_per_s": B * R / (msr * 1e-3)}
    if args.paged:
        # The same step on paged caches: 128-token pages in a seeded random order and a block table.
        nbs = -(-C // w.block_size)
        perm = torch.randperm(B * nbs, generator=torch.Generator().manual_seed(7)).to(torch.int32)
        table = perm.view(B, nbs).to(dev)
        pools = {}
        for name in ("k_idx", "k", "v"):
            t = x[name]
            pool = torch.empty((B * nbs, w.block_size) + tuple(t.shape[2:]), dtype=t.dtype, device=dev)
            pool[perm.long().to(dev)] = t.reshape((B * nbs, w.block_size) + tuple(t.shape[2:]))
            pools[name] = pool
        bip = torch.empty_like(bi)
        op, lsep = torch.empty_like(o), torch.empty_like(lse)

        def pstep():
            msa.decode_paged(x["q_idx"], pools["k_idx"], x["q"], pools["k"], pools["v"], table, x["seqlens"], w.topk,
                             block_idx=bip, o=op, lse=lsep, workspace=ws)
        for _ in range(args.warmup):
            pstep()
        evp = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for e in evp:
            e[0].record(stream)
            pstep()
            e[1].record(stream)
        torch.cuda.synchronize()
        out["paged"] = {"ms": float(np.mean([e[0].elapsed_time(e[1]) for e in evp])),
                        "same_results": bool(torch.equal(bip, bi) and torch.equal(op, o) and torch.equal(lsep, lse))}
        del pools
    if args.index_fp8:
        # The selection on an fp8 e4m3 index cache (integer values: exact, same selection).
        fp8 = torch.float8_e4m3fn
        qi8, ki8 = x["q_idx"].to(fp8), x["k_idx"].to(fp8)
        bi8 = torch.empty_like(bi)
        for _ in range(args.warmup):
            msa.decode_index_topk(qi8, ki8, x["seqlens"], w.topk, block_idx=bi8, workspace=ws)
        ev8 = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for e in ev8:
            e[0].record(stream)
            msa.decode_index_topk(qi8, ki8, x["seqlens"], w.topk, block_idx=bi8, workspace=ws)
            e[1].record(stream)
        torch.cuda.synchronize()
        ms8 = float(np.mean([e[0].elapsed_time(e[1]) for e in ev8]))
        b8 = (nb["selection"] - B * Hkv * w.index_dim - int(((lens - 1) // w.block_size * w.block_size).sum())
              * w.index_dim)   # one byte per index value instead of two
        out["selection_fp8"] = {"ms": ms8, "algorithmic_bytes": b8, "achieved_gbs": b8 / (ms8 * 1e-3) / 1e9,
                                "frac_of_hbm": b8 / (ms8 * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                "speedup_vs_bf16_selection": stage_ms["selection"] / ms8,
                                "step_ms_with_fp8_selection": ms8 + stage_ms["attention"],
                                "same_selection": bool(torch.equal(bi8, bi))}
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle decode on a bounded sample)")
        out["cpu_baseline"] = decode_cpu_baseline(w, x, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def bench_dense(args, dev):
    """The warm-up's dense causal attention on the 128K workload's shapes."""
    w = CONFIGS["n128k"]
    log(f"[bench] dense attention on {w.name} shapes: generating inputs on {dev}")
    x = make_inputs(w, device=dev, kinds=("q", "k", "v"))
    B, N, Hkv, G, D = w.batch, w.seqlen, w.kv_heads, w.group_size, w.head_dim
    dims = msa.make_dims(B, N, Hkv, G, D, w.index_dim, 1, x["q"].dtype)
    ws = torch.empty(max(1, msa.workspace_bytes(dims, msa.MSA_OP_DENSE_ATTN)), dtype=torch.uint8, device=dev)
    o = torch.empty_like(x["q"])
    lse = torch.empty((B, Hkv * G, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        msa.dense_attn_fwd(x["q"], x["k"], x["v"], o=o, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} dense steps")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e in evs:
        e[0].record(stream)
        msa.dense_attn_fwd(x["q"], x["k"], x["v"], o=o, lse=lse, workspace=ws)
        e[1].record(stream)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    ms_ev = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    # F_dense = 4 * D * Hq * sum_i (i + 1): QK^T and PV over every causally visible key.
    f = 4.0 * D * B * Hkv * G * N * (N + 1) / 2
    a = f / (ms_ev * 1e-3) / 1e12
    out = {
        "metric": "MSA dense (warm-up) causal GQA attention fwd tokens/s and TFLOP/s at N=128K",
        "value": B * N / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"dense causal attention, n128k shapes: B={B} N={N} Hkv={Hkv} G={G} D={D} {w.dtype}",
                   "global_batch": B, "seq_len": N, "parallelism": "single GPU"},
        "tflops": f / (ms_step * 1e-3) / 1e12,
        "roofline": {"kernel": "dense_attn_kernel (+ V^T copy)", "bound": "mfma", "achieved": a,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": a / PEAK_BF16_TFLOPS, "traffic": None,
                     "algorithmic_tflop": f / 1e12, "ms": ms_ev},
    }
    if args.kl:
        # The warm-up's KL over every visible token, on the dense LSE.
        log("[bench] dense KL")
        xi = make_inputs(w, device=dev, kinds=("q_idx", "k_idx"))
        kws = torch.empty(max(1, msa.workspace_bytes(dims, msa.MSA_OP_DENSE_KL)), dtype=torch.uint8, device=dev)
        kl_rows = torch.empty((B, Hkv, N), dtype=torch.float32, device=dev)
        kl_sum = torch.empty((1,), dtype=torch.float32, device=dev)

        def kl():
            msa.dense_kl_align_fwd(x["q"], x["k"], xi["q_idx"], xi["k_idx"], lse, kl_rows=kl_rows, kl_sum=kl_sum,
                                   workspace=kws)
        kl()
        kev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for e in kev:
            e[0].record(stream)
            kl()
            e[1].record(stream)
        torch.cuda.synchronize()
        kl_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in kev]))
        fk = (2.0 * D * Hkv * G + 2.0 * w.index_dim * Hkv) * B * N * (N + 1) / 2
        out["dense_kl_align"] = {"ms": kl_ms, "algorithmic_tflop": fk / 1e12, "tflops": fk / (kl_ms * 1e-3) / 1e12,
                                 "frac_of_peak": fk / (kl_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                                 "kl_sum": float(kl_sum.item())}
    if not args.no_cpu_baseline:
        from oracle import msa_oracle as O
        log("[bench] cpu baseline (oracle dense rows on a bounded sample)")
        kh, vh = x["k"].cpu(), x["v"].cpu()
        workers = max(1, min(16, os.cpu_count() or 1))
        pos = sample_rows(w, n=128, seed=3)
        b = torch.as_tensor(pos[:, 0], device=dev)
        i = torch.as_tensor(pos[:, 1], device=dev)
        q_rows = x["q"][b, i].cpu()
        rows = O.dense_block_idx_rows(pos, Hkv, w.block_size)
        t0 = time.perf_counter()
        O.map_positions(lambda c, br, qr: O.attention_rows(None, kh, vh, br, c, w.block_size, q_rows=qr),
                        pos, (rows, q_rows), workers=workers)
        spent = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": len(pos) / spent, "unit": "tokens/s", "cores": workers, "kind": "oracle",
                               "sample": f"{len(pos)} query positions of the 128K sequence (all 64 heads, every "
                                         f"visible key), float64 oracle; {spent:.1f} s"}
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="n128k", choices=sorted(CONFIGS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--kl", action="store_true",
                    help="also time the KL-alignment forward (msa_kl_align_fwd) on the step's outputs")
    ap.add_argument("--index-fp8", action="store_true",
                    help="also time the step with the selection on fp8 e4m3 copies of the index inputs "
                         "(reported beside the bf16 headline, never as it)")
    ap.add_argument("--index-fp4", action="store_true",
                    help="also time the step with the selection on fp4 e2m1 copies of the index inputs "
                         "(reported beside the bf16 headline, never as it)")
    ap.add_argument("--bwd", action="store_true",
                    help="also time the main-branch backward (msa_sparse_attn_bwd) on the step's outputs")
    ap.add_argument("--fused-only", action="store_true",
                    help="with --bwd --kl: time only the fused backward (msa_fused_bwd), not the separate ones")
    ap.add_argument("--decode", action="store_true",
                    help="time one decode step (64 sequences, 128K-token caches) instead of the forward")
    ap.add_argument("--decode-queries", type=int, default=1,
                    help="with --decode: also time one step with this many new tokens per sequence")
    ap.add_argument("--paged", action="store_true",
                    help="with --decode: also time the step on paged caches (block table, random page order)")
    ap.add_argument("--dense", action="store_true",
                    help="time the warm-up's dense causal attention (msa_dense_attn_fwd) on the 128K shapes instead")
    ap.add_argument("--stream-probe", action="store_true",
                    help="only time plain read/write/copy kernels on cache-resident and HBM-sized buffers")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the MSA forward path here runs on a single MI355X "
              "(multi-GPU sharding by (batch, group) is a design note, not built). Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    dev = torch.device("cuda:0")
    if args.stream_probe:
        # Streaming rates of plain torch kernels on buffers that fit the 256 MB infinity
        # cache (repeated passes stay resident) and on buffers far larger than it.
        res = []
        for mib in (64, 128, 192, 4096):
            n = mib << 18
            a = torch.ones(n, dtype=torch.float32, device=dev)
            b = torch.empty_like(a)
            for name, fn, nbytes in (("read", lambda: a.sum(), n * 4), ("write", lambda: b.fill_(1.0), n * 4),
                                     ("copy", lambda: b.copy_(a), 2 * n * 4)):
                for _ in range(3):
                    fn()
                reps = max(8, (8 << 30) // nbytes)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(reps):
                    fn()
                e1.record()
                torch.cuda.synchronize()
                ms = e0.elapsed_time(e1) / reps
                res.append({"mib": mib, "op": name, "ms": ms, "gbs": nbytes / (ms * 1e-3) / 1e9})
                log(f"[bench] stream {name} {mib} MiB: {res[-1]['gbs']:.0f} GB/s")
            del a, b
        print(json.dumps({"stream_probe": res}), flush=True)
        return
    if args.copy_mib:
        # Reference for HBM byte counters: one launch reads and writes exactly this many bytes.
        src = torch.ones(args.copy_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.copy_mib << 20}), flush=True)
        return
    if args.decode:
        msa.load_library()
        bench_decode(args, dev)
        return
    if args.dense:
        msa.load_library()
        bench_dense(args, dev)
        return
    w = CONFIGS[args.workload]
    msa.load_library()
    log(f"[bench] workload {w.name}: generating inputs on {dev}")
    x = make_inputs(w, device=dev)
    B, N, Hkv, G, D = w.batch, w.seqlen, w.kv_heads, w.group_size, w.head_dim
    block_idx = torch.empty((B, Hkv, N, w.topk), dtype=torch.int32, device=dev)
    o = torch.empty_like(x["q"])
    lse = torch.empty((B, Hkv * G, N), dtype=torch.float32, device=dev)
    dims = msa.make_dims(B, N, Hkv, G, D, w.index_dim, w.topk, x["q"].dtype)
    ws = torch.empty(max(1, msa.workspace_bytes(dims, msa.MSA_OP_FORWARD)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    # The selection runs the software-pipelined 8-wave kernel when 512 rows tile
    # a query block in bf16, else the general one (the name only labels the entry).
    index_kernel = ("index_topk_pipe_kernel" if w.dtype == "bf16" and (w.block_size * Hkv) % 512 == 0
                    else "index_topk_kernel")

    def step(ev, q_idx=x["q_idx"], k_idx=x["k_idx"], bi=block_idx):
        """One step; ev[0..4] bracket the selection and the three attention stages."""
        ev[0].record(stream)
        msa.index_topk(q_idx, k_idx, w.topk, block_idx=bi)
        ev[1].record(stream)
        for s, e in ((msa.STAGE_PREPARE, ev[2]), (msa.STAGE_NONLOCAL, ev[3]), (msa.STAGE_COMBINE, ev[4])):
            msa.sparse_attn_fwd(x["q"], x["k"], x["v"], bi, o=o, lse=lse, workspace=ws, stages=s)
            e.record(stream)

    def events():
        return [torch.cuda.Event(enable_timing=True) for _ in range(5)]

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step(events())
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    evs = [events() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for ev in evs:
        step(ev)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    stage_ms = {name: float(np.mean([ev[a].elapsed_time(ev[a + 1]) for ev in evs]))
                for a, name in enumerate((index_kernel, "prepare", "attn_nonlocal_kernel",
                                          "attn_local_combine_kernel"))}
    # The forward entry point gives the same bits as the four calls.
    ref = (block_idx.clone(), o.clone(), lse.clone())
    msa.forward(x["q_idx"], x["k_idx"], x["q"], x["k"], x["v"], w.topk, block_idx=block_idx, o=o, lse=lse,
                workspace=ws)
    torch.cuda.synchronize()
    same = all(torch.equal(a, b) for a, b in zip(ref, (block_idx, o, lse)))

    f_idx, f_main = flops(w)
    tokens = B * N
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    ab = attention_bytes(w, block_idx)
    wl = w.name

    f_nonlocal, f_local = flops_split(w)

    def mfma_entry(kernel, work_flop, design_bytes=None):
        """Roofline of one kernel against the matrix-core peak: its share of the
        method's algorithmic work (F_idx, or F_main's non-local / local part)
        over its event-timed duration. The bytes this design moves (gathered
        query rows, partial outputs) and their measured rate are reported
        beside it, not as the roofline."""
        a = work_flop / (stage_ms[kernel] * 1e-3) / 1e12
        e = {"kernel": kernel, "bound": "mfma", "achieved": a, "peak": peak, "unit": "TFLOP/s",
             "frac": a / peak, "traffic": traffic_entry(kernel, wl), "algorithmic_tflop": work_flop / 1e12,
             "ms": stage_ms[kernel]}
        if design_bytes is not None:
            e["design_bytes"] = design_bytes
            e["design_gbs"] = design_bytes / (stage_ms[kernel] * 1e-3) / 1e9
        return e

    rooflines = {index_kernel: mfma_entry(index_kernel, f_idx),
                 "attn_nonlocal_kernel": mfma_entry("attn_nonlocal_kernel", f_nonlocal, ab["nonlocal"]),
                 "attn_local_combine_kernel": mfma_entry("attn_local_combine_kernel", f_local, ab["combine"])}
    dominant = max(rooflines, key=lambda k: stage_ms[k])
    comp = compulsory_attention_bytes(w)
    attention_traffic = {"compulsory_bytes": comp, "design_bytes": ab["nonlocal"] + ab["combine"],
                         "design_over_compulsory": (ab["nonlocal"] + ab["combine"]) / comp}
    out = {
        "metric": "MSA fwd tokens/s and TFLOP/s (% bf16 MFMA peak) at N=128K, k=16, Bk=128",
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"{w.name}: B={B} N={N} Hkv={Hkv} G={G} D={D} Di={w.index_dim} "
                               f"Bk={w.block_size} k={w.topk} {w.dtype}"
                               + (f", {int(round(w.stripe_frac * w.nblocks))} stripe blocks +{w.stripe_bias:g}"
                                  if w.stripe_frac else ""),
                   "global_batch": B, "seq_len": N, "parallelism": "single GPU"},
        "tflops": (f_idx + f_main) / (ms_step * 1e-3) / 1e12,
        "frac_of_peak": (f_idx + f_main) / (ms_step * 1e-3) / 1e12 / peak,
        "algorithmic_tflop": {"index": f_idx / 1e12, "attention": f_main / 1e12},
        "stage_ms": stage_ms,
        "forward_matches_stages": same,
        "roofline": rooflines[dominant],
        "rooflines": rooflines,
        "attention_bytes": attention_traffic,
    }
    if args.index_fp8:
        # Same workload with the index inputs held as fp8 e4m3 (their integer
        # values are exact in it, so the selection must not change).
        log("[bench] step with the fp8 selection")
        fp8 = torch.float8_e4m3fn
        qi8, ki8 = x["q_idx"].to(fp8), x["k_idx"].to(fp8)
        bi8 = torch.empty_like(block_idx)
        for _ in range(args.warmup):
            step(events(), qi8, ki8, bi8)
        evs8 = [events() for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for ev in evs8:
            step(ev, qi8, ki8, bi8)
        torch.cuda.synchronize()
        ms8 = (time.perf_counter() - t0) * 1e3 / args.steps
        idx8 = float(np.mean([ev[0].elapsed_time(ev[1]) for ev in evs8]))
        a8 = f_idx / (idx8 * 1e-3) / 1e12
        out["index_fp8"] = {
            "kernel": index_kernel, "dtype": "fp8 e4m3 index inputs, fp32 accumulation", "ms": idx8,
            "achieved": a8, "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s", "frac": a8 / PEAK_FP8_TFLOPS,
            "speedup_vs_bf16_index": stage_ms[index_kernel] / idx8,
            "ms_per_step": ms8, "tokens_per_s": tokens / (ms8 * 1e-3),
            "same_selection": bool(torch.equal(bi8, block_idx))}
    if args.index_fp4:
        # The index inputs as OCP fp4 e2m1 (two per byte): the integers -4..4 are exact, so
        # the selection equals the bf16 one wherever the inputs fit; the 128K stripes' +3
        # bias takes some components to 5..7, which round to 4 or 6.
        log("[bench] step with the fp4 selection")
        qi4, ki4 = to_fp4_e2m1(x["q_idx"]), to_fp4_e2m1(x["k_idx"])
        bi4 = torch.empty_like(block_idx)
        for _ in range(args.warmup):
            step(events(), qi4, ki4, bi4)
        evs4 = [events() for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for ev in evs4:
            step(ev, qi4, ki4, bi4)
        torch.cuda.synchronize()
        ms4 = (time.perf_counter() - t0) * 1e3 / args.steps
        idx4 = float(np.mean([ev[0].elapsed_time(ev[1]) for ev in evs4]))
        a4 = f_idx / (idx4 * 1e-3) / 1e12
        out["index_fp4"] = {
            "kernel": index_kernel, "dtype": "fp4 e2m1 index inputs (unit scales), fp32 accumulation", "ms": idx4,
            "achieved": a4, "peak": PEAK_FP4_TFLOPS, "unit": "TFLOP/s", "frac": a4 / PEAK_FP4_TFLOPS,
            "speedup_vs_bf16_index": stage_ms[index_kernel] / idx4,
            "ms_per_step": ms4, "tokens_per_s": tokens / (ms4 * 1e-3),
            "same_selection": bool(torch.equal(bi4, block_idx)),
            "rows_with_same_selection": float((bi4 == block_idx).all(dim=-1).float().mean())}
    if args.bwd and args.kl:
        # Both branches' gradients from one pass (msa_fused_bwd), query window by query window.
        log("[bench] fused backward of both branches")
        dout_f = make_grad_output(w, device=dev)
        wr_f = make_row_weights(w, device=dev)
        ilse_f = torch.empty((B, Hkv, N), dtype=torch.float32, device=dev)
        kws_f = torch.empty(max(1, msa.workspace_bytes(dims, msa.MSA_OP_KL)), dtype=torch.uint8, device=dev)
        msa.kl_align_fwd(x["q"], x["k"], x["q_idx"], x["k_idx"], block_idx, lse, index_lse=ilse_f, workspace=kws_f)
        del kws_f
        fws = torch.empty(max(1, msa.workspace_bytes(dims, msa.MSA_OP_FUSED_BWD)), dtype=torch.uint8, device=dev)
        fouts = [torch.empty_like(t) for t in (x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"])]

        def fused():
            msa.fused_bwd(x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], block_idx, o, lse, ilse_f, dout_f,
                          dkl_rows=wr_f, dq=fouts[0], dk=fouts[1], dv=fouts[2], dq_idx=fouts[3], dk_idx=fouts[4],
                          workspace=fws)
        fused()
        fev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(max(1, args.steps))]
        for e in fev:
            e[0].record(stream)
            fused()
            e[1].record(stream)
        torch.cuda.synchronize()
        fms = float(np.mean([e[0].elapsed_time(e[1]) for e in fev]))
        fb = 2.5 * f_main + kl_backward_flops(w) - 2.0 * w.head_dim * B * Hkv * G * float(
            ((np.minimum(w.topk, np.arange(N) // w.block_size + 1) - 1) * w.block_size + np.arange(N) % w.block_size
             + 1).sum())   # the teacher's scores are the main branch's: counted once
        out["fused_backward"] = {"ms": fms, "algorithmic_tflop": fb / 1e12, "tflops": fb / (fms * 1e-3) / 1e12,
                                 "frac_of_peak": fb / (fms * 1e-3) / 1e12 / peak,
                                 "workspace_gb": fws.numel() / 1e9, "tokens_per_s": tokens / (fms * 1e-3)}
        del fws, fouts
        if args.fused_only:
            args.bwd = False
    if args.bwd:
        log("[bench] main-branch backward")
        dout = make_grad_output(w, device=dev)
        bws = torch.empty(max(1, msa.workspace_bytes(dims, msa.MSA_OP_ATTN_BWD)), dtype=torch.uint8, device=dev)
        dq, dk, dv = torch.empty_like(x["q"]), torch.empty_like(x["k"]), torch.empty_like(x["v"])

        def bwd():
            msa.sparse_attn_bwd(x["q"], x["k"], x["v"], block_idx, o, lse, dout, dq=dq, dk=dk, dv=dv, workspace=bws)
        for _ in range(max(1, args.warmup)):
            bwd()
        bev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(max(1, args.steps))]
        for e in bev:
            e[0].record(stream)
            bwd()
            e[1].record(stream)
        torch.cuda.synchronize()
        bwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in bev]))
        fb = 2.5 * f_main   # S, dP, dV, dK, dQ: five D-deep products per (row, token) against the forward's two
        out["backward"] = {"ms": bwd_ms, "algorithmic_tflop": fb / 1e12, "tflops": fb / (bwd_ms * 1e-3) / 1e12,
                           "frac_of_peak": fb / (bwd_ms * 1e-3) / 1e12 / peak,
                           "tokens_per_s": tokens / (bwd_ms * 1e-3)}
    if args.kl:
        log("[bench] KL-alignment forward")
        kws = torch.empty(max(1, msa.workspace_bytes(dims, msa.MSA_OP_KL)), dtype=torch.uint8, device=dev)
        kl_rows = torch.empty((B, Hkv, N), dtype=torch.float32, device=dev)
        kl_sum = torch.empty((1,), dtype=torch.float32, device=dev)

        def kl():
            msa.kl_align_fwd(x["q"], x["k"], x["q_idx"], x["k_idx"], block_idx, lse, kl_rows=kl_rows,
                             kl_sum=kl_sum, workspace=kws)
        kl()
        kev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(max(1, args.steps))]
        for e in kev:
            e[0].record(stream)
            kl()
            e[1].record(stream)
        torch.cuda.synchronize()
        kl_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in kev]))
        fk = kl_flops(w)
        out["kl_align"] = {"ms": kl_ms, "algorithmic_tflop": fk / 1e12, "tflops": fk / (kl_ms * 1e-3) / 1e12,
                           "frac_of_peak": fk / (kl_ms * 1e-3) / 1e12 / peak, "kl_sum": float(kl_sum.item())}
        if args.bwd:
            # KL-term backward (index-branch gradients) on the same rows, unit row weights.
            ilse = torch.empty((B, Hkv, N), dtype=torch.float32, device=dev)
            msa.kl_align_fwd(x["q"], x["k"], x["q_idx"], x["k_idx"], block_idx, lse, kl_rows=kl_rows,
                             kl_sum=kl_sum, workspace=kws, index_lse=ilse)
            kbws = torch.empty(max(1, msa.workspace_bytes(dims, msa.MSA_OP_KL_BWD)), dtype=torch.uint8,
                               device=dev)
            dqi, dki = torch.empty_like(x["q_idx"]), torch.empty_like(x["k_idx"])

            def klb():
                msa.kl_align_bwd(x["q"], x["k"], x["q_idx"], x["k_idx"], block_idx, lse, ilse, dq_idx=dqi,
                                 dk_idx=dki, workspace=kbws)
            klb()
            for e in kev:
                e[0].record(stream)
                klb()
                e[1].record(stream)
            torch.cuda.synchronize()
            klb_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in kev]))
            fkb = kl_backward_flops(w)
            out["kl_align_bwd"] = {"ms": klb_ms, "algorithmic_tflop": fkb / 1e12,
                                   "tflops": fkb / (klb_ms * 1e-3) / 1e12,
                                   "frac_of_peak": fkb / (klb_ms * 1e-3) / 1e12 / peak}
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle on a bounded sample)")
        out["cpu_baseline"] = cpu_baseline(w, x, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
