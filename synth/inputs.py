"""Seeded input generation (no method arithmetic here)."""
import math

import numpy as np
import torch

from .configs import Workload

_TORCH_DTYPE = {"bf16": torch.bfloat16, "f32": torch.float32}
_CHUNK = 1 << 26  # elements drawn per call, bounds the fp32/int64 temporaries


def torch_dtype(name: str) -> torch.dtype:
    return _TORCH_DTYPE[name]


def _randint(shape, gen, device, dtype, absmax=4):
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    for s in range(0, flat.numel(), _CHUNK):
        e = min(flat.numel(), s + _CHUNK)
        flat[s:e] = torch.randint(-absmax, absmax + 1, (e - s,), generator=gen, device=device).to(dtype)
    return out


def _randn(shape, gen, device, dtype):
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    for s in range(0, flat.numel(), _CHUNK):
        e = min(flat.numel(), s + _CHUNK)
        flat[s:e] = torch.randn((e - s,), generator=gen, device=device,
                                dtype=torch.float32).to(dtype)
    return out


def stripe_blocks(w: Workload, gen: torch.Generator, device) -> torch.Tensor:
    n = int(round(w.stripe_frac * w.nblocks))
    if n <= 0:
        return torch.empty(0, dtype=torch.long)
    perm = torch.randperm(w.nblocks, generator=gen, device=device)
    return perm[:n].sort().values.cpu()


def make_inputs(w: Workload, device="cpu", seed=None, kinds=("q_idx", "k_idx", "q", "k", "v")):
    """Draw the workload's inputs on ``device`` from one seeded generator.

    Returns a dict with q_idx [B,N,Hkv,Di], k_idx [B,N,Di], q [B,N,Hq,D],
    k/v [B,N,Hkv,D] (all in the workload dtype) and 'stripes' (block ids that got
    the k_idx bias). Tensors not listed in ``kinds`` are still drawn (to keep the
    random stream aligned) but dropped.
    """
    seed = w.seed if seed is None else seed
    dt = torch_dtype(w.dtype)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    B, N, Hkv, G, D, Di, Bk = (w.batch, w.seqlen, w.kv_heads, w.group_size,
                               w.head_dim, w.index_dim, w.block_size)
    out = {}
    out["q_idx"] = _randint((B, N, Hkv, Di), gen, device, dt, w.index_absmax)
    k_idx = _randint((B, N, Di), gen, device, dt, w.index_absmax)
    stripes = stripe_blocks(w, gen, device)
    for j in stripes.tolist():
        k_idx[:, j * Bk:min(N, (j + 1) * Bk), :] += w.stripe_bias
    out["k_idx"] = k_idx
    out["stripes"] = stripes
    out["q"] = _randn((B, N, Hkv * G, D), gen, device, dt)
    out["k"] = _randn((B, N, Hkv, D), gen, device, dt)
    out["v"] = _randn((B, N, Hkv, D), gen, device, dt)
    for name in ("q_idx", "k_idx", "q", "k", "v"):
        if name not in kinds:
            del out[name]
    return out


def edge_positions(w: Workload):
    """Query positions at the block and budget edges: 0, Bk-1, Bk, k*Bk-1, k*Bk, N-1."""
    Bk, k, N = w.block_size, w.topk, w.seqlen
    cand = [0, Bk - 1, Bk, k * Bk - 1, k * Bk, N - 1]
    return sorted({p for p in cand if 0 <= p < N})


def uniform_rows(w: Workload, n=None, seed=1):
    """The uniformly drawn part of ``sample_rows``: ``n`` flat positions
    b * N + i drawn without replacement over all B*N (all of them when n
    covers the workload), unsorted int64."""
    n = w.sampled_rows if n is None else n
    total = w.batch * w.seqlen
    if n <= 0 or n >= total:
        return np.arange(total, dtype=np.int64)
    return np.random.default_rng(seed).choice(total, size=n, replace=False).astype(np.int64)


def sample_rows(w: Workload, n=None, seed=1):
    """(b, i) query positions checked on large workloads: ``n`` drawn without
    replacement over all B*N positions plus the edge positions in every batch.
    Returns an int64 array of shape [M, 2], sorted."""
    flat = uniform_rows(w, n, seed)
    edges = [b * w.seqlen + p for b in range(w.batch) for p in edge_positions(w)]
    flat = np.unique(np.concatenate([flat, np.asarray(edges, dtype=np.int64)]))
    return np.stack([flat // w.seqlen, flat % w.seqlen], axis=1)


def make_grad_output(w: Workload, device="cpu", seed=None):
    """Seeded output gradient dO [B, N, Hq, D] for the backward: standard
    normal in the workload dtype, from its own generator (seed + 1000), so the
    forward inputs do not change."""
    seed = (w.seed if seed is None else seed) + 1000
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return _randn((w.batch, w.seqlen, w.q_heads, w.head_dim), gen, device, torch_dtype(w.dtype))


def make_row_weights(w: Workload, device="cpu", seed=None):
    """Seeded per-row loss weights [B, Hkv, N] for the KL backward, uniform on
    [0.5, 2), fp32, from their own generator (seed + 2000)."""
    seed = (w.seed if seed is None else seed) + 2000
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return 0.5 + 1.5 * torch.rand((w.batch, w.kv_heads, w.seqlen), generator=gen, device=device)


def make_decode_inputs(w: Workload, device="cpu", seed=None, lengths=None):
    """Seeded decode batch: ``w.batch`` sequences with a cache of capacity
    ``w.seqlen`` tokens and one new query each.

    Draw order from one generator: k_idx cache [B, C, Di] (integers, as for the
    forward, with the same stripe rule), stripes, K and V caches [B, C, Hkv, D]
    (standard normal), the new index queries q_idx [B, Hkv, Di] (integers) and
    queries q [B, Hq, D] (standard normal). Cache slots past a sequence's length
    hold random values too (they must never be read). ``lengths`` (cached
    tokens per sequence, the new one included) default to integers uniform on
    [1, C] from their own generator (seed + 3000); returned as int32 on
    ``device`` under 'seqlens'.
    """
    seed = w.seed if seed is None else seed
    dt = torch_dtype(w.dtype)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    B, C, Hkv, G, D, Di, Bk = (w.batch, w.seqlen, w.kv_heads, w.group_size,
                               w.head_dim, w.index_dim, w.block_size)
    out = {}
    k_idx = _randint((B, C, Di), gen, device, dt, w.index_absmax)
    stripes = stripe_blocks(w, gen, device)
    for j in stripes.tolist():
        k_idx[:, j * Bk:min(C, (j + 1) * Bk), :] += w.stripe_bias
    out["k_idx"] = k_idx
    out["stripes"] = stripes
    out["k"] = _randn((B, C, Hkv, D), gen, device, dt)
    out["v"] = _randn((B, C, Hkv, D), gen, device, dt)
    out["q_idx"] = _randint((B, Hkv, Di), gen, device, dt, w.index_absmax)
    out["q"] = _randn((B, Hkv * G, D), gen, device, dt)
    if lengths is None:
        lgen = torch.Generator(device="cpu")
        lgen.manual_seed(seed + 3000)
        lengths = torch.randint(1, C + 1, (B,), generator=lgen)
    out["seqlens"] = torch.as_tensor(lengths, dtype=torch.int32).reshape(B).to(device)
    return out


# OCP fp4 e2m1 magnitudes by code 0..7; the rounding boundaries between codes
# c and c + 1 are the midpoints, a value on a midpoint goes to the even code.
_FP4_MIDPOINTS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def to_fp4_e2m1(x: torch.Tensor) -> torch.Tensor:
    """Round x to OCP fp4 e2m1 (nearest, ties to the even code, saturating at
    +-6) and pack two values per byte, element 2c in bits 0-3 of byte c:
    returns a float4_e2m1fn_x2 tensor with the last dimension halved (it must
    be even). An input conversion for tests and the benchmark; the integers
    -4..4 and +-6 are held exactly."""
    a = x.detach().float().abs()
    code = torch.zeros(a.shape, dtype=torch.uint8, device=x.device)
    for c, t in enumerate(_FP4_MIDPOINTS):
        up = (a > t) | ((a == t) & ((c + 1) % 2 == 0))
        code += up.to(torch.uint8)
    code |= ((x < 0) & (code != 0)).to(torch.uint8) << 3
    packed = code[..., 0::2] | (code[..., 1::2] << 4)
    return packed.contiguous().view(torch.float4_e2m1fn_x2)
