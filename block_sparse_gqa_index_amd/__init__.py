"""MSA (MiniMax Sparse Attention) forward hot path (and the main branch's
backward) on AMD Instinct MI355X.

Thin ctypes binding over ``libmsa.so`` (the C ABI declared in include/msa.h).
This module only marshals arguments: shapes and pointers of torch device
tensors, the current HIP stream, and workspace buffers allocated through
torch. Every step of the computation runs in the library's HIP kernels; if
the library is missing, every call raises.

Entry points (same names as the C ABI, without the ``msa_`` prefix):
  index_topk(q_idx, k_idx, topk)                   -> block_idx int32 [B, Hkv, N, k]
  check_block_idx(block_idx)                       -> int32 [1] on the device: rows breaking the layout
  sparse_attn_fwd(q, k, v, block_idx, scale)       -> (o [B,N,Hq,D], lse fp32 [B,Hq,N])
      (stages=... enqueues only some of its three stages: msa_sparse_attn_fwd_stages)
  kl_align_fwd(q, k, q_idx, k_idx, block_idx, lse) -> (kl_rows fp32 [B,Hkv,N], kl_sum fp32 [1])
      (index_lse=<fp32 [B,Hkv,N] tensor> also receives the student LSE per row)
  kl_align_bwd(q, k, q_idx, k_idx, block_idx, lse, index_lse) -> (dq_idx, dk_idx), bf16
  forward(q_idx, k_idx, q, k, v, topk)             -> (block_idx, o, lse): selection, then attention
  sparse_attn_bwd(q, k, v, block_idx, o, lse, dout) -> (dq, dk, dv), bf16
  fused_bwd(q, k, v, q_idx, k_idx, block_idx, o, lse, index_lse, dout)
                                                   -> (dq, dk, dv, dq_idx, dk_idx): both branches in one pass
  decode_index_topk(q_idx, k_idx, seqlens, topk)   -> block_idx int32 [B, Hkv, k] (one new query per sequence;
                                                      q_idx [B, R, Hkv, Di]: R new queries -> [B, Hkv, R, k])
  decode_attn(q, k, v, seqlens, block_idx)         -> (o [B,Hq,D], lse fp32 [B,Hq]) (or [B,R,Hq,D], [B,Hq,R])
  decode(q_idx, k_idx, q, k, v, seqlens, topk)     -> (block_idx, o, lse): both decode steps
  decode_paged*(..., block_table, ...)             -> the decode calls on page pools [P, 128, ...] + a block table
  decode_noalloc(q_idx, k_idx, q, k, v, seqlens, topk) -> decode() with the library's fixed scratch, no workspace
  dense_attn_fwd(q, k, v)                          -> (o, lse): causal attention over every visible key (warm-up)
  dense_kl_align_fwd(q, k, q_idx, k_idx, lse)      -> (kl_rows, kl_sum): the KL loss over every visible token
  workspace_bytes(dims, op)
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmsa.so")

MSA_BF16, MSA_F32, MSA_FP8_E4M3, MSA_FP4_E2M1 = 0, 1, 2, 3
FP4 = torch.float4_e2m1fn_x2   # two OCP e2m1 values per byte, element 2c in the low nibble
MSA_OP_INDEX, MSA_OP_ATTN, MSA_OP_KL, MSA_OP_FORWARD, MSA_OP_ATTN_BWD, MSA_OP_KL_BWD = 0, 1, 2, 3, 4, 5
MSA_OP_DECODE_INDEX, MSA_OP_DECODE_ATTN, MSA_OP_DECODE, MSA_OP_DENSE_ATTN, MSA_OP_DENSE_KL = 6, 7, 8, 9, 10
MSA_OP_FUSED_BWD = 11
STAGE_PREPARE, STAGE_NONLOCAL, STAGE_COMBINE, STAGE_ALL = 1, 2, 4, 7
STATUS = {0: "MSA_OK", 1: "MSA_ERR_NULL", 2: "MSA_ERR_SHAPE", 3: "MSA_ERR_UNSUPPORTED",
          4: "MSA_ERR_ALIGN", 5: "MSA_ERR_WORKSPACE", 6: "MSA_ERR_HIP", 7: "MSA_ERR_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 64 << 20   # MSA_NOALLOC_SCRATCH_BYTES
EXPORTS = ("msa_index_topk", "msa_check_block_idx", "msa_sparse_attn_fwd", "msa_sparse_attn_fwd_stages",
           "msa_forward", "msa_sparse_attn_bwd", "msa_kl_align_fwd", "msa_kl_align_bwd",
           "msa_decode_index_topk", "msa_decode_attn", "msa_decode", "msa_dense_attn_fwd",
           "msa_dense_kl_align_fwd", "msa_decode_paged_index_topk", "msa_decode_paged_attn", "msa_decode_paged",
           "msa_decode_workspace_bytes", "msa_decode_noalloc", "msa_fused_bwd",
           "msa_workspace_bytes", "msa_strerror", "msa_abi_version")


class MsaDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("kv_heads", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("index_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("causal", ctypes.c_int32)]


class MsaError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libmsa.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m block_sparse_gqa_index_amd.build`")
    lib = ctypes.CDLL(path)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    dp = ctypes.POINTER(MsaDims)
    lib.msa_index_topk.argtypes = [dp, vp, vp, vp, vp, sz, vp]
    lib.msa_check_block_idx.argtypes = [dp, vp, vp, vp]
    lib.msa_sparse_attn_fwd.argtypes = [dp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, sz, vp]
    lib.msa_sparse_attn_fwd_stages.argtypes = [dp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, sz,
                                               ctypes.c_int, vp]
    lib.msa_kl_align_fwd.argtypes = [dp, vp, vp, vp, vp, vp, vp, ctypes.c_float, ctypes.c_float,
                                     vp, vp, vp, vp, sz, vp]
    lib.msa_kl_align_bwd.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, ctypes.c_float, vp,
                                     ctypes.c_float, vp, vp, vp, sz, vp]
    lib.msa_forward.argtypes = [dp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp, sz, vp]
    lib.msa_sparse_attn_bwd.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp, sz, vp]
    i32 = ctypes.c_int32
    lib.msa_decode_index_topk.argtypes = [dp, i32, vp, vp, vp, vp, vp, sz, vp]
    lib.msa_decode_attn.argtypes = [dp, i32, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, sz, vp]
    lib.msa_decode.argtypes = [dp, i32, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp, sz, vp]
    lib.msa_decode_noalloc.argtypes = [dp, i32, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp]
    fl = ctypes.c_float
    lib.msa_fused_bwd.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, fl, fl, vp, fl, vp, vp, vp, vp, vp, vp,
                                  sz, vp]
    lib.msa_decode_workspace_bytes.argtypes = [dp, ctypes.c_int, i32]
    lib.msa_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.msa_dense_attn_fwd.argtypes = [dp, vp, vp, vp, ctypes.c_float, vp, vp, vp, sz, vp]
    lib.msa_dense_kl_align_fwd.argtypes = [dp, vp, vp, vp, vp, vp, ctypes.c_float, ctypes.c_float, vp, vp, vp, vp,
                                           sz, vp]
    lib.msa_decode_paged_index_topk.argtypes = [dp, i32, vp, vp, vp, i32, vp, vp, vp, sz, vp]
    lib.msa_decode_paged_attn.argtypes = [dp, i32, vp, vp, vp, vp, i32, vp, vp, ctypes.c_float, vp, vp, vp, sz, vp]
    lib.msa_decode_paged.argtypes = [dp, i32, vp, vp, vp, vp, vp, vp, i32, vp, ctypes.c_float, vp, vp, vp, vp, sz,
                                     vp]
    lib.msa_workspace_bytes.argtypes = [dp, ctypes.c_int]
    lib.msa_workspace_bytes.restype = ctypes.c_size_t
    lib.msa_strerror.argtypes = [ctypes.c_int]
    lib.msa_strerror.restype = ctypes.c_char_p
    lib.msa_abi_version.restype = ctypes.c_int
    for f in (lib.msa_index_topk, lib.msa_check_block_idx, lib.msa_sparse_attn_fwd, lib.msa_sparse_attn_fwd_stages,
              lib.msa_kl_align_fwd, lib.msa_forward, lib.msa_kl_align_bwd, lib.msa_sparse_attn_bwd,
              lib.msa_decode_index_topk, lib.msa_decode_attn, lib.msa_decode, lib.msa_dense_attn_fwd,
              lib.msa_dense_kl_align_fwd, lib.msa_decode_paged_index_topk, lib.msa_decode_paged_attn,
              lib.msa_decode_paged, lib.msa_decode_noalloc, lib.msa_fused_bwd):
        f.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status):
    if status != 0:
        raise MsaError(status, load_library().msa_strerror(status).decode())


def make_dims(batch, seqlen, kv_heads, group_size, head_dim, index_dim, topk, dtype,
              block_size=128, causal=1) -> MsaDims:
    if isinstance(dtype, torch.dtype):
        dtype = {torch.bfloat16: MSA_BF16, torch.float32: MSA_F32,
                 torch.float8_e4m3fn: MSA_FP8_E4M3, FP4: MSA_FP4_E2M1}.get(dtype, -1)
    return MsaDims(batch, seqlen, kv_heads, group_size, head_dim, index_dim, block_size, topk,
                   dtype, causal)


def workspace_bytes(dims: MsaDims, op: int) -> int:
    return int(load_library().msa_workspace_bytes(ctypes.byref(dims), op))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _workspace(nbytes, device, ws):
    if nbytes == 0:
        return None, 0
    if ws is not None:
        _req(ws, "workspace", device=device)
    if ws is None or ws.numel() * ws.element_size() < nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


def _on_gpu(t):
    """Whether t lives in device memory (its own function so that host-only
    tests can stand in for it and reach the shape checks)."""
    return t.is_cuda


def _req(t, name, dtype=None, ndim=None, shape=None, device=None):
    """Checks a tensor argument before anything is enqueued: type, dtype, rank,
    exact shape, contiguity, device memory and (if given) the device the call
    runs on. An output the kernels write must pass `shape`, so that a short
    buffer is refused here instead of being written past its end."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not _on_gpu(t):
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def index_topk(q_idx, k_idx, topk, block_idx=None, block_size=128):
    """Block selection. q_idx [B,N,Hkv,Di], k_idx [B,N,Di] (bf16, fp32 or
    float8_e4m3fn; or float4_e2m1fn_x2 with the last dimension Di/2, two values
    per byte) -> int32 [B,Hkv,N,topk]."""
    lib = load_library()
    _req(q_idx, "q_idx", ndim=4)
    _req(k_idx, "k_idx", dtype=q_idx.dtype, ndim=3)
    B, N, Hkv, Di = q_idx.shape
    if q_idx.dtype == FP4:
        Di *= 2
    if tuple(k_idx.shape) != (B, N, q_idx.shape[3]):
        raise ValueError(f"k_idx shape {tuple(k_idx.shape)} != {(B, N, q_idx.shape[3])}")
    _req(k_idx, "k_idx", device=q_idx.device)
    if block_idx is None:
        block_idx = torch.empty((B, Hkv, N, topk), dtype=torch.int32, device=q_idx.device)
    _req(block_idx, "block_idx", dtype=torch.int32, shape=(B, Hkv, N, topk), device=q_idx.device)
    dims = make_dims(B, N, Hkv, 1, 64, Di, topk, q_idx.dtype, block_size)
    _check(lib.msa_index_topk(ctypes.byref(dims), _ptr(q_idx), _ptr(k_idx), _ptr(block_idx),
                              None, 0, _stream(q_idx.device)))
    return block_idx


def check_block_idx(block_idx, bad_rows=None, block_size=128):
    """Number of rows of block_idx [B, Hkv, N, k] that do not follow the layout
    index_topk writes (int32 [1] on the device, filled on the current stream)."""
    lib = load_library()
    _req(block_idx, "block_idx", dtype=torch.int32, ndim=4)
    B, Hkv, N, topk = block_idx.shape
    if bad_rows is None:
        bad_rows = torch.empty((1,), dtype=torch.int32, device=block_idx.device)
    _req(bad_rows, "bad_rows", dtype=torch.int32, shape=(1,), device=block_idx.device)
    dims = make_dims(B, N, Hkv, 1, 64, 64, topk, MSA_BF16, block_size)
    _check(lib.msa_check_block_idx(ctypes.byref(dims), _ptr(block_idx), _ptr(bad_rows), _stream(block_idx.device)))
    return bad_rows


def sparse_attn_fwd(q, k, v, block_idx, softmax_scale=0.0, o=None, lse=None, workspace=None,
                    block_size=128, stages=STAGE_ALL):
    """Block-sparse GQA attention. q [B,N,Hq,D], k/v [B,N,Hkv,D], block_idx int32
    [B,Hkv,N,topk] -> (o [B,N,Hq,D], lse fp32 [B,Hq,N]). `stages` (a subset of
    STAGE_ALL) enqueues only those stages; the stages of one result must run
    in order on the same workspace, which the caller then passes in."""
    lib = load_library()
    _req(q, "q", ndim=4)
    _req(k, "k", dtype=q.dtype, ndim=4)
    _req(v, "v", dtype=q.dtype, ndim=4)
    _req(block_idx, "block_idx", dtype=torch.int32, ndim=4)
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    if tuple(k.shape) != (B, N, Hkv, D) or tuple(v.shape) != (B, N, Hkv, D) or Hq % Hkv:
        raise ValueError("k/v must be [B, N, Hkv, D] with Hq a multiple of Hkv")
    topk = block_idx.shape[3]
    if tuple(block_idx.shape) != (B, Hkv, N, topk):
        raise ValueError("block_idx must be [B, Hkv, N, topk]")
    for name, t in (("k", k), ("v", v), ("block_idx", block_idx)):
        _req(t, name, device=q.device)
    dims = make_dims(B, N, Hkv, Hq // Hkv, D, 64, topk, q.dtype, block_size)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    _req(o, "o", dtype=q.dtype, shape=q.shape, device=q.device)
    _req(lse, "lse", dtype=torch.float32, shape=(B, Hq, N), device=q.device)
    ws, nws = _workspace(workspace_bytes(dims, MSA_OP_ATTN), q.device, workspace)
    if stages == STAGE_ALL:
        _check(lib.msa_sparse_attn_fwd(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(block_idx),
                                       float(softmax_scale), _ptr(o), _ptr(lse), _ptr(ws), nws,
                                       _stream(q.device)))
    else:
        if stages != STAGE_PREPARE and ws is not None and ws is not workspace:
            raise ValueError("a later stage needs the workspace of the earlier ones: pass workspace=")
        _check(lib.msa_sparse_attn_fwd_stages(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(block_idx),
                                              float(softmax_scale), _ptr(o), _ptr(lse), _ptr(ws), nws,
                                              int(stages), _stream(q.device)))
    return o, lse


def sparse_attn_bwd(q, k, v, block_idx, o, lse, dout, softmax_scale=0.0, dq=None, dk=None, dv=None,
                    workspace=None, block_size=128):
    """Backward of sparse_attn_fwd for the loss <dout, o> (bf16): o and lse
    from the forward of the same inputs -> (dq [B,N,Hq,D], dk, dv [B,N,Hkv,D])."""
    lib = load_library()
    _req(q, "q", ndim=4)
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout)):
        _req(t, name, dtype=q.dtype, ndim=4)
    _req(block_idx, "block_idx", dtype=torch.int32, ndim=4)
    _req(lse, "lse", dtype=torch.float32, ndim=3)
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    if tuple(k.shape) != (B, N, Hkv, D) or tuple(v.shape) != (B, N, Hkv, D) or Hq % Hkv:
        raise ValueError("k/v must be [B, N, Hkv, D] with Hq a multiple of Hkv")
    if tuple(o.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape) or tuple(lse.shape) != (B, Hq, N):
        raise ValueError("o/dout must be [B, N, Hq, D] and lse [B, Hq, N]")
    topk = block_idx.shape[3]
    if tuple(block_idx.shape) != (B, Hkv, N, topk):
        raise ValueError("block_idx must be [B, Hkv, N, topk]")
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout), ("block_idx", block_idx), ("lse", lse)):
        _req(t, name, device=q.device)
    dims = make_dims(B, N, Hkv, Hq // Hkv, D, 64, topk, q.dtype, block_size)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _req(t, name, dtype=q.dtype, shape=ref.shape, device=q.device)
    ws, nws = _workspace(workspace_bytes(dims, MSA_OP_ATTN_BWD), q.device, workspace)
    _check(lib.msa_sparse_attn_bwd(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(block_idx), _ptr(o),
                                   _ptr(lse), _ptr(dout), float(softmax_scale), _ptr(dq), _ptr(dk), _ptr(dv),
                                   _ptr(ws), nws, _stream(q.device)))
    return dq, dk, dv


def _kl_input_shapes(q, k, q_idx, k_idx, lse, block_idx):
    """Shapes and device of the KL calls' inputs (q [B,N,Hq,D] sets B, N, Hq, D;
    q_idx [., ., Hkv, Di] sets Hkv and Di; block_idx sets topk)."""
    B, N, Hq, D = q.shape
    Hkv, Di = q_idx.shape[2], q_idx.shape[3]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    _req(k, "k", shape=(B, N, Hkv, D), device=q.device)
    _req(q_idx, "q_idx", shape=(B, N, Hkv, Di), device=q.device)
    _req(k_idx, "k_idx", shape=(B, N, Di), device=q.device)
    _req(lse, "lse", shape=(B, Hq, N), device=q.device)
    _req(block_idx, "block_idx", shape=(B, Hkv, N, block_idx.shape[3]), device=q.device)


def fused_bwd(q, k, v, q_idx, k_idx, block_idx, o, lse, index_lse, dout, softmax_scale=0.0, index_scale=0.0,
              dkl_rows=None, kl_weight=1.0, dq=None, dk=None, dv=None, dq_idx=None, dk_idx=None, workspace=None,
              block_size=128):
    """Both branches' gradients in one pass (msa_fused_bwd, bf16): the main
    branch's (dq, dk, dv) for <dout, o> and the KL term's (dq_idx, dk_idx) for
    sum_rows w_row KL_row -> (dq, dk, dv, dq_idx, dk_idx). o, lse come from
    sparse_attn_fwd and index_lse from kl_align_fwd on the same inputs."""
    lib = load_library()
    _req(q, "q", ndim=4)
    B, N, Hq, D = q.shape
    Hkv, Di = q_idx.shape[2], q_idx.shape[3]
    _kl_input_shapes(q, k, q_idx, k_idx, lse, block_idx)
    topk = block_idx.shape[3]
    for name, t in (("k", k), ("v", v), ("q_idx", q_idx), ("k_idx", k_idx), ("o", o), ("dout", dout)):
        _req(t, name, dtype=q.dtype)
    _req(v, "v", shape=k.shape, device=q.device)
    _req(o, "o", shape=q.shape, device=q.device)
    _req(dout, "dout", shape=q.shape, device=q.device)
    _req(block_idx, "block_idx", dtype=torch.int32)
    _req(lse, "lse", dtype=torch.float32)
    _req(index_lse, "index_lse", dtype=torch.float32, shape=(B, Hkv, N), device=q.device)
    if dkl_rows is not None:
        _req(dkl_rows, "dkl_rows", dtype=torch.float32, shape=(B, Hkv, N), device=q.device)
    dims = make_dims(B, N, Hkv, Hq // Hkv, D, Di, topk, q.dtype, block_size)
    outs = []
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v), ("dq_idx", dq_idx, q_idx), ("dk_idx", dk_idx, k_idx)):
        t = torch.empty_like(ref) if t is None else t
        _req(t, name, dtype=q.dtype, shape=ref.shape, device=q.device)
        outs.append(t)
    ws, nws = _workspace(workspace_bytes(dims, MSA_OP_FUSED_BWD), q.device, workspace)
    _check(lib.msa_fused_bwd(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(q_idx), _ptr(k_idx), _ptr(block_idx),
                             _ptr(o), _ptr(lse), _ptr(index_lse), _ptr(dout), float(softmax_scale),
                             float(index_scale), _ptr(dkl_rows), float(kl_weight), *[_ptr(t) for t in outs],
                             _ptr(ws), nws, _stream(q.device)))
    return tuple(outs)


def kl_align_fwd(q, k, q_idx, k_idx, block_idx, lse, softmax_scale=0.0, index_scale=0.0,
                 kl_rows=None, kl_sum=None, workspace=None, block_size=128, index_lse=None):
    """KL(group-mean main softmax || index softmax) over the selected tokens,
    per row -> (kl_rows fp32 [B,Hkv,N], kl_sum fp32 [1]); `index_lse` (an fp32
    [B,Hkv,N] tensor, optional) receives the student's LSE per row."""
    lib = load_library()
    _req(q, "q", ndim=4)
    _req(k, "k", dtype=q.dtype, ndim=4)
    _req(q_idx, "q_idx", dtype=q.dtype, ndim=4)
    _req(k_idx, "k_idx", dtype=q.dtype, ndim=3)
    _req(block_idx, "block_idx", dtype=torch.int32, ndim=4)
    _req(lse, "lse", dtype=torch.float32, ndim=3)
    B, N, Hq, D = q.shape
    Hkv, Di = q_idx.shape[2], q_idx.shape[3]
    topk = block_idx.shape[3]
    _kl_input_shapes(q, k, q_idx, k_idx, lse, block_idx)
    dims = make_dims(B, N, Hkv, Hq // Hkv, D, Di, topk, q.dtype, block_size)
    if kl_rows is None:
        kl_rows = torch.empty((B, Hkv, N), dtype=torch.float32, device=q.device)
    if kl_sum is None:
        kl_sum = torch.empty((1,), dtype=torch.float32, device=q.device)
    _req(kl_rows, "kl_rows", dtype=torch.float32, shape=(B, Hkv, N), device=q.device)
    _req(kl_sum, "kl_sum", dtype=torch.float32, shape=(1,), device=q.device)
    if index_lse is not None:
        _req(index_lse, "index_lse", dtype=torch.float32, shape=(B, Hkv, N), device=q.device)
    ws, nws = _workspace(workspace_bytes(dims, MSA_OP_KL), q.device, workspace)
    _check(lib.msa_kl_align_fwd(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(q_idx), _ptr(k_idx),
                                _ptr(block_idx), _ptr(lse), float(softmax_scale), float(index_scale),
                                _ptr(kl_rows), _ptr(kl_sum), _ptr(index_lse), _ptr(ws), nws, _stream(q.device)))
    return kl_rows, kl_sum


def kl_align_bwd(q, k, q_idx, k_idx, block_idx, lse, index_lse, softmax_scale=0.0, index_scale=0.0,
                 dkl_rows=None, kl_weight=1.0, dq_idx=None, dk_idx=None, workspace=None, block_size=128):
    """Gradients of sum_rows w_row KL_row (w_row = kl_weight * dkl_rows, or
    kl_weight) w.r.t. q_idx and k_idx, the teacher held fixed (bf16) ->
    (dq_idx [B,N,Hkv,Di], dk_idx [B,N,Di]). lse and index_lse come from the
    forward of the same inputs."""
    lib = load_library()
    _req(q, "q", ndim=4)
    _req(k, "k", dtype=q.dtype, ndim=4)
    _req(q_idx, "q_idx", dtype=q.dtype, ndim=4)
    _req(k_idx, "k_idx", dtype=q.dtype, ndim=3)
    _req(block_idx, "block_idx", dtype=torch.int32, ndim=4)
    _req(lse, "lse", dtype=torch.float32, ndim=3)
    _req(index_lse, "index_lse", dtype=torch.float32, ndim=3)
    B, N, Hq, D = q.shape
    Hkv, Di = q_idx.shape[2], q_idx.shape[3]
    topk = block_idx.shape[3]
    _kl_input_shapes(q, k, q_idx, k_idx, lse, block_idx)
    _req(index_lse, "index_lse", shape=(B, Hkv, N), device=q.device)
    if dkl_rows is not None:
        _req(dkl_rows, "dkl_rows", dtype=torch.float32, shape=(B, Hkv, N), device=q.device)
    dims = make_dims(B, N, Hkv, Hq // Hkv, D, Di, topk, q.dtype, block_size)
    dq_idx = torch.empty_like(q_idx) if dq_idx is None else dq_idx
    dk_idx = torch.empty_like(k_idx) if dk_idx is None else dk_idx
    _req(dq_idx, "dq_idx", dtype=q.dtype, shape=q_idx.shape, device=q.device)
    _req(dk_idx, "dk_idx", dtype=q.dtype, shape=k_idx.shape, device=q.device)
    ws, nws = _workspace(workspace_bytes(dims, MSA_OP_KL_BWD), q.device, workspace)
    _check(lib.msa_kl_align_bwd(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(q_idx), _ptr(k_idx), _ptr(block_idx),
                                _ptr(lse), _ptr(index_lse), float(softmax_scale), float(index_scale),
                                _ptr(dkl_rows), float(kl_weight), _ptr(dq_idx), _ptr(dk_idx), _ptr(ws), nws,
                                _stream(q.device)))
    return dq_idx, dk_idx


def forward(q_idx, k_idx, q, k, v, topk, softmax_scale=0.0, block_idx=None, o=None, lse=None,
            workspace=None, block_size=128):
    """The whole hot path (msa_forward): the selection, then the sparse
    attention on the same stream. Returns (block_idx int32 [B,Hkv,N,topk], o [B,N,Hq,D], lse fp32 [B,Hq,N])."""
    lib = load_library()
    _req(q_idx, "q_idx", ndim=4)
    _req(k_idx, "k_idx", dtype=q_idx.dtype, ndim=3)
    _req(q, "q", dtype=q_idx.dtype, ndim=4)
    _req(k, "k", dtype=q.dtype, ndim=4)
    _req(v, "v", dtype=q.dtype, ndim=4)
    B, N, Hq, D = q.shape
    Hkv, Di = q_idx.shape[2], q_idx.shape[3]
    if (tuple(k_idx.shape) != (B, N, Di) or tuple(k.shape) != (B, N, Hkv, D) or tuple(v.shape) != (B, N, Hkv, D)
            or tuple(q_idx.shape[:2]) != (B, N) or Hq % Hkv):
        raise ValueError("inconsistent shapes")
    dims = make_dims(B, N, Hkv, Hq // Hkv, D, Di, topk, q.dtype, block_size)
    if block_idx is None:
        block_idx = torch.empty((B, Hkv, N, topk), dtype=torch.int32, device=q.device)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    for name, t in (("q_idx", q_idx), ("k_idx", k_idx), ("k", k), ("v", v)):
        _req(t, name, device=q.device)
    _req(block_idx, "block_idx", dtype=torch.int32, shape=(B, Hkv, N, topk), device=q.device)
    _req(o, "o", dtype=q.dtype, shape=q.shape, device=q.device)
    _req(lse, "lse", dtype=torch.float32, shape=(B, Hq, N), device=q.device)
    ws, nws = _workspace(workspace_bytes(dims, MSA_OP_FORWARD), q.device, workspace)
    _check(lib.msa_forward(ctypes.byref(dims), _ptr(q_idx), _ptr(k_idx), _ptr(q), _ptr(k), _ptr(v),
                           float(softmax_scale), _ptr(block_idx), _ptr(o), _ptr(lse), _ptr(ws), nws,
                           _stream(q.device)))
    return block_idx, o, lse


def _rows(t, name, inner):
    """Decode query tensor: [B, inner...] (one new token) or [B, R, inner...];
    returns R and whether the R axis is present."""
    _req(t, name)
    if t.dim() == 1 + inner:
        return 1, False
    if t.dim() == 2 + inner:
        return t.shape[1], True
    raise ValueError(f"{name} must have {1 + inner} or {2 + inner} dimensions")


def _decode_outputs(B, R, multi, Hkv, Hq, D, topk, like, block_idx, o, lse, want_sel=True, want_attn=True):
    dev = like.device
    if want_sel and block_idx is None:
        block_idx = torch.empty((B, Hkv, R, topk) if multi else (B, Hkv, topk), dtype=torch.int32, device=dev)
    if want_attn:
        if o is None:
            o = torch.empty((B, R, Hq, D) if multi else (B, Hq, D), dtype=like.dtype, device=dev)
        if lse is None:
            lse = torch.empty((B, Hq, R) if multi else (B, Hq), dtype=torch.float32, device=dev)
    return block_idx, o, lse


def _check_sel(block_idx, B, Hkv, R, multi, device, topk=None):
    """block_idx of a decode call: [B, Hkv, (R,) topk] int32 on `device`
    (topk = the call's argument when it has one, else the tensor's last
    dimension). Returns topk."""
    _req(block_idx, "block_idx", dtype=torch.int32)
    want = (B, Hkv, R) if multi else (B, Hkv)
    k = block_idx.shape[-1] if topk is None else int(topk)
    _req(block_idx, "block_idx", shape=want + (k,), device=device)
    return k


def _check_decode_out(o, lse, B, R, multi, Hq, D, dtype, device):
    _req(o, "o", dtype=dtype, shape=(B, R, Hq, D) if multi else (B, Hq, D), device=device)
    _req(lse, "lse", dtype=torch.float32, shape=(B, Hq, R) if multi else (B, Hq), device=device)


def decode_workspace_bytes(dims: MsaDims, op: int, num_queries: int = 1) -> int:
    return int(load_library().msa_decode_workspace_bytes(ctypes.byref(dims), op, num_queries))


def decode_index_topk(q_idx, k_idx, seqlens, topk, block_idx=None, workspace=None, block_size=128):
    """Selection for the new queries of each sequence: q_idx [B, Hkv, Di] (one
    new token) or [B, R, Hkv, Di] (R new tokens, the r-th at position
    n_b - R + r), index-key cache k_idx [B, C, Di], seqlens int32 [B] (cached
    tokens, the new ones included) -> block_idx int32 [B, Hkv, topk] or
    [B, Hkv, R, topk]."""
    lib = load_library()
    R, multi = _rows(q_idx, "q_idx", 2)
    _req(k_idx, "k_idx", dtype=q_idx.dtype, ndim=3)
    _req(seqlens, "seqlens", dtype=torch.int32, ndim=1)
    B, C, Di = k_idx.shape
    Hkv = q_idx.shape[-2]
    if q_idx.shape[0] != B or q_idx.shape[-1] != Di or seqlens.shape[0] != B:
        raise ValueError("q_idx must be [B, (R,) Hkv, Di], k_idx [B, C, Di], seqlens [B]")
    for name, t in (("k_idx", k_idx), ("seqlens", seqlens)):
        _req(t, name, device=q_idx.device)
    block_idx, _, _ = _decode_outputs(B, R, multi, Hkv, 0, 0, topk, q_idx, block_idx, None, None, want_attn=False)
    _check_sel(block_idx, B, Hkv, R, multi, q_idx.device, topk)
    dims = make_dims(B, C, Hkv, 1, 64, Di, topk, q_idx.dtype, block_size)
    ws, nws = _workspace(decode_workspace_bytes(dims, MSA_OP_DECODE_INDEX, R), q_idx.device, workspace)
    _check(lib.msa_decode_index_topk(ctypes.byref(dims), R, _ptr(q_idx), _ptr(k_idx), _ptr(seqlens),
                                     _ptr(block_idx), _ptr(ws), nws, _stream(q_idx.device)))
    return block_idx


def decode_attn(q, k, v, seqlens, block_idx, softmax_scale=0.0, o=None, lse=None, workspace=None,
                block_size=128):
    """Attention of the new queries of each sequence: q [B, Hq, D] or
    [B, R, Hq, D], caches k/v [B, C, Hkv, D], seqlens int32 [B], block_idx
    int32 [B, Hkv, (R,) topk] -> (o like q, lse fp32 [B, Hq] or [B, Hq, R])."""
    lib = load_library()
    R, multi = _rows(q, "q", 2)
    _req(k, "k", dtype=q.dtype, ndim=4)
    _req(v, "v", dtype=q.dtype, ndim=4)
    _req(seqlens, "seqlens", dtype=torch.int32, ndim=1)
    B, C, Hkv, D = k.shape
    Hq = q.shape[-2]
    if (tuple(v.shape) != tuple(k.shape) or q.shape[0] != B or q.shape[-1] != D or Hq % Hkv
            or seqlens.shape[0] != B):
        raise ValueError("q must be [B, (R,) Hq, D] with Hq a multiple of Hkv; k, v [B, C, Hkv, D]")
    for name, t in (("k", k), ("v", v), ("seqlens", seqlens)):
        _req(t, name, device=q.device)
    topk = _check_sel(block_idx, B, Hkv, R, multi, q.device)
    _, o, lse = _decode_outputs(B, R, multi, Hkv, Hq, D, topk, q, None, o, lse, want_sel=False)
    _check_decode_out(o, lse, B, R, multi, Hq, D, q.dtype, q.device)
    dims = make_dims(B, C, Hkv, Hq // Hkv, D, 64, topk, q.dtype, block_size)
    ws, nws = _workspace(decode_workspace_bytes(dims, MSA_OP_DECODE_ATTN, R), q.device, workspace)
    _check(lib.msa_decode_attn(ctypes.byref(dims), R, _ptr(q), _ptr(k), _ptr(v), _ptr(seqlens), _ptr(block_idx),
                               float(softmax_scale), _ptr(o), _ptr(lse), _ptr(ws), nws, _stream(q.device)))
    return o, lse


def decode(q_idx, k_idx, q, k, v, seqlens, topk, softmax_scale=0.0, block_idx=None, o=None, lse=None,
           workspace=None, block_size=128):
    """One decode step (msa_decode): the selection, then the attention.
    Returns (block_idx, o, lse) in the layouts of decode_index_topk and decode_attn."""
    lib = load_library()
    R, multi = _rows(q_idx, "q_idx", 2)
    R2, multi2 = _rows(q, "q", 2)
    if (R2, multi2) != (R, multi) or q.dtype != q_idx.dtype:
        raise ValueError("q and q_idx must have the same new-query axis and dtype")
    _req(k_idx, "k_idx", dtype=q.dtype, ndim=3)
    _req(k, "k", dtype=q.dtype, ndim=4)
    _req(v, "v", dtype=q.dtype, ndim=4)
    _req(seqlens, "seqlens", dtype=torch.int32, ndim=1)
    B, C, Hkv, D = k.shape
    Di, Hq = k_idx.shape[2], q.shape[-2]
    if (tuple(k_idx.shape[:2]) != (B, C) or tuple(v.shape) != tuple(k.shape) or q_idx.shape[-2:] != (Hkv, Di)
            or q.shape[-1] != D or Hq % Hkv or seqlens.shape[0] != B):
        raise ValueError("inconsistent shapes")
    if q_idx.shape[0] != B or q.shape[0] != B:
        raise ValueError("q_idx and q must have the caches' batch")
    for name, t in (("q_idx", q_idx), ("k_idx", k_idx), ("k", k), ("v", v), ("seqlens", seqlens)):
        _req(t, name, device=q.device)
    block_idx, o, lse = _decode_outputs(B, R, multi, Hkv, Hq, D, topk, q, block_idx, o, lse)
    _check_sel(block_idx, B, Hkv, R, multi, q.device, topk)
    _check_decode_out(o, lse, B, R, multi, Hq, D, q.dtype, q.device)
    dims = make_dims(B, C, Hkv, Hq // Hkv, D, Di, topk, q.dtype, block_size)
    ws, nws = _workspace(decode_workspace_bytes(dims, MSA_OP_DECODE, R), q.device, workspace)
    _check(lib.msa_decode(ctypes.byref(dims), R, _ptr(q_idx), _ptr(k_idx), _ptr(q), _ptr(k), _ptr(v), _ptr(seqlens),
                          float(softmax_scale), _ptr(block_idx), _ptr(o), _ptr(lse), _ptr(ws), nws,
                          _stream(q.device)))
    return block_idx, o, lse


def decode_noalloc(q_idx, k_idx, q, k, v, seqlens, topk, softmax_scale=0.0, block_idx=None, o=None, lse=None,
                   block_size=128):
    """decode() through msa_decode_noalloc: the library's fixed scratch array
    (64 MiB per GPU) instead of a workspace; the library allocates nothing
    (the outputs, if not given, are still allocated here by torch). Calls that
    overlap on one GPU race on that array."""
    lib = load_library()
    R, multi = _rows(q_idx, "q_idx", 2)
    R2, multi2 = _rows(q, "q", 2)
    if (R2, multi2) != (R, multi) or q.dtype != q_idx.dtype:
        raise ValueError("q and q_idx must have the same new-query axis and dtype")
    _req(k_idx, "k_idx", dtype=q.dtype, ndim=3)
    _req(k, "k", dtype=q.dtype, ndim=4)
    _req(v, "v", dtype=q.dtype, ndim=4)
    _req(seqlens, "seqlens", dtype=torch.int32, ndim=1)
    B, C, Hkv, D = k.shape
    Di, Hq = k_idx.shape[2], q.shape[-2]
    if (tuple(k_idx.shape[:2]) != (B, C) or tuple(v.shape) != tuple(k.shape) or q_idx.shape[-2:] != (Hkv, Di)
            or q.shape[-1] != D or Hq % Hkv or seqlens.shape[0] != B or q_idx.shape[0] != B or q.shape[0] != B):
        raise ValueError("inconsistent shapes")
    for name, t in (("q_idx", q_idx), ("k_idx", k_idx), ("k", k), ("v", v), ("seqlens", seqlens)):
        _req(t, name, device=q.device)
    block_idx, o, lse = _decode_outputs(B, R, multi, Hkv, Hq, D, topk, q, block_idx, o, lse)
    _check_sel(block_idx, B, Hkv, R, multi, q.device, topk)
    _check_decode_out(o, lse, B, R, multi, Hq, D, q.dtype, q.device)
    dims = make_dims(B, C, Hkv, Hq // Hkv, D, Di, topk, q.dtype, block_size)
    _check(lib.msa_decode_noalloc(ctypes.byref(dims), R, _ptr(q_idx), _ptr(k_idx), _ptr(q), _ptr(k), _ptr(v),
                                  _ptr(seqlens), float(softmax_scale), _ptr(block_idx), _ptr(o), _ptr(lse),
                                  _stream(q.device)))
    return block_idx, o, lse


def dense_attn_fwd(q, k, v, softmax_scale=0.0, o=None, lse=None, workspace=None, block_size=128):
    """Dense causal GQA attention (the warm-up's full attention): q [B,N,Hq,D],
    k/v [B,N,Hkv,D] -> (o [B,N,Hq,D], lse fp32 [B,Hq,N])."""
    lib = load_library()
    _req(q, "q", ndim=4)
    _req(k, "k", dtype=q.dtype, ndim=4)
    _req(v, "v", dtype=q.dtype, ndim=4)
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    if tuple(k.shape) != (B, N, Hkv, D) or tuple(v.shape) != (B, N, Hkv, D) or Hq % Hkv:
        raise ValueError("k/v must be [B, N, Hkv, D] with Hq a multiple of Hkv")
    for name, t in (("k", k), ("v", v)):
        _req(t, name, device=q.device)
    dims = make_dims(B, N, Hkv, Hq // Hkv, D, 64, 1, q.dtype, block_size)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    _req(o, "o", dtype=q.dtype, shape=q.shape, device=q.device)
    _req(lse, "lse", dtype=torch.float32, shape=(B, Hq, N), device=q.device)
    ws, nws = _workspace(workspace_bytes(dims, MSA_OP_DENSE_ATTN), q.device, workspace)
    _check(lib.msa_dense_attn_fwd(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), float(softmax_scale), _ptr(o),
                                  _ptr(lse), _ptr(ws), nws, _stream(q.device)))
    return o, lse


def dense_kl_align_fwd(q, k, q_idx, k_idx, lse, softmax_scale=0.0, index_scale=0.0, kl_rows=None, kl_sum=None,
                       index_lse=None, workspace=None, block_size=128):
    """The warm-up's KL loss over every visible token (lse from dense_attn_fwd)
    -> (kl_rows fp32 [B,Hkv,N], kl_sum fp32 [1])."""
    lib = load_library()
    _req(q, "q", ndim=4)
    _req(k, "k", dtype=q.dtype, ndim=4)
    _req(q_idx, "q_idx", dtype=q.dtype, ndim=4)
    _req(k_idx, "k_idx", dtype=q.dtype, ndim=3)
    _req(lse, "lse", dtype=torch.float32, ndim=3)
    B, N, Hq, D = q.shape
    Hkv, Di = q_idx.shape[2], q_idx.shape[3]
    if (tuple(k.shape) != (B, N, Hkv, D) or tuple(k_idx.shape) != (B, N, Di) or tuple(lse.shape) != (B, Hq, N)
            or Hq % Hkv):
        raise ValueError("inconsistent shapes")
    for name, t in (("k", k), ("q_idx", q_idx), ("k_idx", k_idx), ("lse", lse)):
        _req(t, name, device=q.device)
    if tuple(q_idx.shape[:2]) != (B, N):
        raise ValueError("q_idx must be [B, N, Hkv, Di]")
    dims = make_dims(B, N, Hkv, Hq // Hkv, D, Di, 1, q.dtype, block_size)
    if kl_rows is None:
        kl_rows = torch.empty((B, Hkv, N), dtype=torch.float32, device=q.device)
    if kl_sum is None:
        kl_sum = torch.empty((1,), dtype=torch.float32, device=q.device)
    _req(kl_rows, "kl_rows", dtype=torch.float32, shape=(B, Hkv, N), device=q.device)
    _req(kl_sum, "kl_sum", dtype=torch.float32, shape=(1,), device=q.device)
    if index_lse is not None:
        _req(index_lse, "index_lse", dtype=torch.float32, shape=(B, Hkv, N), device=q.device)
    ws, nws = _workspace(workspace_bytes(dims, MSA_OP_DENSE_KL), q.device, workspace)
    _check(lib.msa_dense_kl_align_fwd(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(q_idx), _ptr(k_idx), _ptr(lse),
                                      float(softmax_scale), float(index_scale), _ptr(kl_rows), _ptr(kl_sum),
                                      _ptr(index_lse), _ptr(ws), nws, _stream(q.device)))
    return kl_rows, kl_sum


def _paged_shapes(block_table, seqlens, k_idx_pages=None, k_pages=None, v_pages=None):
    _req(block_table, "block_table", dtype=torch.int32, ndim=2)
    _req(seqlens, "seqlens", dtype=torch.int32, ndim=1)
    B, MB = block_table.shape
    if seqlens.shape[0] != B:
        raise ValueError("seqlens must be [B] with B = block_table.shape[0]")
    P = None
    if k_idx_pages is not None:
        _req(k_idx_pages, "k_idx_pages", ndim=3)
        if k_idx_pages.shape[1] != 128:
            raise ValueError("k_idx_pages must be [P, 128, Di]")
        P = k_idx_pages.shape[0]
    if k_pages is not None:
        _req(k_pages, "k_pages", ndim=4)
        _req(v_pages, "v_pages", dtype=k_pages.dtype, ndim=4)
        if k_pages.shape[1] != 128 or tuple(v_pages.shape) != tuple(k_pages.shape):
            raise ValueError("k_pages and v_pages must be [P, 128, Hkv, D]")
        if P is not None and k_pages.shape[0] != P:
            raise ValueError("the page pools must hold the same number of pages")
        P = k_pages.shape[0]
    return B, MB * 128, P


def decode_paged_index_topk(q_idx, k_idx_pages, block_table, seqlens, topk, block_idx=None, workspace=None):
    """decode_index_topk on a paged index-key cache: k_idx_pages [P, 128, Di],
    block_table int32 [B, max_blocks] (page of each block)."""
    lib = load_library()
    B, C, P = _paged_shapes(block_table, seqlens, k_idx_pages=k_idx_pages)
    R, multi = _rows(q_idx, "q_idx", 2)
    Hkv, Di = q_idx.shape[-2], q_idx.shape[-1]
    if q_idx.dtype != k_idx_pages.dtype or q_idx.shape[0] != B or k_idx_pages.shape[2] != Di:
        raise ValueError("q_idx must be [B, (R,) Hkv, Di] in the pool's dtype")
    for name, t in (("k_idx_pages", k_idx_pages), ("block_table", block_table), ("seqlens", seqlens)):
        _req(t, name, device=q_idx.device)
    block_idx, _, _ = _decode_outputs(B, R, multi, Hkv, 0, 0, topk, q_idx, block_idx, None, None, want_attn=False)
    _check_sel(block_idx, B, Hkv, R, multi, q_idx.device, topk)
    dims = make_dims(B, C, Hkv, 1, 64, Di, topk, q_idx.dtype)
    ws, nws = _workspace(decode_workspace_bytes(dims, MSA_OP_DECODE_INDEX, R), q_idx.device, workspace)
    _check(lib.msa_decode_paged_index_topk(ctypes.byref(dims), R, _ptr(q_idx), _ptr(k_idx_pages), _ptr(block_table),
                                           P, _ptr(seqlens), _ptr(block_idx), _ptr(ws), nws, _stream(q_idx.device)))
    return block_idx


def decode_paged_attn(q, k_pages, v_pages, block_table, seqlens, block_idx, softmax_scale=0.0, o=None, lse=None,
                      workspace=None):
    """decode_attn on paged K/V caches [P, 128, Hkv, D]."""
    lib = load_library()
    B, C, P = _paged_shapes(block_table, seqlens, k_pages=k_pages, v_pages=v_pages)
    R, multi = _rows(q, "q", 2)
    Hkv, D = k_pages.shape[2], k_pages.shape[3]
    Hq = q.shape[-2]
    if q.dtype != k_pages.dtype or q.shape[0] != B or q.shape[-1] != D or Hq % Hkv:
        raise ValueError("q must be [B, (R,) Hq, D] with Hq a multiple of Hkv")
    for name, t in (("k_pages", k_pages), ("v_pages", v_pages), ("block_table", block_table), ("seqlens", seqlens)):
        _req(t, name, device=q.device)
    topk = _check_sel(block_idx, B, Hkv, R, multi, q.device)
    _, o, lse = _decode_outputs(B, R, multi, Hkv, Hq, D, topk, q, None, o, lse, want_sel=False)
    _check_decode_out(o, lse, B, R, multi, Hq, D, q.dtype, q.device)
    dims = make_dims(B, C, Hkv, Hq // Hkv, D, 64, topk, q.dtype)
    ws, nws = _workspace(decode_workspace_bytes(dims, MSA_OP_DECODE_ATTN, R), q.device, workspace)
    _check(lib.msa_decode_paged_attn(ctypes.byref(dims), R, _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table),
                                     P, _ptr(seqlens), _ptr(block_idx), float(softmax_scale), _ptr(o), _ptr(lse),
                                     _ptr(ws), nws, _stream(q.device)))
    return o, lse


def decode_paged(q_idx, k_idx_pages, q, k_pages, v_pages, block_table, seqlens, topk, softmax_scale=0.0,
                 block_idx=None, o=None, lse=None, workspace=None):
    """One decode step on paged caches (msa_decode_paged) -> (block_idx, o, lse)."""
    lib = load_library()
    B, C, P = _paged_shapes(block_table, seqlens, k_idx_pages=k_idx_pages, k_pages=k_pages, v_pages=v_pages)
    R, multi = _rows(q_idx, "q_idx", 2)
    R2, multi2 = _rows(q, "q", 2)
    if (R2, multi2) != (R, multi) or q.dtype != q_idx.dtype or q.dtype != k_pages.dtype:
        raise ValueError("q and q_idx must have the same new-query axis and dtype")
    Hkv, Di, D = q_idx.shape[-2], q_idx.shape[-1], k_pages.shape[3]
    Hq = q.shape[-2]
    if k_pages.shape[2] != Hkv or Hq % Hkv or q.shape[-1] != D:
        raise ValueError("inconsistent shapes")
    if q_idx.shape[0] != B or q.shape[0] != B or k_idx_pages.shape[2] != Di:
        raise ValueError("q_idx and q must have the block table's batch, k_idx_pages the index dim of q_idx")
    for name, t in (("q_idx", q_idx), ("k_idx_pages", k_idx_pages), ("k_pages", k_pages), ("v_pages", v_pages),
                    ("block_table", block_table), ("seqlens", seqlens)):
        _req(t, name, device=q.device)
    block_idx, o, lse = _decode_outputs(B, R, multi, Hkv, Hq, D, topk, q, block_idx, o, lse)
    _check_sel(block_idx, B, Hkv, R, multi, q.device, topk)
    _check_decode_out(o, lse, B, R, multi, Hq, D, q.dtype, q.device)
    dims = make_dims(B, C, Hkv, Hq // Hkv, D, Di, topk, q.dtype)
    ws, nws = _workspace(decode_workspace_bytes(dims, MSA_OP_DECODE, R), q.device, workspace)
    _check(lib.msa_decode_paged(ctypes.byref(dims), R, _ptr(q_idx), _ptr(k_idx_pages), _ptr(q), _ptr(k_pages),
                                _ptr(v_pages), _ptr(block_table), P, _ptr(seqlens), float(softmax_scale),
                                _ptr(block_idx), _ptr(o), _ptr(lse), _ptr(ws), nws, _stream(q.device)))
    return block_idx, o, lse
