"""The C ABI library on the host (no GPU needed): it loads, exports every
function include/msa.h declares, and rejects bad arguments with the documented
status before touching the device."""
import ctypes
import os
import re
import subprocess

import pytest

import block_sparse_gqa_index_amd as msa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(msa.LIB_PATH):
        from block_sparse_gqa_index_amd import build
        build.build()
    return msa.load_library()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^MSA_API\s+[\w\s\*]*?\b(msa_\w+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    assert _declared() == sorted(msa.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", msa.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in _declared():
        assert name in exported, name
        assert hasattr(lib, name)
    # nothing but the C ABI is exported
    assert {n for n in exported if not n.startswith("_")} == set(_declared())


def test_version_and_strings(lib):
    assert lib.msa_abi_version() == 6
    for s in range(8):
        assert lib.msa_strerror(s)
    assert lib.msa_strerror(99) == b"unknown status"


def _dims(**kw):
    base = dict(batch=1, seqlen=1024, kv_heads=2, group_size=4, head_dim=128, index_dim=64,
                topk=16, dtype=msa.MSA_BF16)
    base.update(kw)
    return msa.make_dims(**base)


FAKE = ctypes.c_void_p(0x1000)      # aligned, never dereferenced: every call below is rejected
MISALIGNED = ctypes.c_void_p(0x1008)


def _index(lib, d, q=FAKE, k=FAKE, out=FAKE):
    return lib.msa_index_topk(ctypes.byref(d), q, k, out, None, 0, None)


def _attn(lib, d, ptrs=None, ws=None, nws=0):
    p = dict(q=FAKE, k=FAKE, v=FAKE, bi=FAKE, o=FAKE, lse=FAKE)
    p.update(ptrs or {})
    return lib.msa_sparse_attn_fwd(ctypes.byref(d), p["q"], p["k"], p["v"], p["bi"], 0.0,
                                   p["o"], p["lse"], ws, nws, None)


def _kl(lib, d, ptrs=None, ws=None, nws=0):
    p = dict(q=FAKE, k=FAKE, qi=FAKE, ki=FAKE, bi=FAKE, lse=FAKE, rows=FAKE, sum=FAKE)
    p.update(ptrs or {})
    return lib.msa_kl_align_fwd(ctypes.byref(d), p["q"], p["k"], p["qi"], p["ki"], p["bi"], p["lse"],
                                0.0, 0.0, p["rows"], p["sum"], p.get("ilse"), ws, nws, None)


@pytest.mark.parametrize("kw,status", [
    (dict(block_size=96), 3), (dict(block_size=512), 3), (dict(block_size=64, dtype=msa.MSA_FP8_E4M3), 3),
    (dict(block_size=256, dtype=msa.MSA_FP4_E2M1), 3), (dict(topk=0), 2), (dict(topk=33), 3), (dict(dtype=7), 3),
    (dict(causal=0), 3), (dict(index_dim=96), 3), (dict(kv_heads=0), 2), (dict(seqlen=-1), 2),
    (dict(batch=-2), 2), (dict(seqlen=1 << 26), 2),
])
def test_index_rejects_bad_dims(lib, kw, status):
    assert _index(lib, _dims(**kw)) == status


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), 3), (dict(group_size=3), 3), (dict(group_size=64), 3),
    (dict(block_size=256, topk=17), 3), (dict(block_size=96), 3), (dict(block_size=64, dtype=msa.MSA_FP8_E4M3), 3),
    (dict(topk=40), 3), (dict(group_size=0), 2),
    # (batch, group, 64K-position window, key block) keys past 2^31 - 1
    (dict(kv_heads=16, seqlen=1 << 25, topk=2), 2),
])
def test_attention_rejects_bad_dims(lib, kw, status):
    assert _attn(lib, _dims(**kw)) == status


def test_fp8_is_for_the_selection_only(lib):
    d = _dims(dtype=msa.MSA_FP8_E4M3)
    assert _index(lib, d, out=None) == 1          # accepted: goes on to the pointer checks
    assert _attn(lib, d) == 3
    assert _kl(lib, d) == 3
    p = [FAKE] * 5
    assert lib.msa_forward(ctypes.byref(d), *p, 0.0, FAKE, FAKE, FAKE, None, 0, None) == 3
    assert lib.msa_check_block_idx(ctypes.byref(d), FAKE, None, None) == 1


def _bwd(lib, d, ptrs=None, ws=FAKE, nws=1 << 50):
    p = dict(q=FAKE, k=FAKE, v=FAKE, bi=FAKE, o=FAKE, lse=FAKE, do=FAKE, dq=FAKE, dk=FAKE, dv=FAKE)
    p.update(ptrs or {})
    return lib.msa_sparse_attn_bwd(ctypes.byref(d), p["q"], p["k"], p["v"], p["bi"], p["o"], p["lse"], p["do"],
                                   0.0, p["dq"], p["dk"], p["dv"], ws, nws, None)


def test_backward_rejects_before_any_launch(lib):
    d = _dims()
    need = lib.msa_workspace_bytes(ctypes.byref(d), msa.MSA_OP_ATTN_BWD)
    assert need > lib.msa_workspace_bytes(ctypes.byref(d), msa.MSA_OP_ATTN) > 0
    assert _bwd(lib, _dims(dtype=msa.MSA_F32)) == 3              # bf16 only
    assert lib.msa_workspace_bytes(ctypes.byref(_dims(dtype=msa.MSA_F32)), msa.MSA_OP_ATTN_BWD) == 0
    assert _bwd(lib, _dims(dtype=msa.MSA_FP8_E4M3)) == 3
    assert _bwd(lib, _dims(head_dim=96)) == 3
    assert _bwd(lib, _dims(index_dim=96), ws=None, nws=0) == 5   # index_dim is not read
    for name in ("q", "k", "v", "bi", "o", "lse", "do", "dq", "dk", "dv"):
        assert _bwd(lib, d, ptrs={name: None}) == 1, name
        assert _bwd(lib, d, ptrs={name: MISALIGNED}) == 4, name
    assert _bwd(lib, d, ws=None, nws=0) == 5
    assert _bwd(lib, d, nws=need - 1) == 5
    assert _bwd(lib, d, ws=MISALIGNED, nws=need) == 5
    none = {n: None for n in ("q", "k", "v", "bi", "o", "lse", "do", "dq", "dk", "dv")}
    assert _bwd(lib, _dims(batch=0), ptrs=none, ws=None, nws=0) == 0
    assert _bwd(lib, _dims(seqlen=0), ptrs=none, ws=None, nws=0) == 0


def _klb(lib, d, ptrs=None, ws=FAKE, nws=1 << 50):
    p = dict(q=FAKE, k=FAKE, qi=FAKE, ki=FAKE, bi=FAKE, lse=FAKE, ilse=FAKE, w=None, dqi=FAKE, dki=FAKE)
    p.update(ptrs or {})
    return lib.msa_kl_align_bwd(ctypes.byref(d), p["q"], p["k"], p["qi"], p["ki"], p["bi"], p["lse"], p["ilse"],
                                0.0, 0.0, p["w"], 1.0, p["dqi"], p["dki"], ws, nws, None)


def test_kl_backward_rejects_before_any_launch(lib):
    d = _dims()
    need = lib.msa_workspace_bytes(ctypes.byref(d), msa.MSA_OP_KL_BWD)
    assert need > 0
    assert _klb(lib, _dims(dtype=msa.MSA_F32)) == 3
    assert _klb(lib, _dims(index_dim=96)) == 3
    for name in ("q", "k", "qi", "ki", "bi", "lse", "ilse", "dqi", "dki"):
        assert _klb(lib, d, ptrs={name: None}) == 1, name
        assert _klb(lib, d, ptrs={name: MISALIGNED}) == 4, name
    assert _klb(lib, d, ptrs={"w": MISALIGNED}) == 4
    assert _klb(lib, d, ws=None, nws=0) == 5
    assert _klb(lib, d, nws=need - 1) == 5
    none = {n: None for n in ("q", "k", "qi", "ki", "bi", "lse", "ilse", "dqi", "dki")}
    assert _klb(lib, _dims(seqlen=0), ptrs=none, ws=None, nws=0) == 0
    # the forward's optional student-LSE output: 4-byte alignment only
    assert _kl(lib, _dims(), ptrs={"ilse": ctypes.c_void_p(0x1002)}) == 4


def test_index_ignores_attention_fields(lib):
    # group_size/head_dim are not read by the selection: the call goes on to
    # the pointer checks (NULL output -> MSA_ERR_NULL, not UNSUPPORTED)
    assert _index(lib, _dims(group_size=3, head_dim=7), out=None) == 1


def test_null_and_alignment(lib):
    d = _dims()
    assert lib.msa_index_topk(None, FAKE, FAKE, FAKE, None, 0, None) == 1
    assert _index(lib, d, q=None) == 1
    assert _index(lib, d, k=MISALIGNED) == 4
    assert _attn(lib, d, {"lse": None}) == 1
    assert _attn(lib, d, {"v": MISALIGNED}) == 4
    assert _kl(lib, d, {"sum": None}) == 1
    assert _kl(lib, d, {"rows": None}) == 1
    assert _kl(lib, d, {"ki": MISALIGNED}) == 4


def test_layout_check_arguments(lib):
    chk = lambda d, bi=FAKE, out=FAKE: lib.msa_check_block_idx(ctypes.byref(d), bi, out, None)
    assert chk(_dims(topk=0)) == 2
    assert chk(_dims(topk=33)) == 3
    assert chk(_dims(block_size=96)) == 3
    assert chk(_dims(block_size=64), out=None) == 1     # 64 and 256 are accepted: goes on to the pointers
    assert chk(_dims(block_size=256), out=None) == 1
    # head and index dims are not read
    assert chk(_dims(head_dim=96, index_dim=96, group_size=3), out=None) == 1
    assert chk(_dims(), bi=None) == 1
    assert chk(_dims(), bi=MISALIGNED) == 4
    assert chk(_dims(), out=ctypes.c_void_p(0x1002)) == 4
    assert lib.msa_check_block_idx(None, FAKE, FAKE, None) == 1


def test_attention_stages_argument(lib):
    d = _dims()
    p = [FAKE] * 4
    for bad in (0, 8, -1, 9):
        assert lib.msa_sparse_attn_fwd_stages(ctypes.byref(d), *p, 0.0, FAKE, FAKE, None, 0, bad, None) == 3
    # a valid stage set goes on to the workspace check
    assert lib.msa_sparse_attn_fwd_stages(ctypes.byref(d), *p, 0.0, FAKE, FAKE, None, 0, 2, None) == 5
    # bad dims are reported before the stage set
    assert lib.msa_sparse_attn_fwd_stages(ctypes.byref(_dims(head_dim=96)), *p, 0.0, FAKE, FAKE, None, 0, 0,
                                          None) == 3


def test_workspace_checks(lib):
    d = _dims()
    need = msa.workspace_bytes(d, msa.MSA_OP_ATTN)
    assert need > 0
    assert _attn(lib, d) == 5                           # no workspace
    assert _attn(lib, d, ws=FAKE, nws=need - 1) == 5    # too small
    assert _attn(lib, d, ws=MISALIGNED, nws=need) == 5  # misaligned
    needk = msa.workspace_bytes(d, msa.MSA_OP_KL)
    assert needk > 0
    assert _kl(lib, d, ws=FAKE, nws=needk - 1) == 5


def test_empty_problems_are_accepted_without_device_work(lib):
    for kw in (dict(batch=0), dict(seqlen=0)):
        d = _dims(**kw)
        assert _index(lib, d, q=None, k=None, out=None) == 0
        assert _attn(lib, d, {k: None for k in ("q", "k", "v", "bi", "o", "lse")}) == 0
        assert msa.workspace_bytes(d, msa.MSA_OP_ATTN) == 0


def test_workspace_sizes(lib):
    # a single query block, or k = 1: no non-local block anywhere -> only the
    # transposed copy of V (B * Hkv * nb * D * 128 elements)
    assert msa.workspace_bytes(_dims(seqlen=128), msa.MSA_OP_ATTN) == 2 * 128 * 128 * 2
    assert msa.workspace_bytes(_dims(topk=1), msa.MSA_OP_ATTN) == 2 * 8 * 128 * 128 * 2
    assert msa.workspace_bytes(_dims(), msa.MSA_OP_INDEX) == 0
    assert msa.workspace_bytes(_dims(), 12) == 0
    assert msa.workspace_bytes(_dims(), msa.MSA_OP_FUSED_BWD) > msa.workspace_bytes(_dims(), msa.MSA_OP_ATTN_BWD) > 0
    # the partial outputs dominate: rows * (k-1) * G * D * 2 bytes for bf16
    d = _dims(seqlen=131072, kv_heads=8, group_size=8, topk=16)
    need = msa.workspace_bytes(d, msa.MSA_OP_ATTN)
    partial = 131072 * 8 * 15 * 8 * 128 * 2
    assert partial < need < partial * 1.1
    d32 = _dims(seqlen=131072, kv_heads=8, group_size=8, topk=16, dtype=msa.MSA_F32)
    assert msa.workspace_bytes(d32, msa.MSA_OP_ATTN) > 1.9 * need


# ------------------------------------------------------------------ decode --

def _dec_index(lib, d, ptrs=None, ws=None, nws=0):
    p = dict(qi=FAKE, ki=FAKE, lens=FAKE, bi=FAKE)
    p.update(ptrs or {})
    return lib.msa_decode_index_topk(ctypes.byref(d), p.get("R", 1), p["qi"], p["ki"], p["lens"], p["bi"], ws, nws,
                                     None)


def _dec_attn(lib, d, ptrs=None, ws=None, nws=0):
    p = dict(q=FAKE, k=FAKE, v=FAKE, lens=FAKE, bi=FAKE, o=FAKE, lse=FAKE)
    p.update(ptrs or {})
    return lib.msa_decode_attn(ctypes.byref(d), p.get("R", 1), p["q"], p["k"], p["v"], p["lens"], p["bi"], 0.0,
                               p["o"], p["lse"], ws, nws, None)


def _dec(lib, d, ptrs=None, ws=None, nws=0):
    p = dict(qi=FAKE, ki=FAKE, q=FAKE, k=FAKE, v=FAKE, lens=FAKE, bi=FAKE, o=FAKE, lse=FAKE)
    p.update(ptrs or {})
    return lib.msa_decode(ctypes.byref(d), p.get("R", 1), p["qi"], p["ki"], p["q"], p["k"], p["v"], p["lens"], 0.0,
                          p["bi"], p["o"], p["lse"], ws, nws, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=msa.MSA_FP8_E4M3), 3), (dict(topk=33), 3), (dict(block_size=64), 3), (dict(causal=0), 3),
    (dict(batch=65536), 2), (dict(batch=2048, kv_heads=1024), 2), (dict(seqlen=1 << 26), 2),
    (dict(index_dim=96), 3), (dict(head_dim=96), 3), (dict(group_size=64), 3),
])
def test_decode_rejects_bad_dims(lib, kw, status):
    d = _dims(**kw)
    assert _dec(lib, d) == status
    # the selection alone ignores the head fields and takes fp8; the attention alone ignores the index dim
    if kw.get("dtype") == msa.MSA_FP8_E4M3:
        assert _dec_index(lib, d, dict(lens=None)) == 1      # accepted: goes on to the pointer checks
    elif "head_dim" not in kw and "group_size" not in kw:
        assert _dec_index(lib, d) == status
    if "index_dim" not in kw:
        assert _dec_attn(lib, d) == status


def test_decode_pointers_workspace_and_sizes(lib):
    d = _dims(batch=4, seqlen=5000, kv_heads=8, group_size=8, topk=16)
    nbs = (5000 + 127) // 128
    need_i = msa.workspace_bytes(d, msa.MSA_OP_DECODE_INDEX)
    need_a = msa.workspace_bytes(d, msa.MSA_OP_DECODE_ATTN)
    # block scores [B, Hkv, nb] fp32; partial outputs and LSEs [B, Hkv, k, G, D + 1] fp32 (256-byte aligned pieces)
    assert need_i == -(-4 * 8 * nbs * 4 // 256) * 256
    assert need_a == 4 * 8 * 16 * 8 * 128 * 4 + -(-4 * 8 * 16 * 8 * 4 // 256) * 256
    assert msa.workspace_bytes(d, msa.MSA_OP_DECODE) == max(need_i, need_a)
    assert _dec_index(lib, d, dict(lens=None), ws=FAKE, nws=need_i) == 1
    assert _dec_index(lib, d, dict(bi=MISALIGNED), ws=FAKE, nws=need_i) == 4
    assert _dec_index(lib, d, ws=FAKE, nws=need_i - 1) == 5
    assert _dec_index(lib, d, ws=MISALIGNED, nws=need_i) == 5
    assert _dec_attn(lib, d, dict(o=None), ws=FAKE, nws=need_a) == 1
    assert _dec_attn(lib, d, ws=None, nws=0) == 5
    assert _dec(lib, d, dict(q=MISALIGNED), ws=FAKE, nws=need_a) == 4


def test_decode_empty_batch_needs_nothing(lib):
    for kw in (dict(batch=0), dict(seqlen=0)):
        d = _dims(**kw)
        none = dict(qi=None, ki=None, q=None, k=None, v=None, lens=None, bi=None, o=None, lse=None)
        assert _dec(lib, d, none) == 0
        assert msa.workspace_bytes(d, msa.MSA_OP_DECODE) == 0


def test_dense_attention_arguments(lib):
    d = _dims(topk=0)                    # topk is not read by the dense attention
    need = msa.workspace_bytes(d, msa.MSA_OP_DENSE_ATTN)
    nb = (1024 + 127) // 128
    assert need == 1 * 2 * nb * 128 * 128 * 2   # V^T copy [B, Hkv, nb, D, 128] bf16

    def call(ptrs=None, ws=FAKE, nws=need, dd=d):
        p = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE)
        p.update(ptrs or {})
        return lib.msa_dense_attn_fwd(ctypes.byref(dd), p["q"], p["k"], p["v"], 0.0, p["o"], p["lse"], ws, nws, None)
    assert call(dict(v=None)) == 1
    assert call(dict(o=MISALIGNED)) == 4
    assert call(nws=need - 1) == 5
    assert call(dd=_dims(head_dim=96)) == 3
    assert call(dd=_dims(dtype=msa.MSA_FP8_E4M3)) == 3
    assert call(dd=_dims(seqlen=0), ptrs=dict(q=None, k=None, v=None, o=None, lse=None), ws=None, nws=0) == 0


def test_dense_kl_arguments(lib):
    d = _dims(topk=0)
    need = msa.workspace_bytes(d, msa.MSA_OP_DENSE_KL)
    assert need == 256                  # one double per reduction block, 256-byte aligned

    def call(ptrs=None, ws=FAKE, nws=need, dd=d):
        p = dict(q=FAKE, k=FAKE, qi=FAKE, ki=FAKE, lse=FAKE, rows=FAKE, sum=FAKE, ilse=None)
        p.update(ptrs or {})
        return lib.msa_dense_kl_align_fwd(ctypes.byref(dd), p["q"], p["k"], p["qi"], p["ki"], p["lse"], 0.0, 0.0,
                                          p["rows"], p["sum"], p["ilse"], ws, nws, None)
    assert call(dict(sum=None)) == 1
    assert call(dict(ki=None)) == 1
    assert call(dict(lse=MISALIGNED)) == 4
    assert call(ws=None, nws=0) == 5
    assert call(dd=_dims(index_dim=96)) == 3


def test_paged_decode_arguments(lib):
    d = _dims(batch=4, seqlen=5000, kv_heads=8, group_size=8, topk=16)
    need = msa.workspace_bytes(d, msa.MSA_OP_DECODE)

    def call(ptrs=None, pages=10, ws=FAKE, nws=need, dd=d):
        p = dict(qi=FAKE, ki=FAKE, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, lens=FAKE, bi=FAKE, o=FAKE, lse=FAKE)
        p.update(ptrs or {})
        return lib.msa_decode_paged(ctypes.byref(dd), 1, p["qi"], p["ki"], p["q"], p["k"], p["v"], p["bt"], pages,
                                    p["lens"], 0.0, p["bi"], p["o"], p["lse"], ws, nws, None)
    assert call(dict(bt=None)) == 1
    assert call(dict(bt=MISALIGNED)) == 4
    assert call(pages=-1) == 2
    assert call(nws=need - 1) == 5
    assert call(dd=_dims(dtype=msa.MSA_FP8_E4M3)) == 3
    assert lib.msa_decode_paged_index_topk(ctypes.byref(_dims(dtype=msa.MSA_FP8_E4M3)), 1, FAKE, FAKE, None, 10,
                                           FAKE, FAKE, FAKE, 1 << 20, None) == 1
    assert lib.msa_decode_paged_attn(ctypes.byref(d), 1, FAKE, FAKE, FAKE, FAKE, -3, FAKE, FAKE, 0.0, FAKE, FAKE,
                                     FAKE, need, None) == 2


def test_multi_query_decode_arguments(lib):
    d = _dims(batch=4, seqlen=5000, kv_heads=8, group_size=8, topk=16)
    one = msa.decode_workspace_bytes(d, msa.MSA_OP_DECODE_ATTN, 1)
    assert one == msa.workspace_bytes(d, msa.MSA_OP_DECODE_ATTN)
    four = msa.decode_workspace_bytes(d, msa.MSA_OP_DECODE_ATTN, 4)
    assert four == 4 * 8 * 4 * 16 * 8 * 128 * 4 + -(-4 * 4 * 8 * 16 * 8 * 4 // 256) * 256
    assert msa.decode_workspace_bytes(d, msa.MSA_OP_DECODE_INDEX, 3) == -(-4 * 3 * 8 * 40 * 4 // 256) * 256
    assert msa.decode_workspace_bytes(d, msa.MSA_OP_DECODE, 0) == 0
    assert msa.decode_workspace_bytes(d, msa.MSA_OP_ATTN, 2) == 0
    assert _dec(lib, d, dict(R=0)) == 2
    assert _dec(lib, _dims(batch=20000), dict(R=4)) == 2              # B * R > 65535
    assert _dec(lib, d, dict(R=4), ws=FAKE, nws=four - 1) == 5       # the R-query workspace is required
    assert _dec_attn(lib, d, dict(R=4, o=None), ws=FAKE, nws=four) == 1


def test_noalloc_decode_arguments(lib):
    """msa_decode_noalloc: the decode checks, then problems whose decode
    workspace exceeds its 64 MiB scratch array are refused (MSA_ERR_SCRATCH)
    before any device work; an empty batch needs nothing."""
    def call(d, R=1, **ptrs):
        p = dict(qi=FAKE, ki=FAKE, q=FAKE, k=FAKE, v=FAKE, sl=FAKE, bi=FAKE, o=FAKE, lse=FAKE)
        p.update(ptrs)
        return lib.msa_decode_noalloc(ctypes.byref(d), R, p["qi"], p["ki"], p["q"], p["k"], p["v"], p["sl"], 0.0,
                                      p["bi"], p["o"], p["lse"], None)
    big = _dims(batch=200, seqlen=131072, kv_heads=8, group_size=8, head_dim=128, index_dim=128, topk=16)
    assert msa.decode_workspace_bytes(big, msa.MSA_OP_DECODE, 1) > msa.NOALLOC_SCRATCH_BYTES
    assert call(big) == 7
    assert call(big, R=2) == 7
    assert call(big, q=None) == 1                      # pointer checks come first
    assert call(big, o=MISALIGNED) == 4
    assert call(_dims(block_size=64)) == 3
    assert call(_dims(), R=0) == 2
    assert call(_dims(batch=0)) == 0                   # empty: nothing to do, no device touched
    assert b"scratch" in lib.msa_strerror(7)
