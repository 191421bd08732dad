"""The Python binding refuses mis-shaped, mis-typed or misplaced tensors before
anything reaches the library (host only: CPU tensors stand in for device
tensors, and the library's compute entry points are replaced by a stub that
fails the test if any of them is called)."""
import pytest
import torch

import block_sparse_gqa_index_amd as msa

B, N, HKV, G, D, DI, K = 1, 256, 2, 4, 64, 64, 4
HQ = HKV * G


class _Stub:
    """The real library for its host-only helpers; any other call fails."""

    def __init__(self, real):
        self._real = real

    def __getattr__(self, name):
        if name in ("msa_workspace_bytes", "msa_decode_workspace_bytes", "msa_strerror", "msa_abi_version"):
            return getattr(self._real, name)

        def called(*a, **k):
            raise AssertionError(f"{name} was called with bad arguments")
        return called


@pytest.fixture
def host(monkeypatch):
    real = msa.load_library()
    monkeypatch.setattr(msa, "_on_gpu", lambda t: t.device.type == "cpu")
    monkeypatch.setattr(msa, "load_library", lambda *a, **k: _Stub(real))
    monkeypatch.setattr(msa, "_stream", lambda dev: None)


def t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def meta(*shape, dtype=torch.float32):
    return torch.empty(shape, dtype=dtype, device="meta")


def inputs():
    return dict(q_idx=t(B, N, HKV, DI), k_idx=t(B, N, DI), q=t(B, N, HQ, D), k=t(B, N, HKV, D), v=t(B, N, HKV, D),
                bi=t(B, HKV, N, K, dtype=torch.int32), lse=t(B, HQ, N, dtype=torch.float32))


@pytest.mark.parametrize("kw", [
    dict(block_idx=t(B, HKV, N, K - 1, dtype=torch.int32)),
    dict(block_idx=t(B, HKV, N - 1, K, dtype=torch.int32)),
    dict(block_idx=t(B, HKV, N, K)),                       # wrong dtype
])
def test_index_topk_output(host, kw):
    x = inputs()
    with pytest.raises(ValueError):
        msa.index_topk(x["q_idx"], x["k_idx"], K, **kw)


@pytest.mark.parametrize("kw", [
    dict(o=t(B, N, HQ, D - 1)), dict(o=t(B, N - 1, HQ, D)), dict(o=t(B, N, HQ, D, dtype=torch.float32)),
    dict(lse=t(B, HQ, N - 1, dtype=torch.float32)), dict(lse=t(B, HKV, N, dtype=torch.float32)),
    dict(o=meta(B, N, HQ, D, dtype=torch.bfloat16)),       # not a device tensor
])
def test_sparse_attn_outputs(host, kw):
    x = inputs()
    with pytest.raises(ValueError):
        msa.sparse_attn_fwd(x["q"], x["k"], x["v"], x["bi"], **kw)


@pytest.mark.parametrize("kw", [
    dict(block_idx=t(B, HKV, N, K + 1, dtype=torch.int32)), dict(o=t(B, N, HQ - 1, D)),
    dict(lse=t(B, HQ, 1, dtype=torch.float32)),
])
def test_forward_outputs(host, kw):
    x = inputs()
    with pytest.raises(ValueError):
        msa.forward(x["q_idx"], x["k_idx"], x["q"], x["k"], x["v"], K, **kw)


@pytest.mark.parametrize("kw", [
    dict(kl_rows=t(B, HKV, N - 1, dtype=torch.float32)), dict(kl_rows=t(B, HKV, N)),
    dict(kl_rows=meta(B, HKV, N)), dict(kl_sum=t(2, dtype=torch.float32)), dict(kl_sum=meta(1)),
    dict(kl_sum=t(1, dtype=torch.float64)), dict(index_lse=t(B, HKV, 1, dtype=torch.float32)),
])
def test_kl_outputs(host, kw):
    x = inputs()
    with pytest.raises(ValueError):
        msa.kl_align_fwd(x["q"], x["k"], x["q_idx"], x["k_idx"], x["bi"], x["lse"], **kw)


def test_kl_inputs(host):
    x = inputs()
    with pytest.raises(ValueError):
        msa.kl_align_fwd(x["q"], x["k"], x["q_idx"], x["k_idx"], x["bi"], t(B, HQ, N - 1, dtype=torch.float32))
    with pytest.raises(ValueError):
        msa.kl_align_fwd(x["q"], x["k"], x["q_idx"], t(B, N - 1, DI), x["bi"], x["lse"])


@pytest.mark.parametrize("kw", [
    dict(dq=t(B, N, HQ, D - 1)), dict(dk=t(B, N, HKV + 1, D)), dict(dv=meta(B, N, HKV, D, dtype=torch.bfloat16)),
])
def test_backward_outputs(host, kw):
    x = inputs()
    with pytest.raises(ValueError):
        msa.sparse_attn_bwd(x["q"], x["k"], x["v"], x["bi"], x["q"], x["lse"], x["q"], **kw)


@pytest.mark.parametrize("kw", [dict(dq_idx=t(B, N, HKV, DI - 1)), dict(dk_idx=t(B, N, DI + 1))])
def test_kl_backward_outputs(host, kw):
    x = inputs()
    ilse = t(B, HKV, N, dtype=torch.float32)
    with pytest.raises(ValueError):
        msa.kl_align_bwd(x["q"], x["k"], x["q_idx"], x["k_idx"], x["bi"], x["lse"], ilse, **kw)


def test_dense_outputs(host):
    x = inputs()
    with pytest.raises(ValueError):
        msa.dense_attn_fwd(x["q"], x["k"], x["v"], lse=t(B, HQ, N + 1, dtype=torch.float32))
    with pytest.raises(ValueError):
        msa.dense_kl_align_fwd(x["q"], x["k"], x["q_idx"], x["k_idx"], x["lse"], kl_sum=t(1))


def _decode():
    Bd, C = 3, 512
    return dict(q_idx=t(Bd, HKV, DI), k_idx=t(Bd, C, DI), q=t(Bd, HQ, D), k=t(Bd, C, HKV, D), v=t(Bd, C, HKV, D),
                seqlens=t(Bd, dtype=torch.int32), bi=t(Bd, HKV, K, dtype=torch.int32), B=Bd)


@pytest.mark.parametrize("kw", [
    dict(block_idx=t(3, HKV, K - 1, dtype=torch.int32)),    # shorter than topk: the kernels write K ids
    dict(o=t(3, HQ, D + 1)), dict(lse=t(3, HQ + 1, dtype=torch.float32)), dict(lse=meta(3, HQ)),
])
def test_decode_outputs(host, kw):
    x = _decode()
    with pytest.raises(ValueError):
        msa.decode(x["q_idx"], x["k_idx"], x["q"], x["k"], x["v"], x["seqlens"], K, **kw)


def test_decode_selection_and_attention_outputs(host):
    x = _decode()
    with pytest.raises(ValueError):
        msa.decode_index_topk(x["q_idx"], x["k_idx"], x["seqlens"], K, block_idx=t(3, HKV, K + 1, dtype=torch.int32))
    with pytest.raises(ValueError):
        msa.decode_attn(x["q"], x["k"], x["v"], x["seqlens"], x["bi"], o=t(3, HQ, D - 1))
    with pytest.raises(ValueError):
        msa.decode_attn(x["q"], x["k"], x["v"], x["seqlens"], x["bi"], lse=t(3, HQ, 2, dtype=torch.float32))


def test_workspace_must_be_a_device_tensor(host):
    x = inputs()
    with pytest.raises(ValueError):
        msa.sparse_attn_fwd(x["q"], x["k"], x["v"], x["bi"], workspace=meta(1 << 20, dtype=torch.uint8))


def test_good_arguments_reach_the_library(host):
    """Sanity check of the set-up: well-formed calls pass every check and
    arrive at the (stubbed) library call."""
    x = inputs()
    with pytest.raises(AssertionError, match="msa_sparse_attn_fwd"):
        msa.sparse_attn_fwd(x["q"], x["k"], x["v"], x["bi"])
    with pytest.raises(AssertionError, match="msa_kl_align_fwd"):
        msa.kl_align_fwd(x["q"], x["k"], x["q_idx"], x["k_idx"], x["bi"], x["lse"])
    d = _decode()
    with pytest.raises(AssertionError, match="msa_decode"):
        msa.decode(d["q_idx"], d["k_idx"], d["q"], d["k"], d["v"], d["seqlens"], K)
