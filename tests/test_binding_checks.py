"""Host-side argument checks of the Python binding (CPU only).

The binding passes raw pointers to kernels that write every row of their
outputs, so an undersized output must be rejected before anything is
launched.  These tests run the binding's own checks on CPU tensors with the
device test relaxed and a stand-in library whose compute entry points fail
the test if they are ever reached.
"""
import pytest
import torch

import transformer_attention_amd as ta


class _NoLaunch:
    """Workspace sizes as plain numbers; any compute call is a test failure."""

    def __getattr__(self, name):
        if name.endswith("_workspace_size"):
            return lambda *a: 4096
        if name == "attn_status_string":
            return lambda s: b"stub"

        def launched(*a):
            raise AssertionError(f"{name} was launched")
        return launched


@pytest.fixture
def host_binding(monkeypatch):
    def require_on_host(t, name, dtype, device=None, ndim=None):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if dtype is not None and t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
        if ndim is not None and t.dim() != ndim:
            raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")

    monkeypatch.setattr(ta, "_require", require_on_host)
    monkeypatch.setattr(ta, "_lib", _NoLaunch())
    monkeypatch.setattr(ta, "_stream", lambda device: None)


B, HQ, HKV, S, D = 3, 8, 2, 64, 128
BAD_LSE = (torch.empty(B * HQ - 1), torch.empty(B, HQ + 1))


def _bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def _lens():
    return torch.full((B,), S, dtype=torch.int32)


def _table():
    return torch.zeros((B, 1), dtype=torch.int32)


CALLS = {
    "attn_decode": lambda lse: ta.attn_decode(_bf(B, HQ, D), _bf(B, HKV, S, D), _bf(B, HKV, S, D),
                                              _lens(), lse=lse),
    "mla_decode": lambda lse: ta.mla_decode(_bf(B, HQ, 576), _bf(B, S, 576), _lens(), scale=0.1,
                                            lse=lse),
    "attn_decode_paged": lambda lse: ta.attn_decode_paged(
        _bf(B, HQ, D), _bf(4, HKV, S, D), _bf(4, HKV, S, D), _lens(), _table(), lse=lse),
    "mla_decode_paged": lambda lse: ta.mla_decode_paged(
        _bf(B, HQ, 576), _bf(4, S, 576), _lens(), _table(), scale=0.1, lse=lse),
    "attn_decode_fp8": lambda lse: ta.attn_decode_fp8(
        _bf(B, HQ, D), torch.zeros((B, HKV, S, D), dtype=torch.uint8),
        torch.zeros((B, HKV, S, D), dtype=torch.uint8), torch.ones(B, HKV, 2),
        torch.ones(B, HKV, 2), _lens(), lse=lse),
    "attn_decode_paged_fp8": lambda lse: ta.attn_decode_paged_fp8(
        _bf(B, HQ, D), torch.zeros((4, HKV, S, D), dtype=torch.uint8),
        torch.zeros((4, HKV, S, D), dtype=torch.uint8), torch.ones(4, HKV, 2),
        torch.ones(4, HKV, 2), _lens(), _table(), lse=lse),
}


@pytest.mark.parametrize("entry", sorted(CALLS))
@pytest.mark.parametrize("bad", range(len(BAD_LSE)))
def test_wrong_size_lse_is_rejected_before_launch(host_binding, entry, bad):
    with pytest.raises(ValueError, match="lse"):
        CALLS[entry](BAD_LSE[bad])


@pytest.mark.parametrize("entry", sorted(CALLS))
def test_right_size_lse_reaches_the_launch(host_binding, entry):
    """With a correctly sized lse the checks pass and the call reaches the
    library (the stand-in then stops it)."""
    with pytest.raises(AssertionError, match="was launched"):
        CALLS[entry](torch.empty(B, HQ))
