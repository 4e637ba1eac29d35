"""QLORA_DEBUG=1 guard bands, exercised on host tensors (no GPU needed)."""

import pytest
import torch

from bit_quantized_finetuning_nf4_amd import debug


@pytest.fixture
def enabled(monkeypatch):
    monkeypatch.setattr(debug, "ENABLED", True)
    monkeypatch.setattr(debug, "_live", [])


def test_disabled_is_plain_empty(monkeypatch):
    monkeypatch.setattr(debug, "ENABLED", False)
    t = debug.empty((3, 5), torch.bfloat16, "cpu")
    assert t.shape == (3, 5) and not hasattr(t, "_qlora_guard")


def test_guarded_view_shape_alignment_and_clean_check(enabled):
    t = debug.empty((7, 9), torch.float32, "cpu")
    assert t.shape == (7, 9) and t.dtype == torch.float32 and t.is_contiguous()
    assert t.data_ptr() % 256 == t._qlora_guard[0].data_ptr() % 256
    t.fill_(1.0)                       # writing the whole view leaves the guards alone
    debug.after_call("fill")


@pytest.mark.parametrize("where", ["before", "after"])
def test_write_into_a_guard_is_caught(enabled, where):
    t = debug.empty(100, torch.uint8, "cpu")
    base, n = t._qlora_guard
    base[debug.GUARD_BYTES - 1 if where == "before" else debug.GUARD_BYTES + n] = 0
    with pytest.raises(debug.CanaryError, match="qlora_test_call"):
        debug.after_call("qlora_test_call")
    del t, base
    debug.after_call("after the buffer is gone")   # dead buffers are dropped from the check


@pytest.mark.parametrize("on", [False, True])
def test_binding_allocator_takes_sizes_or_one_tuple(monkeypatch, on):
    from bit_quantized_finetuning_nf4_amd import ops
    monkeypatch.setattr(debug, "ENABLED", on)
    monkeypatch.setattr(debug, "_live", [])
    for args in ((2, 3), ((2, 3),), ([2, 3],), (torch.Size([2, 3]),)):
        t = ops._empty(*args, dtype=torch.bfloat16, device="cpu")
        assert t.shape == (2, 3) and t.dtype == torch.bfloat16
    assert ops._empty(5, dtype=torch.uint8, device="cpu").shape == (5,)
