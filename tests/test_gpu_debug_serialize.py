"""GPU checks of the debug mode (QLORA_DEBUG=1) and of serialized weights.

Debug mode must leave every result bit-identical and find every guard band
intact after the library's calls; a weight written by save_quantized and
read back onto the GPU must dequantize to the same bits.
"""

import numpy as np
import pytest
import torch

from bit_quantized_finetuning_nf4_amd import debug, ops, synth
from tests.helpers import bits_to_torch

pytestmark = pytest.mark.gpu


def _inputs():
    d = synth.small_numpy(0)
    W, X, A, B, dY = (bits_to_torch(d[k], "cuda:0") for k in ("W", "X", "A", "B", "dY"))
    return W, X, A, B, dY, d["alpha"]


def _run(W, X, A, B, dY, alpha):
    q = ops.quantize(W)
    Y, U = ops.linear_fwd(q, X, A, B, alpha, save_u=True)
    dX, dA, dB = ops.linear_bwd(q, X, dY, A, B, alpha, U=U)
    y = ops.gemv([ops.GemvJob(q, X[0].contiguous(), A, B, alpha)])[0]
    Wd = ops.dequant(q)
    torch.cuda.synchronize()
    return [q.codes, q.absmax_q, q.group_scale, Y, U, dX, dA, dB, y, Wd]


def test_debug_mode_gives_identical_results(monkeypatch):
    args = _inputs()
    plain = _run(*args)
    monkeypatch.setattr(debug, "ENABLED", True)
    monkeypatch.setattr(debug, "_live", [])
    guarded = _run(*args)
    debug.after_call("final check")
    # every output of the debug run is a guarded view, alive and intact
    assert all(hasattr(t, "_qlora_guard") and debug.guards_intact(t) for t in guarded)
    assert len(debug._live) >= len(guarded)
    for a, b in zip(plain, guarded):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_serialized_weight_round_trip_on_gpu(tmp_path):
    W = _inputs()[0]
    for codebook, fmt in (("nf4", "linear"), ("fp4", "fp8")):
        q = ops.quantize(W, codebook=codebook, absmax_format=fmt)
        ops.save_quantized(q, tmp_path / f"{codebook}.qt")
        r = ops.load_quantized(tmp_path / f"{codebook}.qt", "cuda:0")
        assert (r.codebook, r.absmax_format) == (codebook, fmt)
        a, b = ops.dequant(q), ops.dequant(r)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        assert np.array_equal(q.codes.cpu().numpy(), r.codes.cpu().numpy())
