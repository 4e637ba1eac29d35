"""GPU parity of qlora_gemv (batch-1 decode) against the fp64 oracle.

y = deq(W) x + s B (A x) within the forward tolerances, for single jobs,
ragged row counts and block counts, r = 0, and batches larger than one
kernel-argument batch with mixed shapes (the grouped decode path).
"""

import numpy as np
import pytest
import torch

import oracle
from bit_quantized_finetuning_nf4_amd import ops, synth
from tests.helpers import assert_close, bits_to_torch, torch_to_f64

pytestmark = pytest.mark.gpu


def _job(N, K, r, seed, ab_std=0.01, w_std=0.02):
    """w_std = 0 gives W = 0 exactly (every block all-zero), so y is the
    LoRA term alone."""
    rng = np.random.default_rng(seed)
    g = lambda shape, std: synth.to_bf16_bits(rng.standard_normal(shape) * std)
    W = g((N, K), w_std) if w_std else np.zeros((N, K), dtype=np.uint16)
    return dict(W=W, x=g((K,), 1.0), A=g((r, K), ab_std) if r else None,
                B=g((N, r), ab_std) if r else None, alpha=16.0)


def _oracle_y(d, codebook="nf4"):
    c, a, s = oracle.quantize(d["W"], codebook)
    Wd = oracle.bf16_bits_to_f64(oracle.dequant(c, a, s, d["W"].size, codebook)).reshape(d["W"].shape)
    f = lambda k: None if d[k] is None else oracle.bf16_bits_to_f64(d[k]).reshape(d[k].shape)
    return oracle.gemv(Wd, f("x"), f("A"), f("B"), d["alpha"])


def _run(ds, label, codebook="nf4"):
    print(f"[gemv parity] {codebook} {label}: {len(ds)} jobs", flush=True)
    jobs = []
    for d in ds:
        q = ops.quantize(bits_to_torch(d["W"]), codebook=codebook)
        jobs.append(ops.GemvJob(q, bits_to_torch(d["x"]),
                                None if d["A"] is None else bits_to_torch(d["A"]),
                                None if d["B"] is None else bits_to_torch(d["B"]), d["alpha"]))
    ys = ops.gemv(jobs)
    torch.cuda.synchronize()
    for i, (d, y) in enumerate(zip(ds, ys)):
        assert_close(torch_to_f64(y), _oracle_y(d, codebook), f"{label} job {i}")


def test_small_config_one_token():
    d = synth.small_numpy(0)
    _run([dict(W=d["W"], x=d["X"][0], A=d["A"], B=d["B"], alpha=d["alpha"])], "1024^2 r8")


# (37, 22016): a row's absmax codes end mid-way through a 16-block load unit
# (344 blocks), and the last row's last two steps read up to the array end.
@pytest.mark.parametrize("N,K,r", [(1024, 1024, 64), (1000, 576, 16), (130, 64, 8), (257, 8192, 128),
                                   (64, 320, 0), (37, 22016, 64), (300, 1536, 8)])
def test_single_job_shapes(N, K, r):
    _run([_job(N, K, r, seed=N + K + r)], f"N{N} K{K} r{r}")


# The LoRA side path carries y, so a mistake in u = A x, in its scale or in
# the up-projection at tile start cannot hide inside the tolerance of a base
# product that dominates y (deepfa.ir blog, "LoRA: Prerequisite": the
# adapter's low-rank product is added to the frozen layer's).
@pytest.mark.parametrize("N,K,r", [(1024, 1024, 64), (257, 8192, 128), (37, 22016, 64), (300, 1536, 128)])
def test_lora_only_weight_zero(N, K, r):
    d = _job(N, K, r, seed=7000 + N + r, ab_std=1.0, w_std=0.0)
    _run([d], f"W=0 N{N} K{K} r{r}")


@pytest.mark.parametrize("r,ab_std", [(64, 1.0), (128, 1.0), (128, 0.2)])
def test_lora_dominant_stress(r, ab_std):
    d = _job(768, 4096, r, seed=7100 + r, ab_std=ab_std)
    ref = _oracle_y(d)
    # the case is only a stress case if the LoRA term carries most of y
    f = lambda k: oracle.bf16_bits_to_f64(d[k]).reshape(d[k].shape)
    lora = d["alpha"] / r * f("B") @ (f("A") @ f("x"))
    assert np.linalg.norm(lora) > 0.9 * np.linalg.norm(ref)
    _run([d], f"stress r{r} ab{ab_std}")


def test_lora_stress_mixed_call():
    # W = 0, LoRA-dominant and ordinary jobs of several shapes in one call
    ds = [_job(1024, 1024, 64, seed=7200, ab_std=1.0, w_std=0.0), _job(512, 8192, 128, seed=7201, ab_std=1.0),
          _job(37, 22016, 64, seed=7202), _job(300, 1536, 128, seed=7203, ab_std=0.2, w_std=0.0),
          _job(64, 320, 0, seed=7204), _job(1536, 512, 8, seed=7205, ab_std=1.0)]
    _run(ds, "stress mixed")


def test_jobs_sharing_x_with_different_lengths():
    """Two jobs read one x buffer, over different lengths K: each must see
    its own K columns with zero beyond (the x staged for the first job must
    not serve the second)."""
    x_full = synth.to_bf16_bits(np.random.default_rng(7300).standard_normal(4096))
    x = bits_to_torch(x_full)
    ds, jobs = [], []
    for i, (N, K) in enumerate([(512, 4096), (300, 1088), (700, 4096), (64, 2112)]):
        d = _job(N, K, 64, seed=7310 + i, ab_std=0.2)
        d["x"] = x_full[:K]
        ds.append(d)
        q = ops.quantize(bits_to_torch(d["W"]))
        jobs.append(ops.GemvJob(q, x[:K], bits_to_torch(d["A"]), bits_to_torch(d["B"]), d["alpha"]))
    assert all(j.x.data_ptr() == x.data_ptr() for j in jobs)
    print("[gemv parity] one x buffer, four lengths", flush=True)
    ys = ops.gemv(jobs)
    torch.cuda.synchronize()
    for i, (d, y) in enumerate(zip(ds, ys)):
        assert_close(torch_to_f64(y), _oracle_y(d), f"shared x job {i}")


def test_grouped_batch_mixed_shapes():
    shapes = [(512, 512, 64), (1536, 512, 64), (512, 1536, 64), (264, 1088, 32), (64, 64, 0)] * 6
    _run([_job(N, K, r, seed=100 + i) for i, (N, K, r) in enumerate(shapes)], "grouped")


def test_gemv_matches_forward_at_one_token():
    d = _job(768, 1024, 64, seed=3)
    q = ops.quantize(bits_to_torch(d["W"]))
    x, A, B = bits_to_torch(d["x"]), bits_to_torch(d["A"]), bits_to_torch(d["B"])
    y = ops.gemv([ops.GemvJob(q, x, A, B, 16.0)])[0]
    Y = ops.linear_fwd(q, x.view(1, -1), A, B, 16.0)
    torch.cuda.synchronize()
    ref = _oracle_y(d)
    assert_close(torch_to_f64(y), ref, "gemv")
    assert_close(torch_to_f64(Y)[0], ref, "fwd M=1")


def test_prepared_plan_reruns_with_new_inputs():
    """qlora_gemv_prepare once, qlora_gemv_run three times: the inputs change
    in place between runs and every run matches the oracle."""
    shapes = [(512, 1024, 64), (1536, 1024, 64), (300, 22016, 16), (64, 576, 8)]
    ds = [_job(N, K, r, seed=500 + i) for i, (N, K, r) in enumerate(shapes)]
    qs = [ops.quantize(bits_to_torch(d["W"])) for d in ds]
    xs = [bits_to_torch(d["x"]) for d in ds]
    plan = ops.GemvPlan([ops.GemvJob(q, x, bits_to_torch(d["A"]), bits_to_torch(d["B"]), d["alpha"])
                         for q, x, d in zip(qs, xs, ds)])
    for run in range(3):
        print(f"[gemv parity] prepared plan, run {run}", flush=True)
        for i, d in enumerate(ds):
            rng = np.random.default_rng(1000 * run + i)
            d["x"] = synth.to_bf16_bits(rng.standard_normal(d["x"].shape))
            xs[i].copy_(bits_to_torch(d["x"]))
        ys = plan()
        torch.cuda.synchronize()
        for i, (d, y) in enumerate(zip(ds, ys)):
            assert_close(torch_to_f64(y), _oracle_y(d), f"run {run} job {i}")


@pytest.mark.parametrize("codebook", ["fp4", "int4"])
def test_other_codebooks(codebook):
    # FP4 and Int4 weights (one codebook per call), single and grouped jobs
    _run([_job(1024, 1024, 64, seed=31)], "N1024 K1024 r64", codebook)
    _run([_job(37, 22016, 64, seed=32), _job(300, 1536, 8, seed=33), _job(64, 320, 0, seed=34)], "grouped",
         codebook)


def test_mixed_codebooks_in_one_call_are_rejected():
    d = _job(64, 128, 0, seed=35)
    W = bits_to_torch(d["W"])
    jobs = [ops.GemvJob(ops.quantize(W, codebook="nf4"), bits_to_torch(d["x"]), None, None, 0.0),
            ops.GemvJob(ops.quantize(W, codebook="fp4"), bits_to_torch(d["x"]), None, None, 0.0)]
    with pytest.raises(RuntimeError, match="UNSUPPORTED"):
        ops.gemv(jobs)
