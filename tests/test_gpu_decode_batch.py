"""GPU parity of small-batch decode (qlora_gemv jobs of m = 2..16 tokens)
against the fp64 oracle.

Y [m x N] = X deq(W)^T + s (X A^T) B^T is the forward product at M = m, so
the oracle is its forward, within the forward tolerances.  The cases span
partial 512-row tiles, odd block counts (a last step of one block), several
1024-column x chunks with a short last one, r = 0 and r = 128, 16 tokens,
batch-1 and batch jobs in one call, a prepared plan re-run on new inputs,
and the other codebooks.
"""

import numpy as np
import pytest
import torch

import oracle
from bit_quantized_finetuning_nf4_amd import ops, synth
from tests.helpers import assert_close, bits_to_torch, torch_to_f64

pytestmark = pytest.mark.gpu


def _job(N, K, r, m, seed, ab_std=0.01, w_std=0.02):
    """w_std = 0 gives W = 0 exactly, so Y is the LoRA term alone."""
    rng = np.random.default_rng(seed)
    g = lambda shape, std: synth.to_bf16_bits(rng.standard_normal(shape) * std)
    W = g((N, K), w_std) if w_std else np.zeros((N, K), dtype=np.uint16)
    return dict(W=W, x=g((m, K) if m else (K,), 1.0), A=g((r, K), ab_std) if r else None,
                B=g((N, r), ab_std) if r else None, alpha=16.0)


def _oracle_y(d, codebook="nf4"):
    c, a, s = oracle.quantize(d["W"], codebook)
    Wd = oracle.bf16_bits_to_f64(oracle.dequant(c, a, s, d["W"].size, codebook)).reshape(d["W"].shape)
    f = lambda k: None if d[k] is None else oracle.bf16_bits_to_f64(d[k]).reshape(d[k].shape)
    X = f("x")
    Y = oracle.linear_fwd(Wd, X.reshape(-1, X.shape[-1]), f("A"), f("B"), d["alpha"])
    return Y.reshape(X.shape[:-1] + (Wd.shape[0],))


def _jobs(ds, codebook="nf4"):
    out = []
    for d in ds:
        q = ops.quantize(bits_to_torch(d["W"]), codebook=codebook)
        out.append(ops.GemvJob(q, bits_to_torch(d["x"]), None if d["A"] is None else bits_to_torch(d["A"]),
                               None if d["B"] is None else bits_to_torch(d["B"]), d["alpha"]))
    return out


def _run(ds, label, codebook="nf4"):
    print(f"[decode batch parity] {codebook} {label}: {len(ds)} jobs", flush=True)
    ys = ops.gemv(_jobs(ds, codebook))
    torch.cuda.synchronize()
    for i, (d, y) in enumerate(zip(ds, ys)):
        assert tuple(y.shape) == _oracle_y(d, codebook).shape
        assert_close(torch_to_f64(y), _oracle_y(d, codebook), f"{label} job {i}")


# (1100, 2112): 33 blocks per row (a last step of one block), three x chunks
# with a short last one, three tiles with a partial last one.
# (70, 64) and (130, 192): rows of one and three blocks, so most of a
# chunk's spans lie past the row end and read other rows' codes (or nothing).
@pytest.mark.parametrize("N,K,r,m", [(300, 640, 16, 2), (1100, 2112, 8, 3), (520, 1024, 0, 16),
                                     (512, 4096, 64, 16), (64, 128, 32, 5), (96, 3072, 128, 8),
                                     (40, 22016, 64, 4), (70, 64, 8, 3), (130, 192, 16, 16)])
def test_single_job_shapes(N, K, r, m):
    _run([_job(N, K, r, m, seed=N + K + r + m)], f"N{N} K{K} r{r} m{m}")


# The LoRA term carries Y in these cases, so a mistake in the m-token
# u = A x, in the staged s u or in the up-projection MFMAs at tile end
# cannot hide inside the tolerance of the base product.
@pytest.mark.parametrize("N,K,r,m", [(1024, 1024, 64, 2), (520, 8192, 128, 16), (40, 22016, 64, 5),
                                     (1100, 2112, 128, 9), (300, 640, 64, 16)])
def test_lora_only_weight_zero(N, K, r, m):
    _run([_job(N, K, r, m, seed=8000 + N + r + m, ab_std=1.0, w_std=0.0)], f"W=0 N{N} K{K} r{r} m{m}")


@pytest.mark.parametrize("r,ab_std,m", [(64, 1.0, 4), (128, 1.0, 16), (128, 0.2, 8), (64, 0.2, 2)])
def test_lora_dominant_stress(r, ab_std, m):
    d = _job(768, 4096, r, m, seed=8100 + r + m, ab_std=ab_std)
    f = lambda k: oracle.bf16_bits_to_f64(d[k]).reshape(d[k].shape)
    lora = d["alpha"] / r * (f("x") @ f("A").T) @ f("B").T
    assert np.linalg.norm(lora) > 0.9 * np.linalg.norm(_oracle_y(d))
    _run([d], f"stress r{r} ab{ab_std} m{m}")


def test_lora_stress_mixed_call():
    # batch-1 and m-token jobs, W = 0 and LoRA-dominant and ordinary, in one call
    ds = [_job(1024, 1024, 64, 16, seed=8200, ab_std=1.0, w_std=0.0),
          _job(512, 8192, 128, 0, seed=8201, ab_std=1.0),
          _job(40, 22016, 64, 3, seed=8202),
          _job(300, 1536, 128, 8, seed=8203, ab_std=0.2, w_std=0.0),
          _job(1536, 512, 8, 1, seed=8204, ab_std=1.0, w_std=0.0),
          _job(700, 1088, 32, 12, seed=8205, ab_std=1.0)]
    _run(ds, "stress mixed")


def test_tokens_past_the_first_are_not_the_first_token_repeated():
    # every token row of the output follows its own x row
    d = _job(256, 512, 16, 7, seed=41)
    y = torch_to_f64(ops.gemv(_jobs([d]))[0])
    torch.cuda.synchronize()
    ref = _oracle_y(d)
    for t in range(7):
        assert_close(y[t], ref[t], f"token {t}")
    assert np.linalg.norm(ref[1] - ref[0]) > 0.5 * np.linalg.norm(ref[0])


def test_batch_and_single_token_jobs_in_one_call():
    shapes = [(512, 1024, 64, 0), (1536, 1024, 64, 4), (300, 22016, 16, 16), (64, 576, 8, 1), (700, 1088, 32, 2),
              (130, 64, 8, 0), (1024, 512, 0, 9)]
    _run([_job(N, K, r, m, seed=200 + i) for i, (N, K, r, m) in enumerate(shapes)], "mixed")


def test_one_workgroup_walks_jobs_of_different_token_counts():
    # 300 one-tile jobs are more than the device's persistent workgroups, so
    # some workgroups take several jobs in a row; token counts rise and fall
    # from job to job (staged x rows past m must not reach any output).  The
    # last two jobs read one x tensor, the second its first 5 rows only.
    ms = [2 + (7 * i) % 15 for i in range(300)]
    ds = [_job(64, 128, 8 if i % 3 else 0, m, seed=9000 + i) for i, m in enumerate(ms)]
    ds.append(_job(64, 128, 8, 16, seed=9998))
    ds.append(dict(_job(64, 128, 8, 5, seed=9999), x=ds[-1]["x"][:5]))
    jobs = _jobs(ds)
    jobs[-1].x = jobs[-2].x[:5]   # the same memory as the 16-token job's first rows
    print(f"[decode batch parity] {len(ds)} small jobs", flush=True)
    ys = ops.gemv(jobs)
    torch.cuda.synchronize()
    for i, (d, y) in enumerate(zip(ds, ys)):
        assert_close(torch_to_f64(y), _oracle_y(d), f"job {i} (m = {d['x'].shape[0]})")


def test_prepared_plan_reruns_with_new_inputs():
    shapes = [(512, 1024, 64, 8), (1536, 1024, 64, 16), (300, 2048, 16, 0)]
    ds = [_job(N, K, r, m, seed=600 + i) for i, (N, K, r, m) in enumerate(shapes)]
    jobs = _jobs(ds)
    plan = ops.GemvPlan(jobs)
    for run in range(3):
        print(f"[decode batch parity] prepared plan, run {run}", flush=True)
        for i, (d, j) in enumerate(zip(ds, jobs)):
            rng = np.random.default_rng(2000 * run + i)
            d["x"] = synth.to_bf16_bits(rng.standard_normal(d["x"].shape))
            j.x.copy_(bits_to_torch(d["x"]))
        ys = plan()
        torch.cuda.synchronize()
        for i, (d, y) in enumerate(zip(ds, ys)):
            assert_close(torch_to_f64(y), _oracle_y(d), f"run {run} job {i}")


def test_matches_the_fused_forward():
    # the decode batch and qlora_linear_fwd compute the same product at M = m
    d = _job(768, 1024, 64, 6, seed=43)
    job = _jobs([d])[0]
    y = ops.gemv([job])[0]
    Y = ops.linear_fwd(job.q, job.x, job.A, job.B, 16.0)
    torch.cuda.synchronize()
    ref = _oracle_y(d)
    assert_close(torch_to_f64(y), ref, "decode batch")
    assert_close(torch_to_f64(Y), ref, "fwd M=6")


@pytest.mark.parametrize("codebook", ["fp4", "int4"])
def test_other_codebooks(codebook):
    _run([_job(1024, 1024, 64, 4, seed=51), _job(37, 22016, 64, 16, seed=52), _job(300, 1536, 8, 1, seed=53)],
         "grouped", codebook)


def test_more_than_16_tokens_is_rejected():
    d = _job(64, 128, 0, 17, seed=55)
    with pytest.raises(RuntimeError, match="UNSUPPORTED"):
        ops.gemv(_jobs([d]))
