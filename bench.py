#!/usr/bin/env python3
"""Throughput of the QLoRA NF4 linear hot path on one MI355X.

One step is one pass of every stage of the path over the LLaMA-65B-shaped
layer set (q/k/v/o 8192x8192, gate/up 22016x8192, down 8192x22016; 4096
tokens; LoRA r = 64, alpha = 16; NF4 blocksize 64 with 8-bit double
quantization over 256-block groups):

  1. quantize the seven bf16 weights (block absmax, NF4 codes, 8-bit absmax
     codes against fp32 group scales);
  2. forward: U = X A^T, then the fused NF4 GEMM Y = X deq(W)^T + s U B^T;
  3. backward: G = dY B, the fused NF4 GEMM dX = dY deq(W) + s G A, then
     dA = s G^T X and dB = s dY^T U;
  4. batch-1 decode: y = deq(W) x + s B (A x) for the seven linears in one
     grouped call.

`value` is the fwd+bwd algorithmic work, sum over linears of
4MNK + 6Mr(N+K) flops, divided by the wall time of whole steps (quantize and
decode included).  HIP events on the launch stream bracket every fused GEMM
launch; the slower of the two fused GEMMs is reported against the dense bf16
MFMA peak.  The CPU oracle (fp64 numpy) is timed on one linear of the same
workload.  With --decode-layers > 0 the 80-layer decode pass (about 65e9
weights) is also timed and reported as HBM bandwidth.

Inputs are synthetic and seeded (bit_quantized_finetuning_nf4_amd.synth);
they are resident in HBM before timing starts.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E
METRIC = "QLoRA linear fwd+bwd TFLOP/s at 7B/65B shapes; NF4 decode GEMV HBM GB/s"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def linear_flops(M, N, K, r):
    return 4 * M * N * K + 6 * M * r * (N + K)


def gemv_bytes(N, K, r, m=1):
    # codes, absmax codes, group scales, A and B, and m rows of x and y
    return N * K // 2 + N * K // 64 + 4 * (-(-N * K // 16384)) + 2 * r * (N + K) + 2 * m * (N + K)


def decode_batch_study(jobs, layers, r, alpha, passes, dev):
    """Decode of m = 2..16 tokens over the same quantized layers as the
    batch-1 pass (one grouped call of 7 jobs per layer), and dense bf16
    decode (F.linear on bf16 weights) timed on 8 layers and scaled to the
    layer count, for the 4-bit versus 16-bit decode comparison."""
    import torch
    from bit_quantized_finetuning_nf4_amd import ops, synth
    E = lambda: torch.cuda.Event(enable_timing=True)

    def timed(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        evs = [(E(), E()) for _ in range(passes)]
        for a, b in evs:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in evs) / len(evs)

    shapes = [(j.q.rows, j.q.cols) for j in jobs]
    out = {"workload": f"{layers} layers x 7 LLaMA-65B-shaped linears, m tokens per linear, LoRA r={r} fused; "
                       f"{len(jobs)} jobs in one grouped call", "tokens": {}}
    one_ms = None
    for m in (1, 2, 4, 8, 16):
        xs = {}
        mj = []
        for li, j in enumerate(jobs):
            key = (li // 7, j.q.cols)
            if key not in xs:
                shape = (j.q.cols,) if m == 1 else (m, j.q.cols)
                xs[key] = synth.normal_bf16(shape, 1.0, 20_000_000 + 1000 * m + 2 * key[0] + (j.q.cols > 8192), dev)
            mj.append(ops.GemvJob(j.q, xs[key], j.A, j.B, alpha))
        plan = ops.GemvPlan(mj)
        ms = timed(plan)
        nbytes = sum(gemv_bytes(N, K, r, m) for N, K in shapes)
        one_ms = ms if m == 1 else one_ms
        out["tokens"][str(m)] = {"ms_per_pass": ms, "gbps": nbytes / (ms * 1e-3) / 1e9,
                                 "frac_of_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                                 "tokens_per_s": m / (ms * 1e-3), "vs_batch1_tokens_per_s": m * one_ms / ms}
        log(f"[bench] decode m={m}: {ms:.3f} ms per pass, {out['tokens'][str(m)]['gbps']:.0f} GB/s")
        del plan, mj, xs
    # dense bf16 weights: 8 layers (about 13 GB), scaled to `layers`
    dl = min(8, layers)
    Ws = [synth.normal_bf16((N, K), 0.02, 30_000_000 + i, dev) for i, (N, K) in enumerate(shapes[:7 * dl])]
    dense = {"layers_timed": dl, "how": "torch.nn.functional.linear on bf16 weights, one call per linear"}
    for m in (1, 16):
        xa = synth.normal_bf16((m, 8192), 1.0, 31_000_000 + m, dev)
        xd = synth.normal_bf16((m, 22016), 1.0, 32_000_000 + m, dev)

        def run():
            for W in Ws:
                torch.nn.functional.linear(xd if W.shape[1] == 22016 else xa, W)

        ms = timed(run) * layers / dl
        nf4 = out["tokens"][str(m)]["ms_per_pass"]
        dense[f"m{m}"] = {"ms_per_pass": ms, "gbps": sum(2 * N * K for N, K in shapes) / (ms * 1e-3) / 1e9,
                          "tokens_per_s": m / (ms * 1e-3), "nf4_speedup": ms / nf4}
        log(f"[bench] dense bf16 decode m={m}: {ms:.3f} ms per {layers}-layer pass (NF4 {ms / nf4:.2f}x faster)")
    out["bf16_dense"] = dense
    del Ws
    torch.cuda.empty_cache()
    return out


# the device code of each kernel whose traffic is reported: its source file
# and the device headers it includes
KERNEL_SOURCES = {"fwd_kernel": ["gemm_nf4.hip"], "dx_kernel": ["gemm_nf4.hip"],
                  "quantize_kernel": ["quantize.hip"], "gemv_kernel": ["gemv.hip"]}
DEVICE_HEADERS = ["device.h", "lds.h"]


def source_digest(kernel):
    """Digest of a kernel's device code: traffic figures taken on other code are not reported."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "bit_quantized_finetuning_nf4_amd", "csrc")
    for f in KERNEL_SOURCES[kernel] + DEVICE_HEADERS:
        h.update(f.encode())
        h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


def traffic_for(kernel):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source (else None)."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    e = d.get(kernel)
    if not e or e.get("source_digest") != source_digest(kernel):
        return None
    return e.get("hbm_bytes_per_launch")


# rocprofv3 kernel name -> bench kernel; a launch of the fused GEMMs may add a
# half-tile tail dispatch, whose bytes count towards that launch
TRAFFIC_KERNELS = {"nf4_fwd_r_kernel": "fwd_kernel", "nf4_fwd_kernel": "fwd_kernel", "nf4_dx_kernel": "dx_kernel",
                   "quantize_kernel": "quantize_kernel", "nf4_gemv_kernel": "gemv_kernel"}
TAIL_KERNELS = {"nf4_fwd_n32_kernel": "fwd_kernel", "nf4_dx_half_kernel": "dx_kernel"}


def summarize_pmc(fetch_csv, write_csv, copy_mib):
    """Average FETCH_SIZE / WRITE_SIZE (KiB per dispatch) per kernel from two
    rocprofv3 counter runs, each scaled by what the same counter reads for the
    elementwise copy probe of known size (copy_mib MiB read and written)."""
    import csv
    import re

    def per_kernel(path, counter):
        acc = {}
        for row in csv.DictReader(open(path)):
            if row["Counter_Name"] != counter:
                continue
            name = row["Kernel_Name"]
            m = re.search(r"(\w+_kernel)\b", name)
            key = m.group(1) if m else name
            if "neg_kernel" in name or ("elementwise" in name and "neg" in name):
                key = "copy_probe"
            acc.setdefault(key, {}).setdefault(row["Dispatch_Id"], 0.0)
            acc[key][row["Dispatch_Id"]] += float(row["Counter_Value"])
        # bytes summed over the dispatches, and the dispatch count
        return {k: (sum(v.values()) * 1024.0, len(v)) for k, v in acc.items()}

    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")
    probe = copy_mib * 1024 * 1024
    f_scale = probe / (fetch["copy_probe"][0] / fetch["copy_probe"][1])
    w_scale = probe / (write["copy_probe"][0] / write["copy_probe"][1])
    out = {"_note": "HBM bytes per launch = FETCH_SIZE x fetch_scale + WRITE_SIZE x write_scale, summed over the "
                    "dispatches of one bench run (a fused GEMM's half-tile tail dispatches included) and divided by "
                    "the number of launches; scales from an elementwise copy of copy_probe_bytes",
           "copy_probe_bytes": probe, "fetch_scale": f_scale, "write_scale": w_scale}
    for k, name in TRAFFIC_KERNELS.items():
        if k in fetch and k in write:
            tails = [t for t, n in TAIL_KERNELS.items() if n == name]
            fb = fetch[k][0] + sum(fetch[t][0] for t in tails if t in fetch)
            wb = write[k][0] + sum(write[t][0] for t in tails if t in write)
            fpl, wpl = fb / fetch[k][1] * f_scale, wb / write[k][1] * w_scale
            out[name] = {"source_digest": source_digest(name), "fetch_bytes_per_launch": fpl,
                         "write_bytes_per_launch": wpl, "hbm_bytes_per_launch": fpl + wpl}
    return out


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_MFMA", "SQ_INSTS_VALU",
                 "SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE", "GRBM_COUNT")


def summarize_mfma(csv_path, simds=1024, xccs=8):
    """Per-kernel MFMA figures from one rocprofv3 counter run of MFMA_COUNTERS:
    MFMA busy fraction (busy SIMD-cycles over SIMDs x active cycles of one
    XCC), bf16 MFMA flops per launch (MOPS x 512), VALU instructions per MFMA
    instruction, and the shader clock the active cycles imply over the
    dispatch's duration.  The counter values in the file are sums over all
    XCCs, shader engines and SIMDs."""
    import csv
    import re

    per = {}
    for row in csv.DictReader(open(csv_path)):
        m = re.search(r"(\w+_kernel)\b", row["Kernel_Name"])
        if not m or not any(k in row["Kernel_Name"] for k in ("qlora", "nf4", "skinny")):
            continue
        d = per.setdefault(m.group(1), {}).setdefault(row["Dispatch_Id"], {})
        d[row["Counter_Name"]] = d.get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
        d["ns"] = int(row["End_Timestamp"]) - int(row["Start_Timestamp"])
    out = {"_note": "from one rocprofv3 --pmc run of " + " ".join(MFMA_COUNTERS) + "; averages over the "
                    "dispatches; busy = SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x GRBM_GUI_ACTIVE / XCCs); "
                    "clock = GRBM_GUI_ACTIVE / XCCs / duration",
           "simds": simds, "xccs": xccs}
    for k, ds in sorted(per.items()):
        ds = [d for d in ds.values() if all(c in d for c in MFMA_COUNTERS) and d["ns"] > 0]
        if not ds:
            continue
        avg = lambda f: sum(f(d) for d in ds) / len(ds)
        out[k] = {"dispatches": len(ds),
                  "avg_us": avg(lambda d: d["ns"] / 1e3),
                  "mfma_busy": avg(lambda d: d["SQ_VALU_MFMA_BUSY_CYCLES"] / (simds * d["GRBM_GUI_ACTIVE"] / xccs)),
                  "bf16_mfma_tflop_per_launch": avg(lambda d: d["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / 1e12),
                  "valu_per_mfma": avg(lambda d: d["SQ_INSTS_VALU"] / max(d["SQ_INSTS_MFMA"], 1.0)),
                  "clock_ghz": avg(lambda d: d["GRBM_GUI_ACTIVE"] / xccs / d["ns"])}
    return out


def cpu_baseline(lin, M, r, alpha, dev_tensors, min_seconds=10.0, max_reps=20):
    """fp64 oracle fwd+bwd on one linear of the workload (host cores)."""
    import numpy as np
    import oracle
    from tests.helpers import torch_to_bits
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    name, N, K = lin
    W, X, A, B, dY = (dev_tensors[k] for k in ("W", "X", "A", "B", "dY"))
    wb = torch_to_bits(W)
    c, a, s = oracle.quantize(wb)
    Wd = oracle.bf16_bits_to_f64(oracle.dequant(c, a, s, wb.size)).reshape(N, K)
    f = lambda t: oracle.bf16_bits_to_f64(torch_to_bits(t)).reshape(tuple(t.shape))
    Xf, Af, Bf, dYf = f(X), f(A), f(B), f(dY)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.linear_fwd(Wd, Xf, Af, Bf, alpha)
        oracle.linear_bwd(Wd, Xf, dYf, Af, Bf, alpha)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or reps >= max_reps:
            break
    fl = linear_flops(M, N, K, r) * reps
    return {"value": fl / el / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 numpy forward+backward of the {name} linear ({N}x{K}, M={M}, r={r}) x{reps}, "
                      f"{el:.1f} s; weight quantized and dequantized by the oracle beforehand (not timed)",
            "host_cpu_count": os.cpu_count()}


def codebook_study(L, dev, q_bytes, reps=5):
    """Quantize the layer set with each 4-bit codebook (HBM rate, same bytes
    as NF4) and the relative RMS error of its dequantized q weight: the
    pages' comparison of NF4 with FP4 and Int4, on the synthetic weights."""
    import torch
    from bit_quantized_finetuning_nf4_amd import ops
    qs = [ops.QuantizedWeight.empty(o["N"], o["K"], dev) for o in L]
    W0 = L[0]["W"]
    back = torch.empty_like(W0)
    ref = W0.double()
    res = {}
    for cb in ("nf4", "fp4", "int4"):
        for o, q in zip(L, qs):
            ops.quantize(o["W"], out=q, codebook=cb)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            for o, q in zip(L, qs):
                ops.quantize(o["W"], out=q, codebook=cb)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        ops.dequant(qs[0], out=back)
        err = ((back.double() - ref).pow(2).mean().sqrt() / ref.pow(2).mean().sqrt()).item()
        res[cb] = {"quantize_ms": ms, "quantize_gbps": q_bytes / (ms * 1e-3) / 1e9,
                   f"rel_rmse_{L[0]['name']}": err}
    del qs, back, ref
    return res


def optimizer_study(L, r, dev, reps=5):
    """The AdamW step over every LoRA value of the layer set (one flat fp32
    buffer each for p, g, m, v and a bf16 copy; 30 bytes per value), with the
    moments on the device and, as a paged optimizer's CPU-resident states,
    in pinned host memory."""
    import torch
    from bit_quantized_finetuning_nf4_amd import ops
    n = sum(r * (o["N"] + o["K"]) for o in L)
    g = torch.randn(n, device=dev) * 1e-3
    p = torch.randn(n, device=dev) * 1e-2
    pb = torch.empty(n, dtype=torch.bfloat16, device=dev)
    res = {"values": n, "bytes_per_value": 30}
    for where in ("device", "pinned_host"):
        if where == "device":
            m, v = torch.zeros(n, device=dev), torch.zeros(n, device=dev)
        else:
            m, v = torch.zeros(n, pin_memory=True), torch.zeros(n, pin_memory=True)
        ops.adamw(p, g, m, v, 1, p_bf16=pb)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for t in range(reps):
            ops.adamw(p, g, m, v, t + 2, p_bf16=pb)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        res[f"{where}_moments"] = {"ms": ms, "gbps": 30 * n / (ms * 1e-3) / 1e9}
        del m, v
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama65b", choices=["llama65b", "llama13b", "llama7b"])
    ap.add_argument("--decode-layers", type=int, default=80)
    ap.add_argument("--decode-passes", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-codebook-study", action="store_true",
                    help="skip the side studies after the timed steps: the layer set quantized with FP4 and "
                         "Int4, the AdamW step over its LoRA values, and decode of 2-16 tokens (and of dense bf16 "
                         "weights) over the decode layers")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the timed steps, run one elementwise copy (negation) of this many MiB: "
                         "a kernel of known traffic for scaling the FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="do not run: turn two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, "
                         "WRITE_SIZE) of a --copy-probe-mib run into profiles/traffic.json on stdout")
    ap.add_argument("--summarize-mfma", metavar="CSV",
                    help="do not run: per-kernel MFMA busy fraction, MFMA flops, VALU per MFMA and implied "
                         "clock from a rocprofv3 --pmc counter_collection.csv of the MFMA_COUNTERS, on stdout")
    args = ap.parse_args()
    if args.summarize_mfma:
        print(json.dumps(summarize_mfma(args.summarize_mfma), indent=1))
        return
    if args.summarize_pmc:
        print(json.dumps(summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.copy_probe_mib), indent=1))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(sharding is described in DESIGN.md); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from bit_quantized_finetuning_nf4_amd import ops, synth
    from bit_quantized_finetuning_nf4_amd import _lib

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = synth.LAYER_SETS[args.workload]
    M, r, alpha = cfg["M"], cfg["r"], cfg["alpha"]
    set_index = {"llama7b": 1, "llama13b": 2, "llama65b": 3}[args.workload]
    lins = cfg["linears"]
    log(f"[bench] workload {args.workload}: {len(lins)} linears, M={M}, r={r}")

    # ---- inputs and outputs, resident before timing ----
    L = []
    for i, (name, N, K) in enumerate(lins):
        t = synth.linear_inputs(N, K, M, r, synth.layer_set_seed(set_index, i), dev, outliers=cfg["outliers"])
        q = ops.QuantizedWeight.empty(N, K, dev)
        o = dict(name=name, N=N, K=K, q=q, **t,
                 x=t["X"][0].contiguous(),
                 Y=torch.empty(M, N, dtype=torch.bfloat16, device=dev),
                 U=torch.empty(M, r, dtype=torch.bfloat16, device=dev),
                 G=torch.empty(M, r, dtype=torch.bfloat16, device=dev),
                 dX=torch.empty(M, K, dtype=torch.bfloat16, device=dev),
                 dA=torch.empty(r, K, dtype=torch.float32, device=dev),
                 dB=torch.empty(N, r, dtype=torch.float32, device=dev))
        L.append(o)
    ws_bytes = max(ops.workspace_bytes(_lib.QLORA_OP_LORA, M, o["N"], o["K"], r) for o in L)
    ws = ops.workspace(ws_bytes, dev)
    plan = ops.GemvPlan([ops.GemvJob(o["q"], o["x"], o["A"], o["B"], alpha) for o in L])
    torch.cuda.synchronize()

    fl_step = sum(linear_flops(M, o["N"], o["K"], r) for o in L)
    fl_fwd = [2 * M * o["N"] * o["K"] + 2 * M * o["N"] * r for o in L]   # fused forward GEMM
    fl_dx = [2 * M * o["N"] * o["K"] + 2 * M * o["K"] * r for o in L]    # fused dX GEMM
    q_bytes = sum(2 * o["N"] * o["K"] + o["q"].nbytes() for o in L)
    g_bytes = sum(gemv_bytes(o["N"], o["K"], r) for o in L)

    E = lambda: torch.cuda.Event(enable_timing=True)
    record = []

    def step(timed):
        ev = dict(p=[E() for _ in range(5)], f=[(E(), E()) for _ in L], d=[(E(), E()) for _ in L]) if timed else None
        if timed:
            ev["p"][0].record()
        for o in L:
            ops.quantize(o["W"], out=o["q"])
        if timed:
            ev["p"][1].record()
        for i, o in enumerate(L):
            ops.lora_down(o["X"], o["A"], U=o["U"], ws=ws)
            if timed:
                ev["f"][i][0].record()
            ops.nf4_fwd(o["q"], o["X"], o["U"], o["B"], alpha, out=o["Y"])
            if timed:
                ev["f"][i][1].record()
        if timed:
            ev["p"][2].record()
        for i, o in enumerate(L):
            ops.lora_dy_b(o["dY"], o["B"], G=o["G"], ws=ws)
            if timed:
                ev["d"][i][0].record()
            ops.nf4_dx(o["q"], o["dY"], o["G"], o["A"], alpha, out=o["dX"])
            if timed:
                ev["d"][i][1].record()
            ops.lora_grads(o["X"], o["dY"], o["U"], o["G"], alpha, dA=o["dA"], dB=o["dB"], ws=ws)
        if timed:
            ev["p"][3].record()
        plan()
        if timed:
            ev["p"][4].record()
            record.append(ev)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * 1024 * 1024 // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    ph = {"quantize": 0.0, "forward": 0.0, "backward": 0.0, "decode_gemv": 0.0}
    fwd_ms, dx_ms = 0.0, 0.0
    for ev in record:
        p = ev["p"]
        ph["quantize"] += p[0].elapsed_time(p[1])
        ph["forward"] += p[1].elapsed_time(p[2])
        ph["backward"] += p[2].elapsed_time(p[3])
        ph["decode_gemv"] += p[3].elapsed_time(p[4])
        fwd_ms += sum(a.elapsed_time(b) for a, b in ev["f"])
        dx_ms += sum(a.elapsed_time(b) for a, b in ev["d"])
    K_ = args.steps
    ph = {k: v / K_ for k, v in ph.items()}
    fwd_ms /= K_
    dx_ms /= K_
    fwd_tf = sum(fl_fwd) / (fwd_ms * 1e-3) / 1e12
    dx_tf = sum(fl_dx) / (dx_ms * 1e-3) / 1e12
    kernels = {
        "fwd_kernel": {"launches_per_step": len(L), "avg_launch_ms": fwd_ms / len(L), "tflops": fwd_tf,
                       "flops_per_step": sum(fl_fwd)},
        "dx_kernel": {"launches_per_step": len(L), "avg_launch_ms": dx_ms / len(L), "tflops": dx_tf,
                      "flops_per_step": sum(fl_dx)},
    }
    dom = "dx_kernel" if dx_ms >= fwd_ms else "fwd_kernel"
    k = kernels[dom]
    traffic = traffic_for(dom)
    roof = {"kernel": dom, "bound": "mfma", "achieved": k["tflops"], "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": k["tflops"] / PEAK_BF16_TFLOPS,
            "traffic": traffic,
            "per_launch": "flops of the fused GEMM = 2MNK + 2Mr(N or K) for each of the 7 linears; "
                          "achieved = their sum / the sum of the launches' HIP-event durations"}
    value = fl_step / (ms_step * 1e-3) / 1e12
    out = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{args.workload} layer set: " + ", ".join(f"{o['name']} {o['N']}x{o['K']}" for o in L)
                   + f"; M={M} tokens; LoRA r={r} alpha={alpha}; NF4 blocksize 64, 8-bit double quant per 256 blocks"
                   + "; step = quantize + fwd + bwd + batch-1 decode GEMV",
                   "global_batch": M, "seq_len": M, "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "phases_ms": ph,
        "kernels": kernels,
        "fwd_bwd_tflops": fl_step / ((ph["forward"] + ph["backward"]) * 1e-3) / 1e12,
        "quantize_gbps": q_bytes / (ph["quantize"] * 1e-3) / 1e9,
        "layer_gemv_gbps": g_bytes / (ph["decode_gemv"] * 1e-3) / 1e9,
    }
    log(f"[bench] step {ms_step:.3f} ms, {value:.1f} TFLOP/s; phases {ph}")
    if not args.no_codebook_study:
        out["codebooks"] = codebook_study(L, dev, q_bytes)
        log(f"[bench] codebooks {out['codebooks']}")
        out["optimizer"] = optimizer_study(L, r, dev)
        log(f"[bench] optimizer {out['optimizer']}")

    # ---- 80-layer batch-1 decode pass (about 65e9 weights) ----
    if args.decode_layers > 0:
        del L, plan
        torch.cuda.empty_cache()
        c65 = synth.LAYER_SETS["llama65b"]
        jobs, nbytes = [], 0
        for layer in range(args.decode_layers):
            x_attn = synth.normal_bf16((8192,), 1.0, 10_000_000 + 2 * layer, dev)
            x_down = synth.normal_bf16((22016,), 1.0, 10_000_001 + 2 * layer, dev)
            for i, (name, N, K) in enumerate(c65["linears"]):
                seed = synth.layer_set_seed(4, i, layer=layer + 1)
                W = synth.normal_bf16((N, K), 0.02, seed * 16, dev, outliers=c65["outliers"])
                q = ops.quantize(W)
                del W
                A = synth.normal_bf16((r, K), 0.01, seed * 16 + 1, dev)
                B = synth.normal_bf16((N, r), 0.01, seed * 16 + 2, dev)
                jobs.append(ops.GemvJob(q, x_down if name == "down" else x_attn, A, B, alpha))
                nbytes += gemv_bytes(N, K, r)
            if layer % 20 == 19:
                log(f"[bench] decode weights: {layer + 1} layers quantized")
        dplan = ops.GemvPlan(jobs)
        for _ in range(2):
            dplan()
        torch.cuda.synchronize()
        evs = [(E(), E()) for _ in range(args.decode_passes)]
        for a, b in evs:
            a.record()
            dplan()
            b.record()
        torch.cuda.synchronize()
        pass_ms = sum(a.elapsed_time(b) for a, b in evs) / len(evs)
        gbps = nbytes / (pass_ms * 1e-3) / 1e9
        out["decode"] = {"workload": f"{args.decode_layers} layers x 7 LLaMA-65B-shaped linears, batch 1, "
                                     f"LoRA r={r} fused; {len(jobs)} jobs in one grouped call",
                         "bytes_per_pass": nbytes, "ms_per_pass": pass_ms, "gbps": gbps,
                         "frac_of_hbm_peak": gbps / PEAK_HBM_GBPS}
        log(f"[bench] decode pass {pass_ms:.3f} ms, {gbps:.0f} GB/s")
        del dplan
        if not args.no_codebook_study:
            out["decode_batch"] = decode_batch_study(jobs, args.decode_layers, r, alpha, args.decode_passes, dev)
        del jobs
        torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        lin = synth.LAYER_SETS[args.workload]["linears"][0]
        t = synth.linear_inputs(lin[1], lin[2], M, r, synth.layer_set_seed(set_index, 0), dev,
                                outliers=cfg["outliers"])
        log("[bench] timing the CPU oracle ...")
        out["cpu_baseline"] = cpu_baseline(lin, M, r, alpha, t)
        log(f"[bench] cpu oracle {out['cpu_baseline']['value']:.4f} TFLOP/s")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
