#!/usr/bin/env python3
"""Throughput of the QLoRA NF4 linear hot path on one MI355X.

One step is one pass of every stage of the path over the LLaMA-65B-shaped
layer set (q/k/v/o 8192x8192, gate/up 22016x8192, down 8192x22016; 4096
tokens; LoRA r = 64, alpha = 16; NF4 blocksize 64 with 8-bit double
quantization over 256-block groups):

  1. quantize the seven bf16 weights (block absmax, NF4 codes, 8-bit absmax
     codes against fp32 group scales);
  2. forward, per group of linears that read the same input (q/k/v, o,
     gate/up, down): U = X A^T for the group's stacked adapters; the group's
     weights dequantized once into one bf16 stack; one dense bf16 GEMM
     Y = X deq(W)^T + s U B^T over the stack, each row group with its own
     adapter;
  3. backward, per group: G = dY B; the weights dequantized once, transposed,
     side by side; one dense GEMM dX = dY deq(W) + s G A contracting over the
     group's outputs; dA = s G^T X and dB = s dY^T U;
  4. batch-1 decode: y = deq(W) x + s B (A x) for the seven linears in one
     grouped call.

Steps 2 and 3 are the building blocks of qlora_group_fwd / qlora_group_bwd.
The same step with one product per linear (the staged path of
qlora_linear_fwd / _bwd, taken from 1024 tokens on), and with the fused path
(W decoded inside each 256-token product tile), is timed beside it.

`value` is the fwd+bwd algorithmic work, sum over linears of
4MNK + 6Mr(N+K) flops, divided by the wall time of whole steps (quantize and
decode included).  HIP events on the launch stream bracket every dense GEMM
call; their flops over their summed durations is the roofline figure
against the dense bf16 MFMA peak.  The 7B and 13B layer sets and the small
1024x1024 case are timed the same way (fwd + bwd phases), dequantization is
timed on the 65B gate weight (360 MB of bf16 out), and the shader clock is
sampled with the box's smi tool while steps run.  The CPU oracle (fp64
numpy) is timed on one linear of the same workload.  With --decode-layers > 0
the 80-layer decode pass (about 65e9 weights) is also timed and reported as
HBM bandwidth.

Inputs are synthetic and seeded (bit_quantized_finetuning_nf4_amd.synth);
they are resident in HBM before timing starts.
"""

import argparse
import ctypes
import hashlib
import json
import os
import subprocess
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E
# Untimed decode passes before the timed ones: after an idle gap the first
# passes run 10-20 % slower and speed up pass by pass (the clocks ramp back
# up); ten passes (about 70 ms) reach the steady rate a serving loop sees.
DECODE_WARMUP = 10
METRIC = "QLoRA linear fwd+bwd TFLOP/s at 7B/65B shapes; NF4 decode GEMV HBM GB/s"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# hipEventCreateWithFlags flag (hip_runtime_api.h): no system-scope fence.
# A default event (torch.cuda.Event) writes back and invalidates the caches
# when it is recorded; between two kernels that left a gap of about 6 us,
# more than 4 % of a 7B-set step with its 21 events.  Events made for timing
# do not need the fence: the timed loops end with a full device
# synchronization before any result is read on the host.
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class TimingEvent:
    """A HIP timing event recorded on torch's current stream (the stream the
    library's kernels are launched on), from the HIP runtime torch loaded."""
    _hip = None

    @classmethod
    def hip(cls):
        if cls._hip is None:
            import torch
            torch.cuda.init()
            path = next((ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64" in ln), None)
            if path is None:
                raise RuntimeError("the HIP runtime is not loaded in this process")
            h = ctypes.CDLL(path)
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            h.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = h
        return cls._hip

    def __init__(self):
        import torch
        self._torch = torch
        self.h = ctypes.c_void_p()
        rc = self.hip().hipEventCreateWithFlags(
            ctypes.byref(self.h), HIP_EVENT_DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self):
        rc = self.hip().hipEventRecord(self.h, ctypes.c_void_p(self._torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end):
        """Milliseconds from this event to `end` (both recorded and done)."""
        ms = ctypes.c_float()
        rc = self.hip().hipEventElapsedTime(ctypes.byref(ms), self.h, end.h)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        if self._hip is not None and self.h:
            self._hip.hipEventDestroy(self.h)


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
    E = TimingEvent

    def timed(fn):
        for _ in range(DECODE_WARMUP):
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
KERNEL_SOURCES = {"fwd_kernel": ["gemm_nf4.hip", "gemm_common.h"], "dx_kernel": ["gemm_nf4.hip", "gemm_common.h"],
                  "dense_gemm": ["gemm_bf16.hip", "gemm_common.h"],
                  "quantize_kernel": ["quantize.hip"], "gemv_kernel": ["gemv.hip"],
                  "dequant_kernel": ["quantize.hip"], "dequant_t_kernel": ["quantize.hip"]}
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


def mfma_counters_for(kernel, source):
    """MFMA busy fraction, VALU per MFMA and clock of a kernel from the
    committed counter summary, if it was taken on the current source."""
    p = os.path.join(ROOT, "profiles", "mfma.json")
    if not os.path.exists(p):
        return None
    e = json.load(open(p)).get(kernel)
    if not e or e.get("source_digest") != source_digest(source):
        return None
    return e


# rocprofv3 kernel name -> bench kernel; a launch of the fused GEMMs may add a
# half-tile tail dispatch, whose bytes count towards that launch
TRAFFIC_KERNELS = {"nf4_fwd_r_kernel": "fwd_kernel", "nf4_dx_kernel": "dx_kernel", "bf16_fwd_kernel": "dense_gemm",
                   "quantize_kernel": "quantize_kernel", "nf4_gemv_kernel": "gemv_kernel",
                   "dequant_kernel": "dequant_kernel", "dequant_t_kernel": "dequant_t_kernel"}
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
    # steps in the run: the step's decode GEMV is one dispatch per step
    steps = fetch.get("nf4_gemv_kernel", (0, 0))[1]
    for k, name in TRAFFIC_KERNELS.items():
        if k in fetch and k in write:
            tails = [t for t, n in TAIL_KERNELS.items() if n == name]
            fb = fetch[k][0] + sum(fetch[t][0] for t in tails if t in fetch)
            wb = write[k][0] + sum(write[t][0] for t in tails if t in write)
            # the dense GEMM is timed per product call (8 per grouped step, one
            # or two dispatches each): its bytes are per call, like `achieved`
            calls = steps * 2 * len(GROUPS) if name == "dense_gemm" and steps else fetch[k][1]
            fpl, wpl = fb / calls * f_scale, wb / calls * w_scale
            out[name] = {"source_digest": source_digest(name), "fetch_bytes_per_launch": fpl,
                         "write_bytes_per_launch": wpl, "hbm_bytes_per_launch": fpl + wpl,
                         "dispatches": fetch[k][1], "launches": calls}
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
        if not m or not any(k in row["Kernel_Name"] for k in ("qlora", "nf4", "skinny", "bf16_fwd")):
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
    """Quantize the layer set with each 4-bit codebook and each second-level
    format of the block constants (HBM rate, same bytes as NF4 with the
    linear code) and the relative RMS error of its dequantized q weight: the
    pages' comparison of NF4 with FP4 and Int4, and the linear against the
    FP8 second level, on the synthetic weights."""
    import torch
    from bit_quantized_finetuning_nf4_amd import ops
    qs = [ops.QuantizedWeight.empty(o["N"], o["K"], dev) for o in L]
    W0 = L[0]["W"]
    back = torch.empty_like(W0)
    ref = W0.double()
    res = {}
    for cb, fmt in (("nf4", "linear"), ("fp4", "linear"), ("int4", "linear"), ("nf4", "fp8")):
        for o, q in zip(L, qs):
            ops.quantize(o["W"], out=q, codebook=cb, absmax_format=fmt)
        torch.cuda.synchronize()
        a, b = TimingEvent(), TimingEvent()
        a.record()
        for _ in range(reps):
            for o, q in zip(L, qs):
                ops.quantize(o["W"], out=q, codebook=cb, absmax_format=fmt)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        ops.dequant(qs[0], out=back)
        err = ((back.double() - ref).pow(2).mean().sqrt() / ref.pow(2).mean().sqrt()).item()
        res[cb if fmt == "linear" else f"{cb}_fp8_absmax"] = {
            "quantize_ms": ms, "quantize_gbps": q_bytes / (ms * 1e-3) / 1e9, f"rel_rmse_{L[0]['name']}": err}
    del qs, back, ref
    return res


def optimizer_study(L, r, dev, reps=5):
    """The AdamW step over every LoRA value of the layer set (one flat fp32
    buffer each for p, g, m, v and a bf16 copy; 30 bytes per value), with the
    moments on the device and, as a paged optimizer's CPU-resident states,
    in pinned host memory; then the paged optimizer (qlora_paged_adamw) on
    the 14 adapter tensors with its moments in a pinned host backing store,
    at a device budget that holds them all and at a quarter of that."""
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
        a, b = TimingEvent(), TimingEvent()
        a.record()
        for t in range(reps):
            ops.adamw(p, g, m, v, t + 2, p_bf16=pb)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        res[f"{where}_moments"] = {"ms": ms, "gbps": 30 * n / (ms * 1e-3) / 1e9}
        del m, v
    # paged: the adapters of the set as separate tensors (A and B per linear)
    sizes = [r * o["K"] for o in L] + [o["N"] * r for o in L]
    ps = [torch.randn(k, device=dev) * 1e-2 for k in sizes]
    gs = [torch.randn(k, device=dev) * 1e-3 for k in sizes]
    bs = [torch.empty(k, dtype=torch.bfloat16, device=dev) for k in sizes]
    state = sum(2 * (-(-4 * k // 256) * 256) for k in sizes)
    copy_stream = torch.cuda.Stream()
    paged = {"tensors": len(sizes), "moment_bytes": state}
    for name, budget in (("all_resident", state), ("quarter_budget", state // 4)):
        opt = ops.PagedAdamW(ps, gs, budget, p_bf16=bs, copy_stream=copy_stream)
        opt.step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            opt.step()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / reps
        paged[name] = {"budget_bytes": budget, "layout": opt.layout, "ms_per_step": ms}
        del opt
    res["paged"] = paged
    del ps, gs, bs
    return res


class ClockSampler:
    """Samples the shader clock (MHz, mean over the XCDs) with the box's smi
    tool in a subprocess loop while the GPU works; the median of the samples
    taken inside [start, stop] is the clock observed during the timed steps."""

    def __init__(self):
        self.samples, self._stop, self.tool = [], threading.Event(), None
        for tool in (["amd-smi", "metric", "-c", "--json"], ["rocm-smi", "--showclocks", "--json"]):
            try:
                if self._read(tool) is not None:
                    self.tool = tool
                    break
            except Exception:
                pass

    @staticmethod
    def _read(tool):
        out = subprocess.run(tool, capture_output=True, text=True, timeout=5).stdout
        j = json.loads(out[out.index("{") if out.lstrip().startswith("{") else out.index("["):])
        vals = []

        def walk(o):
            if isinstance(o, dict):
                for k, v in o.items():
                    if k.startswith("gfx_") and isinstance(v, dict) and isinstance(v.get("clk"), dict):
                        vals.append(float(v["clk"]["value"]))
                    elif "sclk clock speed" in k and isinstance(v, str):
                        vals.append(float(v.strip("()Mhz")))
                    else:
                        walk(v)
            elif isinstance(o, list):
                for v in o:
                    walk(v)
        walk(j)
        return sum(vals) / len(vals) if vals else None

    def _run(self):
        while not self._stop.is_set():
            try:
                v = self._read(self.tool)
                if v is not None:
                    self.samples.append(v)
            except Exception:
                pass

    def __enter__(self):
        if self.tool:
            self._t = threading.Thread(target=self._run, daemon=True)
            self._t.start()
        return self

    def __exit__(self, *a):
        self._stop.set()
        if self.tool:
            self._t.join(timeout=10)

    def result(self):
        if not self.samples:
            return None
        v = sorted(self.samples)
        return {"tool": " ".join(self.tool), "samples": len(v), "median_mhz": v[len(v) // 2],
                "min_mhz": v[0], "max_mhz": v[-1]}


# linears of a LLaMA layer that read the same input: the attention
# projections q/k/v read the normalised hidden state, gate/up the second one
GROUPS = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))


def dy_late(dY):
    """The staged backward's order, as qlora_linear_bwd / qlora_group_bwd take
    it: G = dY B after the transposed dequantization (right before the dX
    product, so dY is still in the last-level cache there) when dY is at most
    128 MB, else first."""
    return dY.numel() * 2 <= (128 << 20)


class LayerSet:
    """Inputs, outputs and scratch of one layer set, resident on the device,
    and one step of the path over it: grouped, per-linear staged, or fused
    products."""

    def __init__(self, name, dev, with_decode=True):
        import torch
        from bit_quantized_finetuning_nf4_amd import ops, synth
        from bit_quantized_finetuning_nf4_amd import _lib
        self.ops, self.torch = ops, torch
        cfg = synth.LAYER_SETS[name]
        self.name, self.M, self.r, self.alpha = name, cfg["M"], cfg["r"], cfg["alpha"]
        set_index = {"small": 0, "llama7b": 1, "llama13b": 2, "llama65b": 3}[name]
        M, r = self.M, self.r
        self.L = []
        for i, (lname, N, K) in enumerate(cfg["linears"]):
            t = synth.linear_inputs(N, K, M, r, synth.layer_set_seed(set_index, i), dev, outliers=cfg["outliers"])
            o = dict(name=lname, N=N, K=K, q=ops.QuantizedWeight.empty(N, K, dev), **t,
                     x=t["X"][0].contiguous(),
                     Y=torch.empty(M, N, dtype=torch.bfloat16, device=dev),
                     U=torch.empty(M, r, dtype=torch.bfloat16, device=dev),
                     G=torch.empty(M, r, dtype=torch.bfloat16, device=dev),
                     dX=torch.empty(M, K, dtype=torch.bfloat16, device=dev),
                     dA=torch.empty(r, K, dtype=torch.float32, device=dev),
                     dB=torch.empty(N, r, dtype=torch.float32, device=dev))
            self.L.append(o)
        # linears that read the same input run as one group on the grouped path
        names = [o["name"] for o in self.L]
        parts = GROUPS if all(n in names for grp in GROUPS for n in grp) else tuple((n,) for n in names)
        self.groups = []
        for grp in parts:
            mem = [self.L[names.index(n)] for n in grp]
            G, N, K = len(mem), mem[0]["N"], mem[0]["K"]
            cat = lambda key, dim=0: torch.cat([o[key] for o in mem], dim=dim).contiguous() if G > 1 else mem[0][key]
            self.groups.append(dict(
                name="/".join(grp), G=G, N=N, K=K, qs=[o["q"] for o in mem], X=mem[0]["X"],
                A=cat("A"), B=cat("B"), dY=cat("dY", 1),
                Y=torch.empty(M, G * N, dtype=torch.bfloat16, device=dev),
                U=torch.empty(M, G * r, dtype=torch.bfloat16, device=dev),
                Gm=torch.empty(M, G * r, dtype=torch.bfloat16, device=dev),
                dX=torch.empty(M, K, dtype=torch.bfloat16, device=dev),
                dA=torch.empty(G * r, K, dtype=torch.float32, device=dev),
                dB=torch.empty(G * N, r, dtype=torch.float32, device=dev)))
        self.ws = ops.workspace(max([ops.workspace_bytes(_lib.QLORA_OP_LORA, M, o["N"], o["K"], r) for o in self.L]
                                    + [ops.workspace_bytes(_lib.QLORA_OP_GROUP_LORA, M, g["N"], g["K"], r, g["G"])
                                       for g in self.groups]
                                    + [ops.workspace_bytes(_lib.QLORA_OP_BF16_DX, M, o["N"], o["K"], r, 1)
                                       for o in self.L]
                                    + [ops.workspace_bytes(_lib.QLORA_OP_BF16_DX, M, g["N"], g["K"], r, g["G"])
                                       for g in self.groups]), dev)
        self.wbuf = torch.empty(max(g["G"] * g["N"] * g["K"] for g in self.groups), dtype=torch.bfloat16,
                                device=dev)
        self.plan = (ops.GemvPlan([ops.GemvJob(o["q"], o["x"], o["A"], o["B"], self.alpha) for o in self.L])
                     if with_decode else None)
        self.fl_step = sum(linear_flops(M, o["N"], o["K"], r) for o in self.L)
        self.fl_fwd = [2 * M * o["N"] * o["K"] + 2 * M * o["N"] * r for o in self.L]
        self.fl_dx = [2 * M * o["N"] * o["K"] + 2 * M * o["K"] * r for o in self.L]
        self.q_bytes = sum(2 * o["N"] * o["K"] + o["q"].nbytes() for o in self.L)
        self.g_bytes = sum(gemv_bytes(o["N"], o["K"], r) for o in self.L)
        for o in self.L:
            ops.quantize(o["W"], out=o["q"])
        torch.cuda.synchronize()

    def units(self, path):
        """The products of one step: one per group on the grouped path, else
        one per linear."""
        return self.groups if path == "grouped" else self.L

    def step(self, path, record=None):
        """One step; with `record` (a list) HIP events bracket the phases and
        every dense (or fused) product call."""
        ops, torch, a, L = self.ops, self.torch, self.alpha, self.L
        E = TimingEvent
        nu = len(self.units(path))
        ev = dict(p=[E() for _ in range(5)], f=[(E(), E()) for _ in range(nu)], d=[(E(), E()) for _ in range(nu)]) \
            if record is not None else None
        mark = (lambda e: e.record()) if ev else (lambda e: None)
        if ev:
            mark(ev["p"][0])
        for o in L:
            ops.quantize(o["W"], out=o["q"])
        if ev:
            mark(ev["p"][1])
        if path == "grouped":
            self._grouped(ev, mark)
        else:
            self._per_linear(path, ev, mark)
        if ev:
            mark(ev["p"][3])
        if self.plan is not None:
            self.plan()
        if ev:
            mark(ev["p"][4])
            record.append(ev)

    def _grouped(self, ev, mark):
        """Forward and backward with q/k/v and gate/up as one group each (the
        building blocks of qlora_group_fwd / _bwd, so the dense products can
        be timed on their own)."""
        ops, a = self.ops, self.alpha
        for i, g in enumerate(self.groups):
            G, N, K = g["G"], g["N"], g["K"]
            ops.lora_down(g["X"], g["A"], U=g["U"], ws=self.ws)
            Wd = ops.group_dequant(g["qs"], out=self.wbuf[:G * N * K].view(G * N, K))
            if ev:
                mark(ev["f"][i][0])
            ops.bf16_group_fwd(Wd, G, g["X"], g["U"], g["B"], a, out=g["Y"])
            if ev:
                mark(ev["f"][i][1])
        if ev:
            mark(ev["p"][2])
        for i, g in enumerate(self.groups):
            G, N, K = g["G"], g["N"], g["K"]
            late = dy_late(g["dY"])
            if not late:
                ops.group_lora_dy_b(g["dY"], g["B"], G, Gm=g["Gm"], ws=self.ws)
            WdT = ops.group_dequant(g["qs"], out=self.wbuf[:G * N * K].view(K, G * N), transposed=True)
            if late:
                ops.group_lora_dy_b(g["dY"], g["B"], G, Gm=g["Gm"], ws=self.ws)
            if ev:
                mark(ev["d"][i][0])
            ops.bf16_group_dx(WdT, G, g["dY"], g["Gm"], g["A"], a, out=g["dX"], ws=self.ws)
            if ev:
                mark(ev["d"][i][1])
            ops.group_lora_grads(g["X"], g["dY"], g["U"], g["Gm"], G, a, dA=g["dA"], dB=g["dB"], ws=self.ws)

    def _per_linear(self, path, ev, mark):
        ops, a, L = self.ops, self.alpha, self.L
        for i, o in enumerate(L):
            ops.lora_down(o["X"], o["A"], U=o["U"], ws=self.ws)
            if path == "staged":
                Wd = ops.dequant(o["q"], out=self.wbuf[:o["N"] * o["K"]].view(o["N"], o["K"]))
                if ev:
                    mark(ev["f"][i][0])
                ops.bf16_fwd(Wd, o["X"], o["U"], o["B"], a, out=o["Y"])
            else:
                if ev:
                    mark(ev["f"][i][0])
                ops.nf4_fwd(o["q"], o["X"], o["U"], o["B"], a, out=o["Y"])
            if ev:
                mark(ev["f"][i][1])
        if ev:
            mark(ev["p"][2])
        for i, o in enumerate(L):
            late = path == "staged" and dy_late(o["dY"])
            if not late:
                ops.lora_dy_b(o["dY"], o["B"], G=o["G"], ws=self.ws)
            if path == "staged":
                WdT = ops.dequant_t(o["q"], out=self.wbuf[:o["N"] * o["K"]].view(o["K"], o["N"]))
                if late:
                    ops.lora_dy_b(o["dY"], o["B"], G=o["G"], ws=self.ws)
                if ev:
                    mark(ev["d"][i][0])
                ops.bf16_dx(WdT, o["dY"], o["G"], o["A"], a, out=o["dX"], ws=self.ws)
            else:
                if ev:
                    mark(ev["d"][i][0])
                ops.nf4_dx(o["q"], o["dY"], o["G"], o["A"], a, out=o["dX"])
            if ev:
                mark(ev["d"][i][1])
            ops.lora_grads(o["X"], o["dY"], o["U"], o["G"], a, dA=o["dA"], dB=o["dB"], ws=self.ws)

    def run(self, path, steps, warmup):
        """Timed steps: wall time per step, phases and per-product times."""
        torch = self.torch
        for _ in range(warmup):
            self.step(path)
        torch.cuda.synchronize()
        record = []
        t0 = time.perf_counter()
        for _ in range(steps):
            self.step(path, record)
        torch.cuda.synchronize()
        ms_step = (time.perf_counter() - t0) * 1e3 / steps
        ph = {"quantize": 0.0, "forward": 0.0, "backward": 0.0, "decode_gemv": 0.0}
        fwd_ms = dx_ms = 0.0
        for ev in record:
            p = ev["p"]
            ph["quantize"] += p[0].elapsed_time(p[1])
            ph["forward"] += p[1].elapsed_time(p[2])
            ph["backward"] += p[2].elapsed_time(p[3])
            ph["decode_gemv"] += p[3].elapsed_time(p[4])
            fwd_ms += sum(x.elapsed_time(y) for x, y in ev["f"])
            dx_ms += sum(x.elapsed_time(y) for x, y in ev["d"])
        ph = {k: v / steps for k, v in ph.items()}
        fwd_ms, dx_ms = fwd_ms / steps, dx_ms / steps
        n = len(self.units(path))
        gemm_tf = (sum(self.fl_fwd) + sum(self.fl_dx)) / ((fwd_ms + dx_ms) * 1e-3) / 1e12
        return {
            "path": path, "ms_per_step": ms_step, "phases_ms": ph,
            "fwd_bwd_tflops": self.fl_step / ((ph["forward"] + ph["backward"]) * 1e-3) / 1e12,
            "products": {
                "kernel": "nf4_fwd_r_kernel / nf4_dx_kernel (fused NF4 GEMMs)" if path == "fused"
                          else "bf16_fwd_kernel (dense bf16 GEMM)",
                "calls_per_step": 2 * n,
                "products": [u["name"] for u in self.units(path)],
                "fwd_avg_call_ms": fwd_ms / n, "dx_avg_call_ms": dx_ms / n,
                "fwd_tflops": sum(self.fl_fwd) / (fwd_ms * 1e-3) / 1e12,
                "dx_tflops": sum(self.fl_dx) / (dx_ms * 1e-3) / 1e12,
                "tflops": gemm_tf, "frac_of_bf16_peak": gemm_tf / PEAK_BF16_TFLOPS},
        }


def dequant_study(dev, reps=10):
    """qlora_dequant and qlora_dequant_t on the 65B gate weight (22016 x 8192:
    0.516 B/weight read, 360 MB of bf16 written, beyond the 256 MB last-level
    cache), as HBM bandwidth."""
    import torch
    from bit_quantized_finetuning_nf4_amd import ops, synth
    N, K = 22016, 8192
    W = synth.normal_bf16((N, K), 0.02, 77, dev, outliers=0.001)
    q = ops.quantize(W)
    out = torch.empty_like(W)
    outT = torch.empty(K, N, dtype=torch.bfloat16, device=dev)
    del W
    nbytes = N * K * 2 + q.nbytes()
    res = {"weight": f"{N}x{K}", "bytes_per_call": nbytes}
    for name, fn in (("dequant", lambda: ops.dequant(q, out=out)), ("dequant_t", lambda: ops.dequant_t(q, out=outT))):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = TimingEvent(), TimingEvent()
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        res[name] = {"ms": ms, "gbps": nbytes / (ms * 1e-3) / 1e9,
                     "frac_of_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS}
    del q, out, outT
    torch.cuda.empty_cache()
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
    ap.add_argument("--no-other-sets", action="store_true",
                    help="skip the 7B, 13B and small layer sets and the dequant leg")
    ap.add_argument("--headline-only", action="store_true",
                    help="time the grouped steps only (no clock window, no per-linear or fused steps): for "
                         "counter runs, where every dispatch should belong to the headline step")
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
        res = summarize_mfma(args.summarize_mfma)
        if "bf16_fwd_kernel" in res:
            res["bf16_fwd_kernel"]["source_digest"] = source_digest("dense_gemm")
        print(json.dumps(res, indent=1))
        return
    if args.summarize_pmc:
        print(json.dumps(summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.copy_probe_mib), indent=1))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path (tokens would shard "
              "data-parallel, with one all-reduce of the adapter gradients per layer); use --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from bit_quantized_finetuning_nf4_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = synth.LAYER_SETS[args.workload]
    M, r, alpha = cfg["M"], cfg["r"], cfg["alpha"]
    set_index = {"llama7b": 1, "llama13b": 2, "llama65b": 3}[args.workload]
    log(f"[bench] workload {args.workload}: {len(cfg['linears'])} linears, M={M}, r={r}")
    S = LayerSet(args.workload, dev)
    L = S.L
    head = S.run("grouped", args.steps, args.warmup)
    ms_step = head["ms_per_step"]
    log(f"[bench] grouped step {ms_step:.3f} ms; phases {head['phases_ms']}; products {head['products']}")

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * 1024 * 1024 // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    clock = per_linear = fused = None
    if not args.headline_only:
        # the shader clock while the same steps run (a separate window, so the
        # sampling subprocess stays out of the timed region above)
        sampler = ClockSampler()
        with sampler:
            t_end = time.perf_counter() + 2.0
            while time.perf_counter() < t_end:
                for _ in range(10):
                    S.step("grouped")
                torch.cuda.synchronize()
        clock = sampler.result()
        log(f"[bench] clock {clock}")
        per_linear = S.run("staged", args.steps, args.warmup)
        log(f"[bench] per-linear staged step {per_linear['ms_per_step']:.3f} ms; "
            f"fwd+bwd {per_linear['fwd_bwd_tflops']:.0f} TFLOP/s")
        fused = S.run("fused", args.steps, args.warmup)
        log(f"[bench] fused step {fused['ms_per_step']:.3f} ms; fwd+bwd {fused['fwd_bwd_tflops']:.0f} TFLOP/s")

    prod = head["products"]
    traffic = traffic_for("dense_gemm")
    roof = {"kernel": "dense_gemm (bf16_fwd_kernel, forward and dX products)", "bound": "mfma",
            "achieved": prod["tflops"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": prod["tflops"] / PEAK_BF16_TFLOPS, "traffic": traffic,
            "per_launch": "flops of the dense GEMM = 2MNK + 2Mr(N) (forward) or 2MNK + 2Mr(K) (dX) summed over the "
                          "linears of each product (q/k/v, o, gate/up, down); achieved = the sum over the 7 "
                          "linears / the sum of the 8 product calls' HIP-event durations (a call is one launch, or "
                          "two when its last round of tiles takes a narrower tile width)"}
    mc = mfma_counters_for("bf16_fwd_kernel", "dense_gemm")
    if mc:
        roof["counters"] = {"source": "profiles/mfma.json (rocprofv3 --pmc on the same device code)",
                            "mfma_busy": mc["mfma_busy"], "valu_per_mfma": mc["valu_per_mfma"],
                            "clock_ghz": mc["clock_ghz"]}
    if clock:
        roof["clock_mhz_median"] = clock["median_mhz"]
        roof["frac_at_measured_clock"] = prod["tflops"] / (PEAK_BF16_TFLOPS * clock["median_mhz"] / 2400.0)
    value = S.fl_step / (ms_step * 1e-3) / 1e12
    fb = head["fwd_bwd_tflops"]
    out = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{args.workload} layer set: " + ", ".join(f"{o['name']} {o['N']}x{o['K']}" for o in L)
                   + f"; M={M} tokens; LoRA r={r} alpha={alpha}; NF4 blocksize 64, 8-bit double quant per 256 blocks"
                   + "; step = quantize + fwd + bwd (q/k/v and gate/up as one group each; staged: W "
                     "dequantized once per product, dense bf16 GEMM) + batch-1 decode GEMV",
                   "global_batch": M, "seq_len": M, "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "phases_ms": head["phases_ms"],
        "products": prod,
        "fwd_bwd_tflops": fb,
        "targets": {"fwd_bwd_frac_of_bf16_peak": fb / PEAK_BF16_TFLOPS, "fwd_bwd_target_frac": 0.50,
                    "fwd_bwd_shortfall_ms": max(0.0, (head["phases_ms"]["forward"] + head["phases_ms"]["backward"])
                                                - S.fl_step / (0.5 * PEAK_BF16_TFLOPS * 1e12) * 1e3)},
        "per_linear_path": per_linear and {k: per_linear[k] for k in ("ms_per_step", "phases_ms", "fwd_bwd_tflops",
                                                                     "products")},
        "fused_path": fused and {k: fused[k] for k in ("ms_per_step", "phases_ms", "fwd_bwd_tflops", "products")},
        "clock": clock,
        "quantize_gbps": S.q_bytes / (head["phases_ms"]["quantize"] * 1e-3) / 1e9,
        "layer_gemv_gbps": S.g_bytes / (head["phases_ms"]["decode_gemv"] * 1e-3) / 1e9,
    }
    if not args.no_codebook_study and not args.headline_only:
        out["codebooks"] = codebook_study(L, dev, S.q_bytes)
        log(f"[bench] codebooks {out['codebooks']}")
        out["optimizer"] = optimizer_study(L, r, dev)
        log(f"[bench] optimizer {out['optimizer']}")
    del S, L
    torch.cuda.empty_cache()

    if not args.no_other_sets and not args.headline_only:
        out["dequant"] = dequant_study(dev)
        log(f"[bench] dequant {out['dequant']}")
        sets = {}
        for name in ("llama7b", "llama13b", "small"):
            if name == args.workload:
                continue
            T = LayerSet(name, dev, with_decode=False)
            paths = ("grouped", "staged", "fused") if T.M >= 1024 else ("grouped", "fused")
            res = {"M": T.M, "r": T.r, "linears": [f"{o['name']} {o['N']}x{o['K']}" for o in T.L],
                   "flops_per_step": T.fl_step}
            for pth in paths:
                rr = T.run(pth, args.steps, args.warmup)
                res[pth] = {"fwd_bwd_tflops": rr["fwd_bwd_tflops"],
                            "fwd_bwd_frac_of_bf16_peak": rr["fwd_bwd_tflops"] / PEAK_BF16_TFLOPS,
                            "phases_ms": rr["phases_ms"], "products_tflops": rr["products"]["tflops"],
                            "products_frac": rr["products"]["frac_of_bf16_peak"]}
            res["path_taken_by_qlora_linear"] = "staged" if T.M >= 1024 else "fused"
            sets[name] = res
            log(f"[bench] {name}: " + ", ".join(f"{pth} {res[pth]['fwd_bwd_tflops']:.0f} TF/s" for pth in paths))
            del T
            torch.cuda.empty_cache()
        out["layer_sets"] = sets

    # ---- 80-layer batch-1 decode pass (about 65e9 weights) ----
    if args.decode_layers > 0:
        from bit_quantized_finetuning_nf4_amd import ops
        E = TimingEvent
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
        for _ in range(DECODE_WARMUP):
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
                         "frac_of_hbm_peak": gbps / PEAK_HBM_GBPS, "target_frac": 0.70,
                         "target_shortfall_ms": max(0.0, pass_ms - nbytes / (0.7 * PEAK_HBM_GBPS * 1e9) * 1e3)}
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
