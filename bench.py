"""Benchmark of the FP8 block-scaled linear-layer flow on one MI355X.

One step = the whole hot path for every linear of the workload:
    quantize_weight_128x128(W)            (with the transposed copy for DGrad)
    quantize_dual_1x128_128x1(X)  -> fp8_gemm_fwd      Y  = Xq Wq^T   (+ Xq_t saved for WGrad)
    quantize_dual_1x128_128x1(dY) -> fp8_gemm_dgrad    dX = dYq Wq
    fp8_gemm_wgrad_grouped over all linears              dW = dYq^T Xq
on synthetic inputs already resident in HBM. The dual quantizer emits the
1x128 and the transposed 128x1 groupings from one read; --separate-quant runs
quantize_act_1x128 and transpose_quantize_128x1 as separate launches instead.
The WGrads of all linears go out as one grouped launch (their tiles fill the
compute units that the small qkv / o outputs alone leave idle); --no-grouped
launches them one per linear. Default workload: the four
linears of a Qwen2.5-32B-shaped layer (qkv 5120->7168, o 5120->5120,
up 5120->27648, down 27648->5120) at 32768 tokens.

Prints ONE JSON line. `value` is GEMM TFLOP/s over the whole step (every
quantizer and GEMM launch inside the timed region of K steps). The per-launch
table comes from HIP events around every launch in a pass of the same K steps
run just before the timed region; inside the timed region only the launch that
takes the most time is bracketed by HIP events (on the stream the kernels run
on), and `roofline` reports that launch with its average duration there (and
the median and minimum over the K steps; every launch in `kernels` carries the
same three from the instrumented pass).
`cpu_baseline` times the CPU oracle on a bounded sample of the same
workload.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload NAME]
                    [--no-cpu-baseline] [--traffic-from profiles/<file>.json]
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "FP8 block-scaled GEMM TFLOP/s (fwd/DGrad/WGrad), % of FP8 MFMA peak"
PEAK_FP8_TFLOPS = 5000.0        # MI355X dense FP8 MFMA, published
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E, published
DEFAULT_WORKLOAD = "qwen25_32b_linears_m32768"
RIDGE = PEAK_FP8_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)   # 625 FLOP per byte: MFMA- vs HBM-bound
ROTATE_BYTES = 640 << 20        # > 256 MB last-level cache + 8 x 4 MB L2, with margin


def attainable_tflops(flop_per_byte):
    """Roofline: min(FP8 MFMA peak, arithmetic intensity x HBM peak), TFLOP/s."""
    return min(PEAK_FP8_TFLOPS, flop_per_byte * PEAK_HBM_GBS / 1e3)
MAX_SETS = 32


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-producers", action="store_true",
                    help="skip timing the fused RMSNorm / SwiGLU producers (reported outside the step)")
    ap.add_argument("--no-grouped", action="store_true",
                    help="one WGrad launch per linear instead of one grouped launch for all of them")
    ap.add_argument("--separate-quant", action="store_true",
                    help="quantize X and dY with the single-output kernels (two reads each)")
    ap.add_argument("--weights-prequantized", action="store_true",
                    help="quantize the weights once per input set outside the timed step "
                         "(rollout: weights change once per optimizer update)")
    ap.add_argument("--no-stream", action="store_true",
                    help="run decode-sized forward-only linears on the row-major tile forward instead of the "
                         "weight-streaming layout and its forward")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured in a HIP graph (one graph per input set) and "
                         "replayed: graph_ms_per_step")
    ap.add_argument("--rotate", type=int, default=0,
                    help="input/weight sets rotated between steps (0: enough that one rotation "
                         "touches more than the 256 MB last-level cache plus L2)")
    ap.add_argument("--traffic-from", default=None,
                    help="JSON with measured HBM bytes per launch of the dominant kernel")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="before timing, run one plain 1 GiB device copy (y = x + 0 on bf16) whose "
                         "FETCH_SIZE / WRITE_SIZE calibrate the HBM counters")
    ap.add_argument("--summarize-trace", metavar="CSV", default=None,
                    help="host only: per (kernel, grid) average durations from a rocprofv3 kernel trace")
    ap.add_argument("--summarize-runs", metavar="JSON", nargs="+", default=None,
                    help="print a markdown table of the launches of bench.py result lines (files)")
    ap.add_argument("--summarize-counters", metavar="CSV", nargs="+", default=None,
                    help="host only: per (kernel, grid) averages of rocprofv3 --pmc counter CSVs")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the measured-ceilings micro-benchmark (bench_ceilings) run before the step")
    return ap.parse_args()


CEILINGS_EXE = os.path.join(ROOT, "bench_ceilings")


def measured_ceilings():
    """Run the ceilings micro-benchmark (a separate process, before this one
    touches the GPU) and return its streams and MFMA loops by name."""
    import subprocess
    if not os.path.exists(CEILINGS_EXE):
        return None
    r = subprocess.run([CEILINGS_EXE], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=120)
    if r.returncode != 0:
        print(f"[bench] bench_ceilings failed: {r.stdout[-500:]}", file=sys.stderr, flush=True)
        return None
    out = {"streams": {}, "mfma_loops": {}}
    for line in r.stdout.splitlines():
        d = json.loads(line)
        if "stream" in d:
            out["streams"][d.pop("stream")] = d
        elif "loop" in d:
            out["mfma_loops"][d.pop("loop")] = d
        elif "device" in d:
            out["device"] = d["device"]
    return out


# The measured stream whose read/write mix matches each quantizer kind:
# 2 B read + 1 B written per element (1x128, 128x1, 128x128 without the
# transposed copy) or 2 B read + 2 B written (dual, 128x128 with it).
STREAM_FOR = {"quant_act": "read2_write1", "quant_transpose": "read2_write1", "quant_dual": "copy_nt",
              "quant_weight": "copy_nt", "quant_weight_nt": "read2_write1",
              "quant_weight_stream": "read2_write1"}

# Forward-only linears with at most this many tokens (decode) run on the
# weight-streaming layout: the weight quantizer writes it, the stream forward
# reads it (the same bytes as the row-major codes, rearranged).
STREAM_MAX_TOKENS = 64


def act_bytes(rows, cols):
    return rows * cols * 3 + rows * (cols // 128) * 4


def dual_bytes(rows, cols):
    return rows * cols * 4 + rows * (cols // 128) * 4 + cols * (rows // 128) * 4


def launch_stats(samples):
    """Mean, median and minimum of one launch's per-step durations (ms)."""
    v = sorted(samples)
    n = len(v)
    med = v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])
    return {"ms": sum(v) / n, "ms_median": med, "ms_min": v[0]}


def host_cpu_model():
    """The host CPU's model name (Linux /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def weight_bytes(n, k, transposed):
    return n * k * (4 if transposed else 3) + (n // 128) * (k // 128) * 4


class Linear:
    """Device buffers and the launch list of one linear layer."""

    def __init__(self, lin, passes, seed, fq, inputs, torch, dual=True, stream=True):
        self.name, self.M, self.N, self.K = lin["name"], lin["M"], lin["N"], lin["K"]
        self.stream = stream and tuple(passes) == ("fwd",) and lin["M"] <= STREAM_MAX_TOKENS
        M, N, K = self.M, self.N, self.K
        dev = "cuda"
        t = inputs.linear_tensors_device(lin, seed=seed)
        self.x, self.w, self.dy = t["x"], t["w"], t["dy"]
        e = lambda shape, dt: torch.empty(shape, dtype=dt, device=dev)
        u8, f32, bf = torch.uint8, torch.float32, torch.bfloat16
        self.passes = passes
        dgrad, wgrad = "dgrad" in passes, "wgrad" in passes
        self.dual = dual
        self.wq, self.ws = e((N, K), u8), e((N // 128, K // 128), f32)
        self.wq_t = e((K, N), u8) if dgrad else None
        if "fwd" in passes:
            self.xq, self.xs = e((M, K), u8), e((M, K // 128), f32)
            self.y = e((M, N), bf)
        if dgrad:
            self.dyq, self.dys = e((M, N), u8), e((M, N // 128), f32)
        if dgrad:
            self.dx = e((M, K), bf)
        if wgrad:
            self.xq_t, self.xs_t = e((K, M), u8), e((K, M // 128), f32)
            self.dyq_t, self.dys_t = e((N, M), u8), e((N, M // 128), f32)
            self.dw = e((N, K), bf)
        self.fq = fq
        self.defer_wgrad = False

    def launches(self):
        """(kind, key, flops, bytes, callable) for every launch of one step, in order.

        X feeds the forward (1x128) and WGrad (128x1); dY feeds DGrad (1x128)
        and WGrad (128x1). Where a tensor needs both groupings the dual
        quantizer makes them in one launch (unless --separate-quant).
        """
        fq, M, N, K = self.fq, self.M, self.N, self.K
        fwd, dgrad, wgrad = ("fwd" in self.passes), ("dgrad" in self.passes), ("wgrad" in self.passes)
        x_dual, dy_dual = self.dual and fwd and wgrad, self.dual and dgrad and wgrad
        L = []
        if self.stream:
            # wq holds the codes in the weight-streaming layout
            L.append(("quant_weight_stream", f"{self.name}.w_stream[{N},{K}]", 0, weight_bytes(N, K, False),
                      lambda: fq.quantize_weight_128x128_stream(self.w, self.wq, self.ws)))
        else:
            L.append(("quant_weight" if self.wq_t is not None else "quant_weight_nt", f"{self.name}.w[{N},{K}]", 0,
                      weight_bytes(N, K, self.wq_t is not None),
                      lambda: fq.quantize_weight_128x128(self.w, self.wq_t is not None, self.wq, self.ws, self.wq_t)))
        if x_dual:
            L.append(("quant_dual", f"{self.name}.x_dual[{M},{K}]", 0, dual_bytes(M, K),
                      lambda: fq.quantize_dual_1x128_128x1(self.x, self.xq, self.xs, self.xq_t, self.xs_t)))
        elif fwd:
            L.append(("quant_act", f"{self.name}.x[{M},{K}]", 0, act_bytes(M, K),
                      lambda: fq.quantize_act_1x128(self.x, self.xq, self.xs)))
        if fwd and self.stream:
            L.append(("gemm_fwd", f"{self.name}.fwd_stream[{M}x{N}x{K}]", 2 * M * N * K, M * K + N * K + 2 * M * N,
                      lambda: fq.fp8_gemm_fwd_stream(self.xq, self.xs, self.wq, self.ws, out=self.y)))
        elif fwd:
            L.append(("gemm_fwd", f"{self.name}.fwd[{M}x{N}x{K}]", 2 * M * N * K, M * K + N * K + 2 * M * N,
                      lambda: fq.fp8_gemm_fwd(self.xq, self.xs, self.wq, self.ws, out=self.y)))
        if dy_dual:
            L.append(("quant_dual", f"{self.name}.dy_dual[{M},{N}]", 0, dual_bytes(M, N),
                      lambda: fq.quantize_dual_1x128_128x1(self.dy, self.dyq, self.dys, self.dyq_t, self.dys_t)))
        elif dgrad:
            L.append(("quant_act", f"{self.name}.dy[{M},{N}]", 0, act_bytes(M, N),
                      lambda: fq.quantize_act_1x128(self.dy, self.dyq, self.dys)))
        if dgrad:
            L.append(("gemm_dgrad", f"{self.name}.dgrad[{M}x{K}x{N}]", 2 * M * N * K, M * N + N * K + 2 * M * K,
                      lambda: fq.fp8_gemm_dgrad(self.dyq, self.dys, self.wq_t, self.ws, out=self.dx)))
        if wgrad:
            if not x_dual:
                L.append(("quant_transpose", f"{self.name}.x_t[{M},{K}]", 0, act_bytes(M, K),
                          lambda: fq.transpose_quantize_128x1(self.x, self.xq_t, self.xs_t)))
            if not dy_dual:
                L.append(("quant_transpose", f"{self.name}.dy_t[{M},{N}]", 0, act_bytes(M, N),
                          lambda: fq.transpose_quantize_128x1(self.dy, self.dyq_t, self.dys_t)))
            if not self.defer_wgrad:
                L.append(("gemm_wgrad", f"{self.name}.wgrad[{N}x{K}x{M}]", 2 * M * N * K, M * N + M * K + 2 * N * K,
                          lambda: fq.fp8_gemm_wgrad(self.dyq_t, self.dys_t, self.xq_t, self.xs_t, out=self.dw)))
        return L

    def wgrad_problem(self):
        """(operands, output, flops, bytes) of this linear's WGrad for a grouped launch."""
        M, N, K = self.M, self.N, self.K
        return ((self.dyq_t, self.dys_t, self.xq_t, self.xs_t), self.dw, 2 * M * N * K,
                M * N + M * K + 2 * N * K)


def time_producers(fq, inputs, torch, wl, reps=10):
    """The fused producers at the workload's shapes, timed outside the step.

    RMSNorm of the hidden input [M, K] and SwiGLU of the intermediate [M, N]
    (the up linear's width), each with both groupings quantized and no bf16
    copy written. Algorithmic bytes: 2 B read per input element + 2 B of codes
    + 8 B of scales per 128 elements (+ 4 B of rstd per row); the RMSNorm
    implementation reads x twice (row statistics, then the quantizing pass).
    """
    lins = {l["name"]: l for l in wl["linears"]}
    if "fwd" not in wl["passes"] or not ({"qkv", "up"} <= set(lins)):
        return None
    M, K, N = lins["qkv"]["M"], lins["qkv"]["K"], lins["up"]["N"]
    x = inputs.bf16_normal_device((M, K), 1.0, 0.01, seed=41)
    g = inputs.bf16_normal_device((K,), 0.5, 0.0, seed=42)
    gate = inputs.bf16_normal_device((M, N), 2.0, 0.0, seed=43)
    up = inputs.bf16_normal_device((M, N), 1.0, 0.0, seed=44)
    out_r = fq.rmsnorm_quantize_1x128(x, g, 1e-6, True)
    out_s = fq.swiglu_quantize_1x128(gate, up, True)
    cases = [
        (f"rmsnorm_quantize[{M},{K}]", M * K * 4 + M * K // 16 + M * 4,
         lambda: fq.rmsnorm_quantize_1x128(x, g, 1e-6, True, False, *out_r[:5])),
        (f"swiglu_quantize[{M},{N}]", M * N * 6 + M * N // 16,
         lambda: fq.swiglu_quantize_1x128(gate, up, True, False, *out_s[:4])),
    ]
    res = {}
    stream = torch.cuda.current_stream()
    for key, nbytes, fn in cases:
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        gbs = nbytes / (ms * 1e-3) / 1e9
        res[key] = {"ms": round(ms, 4), "gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
    del x, g, gate, up, out_r, out_s
    torch.cuda.empty_cache()
    return res


def cpu_baseline(inputs, wl, tokens=16384):
    """Time the CPU oracle on a bounded sample: every pass of the o-proj linear at `tokens` tokens."""
    import numpy as np
    from oracle import gemm, quant

    lin = dict(next(l for l in wl["linears"] if l["name"] == "o") if any(l["name"] == "o" for l in wl["linears"])
               else wl["linears"][0])
    lin["M"] = tokens
    t = inputs.linear_tensors(lin, seed=0)
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    M, N, K = lin["M"], lin["N"], lin["K"]
    t0 = time.perf_counter()
    xq, xs = quant.quantize_act_1x128(t["x"])
    wq, ws, _ = quant.quantize_weight_128x128(t["w"])
    dyq, dys = quant.quantize_act_1x128(t["dy"])
    xq_t, xs_t = quant.transpose_quantize_128x1(t["x"])
    dyq_t, dys_t = quant.transpose_quantize_128x1(t["dy"])
    gemm.gemm_fwd(xq, xs, wq, ws)
    gemm.gemm_dgrad(dyq, dys, wq, ws)
    gemm.gemm_wgrad(dyq_t, dys_t, xq_t, xs_t)
    dt = time.perf_counter() - t0
    flops = 3 * 2 * M * N * K
    import hashlib
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{lin['name']} linear ({K}->{N}) at {M} tokens: all five quantizations and "
                      f"fwd/dgrad/wgrad in fp64, {dt:.1f} s wall; inputs drawn on the host (numpy PCG64, "
                      f"seed 0, the same recipe as the step's), not the step's device-drawn tensors",
            "inputs_sha256": {k: hashlib.sha256(t[k].tobytes()).hexdigest()[:16] for k in ("x", "w", "dy")},
            "seconds": dt, "blas_threads": int(threads), "host_cpus": len(os.sched_getaffinity(0)),
            "cpu_model": host_cpu_model()}


def measured_traffic(path, key):
    """HBM bytes per launch of `key` from a counter summary, or None.

    The summary holds FETCH_SIZE and WRITE_SIZE per launch, each scaled by the
    ratio of the known bytes of a plain copy kernel to what the same counter
    read for it. It is ignored once a kernel source it names has changed since
    the counters were taken (a stored source hash no longer matches).
    """
    import hashlib
    if not os.path.exists(path):
        return None
    tr = json.load(open(path))
    hashes = tr.get("source_sha256_16", {})
    if not hashes:
        return None
    for name, want in hashes.items():
        src = os.path.join(ROOT, "fp8_block_scaled_quantize_amd", "csrc", name)
        if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest()[:16] != want:
            return None
    return tr.get("bytes_per_launch", {}).get(key)


def _short(name):
    name = name.split("(")[0].replace("void ", "")
    return name[-80:]


def summarize_trace(path):
    """Average duration per (kernel, grid size) from a rocprofv3 --kernel-trace CSV."""
    import csv
    groups = {}
    for r in csv.DictReader(open(path)):
        if "Grid_Size" in r:
            grid = r["Grid_Size"]
        else:
            grid = str(int(r["Grid_Size_X"]) * int(r.get("Grid_Size_Y") or 1) * int(r.get("Grid_Size_Z") or 1))
        key = (_short(r["Kernel_Name"]), grid)
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6
        groups.setdefault(key, []).append(d)
    rows = sorted(groups.items(), key=lambda kv: -sum(kv[1]))
    print(f"{'kernel':80s} {'grid':>10s} {'calls':>6s} {'avg_ms':>9s} {'total_ms':>9s}")
    for (k, g), v in rows:
        print(f"{k:80s} {g:>10s} {len(v):6d} {sum(v)/len(v):9.4f} {sum(v):9.3f}")


def summarize_counters(paths):
    """Average counter value per (kernel, grid size, counter) from rocprofv3 --pmc CSVs."""
    import csv
    groups = {}
    for path in paths:
        for r in csv.DictReader(open(path)):
            key = (_short(r["Kernel_Name"]), r["Grid_Size"], r["Counter_Name"])
            groups.setdefault(key, {}).setdefault(r["Dispatch_Id"], 0.0)
            groups[key][r["Dispatch_Id"]] += float(r["Counter_Value"])
    print(f"{'kernel':80s} {'grid':>10s} {'counter':>12s} {'dispatches':>10s} {'avg':>14s}")
    for (k, g, c), d in sorted(groups.items()):
        vals = list(d.values())
        print(f"{k:80s} {g:>10s} {c:>12s} {len(vals):10d} {sum(vals)/len(vals):14.1f}")


def summarize_runs(paths):
    """Markdown table of the per-launch timings of bench.py result lines."""
    for path in paths:
        r = json.loads(open(path).read().strip().splitlines()[-1])
        c = r["config"]
        print(f"### {c['workload']}  ({', '.join(c['passes'])}; {r['input_sets']} input set(s); "
              f"weights {r.get('weights', 'quantized inside the step')})\n")
        print(f"step {r['ms_per_step']} ms, {r['value']} TFLOP/s over the step, GEMMs alone "
              f"{r['gemm_only_tflops']} TFLOP/s\n")
        print("| launch | ms | rate | of peak |\n|---|---|---|---|")
        for key, k in r["kernels"].items():
            if "tflops" in k:
                gbs = f", {k['gbs']} GB/s ({100 * k['gbs'] / PEAK_HBM_GBS:.1f} % HBM)" if "gbs" in k else ""
                if k.get("bound") == "hbm":
                    roof = f"{100 * k['gbs'] / PEAK_HBM_GBS:.1f} % HBM (HBM-bound, {k['flop_per_byte']} FLOP/B)"
                else:
                    roof = f"{100 * k['frac_fp8_peak']:.1f} % FP8"
                print(f"| {key} | {k['ms']} | {k['tflops']} TFLOP/s{gbs} | {roof} |")
            else:
                print(f"| {key} | {k['ms']} | {k['gbs']} GB/s | {100 * k['frac_hbm_peak']:.1f} % HBM |")
        print()


def main():
    args = parse()
    if args.summarize_runs:
        summarize_runs(args.summarize_runs)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); a multi-GPU layout "
              "is not measured here.", file=sys.stderr)
        sys.exit(2)

    ceilings = None if args.no_ceilings else measured_ceilings()

    import torch
    import fp8_block_scaled_quantize_amd as fq
    from fp8_block_scaled_quantize_amd import inputs

    if not os.path.exists(fq.library_path()):
        from fp8_block_scaled_quantize_amd.build import build
        build()
    fq.load_library()
    wl = inputs.WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    print(f"[bench] workload {args.workload}: generating inputs", file=sys.stderr, flush=True)
    grouped = not args.no_grouped and "wgrad" in wl["passes"] and len(wl["linears"]) > 1

    def build_step(seed):
        layers = [Linear(lin, wl["passes"], seed + 17 * i, fq, inputs, torch, dual=not args.separate_quant,
                         stream=not args.no_stream)
                  for i, lin in enumerate(wl["linears"])]
        for layer in layers:
            layer.defer_wgrad = grouped
        steps = [l for layer in layers for l in layer.launches()]
        if args.weights_prequantized:
            for l in [l for l in steps if l[0].startswith("quant_weight")]:
                l[4]()
            steps = [l for l in steps if not l[0].startswith("quant_weight")]
        if grouped:
            # the WGrads of all linears in one launch (they are independent of the
            # rest of the step; a backward pass can defer them to the end)
            probs = [layer.wgrad_problem() for layer in layers]
            outs = [p[1] for p in probs]
            ops = [p[0] for p in probs]
            names = "+".join(layer.name for layer in layers)
            steps.append(("gemm_wgrad", f"wgrad_grouped[{names}]", sum(p[2] for p in probs),
                          sum(p[3] for p in probs), lambda: fq.fp8_gemm_wgrad_grouped(ops, outs)))
        return steps

    # Small workloads rotate through independent input sets, so that no step
    # finds its operands in the 256 MB last-level cache from the step before.
    sets = [build_step(1000)]
    step_bytes = sum(l[3] for l in sets[0])
    nsets = args.rotate if args.rotate > 0 else min(MAX_SETS, -(-ROTATE_BYTES // step_bytes))
    for r in range(1, nsets):
        sets.append(build_step(1000 + 7919 * r))
    launches = sets[0]
    torch.cuda.synchronize()
    if args.calibrate_copy:
        cx = torch.ones((1 << 29,), dtype=torch.bfloat16, device="cuda")    # 1 GiB
        cy = torch.empty_like(cx)
        torch.add(cx, 0, out=cy)
        torch.cuda.synchronize()
        del cx, cy

    for s in range(max(args.warmup, nsets)):
        for _, _, _, _, fn in sets[s % nsets]:
            fn()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps); timing {args.steps} steps", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()

    def event_pair():
        return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    # Per-launch breakdown: the same K steps with HIP events around every
    # launch, before the timed region (an event record between every pair of
    # launches would add its own gaps to the step).
    ev = [[event_pair() for _ in launches] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        for i, (_, _, _, _, fn) in enumerate(sets[s % nsets]):
            ev[s][i][0].record(stream)
            fn()
            ev[s][i][1].record(stream)
    torch.cuda.synchronize()
    per_stats = [launch_stats([ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(args.steps)])
                 for i in range(len(launches))]
    per_ms = [st["ms"] for st in per_stats]
    dom_i = max(range(len(launches)), key=lambda i: per_ms[i])

    # The timed region: exactly K steps; HIP events bracket only the dominant
    # launch (its average duration is the roofline's avg_ms).
    dev = [event_pair() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        for i, (_, _, _, _, fn) in enumerate(sets[s % nsets]):
            if i == dom_i:
                dev[s][0].record(stream)
            fn()
            if i == dom_i:
                dev[s][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    dom_stats = launch_stats([a.elapsed_time(b) for a, b in dev])
    dom_ms = dom_stats["ms"]

    graph_ms = None
    if args.graph:
        # The same launches captured once per input set and replayed: what a
        # launch-bound step (decode) costs without per-launch host overhead.
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for st in sets:
                for _, _, _, _, fn in st:
                    fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graphs = []
        for st in sets:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _, _, _, _, fn in st:
                    fn()
            graphs.append(g)
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(args.steps):
            graphs[s % nsets].replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) * 1e3 / args.steps

    # Per-launch average durations (ms) from the instrumented pass.
    per = []
    for i, (kind, key, flops, nbytes, _) in enumerate(launches):
        per.append({"kind": kind, "key": key, "flops": flops, "bytes": nbytes, **per_stats[i]})
    gemm_flops = sum(p["flops"] for p in per)
    gemm_ms = sum(p["ms"] for p in per if p["flops"])
    quant_ms = sum(p["ms"] for p in per if not p["flops"])
    value = gemm_flops / (ms_per_step * 1e-3) / 1e12

    kernels = {}
    for p in per:
        if p["flops"]:
            tf = p["flops"] / (p["ms"] * 1e-3) / 1e12
            ai = p["flops"] / p["bytes"]
            kernels[p["key"]] = {"ms": round(p["ms"], 4), "ms_median": round(p["ms_median"], 4),
                                 "ms_min": round(p["ms_min"], 4), "tflops": round(tf, 1),
                                 "frac_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4),
                                 "gbs": round(p["bytes"] / (p["ms"] * 1e-3) / 1e9, 1),
                                 "flop_per_byte": round(ai, 1),
                                 "bound": "mfma" if ai >= RIDGE else "hbm",
                                 "frac_attainable": round(tf / attainable_tflops(ai), 4)}
            # the decode forward against a read of the same weight bytes in its own order
            if ceilings and "fwd_stream" in p["key"] and "stream_ring8" in ceilings["streams"]:
                gbs = p["bytes"] / (p["ms"] * 1e-3) / 1e9
                kernels[p["key"]]["frac_stream_ceiling"] = round(gbs / ceilings["streams"]["stream_ring8"]["gbs"], 4)
                kernels[p["key"]]["stream_ceiling"] = "stream_ring8"
        else:
            gbs = p["bytes"] / (p["ms"] * 1e-3) / 1e9
            kernels[p["key"]] = {"ms": round(p["ms"], 4), "ms_median": round(p["ms_median"], 4),
                                 "ms_min": round(p["ms_min"], 4), "gbs": round(gbs, 1),
                                 "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
            kind = p["kind"]
            if ceilings and STREAM_FOR.get(kind) in ceilings["streams"]:
                name = STREAM_FOR[kind]
                kernels[p["key"]]["frac_stream_ceiling"] = round(gbs / ceilings["streams"][name]["gbs"], 4)
                kernels[p["key"]]["stream_ceiling"] = name

    dom = dict(per[dom_i], ms=dom_ms)       # the dominant launch, timed inside the timed region
    if dom["flops"] and dom["flops"] / dom["bytes"] >= RIDGE:
        achieved = dom["flops"] / (dom["ms"] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_FP8_TFLOPS, 4)}
    elif dom["flops"]:
        # A GEMM below the ridge point (decode, a few hundred tokens) is bound by
        # HBM: its algorithmic bytes over the time, against the HBM peak.
        achieved = dom["bytes"] / (dom["ms"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4),
                "flop_per_byte": round(dom["flops"] / dom["bytes"], 1),
                "tflops": round(dom["flops"] / (dom["ms"] * 1e-3) / 1e12, 1)}
    else:
        achieved = dom["bytes"] / (dom["ms"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4)}
    roof["kernel"] = dom["key"]
    roof["avg_ms"] = round(dom["ms"], 4)
    roof["median_ms"] = round(dom_stats["ms_median"], 4)
    roof["min_ms"] = round(dom_stats["ms_min"], 4)
    roof["traffic"] = measured_traffic(args.traffic_from or os.path.join(
        ROOT, "profiles", f"traffic_{args.workload}.json"), dom["key"])

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate, bf16 out)",
        "data": "synthetic",
        "config": {"workload": args.workload,
                   "tokens": wl["linears"][0]["M"],
                   "linears": {l["name"]: [l["N"], l["K"]] for l in wl["linears"]},
                   "passes": list(wl["passes"])},
        "pct_of_fp8_peak": round(100 * value / PEAK_FP8_TFLOPS, 2),
        "gemm_only_tflops": round(gemm_flops / (gemm_ms * 1e-3) / 1e12, 1),
        "gemm_ms_per_step": round(gemm_ms, 3),
        "quant_ms_per_step": round(quant_ms, 3),
        "quantizers": "separate" if args.separate_quant else "dual",
        "wgrad_launch": "grouped" if grouped else "per linear",
        "fwd_path": "weight-streaming layout" if any(l[1].split("[")[0].endswith("fwd_stream") for l in launches)
                    else "row-major tiles",
        "input_sets": nsets,
        "graph_ms_per_step": None if graph_ms is None else round(graph_ms, 4),
        "weights": "quantized once per input set, outside the step" if args.weights_prequantized
                   else "quantized inside the step",
        "roofline": roof,
        "kernels": kernels,
    }
    if ceilings:
        result["ceilings"] = ceilings
    if not args.no_producers:
        prod = time_producers(fq, inputs, torch, wl)
        if prod:
            result["producers"] = prod
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(inputs, wl)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
