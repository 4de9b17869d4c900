#!/usr/bin/env python3
"""Benchmark of the NVFP4 hot path on one MI355X.

One step runs every operation of the path once, at the Qwen-Image attention-projection shapes
(weight 3072 x 3072, 4096 tokens x 3072 channels):
  quantize     W fp32 -> NVFP4 (run-time amax)                     [headline: GB/s]
  requantize   W as FP8 E4M3 + per-tensor scale -> NVFP4
  dequantize   NVFP4 W -> bf16
  act_quantize A bf16 -> NVFP4 (dynamic, per-tensor run-time amax)
  gemm_w4a16   C = A . W_hat^T, bf16 activations                    [headline: TFLOP/s]
  gemm_w4a4    C = A_hat . W_hat^T, NVFP4 activations
  gemv_w4a16   the first 2 rows of A against W (memory-bound form)
  percentile   per-channel p99.9 and max of |A|
The FP8 side path is timed after the step, in a loop of its own over the same inputs ("next_ops"):
  act_quantize_fp8  A bf16 -> FP8 E4M3 tensorwise (dynamic amax)
  gemm_w4a8    C = A_fp8 . W_hat^T, FP8 activations
  weight_stats quality statistics of W and its NVFP4 form (relative error, kurtosis, block max/std)
  gemm_w4a16_lr128  C = A . W_hat^T + (A . V^T) . U^T with a bf16 rank-128 branch (V [128 x K], U [N x 128])
  gemm_w4a4_qa C = A_hat . W_hat^T with A quantized under a static amax (p99.9 calibration) by the same call
               (at N = 3072 the library picks a quantize pass + the W4A4 kernel over the fused kernel)
Inputs are resident in HBM before timing; the step rotates over several input sets whose total
size exceeds the 256 MB Infinity Cache, so repeated steps do not hit in cache.  Each operation is
bracketed by events on the stream it runs on; the dominant kernel's roofline uses those times.  Each
timed step is enqueued behind a short spin kernel, so that the host has issued the step's launches
before the GPU reaches them: the events then time the kernels (and the gaps between back-to-back
launches), not the Python binding's per-call overhead.

The JSON line also carries:
  "graph"        the step and the quantize alone captured in HIP graphs and replayed (no eager
                 dispatch gaps between kernels), for information;
  "configs"      the other workloads, event-timed on the GPU with their own rotating inputs:
                 modulation (18432 x 3072 fp32 quantize; 60 FP8 weights requantized; the M = 2
                 GEMV over the 60 results), the Qwen3-VL MLP chain (dynamic activation quantizes and
                 W4A4 gate / up / down at M = 512), and calibration + layer stack (per-channel p99.9
                 over 217088 x 3072 Student-t(3) activations; 360 FP8 weights of 60 blocks
                 requantized, each block's four 3072 x 3072 weights in one batched call (and, for
                 comparison, every weight in a call of its own); the 360 GEMMs at M = 4096, W4A4
                 under the calibrated static amax and W4A16);
  "achievable_peaks"  a 1 GiB device copy and a bf16 library matmul, measured in the same run;
  "cpu_baseline" the CPU oracle timed on the host's cores (one thread and a worker pool) on bounded
                 samples of the same workloads, before the GPU is initialised.

Prints one JSON line.  Flags: --gpus (1 only), --steps, --warmup, --no-cpu-baseline, --no-peaks,
--sections (a comma list of step, next, graph, configs, peaks, cpu; default all).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NVFP4 quantize GB/s; NVFP4-weight GEMM TFLOP/s at Qwen-Image shapes (1 GPU)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
M_TOK, N_OUT, K_IN = 4096, 3072, 3072
GEMV_M = 2
LR_RANK = 128  # rank of the bf16 low-rank branch ("FP4 with BF16 rank 128 branches")
ROTATE_MIN_BYTES = 320 << 20
CPU_REPS = 4  # repetitions of each CPU-baseline sample (about 20 s of oracle work on a 16-core host)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true")
    ap.add_argument("--peaks", action="store_true", help="(kept for old command lines; peaks are on by default)")
    ap.add_argument("--sections", default="step,next,graph,configs,peaks,cpu",
                    help="comma list of: step (the headline step), next (the next-row ops), graph, configs, "
                         "peaks, cpu")
    ap.add_argument("--config-reps", type=int, default=10, help="timed repetitions of each config op")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="after the timed steps, copy a buffer of this many MiB three times (a plain copy of "
                         "known size, for scaling HBM byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the NVFP4 path here is a single-GPU kernel library "
              "(row-sharding across GPUs needs only an all-reduce(max) of amax); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    sections = set(args.sections.split(","))
    if args.no_cpu_baseline:
        sections.discard("cpu")
    if args.no_peaks:
        sections.discard("peaks")

    import numpy as np
    import torch

    # the CPU oracle first: its worker pool forks before anything touches the GPU
    cpu = cpu_baseline() if "cpu" in sections else None

    import bit_gemm_nvfp4_amd as nv
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if "step" not in sections:
        out = {"metric": METRIC, "sections": sorted(sections)}
        if "configs" in sections:
            out["configs"] = bench_configs(nv, dev, args.config_reps, args.warmup)
        if "peaks" in sections:
            out["achievable_peaks"] = achievable_peaks(dev)
        if cpu is not None:
            out["cpu_baseline"] = cpu
        calibration_copies(args.calibrate_copy_mib, dev)
        print(json.dumps(out), flush=True)
        return

    # ---- inputs (synthetic, seeded), resident in HBM ----
    w_np = synth.attn_proj_weight(N_OUT, K_IN)
    a_bits = synth.attn_proj_activations(M_TOK, K_IN)
    w8_np, w8_scale = synth.fp8_tensorwise(w_np)
    w0 = torch.from_numpy(w_np).to(dev)
    a0 = torch.from_numpy(a_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    w80 = torch.from_numpy(w8_np).to(dev)
    set_bytes = w0.numel() * 4 + a0.numel() * 2 + w80.numel()
    nsets = max(2, -(-ROTATE_MIN_BYTES // set_bytes))
    sets = [(w0.clone(), a0.clone(), w80.clone()) for _ in range(nsets)]
    del w0, a0, w80
    src_scale = torch.tensor([w8_scale], dtype=torch.float32, device=dev)

    # ---- outputs and workspaces, allocated once ----
    qw = nv.NVFP4Tensor.empty(N_OUT, K_IN, dev)
    qw8 = nv.NVFP4Tensor.empty(N_OUT, K_IN, dev)
    qa = nv.NVFP4Tensor.empty(M_TOK, K_IN, dev)
    wd = torch.empty((N_OUT, K_IN), dtype=torch.bfloat16, device=dev)
    c16 = torch.empty((M_TOK, N_OUT), dtype=torch.float32, device=dev)
    c4 = torch.empty((M_TOK, N_OUT), dtype=torch.float32, device=dev)
    cv = torch.empty((GEMV_M, N_OUT), dtype=torch.float32, device=dev)
    qws, qws2, qws3, qws4 = (nv.quantize_workspace(dev) for _ in range(4))
    qflags = torch.zeros(1, dtype=torch.int32, device=dev)
    a8 = nv.FP8Tensor.empty(M_TOK, K_IN, dev)
    c8 = torch.empty((M_TOK, N_OUT), dtype=torch.float32, device=dev)
    st_out = torch.empty(8, dtype=torch.float64, device=dev)
    st_ws = torch.empty(nv.workspace_size(nv.OP_STATS, 0, 0), dtype=torch.uint8, device=dev)
    gl = torch.Generator(device="cpu").manual_seed(128)
    lr_v = (torch.randn((LR_RANK, K_IN), generator=gl) * 0.05).to(torch.bfloat16).to(dev)
    lr_u = (torch.randn((N_OUT, LR_RANK), generator=gl) * 0.05).to(torch.bfloat16).to(dev)
    lr_ws = torch.empty(nv.workspace_size(nv.OP_LOWRANK, M_TOK, N_OUT, K_IN), dtype=torch.uint8, device=dev)
    clr = torch.empty((M_TOK, N_OUT), dtype=torch.float32, device=dev)
    # static activation amax, calibrated once: max over channels of the per-channel p99.9 of |A|
    qa_amax = nv.amax_percentile(sets[0][1], 99.9, per_channel=True)[0].max().reshape(1).contiguous()
    qa_ws = nv.gemm_qa_workspace(M_TOK, N_OUT, K_IN, dev)
    cqa = torch.empty((M_TOK, N_OUT), dtype=torch.float32, device=dev)

    ops = ["quantize", "requantize", "dequantize", "act_quantize", "gemm_w4a16", "gemm_w4a4", "gemv_w4a16",
           "percentile"]
    next_ops = ["act_quantize_fp8", "gemm_w4a8", "weight_stats", "gemm_w4a16_lr128", "gemm_w4a4_qa"]
    # kernels each op launches (the roofline is reported for the longest single-kernel op); the
    # percentile at p99.9 over 4096 rows takes the one-pass top-M path (selection + merge)
    n_kernels = {"quantize": 1, "requantize": 1, "dequantize": 1, "act_quantize": 1, "gemm_w4a16": 1,
                 "gemm_w4a4": 1, "gemv_w4a16": 1, "percentile": 2, "act_quantize_fp8": 1, "gemm_w4a8": 1,
                 "weight_stats": 2, "gemm_w4a16_lr128": 2, "gemm_w4a4_qa": 2}

    def step(i, events=None):
        w, a, w8 = sets[i % nsets]
        e = events
        if e: e[0].record()
        nv.quantize(w, out=qw, workspace=qws, flags=qflags)
        if e: e[1].record()
        nv.quantize(w8, src_scale=src_scale, out=qw8, workspace=qws2, flags=qflags)
        if e: e[2].record()
        nv.dequantize(qw, out=wd)
        if e: e[3].record()
        nv.quantize(a, out=qa, workspace=qws3, flags=qflags)
        if e: e[4].record()
        nv.gemm(a, qw, out=c16)
        if e: e[5].record()
        nv.gemm(qa, qw, out=c4)
        if e: e[6].record()
        nv.gemm(a[:GEMV_M], qw, out=cv)
        if e: e[7].record()
        nv.amax_percentile(a, 99.9, per_channel=True)
        if e: e[8].record()

    def step_next(i, events=None):
        w, a, w8 = sets[i % nsets]
        e = events
        if e: e[0].record()
        nv.quantize_fp8(a, out=a8, workspace=qws4, flags=qflags)
        if e: e[1].record()
        nv.gemm(a8, qw, out=c8)
        if e: e[2].record()
        nv.matrix_stats(w, qw, out=st_out, workspace=st_ws)
        if e: e[3].record()
        nv.gemm_lowrank(a, qw, lr_v, lr_u, out=clr, workspace=lr_ws)
        if e: e[4].record()
        nv.gemm_qa(a, qw, qa_amax, out=cqa, workspace=qa_ws)
        if e: e[5].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(ops) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step(0)
    host_ms = (time.perf_counter() - t0) * 1e3
    torch.cuda.synchronize()
    for i in range(args.steps):
        # each step is enqueued behind a hold, so its events time the kernels, not the host's launches
        gpu_hold(2.0 * host_ms + 1.0)
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    ms_per_step = float(np.mean([evs[s][0].elapsed_time(evs[s][-1]) for s in range(args.steps)]))
    op_ms = {op: float(np.mean([evs[s][j].elapsed_time(evs[s][j + 1]) for s in range(args.steps)]))
             for j, op in enumerate(ops)}
    # the next-row ops, in their own loop (the step above stays the NVFP4 path alone)
    if "next" in sections:
        for i in range(args.warmup):
            step_next(i)
        torch.cuda.synchronize()
        evn = [[torch.cuda.Event(enable_timing=True) for _ in range(len(next_ops) + 1)] for _ in range(args.steps)]
        for i in range(args.steps):
            step(args.warmup + i)
            gpu_hold(2.0 * host_ms + 1.0)
            step_next(args.warmup + i, evn[i])
        torch.cuda.synchronize()
        op_ms.update({op: float(np.mean([evn[s][j].elapsed_time(evn[s][j + 1]) for s in range(args.steps)]))
                      for j, op in enumerate(next_ops)})
    else:
        next_ops = []

    def graph_rates():
        """The step, and the quantize alone, captured in HIP graphs (one call per rotating input set)
        and replayed: the same kernels without the eager stream's dispatch gaps.  Informational; the
        headline stays the eager figure."""
        try:
            graphs = []
            for body in (lambda: [step(i) for i in range(nsets)],
                         lambda: [nv.quantize(sets[i][0], out=qw, workspace=qws, flags=qflags) for i in range(nsets)]):
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    body()
                graphs.append(g)
            res = []
            for g in graphs:
                g.replay()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                reps = 10
                e0.record()
                for _ in range(reps):
                    g.replay()
                e1.record()
                torch.cuda.synchronize()
                res.append(e0.elapsed_time(e1) / (reps * nsets))
            return {"ms_per_step": round(res[0], 4),
                    "quantize_ms": round(res[1], 5),
                    "quantize_GBps": round((nW * 4.5625 + 4) / (res[1] * 1e-3) / 1e9, 2),
                    "note": "each replayed graph holds one call per rotating input set; times per call"}
        except Exception as exc:  # capture is informational: report, do not fail the run
            return {"error": f"{type(exc).__name__}: {exc}"[:200]}

    nW, nA = N_OUT * K_IN, M_TOK * K_IN
    graph = graph_rates() if "graph" in sections else None
    nv.check_flags(qflags, "quantizers of the timed steps")

    work = {  # algorithmic bytes (codec / memory-bound ops) or flops (GEMMs)
        "quantize": ("GB/s", nW * 4.5625 + 4, HBM_PEAK_GBS),
        "requantize": ("GB/s", nW * 1.5625 + 4, HBM_PEAK_GBS),
        "dequantize": ("GB/s", nW * 2.5625, HBM_PEAK_GBS),
        "act_quantize": ("GB/s", nA * 2.5625 + 4, HBM_PEAK_GBS),
        "gemm_w4a16": ("TFLOP/s", 2.0 * M_TOK * N_OUT * K_IN, BF16_MFMA_PEAK_TFLOPS),
        "gemm_w4a4": ("TFLOP/s", 2.0 * M_TOK * N_OUT * K_IN, BF16_MFMA_PEAK_TFLOPS),
        "gemv_w4a16": ("GB/s", nW * 0.5625 + GEMV_M * K_IN * 2 + GEMV_M * N_OUT * 4, HBM_PEAK_GBS),
        "percentile": ("GB/s", nA * 2.0, HBM_PEAK_GBS),
        "act_quantize_fp8": ("GB/s", nA * 3.0 + 4, HBM_PEAK_GBS),
        "gemm_w4a8": ("TFLOP/s", 2.0 * M_TOK * N_OUT * K_IN, BF16_MFMA_PEAK_TFLOPS),
        "weight_stats": ("GB/s", nW * 4.5625 + 4, HBM_PEAK_GBS),
        "gemm_w4a16_lr128": ("TFLOP/s", 2.0 * M_TOK * N_OUT * K_IN + 2.0 * M_TOK * LR_RANK * (K_IN + N_OUT),
                             BF16_MFMA_PEAK_TFLOPS),
        "gemm_w4a4_qa": ("TFLOP/s", 2.0 * M_TOK * N_OUT * K_IN, BF16_MFMA_PEAK_TFLOPS),
    }
    op_report, next_report = {}, {}
    for op in ops + next_ops:
        unit, amount, peak = work[op]
        rate = amount / (op_ms[op] * 1e-3) / (1e9 if unit == "GB/s" else 1e12)
        (op_report if op in ops else next_report)[op] = {
            "ms": round(op_ms[op], 5), "rate": round(rate, 2), "unit": unit, "frac_of_peak": round(rate / peak, 4),
            "kernels": n_kernels[op]}

    gemm_ms = op_ms["gemm_w4a16"]
    dom = max((o for o in ops if n_kernels[o] == 1), key=lambda o: op_ms[o])
    d_unit, d_amount, d_peak = work[dom]
    d_rate = d_amount / (op_ms[dom] * 1e-3) / (1e9 if d_unit == "GB/s" else 1e12)
    roofline = {"bound": "mfma" if d_unit == "TFLOP/s" else "hbm", "kernel": dom, "achieved": round(d_rate, 2),
                "peak": d_peak, "unit": d_unit, "frac": round(d_rate / d_peak, 4),
                "traffic": measured_traffic(dom)}

    q_gbs = work["quantize"][1] / (op_ms["quantize"] * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(q_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "Qwen-Image attention projection: W 3072x3072 fp32 N(0,0.02^2); A 4096x3072 bf16 N(0,1) "
                        "with 3 of 3072 channels x20; W also as FP8 E4M3 tensorwise; every NVFP4 hot-path op once "
                        "per step",
            "M": M_TOK, "N": N_OUT, "K": K_IN, "gemv_m": GEMV_M, "rotating_input_sets": nsets,
            "rotating_bytes": nsets * set_bytes,
        },
        "gemm_tflops": round(2.0 * M_TOK * N_OUT * K_IN / (gemm_ms * 1e-3) / 1e12, 2),
        "ops": op_report,
        "next_ops": next_report,
        "roofline": roofline,
        "graph": graph,
    }
    if "configs" in sections:
        sets.clear()
        torch.cuda.empty_cache()
        out["configs"] = bench_configs(nv, dev, args.config_reps, args.warmup)
    if "peaks" in sections:
        peaks = achievable_peaks(dev)
        out["achievable_peaks"] = peaks
        # the step's ops against the measured peaks too
        for rep in (op_report, next_report):
            for op, r in rep.items():
                meas = peaks["hbm_copy_GBps"] if r["unit"] == "GB/s" else peaks["bf16_matmul_TFLOPs"]
                r["frac_of_measured"] = round(r["rate"] / meas, 4)
    if cpu is not None:
        out["cpu_baseline"] = cpu
    calibration_copies(args.calibrate_copy_mib, dev)
    print(json.dumps(out), flush=True)


def calibration_copies(mib, dev):
    """Three device-to-device copies of `mib` MiB (a plain copy of known size, whose HBM byte counters
    scale those of the other kernels in a counter run); nothing when mib is 0."""
    import torch
    if mib > 0:
        src = torch.empty(mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()


def measured_traffic(op):
    """HBM bytes per launch of the op's kernel from the committed counter summary, if that summary was
    taken on the current kernel source (it records the source's SHA-256); otherwise None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic_attention_projection.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    src = fields.get(f"{op}.source")
    if not src or f"{op}.bytes" not in fields:
        return None
    h = hashlib.sha256()
    for p in src.split(","):
        h.update(open(os.path.join(ROOT, p.strip()), "rb").read())
    if h.hexdigest() != fields.get(f"{op}.source_sha256"):
        return None
    return float(fields[f"{op}.bytes"])


def achievable_peaks(dev):
    """Achievable peaks on this GPU from library calls (no code of this repository): HBM read+write
    rate of a 1 GiB device-to-device copy, and the bf16 matmul rate of torch (hipBLASLt) at the
    attention-projection shape.  Event-timed medians over 20 runs after 3 warmups."""
    import numpy as np
    import torch

    def timed(fn, n=20):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(n):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    src.fill_(1)
    dst = torch.empty_like(src)
    copy_ms = timed(lambda: dst.copy_(src))
    del src, dst
    # the GEMM's own layout: A [M x K] times W [N x K] transposed (a 2-D product, no batching)
    a = torch.randn(M_TOK, K_IN, device=dev, dtype=torch.bfloat16)
    w = torch.randn(N_OUT, K_IN, device=dev, dtype=torch.bfloat16)
    mm_ms = timed(lambda: torch.matmul(a, w.T))
    return {"hbm_copy_GBps": round(2 * n / (copy_ms * 1e-3) / 1e9, 1), "hbm_copy_bytes": 2 * n,
            "bf16_matmul_TFLOPs": round(2.0 * M_TOK * N_OUT * K_IN / (mm_ms * 1e-3) / 1e12, 1),
            "bf16_matmul_shape": [M_TOK, N_OUT, K_IN]}


# ------------------------------------------------------------------------------------------------
# the other workloads on the GPU
# ------------------------------------------------------------------------------------------------
def _median_ms(events):
    import numpy as np
    return float(np.median([a.elapsed_time(b) for a, b in events]))


_HOLD = {}


def gpu_hold(ms):
    """Keep the stream busy for about `ms` milliseconds (torch's spin kernel, calibrated once), so
    that the host can enqueue what follows before the GPU reaches it: event times then cover the
    kernels and not the host's launch overhead."""
    import torch
    if "per_ms" not in _HOLD:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000)
        e0.record()
        torch.cuda._sleep(2_000_000)
        e1.record()
        torch.cuda.synchronize()
        _HOLD["per_ms"] = 2_000_000 / max(e0.elapsed_time(e1), 1e-3)
    torch.cuda._sleep(int(ms * _HOLD["per_ms"]))


def _timed(fn, reps, warmup=2):
    """Median event time (ms) of fn(i) on the current stream over reps calls after warmup calls
    (i = the repetition index, for rotating inputs).  Each timed call is enqueued behind a hold
    longer than the host needs to issue it."""
    import torch
    t0 = time.perf_counter()
    for i in range(warmup):
        fn(i)
    host_ms = (time.perf_counter() - t0) * 1e3 / max(warmup, 1)
    torch.cuda.synchronize()
    evs = []
    for i in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        gpu_hold(2.0 * host_ms + 1.0)
        e0.record()
        fn(warmup + i)
        e1.record()
        evs.append((e0, e1))
        torch.cuda.synchronize()
    return _median_ms(evs)


def _graph_ms(fn, reps=5):
    """Median time (ms) of one replay of fn captured in a HIP graph (fn issues only kernels of this
    library on the current stream): the same kernels without the eager stream's per-launch gaps.  None
    if the capture fails (informational)."""
    import torch
    try:
        fn(0)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn(0)
        g.replay()
        torch.cuda.synchronize()
        evs = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            evs.append((e0, e1))
        torch.cuda.synchronize()
        del g
        return _median_ms(evs)
    except Exception:  # capture is informational: report nothing rather than fail the run
        return None


def _rate(amount, ms, unit):
    r = amount / (ms * 1e-3) / (1e9 if unit == "GB/s" else 1e12)
    peak = HBM_PEAK_GBS if unit == "GB/s" else BF16_MFMA_PEAK_TFLOPS
    return {"ms": round(ms, 5), "rate": round(r, 2), "unit": unit, "frac_of_peak": round(r / peak, 4)}


def _fp8_weight(rows, cols, sigma, seed, dev):
    """A per-tensor FP8 E4M3 checkpoint weight made on the GPU: w = sigma N(0, 1) (torch's seeded
    generator), scale = amax / 448, bytes = torch's float8_e4m3fn cast of w / scale."""
    import torch
    g = torch.Generator(device=dev).manual_seed(seed)
    w = torch.randn((rows, cols), generator=g, device=dev, dtype=torch.float32) * sigma
    scale = (w.abs().max() / 448.0).reshape(1)
    b = (w / scale).to(torch.float8_e4m3fn).view(torch.uint8)
    return b, scale


def bench_configs(nv, dev, reps, warmup):
    import torch
    out = {}
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = nv.quantize_workspace(dev)

    # ---- modulation: 18432 x 3072 ------------------------------------------------------------
    R, C = 18432, 3072
    g = torch.Generator(device=dev).manual_seed(3000)
    wmod = [torch.randn((R, C), generator=g, device=dev) * 0.01 for _ in range(2)]  # 453 MB, rotating
    qmod = nv.NVFP4Tensor.empty(R, C, dev)
    q_ms = _timed(lambda i: nv.quantize(wmod[i % 2], out=qmod, workspace=ws, flags=flags), reps, warmup)
    fp8 = [_fp8_weight(R, C, 0.01, 3100 + i, dev) for i in range(60)]  # 3.4 GB of E4M3 sources
    qs = [nv.NVFP4Tensor.empty(R, C, dev) for _ in range(60)]

    def requant_all(_):
        for (b, sc), q in zip(fp8, qs):
            nv.quantize(b, src_scale=sc, out=q, workspace=ws, flags=flags)
    rq_ms = _timed(requant_all, max(3, reps // 3), 1)
    rq_graph_ms = _graph_ms(requant_all)
    a2 = torch.randn((2, C), generator=g, device=dev).to(torch.bfloat16)
    cv = torch.empty((2, R), dtype=torch.float32, device=dev)

    def gemv_all(_):
        for q in qs:
            nv.gemm(a2, q, out=cv)
    gv_ms = _timed(gemv_all, max(3, reps // 3), 1)
    gv_graph_ms = _graph_ms(gemv_all)
    n = R * C
    rq_bytes, gv_bytes = 60 * (n * 1.5625 + 4), 60 * (n * 0.5625 + 2 * C * 2 + 2 * R * 4)
    out["modulation_18432x3072"] = {
        "quantize_fp32": _rate(n * 4.5625 + 4, q_ms, "GB/s"),
        "requantize_fp8_x60": dict(_rate(rq_bytes, rq_ms, "GB/s"), per_weight_ms=round(rq_ms / 60, 5)),
        "gemv_m2_x60": dict(_rate(gv_bytes, gv_ms, "GB/s"), per_call_ms=round(gv_ms / 60, 5)),
    }
    if rq_graph_ms:
        out["modulation_18432x3072"]["requantize_fp8_x60_graph"] = dict(
            _rate(rq_bytes, rq_graph_ms, "GB/s"), note="the 60 calls replayed from a HIP graph")
    if gv_graph_ms:
        out["modulation_18432x3072"]["gemv_m2_x60_graph"] = dict(
            _rate(gv_bytes, gv_graph_ms, "GB/s"), note="the 60 calls replayed from a HIP graph")
    del wmod, fp8, qs, qmod
    torch.cuda.empty_cache()

    # ---- Qwen3-VL MLP at M = 512 -------------------------------------------------------------
    H, I, M = 4096, 12288, 512
    g = torch.Generator(device=dev).manual_seed(4000)
    layers = []
    wg, wu, wd = (torch.randn(s_, generator=g, device=dev) * 0.015 for s_ in ((I, H), (I, H), (H, I)))
    for _ in range(4):  # four copies of the layer (340 MB) so that repeats do not hit in cache
        layers.append(tuple(nv.quantize(w, workspace=ws, flags=flags) for w in (wg, wu, wd)))
    del wg, wu, wd
    a = torch.randn((M, H), generator=g, device=dev).to(torch.bfloat16)
    qa = nv.NVFP4Tensor.empty(M, H, dev)
    cg = torch.empty((M, I), dtype=torch.float32, device=dev)
    cu = torch.empty((M, I), dtype=torch.float32, device=dev)
    qu = nv.NVFP4Tensor.empty(M, I, dev)
    cd = torch.empty((M, H), dtype=torch.float32, device=dev)
    ws2 = nv.quantize_workspace(dev)
    steps = ["quantize_a", "gemm_gate", "gemm_up", "quantize_up", "gemm_down"]

    def chain(i, ev=None):
        lg, lu, ld = layers[i % 4]
        fns = [lambda: nv.quantize(a, out=qa, workspace=ws2, flags=flags),
               lambda: nv.gemm(qa, lg, out=cg), lambda: nv.gemm(qa, lu, out=cu),
               lambda: nv.quantize(cu, out=qu, workspace=ws2, flags=flags), lambda: nv.gemm(qu, ld, out=cd)]
        for k, f in enumerate(fns):
            if ev:
                ev[k].record()
            f()
        if ev:
            ev[len(fns)].record()
    t0 = time.perf_counter()
    for i in range(warmup):
        chain(i)
    host_ms = (time.perf_counter() - t0) * 1e3 / max(warmup, 1)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(steps) + 1)] for _ in range(reps)]
    for i in range(reps):
        gpu_hold(2.0 * host_ms + 1.0)
        chain(warmup + i, evs[i])
        torch.cuda.synchronize()
    import numpy as np
    ms = {st: float(np.median([e[k].elapsed_time(e[k + 1]) for e in evs])) for k, st in enumerate(steps)}
    total = float(np.median([e[0].elapsed_time(e[-1]) for e in evs]))
    fl = 2.0 * M * I * H
    out["qwen3vl_mlp_m512"] = {
        "quantize_a": _rate(M * H * 2.5625 + 4, ms["quantize_a"], "GB/s"),
        "gemm_gate": _rate(fl, ms["gemm_gate"], "TFLOP/s"),
        "gemm_up": _rate(fl, ms["gemm_up"], "TFLOP/s"),
        "quantize_up": _rate(M * I * 4.5625 + 4, ms["quantize_up"], "GB/s"),
        "gemm_down": _rate(fl, ms["gemm_down"], "TFLOP/s"),
        "chain": dict(_rate(3 * fl, total, "TFLOP/s"), note="quantize A, gate, up, quantize up output, down"),
    }
    chain_graph_ms = _graph_ms(lambda _: [chain(j) for j in range(4)])
    if chain_graph_ms:
        out["qwen3vl_mlp_m512"]["chain_graph"] = dict(
            _rate(4 * 3 * fl, chain_graph_ms, "TFLOP/s"), per_chain_ms=round(chain_graph_ms / 4, 5),
            note="the chain over the four layer copies replayed from a HIP graph")
    del layers, a, qa, cg, cu, qu, cd
    torch.cuda.empty_cache()

    # ---- calibration + layer stack -----------------------------------------------------------
    rows, C = 53 * 4096, 3072
    x = torch.empty((rows, C), dtype=torch.bfloat16, device=dev)
    g = torch.Generator(device=dev).manual_seed(5000)
    for r0 in range(0, rows, 8192):  # Student-t(3) = z / sqrt(chi2_3 / 3)
        r1 = min(rows, r0 + 8192)
        z = torch.randn((r1 - r0, C), generator=g, device=dev)
        chi = sum(torch.randn((r1 - r0, C), generator=g, device=dev) ** 2 for _ in range(3))
        x[r0:r1] = (z / torch.sqrt(chi / 3.0)).to(torch.bfloat16)
    pct_ms = _timed(lambda i: nv.amax_percentile(x, 99.9, per_channel=True), max(3, reps // 2), 1)
    pct, _ = nv.amax_percentile(x, 99.9, per_channel=True)
    amax_a = pct.max().reshape(1).contiguous()
    a1 = x[:4096].contiguous()
    del x
    torch.cuda.empty_cache()
    shapes = [(3072, 3072)] * 4 + [(12288, 3072), (3072, 12288)]
    stack = [[_fp8_weight(r, c, 0.02, 5100 + 6 * blk + j, dev) for j, (r, c) in enumerate(shapes)]
             for blk in range(60)]
    qstack = [[nv.NVFP4Tensor.empty(r, c, dev) for (r, c) in shapes] for _ in range(60)]

    def requant_stack(_):
        # per block: the four 3072 x 3072 weights in one batched call, the two larger ones one call each
        for blk in range(60):
            nv.quantize_batch([b for b, _ in stack[blk][:4]], src_scales=[sc for _, sc in stack[blk][:4]],
                              outs=qstack[blk][:4], workspace=ws, flags=flags)
            for j in range(4, 6):
                b, sc = stack[blk][j]
                nv.quantize(b, src_scale=sc, out=qstack[blk][j], workspace=ws, flags=flags)

    def requant_stack_single(_):
        for blk in range(60):
            for j in range(6):
                b, sc = stack[blk][j]
                nv.quantize(b, src_scale=sc, out=qstack[blk][j], workspace=ws, flags=flags)
    rs_ms = _timed(requant_stack, 3, 1)
    rs1_ms = _timed(requant_stack_single, 3, 1)
    rs_graph_ms = _graph_ms(requant_stack, 3)
    n_el = 60 * sum(r * c for r, c in shapes)
    del stack
    torch.cuda.empty_cache()
    t3 = torch.randn((4096, 12288), generator=g, device=dev).to(torch.bfloat16)
    amax_t3 = nv.amax_percentile(t3, 99.9, per_channel=True)[0].max().reshape(1).contiguous()
    c_out = {s_: torch.empty((4096, s_[0]), dtype=torch.float32, device=dev) for s_ in set(shapes)}
    qa_ws = torch.zeros(max(nv.workspace_size(nv.OP_GEMM_QA, 4096, r, c) for r, c in shapes), dtype=torch.uint8,
                        device=dev)

    def gemms(form):
        def run(_):
            for blk in range(60):
                for j, sh in enumerate(shapes):
                    act, am = (a1, amax_a) if sh[1] == 3072 else (t3, amax_t3)
                    if form == "w4a4":
                        nv.gemm_qa(act, qstack[blk][j], am, out=c_out[sh], workspace=qa_ws)
                    else:
                        nv.gemm(act, qstack[blk][j], out=c_out[sh])
        return run
    fl5 = 60 * sum(2.0 * 4096 * r * c for r, c in shapes)
    g4_ms = _timed(gemms("w4a4"), 2, 1)
    g16_ms = _timed(gemms("w4a16"), 2, 1)
    nv.check_flags(flags, "config quantizers")
    out["calibration_stack"] = {
        "percentile_p999_217088x3072": _rate(rows * C * 2.0, pct_ms, "GB/s"),
        "requantize_360": dict(_rate(n_el * 1.5625 + 360 * 4, rs_ms, "GB/s"), per_weight_ms=round(rs_ms / 360, 5),
                               note="per block: the four 3072 x 3072 weights in one nvfp4_quantize_batch call, "
                                    "the two 3072 x 12288 ones one nvfp4_quantize call each"),
        "requantize_360_one_call_each": _rate(n_el * 1.5625 + 360 * 4, rs1_ms, "GB/s"),
        "gemm_w4a4_static_amax_360": dict(_rate(fl5, g4_ms, "TFLOP/s"),
                                          note="activations quantized under the calibrated amax by the same call"),
        "gemm_w4a16_360": _rate(fl5, g16_ms, "TFLOP/s"),
    }
    if rs_graph_ms:
        out["calibration_stack"]["requantize_360_graph"] = dict(
            _rate(n_el * 1.5625 + 360 * 4, rs_graph_ms, "GB/s"), note="the 180 calls replayed from a HIP graph")
    return out


# ------------------------------------------------------------------------------------------------
# the CPU oracle on the host's cores
# ------------------------------------------------------------------------------------------------
_CPU = {}  # inputs of the CPU baseline, inherited by the forked workers


def _cpu_op(name, lo, hi):
    """One slice [lo, hi) of one baseline op, with the oracle as it stands (one BLAS thread)."""
    import oracle
    d = _CPU
    if name == "quantize_attn_w":
        oracle.quantize(d["w2"][lo:hi])
    elif name == "dequantize_attn_w":
        q = d["q2"]
        oracle.dequantize(oracle.QTensor(q.codes[lo:hi], q.scales[lo:hi], q.g), "bf16")
    elif name == "gemm_w4a16_attn":
        oracle.gemm_w4a16(d["a2"][lo:hi], d["q2"])
    elif name == "percentile_attn_a":
        oracle.amax_percentile(d["a2"][:, lo:hi], 99.9, per_channel=True, dtype=oracle.BF16)
    elif name == "quantize_modulation":
        oracle.quantize(d["w3"][lo:hi])
    elif name == "requantize_modulation_fp8":
        oracle.quantize(d["b3"][lo:hi], oracle.E4M3, d["s3"])
    elif name == "gemv_modulation":
        q = d["q3"]
        oracle.gemm_w4a16(d["a3"], oracle.QTensor(q.codes[lo:hi], q.scales[lo:hi], q.g))
    elif name == "gemm_w4a4_mlp_gate":
        oracle.gemm_w4a4(oracle.QTensor(d["qa4"].codes[lo:hi], d["qa4"].scales[lo:hi], d["qa4"].g), d["qg4"])
    elif name == "percentile_calibration":
        oracle.amax_percentile(d["x5"][:, lo:hi], 99.9, per_channel=True, dtype=oracle.BF16)
    elif name == "requantize_stack_block":
        oracle.quantize(d["b5"][lo:hi], oracle.E4M3, d["s5"])
    else:
        raise ValueError(name)


def _cpu_worker(task):
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        _cpu_op(*task)


def cpu_baseline():
    """The CPU oracle (plain scalar C with numpy float64 matmuls; never tuned for speed) on bounded
    samples of the workloads, timed once on one thread and once split by rows (or channels) over a
    pool of worker processes, one per usable core (at most 16).  Runs before the GPU is
    initialised: the pool forks."""
    import multiprocessing as mp

    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    import synth
    t_gen = time.perf_counter()
    d = _CPU
    d["w2"] = synth.attn_proj_weight(N_OUT, K_IN)
    d["q2"], _ = oracle.quantize(d["w2"])
    d["a2"] = synth.attn_proj_activations(M_TOK, K_IN)[:, :]
    d["w3"] = synth.normal_f32((4608, 3072), 0.01, 3000)       # first quarter of the modulation weight
    d["b3"], d["s3"] = synth.modulation_fp8(0, rows=4608)       # a quarter-size FP8 weight of the batch
    d["q3"], _ = oracle.quantize(synth.normal_f32((4608, 3072), 0.01, 3000))
    d["a3"] = synth.modulation_activations(2, 3072)
    wg = synth.normal_f32((1536, 4096), 0.015, 4000)            # first 1536 of 12288 rows of the gate weight
    d["qg4"], _ = oracle.quantize(wg)
    d["qa4"], _ = oracle.quantize(synth.mlp_activations(512, 4096), oracle.BF16)
    d["x5"] = synth.bf16_bits(np.random.default_rng(5000).standard_t(3, size=(53 * 4096, 32)).astype(np.float32))
    d["b5"], d["s5"] = synth.stack_weight_fp8(0, 0)
    t_gen = time.perf_counter() - t_gen

    # (op, unit, work per item, items, item axis description, sample description)
    N2 = N_OUT * K_IN
    ops = [
        ("quantize_attn_w", "GB/s", 4.5625 * K_IN, N_OUT, "rows", "attention W 3072x3072 fp32"),
        ("dequantize_attn_w", "GB/s", 2.5625 * K_IN, N_OUT, "rows", "attention W NVFP4 -> bf16"),
        ("gemm_w4a16_attn", "TFLOP/s", 2.0 * N_OUT * K_IN, 1024, "rows", "1024 of 4096 activation rows x W 3072x3072"),
        ("percentile_attn_a", "GB/s", 2.0 * M_TOK, 768, "channels", "768 of 3072 channels x 4096 rows"),
        ("quantize_modulation", "GB/s", 4.5625 * 3072, 4608, "rows", "4608 of 18432 rows, fp32"),
        ("requantize_modulation_fp8", "GB/s", 1.5625 * 3072, 4608, "rows", "4608x3072 FP8 weight"),
        ("gemv_modulation", "GB/s", 0.5625 * 3072, 4608, "rows", "M=2 against 4608 of 18432 rows"),
        ("gemm_w4a4_mlp_gate", "TFLOP/s", 2.0 * 1536 * 4096, 512, "rows",
         "512 activation rows x the first 1536 of 12288 gate rows"),
        ("percentile_calibration", "GB/s", 2.0 * 53 * 4096, 32, "channels", "32 of 3072 channels x 217088 rows"),
        ("requantize_stack_block", "GB/s", 1.5625 * 3072, 3072, "rows", "block 0, weight 0: 3072x3072 FP8"),
    ]
    usable = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    workers = max(1, min(16, usable))
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    res = {}
    t_all = 0.0
    reps = CPU_REPS
    ctx = mp.get_context("fork")
    with ctx.Pool(workers) as pool:
        pool.map(_cpu_worker, [("quantize_attn_w", 0, 8)] * workers)  # start the workers
        for name, unit, per_item, items, axis, sample in ops:
            with threadpool_limits(1):
                t0 = time.perf_counter()
                for _ in range(reps):
                    _cpu_op(name, 0, items)
                t1 = time.perf_counter() - t0
            cuts = np.linspace(0, items, workers + 1).astype(int)
            tasks = [(name, int(cuts[k]), int(cuts[k + 1])) for k in range(workers) if cuts[k + 1] > cuts[k]]
            t0 = time.perf_counter()
            pool.map(_cpu_worker, tasks * reps, chunksize=1)
            tn = time.perf_counter() - t0
            t_all += t1 + tn
            amount = per_item * items * reps
            scale = 1e9 if unit == "GB/s" else 1e12
            res[name] = {"unit": unit, "one_thread": round(amount / t1 / scale, 5),
                         "all_cores": round(amount / tn / scale, 5), "threads": len(tasks),
                         "s_one_thread": round(t1, 3), "s_all_cores": round(tn, 3),
                         "sample": f"{sample}, {reps} times, split by {axis} over the workers"}
    head = res["quantize_attn_w"]
    return {"value": head["all_cores"], "unit": "GB/s", "cores": head["threads"], "kind": "oracle",
            "sample": "quantize of the attention W 3072x3072 fp32 (the headline op), rows split over the "
                      "worker processes, each slice quantized as a tensor of its own (the same work per element)",
            "nproc": os.cpu_count(), "usable_cpus": usable, "cpu_model": model, "threads": workers,
            "seconds": round(t_all, 1), "input_generation_s": round(t_gen, 1), "ops": res}


if __name__ == "__main__":
    main()
