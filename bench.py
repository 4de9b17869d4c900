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
bracketed by events on the stream it runs on; the dominant kernel's roofline uses those times.

The JSON line also carries "graph": the step and the quantize alone captured in HIP graphs and
replayed (no eager dispatch gaps between kernels), for information.

Prints one JSON line.  Flags: --gpus (1 only), --steps, --warmup, --no-cpu-baseline, --peaks (adds the
achievable peaks measured with library calls: a 1 GiB device copy and a bf16 matmul of the GEMM's shape).
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--peaks", action="store_true",
                    help="also measure achievable peaks: HBM by a 1 GiB device-to-device copy, matrix cores by "
                         "a bf16 torch.matmul of the attention-projection shape")
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

    import numpy as np
    import torch

    import bit_gemm_nvfp4_amd as nv
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

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
    qa_ws = torch.empty(max(nv.workspace_size(nv.OP_GEMM_QA, M_TOK, N_OUT, K_IN), 1), dtype=torch.uint8, device=dev)
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
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    op_ms = {op: float(np.mean([evs[s][j].elapsed_time(evs[s][j + 1]) for s in range(args.steps)]))
             for j, op in enumerate(ops)}
    # the FP8 side path, in its own loop (the step above stays the NVFP4 path alone)
    for i in range(args.warmup):
        step_next(i)
    torch.cuda.synchronize()
    evn = [[torch.cuda.Event(enable_timing=True) for _ in range(len(next_ops) + 1)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(args.warmup + i)
        step_next(args.warmup + i, evn[i])
    torch.cuda.synchronize()
    op_ms.update({op: float(np.mean([evn[s][j].elapsed_time(evn[s][j + 1]) for s in range(args.steps)]))
                  for j, op in enumerate(next_ops)})

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
    graph = graph_rates()
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
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w_np)
    if args.peaks:
        out["achievable_peaks"] = achievable_peaks(dev)
    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    print(json.dumps(out), flush=True)


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


def cpu_baseline(w_np):
    """The oracle's quantizer (plain scalar C, one thread) on the same 3072 x 3072 fp32 weight,
    repeated until about 10 s of CPU time have passed."""
    import oracle
    n_bytes = w_np.size * 4.5625 + 4
    reps, t = 0, 0.0
    while t < 10.0 and reps < 20:
        t0 = time.perf_counter()
        oracle.quantize(w_np)
        t += time.perf_counter() - t0
        reps += 1
    return {"value": round(n_bytes * reps / t / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} x quantize of the 3072x3072 fp32 weight (oracle C, single thread), {t:.1f} s"}


if __name__ == "__main__":
    main()
