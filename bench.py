#!/usr/bin/env python3
"""Throughput of the I2_S W2A8 matmul hot path on one MI355X.

One step = the whole hot path on one batch: quantize the F32 activation rows
(amax/127 scale, int8 values, int8 row sums) and run the ternary contraction
with its fused epilogue (i2s_mul_mat).  Packing the weights happens once,
before timing, as it does offline for a checkpoint.

Default workload: the Qwen2-1.5B FFN up projection at decode time, ternary
weight [8960][1536] (P(-1,0,+1) = 0.3/0.4/0.3, scale 0.015) against one F32
activation row ~ N(0,1) with 1% of its entries scaled by 20, seed 0 (the
line's value, against HBM); beside it, under "prefill_gemm", the gate
projection's prefill: the same weight shape against 512 rows ~ N(0,1), whose
contraction is the int8-MFMA GEMM (its roofline against int8 MFMA).

Measurement:
  * every input is resident in device memory before the timed region; the
    packed weight is replicated into enough distinct copies (>= 512 MiB in
    total, twice the 256 MiB Infinity Cache) and step i uses copy i mod R,
    so each step reads its weights from HBM, as a 28-layer decode does;
  * the K timed steps are captured in a HIP graph (launches from Python
    would otherwise be slower than the kernels), repeated inside it as many
    times as make a run of about --min-region-ms (starting a graph costs a
    few microseconds, which a 20-step graph would spread over its steps), and
    the graph is replayed between two HIP events on the launch stream,
    bracketed by device synchronizations; ms_per_step is the region over the
    steps it ran (config.timed_steps);
  * the dominant kernel's average launch duration comes from a second graph of
    back-to-back launches of that kernel alone, timed the same way inside the
    same bracket; roofline.achieved = algorithmic bytes per launch / that time;
  * cpu_baseline: the CPU oracle (plain scalar C) on the same workload,
    repeated for about --cpu-seconds: half of it on all host cores (up to
    16 threads, output features split), half on one thread.

--workload encoder_mlp times one I8_S encoder block MLP instead (stage 3 of a
4-second clip: FC1 256 -> 1024 with bias and ReLU, then FC2 1024 -> 256 with
bias, 6000 positions, I8_S in and out: i8s_mul_mat_add_relu then
i8s_mul_mat_add, four launches); its roofline line is the FC1 op (both of its
passes) against HBM.

--workload w8a8_prefill / w8a8_decode time the per-channel W8A8 matmul of
the NPU page on the gate projection's shape (8960 x 1536; 512 rows, or one):
quantize the activation rows, then the int8-MFMA contraction with its F32
dequantizing epilogue (two launches); weights quantized once beforehand.

--workload decode_layer times one Qwen2-1.5B decoder layer's seven ternary
projections at N = 1 instead (q/k/v grouped with their F32 biases, o,
gate/up grouped, down: four launches), rotating over 28 layers of weights
(327.5 MB), beside the same projections as seven separate calls.

--workload layer_sweep times each of the seven projections on its own at
N = 1 and at N = 64 (fourteen i2s_mul_mat calls per step, each weight
rotating over >= 512 MiB of copies) and reports every one of them: step and
dominant-kernel time, weight GB/s, int8 TOPS and its roofline fraction.

Prints one JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "I2_S W2A8 matmul: weight GB/s & int8 TOPS at 1 GPU; % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, 8.0 TB/s
INT8_MFMA_PEAK_TOPS = 5000.0  # MI355X dense int8 MFMA, 5.0 POP/s
ROTATE_BYTES = 512 << 20
KERNEL_SRC = os.path.join(ROOT, "ternary_weight_integer_amd", "csrc", "i2s.hip")
KERNEL_SRC_I8S = os.path.join(ROOT, "ternary_weight_integer_amd", "csrc", "i8s.hip")


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=1000)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--workload", default="decode_up",
                   choices=["decode_up", "prefill_gate", "down_small_batch", "small", "decode_layer", "encoder_mlp",
                            "w8a8_prefill", "w8a8_decode", "layer_sweep"])
    p.add_argument("--stage", type=int, default=3, help="encoder stage of --workload encoder_mlp (0..6)")
    p.add_argument("--copies", type=int, default=0, help="weight copies to rotate over (0 = enough for 512 MiB)")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--eager", action="store_true",
                   help="launch from Python without graphs (for counter collection runs)")
    p.add_argument("--no-prefill", action="store_true",
                   help="default workload only: skip the prefill GEMM reported beside the decode GEMV")
    p.add_argument("--min-region-ms", type=float, default=3.0,
                   help="repeat the K steps inside the timed graph until it runs for about this long")
    p.add_argument("--copy-kernel-mib", type=int, default=0,
                   help="only run a plain copy of this many MiB (counter calibration) and exit")
    return p.parse_args(argv)


def make_case(name):
    from ternary_weight_integer_amd import workloads
    return {
        "decode_up": workloads.decode_up_case,
        "prefill_gate": workloads.prefill_gate_case,
        "down_small_batch": workloads.down_small_batch_case,
        "small": workloads.small_case,
    }[name]()


CASE_WORKLOAD = {"decode_up_8960x1536_N1": "decode_up", "prefill_gate_8960x1536_N512": "prefill_gate",
                 "down_1536x8960_N8": "down_small_batch"}


def case_workload(case) -> str:
    """The --workload name of a case (the key of its traffic summary)."""
    return CASE_WORKLOAD.get(case.name, case.name)


def kernel_source_digest(workload: str = "") -> str:
    i8s = workload == "encoder_mlp" or workload.startswith("w8a8_")
    with open(KERNEL_SRC_I8S if i8s else KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, or None if there is none or the kernel source changed since."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_b = re.search(r"^traffic_bytes_per_launch:\s*([0-9.]+)", text, re.M)
    m_h = re.search(r"^kernel_source_sha256_16:\s*([0-9a-f]+)", text, re.M)
    if not m_b or not m_h or m_h.group(1) != kernel_source_digest(workload):
        return None
    return float(m_b.group(1))


def cpu_baseline(case, seconds: float):
    """The oracle, unchanged, on all host cores: the output features are split
    into one row slice per thread (a row slice of the packed payload plus the
    scale slot is itself a packed tensor), each thread calls the scalar C
    oracle on its slice (ctypes releases the GIL), as the pages' schedule
    splits output features over threads.  Also timed on one thread."""
    import concurrent.futures

    import numpy as np

    import oracle
    packed = oracle.pack(case.w, case.ws)
    rb = case.K // 4
    slot = packed[case.rows * rb:]
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    bounds = [case.rows * i // cores for i in range(cores + 1)]
    slices = [(np.concatenate([packed[a * rb:b * rb], slot]), b - a) for a, b in zip(bounds, bounds[1:]) if b > a]

    def run(sl):
        oracle.mul_mat(sl[0], sl[1], case.K, case.x)

    def timed(fn, budget):
        calls, t0 = 0, time.perf_counter()
        while True:
            fn()
            calls += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return calls, el

    with concurrent.futures.ThreadPoolExecutor(max_workers=len(slices)) as pool:
        calls, el = timed(lambda: list(pool.map(run, slices)), seconds / 2)
    calls1, el1 = timed(lambda: oracle.mul_mat(packed, case.rows, case.K, case.x), seconds / 2)
    wbytes = case.rows * case.K // 4
    return {"value": round(wbytes * calls / el / 1e9, 6), "unit": "GB/s", "cores": len(slices), "kind": "oracle",
            "sample": f"{calls} full calls of the same workload ({case.name}, quantize+contract+epilogue, scalar C) "
                      f"on {len(slices)} threads, output features split, in {el:.1f} s",
            "one_thread": {"value": round(wbytes * calls1 / el1 / 1e9, 6), "calls": calls1,
                           "ms_per_call": round(el1 / calls1 * 1e3, 3)},
            "cpu_model": cpu_model(), "host_cores": len(os.sched_getaffinity(0)),
            "ms_per_call": round(el / calls * 1e3, 3)}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def graph_of(fn, torch):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm the allocator and the launch path outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def copy_kernel_only(mib: int):
    import torch
    dev = torch.device("cuda:0")
    n = (mib << 20) // 4
    a = torch.ones(n, device=dev)
    b = torch.empty(n, device=dev)
    for _ in range(5):
        torch.mul(a, 1.0, out=b)
    torch.cuda.synchronize()
    print(json.dumps({"copy_kernel_mib": mib, "bytes_read": n * 4, "bytes_written": n * 4, "launches": 5}), flush=True)


def kernel_name_of(kind: int, variant: int) -> str:
    if kind == 2:
        if variant == 15:
            return "gemm_wk_kernel"
        return "gemm_pipe_kernel" if variant == 10 else ("gemm_res_kernel" if variant >= 5 else "gemm_kernel")
    return {1: "gemv_kernel", 3: "gemv_fused_kernel", 4: "gemv_mfma_kernel"}[kind]


def alg_bytes_of(kind: int, rows: int, K: int, N: int) -> int:
    """Algorithmic bytes of one launch of the dominant kernel.  Fused: packed
    weights + F32 activations + F32 outputs + the weight scale.  Otherwise:
    packed weights + int8 activations + F32 outputs + per-row scale and row
    sum + the weight scale."""
    if kind == 3:
        return rows * K // 4 + 4 * N * K + 4 * N * rows + 4
    return rows * K // 4 + N * K + 4 * N * rows + 8 * N + 4


def copy_ceiling(torch, nbytes: int):
    """A plain copy kernel moving the same number of bytes as one launch of
    the dominant kernel (half read, half written; F32 elementwise copy),
    sources rotating over >= 512 MiB so reads come from HBM: the attainable
    time of a memory-bound kernel this short on this GPU."""
    dev = torch.device("cuda:0")
    n = max(64, (nbytes // 2 + 255) // 256 * 64)   # floats per copy, 256-byte multiple
    R = max(1, -(-ROTATE_BYTES // (4 * n)))
    src = torch.ones(R * n, dtype=torch.float32, device=dev)
    dst = torch.empty(n, dtype=torch.float32, device=dev)
    launches = max(R, 256)
    g = graph_of(lambda: [torch.mul(src[(i % R) * n:(i % R + 1) * n], 1.0, out=dst) for i in range(launches)], torch)
    g.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / launches
    moved = 8 * n
    del g, src, dst
    return {"bytes_moved": moved, "us": round(us, 4), "gbs": round(moved / (us * 1e-6) / 1e9, 2),
            "frac_of_hbm": round(moved / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "sources_rotated": R}


LAYER_PROJ = ("q", "k", "v", "o", "gate", "up", "down")
LAYERS = 28


def bench_layer(args, torch, i2s):
    """One Qwen2-1.5B decoder layer's seven ternary projections at decode time
    (N = 1) per step, weights rotating over 28 layers (327.5 MB, beyond the
    Infinity Cache): grouped as q/k/v (one launch, F32 biases), o, gate/up
    (one launch), down -- four launches -- and, for comparison, as seven
    separate calls."""
    from ternary_weight_integer_amd import workloads
    dev = torch.device("cuda:0")
    case = workloads.decode_layer_case(N=1)
    shp = workloads.QWEN2_1P5B_PROJ
    p0 = {n: i2s.i2s_pack(torch.from_numpy(case.w[n]).to(dev), case.ws) for n in LAYER_PROJ}
    layers = [p0] + [{n: p0[n].clone() for n in LAYER_PROJ} for _ in range(LAYERS - 1)]
    bias = {n: torch.from_numpy(case.bias[n]).to(dev) for n in ("q", "k", "v")}
    xh, xa, xf = (torch.from_numpy(a).to(dev) for a in (case.x_hidden, case.x_attn, case.x_ffn))
    ws = i2s.new_workspace(1, 8960, dev)
    y = {n: torch.empty((1, shp[n][0]), dtype=torch.float32, device=dev) for n in LAYER_PROJ}
    y2 = {n: torch.empty((1, shp[n][0]), dtype=torch.float32, device=dev) for n in LAYER_PROJ}
    wbytes = sum(shp[n][0] * shp[n][1] // 4 for n in LAYER_PROJ)

    def grouped(i, out=y):
        lw = layers[i % LAYERS]
        i2s.i2s_mul_mat_group([(lw["q"], 1536), (lw["k"], 256), (lw["v"], 256)], 1536, xh,
                              biases=[bias["q"], bias["k"], bias["v"]], workspace=ws, ys=[out["q"], out["k"], out["v"]])
        i2s.i2s_mul_mat(lw["o"], 1536, 1536, xa, workspace=ws, y=out["o"])
        i2s.i2s_mul_mat_group([(lw["gate"], 8960), (lw["up"], 8960)], 1536, xa, workspace=ws,
                              ys=[out["gate"], out["up"]])
        i2s.i2s_mul_mat(lw["down"], 1536, 8960, xf, workspace=ws, y=out["down"])

    def separate(i, out=y2):
        lw = layers[i % LAYERS]
        for n, x in (("q", xh), ("k", xh), ("v", xh), ("o", xa), ("gate", xa), ("up", xa), ("down", xf)):
            rows, K = shp[n]
            i2s.i2s_mul_mat_group([(lw[n], rows)], K, x, biases=[bias.get(n)], workspace=ws, ys=[out[n]])

    def gate_up(i):
        lw = layers[i % LAYERS]
        i2s.i2s_mul_mat_group([(lw["gate"], 8960), (lw["up"], 8960)], 1536, xa, workspace=ws,
                              ys=[y["gate"], y["up"]])

    for i in range(args.warmup):
        grouped(i)
        separate(i)
    torch.cuda.synchronize()
    if args.eager:  # launches from Python, one dispatch at a time (counter collection runs)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(args.steps):
            grouped(i)
        e1.record()
        torch.cuda.synchronize()
        return {"metric": METRIC, "value": None, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
                "warmup": args.warmup, "ms_per_step": round(e0.elapsed_time(e1) / args.steps, 6),
                "config": {"workload": case.name, "timing": "eager"}}
    for n in LAYER_PROJ:  # grouping changes no result bit
        if not torch.equal(y[n].view(torch.int32), y2[n].view(torch.int32)):
            raise RuntimeError(f"grouped and separate results differ for {n}")
    K_steps = args.steps
    g1 = graph_of(lambda: [grouped(i) for i in range(K_steps)], torch)
    g2 = graph_of(lambda: [separate(i) for i in range(K_steps)], torch)
    n_kern = 256
    g3 = graph_of(lambda: [gate_up(i) for i in range(n_kern)], torch)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record()
    g1.replay()
    ev[1].record()
    g2.replay()
    ev[2].record()
    g3.replay()
    ev[3].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = ev[0].elapsed_time(ev[1]) / K_steps
    sep_ms = ev[1].elapsed_time(ev[2]) / K_steps
    kern_us = ev[2].elapsed_time(ev[3]) * 1e3 / n_kern
    alg = 2 * 8960 * 1536 // 4 + 4 * 1536 + 2 * 4 * 8960 + 8   # gate+up weights, x, outputs, two scales
    achieved = alg / (kern_us * 1e-6) / 1e9
    out = {
        "metric": METRIC,
        "value": round(wbytes / (step_ms * 1e-3) / 1e9, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": case.name, "layers_rotated": LAYERS, "weight_bytes_per_step": wbytes,
                   "rotated_bytes": LAYERS * sum(p.numel() for p in p0.values()), "launches_per_step": 4,
                   "timing": "hip_graph"},
        "separate_calls": {"launches_per_step": 7, "ms_per_step": round(sep_ms, 6),
                           "value": round(wbytes / (sep_ms * 1e-3) / 1e9, 3)},
        "int8_tops": round(2 * (wbytes * 4) / (step_ms * 1e-3) / 1e12, 4),
        "wall_s": round(wall, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(args.workload),
                     "kernel": "gemv_fused_pair_kernel (gate+up)", "kernel_us": round(kern_us, 4),
                     "alg_bytes_per_launch": alg},
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline_layer(case, args.cpu_seconds)
    return out


def bench_encoder(args, torch):
    """One I8_S encoder block MLP per step: FC1 (+bias, ReLU, requantize) then
    FC2 (+bias, requantize), FC2 reading FC1's I8_S output.  The inputs stay
    hot in the Infinity Cache across steps, as they are when the previous op
    of the block has just written them."""
    from ternary_weight_integer_amd import i8s, workloads
    dev = torch.device("cuda:0")
    case = workloads.encoder_mlp_case(stage=args.stage)
    C, N, H = case.C, case.N, case.w1.shape[0]
    W1 = i8s.i8s_tensor(case.w1, case.w1_scale, dev)
    W2 = i8s.i8s_tensor(case.w2, case.w2_scale, dev)
    X = i8s.i8s_tensor(case.x, case.x_scale, dev)
    b1, b2 = torch.from_numpy(case.b1).to(dev), torch.from_numpy(case.b2).to(dev)
    Hb = torch.empty(i8s.i8s_bytes(N * H), dtype=torch.uint8, device=dev)
    Yb = torch.empty(i8s.i8s_bytes(N * C), dtype=torch.uint8, device=dev)
    ws1, ws2 = i8s.new_workspace(dev), i8s.new_workspace(dev)

    def step():
        i8s.i8s_mul_mat_add_relu(W1, H, C, X, N, b1, out=Hb, workspace=ws1)
        i8s.i8s_mul_mat_add(W2, C, H, Hb, N, b2, out=Yb, workspace=ws2)

    def fc1():
        i8s.i8s_mul_mat_add_relu(W1, H, C, X, N, b1, out=Hb, workspace=ws1)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    h_eager, y_eager = Hb.clone(), Yb.clone()
    K_steps = args.steps
    if args.eager:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(K_steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        step_ms, kern_us, wall = e0.elapsed_time(e1) / K_steps, None, None
    else:
        g_step = graph_of(lambda: [step() for _ in range(K_steps)], torch)
        n_kern = 256
        g_kern = graph_of(lambda: [fc1() for _ in range(n_kern)], torch)
        g_step.replay()
        g_kern.replay()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        t0 = time.perf_counter()
        ev[0].record()
        g_step.replay()
        ev[1].record()
        g_kern.replay()
        ev[2].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        step_ms = ev[0].elapsed_time(ev[1]) / K_steps
        kern_us = ev[1].elapsed_time(ev[2]) * 1e3 / n_kern
    if not (torch.equal(Hb, h_eager) and torch.equal(Yb, y_eager)):
        raise RuntimeError("graph replay result differs from the eager result")
    slot = i8s.I8S_SCALE_SLOT
    fc1_bytes = H * C + N * C + 4 * H + N * H + 3 * slot
    fc2_bytes = C * H + N * H + 4 * C + N * C + 3 * slot
    ops = 2 * 2 * N * H * C
    out = {
        "metric": METRIC,
        "value": round((fc1_bytes + fc2_bytes) / (step_ms * 1e-3) / 1e9, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": case.name, "stage": case.stage, "C": C, "hidden": H, "N": N,
                   "launches_per_step": 4, "variant_fc1": i8s.i8s_mul_mat_add_variant(H, C, N),
                   "variant_fc2": i8s.i8s_mul_mat_add_variant(C, H, N),
                   "timing": "eager" if args.eager else "hip_graph",
                   "value_is": "algorithmic bytes (weights, I8_S input and output, biases) per second"},
        "int8_tops": round(ops / (step_ms * 1e-3) / 1e12, 4),
        "wall_s": None if wall is None else round(wall, 4),
    }
    if kern_us is not None:
        achieved = fc1_bytes / (kern_us * 1e-6) / 1e9
        out["roofline"] = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(args.workload),
                           "kernel": "i8s_mm_mfma_kernel (FC1: max|f| pass + requantize pass)",
                           "kernel_us": round(kern_us, 4), "alg_bytes_per_launch": fc1_bytes,
                           "int8_tops": round(2 * N * H * C / (kern_us * 1e-6) / 1e12, 3)}
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline_encoder(case, args.cpu_seconds, fc1_bytes + fc2_bytes)
    return out


def bench_w8a8(args, torch):
    """Per-channel W8A8: quantize the activation rows and contract (two
    launches, or for M <= 4 one launch that does both); weight copies rotate
    through >= 512 MiB as for I2_S."""
    from ternary_weight_integer_amd import w8a8, workloads
    dev = torch.device("cuda:0")
    case = workloads.w8a8_case(args.workload.split("_", 1)[1])
    OC, K, M = case.OC, case.K, case.M
    wq0, ws0 = w8a8.w8a8_quantize_weight(torch.from_numpy(case.w).to(dev))
    R = args.copies or max(1, -(-ROTATE_BYTES // wq0.numel()))
    copies = [(wq0, ws0)] + [(wq0.clone(), ws0.clone()) for _ in range(R - 1)]
    x = torch.from_numpy(case.x).to(dev)
    ws = w8a8.new_workspace(M, K, dev)
    y = torch.empty((M, OC), dtype=torch.float32, device=dev)
    aq = torch.empty((M, K), dtype=torch.int8, device=dev)
    asc = torch.empty(M, dtype=torch.float32, device=dev)
    w8a8.w8a8_quantize_act(x, aq, asc)
    variant = w8a8.w8a8_mul_mat_variant(OC, K, M)
    fused = variant == 11  # the step is one launch: quantizer and contraction together

    def step(i):
        wq, wsc = copies[i % R]
        w8a8.w8a8_mul_mat(wq, wsc, x, workspace=ws, y=y)

    def contraction(i):
        wq, wsc = copies[i % R]
        if fused:
            w8a8.w8a8_mul_mat(wq, wsc, x, workspace=ws, y=y)
        else:
            w8a8.w8a8_matmul(wq, wsc, aq, asc, y=y)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    y_eager = y.clone()
    K_steps = args.steps
    if args.eager:  # launches from Python, one dispatch at a time (counter collection runs)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(K_steps):
            step(i)
        e1.record()
        torch.cuda.synchronize()
        return {"metric": METRIC, "value": None, "unit": "GB/s", "n_gpus": 1, "steps": K_steps,
                "warmup": args.warmup, "ms_per_step": round(e0.elapsed_time(e1) / K_steps, 6),
                "config": {"workload": case.name, "timing": "eager"}}
    g_step = graph_of(lambda: [step(i) for i in range(K_steps)], torch)
    n_kern = max(R, 64)
    g_kern = graph_of(lambda: [contraction(i) for i in range(n_kern)], torch)
    g_step.replay()
    g_kern.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    t0 = time.perf_counter()
    ev[0].record()
    g_step.replay()
    ev[1].record()
    g_kern.replay()
    ev[2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if not torch.equal(y.view(torch.int32), y_eager.view(torch.int32)):
        raise RuntimeError("graph replay result differs from the eager result")
    step_ms = ev[0].elapsed_time(ev[1]) / K_steps
    kern_us = ev[1].elapsed_time(ev[2]) * 1e3 / n_kern
    ops = 2 * OC * K * M
    wbytes = OC * K + 4 * OC
    # the dominant launch's operands: F32 rows for the fused launch, else the codes and scales
    alg_bytes = wbytes + (4 * M * K if fused else M * K + 4 * M) + 4 * M * OC
    out = {
        "metric": METRIC,
        "value": round(wbytes / (step_ms * 1e-3) / 1e9, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": case.name, "OC": OC, "K": K, "M": M, "weight_copies_rotated": R,
                   "variant": variant, "timing": "hip_graph",
                   "value_is": "int8 weight bytes (+ channel scales) per second"},
        "int8_tops": round(ops / (step_ms * 1e-3) / 1e12, 4),
        "wall_s": round(wall, 4),
    }
    if fused:
        kname = "w8a8_gemv_fused_kernel (activation quantizer, int8 GEMV and F32 dequantizing epilogue in one launch)"
    else:
        kname = {9: "i8s_mm_skinny_kernel", 10: "w8a8_res_kernel"}.get(variant, "i8s_mm_mfma_kernel") + \
            " (F32 dequantizing epilogue)"
    if M >= 64:
        achieved = ops / (kern_us * 1e-6) / 1e12
        out["roofline"] = {"bound": "mfma", "achieved": round(achieved, 2), "peak": INT8_MFMA_PEAK_TOPS,
                           "unit": "TOP/s", "frac": round(achieved / INT8_MFMA_PEAK_TOPS, 4),
                           "traffic": measured_traffic(args.workload), "kernel": kname, "kernel_variant": variant,
                           "kernel_us": round(kern_us, 4), "alg_ops_per_launch": ops, "alg_bytes_per_launch": alg_bytes}
    else:
        achieved = alg_bytes / (kern_us * 1e-6) / 1e9
        out["roofline"] = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(args.workload),
                           "kernel": kname, "kernel_variant": variant, "kernel_us": round(kern_us, 4),
                           "alg_bytes_per_launch": alg_bytes}
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline_w8a8(case, args.cpu_seconds)
    return out


def bench_sweep(args, torch, i2s):
    """Each Qwen2-1.5B projection alone at N = 1 and N = 64 (ws 0.015, x ~
    N(0,1)).  A step is the fourteen i2s_mul_mat calls once each; every
    projection's packed weight is replicated into >= 512 MiB of copies and
    call i of a case uses copy i mod R, so weights come from HBM.  Per case,
    its own graph of the whole call (max(R, 256) launches) and one of the
    dominant kernel alone give the step and kernel times."""
    from ternary_weight_integer_amd import workloads
    dev = torch.device("cuda:0")
    cases = workloads.layer_sweep_cases()
    ws = i2s.new_workspace(64, 8960, dev)
    copies = {}
    prepared = []
    for c in cases:
        proj = c.meta["proj"]
        if proj not in copies:
            p0 = i2s.i2s_pack(torch.from_numpy(c.w).to(dev), c.ws)
            R = max(1, -(-ROTATE_BYTES // p0.numel()))
            copies[proj] = [p0] + [p0.clone() for _ in range(R - 1)]
        x = torch.from_numpy(c.x).to(dev)
        y = torch.empty((c.N, c.rows), dtype=torch.float32, device=dev)
        prepared.append((c, copies[proj], x, y))
    torch.cuda.synchronize()

    def call(pc, i):
        c, cp, x, y = pc
        i2s.i2s_mul_mat(cp[i % len(cp)], c.rows, c.K, x, workspace=ws, y=y)

    def timed_graph(fn, n):
        g = graph_of(lambda: [fn(i) for i in range(n)], torch)
        g.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n  # us per launch

    for i in range(args.warmup):
        for pc in prepared:
            call(pc, i)
    torch.cuda.synchronize()
    eager = [pc[3].clone() for pc in prepared]
    K_steps = args.steps
    g = graph_of(lambda: [call(pc, i) for i in range(K_steps) for pc in prepared], torch)
    g.replay()
    torch.cuda.synchronize()
    for pc, ye in zip(prepared, eager):
        if not torch.equal(pc[3].view(torch.int32), ye.view(torch.int32)):
            raise RuntimeError(f"graph replay result differs from the eager result for {pc[0].name}")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = e0.elapsed_time(e1) / K_steps

    rows_out, wbytes_step, ops_step, kern_total = [], 0, 0, {}
    for j, pc in enumerate(prepared):
        c, cp, x, y = pc
        rows, K, N = c.rows, c.K, c.N
        n = max(len(cp), 256)
        call_us = timed_graph(lambda i: call(pc, i), n)
        kind = i2s.i2s_mul_mat_kernel(rows, K, N)
        variant = i2s.i2s_mul_mat_variant(rows, K, N)
        if kind == i2s.KERNEL_FUSED:
            kern = lambda i: i2s.i2s_mul_mat_ex(cp[i % len(cp)], rows, K, x, workspace=ws, y=y, kernel=kind)
        else:
            i2s.i2s_quantize_act_ws(x, ws)
            kern = lambda i: i2s.i2s_mul_mat_ws(cp[i % len(cp)], rows, K, N, ws, y=y, kernel=kind)
        kern_us = timed_graph(kern, n)
        if not torch.equal(y.view(torch.int32), eager[j].view(torch.int32)):
            raise RuntimeError(f"kernel-only result differs from the eager result for {c.name}")
        wb = rows * K // 4
        alg = alg_bytes_of(kind, rows, K, N)
        gbs = alg / (kern_us * 1e-6) / 1e9
        name = kernel_name_of(kind, variant)
        wbytes_step += wb
        ops_step += 2 * rows * K * N
        kern_total[name] = kern_total.get(name, 0.0) + kern_us
        ceiling = copy_ceiling(torch, alg)
        rows_out.append({"case": c.name, "rows": rows, "K": K, "N": N, "copies_rotated": len(cp),
                         "call_us": round(call_us, 3), "weight_gbs": round(wb / (call_us * 1e-6) / 1e9, 2),
                         "int8_tops": round(2 * rows * K * N / (call_us * 1e-6) / 1e12, 3),
                         "kernel": name, "kernel_variant": variant, "kernel_us": round(kern_us, 3),
                         "kernel_alg_bytes": alg, "kernel_gbs": round(gbs, 2),
                         "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                         "mfma_frac": round(2 * rows * K * N / (kern_us * 1e-6) / 1e12 / INT8_MFMA_PEAK_TOPS, 4),
                         "copy_ceiling_us": ceiling["us"]})
    # The dominant kernel of the sweep: the one with the most time summed over
    # the cases; its roofline line is its largest single case.
    dom = max(kern_total, key=kern_total.get)
    big = max((r for r in rows_out if r["kernel"] == dom), key=lambda r: r["kernel_us"])
    out = {
        "metric": METRIC,
        "value": round(wbytes_step / (step_ms * 1e-3) / 1e9, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": "qwen2_1p5b_projection_sweep_N1_N64", "calls_per_step": len(prepared),
                   "weight_bytes_per_step": wbytes_step, "timing": "hip_graph"},
        "int8_tops": round(ops_step / (step_ms * 1e-3) / 1e12, 4),
        "wall_s": round(wall, 4),
        "sweep": rows_out,
        "roofline": {"bound": "hbm", "achieved": big["kernel_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": big["hbm_frac"], "traffic": None, "kernel": f"{dom} ({big['case']})",
                     "kernel_us": big["kernel_us"], "alg_bytes_per_launch": big["kernel_alg_bytes"]},
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline_sweep(cases, args.cpu_seconds)
    return out


def cpu_baseline_sweep(cases, seconds: float):
    import oracle
    packed = {}
    for c in cases:
        packed.setdefault(c.meta["proj"], oracle.pack(c.w, c.ws))
    wbytes = sum(c.rows * c.K // 4 for c in cases)
    calls, t0 = 0, time.perf_counter()
    while True:
        for c in cases:
            oracle.mul_mat(packed[c.meta["proj"]], c.rows, c.K, c.x)
        calls += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": round(wbytes * calls / el / 1e9, 6), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{calls} full sweeps (14 calls: 7 projections at N = 1 and 64, scalar C, 1 thread) "
                      f"in {el:.1f} s",
            "cpu_model": cpu_model(), "host_cores": len(os.sched_getaffinity(0)),
            "ms_per_call": round(el / calls * 1e3, 3)}


def cpu_baseline_w8a8(case, seconds: float):
    import oracle
    wq, wsc = oracle.w8a8_quantize_weight(case.w)
    rows = min(case.M, 8)   # a bounded sample: rows are independent
    calls, t0 = 0, time.perf_counter()
    while True:
        oracle.w8a8_mul_mat(wq, wsc, case.x[:rows])
        calls += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    wbytes = case.OC * case.K + 4 * case.OC
    per_step = el / calls * case.M / rows
    return {"value": round(wbytes / per_step / 1e9, 6), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{calls} calls on {rows} of the {case.M} activation rows ({case.name}, scalar C, 1 thread) "
                      f"in {el:.1f} s, scaled to the full {case.M} rows",
            "cpu_model": cpu_model(), "host_cores": len(os.sched_getaffinity(0)),
            "ms_per_step": round(per_step * 1e3, 3)}


def cpu_baseline_encoder(case, seconds: float, step_bytes: int):
    import oracle
    H, C, N = case.w1.shape[0], case.C, case.N
    W1 = oracle.i8s_make(case.w1, case.w1_scale)
    W2 = oracle.i8s_make(case.w2, case.w2_scale)
    X = oracle.i8s_make(case.x, case.x_scale)
    calls, t0 = 0, time.perf_counter()
    while True:
        h = oracle.i8s_mul_mat_add(W1, H, C, X, N, case.b1, True)
        oracle.i8s_mul_mat_add(W2, C, H, h, N, case.b2, False)
        calls += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": round(step_bytes * calls / el / 1e9, 6), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{calls} full block MLPs ({case.name}, FC1+ReLU and FC2 with requantization, scalar C, "
                      f"1 thread) in {el:.1f} s",
            "cpu_model": cpu_model(), "host_cores": len(os.sched_getaffinity(0)),
            "ms_per_call": round(el / calls * 1e3, 3)}


def cpu_baseline_layer(case, seconds: float):
    import oracle
    shp_x = {"q": case.x_hidden, "k": case.x_hidden, "v": case.x_hidden, "o": case.x_attn, "gate": case.x_attn,
             "up": case.x_attn, "down": case.x_ffn}
    packed = {n: oracle.pack(case.w[n], case.ws) for n in LAYER_PROJ}
    wbytes = sum(case.w[n].size // 4 for n in LAYER_PROJ)
    calls, t0 = 0, time.perf_counter()
    while True:
        for n in LAYER_PROJ:
            rows, K = case.w[n].shape
            oracle.mul_mat_group([(packed[n], rows, case.bias.get(n))], K, shp_x[n])
        calls += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": round(wbytes * calls / el / 1e9, 6), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{calls} full layers (7 projections, N = 1, scalar C, 1 thread) in {el:.1f} s",
            "cpu_model": cpu_model(), "host_cores": len(os.sched_getaffinity(0)),
            "ms_per_call": round(el / calls * 1e3, 3)}


def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU; --gpus {args.gpus} is not supported "
              "(the kernel runs on one GPU's share; see the sharding note in the design document)",
              file=sys.stderr, flush=True)
        return 2
    if args.copy_kernel_mib:
        copy_kernel_only(args.copy_kernel_mib)
        return 0

    import numpy as np
    import torch

    from ternary_weight_integer_amd import i2s

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.workload == "decode_layer":
        print(json.dumps(bench_layer(args, torch, i2s)), flush=True)
        return 0
    if args.workload == "encoder_mlp":
        print(json.dumps(bench_encoder(args, torch)), flush=True)
        return 0
    if args.workload.startswith("w8a8_"):
        print(json.dumps(bench_w8a8(args, torch)), flush=True)
        return 0
    if args.workload == "layer_sweep":
        print(json.dumps(bench_sweep(args, torch, i2s)), flush=True)
        return 0
    out = bench_case(args, torch, i2s, make_case(args.workload))
    if args.workload == "decode_up" and not args.no_prefill and not args.eager:
        # The prefill GEMM beside the decode GEMV: the same metric's int8-MFMA
        # half, reported under its own key (the line's value stays the decode).
        pre = bench_case(args, torch, i2s, make_case("prefill_gate"))
        out["prefill_gemm"] = {k: pre[k] for k in ("value", "unit", "ms_per_step", "int8_tops", "config",
                                                   "roofline", "quantize", "cpu_baseline") if k in pre}
        out["prefill_gemm"]["value_is"] = "packed weight bytes per second of the whole step (quantize + GEMM)"
    print(json.dumps(out), flush=True)
    return 0


def quantize_line(torch, i2s, x, ws, N: int, K: int, in_step_us: float):
    """The activation quantize launch of a GEMM step on its own: a graph of
    back-to-back i2s_quantize_act_ws calls on the step's rows (which then
    stay cache-resident), against the HBM roofline of its algorithmic bytes
    (F32 rows read, int8 rows, scales and row sums written); in_step_us is
    the step time less the contraction's, i.e. what the launch costs after
    a contraction."""
    n = 256
    g = graph_of(lambda: [i2s.i2s_quantize_act_ws(x, ws) for _ in range(n)], torch)
    g.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / n
    del g
    qbytes = N * K * 4 + N * K + 8 * N
    achieved = qbytes / (us * 1e-6) / 1e9
    return {"kernel": "quantize_rowsum_reg_kernel", "kernel_us": round(us, 4), "in_step_us": round(in_step_us, 4),
            "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "alg_bytes_per_launch": qbytes}}


def graph_repeats(torch, step, steps: int, target_ms: float) -> int:
    """How many times the K timed steps are repeated inside the timed graph so
    that it runs for about target_ms: starting a graph costs a few
    microseconds of its own, which a short graph would add to every step."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g = graph_of(lambda: [step(i) for i in range(steps)], torch)
    g.replay()
    torch.cuda.synchronize()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    once = max(e0.elapsed_time(e1), 1e-3)
    del g
    return max(1, int(-(-target_ms // once)))


def bench_case(args, torch, i2s, case):
    """One I2_S matmul workload: the step (i2s_mul_mat: quantize + contraction
    + epilogue), the dominant kernel alone, its roofline line and the CPU
    oracle baseline."""
    dev = torch.device("cuda:0")
    rows, K, N = case.rows, case.K, case.N
    wbytes = rows * K // 4
    packed0 = i2s.i2s_pack(torch.from_numpy(case.w).to(dev), case.ws)
    R = args.copies or max(1, -(-ROTATE_BYTES // packed0.numel()))
    copies = [packed0] + [packed0.clone() for _ in range(R - 1)]
    x = torch.from_numpy(case.x).to(dev)
    ws = i2s.new_workspace(N, K, dev)
    y = torch.empty((N, rows), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step(i):
        i2s.i2s_mul_mat(copies[i % R], rows, K, x, workspace=ws, y=y)

    # The kernel that dominates a step, timed on its own: the fused quantize +
    # GEMV is the whole step; otherwise the contraction after the quantize.
    kernel_kind = i2s.i2s_mul_mat_kernel(rows, K, N)
    i2s.i2s_quantize_act_ws(x, ws)

    def contraction(i):
        if kernel_kind == i2s.KERNEL_FUSED:
            i2s.i2s_mul_mat_ex(copies[i % R], rows, K, x, workspace=ws, y=y, kernel=kernel_kind)
        else:
            i2s.i2s_mul_mat_ws(copies[i % R], rows, K, N, ws, y=y, kernel=kernel_kind)

    # Warm-up steps (eager), then a correctness check of the graph path.
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    y_eager = y.clone()

    K_steps = args.steps
    repeats = 1
    if args.eager:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        for i in range(K_steps):
            step(i)
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        step_ms = e0.elapsed_time(e1) / K_steps
        kern_us = None
    else:
        repeats = graph_repeats(torch, step, K_steps, args.min_region_ms)
        g_step = graph_of(lambda: [step(i) for i in range(K_steps * repeats)], torch)
        n_kern = max(R, 256)
        g_kern = graph_of(lambda: [contraction(i) for i in range(n_kern)], torch)
        g_step.replay()
        g_kern.replay()
        torch.cuda.synchronize()
        # y now holds the last contraction of copy (n_kern-1) % R; every copy is identical.
        if not torch.equal(y.view(torch.int32), y_eager.view(torch.int32)):
            raise RuntimeError("graph replay result differs from the eager result")
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev[0].record()
        g_step.replay()
        ev[1].record()
        g_kern.replay()
        ev[2].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        step_ms = ev[0].elapsed_time(ev[1]) / (K_steps * repeats)
        kern_us = ev[1].elapsed_time(ev[2]) * 1e3 / n_kern
        if not torch.equal(y.view(torch.int32), y_eager.view(torch.int32)):
            raise RuntimeError("graph replay result differs from the eager result")

    ops = 2 * rows * K * N
    value = wbytes / (step_ms * 1e-3) / 1e9
    alg_bytes = alg_bytes_of(kernel_kind, rows, K, N)
    variant = i2s.i2s_mul_mat_variant(rows, K, N)
    kernel_name = kernel_name_of(kernel_kind, variant)
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": case.name, "rows": rows, "K": K, "N": N, "weight_scale": case.ws,
                   "weight_copies_rotated": R, "rotated_bytes": R * packed0.numel(),
                   "timing": "eager" if args.eager else "hip_graph",
                   "step_repeats": repeats, "timed_steps": K_steps * repeats},
        "int8_tops": round(ops / (step_ms * 1e-3) / 1e12, 4),
        "wall_s": round(wall, 4),
    }
    if kern_us is not None:
        if kernel_kind != 2:
            achieved = alg_bytes / (kern_us * 1e-6) / 1e9
            out["roofline"] = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                               "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(case_workload(case)),
                               "kernel": kernel_name, "kernel_variant": variant, "kernel_us": round(kern_us, 4),
                               "alg_bytes_per_launch": alg_bytes}
        else:
            achieved = ops / (kern_us * 1e-6) / 1e12
            out["roofline"] = {"bound": "mfma", "achieved": round(achieved, 2), "peak": INT8_MFMA_PEAK_TOPS,
                               "unit": "TOP/s", "frac": round(achieved / INT8_MFMA_PEAK_TOPS, 4),
                               "traffic": measured_traffic(case_workload(case)), "kernel": kernel_name,
                               "kernel_variant": variant, "kernel_us": round(kern_us, 4), "alg_ops_per_launch": ops,
                               "alg_bytes_per_launch": alg_bytes}
    if kern_us is not None and kernel_kind != 2:
        out["roofline"]["copy_ceiling"] = copy_ceiling(torch, alg_bytes)
    if kern_us is not None and kernel_kind == 2:
        out["quantize"] = quantize_line(torch, i2s, x, ws, N, K, step_ms * 1e3 - kern_us)
    props = torch.cuda.get_device_properties(0)
    out["gpu"] = {"name": props.name, "cus": props.multi_processor_count,
                  "arch": getattr(props, "gcnArchName", "")}
    del copies, packed0, ws, y, x
    torch.cuda.empty_cache()
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
        out["cpu_baseline"]["gpu_over_cpu"] = round(out["value"] / out["cpu_baseline"]["value"], 1)
    return out


if __name__ == "__main__":
    sys.exit(main())
