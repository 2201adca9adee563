"""Benchmark of the MACaQ online W4A4 linear layer on one MI355X.

Default workload (the headline): the prefill 8B-shaped layer set, M = 2048
tokens through (K, N) = (4096, 4096), (4096, 14336), (14336, 4096), Hadamard
block 32. One step = macaq_linear on each of the three layers (activation
scale + block-Hadamard + MXFP4 quantize + scaled-FP4 GEMM), bf16 in and out.
Weights are prepared beforehand (offline). Inputs are resident in HBM; the
timed steps rotate through several copies of activations and weights so that
no step finds its operands in the 256 MB last-level cache.

Steps are captured into HIP graphs (one per operand copy) and replayed, so
the timed region has no host launch gaps. Prints one JSON line with the
metric, the plain-MXFP4 overhead, the GEMM kernel's roofline (HIP events on
the launch stream around graph replays of that kernel alone, per layer) and
the CPU oracle's throughput on a bounded sample of the same work.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "W4A4 fused linear TFLOPS (% MXFP4 peak); transform overhead vs plain MXFP4"
PEAK_FP4_TFLOPS = 10100.0   # MI355X dense MXFP4 matrix-core peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
ROTATE = 4                  # operand copies cycled through by the timed steps
ORACLE_THREADS_CAP = 16     # the GPU machine's CPU share for one GPU


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="prefill-8b",
                   choices=["prefill-8b", "decode-32b", "moe-128e", "prefill-large", "tiny"])
    p.add_argument("--block", type=int, default=None, help="Hadamard block (default: the workload's first)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    p.add_argument("--profile-steps", type=int, default=0,
                   help="if > 0: only run this many steps of the fused path (for rocprofv3) and exit")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="if > 0: only copy a MIB-MiB device buffer 3 times (the known-size reference for the "
                        "rocprofv3 FETCH_SIZE / WRITE_SIZE counters) and exit")
    return p.parse_args()


class Timer:
    """HIP events on the current (launch) stream."""

    def __init__(self, torch):
        self.torch = torch

    def __enter__(self):
        self.s = self.torch.cuda.Event(enable_timing=True)
        self.e = self.torch.cuda.Event(enable_timing=True)
        self.s.record(self.torch.cuda.current_stream())
        return self

    def __exit__(self, *a):
        self.e.record(self.torch.cuda.current_stream())

    def ms(self):
        return self.s.elapsed_time(self.e)


def source_digest(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def build_layers(torch, binding, inputs, cfg, shapes, M, b, dev):
    """Per (K, N): rotating copies of x and of the prepared weights (fused and plain)."""
    layers = []
    for si, (K, N) in enumerate(shapes):
        case = inputs.linear_case(cfg, si, M=M, b=b)
        x = case.x.to(dev)
        w = case.w.to(dev)
        s = binding.calibrate(case.xcal.to(dev))
        a, r = binding.make_multipliers(s, b)
        w_fused = binding.prepare_weights(w, r, b)
        w_plain = binding.prepare_weights(w, None, 0)
        del w

        def clone(p):
            return binding.Packed(p.codes.clone(), p.scales.clone(), p.rows, p.K)

        copies = [dict(x=x.clone(), w=clone(w_fused), wp=clone(w_plain)) for _ in range(ROTATE)]
        del x, w_fused, w_plain
        ws_bytes = binding.linear_workspace_size(M, K, N)
        qa = binding.Packed(torch.empty(binding.packed_codes_bytes(M, K), dtype=torch.uint8, device=dev),
                            torch.empty(binding.packed_scales_bytes(M, K), dtype=torch.uint8, device=dev), M, K)
        layers.append(dict(K=K, N=N, M=M, a=a, b=b, case=case, copies=copies,
                           y=torch.empty(M, N, dtype=torch.bfloat16, device=dev),
                           work=torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev),
                           gwork=torch.empty(max(binding.gemm_workspace_size(M, K, N), 1), dtype=torch.uint8,
                                             device=dev),
                           qa=qa))
    return layers


def enqueue_step(binding, layers, copy, plain=False):
    for L in layers:
        c = L["copies"][copy]
        if plain:
            binding.linear(c["x"], None, 0, c["wp"], out=L["y"], workspace=L["work"])
        else:
            binding.linear(c["x"], L["a"], L["b"], c["w"], out=L["y"], workspace=L["work"])


def capture(torch, fn):
    """A HIP graph of the kernels that fn enqueues on the current stream."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # eager once on the capture stream (argument checks, warm caches)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn()
    torch.cuda.synchronize()
    return g


def timed_graphs(torch, graphs, steps, warmup):
    """Replay graphs[i % len] for warmup untimed and `steps` timed steps."""
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with Timer(torch) as t:
        for i in range(steps):
            graphs[(warmup + i) % len(graphs)].replay()
    torch.cuda.synchronize()
    return t.ms() / steps, time.perf_counter() - t0


def kernel_breakdown(torch, binding, layers, reps):
    """Per layer: the two kernels of macaq_linear (quantize, GEMM) each alone,
    `reps` launches captured in one graph, timed with HIP events on the launch
    stream around the replay; returns average ms per launch."""
    q_ms, g_ms = [], []
    for L in layers:
        def quant():
            for i in range(reps):
                c = L["copies"][i % ROTATE]
                binding.quant_act(c["x"], L["a"], L["b"], layout="gemm", codes=L["qa"].codes, scales=L["qa"].scales)

        def gemm():
            for i in range(reps):
                c = L["copies"][i % ROTATE]
                binding.linear_plain_gemm(L["qa"], c["w"], out=L["y"], workspace=L["gwork"])

        for fn, acc in ((quant, q_ms), (gemm, g_ms)):
            g = capture(torch, fn)
            g.replay()
            torch.cuda.synchronize()
            with Timer(torch) as t:
                g.replay()
            torch.cuda.synchronize()
            acc.append(t.ms() / reps)
    return q_ms, g_ms


def cpu_baseline(layers, target_s):
    """The oracle (C, fp64 GEMM over codes, as it stands) on a bounded row sample."""
    import numpy as np

    import oracle
    from mxfp4_w4a4_post_amd import inputs as inp

    threads = min(oracle.default_threads(), ORACLE_THREADS_CAP)
    prepared = []
    for L in layers:
        case = L["case"]
        s = oracle.calibrate(inp.bf16_bits(case.xcal))
        a, r = oracle.multipliers(s, case.b)
        wc, ws = oracle.prepare_weights(inp.bf16_bits(case.w), r, case.b)
        prepared.append((inp.bf16_bits(case.x), a, case.b, wc, ws, L["K"], L["N"]))
    rows = 4
    while True:
        t0 = time.perf_counter()
        flops = 0
        for xb, a, b, wc, ws, K, N in prepared:
            oracle.linear(np.ascontiguousarray(xb[:rows]), a, b, wc, ws, threads=threads)
            flops += 2 * rows * K * N
        dt = time.perf_counter() - t0
        if dt >= target_s * 0.5 or rows >= layers[0]["M"]:
            break
        rows = min(layers[0]["M"], max(rows * 2, int(rows * target_s / max(dt, 1e-3))))
    return dict(value=round(flops / dt / 1e12, 6), unit="TFLOP/s", cores=threads, kind="oracle",
                sample="%d of %d token rows through all %d layers (quantize + fp64 GEMM over codes), %.1f s"
                       % (rows, layers[0]["M"], len(layers), dt))


def copy_mb(layers):
    total = 0
    for L in layers:
        c = L["copies"][0]
        total += c["x"].numel() * 2 + c["w"].codes.numel() + c["w"].scales.numel()
    return total / 1e6


def load_traffic(kernel_digest):
    """HBM bytes (FETCH_SIZE + WRITE_SIZE, each scaled by a plain copy of known
    size) per GEMM launch, the mean over the step's layers, from the committed
    rocprofv3 counter summary; None unless it was taken on the current kernel
    source."""
    path = os.path.join(ROOT, "profiles", "gemm_prefill_8b_pmc.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_digest") != kernel_digest:
        return None
    return d.get("hbm_bytes_per_launch_mean")


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (see DESIGN.md for how the layer "
              "would shard); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    from mxfp4_w4a4_post_amd import binding, inputs

    binding.load_library()
    dev = torch.device("cuda:0")
    if args.calibrate_copy > 0:
        n = args.calibrate_copy << 20
        src = torch.ones(n // 4, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copied_bytes": n, "copies": 3}), flush=True)
        return
    wl = {"tiny": 1, "prefill-8b": 2, "decode-32b": 3, "moe-128e": 4, "prefill-large": 5}[args.workload]
    if wl in (3, 4):
        print("workload %s: not wired into bench.py yet" % args.workload, file=sys.stderr)
        sys.exit(2)
    spec = inputs.CONFIGS[wl]
    b = args.block if args.block is not None else spec["blocks"][0]
    M = spec["M"]
    shapes = spec["shapes"]
    layers = build_layers(torch, binding, inputs, wl, shapes, M, b, dev)
    torch.cuda.synchronize()

    if args.profile_steps > 0:
        for i in range(args.profile_steps):
            enqueue_step(binding, layers, i % ROTATE)
        torch.cuda.synchronize()
        print(json.dumps({"profiled_steps": args.profile_steps, "workload": spec["name"]}), flush=True)
        return

    flops = sum(2 * M * K * N for K, N in shapes)
    fused = [capture(torch, lambda c=c: enqueue_step(binding, layers, c)) for c in range(ROTATE)]
    plain = [capture(torch, lambda c=c: enqueue_step(binding, layers, c, plain=True)) for c in range(ROTATE)]
    ms, wall = timed_graphs(torch, fused, args.steps, args.warmup)
    ms_plain, _ = timed_graphs(torch, plain, args.steps, args.warmup)
    q_ms, g_ms = kernel_breakdown(torch, binding, layers, 20)
    tflops = flops / (ms * 1e-3) / 1e12
    gemm_ms = sum(g_ms)
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12
    digest = source_digest([os.path.join(ROOT, "mxfp4_w4a4_post_amd", "csrc", "gemm.hip")])
    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4 (MXFP4 E2M1/E8M0 operands, fp32 accumulate, fp32 transform, bf16 in/out)",
        "data": "synthetic (seeded Student-t(3) activations with 1% outlier channels x30, N(0,0.02^2) weights)",
        "config": {"workload": "%s: M=%d tokens, (K,N) in %s, Hadamard block %d, bf16 in/out"
                               % (spec["name"], M, shapes, b),
                   "tokens": M, "layers": [list(s) for s in shapes], "hadamard_block": b},
        "pct_mxfp4_peak": round(100 * tflops / PEAK_FP4_TFLOPS, 2),
        "tokens_per_s": round(M / (ms * 1e-3), 1),
        "plain_mxfp4_ms_per_step": round(ms_plain, 5),
        "transform_overhead_pct": round(100 * (ms / ms_plain - 1), 2),
        "wall_s_timed": round(wall, 4),
        "timing": "HIP graphs of one step per operand copy (%d copies, %.0f MB each, cycled past the 256 MB "
                  "last-level cache), HIP events on the launch stream" % (ROTATE, copy_mb(layers)),
        "kernels_ms": {"quant": [round(v, 5) for v in q_ms], "gemm": [round(v, 5) for v in g_ms]},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 2), "peak": PEAK_FP4_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / PEAK_FP4_TFLOPS, 4),
                     "traffic": load_traffic(digest), "kernel": "gemm_kernel (scaled-FP4 MFMA)",
                     "kernel_source_digest": digest},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(layers, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
