"""Benchmark of the MACaQ online W4A4 linear layer on one MI355X.

Default workload (the headline): the large prefill layer pair, M = 8192
tokens through (K, N) = (8192, 28672) and (28672, 8192), Hadamard block 32
(blocks 64 and 128 reported alongside as a sweep). One step = macaq_linear
on each layer (activation scale + block-Hadamard + MXFP4 quantize +
scaled-FP4 GEMM), bf16 in and out. Weights are prepared beforehand
(offline). Other workloads (--workload): prefill-8b (M = 2048 through
4096x4096, 4096x14336, 14336x4096), decode-32b (M = 1, 8, 32, 64 through
5120x25600 and 25600x5120), moe-128e
(grouped gate/up and down projections of 4096 tokens routed top-8 over 128
experts), moe-block (the same 4096 tokens through the whole MoE block:
routing, gathered gate/up with the SwiGLU epilogue that quantizes the down
input, down, weighted top-8 combine), prefill-large (M = 8192 through
8192x28672 and 28672x8192, Hadamard block from --block; the default),
refine-8b (offline
Flip-Refinement of the prefill layers' weights: Hessian of 512 transformed
calibration rows, up to 64 greedy code moves per weight row), quant-error
(relative output error of the layer against the exact bf16 product for the
calibration variants s = max^(q/4) and Hadamard blocks b in {0, 32, 64, 128}
on three activation recipes), prepare-stream (weights of 8 blocks of 8B-shaped
linears prepared from pinned host memory back to pinned host memory with one
layer resident, copies overlapped with preparation), tiny, and peaks (the
chip's measured ceilings: scaled-FP4 MFMA rate with constant and random
operands, plain-read and copy bandwidth).

Inputs are resident in HBM; the timed steps rotate through several copies of
activations and weights so that no step finds its operands in the 256 MB
last-level cache. Steps are captured into HIP graphs (one per operand copy)
and replayed, so the timed region has no host launch gaps. Prints one JSON
line with the metric, the overhead of the fused transform over plain MXFP4
(same kernels with no scale and no Hadamard), the dominant kernel's roofline
(HIP events on the launch stream around graph replays of that kernel alone)
and the CPU oracle's throughput on a bounded sample of the same work.
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
ORACLE_THREADS_CAP = 16     # one GPU's share of the host CPU
WORKLOADS = {"tiny": 1, "prefill-8b": 2, "decode-32b": 3, "moe-128e": 4, "prefill-large": 5, "moe-block": 6,
             "refine-8b": 7, "quant-error": 8, "prepare-stream": 9, "peaks": 10}
PEAKS = 10  # the chip's measured ceilings: scaled-FP4 MFMA rate and plain-read / copy bandwidth
MFMA_FLOPS = 2 * 32 * 32 * 64  # one scaled-FP4 MFMA 32x32x64
PREPARE_STREAM = 9  # offline: a stack of 8B-shaped blocks prepared from pinned host memory, one layer resident
STREAM_BLOCKS = 8
BLOCK_SHAPES = [(4096, 4096), (1024, 4096), (1024, 4096), (4096, 4096), (14336, 4096), (14336, 4096), (4096, 14336)]
QUANT_ERROR = 8  # study: layer output error against the calibration variant and the Hadamard block
REFINE = 7  # offline Flip-Refinement of the prefill 8B-shaped layers' weights
REFINE_ROWS = 512  # calibration rows of the Hessian
REFINE_CAP = 64    # moves per weight row
PEAK_FP64_TFLOPS = 78.6
MOE_BLOCK = 6  # the MoE workload as a whole block: routing, gathered gate/up + SwiGLU, down, combine


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="prefill-large", choices=sorted(WORKLOADS))
    p.add_argument("--block", type=int, default=None, help="Hadamard block (default: the workload's first)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    p.add_argument("--profile-steps", type=int, default=0,
                   help="if > 0: only run this many eager steps of the fused path (for rocprofv3) and exit")
    p.add_argument("--gemm-only", default=None, metavar="MxNxK",
                   help="only run the GEMM (macaq_gemm) on random MXFP4 operands of this shape --profile-steps "
                        "times (for counter collection) and exit")
    p.add_argument("--results", default=None, metavar="FILE",
                   help="also append the JSON line to FILE (one line per run)")
    p.add_argument("--no-block-sweep", action="store_true",
                   help="prefill-large: skip the Hadamard blocks 64 and 128 reported beside the headline block")
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


def emit(args, out):
    """Print the result line, and append it to --results when given."""
    line = json.dumps(out)
    print(line, flush=True)
    if args.results:
        with open(args.results, "a") as f:
            f.write(line + "\n")


def source_digest(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def packed_clone(binding, p):
    return binding.Packed(p.codes.clone(), p.scales.clone(), p.rows, p.K)


class Entry:
    """One layer call of a step: the fused and plain calls on operand copy c,
    and (dense layers) the quantize and GEMM kernels alone."""

    def __init__(self, name, flops, nbytes, gemm_bytes):
        self.name, self.flops, self.bytes, self.gemm_bytes = name, flops, nbytes, gemm_bytes
        self.fused = self.plain = None
        self.quant = self.gemm = self.quant_plain = self.gemm_plain = None
        self.oracle_case = None  # (inputs case, rows) for the CPU baseline


def dense_entries(torch, binding, inputs, wl, b, dev):
    spec = inputs.WORKLOAD_SPECS[wl]
    Ms = [spec["M"]] if "M" in spec else list(spec["Ms"])
    entries = []
    for si, (K, N) in enumerate(spec["shapes"]):
        case = inputs.linear_case(wl, si, M=max(Ms), b=b)
        w = case.w.to(dev)
        s = binding.calibrate(case.xcal.to(dev))
        a, r = binding.make_multipliers(s, b)
        wf = [binding.prepare_weights(w, r, b)]
        wp = [binding.prepare_weights(w, None, 0)]
        del w
        wf += [packed_clone(binding, wf[0]) for _ in range(ROTATE - 1)]
        wp += [packed_clone(binding, wp[0]) for _ in range(ROTATE - 1)]
        xs_full = case.x.to(dev)
        for M in Ms:
            xs = [xs_full[:M].clone() for _ in range(ROTATE)]
            wbytes = N * K * 17 / 32
            e = Entry("M=%d K=%d N=%d" % (M, K, N), 2.0 * M * N * K, 2 * M * K + wbytes + 2 * M * N,
                      M * K * 17 / 32 + wbytes + 2 * M * N)
            y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
            y32 = torch.empty(M, N, dtype=torch.float32, device=dev)
            work = torch.empty(max(binding.linear_workspace_size(M, K, N), 1), dtype=torch.uint8, device=dev)
            gwork = torch.empty(max(binding.gemm_workspace_size(M, K, N), 1), dtype=torch.uint8, device=dev)
            qa = binding.Packed(torch.empty(binding.packed_codes_bytes(M, K), dtype=torch.uint8, device=dev),
                                torch.empty(binding.packed_scales_bytes(M, K), dtype=torch.uint8, device=dev), M, K)
            qp = binding.Packed(torch.empty_like(qa.codes), torch.empty_like(qa.scales), M, K)
            binding.quant_act(xs[0], a, b, layout="gemm", codes=qa.codes, scales=qa.scales)
            binding.quant_act(xs[0], None, 0, layout="gemm", codes=qp.codes, scales=qp.scales)
            e.fused = lambda c, xs=xs, a=a, wf=wf, y=y, work=work: binding.linear(xs[c], a, b, wf[c], out=y,
                                                                                   workspace=work)
            e.plain = lambda c, xs=xs, wp=wp, y=y, work=work: binding.linear(xs[c], None, 0, wp[c], out=y,
                                                                              workspace=work)
            e.fused_f32 = lambda c, xs=xs, a=a, wf=wf, y32=y32, work=work: binding.linear(xs[c], a, b, wf[c], out=y32,
                                                                                       workspace=work)
            e.quant = lambda c, xs=xs, a=a, qa=qa: binding.quant_act(xs[c], a, b, layout="gemm", codes=qa.codes,
                                                                     scales=qa.scales)
            e.quant_plain = lambda c, xs=xs, qp=qp: binding.quant_act(xs[c], None, 0, layout="gemm",
                                                                      codes=qp.codes, scales=qp.scales)
            e.gemm = lambda c, qa=qa, wf=wf, y=y, gwork=gwork: binding.linear_plain_gemm(qa, wf[c], out=y,
                                                                                        workspace=gwork)
            e.gemm_plain = lambda c, qp=qp, wp=wp, y=y, gwork=gwork: binding.linear_plain_gemm(qp, wp[c], out=y,
                                                                                              workspace=gwork)
            e.oracle_case = (case, M)
            entries.append(e)
        del xs_full
    return entries, Ms


def moe_entries(torch, binding, inputs, b, dev):
    entries = []
    for proj in ("gate_up", "down"):
        case = inputs.moe_case(proj)
        E, K, N, T = case.E, case.K, case.N, case.T
        offsets = torch.from_numpy(case.offsets.astype("int32")).to(dev)
        a = torch.empty(E, K, dtype=torch.float32, device=dev)
        wf = binding.empty_grouped_weights(E, N, K, dev)
        wp = binding.empty_grouped_weights(E, N, K, dev)
        for ex in range(E):
            s = binding.calibrate(case.xcal[ex].to(dev))
            ae, re_ = binding.make_multipliers(s, b)
            a[ex].copy_(ae)
            w = case.w[ex].to(dev)
            binding.prepare_weights(w, re_, b, out=binding.expert(wf, ex))
            binding.prepare_weights(w, None, 0, out=binding.expert(wp, ex))
        wfs = [wf] + [packed_clone(binding, wf) for _ in range(ROTATE - 1)]
        wps = [wp] + [packed_clone(binding, wp) for _ in range(ROTATE - 1)]
        xs = [case.x.to(dev) for _ in range(ROTATE)]
        y = torch.empty(T, N, dtype=torch.bfloat16, device=dev)
        work = torch.empty(max(binding.linear_grouped_workspace_size(T, E, K, N), 1), dtype=torch.uint8,
                           device=dev)
        wbytes = E * N * K * 17 / 32
        e = Entry("%s T=%d E=%d K=%d N=%d" % (proj, T, E, K, N), 2.0 * T * N * K, 2 * T * K + wbytes + 2 * T * N,
                  T * K * 17 / 32 + wbytes + 2 * T * N)
        e.fused = lambda c, xs=xs, a=a, wfs=wfs, y=y, work=work, off=offsets: binding.linear_grouped(
            xs[c], off, a, b, wfs[c], out=y, workspace=work)
        e.plain = lambda c, xs=xs, wps=wps, y=y, work=work, off=offsets: binding.linear_grouped(
            xs[c], off, None, 0, wps[c], out=y, workspace=work)
        e.oracle_case = (case, None)
        entries.append(e)
        del case
    return entries


def moe_block_entries(torch, binding, inputs, b, dev):
    """One entry: the MoE block on the MoE workload's tokens, with the fused
    (MACaQ) and plain MXFP4 prepared experts; the parts of the block alone for
    the per-kernel split."""
    case = inputs.moe_block_case(b=b)
    T, E, k, H, F = case.T, case.E, case.k, case.H, case.F
    wg, wu, wd = case.w_gate.to(dev), case.w_up.to(dev), case.w_dn.to(dev)
    lf = binding.prepare_moe(wg, wu, wd, case.xcal_gu.to(dev), case.xcal_dn.to(dev), b)
    lp = binding.prepare_moe(wg, wu, wd, None, None, 0)
    del wg, wu, wd

    def copies(lay):
        out = [lay]
        for _ in range(ROTATE - 1):
            out.append(binding.MoELayer(lay.a_gu, packed_clone(binding, lay.wgu), lay.a_dn,
                                        packed_clone(binding, lay.wdn), lay.b))
        return out

    lfs, lps = copies(lf), copies(lp)
    xs = [case.x.to(dev) for _ in range(ROTATE)]
    ids = torch.from_numpy(case.ids).to(dev)
    w = torch.from_numpy(case.w).to(dev)
    y = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    work = torch.empty(binding.moe_workspace_size(T, k, E, H, F), dtype=torch.uint8, device=dev)
    R = T * k
    wbytes = E * (2 * F * H + H * F) * 17 / 32
    flops = 2.0 * R * (2 * F) * H + 2.0 * R * H * F
    e = Entry("moe block T=%d k=%d E=%d H=%d F=%d" % (T, k, E, H, F), flops, 2 * T * H + wbytes + 2 * T * H, None)
    e.fused = lambda c: lfs[c](xs[c], ids, w, out=y, workspace=work)
    e.plain = lambda c: lps[c](xs[c], ids, w, out=y, workspace=work)
    off, tok, pos = binding.moe_route(ids, E)
    dn = binding.moe_gate_up(xs[0], k, tok, off, lf.a_gu, b, lf.wgu, lf.a_dn, workspace=work)
    e.route = lambda c: binding.moe_route(ids, E)
    e.gate_up = lambda c: binding.moe_gate_up(xs[c], k, tok, off, lfs[c].a_gu, b, lfs[c].wgu, lfs[c].a_dn, out=dn,
                                              workspace=work)
    e.down_combine = lambda c: binding.moe_down_combine(dn, off, pos, w, lfs[c].wdn, out=y, workspace=work)
    # the same parts of the plain MXFP4 block (no multipliers, no Hadamard)
    dnp = binding.moe_gate_up(xs[0], k, tok, off, lp.a_gu, 0, lp.wgu, lp.a_dn, workspace=work)
    e.gate_up_plain = lambda c: binding.moe_gate_up(xs[c], k, tok, off, lps[c].a_gu, 0, lps[c].wgu, lps[c].a_dn,
                                                    out=dnp, workspace=work)
    e.down_combine_plain = lambda c: binding.moe_down_combine(dnp, off, pos, w, lps[c].wdn, out=y, workspace=work)
    e.parts_bytes = {"gate_up": 2 * R * H + E * 2 * F * H * 17 / 32 + R * F * 17 / 32,
                     "down_combine": R * F * 17 / 32 + E * H * F * 17 / 32 + 2 * R * H * 2 + 2 * T * H}
    e.oracle_case = (case, None)
    return [e]


def refine_main(args, torch, binding, inputs, dev):
    """Offline Flip-Refinement of the prefill 8B-shaped layers: per step and
    layer, the Hessian of the calibration rows and the refinement of freshly
    prepared (round-to-nearest) codes. Timed with HIP events, eagerly."""
    import numpy as np
    spec = inputs.WORKLOAD_SPECS[2]
    b = args.block if args.block is not None else spec["blocks"][0]
    layers = []
    for si, (K, N) in enumerate(spec["shapes"]):
        case = inputs.linear_case(2, si, M=16, b=b)
        w = case.w.to(dev)
        a, r = binding.make_multipliers(binding.calibrate(case.xcal.to(dev)), b)
        xcal = inputs.activations(2, si, REFINE_ROWS, K, stream=1).to(dev)
        rtn = binding.prepare_weights(w, r, b)
        work = torch.empty(binding.load_library().macaq_flip_refine_workspace_size(N, K), dtype=torch.uint8,
                           device=dev)
        layers.append(dict(K=K, N=N, w=w, a=a, r=r, xcal=xcal, rtn=rtn, work=work,
                           packed=packed_clone(binding, rtn)))
    flops_h = sum(2.0 * REFINE_ROWS * L["K"] ** 2 for L in layers)
    flops_g = sum(2.0 * L["N"] * L["K"] ** 2 for L in layers)

    def step(parts=("hessian", "refine")):
        out = []
        for L in layers:
            L["packed"].codes.copy_(L["rtn"].codes)
            if "hessian" in parts:
                L["H"] = binding.hessian(L["xcal"], L["a"], b)
            if "refine" in parts:
                out.append(binding.flip_refine(L["w"], L["r"], b, L["H"], REFINE_CAP, L["packed"],
                                               workspace=L["work"]))
            if "gradient" in parts:
                # a refinement call that makes no move: transform, the gradient
                # kernel, the diagonal, and a move launch that stops at once
                out.append(binding.flip_refine(L["w"], L["r"], b, L["H"], 0, L["packed"], workspace=L["work"]))
        return out

    flips = step()
    for _ in range(max(args.warmup, 1) - 1):
        step()
    torch.cuda.synchronize()

    def timed(parts):
        with Timer(torch) as t:
            for _ in range(args.steps):
                step(parts)
        torch.cuda.synchronize()
        return t.ms() / args.steps

    steps = args.steps = max(1, min(args.steps, 10))
    ms = timed(("hessian", "refine"))
    ms_h = timed(("hessian",))
    ms_g = max(timed(("hessian", "gradient")) - ms_h, 1e-6)
    ms_r = max(ms - ms_h, 1e-6)
    fl = torch.cat(flips).float().cpu().numpy()
    value = (flops_h + flops_g) / (ms * 1e-3) / 1e12
    call_tf = flops_g / (ms_r * 1e-3) / 1e12
    g_tf = flops_g / (ms_g * 1e-3) / 1e12
    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f64 (Hessian, gradient and move decisions), MXFP4 codes",
        "data": "synthetic (seeded prefill 8B-shaped weights and calibration rows; recipe in inputs.py)",
        "config": {"workload": "refine-8b: Flip-Refinement of the prefill 8B-shaped layers (K, N) in %s, Hessian of "
                               "%d calibration rows, up to %d moves per row, Hadamard block %d"
                               % (spec["shapes"], REFINE_ROWS, REFINE_CAP, b),
                   "layers": [list(x) for x in spec["shapes"]], "calibration_rows": REFINE_ROWS,
                   "max_flips": REFINE_CAP, "hadamard_block": b},
        "hessian_ms_per_step": round(ms_h, 4), "refine_ms_per_step": round(ms_r, 4),
        "gradient_ms_per_step": round(ms_g, 4), "refine_call_tflops": round(call_tf, 3),
        "weight_rows_per_s": round(sum(L["N"] for L in layers) / (ms * 1e-3), 1),
        "moves_per_row_mean": round(float(fl.mean()), 2), "rows_at_cap_pct": round(100.0 * float((fl >= REFINE_CAP).mean()), 2),
        "roofline": {"bound": "mfma", "achieved": round(g_tf, 3), "peak": PEAK_FP64_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(g_tf / PEAK_FP64_TFLOPS, 4), "traffic": None,
                     "kernel": "gram_kernel: the gradient G = E H (2 N K^2 fp64 flops per layer) on the fp64 matrix "
                               "cores, timed as refinement calls with max_flips = 0 (transform, gradient, diagonal, "
                               "a move launch that stops at once)",
                     "avg_launch_us": round(1e3 * ms_g / len(layers), 2)},
        "timing": "HIP events on the launch stream around %d eager steps; each step restores the round-to-nearest "
                  "codes (a device copy) before refining" % steps,
    }
    if not args.no_cpu_baseline:
        import oracle
        L = layers[0]
        K = L["K"]
        threads = min(oracle.default_threads(), ORACLE_THREADS_CAP)
        case = inputs.linear_case(2, 0, M=16, b=b)
        a_o, r_o = oracle.multipliers(oracle.calibrate(inputs.bf16_bits(case.xcal)), b)
        t0 = time.perf_counter()
        hrows = 128
        H = oracle.hessian(inputs.bf16_bits(inputs.activations(2, 0, hrows, K, stream=1)), a_o, b)
        th = time.perf_counter() - t0
        wb = inputs.bf16_bits(case.w)
        codes, scales = oracle.prepare_weights(wb, r_o, b)
        rows = 4
        t0 = time.perf_counter()
        oracle.flip_refine(wb[:rows], r_o, b, H, REFINE_CAP, codes[:rows], scales[:rows])
        tr = time.perf_counter() - t0
        fl_cpu = 2.0 * hrows * K * K + 2.0 * rows * K * K
        out["cpu_baseline"] = dict(value=round(fl_cpu / (th + tr) / 1e12, 6), unit="TFLOP/s", cores=1,
                                   kind="oracle",
                                   sample="Hessian of %d rows at K=%d (%.1f s) and the refinement of %d weight rows "
                                          "(%.1f s), single-threaded C" % (hrows, K, th, rows, tr))
    emit(args, out)


def quant_error_main(args, torch, binding, inputs, dev):
    """Relative L2 error of the W4A4 layer's fp32 output against the exact
    product of the same bf16 activations and weights (fp64 on the host), for
    every calibration variant q (s = max^(q/4)) and Hadamard block b."""
    import numpy as np
    cases = [("normal, 4 channels x50 (K=N=256, M=256)", inputs.linear_case(1, 0, M=256)),
             ("student-t(3), 1% channels x30 (prefill 4096 x 4096, M=512)", inputs.linear_case(2, 0, M=512)),
             ("student-t(3), 0.5% channels x100 (8192 -> first 2048 of 28672 rows, M=256)",
              inputs.linear_case(5, 0, M=256, N=2048))]
    table = {}
    t0 = time.perf_counter()
    for name, c in cases:
        x64 = (inputs.bf16_bits(c.x).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        w64 = (inputs.bf16_bits(c.w).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        exact = x64 @ w64.T
        x, w, xcal = c.x.to(dev), c.w.to(dev), c.xcal.to(dev)
        row = {}
        for q in (0, 1, 2, 4):
            s = binding.calibrate(xcal, q)
            for b in (0, 32, 64, 128):
                a, r = binding.make_multipliers(s, b)
                y = binding.linear(x, a, b, binding.prepare_weights(w, r, b), out_dtype=torch.float32)
                err = float(np.linalg.norm(y.double().cpu().numpy() - exact) / np.linalg.norm(exact))
                row["q=%d/4 b=%d" % (q, b)] = round(err, 5)
        table[name] = row
    wall = time.perf_counter() - t0
    default = table[cases[1][0]]["q=2/4 b=32"]
    best = {n: min(r, key=r.get) for n, r in table.items()}
    out = {
        "metric": METRIC, "value": default, "unit": "rel-L2 output error (prefill recipe, q=2/4, b=32)",
        "n_gpus": 1, "steps": 1, "warmup": 0, "ms_per_step": round(wall * 1e3, 1), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp4 (MXFP4 E2M1/E8M0 operands, fp32 accumulate), fp32 out",
        "data": "synthetic (seeded activations with outlier channels, N(0,sigma^2) weights; recipe in inputs.py)",
        "config": {"workload": "quant-error: calibration variants s = max|x|^(q/4), q in {0,1,2,4}, x Hadamard "
                               "blocks b in {0,32,64,128} on three activation recipes",
                   "calibration_rows": inputs.CALIB_ROWS},
        "error_table": table, "best_setting": best,
        "timing": "one pass over the grid (GPU layers plus the host's exact fp64 products)",
    }
    if not args.no_cpu_baseline:
        import oracle
        c = cases[1][1]
        threads = min(oracle.default_threads(), ORACLE_THREADS_CAP)
        a_o, r_o = oracle.multipliers(oracle.calibrate(inputs.bf16_bits(c.xcal)), c.b)
        wc, ws = oracle.prepare_weights(inputs.bf16_bits(c.w), r_o, c.b)
        rows = 64
        t1 = time.perf_counter()
        oracle.linear(np.ascontiguousarray(inputs.bf16_bits(c.x)[:rows]), a_o, c.b, wc, ws, threads=threads)
        dt = time.perf_counter() - t1
        out["cpu_baseline"] = dict(value=round(2.0 * rows * c.K * c.N / dt / 1e12, 6), unit="TFLOP/s",
                                   cores=threads, kind="oracle",
                                   sample="%d rows of the prefill recipe's layer (quantize + fp64 GEMM over codes), "
                                          "%.1f s" % (rows, dt))
    emit(args, out)


def prepare_stream_main(args, torch, binding, inputs, dev):
    """Streaming preparation of a synthetic stack: (N, K) per linear of an
    8B-shaped block (q, k, v, o, gate, up, down), STREAM_BLOCKS blocks, bf16
    weights and 64 calibration rows per layer in pinned host memory (drawn on
    the device from a seeded generator, then copied out)."""
    from mxfp4_w4a4_post_amd import streaming
    b = args.block if args.block is not None else 32
    gen = torch.Generator(device=dev)
    gen.manual_seed(9)
    layers = []
    for blk in range(STREAM_BLOCKS):
        for (N, K) in BLOCK_SHAPES:
            w = (torch.randn(N, K, generator=gen, device=dev) * 0.02).to(torch.bfloat16)
            x = torch.randn(inputs.CALIB_ROWS, K, generator=gen, device=dev).to(torch.bfloat16)
            layers.append(streaming.HostLayer(w.cpu().pin_memory(), x.cpu().pin_memory()))
    del w, x
    torch.cuda.synchronize()
    max_n = max(L.w.shape[0] for L in layers)
    max_k = max(L.w.shape[1] for L in layers)
    wbytes = sum(2 * L.w.numel() for L in layers)
    pbytes = sum(L.w.numel() * 17 / 32 for L in layers)
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats(dev)
    base = torch.cuda.memory_allocated(dev)
    prep = streaming.StreamingPreparer(dev, max_n, max_k, inputs.CALIB_ROWS)
    prep.run(layers[:2], b)  # warm
    t0 = time.perf_counter()
    out = prep.run(layers, b)
    t_stream = time.perf_counter() - t0
    peak = torch.cuda.max_memory_allocated(dev) - base
    # the same work without overlap: each copy and preparation waits for the one before
    t0 = time.perf_counter()
    for L in layers:
        w = L.w.to(dev)
        x = L.xcal.to(dev)
        a, r = binding.make_multipliers(binding.calibrate(x), b)
        p = binding.prepare_weights(w, r, b)
        p.codes.cpu(), p.scales.cpu(), a.cpu(), r.cpu()
        torch.cuda.synchronize()
    t_seq = time.perf_counter() - t0
    # the device work alone (weights resident): the prepare kernel's roofline
    dw = [L.w.to(dev) for L in layers[:len(BLOCK_SHAPES)]]
    rr = [torch.ones(L.w.shape[1], dtype=torch.float32, device=dev) for L in layers[:len(BLOCK_SHAPES)]]
    outs = [binding.prepare_weights(w, r, b) for w, r in zip(dw, rr)]
    torch.cuda.synchronize()
    with Timer(torch) as t:
        for w, r, o in zip(dw, rr, outs):
            binding.prepare_weights(w, r, b, out=o)
    torch.cuda.synchronize()
    ms_dev = t.ms()
    dev_bytes = sum(w.numel() * (2 + 17 / 32) for w in dw)
    gbs_dev = dev_bytes / (ms_dev * 1e-3) / 1e9
    flips_note = len(out)
    res = {
        "metric": METRIC, "value": round(wbytes / t_stream / 1e9, 2),
        "unit": "GB/s of bf16 weights, pinned host in -> prepared pinned host out", "n_gpus": 1, "steps": 1,
        "warmup": 1, "ms_per_step": round(t_stream * 1e3, 2), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 weights in, MXFP4 (codes + E8M0 scales) out",
        "data": "synthetic (seeded device generator, N(0, 0.02^2) weights, N(0, 1) calibration rows)",
        "config": {"workload": "prepare-stream: %d blocks x %d linears of an 8B-shaped block %s, %d calibration rows "
                               "each, Hadamard block %d" % (STREAM_BLOCKS, len(BLOCK_SHAPES), BLOCK_SHAPES,
                                                            inputs.CALIB_ROWS, b),
                   "layers": flips_note, "weight_bytes": int(wbytes), "packed_bytes": int(pbytes)},
        "sequential_s": round(t_seq, 3), "overlap_speedup": round(t_seq / t_stream, 2),
        "peak_device_bytes": int(peak), "largest_layer_bytes": int(2 * max_n * max_k),
        "roofline": {"bound": "hbm", "achieved": round(gbs_dev, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs_dev / PEAK_HBM_GBS, 4), "traffic": None,
                     "kernel": "quant_rows_kernel as macaq_prepare_weights (2 B read + 17/32 B written per weight), "
                               "one block's seven layers resident"},
        "timing": "wall clock around the streamed run (host in to host out); device work timed with HIP events",
    }
    if not args.no_cpu_baseline:
        import numpy as np
        import oracle
        L = layers[0]
        wb = inputs.bf16_bits(L.w[:256])
        t0 = time.perf_counter()
        a_o, r_o = oracle.multipliers(oracle.calibrate(inputs.bf16_bits(L.xcal)), b)
        oracle.prepare_weights(wb, r_o, b)
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = dict(value=round(wb.size * 2 / dt / 1e9, 4), unit="GB/s of bf16 weights", cores=1,
                                   kind="oracle", sample="256 rows of a 4096 x 4096 layer (calibrate, multipliers, "
                                                         "prepare), %.2f s" % dt)
    emit(args, res)


def mfma_probe_tflops(torch, binding, dev, operands, iters=20000, reps=5):
    """Back-to-back scaled-FP4 MFMAs on register operands (one workgroup per
    CU): TFLOP/s, the median over reps launches."""
    import statistics
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.empty(cus * 256, dtype=torch.float32, device=dev)
    binding.mfma_probe(operands, cus, 200, out)
    ts = []
    for _ in range(reps):
        with Timer(torch) as t:
            binding.mfma_probe(operands, cus, iters, out)
        torch.cuda.synchronize()
        ts.append(t.ms())
    return cus * 4 * iters * 8 * MFMA_FLOPS / (statistics.median(ts) * 1e-3) / 1e12


def read_probe_gbs(torch, binding, dev, mib, copies, workgroups, reps=16):
    """Plain read of `mib` MiB (copies rotated past the last-level cache) by
    the read probe: GB/s per launch over reps back-to-back launches, the
    median of 3."""
    import statistics
    gen = torch.Generator(device=dev)
    gen.manual_seed(12)
    bufs = [torch.randint(0, 1 << 30, (mib << 18,), dtype=torch.int32, device=dev, generator=gen)
            for _ in range(copies)]
    iout = torch.empty(workgroups * 256, dtype=torch.int32, device=dev)
    for b in bufs:
        binding.read_probe(b, workgroups, iout)
    ts = []
    for _ in range(3):
        with Timer(torch) as t:
            for i in range(reps):
                binding.read_probe(bufs[i % copies], workgroups, iout)
        torch.cuda.synchronize()
        ts.append(t.ms() / reps)
    del bufs
    torch.cuda.empty_cache()
    return (mib << 20) / (statistics.median(ts) * 1e-3) / 1e9


def random_probe_operands(torch, binding, dev):
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    return torch.randint(0, 256, (binding.MFMA_PROBE_OPERAND_BYTES,), dtype=torch.uint8, device=dev, generator=gen)


def peaks_main(args, torch, binding, dev):
    """The ceilings the kernels are read against, measured on this device:
    back-to-back scaled-FP4 MFMAs on register operands (one workgroup of 4
    waves per CU, 8 independent accumulators per wave) with constant and with
    random operand bytes, and plain reads of 70 MiB, 470 MiB and 2 GiB (each
    thread 8 loads of 16 bytes in flight, inputs rotated past the 256 MB
    last-level cache) at several grid sizes, and a device copy of 512 MiB;
    the reads and the copy are timed over back-to-back launches, as a layer's
    launches follow one another in a step."""
    import statistics
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    iters = 20000
    operands = {"constant": torch.full((binding.MFMA_PROBE_OPERAND_BYTES,), 0x22, dtype=torch.uint8, device=dev),
                "random": random_probe_operands(torch, binding, dev)}  # constant: E2M1 1.0 in each nibble
    mfma = {k: round(mfma_probe_tflops(torch, binding, dev, ops, iters), 1) for k, ops in operands.items()}
    gen = torch.Generator(device=dev)
    gen.manual_seed(12)
    reads = {}
    for mib, copies in ((70, 8), (470, 2), (2048, 1)):
        reads["%d MiB" % mib] = {str(w): round(read_probe_gbs(torch, binding, dev, mib, copies, w), 1)
                                 for w in (256, 512, 1024, 4096)}
    src = [torch.randint(0, 1 << 30, (128 << 20,), dtype=torch.int32, device=dev, generator=gen) for _ in range(2)]
    dst = [torch.empty_like(x) for x in src]
    ts = []
    for _ in range(3):
        with Timer(torch) as t:
            for i in range(8):
                dst[i % 2].copy_(src[i % 2])
        torch.cuda.synchronize()
        ts.append(t.ms() / 8)
    copy_gbs = round(2 * (512 << 20) / (statistics.median(ts) * 1e-3) / 1e9, 1)
    best_read = max(v for row in reads.values() for v in row.values())
    res = {
        "metric": "measured ceilings: scaled-FP4 MFMA rate and HBM read bandwidth", "value": mfma["random"],
        "unit": "TFLOP/s (scaled-FP4 MFMA, random operands)", "n_gpus": 1, "steps": 5, "warmup": 1,
        "ms_per_step": None, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp4 (E2M1 x E2M1, fp32 accumulate)", "data": "synthetic (constant and seeded random bytes)",
        "config": {"workload": "peaks: %d workgroups x 4 waves x %d rounds of 8 independent 32x32x64 scaled-FP4 "
                               "MFMAs; plain reads of 70 MiB, 470 MiB, 2 GiB; device copy of 512 MiB" % (cus, iters),
                   "compute_units": cus},
        "mfma_fp4_tflops": dict(mfma, nominal=PEAK_FP4_TFLOPS),
        "mfma_fraction_of_nominal": {k: round(v / PEAK_FP4_TFLOPS, 4) for k, v in mfma.items()},
        "hbm_read_gbs_by_workgroups": reads, "copy_gbs_read_plus_write": copy_gbs,
        "hbm_read_fraction_of_nominal": round(best_read / PEAK_HBM_GBS, 4),
        "timing": "MFMA: HIP events around each launch (median of 5); reads and copy: HIP events around 16 (8) "
                  "back-to-back launches with the buffers rotated, per launch (median of 3)",
    }
    emit(args, res)


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


def timed_steps(torch, step, steps, warmup):
    """`warmup` untimed steps, then exactly `steps` timed steps, each step(c)
    on operand copy c = i % ROTATE. The steps are captured in one HIP graph
    per phase, so the timed replay has no host gaps between steps; HIP events
    on the launch stream bracket it. Returns (ms per step, wall seconds)."""
    gw = capture(torch, lambda: [step(i % ROTATE) for i in range(warmup)]) if warmup > 0 else None
    gt = capture(torch, lambda: [step((warmup + i) % ROTATE) for i in range(steps)])
    if gw is not None:
        gw.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with Timer(torch) as t:
        gt.replay()
    torch.cuda.synchronize()
    return t.ms() / steps, time.perf_counter() - t0


def host_cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def step_distribution(torch, step, reps, warmup):
    """Per-step times: one HIP graph per operand copy (one step each),
    replayed in turn, each replay bracketed by its own HIP events. Returns
    (p10, median, p90) in ms."""
    graphs = [capture(torch, lambda c=c: step(c)) for c in range(ROTATE)]
    for i in range(warmup):
        graphs[i % ROTATE].replay()
    timers = []
    for i in range(reps):
        with Timer(torch) as t:
            graphs[i % ROTATE].replay()
        timers.append(t)
    torch.cuda.synchronize()
    ms = sorted(t.ms() for t in timers)
    pick = lambda q: ms[min(len(ms) - 1, int(round(q * (len(ms) - 1))))]
    return pick(0.1), pick(0.5), pick(0.9)


def overhead_pairs(torch, step, step_plain, reps, warmup):
    """The fused and the plain step (one HIP graph per operand copy each)
    replayed alternately, fused then plain, each replay bracketed by its own
    HIP events: per pair the ratio fused / plain. Returns the ratios' (p10,
    median, p90) and the medians of both step times, in ms."""
    gf = [capture(torch, lambda c=c: step(c)) for c in range(ROTATE)]
    gp = [capture(torch, lambda c=c: step_plain(c)) for c in range(ROTATE)]
    for i in range(warmup):
        gf[i % ROTATE].replay()
        gp[i % ROTATE].replay()
    pairs = []
    for i in range(reps):
        with Timer(torch) as tf:
            gf[i % ROTATE].replay()
        with Timer(torch) as tp:
            gp[i % ROTATE].replay()
        pairs.append((tf, tp))
    torch.cuda.synchronize()
    f = [a.ms() for a, _ in pairs]
    p = [b.ms() for _, b in pairs]
    ratios = sorted(x / y for x, y in zip(f, p))
    pick = lambda v, q: v[min(len(v) - 1, int(round(q * (len(v) - 1))))]
    return (pick(ratios, 0.1), pick(ratios, 0.5), pick(ratios, 0.9)), pick(sorted(f), 0.5), pick(sorted(p), 0.5)


def cpu_baseline(entries, target_s, moe):
    """The oracle (C, fp64 GEMM over codes, as it stands) on a bounded sample
    of the step's rows: rows of every dense layer, or the first experts."""
    import numpy as np

    import oracle
    from mxfp4_w4a4_post_amd import inputs as inp

    threads = min(oracle.default_threads(), ORACLE_THREADS_CAP)
    if moe == "block":
        case = entries[0].oracle_case[0]
        bits = inp.bf16_bits
        x = bits(case.x)
        n, dt, flops = 4, 0.0, 0.0
        while True:
            want = np.zeros(case.T, bool)
            want[:n] = True
            used = np.unique(case.ids[:n])
            a_gu = np.ones((case.E, case.H), np.float32)
            a_dn = np.ones((case.E, case.F), np.float32)
            gc = np.zeros((case.E, 2 * case.F, case.H // 2), np.uint8)
            gs = np.zeros((case.E, 2 * case.F, case.H // 32), np.uint8)
            dc = np.zeros((case.E, case.H, case.F // 2), np.uint8)
            ds = np.zeros((case.E, case.H, case.F // 32), np.uint8)
            for ex in used:
                a, r = oracle.multipliers(oracle.calibrate(bits(case.xcal_gu[ex])), case.b)
                a_gu[ex] = a
                wgu = np.stack([bits(case.w_gate[ex]).reshape(case.F // 32, 32, case.H),
                                bits(case.w_up[ex]).reshape(case.F // 32, 32, case.H)], axis=1)
                gc[ex], gs[ex] = oracle.prepare_weights(wgu.reshape(2 * case.F, case.H), r, case.b)
                a, r = oracle.multipliers(oracle.calibrate(bits(case.xcal_dn[ex])), case.b)
                a_dn[ex] = a
                dc[ex], ds[ex] = oracle.prepare_weights(bits(case.w_dn[ex]), r, case.b)
            t0 = time.perf_counter()
            oracle.moe_block(x, case.ids, case.w, case.E, a_gu, gc, gs, a_dn, dc, ds, case.b, want=want,
                             threads=threads)
            dt = time.perf_counter() - t0
            flops = 2.0 * n * case.k * (2 * case.F * case.H + case.H * case.F)
            if dt >= target_s * 0.7 or n >= case.T:
                break
            n = min(case.T, n * max(2, int(target_s / max(dt, 1e-3))))
        return dict(value=round(flops / dt / 1e12, 6), unit="TFLOP/s", cores=threads, kind="oracle",
                    sample="the whole block (routing, gathered gate/up, SiLU x up, down input quantize, down, "
                           "combine) for the first %d of %d tokens, weights of their experts prepared outside "
                           "the timing, %.1f s" % (n, case.T, dt))
    if moe:
        flops, dt, experts = 0.0, 0.0, 0
        while dt < target_s and experts < entries[0].oracle_case[0].E:
            for e in entries:
                case = e.oracle_case[0]
                lo, hi = int(case.offsets[experts]), int(case.offsets[experts + 1])
                if hi <= lo:
                    continue
                s = oracle.calibrate(inp.bf16_bits(case.xcal[experts]))
                a, r = oracle.multipliers(s, case.b)
                wc, ws = oracle.prepare_weights(inp.bf16_bits(case.w[experts]), r, case.b)
                xb = np.ascontiguousarray(inp.bf16_bits(case.x[lo:hi]))
                t0 = time.perf_counter()
                oracle.linear(xb, a, case.b, wc, ws, threads=threads)
                dt += time.perf_counter() - t0
                flops += 2.0 * (hi - lo) * case.N * case.K
            experts += 1
        return dict(value=round(flops / dt / 1e12, 6), unit="TFLOP/s", cores=threads, kind="oracle",
                    sample="experts 0..%d of both projections (quantize + fp64 GEMM over codes, weights prepared "
                           "outside the timing), %.1f s" % (experts - 1, dt))
    prepared = []
    for e in entries:
        case, M = e.oracle_case
        s = oracle.calibrate(inp.bf16_bits(case.xcal))
        a, r = oracle.multipliers(s, case.b)
        wc, ws = oracle.prepare_weights(inp.bf16_bits(case.w), r, case.b)
        prepared.append((inp.bf16_bits(case.x[:M]), a, case.b, wc, ws, case.K, case.N, M))
    frac = 1.0 / 64
    while True:
        t0 = time.perf_counter()
        flops, rows_done, rows_all = 0.0, 0, 0
        for xb, a, b, wc, ws, K, N, M in prepared:
            rows = max(1, min(M, int(round(M * frac))))
            oracle.linear(np.ascontiguousarray(xb[:rows]), a, b, wc, ws, threads=threads)
            flops += 2.0 * rows * K * N
            rows_done += rows
            rows_all += M
        dt = time.perf_counter() - t0
        if dt >= target_s * 0.7 or frac >= 1.0:
            break
        frac = min(1.0, frac * max(2.0, target_s / max(dt, 1e-3)))
    return dict(value=round(flops / dt / 1e12, 6), unit="TFLOP/s", cores=threads, kind="oracle",
                sample="%d of %d token rows over the step's %d layer calls (quantize + fp64 GEMM over codes, "
                       "weights prepared outside the timing), %.1f s" % (rows_done, rows_all, len(prepared), dt))


def load_traffic(workload, kernel_digest):
    """HBM bytes (FETCH_SIZE + WRITE_SIZE, each scaled by a plain copy of known
    size) per GEMM launch, the mean over the step's layers, from the committed
    rocprofv3 counter summary; None unless it was taken on the current kernel
    source."""
    path = os.path.join(ROOT, "profiles", "gemm_%s_pmc.json" % workload.replace("-", "_"))
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
        print("bench.py measures one GPU: the library has no multi-GPU path (the design notes describe how the "
              "layer would shard); run with --gpus 1", file=sys.stderr)
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
    if args.gemm_only:
        M, N, K = (int(v) for v in args.gemm_only.split("x"))
        gen = torch.Generator(device=dev)
        gen.manual_seed(5)

        def packed(rows):
            return binding.Packed(
                torch.randint(0, 256, (binding.packed_codes_bytes(rows, K),), dtype=torch.uint8, device=dev,
                              generator=gen),
                torch.randint(120, 130, (binding.packed_scales_bytes(rows, K),), dtype=torch.uint8, device=dev,
                              generator=gen), rows, K)
        a, w = packed(M), packed(N)
        y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        work = torch.empty(max(binding.gemm_workspace_size(M, K, N), 1), dtype=torch.uint8, device=dev)
        for _ in range(max(args.profile_steps, 1)):
            binding.linear_plain_gemm(a, w, out=y, workspace=work)
        torch.cuda.synchronize()
        print(json.dumps({"gemm_only": [M, N, K], "launches": max(args.profile_steps, 1)}), flush=True)
        return
    wl = WORKLOADS[args.workload]
    if wl == REFINE:
        refine_main(args, torch, binding, inputs, dev)
        return
    if wl == QUANT_ERROR:
        quant_error_main(args, torch, binding, inputs, dev)
        return
    if wl == PREPARE_STREAM:
        prepare_stream_main(args, torch, binding, inputs, dev)
        return
    if wl == PEAKS:
        peaks_main(args, torch, binding, dev)
        return
    spec = inputs.WORKLOAD_SPECS[4 if wl == MOE_BLOCK else wl]
    b = args.block if args.block is not None else spec["blocks"][0]
    moe = wl == 4
    if wl == MOE_BLOCK:
        entries = moe_block_entries(torch, binding, inputs, b, dev)
        workload = ("moe-block: %d tokens routed top-%d over %d experts (Zipf(%.1f) popularity), hidden %d, expert "
                    "FFN %d (gate/up stacked, SwiGLU epilogue quantizing the down input), down, weighted combine, "
                    "Hadamard block %d, bf16 in/out" % (spec["tokens"], spec["top_k"], spec["experts"], spec["zipf"],
                                                        spec["hidden"], spec["ffn"], b))
        tokens = spec["tokens"]
        cfg_extra = {"tokens": tokens, "experts": spec["experts"], "top_k": spec["top_k"], "hidden": spec["hidden"],
                     "ffn": spec["ffn"], "hadamard_block": b}
    elif moe:
        entries = moe_entries(torch, binding, inputs, b, dev)
        workload = ("%s: %d tokens routed top-%d over %d experts (Zipf(%.1f) popularity), grouped gate/up %d->%d "
                    "and down %d->%d, Hadamard block %d, bf16 in/out"
                    % (spec["name"], spec["tokens"], spec["top_k"], spec["experts"], spec["zipf"], spec["hidden"],
                       2 * spec["ffn"], spec["ffn"], spec["hidden"], b))
        tokens = spec["tokens"]
        cfg_extra = {"tokens": tokens, "experts": spec["experts"], "top_k": spec["top_k"], "hadamard_block": b}
    else:
        entries, Ms = dense_entries(torch, binding, inputs, wl, b, dev)
        workload = ("%s: M=%s tokens, (K,N) in %s, Hadamard block %d, bf16 in/out"
                    % (spec["name"], Ms[0] if len(Ms) == 1 else Ms, spec["shapes"], b))
        tokens = sum(Ms)
        cfg_extra = {"tokens": Ms[0] if len(Ms) == 1 else Ms, "layers": [list(s) for s in spec["shapes"]],
                     "hadamard_block": b}
    torch.cuda.synchronize()

    def step(c, plain=False):
        for e in entries:
            (e.plain if plain else e.fused)(c)

    if args.profile_steps > 0:
        for i in range(args.profile_steps):
            step(i % ROTATE)
        torch.cuda.synchronize()
        print(json.dumps({"profiled_steps": args.profile_steps, "workload": spec["name"]}), flush=True)
        return

    flops = sum(e.flops for e in entries)
    nbytes = sum(e.bytes for e in entries)
    ms, wall = timed_steps(torch, step, args.steps, args.warmup)
    ms_plain, _ = timed_steps(torch, lambda c: step(c, True), args.steps, args.warmup)
    tflops = flops / (ms * 1e-3) / 1e12
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
        "data": "synthetic (seeded activations with outlier channels, N(0,sigma^2) weights; recipe in inputs.py)",
        "config": dict({"workload": workload}, **cfg_extra),
        "pct_mxfp4_peak": round(100 * tflops / PEAK_FP4_TFLOPS, 2),
        "tokens_per_s": round(tokens / (ms * 1e-3), 1),
        "hbm_gbs_algorithmic": round(nbytes / (ms * 1e-3) / 1e9, 1),
        "plain_mxfp4_ms_per_step": round(ms_plain, 5),
        "wall_s_timed": round(wall, 4),
        "timing": "the timed steps in one HIP graph (operand copies cycled, %d copies), HIP events on the launch "
                  "stream" % ROTATE,
    }
    # the overhead from interleaved single steps: fused, plain, fused, plain
    # ... (at least 50 pairs), the median of the per-pair ratios with its
    # spread; it replaces the two-replay figure above
    reps = max(args.steps, 50)
    (r10, r50, r90), f50, p50 = overhead_pairs(torch, step, lambda c: step(c, True), reps, args.warmup)
    out["transform_overhead_pct"] = round(100 * (r50 - 1), 2)
    out["transform_overhead_p10_p90_pct"] = [round(100 * (r10 - 1), 2), round(100 * (r90 - 1), 2)]
    out["transform_overhead_method"] = ("median of %d per-pair ratios fused/plain, the two steps replayed "
                                        "alternately (one graph per operand copy each), HIP events around "
                                        "each replay" % reps)
    out["transform_overhead_two_replays_pct"] = round(100 * (ms / ms_plain - 1), 2)
    out["step_ms_median_fused_plain"] = [round(f50, 5), round(p50, 5)]
    if wl == MOE_BLOCK:
        e = entries[0]
        parts = {k: timed_steps(torch, getattr(e, k), args.steps, args.warmup)[0]
                 for k in ("route", "gate_up", "down_combine", "gate_up_plain", "down_combine_plain")}
        out["calls_ms_per_step"] = {k: round(v, 5) for k, v in parts.items()}
        out["overhead_split_ms"] = {"gate_up": round(parts["gate_up"] - parts["gate_up_plain"], 5),
                                    "down_combine": round(parts["down_combine"] - parts["down_combine_plain"], 5)}
        gb_step = nbytes / (ms * 1e-3) / 1e9
        gu_gb = e.parts_bytes["gate_up"] / (parts["gate_up"] * 1e-3) / 1e9
        out["roofline"] = {"bound": "hbm", "achieved": round(gb_step, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "frac": round(gb_step / PEAK_HBM_GBS, 4), "traffic": None,
                           "kernel": "macaq_moe_block (algorithmic bytes: tokens read once, both expert weight "
                                     "sets, y written once)",
                           "gate_up_call_gbs": round(gu_gb, 1),
                           "kernel_source_digest": digest}
    elif not moe:
        # each kernel of the step alone: the same timed steps with only that
        # kernel of every layer call, on the same operand copies
        def kernel_ms(attr):
            return timed_steps(torch, lambda c: [getattr(e, attr)(c) for e in entries], args.steps,
                               args.warmup)[0]

        q, g, qp, gp = (kernel_ms(k) for k in ("quant", "gemm", "quant_plain", "gemm_plain"))
        out["kernels_ms_per_step"] = {"calls": len(entries), "quant": round(q, 5), "gemm": round(g, 5),
                                      "quant_plain": round(qp, 5), "gemm_plain": round(gp, 5)}
        out["overhead_split_ms"] = {"quantize": round(q - qp, 5), "gemm_on_transformed_codes": round(g - gp, 5)}
        out["transform_overhead_kernel_sum_pct"] = round(100 * ((q + g) / (qp + gp) - 1), 2)
        # the same fused step with fp32 output (the precision the parity
        # tests compare)
        ms32, _ = timed_steps(torch, lambda c: [e.fused_f32(c) for e in entries], args.steps, args.warmup)
        out["fp32_out"] = {"ms_per_step": round(ms32, 5), "tflops": round(flops / (ms32 * 1e-3) / 1e12, 2)}
        gemm_ms = g
        if wl == 3:  # decode: the GEMM streams the weights
            gb = sum(e.gemm_bytes for e in entries) / (gemm_ms * 1e-3) / 1e9
            out["roofline"] = {"bound": "hbm", "achieved": round(gb, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                               "frac": round(gb / PEAK_HBM_GBS, 4), "traffic": load_traffic(spec["name"], digest),
                               "kernel": "gemm_kernel (weights streamed per wave)",
                               "avg_launch_us": round(1e3 * gemm_ms / len(entries), 3),
                               "kernel_source_digest": digest}
            # the practical ceiling at this size in the same run: a plain read
            # of 70 MiB (a call's weights), the better of two grids
            ceil_gbs = max(read_probe_gbs(torch, binding, dev, 70, 8, w) for w in (512, 4096))
            out["read_ceiling_70MiB"] = {"gbs": round(ceil_gbs, 1), "gemm_fraction_of_it": round(gb / ceil_gbs, 4),
                                         "probe": "macaq_debug_read_probe (bench.py --workload peaks)"}
        else:
            tf = flops / (gemm_ms * 1e-3) / 1e12
            kname = ("gemm_wide_kernel (256 x 256 tiles, scaled-FP4 MFMA)" if wl == 5 else
                     "scaled-FP4 MFMA GEMM (gemm_wide_kernel for 4096 x 14336, gemm_kernel 128 x 256 for the "
                     "4096-wide layers)")
            out["roofline"] = {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_FP4_TFLOPS,
                               "unit": "TFLOP/s", "frac": round(tf / PEAK_FP4_TFLOPS, 4),
                               "traffic": load_traffic(spec["name"], digest),
                               "kernel": kname,
                               "avg_launch_us": round(1e3 * gemm_ms / len(entries), 3),
                               "kernel_source_digest": digest}
            if wl in (2, 5):
                # the practical ceiling on this device in the same run: back-to-back
                # MFMAs on random operands, where the matrix cores run power-limited
                probe = mfma_probe_tflops(torch, binding, dev, random_probe_operands(torch, binding, dev), 8000, 3)
                out["mfma_ceiling_random_operands"] = {"tflops": round(probe, 1),
                                                       "gemm_fraction_of_it": round(tf / probe, 4),
                                                       "probe": "macaq_debug_mfma_probe (bench.py --workload peaks)"}
        if wl == 5 and not args.no_block_sweep:
            # the other Hadamard blocks of the large prefill workload: the
            # same layers and plain path, fused step with b = 64 and 128
            # (the headline's device buffers are released first; the oracle
            # baseline needs only their host-side cases)
            import types
            entries = [types.SimpleNamespace(oracle_case=e.oracle_case) for e in entries]
            torch.cuda.empty_cache()
            sweep = {}
            for bb in [v for v in spec["blocks"] if v != b]:
                eb, _ = dense_entries(torch, binding, inputs, wl, bb, dev)

                def step_b(c, plain=False, eb=eb):
                    for e in eb:
                        (e.plain if plain else e.fused)(c)

                msb, _ = timed_steps(torch, step_b, args.steps, args.warmup)
                (b10, b50, b90), _, _ = overhead_pairs(torch, step_b, lambda c: step_b(c, True), reps, args.warmup)
                tfb = flops / (msb * 1e-3) / 1e12
                sweep["b=%d" % bb] = {"ms_per_step": round(msb, 5), "tflops": round(tfb, 2),
                                      "pct_mxfp4_peak": round(100 * tfb / PEAK_FP4_TFLOPS, 2),
                                      "transform_overhead_pct": round(100 * (b50 - 1), 2),
                                      "transform_overhead_p10_p90_pct": [round(100 * (b10 - 1), 2),
                                                                         round(100 * (b90 - 1), 2)]}
                del eb
                torch.cuda.empty_cache()
            out["block_sweep"] = sweep
    else:
        calls = [timed_steps(torch, e.fused, 10, 2)[0] for e in entries]
        gb = nbytes / (sum(calls) * 1e-3) / 1e9
        out["calls_ms"] = {"calls": [e.name for e in entries], "fused": [round(v, 5) for v in calls]}
        out["roofline"] = {"bound": "hbm", "achieved": round(gb, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "frac": round(gb / PEAK_HBM_GBS, 4), "traffic": None,
                           "kernel": "macaq_linear_grouped (quantize + tile map + grouped GEMM per call)",
                           "kernel_source_digest": digest}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(entries, args.cpu_seconds, "block" if wl == MOE_BLOCK else moe)
        out["cpu_baseline"]["cpu_model"] = host_cpu_model()
    emit(args, out)


if __name__ == "__main__":
    main()
