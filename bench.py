#!/usr/bin/env python3
"""Benchmark of the row-typed associative-algebra projection on one MI355X.

One step is one pass of the hot path over one batch of synthetic input at the
Qwen3-8B-shaped workload (M = 2048 tokens, d_in = 4096, d_out = 12288, Q_32,
bf16 in and out, fp32 accumulation):
  1. aa_project_fwd      Y = X * W                      (one leaf-GEMM launch)
  2. aa_swiglu_ffn_fwd   H = silu(X*Wg)(X*Wu), Y2 = H*Wd  (two leaf-GEMM launches)
  3. aa_decode_gemv      32 new tokens, one per row type   (one decode launch)
Inputs are resident in HBM before the timed region.  Two complete input sets
(about 1.1 GB) alternate between steps so that the 256 MB Infinity Cache
cannot hold a step's working set (a flushed-cache measurement).

Printed (one JSON line): dense-equivalent TFLOP/s of the step (2 M d_in d_out
per dense projection counted for every projection in the step), the roofline of
the projection kernel (algorithmic HBM bytes / its duration), the same for
every call, a dense bf16 torch.matmul comparator timed in the same run, and the
fp64 oracle timed on the host on a bounded sample.  Call durations come from HIP
events that the library records from the kernels' own dispatches
(aa_set_kernel_events) inside the timed steps, so they match a kernel trace;
the step time comes from events around the K steps and includes the gaps
between kernels.

    python bench.py [--gpus 1] [--steps 300] [--warmup 10]
                    [--workload qwen3_8b_q32|square|pilot_ffn|expert_ffn|qwen3_1p7b|qwen3_8b_down|
                                backward_qwen3_8b|backward_expert]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300,
                    help="timed steps; the calls of a step take turns being timed by their kernel events, so each "
                         "call gets steps / calls samples (100 for the Qwen3-8B projection by default)")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="qwen3_8b_q32",
                    choices=["qwen3_8b_q32", "square", "pilot_ffn", "expert_ffn", "qwen3_1p7b", "qwen3_8b_down",
                             "qwen3_32b", "qwen3_8b_proj",
                             "digraph_qwen3_8b", "pilot_decode_stack", "pilot_generate",
                             "backward_qwen3_8b", "backward_expert"])
    ap.add_argument("--sets", type=int, default=0, help="rotating input sets (0 = enough to exceed 1 GB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="Qwen3-8B step: skip the other configurations (pilot FFN, expert FFN, square product) "
                         "that the default line also reports")
    ap.add_argument("--no-extras", action="store_true",
                    help="Qwen3-8B step and projections: skip the one-token and back-to-back measurements "
                         "(a kernel trace then holds only the warmup and timed calls)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle time for the CPU baseline")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="first run a 1 GiB device-to-device copy (reference kernel for HBM byte counters)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)
    import torch
    import aa_inputs as inp
    import associative_algebra_block_amd as aa

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU"}), flush=True)
        sys.exit(1)
    aa.load()
    dev = "cuda"
    torch.manual_seed(0)
    if args.calibration_copy:
        # A plain copy of known size: under rocprofv3 --pmc its FETCH_SIZE and
        # WRITE_SIZE give the factors that turn those counters into bytes.
        a = torch.ones(1 << 28, dtype=torch.int32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    if args.workload == "qwen3_8b_q32":
        res = bench_qwen3(args, torch, inp, aa, dev)
    elif args.workload == "qwen3_1p7b":
        res = bench_projection(args, torch, inp, aa, dev, inp.WORKLOADS[6])
    elif args.workload == "qwen3_8b_down":
        res = bench_projection(args, torch, inp, aa, dev, inp.WORKLOADS[7])
    elif args.workload == "qwen3_8b_proj":
        res = bench_projection(args, torch, inp, aa, dev, inp.WORKLOADS[3])
    elif args.workload == "qwen3_32b":
        res = bench_projection(args, torch, inp, aa, dev, inp.WORKLOADS[8])
    elif args.workload == "digraph_qwen3_8b":
        res = bench_projection(args, torch, inp, aa, dev, inp.WORKLOADS[3], digraph_density=0.5)
    elif args.workload.startswith("backward_"):
        res = bench_backward(args, torch, inp, aa, dev, args.workload)
    elif args.workload == "pilot_decode_stack":
        res = bench_decode_stack(args, torch, inp, aa, dev)
    elif args.workload == "pilot_generate":
        res = bench_generate(args, torch, aa, dev)
    elif args.workload == "square":
        res = bench_square(args, torch, inp, aa, dev)
    else:
        res = bench_ffn(args, torch, inp, aa, dev, args.workload)
    if not args.no_extras and isinstance(res.get("roofline"), dict) and res["roofline"].get("bound") == "hbm":
        copy = copy_bandwidth(torch, dev)
        res["achievable_hbm"] = {**copy, "roofline_kernel_frac_of_copy":
                                 round(res["roofline"]["achieved"] / copy["GBs"], 4)}
    print(json.dumps(res), flush=True)


# ------------------------------------------------------------------ helpers ---

def _ev(torch):
    return torch.cuda.Event(enable_timing=True)


class KernelTimer:
    """Durations of library calls taken from their own kernel dispatches
    (aa_set_kernel_events): the start event is a marker recorded just before
    the call's first dispatch, the stop event is recorded by its last kernel,
    so the queue time between calls is not counted.  An armed launch costs the
    host about 13 us more than a plain one, so one call per step is armed, in
    turn (step s times call s mod calls), which keeps small-kernel steps from
    waiting on the host.  Events are recorded once at creation because torch
    creates an event at its first record."""

    def __init__(self, torch, aa, steps, calls):
        if steps < calls:
            raise SystemExit(f"--steps must be at least {calls} here (one call of the step is timed per step)")
        self.aa, self.calls, self.armed = aa, calls, False
        self.ev = [(_ev(torch), _ev(torch)) for _ in range(steps)]
        for pair in self.ev:
            for e in pair:
                e.record()
        torch.cuda.synchronize()

    def arm(self, step, call):
        if step % self.calls == call:
            self.aa.aa_set_kernel_events(*self.ev[step])
            self.armed = True
        else:
            self.disarm()

    def disarm(self):
        if self.armed:
            self.aa.aa_set_kernel_events(None, None)
            self.armed = False

    def samples(self, call):
        return [a.elapsed_time(b) for s, (a, b) in enumerate(self.ev) if s % self.calls == call]

    def ms(self, call):
        """Mean duration of the call over the steps that timed it, in ms."""
        t = self.samples(call)
        return sum(t) / len(t)

    def spread(self, call):
        """Median, 10th and 90th percentile of the call's durations (ms)."""
        t = sorted(self.samples(call))
        q = lambda f: t[min(len(t) - 1, int(round(f * (len(t) - 1))))]
        return {"median_ms": round(q(0.5), 5), "p10_ms": round(q(0.1), 5), "p90_ms": round(q(0.9), 5),
                "samples": len(t)}


def kernel_source_hash():
    """Hash of the kernels' sources (aa_kernels.hip, aa_small.hip,
    aa_backward.hip, aa_tile32.hip and the device header they include): stored
    traffic figures are used only while it matches."""
    h = hashlib.sha256()
    for name in ("aa_kernels.hip", "aa_small.hip", "aa_backward.hip", "aa_tile32.hip", "aa_device.h"):
        with open(os.path.join(HERE, "associative_algebra_block_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel_key):
    """HBM bytes per launch measured with rocprofv3 counters, if the committed
    measurement was taken on the current kernel source; else None."""
    p = os.path.join(HERE, "profiles", "traffic.json")
    try:
        with open(p) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    v = rec.get("kernels", {}).get(kernel_key)
    return None if v is None else v.get("hbm_bytes_per_launch")


def roofline(bytes_alg, ms, traffic=None):
    gbs = bytes_alg / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic}


def proj_bytes(M, d_in, d_out, eb_in=2, eb_out=2):
    return eb_in * (M * d_in + d_in * d_out) + eb_out * M * d_out


def exec_flops(M, d_in, d_out, law, q):
    per = (2 * q - 1) / (q * q) if law == "Qq" else 9 / 16
    return 2.0 * M * d_in * d_out * per


def dense_timer(torch, fn, iters=20, warm=5):
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    a, b = _ev(torch), _ev(torch)
    a.record()
    for _ in range(iters):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / iters


def copy_bandwidth(torch, dev, nbytes=1 << 30, reps=10):
    """What a plain device-to-device copy reaches on this GPU in the same run
    (torch copy_ of 1 GiB, two buffer pairs alternating so that the 256 MB
    Infinity Cache holds neither): read plus write bytes per second.  A
    secondary, achievable reference beside the datasheet peak."""
    bufs = [torch.empty(nbytes // 2, dtype=torch.int16, device=dev) for _ in range(4)]
    for t in bufs:
        t.zero_()
    for r in range(3):
        bufs[2 * (r % 2) + 1].copy_(bufs[2 * (r % 2)])
    torch.cuda.synchronize()
    a, b = _ev(torch), _ev(torch)
    a.record()
    for r in range(reps):
        bufs[2 * (r % 2) + 1].copy_(bufs[2 * (r % 2)])
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del bufs
    return {"kind": "torch copy_ of 1 GiB, device to device, hot loop of 10", "GBs": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}


def cpu_threads():
    """Host threads the oracle's BLAS may use: the cores this process may run
    on (its affinity set), capped by OMP_NUM_THREADS when that is set (a
    shared host's share of cores)."""
    n = len(os.sched_getaffinity(0))
    try:
        cap = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        cap = 0
    return min(n, cap) if cap > 0 else n


def timed_oracle(fn):
    """Run fn() with the BLAS pool pinned to cpu_threads(); returns (fn's
    result, the BLAS thread count actually in effect, the affinity size)."""
    n = cpu_threads()
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        with threadpool_limits(limits=n, user_api="blas"):
            used = max((d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"),
                       default=1)
            out = fn()
    except ImportError:
        used, out = n, fn()
    return out, int(used), len(os.sched_getaffinity(0))


# ---------------------------------------------------- Qwen3-8B-shaped step ---

def bench_qwen3(args, torch, inp, aa, dev):
    wl = inp.WORKLOADS[3]
    M, D, F, q, law = wl.M, wl.d_in, wl.d_out, wl.q, wl.law
    n_dec = wl.decode_tokens
    plan = aa.aa_plan_create(law, q, D, F, "pos_mod", 0, "bf16", "bf16")    # projection and gate/up
    down = aa.aa_plan_create(law, q, F, D, "pos_mod", 0, "bf16", "bf16")

    set_bytes = 2 * (M * D + 3 * D * F + F * D + M * F * 2 + M * D + n_dec * (D + F))
    n_sets = args.sets or max(2, math.ceil(1.0e9 / set_bytes))
    sets = []
    for s in range(n_sets):
        seed_off = 100 * s
        X = inp.gaussian((M, D), inp.seed_for(inp.ROLE_X, 3) + seed_off, 1.0, torch.bfloat16, dev)
        W = inp.gaussian((D, F), inp.seed_for(inp.ROLE_W, 3) + seed_off, D ** -0.5, torch.bfloat16, dev)
        Wu = inp.gaussian((D, F), inp.seed_for(inp.ROLE_WU, 3) + seed_off, D ** -0.5, torch.bfloat16, dev)
        Wd = inp.gaussian((F, D), inp.seed_for(inp.ROLE_WD, 3) + seed_off, F ** -0.5, torch.bfloat16, dev)
        st = {
            "X": X, "Wp": aa.pack(plan, W), "Wup": aa.pack(plan, Wu),
            "Wdp": aa.pack(down, Wd), "Y": torch.empty(M, F, dtype=torch.bfloat16, device=dev),
            "H": torch.empty(M, F, dtype=torch.bfloat16, device=dev),
            "Y2": torch.empty(M, D, dtype=torch.bfloat16, device=dev),
            "x": X[:n_dec].clone(), "y": torch.empty(n_dec, F, dtype=torch.bfloat16, device=dev),
        }
        # the gate weight is its own tensor, not an alias of the projection weight
        st["Wgp"] = aa.pack(plan, inp.gaussian((D, F), inp.seed_for(inp.ROLE_W, 3) + seed_off + 50, D ** -0.5,
                                               torch.bfloat16, dev))
        del W, Wu, Wd
        sets.append(st)
    torch.cuda.synchronize()
    pos_dec = 4096  # decode positions 4096 .. 4127: one token of every type

    def step(st, kt=None, s=0):
        if kt:
            kt.arm(s, 0)
        aa.aa_project_fwd(plan, st["X"], st["Wp"], st["Y"])
        if kt:
            kt.arm(s, 1)
        aa.aa_swiglu_ffn_fwd(plan, down, st["X"], st["Wgp"], st["Wup"], st["Wdp"], st["H"], st["Y2"])
        if kt:
            kt.arm(s, 2)
        aa.aa_decode_gemv(plan, st["x"], st["Wp"], st["y"], None, pos_dec)
        if kt:
            kt.disarm()

    for w in range(args.warmup):
        step(sets[w % n_sets])
    torch.cuda.synchronize()
    K = args.steps
    kt = KernelTimer(torch, aa, K, 3)
    t0e, t1e = _ev(torch), _ev(torch)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0e.record()
    for s in range(K):
        step(sets[s % n_sets], kt, s)
    t1e.record()
    torch.cuda.synchronize()
    wall1 = time.perf_counter()
    ms_step = t0e.elapsed_time(t1e) / K
    ms_proj, ms_swi, ms_dec = kt.ms(0), kt.ms(1), kt.ms(2)

    dense_flops = {"project": 2.0 * M * D * F, "swiglu": 3 * 2.0 * M * D * F, "decode": 2.0 * n_dec * D * F}
    total_dense = sum(dense_flops.values())
    value = total_dense / (ms_step * 1e-3) / 1e12

    b_proj = proj_bytes(M, D, F)
    b_swi = 2 * (M * D + 2 * D * F + M * F) + 2 * (M * F + F * D + M * D)
    b_dec = 2 * (n_dec * D + D * F + n_dec * F)
    ex_proj = exec_flops(M, D, F, law, q)
    parts = {
        "project": {"ms": round(ms_proj, 5), **kt.spread(0),
                    "dense_equiv_tflops": round(dense_flops["project"] / ms_proj / 1e9, 2),
                    "exec_tflops": round(ex_proj / ms_proj / 1e9, 2),
                    "roofline": roofline(b_proj, ms_proj, traffic_for("project_qwen3_8b_q32"))},
        "swiglu": {"ms": round(ms_swi, 5), **kt.spread(1),
                   "dense_equiv_tflops": round(dense_flops["swiglu"] / ms_swi / 1e9, 2),
                   "exec_tflops": round(3 * ex_proj / ms_swi / 1e9, 2),
                   "roofline": roofline(b_swi, ms_swi)},
        "decode32": {"ms": round(ms_dec, 5), **kt.spread(2),
                     "dense_equiv_tflops": round(dense_flops["decode"] / ms_dec / 1e9, 3),
                     "roofline": roofline(b_dec, ms_dec)},
    }

    dense = None
    if not args.no_dense:
        st = sets[0]
        Xd = st["X"]
        Wd1 = inp.gaussian((D, F), 999, D ** -0.5, torch.bfloat16, dev)
        Wd2 = inp.gaussian((D, F), 998, D ** -0.5, torch.bfloat16, dev)
        Wd3 = inp.gaussian((F, D), 997, F ** -0.5, torch.bfloat16, dev)
        xd = st["x"]
        t_p = dense_timer(torch, lambda: torch.matmul(Xd, Wd1))
        t_s = dense_timer(torch, lambda: torch.matmul(
            torch.nn.functional.silu(torch.matmul(Xd, Wd1)) * torch.matmul(Xd, Wd2), Wd3))
        t_d = dense_timer(torch, lambda: torch.matmul(xd, Wd1))
        dense = {"kind": "torch.matmul bf16 (hipBLASLt), hot cache, same run",
                 "project_ms": round(t_p, 5), "swiglu_ms": round(t_s, 5), "decode32_ms": round(t_d, 5),
                 "speedup_project": round(t_p / ms_proj, 3), "speedup_swiglu": round(t_s / ms_swi, 3),
                 "speedup_decode32": round(t_d / ms_dec, 3),
                 "speedup_step": round((t_p + t_s + t_d) / ms_step, 3)}
        del Wd1, Wd2, Wd3

    dec1 = ffn1 = alone = graph_step = None
    if not args.no_extras:
        dec1 = decode_single_token(torch, aa, plan, sets, pos_dec, n_dec, D, F, q,
                                   None if dense is None else sets[0])
        ffn1 = ffn_single_token(torch, aa, plan, down, sets, pos_dec, n_dec, D, F, q, dense is not None)
        alone = projection_alone(torch, aa, plan, [(st["X"], st["Wp"], st["Y"]) for st in sets], b_proj)
        # the same step replayed from HIP graphs (one per input set): no host
        # launch work and no queue gaps between its four kernels
        graphs = []
        for st in sets:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(st)
            graphs.append(g)
        for w in range(3):
            graphs[w % n_sets].replay()
        torch.cuda.synchronize()
        a, b = _ev(torch), _ev(torch)
        a.record()
        for s_ in range(K):
            graphs[s_ % n_sets].replay()
        b.record()
        torch.cuda.synchronize()
        ms_g = a.elapsed_time(b) / K
        graph_step = {"ms": round(ms_g, 5), "dense_equiv_tflops": round(total_dense / (ms_g * 1e-3) / 1e12, 2),
                      "kind": "the step captured in one HIP graph per input set, graphs replayed in turn"}
        del graphs

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_qwen3(args, torch, inp, sets[0], wl)

    configs = None
    if not args.no_configs:
        # the other configurations of the workload list, each against its own
        # binding roofline (after the step's own buffers are released)
        del sets
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        configs = {
            "pilot_ffn_q2xq2": ffn_part(torch, inp, aa, dev, "pilot_ffn", 60, 5, not args.no_dense),
            "qwen3_30b_a3b_expert_ffn_q16": ffn_part(torch, inp, aa, dev, "expert_ffn", 100, 10,
                                                     not args.no_dense),
            "square_n32768_b128": square_part(torch, inp, aa, dev, 20, 2, not args.no_dense),
            "qwen3_32b_q256": projection_part(torch, inp, aa, dev, inp.WORKLOADS[8], 20, 2, not args.no_dense),
        }

    return {
        "metric": "dense-equiv TFLOP/s + % roofline (HBM/MFMA), Qwen3-8B-shape q=32 M=2048 bf16",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "qwen3_8b_q32: project + SwiGLU FFN + 32-token decode", "M": M, "d_in": D,
                   "d_out": F, "q": q, "law": law, "type_map": "pos mod q", "decode_tokens": n_dec,
                   "input_sets": n_sets, "cache": "flushed (rotating input sets)"},
        "roofline": parts["project"]["roofline"],
        "roofline_kernel": "aa_project_fwd at the Qwen3-8B shape (leaf_persist_kernel)",
        "timing": "parts: kernel dispatch events of each call (first kernel start to last kernel end); "
                  "ms_per_step: events around the K steps",
        "ms_between_kernels": round(ms_step - ms_proj - ms_swi - ms_dec, 5),
        "parts": parts, "projection_alone": alone, "graph_step": graph_step, "decode_single_token": dec1,
        "ffn_single_token": ffn1,
        "dense": dense,
        "cpu_baseline": cpu,
        "configs": configs,
        "wall_s_timed": round(wall1 - wall0, 4),
        "kernel_source": kernel_source_hash(),
    }


def projection_alone(torch, aa, plan, sets, bytes_alg, reps=50):
    """The projection launched back to back (no other kernels or events in
    between): rotating the input sets (flushed cache: the sets together exceed
    the 256 MB Infinity Cache) and repeating one set (hot cache, as the pages
    also report)."""
    out = {}
    for name, order in (("flushed", list(range(len(sets)))), ("hot", [0])):
        for r in range(5):
            X, W, Y = sets[order[r % len(order)]]
            aa.aa_project_fwd(plan, X, W, Y)
        torch.cuda.synchronize()
        a, b = _ev(torch), _ev(torch)
        a.record()
        for r in range(reps):
            X, W, Y = sets[order[r % len(order)]]
            aa.aa_project_fwd(plan, X, W, Y)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        out[name] = {"ms": round(ms, 5), "GBs": round(bytes_alg / (ms * 1e-3) / 1e9, 1),
                     "frac_of_8TBs": round(bytes_alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    return out


def bench_projection(args, torch, inp, aa, dev, wl, digraph_density=None):
    """A single row-typed projection shape (position typing), flushed cache
    (rotating input sets of >= 1 GB in total) and hot cache, with a dense bf16
    comparator of the same shape.  With digraph_density the table is that of
    a seeded random directed graph on the q groups (each ordered pair an edge
    with that probability); the weight blocks of non-edges are read by no row,
    so the algorithmic bytes count only the q diagonal and |E| edge blocks."""
    M, D, F, q = wl.M, wl.d_in, wl.d_out, wl.q
    edges = None
    if digraph_density is None:
        plan = aa.aa_plan_create(wl.law, q, D, F, "pos_mod", 0, "bf16", "bf16")
        per_set = 2 * (M * D + D * F + M * F)
    else:
        edges = inp.random_edges(q, digraph_density, inp.seed_for(inp.ROLE_TYPES, wl.index))
        plan = aa.aa_plan_create_digraph(q, edges, D, F, "pos_mod", 0, "bf16", "bf16")
        per_set = 2 * (M * D + (q + len(edges)) * (D // q) * (F // q) + M * F)
    n_sets = args.sets or max(2, math.ceil(1.0e9 / per_set))
    sets = []
    for s in range(n_sets):
        X = inp.gaussian((M, D), inp.seed_for(inp.ROLE_X, wl.index) + 100 * s, 1.0, torch.bfloat16, dev)
        W = inp.gaussian((D, F), inp.seed_for(inp.ROLE_W, wl.index) + 100 * s, D ** -0.5, torch.bfloat16, dev)
        sets.append((X, aa.pack(plan, W), torch.empty(M, F, dtype=torch.bfloat16, device=dev)))
        del W
    torch.cuda.synchronize()
    for w in range(args.warmup):
        X, Wp, Y = sets[w % n_sets]
        aa.aa_project_fwd(plan, X, Wp, Y)
    torch.cuda.synchronize()
    K = args.steps
    a, b = _ev(torch), _ev(torch)
    a.record()
    for s in range(K):
        X, Wp, Y = sets[s % n_sets]
        aa.aa_project_fwd(plan, X, Wp, Y)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / K
    # Kernel durations from the dispatch events, in a second pass over the same
    # K calls: with one call per step an armed launch (~13 us more host time)
    # would hold up the timed steps of a ~20 us kernel.
    kt = KernelTimer(torch, aa, K, 1)
    for s in range(K):
        X, Wp, Y = sets[s % n_sets]
        kt.arm(s, 0)
        aa.aa_project_fwd(plan, X, Wp, Y)
    kt.disarm()
    torch.cuda.synchronize()
    ms_k = kt.ms(0)
    alone = None if args.no_extras else projection_alone(torch, aa, plan, sets, per_set)
    dense = None
    if not args.no_dense:
        Wd = inp.gaussian((D, F), 999, D ** -0.5, torch.bfloat16, dev)
        X0 = sets[0][0]
        t = dense_timer(torch, lambda: torch.matmul(X0, Wd))
        dense = {"kind": "torch.matmul bf16 (hipBLASLt), hot cache", "ms": round(t, 5),
                 "speedup_flushed": round(t / ms, 3)}
        if alone:
            dense["speedup_hot"] = round(t / alone["hot"]["ms"], 3)
    name = wl.name if edges is None else f"{wl.name} digraph ({len(edges)} of {q * (q - 1)} edges)"
    return {"metric": f"dense-equiv TFLOP/s + % roofline, {name} projection bf16",
            "value": round(2.0 * M * D * F / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
            "steps": K, "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": name, "M": M, "d_in": D, "d_out": F, "q": q,
                       "law": wl.law if edges is None else "digraph", "type_map": "pos mod q", "input_sets": n_sets,
                       **({} if edges is None else {"edges": len(edges)})},
            "roofline": roofline(per_set, ms_k, traffic_for(f"project_{wl.name}") if edges is None else None),
            "kernel_ms": round(ms_k, 5), "kernel_spread": kt.spread(0),
            "projection_alone": alone,
            "dense": dense,
            "exec_tflops": round((exec_flops(M, D, F, wl.law, q) if edges is None else
                                  2.0 * (M // q) * (D // q) * (F // q) * (q + 2 * len(edges))) / (ms * 1e-3) / 1e12, 2),
            "kernel_source": kernel_source_hash()}


def bench_backward(args, torch, inp, aa, dev, which):
    """Gradients of the projection(s): aa_project_bwd_data (dX) and
    aa_project_bwd_weight (dW) for an upstream gradient dY, bf16 in and out.
    backward_qwen3_8b: the Qwen3-8B projection (M = 2048, 4096 -> 12288, Q_32).
    backward_expert: the three projections of the Qwen3-30B-A3B expert FFN
    (M = 2048, 2048 -> 768 gate and up, 768 -> 2048 down, Q_16), the shape
    whose forward-plus-gradient the pages report.  A step is dX and dW of
    every projection; input sets rotate (flushed cache).  Each call's bytes
    are those of the forward: 2 (M d_in + d_in d_out + M d_out)."""
    M = 2048
    if which == "backward_qwen3_8b":
        q, shapes = 32, [("proj", 4096, 12288)]
    else:
        q, shapes = 16, [("gate", 2048, 768), ("up", 2048, 768), ("down", 768, 2048)]
    plans = {n: aa.aa_plan_create("Qq", q, di, do, "pos_mod", 0, "bf16", "bf16") for n, di, do in shapes}
    per_set = sum(2 * (2 * M * di + 2 * di * do + 2 * M * do) for _, di, do in shapes)
    n_sets = args.sets or max(2, math.ceil(1.0e9 / per_set))
    sets = []
    for s_ in range(n_sets):
        st = {}
        for j, (n, di, do) in enumerate(shapes):
            base = 1000 * (s_ + 1) + 10 * j
            W = inp.gaussian((di, do), base + 1, di ** -0.5, torch.bfloat16, dev)
            nd, nw = aa.aa_project_bwd_workspace(plans[n], M)
            st[n] = {"X": inp.gaussian((M, di), base + 2, 1.0, torch.bfloat16, dev),
                     "dY": inp.gaussian((M, do), base + 3, 1.0, torch.bfloat16, dev),
                     "Wp": aa.pack(plans[n], W),
                     "dX": torch.empty(M, di, dtype=torch.bfloat16, device=dev),
                     "dWp": torch.empty(di * do, dtype=torch.bfloat16, device=dev),
                     "wsd": torch.empty(max(nd, 1), dtype=torch.uint8, device=dev), "nd": nd,
                     "wsw": torch.empty(max(nw, 1), dtype=torch.uint8, device=dev), "nw": nw}
            del W
        sets.append(st)
    torch.cuda.synchronize()
    calls = [(n, kind) for n, _, _ in shapes for kind in ("dX", "dW")]

    def step(st, kt=None, s=0):
        for c, (n, kind) in enumerate(calls):
            if kt:
                kt.arm(s, c)
            b = st[n]
            if kind == "dX":
                aa.aa_project_bwd_data(plans[n], b["dY"], b["Wp"], b["dX"], None, 0, None, b["wsd"], b["nd"])
            else:
                aa.aa_project_bwd_weight(plans[n], b["X"], b["dY"], b["dWp"], None, 0, None, b["wsw"], b["nw"])
        if kt:
            kt.disarm()

    for w in range(args.warmup):
        step(sets[w % n_sets])
    torch.cuda.synchronize()
    K = args.steps
    kt = KernelTimer(torch, aa, K, len(calls))
    a, b = _ev(torch), _ev(torch)
    torch.cuda.synchronize()
    a.record()
    for s_ in range(K):
        step(sets[s_ % n_sets], kt, s_)
    b.record()
    torch.cuda.synchronize()
    ms_step = a.elapsed_time(b) / K
    dims = {n: (di, do) for n, di, do in shapes}
    parts = {}
    for c, (n, kind) in enumerate(calls):
        ms = kt.ms(c)
        di, do = dims[n]
        tkey = f"{'bwd_data' if kind == 'dX' else 'bwd_weight'}_{which}" if len(shapes) == 1 else None
        parts[f"{n}_{kind}"] = {"ms": round(ms, 5), **kt.spread(c),
                                "roofline": roofline(2 * (M * di + di * do + M * do), ms,
                                                     traffic_for(tkey) if tkey else None),
                                "exec_tflops": round(exec_flops(M, di, do, "Qq", q) / (ms * 1e-3) / 1e12, 2)}
    dense_flops = sum(2 * 2.0 * M * di * do for _, di, do in shapes)
    dense = None
    if not args.no_dense:
        t_total = 0.0
        dense = {"kind": "torch.mm bf16 (hipBLASLt), dY W^T and X^T dY, hot cache, same run"}
        for n, di, do in shapes:
            b0 = sets[0][n]
            Wd = inp.gaussian((di, do), 997, di ** -0.5, torch.bfloat16, dev)
            t_dx = dense_timer(torch, lambda: torch.mm(b0["dY"], Wd.t()))
            t_dw = dense_timer(torch, lambda: torch.mm(b0["X"].t(), b0["dY"]))
            dense[f"{n}_dX_ms"], dense[f"{n}_dW_ms"] = round(t_dx, 5), round(t_dw, 5)
            t_total += t_dx + t_dw
            del Wd
        dense["step_ms"] = round(t_total, 5)
        dense["speedup_step"] = round(t_total / ms_step, 3)
    big = max(parts.items(), key=lambda kv: kv[1]["ms"])
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_backward(args, torch, inp, sets[0], shapes, q, M)
    return {"metric": f"dense-equiv TFLOP/s + % roofline, {which} (dX and dW of each projection) bf16",
            "value": round(dense_flops / (ms_step * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
            "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": which, "M": M, "q": q, "law": "Qq", "type_map": "pos mod q",
                       "projections": [{"name": n, "d_in": di, "d_out": do} for n, di, do in shapes],
                       "input_sets": n_sets, "cache": "flushed (rotating input sets)"},
            "roofline": big[1]["roofline"], "roofline_kernel": big[0], "parts": parts, "dense": dense,
            "timing": "parts: kernel dispatch events of each call (its main kernel and partial-sum reduction); "
                      "ms_per_step: events around the K steps",
            "cpu_baseline": cpu, "kernel_source": kernel_source_hash()}


def cpu_baseline_backward(args, torch, inp, st, shapes, q, M):
    """The fp64 oracle's gradients on the host, on a bounded sample: the rows
    of the first s row types of every projection (dX of those rows and their
    contribution to dW), s grown to about --cpu-seconds of work.  Reported in
    the metric's unit (dense-equivalent TFLOP/s of the sampled rows)."""
    import numpy as np
    import oracle
    host = {}
    for j, (n, di, do) in enumerate(shapes):
        W = inp.gaussian((di, do), 1000 + 10 * j + 1, di ** -0.5, torch.bfloat16, "cuda").float().cpu().numpy()
        host[n] = (st[n]["X"].float().cpu().numpy(), st[n]["dY"].float().cpu().numpy(), W)
    types = oracle.types_pos_mod(M, q)

    def sample(s):
        rows = np.nonzero(types < s)[0]
        for n, _, _ in shapes:
            X, dY, W = host[n]
            oracle.project_grad_input(dY[rows], W, "Qq", q, types[rows])
            oracle.project_grad_weight(X[rows], dY[rows], "Qq", q, types[rows])
        return len(rows)

    def run():
        t0 = time.perf_counter()
        sample(1)
        t_one = time.perf_counter() - t0
        s = int(max(1, min(q, args.cpu_seconds / max(t_one, 1e-6))))
        t0 = time.perf_counter()
        n = sample(s)
        return s, n, time.perf_counter() - t0

    (s, n, t), used, aff = timed_oracle(run)
    dense = sum(2 * 2.0 * n * di * do for _, di, do in shapes)
    return {"value": round(dense / t / 1e12, 5), "unit": "TFLOP/s", "cores": used, "kind": "oracle",
            "sample": f"dX and dW of rows of row types 0..{s - 1} ({n} of {M} tokens) for every projection, "
                      f"fp64 numpy, {t:.2f} s", "seconds": round(t, 3), "affinity_cores": aff}


def decode_single_token(torch, aa, plan, sets, pos0, n_tok, D, F, q, dense_set=None, reps=20):
    """Generation decode: one new token per call (M = 1), n_tok calls at
    positions pos0, pos0 + 1, ... (one per row type).  Timed eagerly (each
    call launched from the host) and with the n_tok calls of an input set
    captured in one HIP graph and replayed, sets alternating.  Each token
    reads its 2q - 1 weight blocks: 2((2q-1) b_in b_out + d_in + d_out) bytes."""
    xs = [[st["x"][j:j + 1] for j in range(n_tok)] for st in sets]
    ys = [[st["y"][j:j + 1] for j in range(n_tok)] for st in sets]

    def calls(si):
        for j in range(n_tok):
            aa.aa_decode_gemv(plan, xs[si][j], sets[si]["Wp"], ys[si][j], None, pos0 + j)

    for si in range(len(sets)):
        calls(si)
    torch.cuda.synchronize()
    a, b = _ev(torch), _ev(torch)
    a.record()
    for r in range(reps):
        calls(r % len(sets))
    b.record()
    torch.cuda.synchronize()
    eager_us = a.elapsed_time(b) * 1e3 / (reps * n_tok)
    graphs = []
    for si in range(len(sets)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            calls(si)
        graphs.append(g)
    torch.cuda.synchronize()
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    a.record()
    for r in range(reps):
        graphs[r % len(graphs)].replay()
    b.record()
    torch.cuda.synchronize()
    graph_us = a.elapsed_time(b) * 1e3 / (reps * n_tok)
    per_tok = 2 * ((2 * q - 1) * (D // q) * (F // q) + D + F)
    out = {"tokens": n_tok, "eager_us_per_token": round(eager_us, 3), "graph_us_per_token": round(graph_us, 3),
           "bytes_per_token": per_tok, "graph_GBs": round(per_tok / graph_us / 1e3, 1)}
    if dense_set is not None:
        Wdn = torch.empty(D, F, dtype=torch.bfloat16, device=dense_set["X"].device).normal_(0.0, D ** -0.5)
        x1 = dense_set["x"][:1]
        t = dense_timer(torch, lambda: torch.matmul(x1, Wdn), iters=50)
        out["dense_us_per_token"] = round(t * 1e3, 3)
        out["speedup_graph_vs_dense"] = round(t * 1e3 / graph_us, 3)
        del Wdn
    return out


def ffn_single_token(torch, aa, up, down, sets, pos0, n_tok, D, F, q, dense=True, reps=20):
    """Generation-time SwiGLU FFN: one new token per call (M = 1), n_tok calls
    at positions pos0, pos0 + 1, ..., eager and replayed from one HIP graph
    per input set.  A token reads its 2q - 1 blocks of each of the three
    weights: 2(3 (2q-1) b_in b_out + 2 D + 2 F) bytes.  The dense comparator
    is the same FFN with torch.matmul (three GEMVs), also graph-replayed."""
    def calls(si):
        st = sets[si]
        for j in range(n_tok):
            aa.aa_swiglu_ffn_fwd(up, down, st["x"][j:j + 1], st["Wgp"], st["Wup"], st["Wdp"], st["H"][j:j + 1],
                                 st["Y2"][j:j + 1], None, pos0 + j)

    def timed(fn):
        a, b = _ev(torch), _ev(torch)
        a.record()
        for r in range(reps):
            fn(r)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / (reps * n_tok)

    for si in range(len(sets)):
        calls(si)
    torch.cuda.synchronize()
    eager_us = timed(lambda r: calls(r % len(sets)))
    graphs = []
    for si in range(len(sets)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            calls(si)
        graphs.append(g)
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    graph_us = timed(lambda r: graphs[r % len(graphs)].replay())
    per_tok = 2 * (3 * (2 * q - 1) * (D // q) * (F // q) + 2 * D + 2 * F)
    out = {"tokens": n_tok, "eager_us_per_token": round(eager_us, 3), "graph_us_per_token": round(graph_us, 3),
           "bytes_per_token": per_tok, "graph_GBs": round(per_tok / graph_us / 1e3, 1)}
    if dense:
        dev = sets[0]["x"].device
        # two weight sets (about 600 MB) so that replays alternate and the cache is cold
        ws = [[torch.empty(shape, dtype=torch.bfloat16, device=dev).normal_(0.0, shape[0] ** -0.5)
               for shape in ((D, F), (D, F), (F, D))] for _ in range(2)]
        x1 = sets[0]["x"][:1].clone()
        dgs = []
        for Wg, Wu, Wd in ws:
            for _ in range(2):
                torch.matmul(torch.nn.functional.silu(torch.matmul(x1, Wg)) * torch.matmul(x1, Wu), Wd)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                torch.matmul(torch.nn.functional.silu(torch.matmul(x1, Wg)) * torch.matmul(x1, Wu), Wd)
            dgs.append(g)
        for g in dgs:
            g.replay()
        torch.cuda.synchronize()
        t = timed(lambda r: dgs[r % 2].replay()) * n_tok
        out["dense_graph_us_per_token"] = round(t, 3)
        out["speedup_graph_vs_dense"] = round(t / graph_us, 3)
        del ws, dgs
    return out


def cpu_baseline_qwen3(args, torch, inp, st, wl):
    """The fp64 oracle on the host, on a bounded sample of the same step.

    The sample is the rows of the first s row types through the projection
    and the SwiGLU FFN, plus s decode tokens; s grows until the sample is
    about --cpu-seconds of work (the whole step when that is cheaper, then
    repeated).  Reported in the metric's unit, dense-equivalent TFLOP/s."""
    import numpy as np
    import oracle
    M, D, F, q = wl.M, wl.d_in, wl.d_out, wl.q
    X = st["X"].float().cpu().numpy()
    # unpacked weights are regenerated from their seeds (the packed copies are device-only)
    gen = lambda role, shape, fan: inp.gaussian(shape, inp.seed_for(role, 3), fan ** -0.5, torch.bfloat16,
                                                "cuda").float().cpu().numpy()
    W, Wu, Wdn = gen(inp.ROLE_W, (D, F), D), gen(inp.ROLE_WU, (D, F), D), gen(inp.ROLE_WD, (F, D), F)
    # the step's gate weight is its own tensor (seed offset 50, as in the step)
    Wg = inp.gaussian((D, F), inp.seed_for(inp.ROLE_W, 3) + 50, D ** -0.5, torch.bfloat16,
                      "cuda").float().cpu().numpy()
    types = oracle.types_pos_mod(M, q)

    def sample(s):
        rows = np.nonzero(types < s)[0]
        oracle.project(X[rows], W, "Qq", q, types[rows])
        oracle.swiglu_ffn(X[rows], Wg, Wu, Wdn, "Qq", q, types[rows])
        oracle.decode(X[:s], W, "Qq", q, np.arange(s))
        return len(rows)

    def run():
        t0 = time.perf_counter()
        sample(1)
        t_one = time.perf_counter() - t0
        s = int(max(1, min(q, args.cpu_seconds / max(t_one, 1e-6))))
        reps = 1
        t0 = time.perf_counter()
        n = sample(s)
        t = time.perf_counter() - t0
        if s == q and t < args.cpu_seconds / 2:
            reps = max(1, int(args.cpu_seconds / max(t, 1e-6)))
            t0 = time.perf_counter()
            for _ in range(reps):
                sample(s)
            t = (time.perf_counter() - t0) / reps
        return s, n, t, reps

    (s, n, t, reps), used, aff = timed_oracle(run)
    dense = 2.0 * n * D * F * 4 + 2.0 * s * D * F
    return {"value": round(dense / t / 1e12, 5), "unit": "TFLOP/s", "cores": used, "kind": "oracle",
            "sample": f"rows of row types 0..{s - 1} ({n} of {M} tokens) through the projection and the SwiGLU "
                      f"FFN plus {s} decode tokens, fp64 numpy, {t:.2f} s per pass, {reps} pass(es)",
            "seconds": round(t * reps, 3), "affinity_cores": aff}


# ----------------------------------------------------- other workloads ------

def projection_part(torch, inp, aa, dev, wl, steps, warmup, dense=True):
    """One row-typed projection shape (position typing) as a part of the
    default line: two input sets alternate (flushed cache when a set exceeds
    the 256 MB Infinity Cache), each call timed by its kernel dispatch events."""
    M, D, F, q = wl.M, wl.d_in, wl.d_out, wl.q
    plan = aa.aa_plan_create(wl.law, q, D, F, "pos_mod", 0, "bf16", "bf16")
    per_set = proj_bytes(M, D, F)
    sets = []
    for s_ in range(2):
        X = inp.gaussian((M, D), inp.seed_for(inp.ROLE_X, wl.index) + 100 * s_, 1.0, torch.bfloat16, dev)
        W = inp.gaussian((D, F), inp.seed_for(inp.ROLE_W, wl.index) + 100 * s_, D ** -0.5, torch.bfloat16, dev)
        sets.append((X, aa.pack(plan, W), torch.empty(M, F, dtype=torch.bfloat16, device=dev)))
        del W
    for w in range(warmup):
        aa.aa_project_fwd(plan, *sets[w % 2])
    torch.cuda.synchronize()
    kt = KernelTimer(torch, aa, steps, 1)
    for s_ in range(steps):
        kt.arm(s_, 0)
        aa.aa_project_fwd(plan, *sets[s_ % 2])
    kt.disarm()
    torch.cuda.synchronize()
    ms = kt.ms(0)
    part = {"workload": f"{wl.name}: {wl.notes}", "M": M, "d_in": D, "d_out": F, "q": q,
            "layout": aa.aa_packed_layout_version(plan), "steps": steps, "ms": round(ms, 5), **kt.spread(0),
            "dense_equiv_tflops": round(2.0 * M * D * F / ms / 1e9, 2),
            "exec_tflops": round(exec_flops(M, D, F, wl.law, q) / ms / 1e9, 2),
            "roofline": roofline(per_set, ms, traffic_for(f"project_{wl.name}"))}
    if dense:
        Wd = inp.gaussian((D, F), 999, D ** -0.5, torch.bfloat16, dev)
        X0 = sets[0][0]
        t = dense_timer(torch, lambda: torch.matmul(X0, Wd), iters=5, warm=2)
        part["dense"] = {"kind": "torch.matmul bf16 (hipBLASLt), same run", "ms": round(t, 4),
                         "speedup": round(t / ms, 3)}
        del Wd
    del sets
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return part


def square_part(torch, inp, aa, dev, steps, warmup, dense=True):
    """Fixed-block square product n = 32768, b = 128, q = 256 (block-row
    typing): K launches on one resident input set (6.4 GB, far above the 256
    MB Infinity Cache), each timed by its own kernel dispatch events."""
    n, q = 32768, 256
    plan = aa.aa_plan_create("Qq", q, n, n, "block_rows", 0, "bf16", "bf16")
    X = inp.gaussian((n, n), inp.seed_for(inp.ROLE_X, 5), 1.0, torch.bfloat16, dev)
    W = inp.gaussian((n, n), inp.seed_for(inp.ROLE_W, 5), n ** -0.5, torch.bfloat16, dev)
    Wp = aa.pack(plan, W)
    del W
    Y = torch.empty(n, n, dtype=torch.bfloat16, device=dev)
    for _ in range(warmup):
        aa.aa_project_fwd(plan, X, Wp, Y)
    torch.cuda.synchronize()
    kt = KernelTimer(torch, aa, steps, 1)
    a, b = _ev(torch), _ev(torch)
    a.record()
    for s_ in range(steps):
        kt.arm(s_, 0)
        aa.aa_project_fwd(plan, X, Wp, Y)
    kt.disarm()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    ms_k = kt.ms(0)
    dense_fl = 2.0 * n ** 3
    part = {"workload": "square_n32768_b128_q256: full X * W, every block-row, block-row typing", "n": n, "q": q,
            "steps": steps, "ms": round(ms_k, 5), **kt.spread(0), "ms_per_call": round(ms, 5),
            "dense_equiv_tflops": round(dense_fl / ms_k / 1e9, 2),
            "exec_tflops": round(exec_flops(n, n, n, "Qq", q) / ms_k / 1e9, 2),
            "roofline": roofline(proj_bytes(n, n, n), ms_k, traffic_for("project_square_n32768"))}
    if dense:
        del Wp
        Wd = inp.gaussian((n, n), 999, n ** -0.5, torch.bfloat16, dev)
        t = dense_timer(torch, lambda: torch.matmul(X, Wd), iters=3, warm=1)
        part["dense"] = {"kind": "torch.matmul bf16 (hipBLASLt), same run", "ms": round(t, 4),
                         "speedup": round(t / ms_k, 3)}
        del Wd
    del X, Y
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return part


def bench_square(args, torch, inp, aa, dev):
    """The square product as its own workload (one JSON line)."""
    part = square_part(torch, inp, aa, dev, args.steps, args.warmup, not args.no_dense)
    return {"metric": "dense-equiv TFLOP/s + % roofline, square n=32768 b=128 q=256 bf16",
            "value": round(2.0 * part["n"] ** 3 / part["ms_per_call"] / 1e9, 2), "unit": "TFLOP/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": part["ms_per_call"],
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "square_n32768_b128_q256", "n": part["n"], "q": part["q"], "law": "Qq",
                       "type_map": "block rows"},
            "roofline": part["roofline"], "kernel_ms": part["ms"],
            "kernel_spread": {k: part[k] for k in ("median_ms", "p10_ms", "p90_ms", "samples")},
            "exec_tflops": part["exec_tflops"], "dense": part.get("dense"), "kernel_source": kernel_source_hash()}


def ffn_part(torch, inp, aa, dev, which, steps, warmup, dense=True):
    """SwiGLU FFN forward (gate/up launch + down launch) at the pilot
    (Q2 x Q2, M = 12288, 768 -> 1536 -> 768) or the Qwen3-30B-A3B expert
    (Q_16, M = 2048, 2048 -> 768 -> 2048) shape.  Input sets of at least 1 GB
    rotate between calls (flushed cache); each call is timed by its kernels'
    dispatch events.  The pilot FFN is bound by the bf16 MFMA rate (its
    executed FLOPs over its bytes exceed the chip's FLOP/byte balance), the
    expert FFN by HBM."""
    wl = inp.WORKLOADS[2 if which == "pilot_ffn" else 4]
    M, D, F, q, law = wl.M, wl.d_in, wl.d_out, wl.q, wl.law
    period = wl.extra.get("period", 0)
    up = aa.aa_plan_create(law, q, D, F, "pos_mod", period, "bf16", "bf16")
    down = aa.aa_plan_create(law, q, F, D, "pos_mod", period, "bf16", "bf16")
    set_bytes = 2 * (M * D + 3 * D * F + M * F + M * D)
    n_sets = max(2, math.ceil(1.0e9 / set_bytes))
    sets = []
    for s_ in range(n_sets):
        off = 100 * s_
        g = lambda role, shape, fan: inp.gaussian(shape, inp.seed_for(role, wl.index) + off, fan ** -0.5,
                                                  torch.bfloat16, dev)
        sets.append({"X": inp.gaussian((M, D), inp.seed_for(inp.ROLE_X, wl.index) + off, 1.0, torch.bfloat16, dev),
                     "Wg": aa.pack(up, g(inp.ROLE_W, (D, F), D)), "Wu": aa.pack(up, g(inp.ROLE_WU, (D, F), D)),
                     "Wd": aa.pack(down, g(inp.ROLE_WD, (F, D), F)),
                     "H": torch.empty(M, F, dtype=torch.bfloat16, device=dev),
                     "Y": torch.empty(M, D, dtype=torch.bfloat16, device=dev)})
    call = lambda st: aa.aa_swiglu_ffn_fwd(up, down, st["X"], st["Wg"], st["Wu"], st["Wd"], st["H"], st["Y"])
    for w in range(warmup):
        call(sets[w % n_sets])
    torch.cuda.synchronize()
    kt = KernelTimer(torch, aa, steps, 1)
    a, b = _ev(torch), _ev(torch)
    a.record()
    for s_ in range(steps):
        kt.arm(s_, 0)
        call(sets[s_ % n_sets])
    kt.disarm()
    b.record()
    torch.cuda.synchronize()
    ms_call = a.elapsed_time(b) / steps
    ms = kt.ms(0)
    dense_fl = 3 * 2.0 * M * D * F
    ex = 3 * exec_flops(M, D, F, law, q)
    by = 2 * (M * D + 2 * D * F + M * F) + 2 * (M * F + F * D + M * D)
    mfma = {"bound": "mfma", "achieved": round(ex / ms / 1e9, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ex / ms / 1e9 / BF16_PEAK_TFLOPS, 4), "traffic": None}
    hbm = roofline(by, ms)
    pilot = which == "pilot_ffn"
    part = {"workload": f"{wl.name}: SwiGLU FFN forward (gate/up + down), {wl.notes}", "M": M, "D": D, "F": F,
            "q": q, "law": law, "input_sets": n_sets, "steps": steps, "ms": round(ms, 5), **kt.spread(0),
            "ms_per_call": round(ms_call, 5), "dense_equiv_tflops": round(dense_fl / ms / 1e9, 2),
            "exec_tflops": round(ex / ms / 1e9, 2),
            "roofline": mfma if pilot else hbm, "roofline_other": hbm if pilot else mfma}
    if dense:
        X = sets[0]["X"]
        Wd1 = inp.gaussian((D, F), 999, D ** -0.5, torch.bfloat16, dev)
        Wd2 = inp.gaussian((D, F), 998, D ** -0.5, torch.bfloat16, dev)
        Wd3 = inp.gaussian((F, D), 997, F ** -0.5, torch.bfloat16, dev)
        t = dense_timer(torch, lambda: torch.matmul(
            torch.nn.functional.silu(torch.matmul(X, Wd1)) * torch.matmul(X, Wd2), Wd3))
        part["dense"] = {"kind": "torch.matmul bf16 x3 + silu*mul (hipBLASLt), hot cache, same run",
                         "ms": round(t, 5), "speedup": round(t / ms, 3)}
        del Wd1, Wd2, Wd3
    del sets
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return part


def bench_ffn(args, torch, inp, aa, dev, which):
    """One FFN workload as its own JSON line."""
    part = ffn_part(torch, inp, aa, dev, which, args.steps, args.warmup, not args.no_dense)
    wl = inp.WORKLOADS[2 if which == "pilot_ffn" else 4]
    return {"metric": f"dense-equiv TFLOP/s, {wl.name} SwiGLU forward bf16",
            "value": round(3 * 2.0 * part["M"] * part["D"] * part["F"] / part["ms_per_call"] / 1e9, 2),
            "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": part["ms_per_call"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16", "data": "synthetic",
            "config": {"workload": wl.name, "M": part["M"], "D": part["D"], "F": part["F"], "q": part["q"],
                       "law": part["law"], "input_sets": part["input_sets"]},
            "kernel_ms": part["ms"], "exec_tflops": part["exec_tflops"], "roofline": part["roofline"],
            "roofline_other": part["roofline_other"], "dense": part.get("dense"),
            "kernel_source": kernel_source_hash()}


STACK_LAYERS = 12   # decoder blocks of the 110M pilot model


def decode_stack_weights(torch, inp, aa, up, down, D, F, dev):
    """Seeded synthetic weights of the FFN stack, packed: one (gate, up,
    down) triple per layer, N(0, 1/fan_in)."""
    wl = inp.WORKLOADS[2]
    out = []
    for layer in range(STACK_LAYERS):
        off = 10 * (layer + 1)
        out.append((aa.pack(up, inp.gaussian((D, F), inp.seed_for(inp.ROLE_W, wl.index) + off, D ** -0.5,
                                             torch.bfloat16, dev)),
                    aa.pack(up, inp.gaussian((D, F), inp.seed_for(inp.ROLE_WU, wl.index) + off, D ** -0.5,
                                             torch.bfloat16, dev)),
                    aa.pack(down, inp.gaussian((F, D), inp.seed_for(inp.ROLE_WD, wl.index) + off, F ** -0.5,
                                               torch.bfloat16, dev))))
    return out


def bench_decode_stack(args, torch, inp, aa, dev):
    """Fixed-length generation through the FFN stack of the 110M pilot model
    (12 blocks, width 768, SwiGLU 1536, Q2xQ2 law, context 1536): one new
    token per call, each token through all 12 FFNs in turn (layer l reads
    layer l - 1's output).  Attention, norms, the LM head and sampling are not
    in this path, so the rate is that of the FFN share of decoding only.  A
    HIP graph holds q = 4 consecutive tokens (every row type once; with the
    context a multiple of q the same graph serves every later group of 4
    positions) and is replayed for the whole length.  The dense comparator
    is the same stack with torch.matmul (three GEMVs and silu * mul per
    layer), one token per graph, replayed as often."""
    wl = inp.WORKLOADS[2]
    D, F, q, law = wl.d_in, wl.d_out, wl.q, wl.law
    period = wl.extra.get("period", 0)
    L = 256   # generated tokens per timed step
    up = aa.aa_plan_create(law, q, D, F, "pos_mod", period, "bf16", "bf16")
    down = aa.aa_plan_create(law, q, F, D, "pos_mod", period, "bf16", "bf16")
    W = decode_stack_weights(torch, inp, aa, up, down, D, F, dev)
    x = inp.gaussian((q, D), inp.seed_for(inp.ROLE_X, wl.index), 1.0, torch.bfloat16, dev)
    H = torch.empty(q, F, dtype=torch.bfloat16, device=dev)
    Ys = [torch.empty(q, D, dtype=torch.bfloat16, device=dev) for _ in range(STACK_LAYERS)]

    def tokens():   # positions 0 .. q - 1, one call per token and layer
        for j in range(q):
            src = x[j:j + 1]
            for layer, (g, u, d) in enumerate(W):
                aa.aa_swiglu_ffn_fwd(up, down, src, g, u, d, H[j:j + 1], Ys[layer][j:j + 1], None, j)
                src = Ys[layer][j:j + 1]

    for _ in range(3):
        tokens()
    torch.cuda.synchronize()
    reps = L // q
    a, b = _ev(torch), _ev(torch)
    a.record()
    for _ in range(reps):
        tokens()
    b.record()
    torch.cuda.synchronize()
    eager_us = a.elapsed_time(b) * 1e3 / L
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        tokens()
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    K = args.steps
    a.record()
    for _ in range(K):
        for _ in range(reps):
            g.replay()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / K            # one step = L tokens
    us_tok = ms * 1e3 / L
    # a token reads its row type's 9 of the 16 blocks of each of the 36 weights
    per_tok = STACK_LAYERS * 2 * (3 * 9 * (D // q) * (F // q) + 2 * D + 2 * F)
    res = {"metric": "FFN-stack decode tokens/s, pilot 110M shape (12 SwiGLU blocks, Q2xQ2), no attention",
           "value": round(L / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
           "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "pilot_decode_stack", "layers": STACK_LAYERS, "D": D, "F": F, "q": q,
                      "law": law, "period": period, "tokens_per_step": L, "batch": 1,
                      "graph": f"{q} tokens x {STACK_LAYERS} layers per replay"},
           "us_per_token": round(us_tok, 3), "eager_us_per_token": round(eager_us, 3),
           "bytes_per_token": per_tok, "GBs": round(per_tok / us_tok / 1e3, 1),
           "weights_resident": f"{STACK_LAYERS * 3 * D * F * 2 / 1e6:.0f} MB of weights, inside the 256 MB "
                               "Infinity Cache across tokens",
           "kernel_source": kernel_source_hash()}
    if not args.no_dense:
        dw = [[torch.empty(shape, dtype=torch.bfloat16, device=dev).normal_(0.0, shape[0] ** -0.5)
               for shape in ((D, F), (D, F), (F, D))] for _ in range(STACK_LAYERS)]
        x1 = x[:1].clone()

        def dense_token():
            h = x1
            for Wg, Wu, Wd in dw:
                h = torch.matmul(torch.nn.functional.silu(torch.matmul(h, Wg)) * torch.matmul(h, Wu), Wd)
            return h

        for _ in range(3):
            dense_token()
        torch.cuda.synchronize()
        dg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(dg):
            dense_token()
        for _ in range(3):
            dg.replay()
        torch.cuda.synchronize()
        a.record()
        for _ in range(L):
            dg.replay()
        b.record()
        torch.cuda.synchronize()
        dense_us = a.elapsed_time(b) * 1e3 / L
        res["dense"] = {"kind": "torch.matmul bf16, 3 GEMVs + silu*mul per layer, one token per HIP graph",
                        "us_per_token": round(dense_us, 3), "tokens_per_s": round(1e6 / dense_us, 1),
                        "speedup": round(dense_us / us_tok, 3)}
        del dw
    return res


def generate_timing(torch, gen, prompt, n_new, reps):
    """Fixed-length generation: the prompt in one prefill pass, then n_new
    decode steps, each replayed from one HIP graph of a decode step (device
    position, so one graph serves every position).  Returns (prefill ms,
    decode ms per token), medians over reps sequences."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gen.prefill(prompt)
        for _ in range(3):
            gen.decode_step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gen.decode_step()
    pre, dec = [], []
    for _ in range(reps + 1):
        a, b, c = _ev(torch), _ev(torch), _ev(torch)
        a.record()
        gen.prefill(prompt)
        b.record()
        for _ in range(n_new):
            g.replay()
        c.record()
        torch.cuda.synchronize()
        pre.append(a.elapsed_time(b))
        dec.append(b.elapsed_time(c) / n_new)
    med = lambda v: sorted(v[1:])[len(v[1:]) // 2]   # the first sequence warms up
    del g
    return med(pre), med(dec)


def bench_generate(args, torch, aa, dev):
    """Fixed-length greedy generation with a decoder stack shaped like the
    pilot 110M model (12 layers, width 768, 32 heads, context 1536, GPT-2
    vocabulary, tied LM head, 110,631,168 parameters), once with a dense
    SwiGLU FFN (torch.matmul) and once with the algebra FFN (Q2 x Q2 through
    aa_swiglu_ffn_fwd), on the same synthetic weights: a 128-token prompt and
    256 new tokens per sequence, batch 1 and batch 8.  Attention over the KV
    cache, LayerNorms, the LM head and argmax run in torch in both models.
    value = the algebra model's decode tokens/s at batch 1."""
    from associative_algebra_block_amd.pilot_stack import PilotConfig, PilotGenerator, make_weights
    cfg = PilotConfig()
    w = make_weights(cfg, 0, dev)
    P, G, reps = 128, 256, max(3, min(args.steps, 10))
    runs = {}
    for B in (1, 8):
        g = torch.Generator(device="cpu")
        g.manual_seed(7 + B)
        prompt = torch.randint(0, cfg.vocab, (B, P), generator=g).to(dev)
        for ffn in ("dense", "algebra"):
            gen = PilotGenerator(cfg, w, ffn, B, dev)
            pre, dec = generate_timing(torch, gen, prompt, G, reps)
            runs[(B, ffn)] = {"prefill_ms": round(pre, 4), "decode_ms_per_step": round(dec, 5),
                              "decode_tokens_per_s": round(B / (dec * 1e-3), 1),
                              "sequence_tokens_per_s": round(B * G / ((pre + G * dec) * 1e-3), 1)}
            del gen
            torch.cuda.synchronize()
    out = {}
    for B in (1, 8):
        d, a = runs[(B, "dense")], runs[(B, "algebra")]
        out[f"batch{B}"] = {"dense_ffn": d, "algebra_ffn": a,
                            "decode_speedup": round(a["decode_tokens_per_s"] / d["decode_tokens_per_s"], 4),
                            "sequence_speedup": round(a["sequence_tokens_per_s"] / d["sequence_tokens_per_s"], 4),
                            "prefill_speedup": round(d["prefill_ms"] / a["prefill_ms"], 4)}
    a1 = runs[(1, "algebra")]
    return {"metric": "fixed-length generation tokens/s, pilot 110M-shaped decoder, algebra FFN vs dense FFN",
            "value": a1["decode_tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": reps,
            "warmup": 1, "ms_per_step": a1["decode_ms_per_step"], "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded random weights and prompts)",
            "config": {"workload": "pilot_generate", "layers": cfg.layers, "d": cfg.d, "heads": cfg.heads,
                       "ffn": cfg.ffn, "ctx": cfg.ctx, "vocab": cfg.vocab, "params": cfg.parameter_count(),
                       "law": "Q2xQ2", "prompt": P, "new_tokens": G, "batches": [1, 8],
                       "decode": "one HIP graph per decode step, replayed"},
            "runs": out,
            "pages": "generation gain of the pilot models: +6.2 to +7.8% tokens/s (tokenization and sampling "
                     "included, hardware not stated)",
            "kernel_source": kernel_source_hash()}


if __name__ == "__main__":
    main()
