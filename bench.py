"""Benchmark of the stitched / GEMM-fused hot path on one MI355X.

One step = one call of each of the five fused entry points (the whole hot
path) on its workload, inputs resident in HBM.  Each call is bracketed by HIP
events on the stream it runs on, with a 512 MiB cache-evicting read sweep
before it (outside the events) so every call reads its inputs from HBM.  The headline
line reports the tall-skinny LayerNorm workload (750000 x 32 fp32); the other
four workloads are reported under "per_config" in the same line, and so are
the back-to-back GEMM with the softmax between (8192 x 8192 x 128 x 128),
RMSNorm and affine LayerNorm (750000 x 32 fp32), which are timed per kernel
but are not part of the step.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only NAME]
                       [--no-unfused] [--no-cpu] [--calibrate-copy]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
METRIC = "effective HBM GB/s per stitched subgraph; TFLOP/s for fused GEMM+LN/softmax"
HEADLINE = "layernorm_750000x32"
FLUSH_BYTES = 512 << 20
# Bytes of other traffic between two timed uses of one buffer set: three times
# the 256 MB infinity cache, so no timed call finds its data in a cache.
ROTATE_BYTES = 768 << 20
# Back-to-back launches per workload in the per-kernel timing loop.
LAUNCHES_PER_KERNEL = 60
# Source files that define each workload's fused kernel; a stored hardware
# byte count is reported only while these files and the launch plan are unchanged.
KERNEL_SOURCES = {
    "softmax_256x1024": ("stitch.hip", "dev.hpp"),
    "layernorm_750000x32": ("stitch.hip", "dev.hpp"),
    "pow_bcast_add_softmax_64x30000": ("stitch.hip", "dev.hpp"),
    "gemm_ln_4096x4096x1024": ("gemm.hip", "dev.hpp"),
    "gemm_softmax_8192x8192x128": ("gemm.hip", "dev.hpp"),
    "gemm_softmax_gemm_8192x8192x128x128": ("gemm.hip", "dev.hpp"),
    "rmsnorm_750000x32": ("stitch.hip", "dev.hpp"),
    "layernorm_affine_750000x32": ("stitch.hip", "dev.hpp"),
    "gemm_gelu_4096x4096x1024": ("gemm.hip", "dev.hpp"),
    "auto_layernorm_750000x32": ("auto.cpp",),
    "auto_silu_ln_scaled_750000x32": ("auto.cpp",),
    "auto_softmax_512x65536": ("auto.cpp",),
}


def source_hash(workload: str, plan: dict | None = None) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[workload]:
        with open(os.path.join(ROOT, "broadcast_subgraphs_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if plan is not None:
        h.update(json.dumps(plan, sort_keys=True).encode())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", default=None, help="run one workload only (for profiling)")
    ap.add_argument("--no-unfused", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-flush", action="store_true")
    ap.add_argument("--flush", choices=["read", "write"], default="read",
                    help="evict caches before each timed call by reading (default) or writing 512 MiB")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run the 256 MiB copy kernel (hardware byte-counter calibration)")
    return ap.parse_args()


# ------------------------------------------------------------------ workloads

class Workload:
    """Inputs, outputs and the fused / unfused calls of one workload.

    The fused call is available on `copies` independent sets of device buffers
    (`fused_on(i)`), enough that at least ROTATE_BYTES of other traffic passes
    between two uses of one set: rotating through them keeps every timed call's
    inputs and outputs out of the caches without a flush kernel in between.
    """

    def __init__(self, name, torch, cf, gen):
        self.name = name
        self.torch = torch
        dev = "cuda"
        d32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
        dbf = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).to(dev).view(torch.bfloat16)
        if name == "softmax_256x1024":
            x = gen.softmax_inputs(seed=1)["x"]
            self.inp = {"x": x}
            bufs = {"X": d32(x), "Y": torch.empty(256, 1024, device=dev)}
            self.bytes, self.flops = 2 * x.nbytes, 0
            call = lambda b, ws, u: cf.cf_stitch_softmax(b["X"], b["Y"], ws=ws, unfused=u)
            self.op, self.dims = cf.CF_OP_STITCH_SOFTMAX, (256, 1024, 0)
        elif name == "layernorm_750000x32":
            x = gen.layernorm_inputs(seed=2)["x"]
            self.inp = {"x": x}
            bufs = {"X": d32(x), "Y": torch.empty(750000, 32, device=dev)}
            self.bytes, self.flops = 2 * x.nbytes, 0
            call = lambda b, ws, u: cf.cf_stitch_layernorm(b["X"], b["Y"], 1e-5, ws=ws, unfused=u)
            self.op, self.dims = cf.CF_OP_STITCH_LAYERNORM, (750000, 32, 0)
        elif name == "pow_bcast_add_softmax_64x30000":
            d = gen.pow_bcast_add_inputs(seed=3)
            self.inp = d
            bufs = {"X": d32(d["x"]), "V": d32(d["v"]), "Y": torch.empty(64, 30000, device=dev)}
            self.bytes, self.flops = 2 * d["x"].nbytes + d["v"].nbytes, 0
            call = lambda b, ws, u: cf.cf_stitch_pow_bcast_add(b["X"], b["V"], 1.5, b["Y"], None, ws=ws, unfused=u)
            self.op, self.dims = cf.CF_OP_STITCH_POW_BCAST_ADD, (64, 30000, 0)
        elif name == "gemm_ln_4096x4096x1024":
            M, N, K = 4096, 4096, 1024
            d = gen.gemm_ln_inputs(seed=4)
            self.inp = d
            bufs = {"A": dbf(d["a_bits"]), "W": dbf(d["w_bits"]), "R": dbf(d["r_bits"]), "bias": d32(d["bias"]),
                    "gamma": d32(d["gamma"]), "beta": d32(d["beta"]),
                    "Y": torch.empty(M, N, dtype=torch.bfloat16, device=dev)}
            self.bytes = 2 * (M * K + K * N + 2 * M * N) + 4 * 3 * N
            self.flops = 2 * M * N * K
            call = lambda b, ws, u: cf.cf_gemm_ln(b["A"], b["W"], b["bias"], b["R"], b["gamma"], b["beta"], b["Y"],
                                                  1e-5, ws=ws, unfused=u)
            self.op, self.dims = cf.CF_OP_GEMM_LN, (M, N, K)
        elif name == "gemm_softmax_8192x8192x128":
            M, N, D = 8192, 8192, 128
            d = gen.gemm_softmax_inputs(seed=5)
            self.inp = d
            bufs = {"Q": dbf(d["q_bits"]), "K": dbf(d["k_bits"]), "S": torch.empty(M, N, dtype=torch.bfloat16, device=dev)}
            self.bytes = 2 * (M * D + N * D + M * N)
            self.flops = 2 * M * N * D
            scale = d["scale"]
            call = lambda b, ws, u: cf.cf_gemm_softmax(b["Q"], b["K"], scale, b["S"], ws=ws, unfused=u)
            self.op, self.dims = cf.CF_OP_GEMM_SOFTMAX, (M, N, D)
        elif name == "gemm_softmax_gemm_8192x8192x128x128":
            M, N, D, Dv = 8192, 8192, 128, 128
            d = gen.gemm_softmax_gemm_inputs(seed=6)
            self.inp = d
            bufs = {"Q": dbf(d["q_bits"]), "K": dbf(d["k_bits"]), "V": dbf(d["v_bits"]),
                    "Y": torch.empty(M, Dv, dtype=torch.bfloat16, device=dev)}
            self.bytes = 2 * (M * D + N * D + N * Dv + M * Dv)
            self.flops = 2 * M * N * D + 2 * M * N * Dv
            scale = d["scale"]
            call = lambda b, ws, u: cf.cf_gemm_softmax_gemm(b["Q"], b["K"], b["V"], scale, b["Y"], ws=ws, unfused=u)
            self.op, self.dims = cf.CF_OP_GEMM_SOFTMAX_GEMM, (M, N, D)
        elif name == "rmsnorm_750000x32":
            d = gen.rmsnorm_inputs(seed=7)
            self.inp = d
            bufs = {"X": d32(d["x"]), "G": d32(d["gamma"]), "Y": torch.empty(750000, 32, device=dev)}
            self.bytes, self.flops = 2 * d["x"].nbytes + d["gamma"].nbytes, 0
            call = lambda b, ws, u: cf.cf_stitch_rmsnorm(b["X"], b["G"], b["Y"], 1e-5, ws=ws, unfused=u)
            self.op, self.dims = cf.CF_OP_STITCH_RMSNORM, (750000, 32, 0)
        elif name == "layernorm_affine_750000x32":
            d = gen.layernorm_affine_inputs(seed=8)
            self.inp = d
            bufs = {"X": d32(d["x"]), "G": d32(d["gamma"]), "B": d32(d["beta"]),
                    "Y": torch.empty(750000, 32, device=dev)}
            self.bytes, self.flops = 2 * d["x"].nbytes + d["gamma"].nbytes + d["beta"].nbytes, 0
            call = lambda b, ws, u: cf.cf_stitch_layernorm_affine(b["X"], b["G"], b["B"], b["Y"], 1e-5, ws=ws,
                                                                  unfused=u)
            self.op, self.dims = cf.CF_OP_STITCH_LAYERNORM_AFFINE, (750000, 32, 0)
        elif name == "gemm_gelu_4096x4096x1024":
            M, N, K = 4096, 4096, 1024
            d = gen.gemm_act_inputs(seed=9)
            self.inp = d
            bufs = {"A": dbf(d["a_bits"]), "W": dbf(d["w_bits"]), "bias": d32(d["bias"]),
                    "Y": torch.empty(M, N, dtype=torch.bfloat16, device=dev)}
            self.bytes = 2 * (M * K + K * N + M * N) + 4 * N
            self.flops = 2 * M * N * K
            call = lambda b, ws, u: cf.cf_gemm_act(b["A"], b["W"], b["bias"], "gelu_tanh", b["Y"], ws=ws, unfused=u)
            self.op, self.dims = cf.CF_OP_GEMM_ACT, (M, N, K)
        elif name in ("auto_layernorm_750000x32", "auto_silu_ln_scaled_750000x32"):
            # the same subgraph as a captured graph, stitched automatically into
            # a generated kernel (and a graph outside the library's stage DAGs)
            d = gen.layernorm_affine_inputs(seed=10)
            v = gen.uniform(10, 5, (750000,), 0.1, 2.0)
            self.inp = {"x": d["x"], "beta": d["beta"], "v": v}
            g = cf.Graph()
            x = g.input(0)
            u = g.op("add", g.op("silu", x), g.rowvec(1)) if name.startswith("auto_silu") else x
            mu = g.op("div", g.op("rowsum", u), g.const(32))
            c = g.op("sub", u, mu)
            var = g.op("div", g.op("rowsum", g.op("square", c)), g.const(32))
            y = g.op("mul", c, g.op("rsqrt", g.op("add", var, g.const(1e-5))))
            if name.startswith("auto_silu"):
                y = g.op("mul", y, g.colvec(2))
            self.graph = (g.nodes, y)
            auto = cf.Auto(g, y, 750000, 32)
            self.plan_auto = auto.describe()
            bufs = {"X": d32(d["x"]), "B": d32(d["beta"]), "V": d32(v), "Y": torch.empty(750000, 32, device=dev)}
            extra = 0 if name.startswith("auto_layernorm") else d["beta"].nbytes + v.nbytes
            self.bytes, self.flops = 2 * d["x"].nbytes + extra, 0
            call = lambda b, ws, u: auto.launch([b["X"], b["B"], b["V"]], b["Y"])
            self.op, self.dims = None, (750000, 32, 0)
        elif name == "auto_softmax_512x65536":
            # rows of 65536 values: the generated kernel's Global scheme (8 member
            # workgroups per row joining at both reductions)
            x = gen.softmax_inputs(seed=11, rows=512, cols=1 << 16)["x"]
            self.inp = {"x": x}
            g = cf.Graph()
            xi = g.input(0)
            e = g.op("exp", g.op("sub", xi, g.op("rowmax", xi)))
            y = g.op("div", e, g.op("rowsum", e))
            self.graph = (g.nodes, y)
            auto = cf.Auto(g, y, 512, 1 << 16)
            self.plan_auto = auto.describe()
            bufs = {"X": d32(x), "Y": torch.empty(512, 1 << 16, device=dev)}
            self.bytes, self.flops = 2 * x.nbytes, 0
            auto_ws = cf.Workspace(auto.workspace_bytes())
            call = lambda b, ws, u: auto.launch([b["X"]], b["Y"], ws=auto_ws)
            self.op, self.dims = None, (512, 1 << 16, 0)
        else:
            raise ValueError(name)
        self.bound = "mfma" if name in ("gemm_ln_4096x4096x1024", "gemm_softmax_gemm_8192x8192x128x128",
                                        "gemm_gelu_4096x4096x1024") else "hbm"
        nb = cf.cf_workspace_bytes(self.op, *self.dims) if self.op is not None else 0
        self.ws = cf.Workspace(nb) if nb else None
        self.uws = None
        self.copies = max(2, -(-ROTATE_BYTES // self.bytes))
        self.sets = [bufs] + [{k: v.clone() for k, v in bufs.items()} for _ in range(self.copies - 1)]
        self.fused_on = lambda i, ws=None: call(self.sets[i % self.copies], ws if ws is not None else self.ws, False)
        self.fused = lambda ws=None: call(self.sets[0], ws, False)
        self.unfused = lambda ws=None: call(self.sets[0], ws, True)
        self.out = self.sets[0]["Y"] if "Y" in bufs else self.sets[0]["S"]
        if self.op is None:
            call(self.sets[0], None, False)  # the code object loads here, not under graph capture
            torch.cuda.synchronize()

    def oracle_once(self, oracle):
        d = self.inp
        if self.name == "softmax_256x1024":
            return oracle.softmax_rows(d["x"])
        if self.name == "layernorm_750000x32":
            return oracle.layernorm_rows(d["x"], 1e-5)
        if self.name == "pow_bcast_add_softmax_64x30000":
            return oracle.pow_bcast_add_softmax(d["x"], d["v"], 1.5)
        if self.name == "gemm_ln_4096x4096x1024":
            return oracle.gemm_ln(d["a"], d["w"], d["bias"], d["r"], d["gamma"], d["beta"], 1e-5)
        if self.name == "gemm_softmax_gemm_8192x8192x128x128":
            return oracle.gemm_softmax_gemm(d["q"], d["k"], d["v"], d["scale"])
        if self.name == "rmsnorm_750000x32":
            return oracle.rmsnorm_rows(d["x"], d["gamma"], 1e-5)
        if self.name == "layernorm_affine_750000x32":
            return oracle.layernorm_affine_rows(d["x"], d["gamma"], d["beta"], 1e-5)
        if self.name == "gemm_gelu_4096x4096x1024":
            return oracle.gemm_act(d["a"], d["w"], d["bias"], "gelu_tanh")
        if self.name == "auto_softmax_512x65536":
            return oracle.graph.evaluate(self.graph[0], self.graph[1], [d["x"]])
        if self.name.startswith("auto_"):
            return oracle.graph.evaluate(self.graph[0], self.graph[1], [d["x"], d["beta"], d["v"]])
        return oracle.gemm_softmax(d["q"], d["k"], d["scale"])


WORKLOAD_NAMES = ["softmax_256x1024", "layernorm_750000x32", "pow_bcast_add_softmax_64x30000",
                  "gemm_ln_4096x4096x1024", "gemm_softmax_8192x8192x128"]
# measured per kernel (and unfused) but outside the step
EXTRA_NAMES = ["gemm_softmax_gemm_8192x8192x128x128", "rmsnorm_750000x32", "layernorm_affine_750000x32",
               "gemm_gelu_4096x4096x1024", "auto_layernorm_750000x32", "auto_silu_ln_scaled_750000x32",
               "auto_softmax_512x65536"]


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def shape_keys(w):
    """The timed workload's sizes for the JSON line's config: rows x cols, or the GEMM's M, N, K."""
    a, b, c = w.dims
    if c:
        return {"M": a, "N": b, "K": c}
    keys = {"rows": a, "cols": b}
    if "layernorm" in w.name or "rmsnorm" in w.name:
        keys["eps"] = 1e-5
    return keys


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU; --gpus must be 1 "
                                   "(the path shards by rows with no exchange; no multi-GPU launch is provided)"}))
        sys.exit(2)

    import torch

    import broadcast_subgraphs_amd as cf
    import gen

    torch.cuda.init()
    stream = torch.cuda.current_stream()
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")

    sink = torch.empty(1, device="cuda")

    def do_flush():
        # A read-only sweep evicts the caches without leaving dirty lines that
        # the timed kernel would have to write back.
        if args.no_flush:
            return
        if args.flush == "read":
            torch.sum(flush, dim=0, keepdim=True, out=sink)
        else:
            cf.cf_util_fill_f32(flush, 0.0)

    if args.calibrate_copy:
        n = (256 << 20) // 4
        src = torch.ones(n, device="cuda")
        dst = torch.empty(n, device="cuda")
        for _ in range(args.warmup + args.steps):
            do_flush()
            cf.cf_util_copy_f32(src, dst)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": n * 4, "calibrate_copy_bytes_written": n * 4,
                          "launches": args.warmup + args.steps}))
        return

    names = [args.only] if args.only else WORKLOAD_NAMES + EXTRA_NAMES
    wl_all = [Workload(n, torch, cf, gen) for n in names]
    wl = [w for w in wl_all if w.name not in EXTRA_NAMES or args.only]  # the step
    torch.cuda.synchronize()

    def run_step(w, fn, ws, ev=None):
        do_flush()
        if ev is not None:
            ev[0].record(stream)
        fn(ws)
        if ev is not None:
            ev[1].record(stream)

    # ---- warmup
    for k in range(args.warmup):
        for w in wl:
            w.fused_on(k)
    torch.cuda.synchronize()

    # ---- timed region: K steps of the whole hot path (each workload once per
    # step, rotating buffer sets so inputs come from HBM)
    t_ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_ev[0].record(stream)
    for k in range(args.steps):
        for w in wl:
            w.fused_on(args.warmup + k)
    t_ev[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = t_ev[0].elapsed_time(t_ev[1]) / args.steps

    # ---- launch duration of each fused kernel: LAUNCHES_PER_KERNEL back-to-back
    # launches over the rotating buffer sets, captured once as a HIP graph (so
    # the host's per-call cost does not gate small kernels) and replayed between
    # one pair of HIP events on the launch stream, five times
    per = {}
    cs = torch.cuda.Stream()
    for w in wl_all:
        with torch.cuda.stream(cs):
            cs.synchronize()
            cf.cf_graph_begin()
            for i in range(LAUNCHES_PER_KERNEL):
                w.fused_on(i)
            gh = cf.cf_graph_end()
            cf.cf_graph_launch(gh)  # first replay uploads the graph
            cs.synchronize()
            reps = []
            for r in range(5):
                ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                ev[0].record(cs)
                cf.cf_graph_launch(gh)
                ev[1].record(cs)
                cs.synchronize()
                reps.append(ev[0].elapsed_time(ev[1]) * 1e3 / LAUNCHES_PER_KERNEL)
            cf.cf_graph_destroy(gh)
        ts = np.array(reps)
        t = float(ts.mean())
        ent = {"us_mean": round(t, 3), "us_min": round(float(ts.min()), 3), "us_max": round(float(ts.max()), 3),
               "launches": LAUNCHES_PER_KERNEL * len(reps), "buffer_sets": w.copies,
               "alg_bytes": w.bytes, "GBps": round(w.bytes / t / 1e3, 1),
               "frac_hbm_peak": round(w.bytes / t / 1e3 / HBM_PEAK_GBS, 4)}
        if w.flops:
            ent["alg_flops"] = w.flops
            ent["TFLOPs"] = round(w.flops / t / 1e6, 1)
            ent["frac_mfma_peak"] = round(w.flops / t / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4)
        ent["bound"] = w.bound
        ent["in_step"] = w in wl
        ent["plan"] = None
        per[w.name] = ent
    # plans (one extra untimed call each)
    for w in wl_all:
        w.fused(w.ws)
        per[w.name]["plan"] = json.loads(cf.last_plan()) if w.op is not None else w.plan_auto
    torch.cuda.synchronize()
    for w in wl_all:
        if w.ws is not None:
            assert w.ws.error_word() == 0, f"{w.name}: a cross-workgroup wait gave up"

    # ---- unfused baselines, stream-launched and graph-replayed
    if not args.no_unfused:
        for w in wl_all:
            if w.op is None:
                continue  # a generated kernel has no unfused twin
            w.uws = cf.Workspace(cf.cf_unfused_workspace_bytes(w.op, *w.dims))
            ks = max(3, min(args.steps, 10))
            for _ in range(2):
                run_step(w, w.unfused, w.uws)
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(ks)]
            for k in range(ks):
                run_step(w, w.unfused, w.uws, ev[k])
            torch.cuda.synchronize()
            t_stream = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
            cs = torch.cuda.Stream()
            with torch.cuda.stream(cs):
                cs.synchronize()
                cf.cf_graph_begin()
                w.unfused(w.uws)
                h = cf.cf_graph_end()
                evg = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(ks)]
                for k in range(ks + 2):
                    do_flush()
                    if k >= 2:
                        evg[k - 2][0].record(cs)
                    cf.cf_graph_launch(h)
                    if k >= 2:
                        evg[k - 2][1].record(cs)
                cs.synchronize()
                cf.cf_graph_destroy(h)
            t_graph = float(np.mean([a.elapsed_time(b) for a, b in evg])) * 1e3
            # Host wall clock from issuing the chain to its completion (a
            # synchronize on each side, the cache sweep outside): stream launches
            # pay every kernel's host enqueue cost, one graph launch pays one,
            # so their difference is the launch saving the graph buys.
            def host_us(issue):
                ts = []
                for k in range(ks + 1):
                    do_flush()
                    torch.cuda.synchronize()
                    t0 = time.perf_counter()
                    issue()
                    torch.cuda.synchronize()
                    if k >= 1:
                        ts.append((time.perf_counter() - t0) * 1e6)
                return float(np.median(ts))
            with torch.cuda.stream(cs):
                cf.cf_graph_begin()
                w.unfused(w.uws)
                h2 = cf.cf_graph_end()
                cf.cf_graph_launch(h2)
                cs.synchronize()
                t_graph_host = host_us(lambda: cf.cf_graph_launch(h2))
                t_stream_host = host_us(lambda: w.unfused(w.uws))
                cf.cf_graph_destroy(h2)
            per[w.name]["unfused_stream_us"] = round(t_stream, 3)
            per[w.name]["unfused_graph_us"] = round(t_graph, 3)
            per[w.name]["unfused_stream_host_us"] = round(t_stream_host, 3)
            per[w.name]["unfused_graph_host_us"] = round(t_graph_host, 3)
            per[w.name]["speedup_vs_unfused_graph"] = round(t_graph / per[w.name]["us_mean"], 2)
            per[w.name]["launch_savings_us"] = round(t_stream_host - t_graph_host, 3)
            per[w.name]["roundtrip_savings_us"] = round(t_graph - per[w.name]["us_mean"], 3)
            del w.uws
            torch.cuda.empty_cache()

    # ---- Fusion Spec IR: the headline subgraph as a captured graph, lowered,
    # matched and launched; host cost of building the spec and of one launch
    # against the direct entry point, and the launched kernel's bits
    spec_info = None
    head = next((w for w in wl if w.name == HEADLINE), wl[0])
    if head.name == "layernorm_750000x32":
        g = cf.Graph()
        x = g.input(0)
        mu = g.op("div", g.op("rowsum", x), g.const(32))
        c = g.op("sub", x, mu)
        var = g.op("div", g.op("rowsum", g.op("square", c)), g.const(32))
        y = g.op("mul", c, g.op("rsqrt", g.op("add", var, g.const(1e-5))))
        t0 = time.perf_counter()
        nb = 200
        for _ in range(nb):
            spec = cf.Spec(g, y, 750000, 32)
        build_us = (time.perf_counter() - t0) / nb * 1e6
        b0 = head.sets[0]
        out = torch.empty_like(b0["Y"])
        spec.launch([b0["X"]], out, ws=head.ws)
        head.fused(head.ws)
        torch.cuda.synchronize()
        same = bool(torch.equal(out, b0["Y"]))
        nl = 200
        t0 = time.perf_counter()
        for _ in range(nl):
            spec.launch([b0["X"]], out, ws=head.ws)
        t_spec = (time.perf_counter() - t0) / nl * 1e6
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(nl):
            head.fused(head.ws)
        t_direct = (time.perf_counter() - t0) / nl * 1e6
        torch.cuda.synchronize()
        spec_info = {"match": spec.describe()["match"]["call"], "build_host_us": round(build_us, 2),
                     "launch_host_us": round(t_spec, 2), "direct_launch_host_us": round(t_direct, 2),
                     "bitwise_equal_to_direct": same}

    # ---- CPU baseline: the oracle, on rank 0, on a bounded sample.  Rows are
    # independent, so the oracle (unchanged) runs on row chunks of the input
    # in a thread pool with one thread per core the process may use (numpy
    # releases the interpreter lock inside each whole-array operator); the
    # single-core rate (one thread, the whole input) is reported beside it.
    cpu = None
    if not args.no_cpu:
        import oracle
        from concurrent.futures import ThreadPoolExecutor
        cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
        inp = head.inp
        rows = inp["x"].shape[0]
        bounds = np.linspace(0, rows, cores + 1).astype(int)

        def chunk(i):
            lo, hi = bounds[i], bounds[i + 1]
            return oracle.layernorm_rows(inp["x"][lo:hi], 1e-5) if head.name == "layernorm_750000x32" \
                else head.oracle_once(oracle)

        def timed(fn, budget):
            reps, t0 = 0, time.perf_counter()
            while True:
                fn()
                reps += 1
                t = time.perf_counter() - t0
                if t >= budget:
                    return reps, t

        reps1, t1 = timed(lambda: head.oracle_once(oracle), 4.0)
        with ThreadPoolExecutor(max_workers=cores) as ex:
            repsn, tn = timed(lambda: list(ex.map(chunk, range(cores))), 8.0)
        cpu = {"value": round(head.bytes * repsn / tn / 1e9, 3), "unit": "GB/s", "cores": cores,
               "kind": "oracle", "single_core_value": round(head.bytes * reps1 / t1 / 1e9, 3),
               "cpu_model": _cpu_model(),
               "sample": f"{repsn} full passes of the fp64 op-by-op oracle over the {head.name} input, rows "
                         f"split over {cores} threads ({tn:.1f} s); single core: {reps1} passes ({t1:.1f} s)"}

    # ---- roofline of the headline kernel
    h = per[head.name]
    achieved = h["GBps"] if head.bound == "hbm" else h["TFLOPs"]
    roof = {"bound": head.bound, "achieved": achieved,
            "peak": HBM_PEAK_GBS if head.bound == "hbm" else MFMA_BF16_PEAK_TFLOPS,
            "unit": "GB/s" if head.bound == "hbm" else "TFLOP/s",
            "frac": round(achieved / (HBM_PEAK_GBS if head.bound == "hbm" else MFMA_BF16_PEAK_TFLOPS), 4),
            "traffic": None}
    tfile = os.path.join(ROOT, "profiles", f"traffic_{head.name}.json")
    cur_hash = source_hash(head.name, h["plan"])
    if os.path.exists(tfile):
        with open(tfile) as f:
            tr = json.load(f)
        if tr.get("source_hash") == cur_hash:
            roof["traffic"] = tr.get("bytes_per_launch")
            roof["traffic_detail"] = {k: tr[k] for k in ("fetch_bytes", "write_bytes", "fetch_scale", "write_scale")
                                      if k in tr}

    ms_per_step = step_ms
    line = {
        "metric": METRIC,
        "value": h["GBps"] if head.bound == "hbm" else h["TFLOPs"],
        "unit": "GB/s" if head.bound == "hbm" else "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "wall_ms_per_step": round(wall / args.steps * 1e3, 3),
        "timing": (f"ms_per_step: HIP events around the K timed steps (direct launches); per kernel: mean of 5 "
                   f"replays of a HIP graph of {LAUNCHES_PER_KERNEL} back-to-back launches, each replay between one "
                   f"HIP event pair on the launch stream, rotating over buffer sets with >= {ROTATE_BYTES >> 20} MiB "
                   f"of other traffic between two uses of one set"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": head.name, **shape_keys(head),
                   "step": "one fused call per workload: " + ", ".join(w.name for w in wl)},
        "roofline": roof,
        "cpu_baseline": cpu,
        "per_config": per,
        "spec_ir": spec_info,
        "source_hash": cur_hash,
        "planner_env": {k: v for k, v in sorted(os.environ.items()) if k.startswith("CF_")},
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
