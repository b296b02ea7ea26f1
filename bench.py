"""Throughput of the MXFP4 MoE layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one pass of the layer's hot path -- route, permute, FC1 grouped
GEMM + SwiGLU, FC2 grouped GEMM, combine -- over one batch of synthetic
input already resident in HBM (weights, activations, logits).  The default
workload is the Kimi-K3-shaped prefill layer (T=8192, hidden 7168, expert
intermediate 3584, 896 experts, top-16, MXFP8 activations, Zipf-skewed
routing, interleaved gate/up).  `--workload streamed` times the layerwise
double-buffered prefill over 43 stacked DeepSeek-V4-Flash-shaped layers
streamed from pinned host memory.

Prints one JSON line.  Before any timing the step's output is checked
(routing invariants, a consistent permutation, finite and repeatable
outputs); a failed check prints no throughput.  Parity against the oracle at
this size, in this launch configuration, is tests/test_gpu_fullsize.py.  The
oracle runs here only in the CPU-baseline leg.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import mxfp4_weight_mixture_amd as mx  # noqa: E402  (fails loudly if libmxmoe.so is missing)
from workloads import gen  # noqa: E402

PEAK = {  # MI355X published dense peaks
    "hbm_GBps": 8000.0,
    "mxfp4_TFLOPs": 10100.0,
    "fp8_TFLOPs": 5000.0,
    "bf16_TFLOPs": 2500.0,
}
METRIC = "MoE-layer prefill tokens/s + TFLOPS (% MI355X MXFP4 peak), 1 GPU"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="prefill896_mxfp8",
                   choices=["prefill896_mxfp8", "prefill256", "decode", "tiny", "streamed"])
    p.add_argument("--tokens", type=int, default=0, help="override T (decode: 1/2/8/32)")
    p.add_argument("--inter", default=None, choices=["bf16", "mxfp8"],
                   help="precision of the SwiGLU output fed to FC2 (default: mxfp8 for MXFP8 "
                        "activations with hidden % 512 == 0, else bf16)")
    p.add_argument("--w-format", default=None, choices=["canonical", "tiled"],
                   help="weight order the GEMMs read (default: tiled at load time, untimed, when hidden "
                        "and intermediate are multiples of 512, else canonical)")
    p.add_argument("--expert-copy", default="all", choices=["all", "routed", "auto"],
                   help="streamed: move every expert per layer, or only the experts the layer's routing hits")
    p.add_argument("--mfma-rate", action="store_true",
                   help="issue rates of the matrix instructions the GEMM uses (libmxmoe_probe.so), one JSON line")
    p.add_argument("--phases", action="store_true",
                   help="where a grouped-GEMM block's time goes, per row-tile class (K loop, the phases between "
                        "units, small units), for the workload's FC1 and FC2 calls: libmxmoe_phases.so, the same "
                        "kernels with timers compiled in, one JSON line")
    p.add_argument("--chunk-stream", action="store_true",
                   help="rate at which blocks stream contiguous 16 KB chunks, global -> LDS and global -> registers, "
                        "against blocks and chunks in flight (libmxmoe_probe.so), one JSON line")
    p.add_argument("--traffic-record", default=None, metavar="DIR",
                   help="write profiles/gemm_traffic_<workload>.json from the rocprofv3 counter runs under DIR "
                        "(subfolders pmc_FETCH_SIZE, pmc_WRITE_SIZE, cal_FETCH_SIZE, cal_WRITE_SIZE); no GPU needed")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-parity", action="store_true", help="skip the output checks (profiling runs)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a 1 GiB device copy three times (the known-size kernel that scales "
                        "rocprofv3's FETCH_SIZE / WRITE_SIZE counters)")
    return p.parse_args()


# ----------------------------------------------------------------- helpers

class Steps:
    """The five ABI calls of one layer, with events between them on one stream."""
    NAMES = ["route", "permute", "fc1", "fc2", "combine"]

    def __init__(self, shape, w, x, xs, logits, inter="bf16", w_format="canonical"):
        self.s = shape
        self.inter = inter
        self.w1p, self.w1s, self.w2p, self.w2s = w
        self.x, self.xs, self.logits = x, xs, logits
        T, k, E, H, I = shape.T, shape.k, shape.E, shape.H, shape.I
        dev = logits.device
        rows = T * k
        self.ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.tw = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.off = torch.empty(E + 1, dtype=torch.int32, device=dev)
        self.ps = torch.empty(rows, dtype=torch.int32, device=dev)
        self.dr = torch.empty(rows, dtype=torch.int32, device=dev)
        mx8 = inter == "mxfp8"
        self.act = torch.empty((rows, I), dtype=torch.uint8 if mx8 else torch.bfloat16, device=dev)
        self.act_s = torch.empty((rows, I // 32), dtype=torch.uint8, device=dev) if mx8 else None
        self.y = torch.empty((rows, H), dtype=torch.bfloat16, device=dev)
        self.out = torch.empty((T, H), dtype=torch.float32, device=dev)
        self.pws_n = mx.lib.moe_permute_workspace_size(T, E, k)
        self.pws = torch.empty(max(self.pws_n, 1), dtype=torch.uint8, device=dev)
        lay = mx.LAYOUT[shape.layout]
        self.g1 = mx.GemmArgs(a=x.data_ptr(), a_scales=xs.data_ptr() if xs is not None else None,
                              a_gather=self.ps.data_ptr(), w_packed=self.w1p.data_ptr(),
                              w_scales=self.w1s.data_ptr(), expert_offsets=self.off.data_ptr(),
                              c=self.act.data_ptr(), c_scales=self.act_s.data_ptr() if mx8 else None,
                              a_dtype=1 if xs is not None else 0, a_gather_div=k, a_rows=T, rows=rows, E=E,
                              N=2 * I, K=H, epilogue=lay, c_dtype=2 if mx8 else 1,
                              w_format=mx.W_FORMAT[w_format])
        self.g2 = mx.GemmArgs(a=self.act.data_ptr(), a_scales=self.act_s.data_ptr() if mx8 else None,
                              a_gather=None, w_packed=self.w2p.data_ptr(), w_scales=self.w2s.data_ptr(),
                              expert_offsets=self.off.data_ptr(), c=self.y.data_ptr(), c_scales=None,
                              a_dtype=1 if mx8 else 0, a_gather_div=1, a_rows=rows, rows=rows, E=E, N=H, K=I,
                              epilogue=0, c_dtype=1, w_format=mx.W_FORMAT[w_format])
        import ctypes
        self.ctypes = ctypes
        n = max(mx.lib.moe_grouped_gemm_workspace_size(ctypes.byref(self.g1)),
                mx.lib.moe_grouped_gemm_workspace_size(ctypes.byref(self.g2)))
        self.gws_n = n
        self.gws = torch.empty(n, dtype=torch.uint8, device=dev)
        self.ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]

    def run(self, timed=False):
        s, c = self.s, self.ctypes
        st = c.c_void_p(torch.cuda.current_stream().cuda_stream)
        p = lambda t: c.c_void_p(t.data_ptr())
        ev = self.ev
        if timed:
            ev[0].record()
        mx._check(mx.lib.moe_route(p(self.logits), s.T, s.E, s.k, p(self.ids), p(self.tw), st))
        if timed:
            ev[1].record()
        mx._check(mx.lib.moe_permute(p(self.ids), s.T, s.E, s.k, p(self.off), p(self.ps), p(self.dr),
                                     p(self.pws), self.pws_n, st))
        if timed:
            ev[2].record()
        mx._check(mx.lib.moe_mxfp4_grouped_gemm(c.byref(self.g1), p(self.gws), self.gws_n, st))
        if timed:
            ev[3].record()
        mx._check(mx.lib.moe_mxfp4_grouped_gemm(c.byref(self.g2), p(self.gws), self.gws_n, st))
        if timed:
            ev[4].record()
        mx._check(mx.lib.moe_combine(p(self.y), 1, p(self.dr), p(self.tw), s.T, s.k, s.H, p(self.out), None, st))
        if timed:
            ev[5].record()

    def split_ms(self):
        return [self.ev[i].elapsed_time(self.ev[i + 1]) for i in range(5)]


def hit_stats(ids, E):
    counts = np.bincount(ids.ravel(), minlength=E)
    return counts, int((counts > 0).sum())


def sanity_gate(shape, steps):
    """Oracle-free checks of one step's output before any timing (the oracle
    comparison at this size and launch configuration is tests/test_gpu_fullsize.py):
    routing invariants, a consistent permutation, finite outputs, and two runs
    bitwise identical."""
    ids = steps.ids.cpu().numpy()
    w = steps.tw.cpu().numpy()
    off = steps.off.cpu().numpy()
    ps = steps.ps.cpu().numpy()
    dr = steps.dr.cpu().numpy()
    out1 = steps.out.clone()
    steps.run()
    torch.cuda.synchronize()
    checks = {
        "ids_in_range": bool(ids.min() >= 0 and ids.max() < shape.E),
        "ids_distinct_per_token": bool(all(len(set(r)) == shape.k for r in ids[:: max(1, shape.T // 512)])),
        "weights_sum_to_1": bool(np.allclose(w.sum(axis=1), 1.0, atol=1e-5)),
        "weights_non_increasing": bool(np.all(np.diff(w, axis=1) <= 0)),
        "offsets_match_counts": bool(np.array_equal(np.diff(off), np.bincount(ids.ravel(), minlength=shape.E))),
        "dest_row_inverts_perm_src": bool(np.array_equal(dr[ps], np.arange(ps.size))),
        "out_finite": bool(torch.isfinite(out1).all()),
        "repeat_bitwise": bool(torch.equal(out1, steps.out)),
    }
    checks["passed"] = all(checks.values())
    return checks


def host_info():
    """The host the CPU baseline ran on: CPU model, cores, NUMA nodes, BLAS library and its threads."""
    import glob
    info = {"cpu_count": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0))}
    try:
        with open("/proc/cpuinfo") as f:
            info["cpu_model"] = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:
        info["cpu_model"] = None
    info["numa_nodes"] = len(glob.glob("/sys/devices/system/node/node[0-9]*")) or None
    try:
        from threadpoolctl import threadpool_info
        info["blas"] = [{k: i.get(k) for k in ("internal_api", "version", "num_threads", "threading_layer",
                                                "architecture")} for i in threadpool_info() if i.get("user_api") == "blas"]
    except Exception:
        info["blas"] = None
    return info


def _blas_threads(host):
    return max([b.get("num_threads") or 1 for b in (host.get("blas") or [])] + [1])


def _time_experts(shape, li, layer, budget_s):
    """The oracle's expert body (dequantise both matrices + the SwiGLU MLP, float64) over this layer's
    hit experts: every hit expert when the largest one's time x their count fits the budget (measured),
    else a stratified sample by row count with t = a + b*rows fitted and summed (extrapolated).
    Weights are generated before each timed expert (input generation, not timed)."""
    from oracle import moe as omoe
    from oracle import mx as omx
    t0 = time.perf_counter()
    rid, rw = omoe.route(li.logits, shape.k)
    offsets, perm_src, dest_row = omoe.permute(rid, shape.E)
    t_rp = time.perf_counter() - t0
    counts = np.diff(offsets)
    hit = np.nonzero(counts)[0]
    order = hit[np.argsort(-counts[hit], kind="stable")]          # largest first
    x_rows = None
    if shape.act == "mxfp8":
        x_rows = lambda tok: omoe.activations(x_codes=li.x_codes[tok].numpy(), x_scales=li.x_scales[tok].numpy())
    else:
        x_rows = lambda tok: omoe.activations(x_bf16=li.x_bf16[tok].view(torch.int16).numpy())

    def one(e):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        X = x_rows(perm_src[lo:hi] // shape.k)
        w1p, w1s, w2p, w2s = [t.numpy() for t in gen.expert_weights(shape, int(e), layer)]
        t1 = time.perf_counter()
        omoe.expert_mlp(X, omx.dequant_mxfp4(w1p, w1s), omx.dequant_mxfp4(w2p, w2s), shape.layout)
        return hi - lo, time.perf_counter() - t1

    first = one(order[0])
    samples = [first]
    if first[1] * len(order) <= budget_s:
        samples += [one(e) for e in order[1:]]
        t_exp, how = float(sum(t for _, t in samples)), f"all {len(hit)} hit experts timed"
    else:
        n_target = min(8, len(order))
        picks = [order[int(round(q))] for q in np.linspace(0, len(order) - 1, n_target)][1:]
        spent = first[1]
        for e in picks:
            if spent > budget_s and len(samples) >= 2:
                break
            samples.append(one(e))
            spent += samples[-1][1]
        n = np.array([s[0] for s in samples], dtype=np.float64)
        t = np.array([s[1] for s in samples], dtype=np.float64)
        if len(samples) >= 2 and np.ptp(n) > 0:
            b, a = np.polyfit(n, t, 1)
            a, b = max(a, 0.0), max(b, 0.0)
        else:
            a, b = float(t.mean()), 0.0
        t_exp = float(len(hit) * a + b * counts[hit].sum())
        how = (f"{len(samples)} of {len(hit)} hit experts timed at evenly spaced row-count ranks "
               f"({', '.join(str(int(v)) for v in n)} rows), t = a + b*rows fitted (a={a:.3f}s, "
               f"b={b * 1e3:.3f}ms/row) and summed over all hit experts")
    # the combine, on all tokens when T is small, else on a slice of tokens scaled by T
    sub = min(shape.T, 512)
    Y = np.random.default_rng(0).standard_normal((sub * shape.k, shape.H))
    t2 = time.perf_counter()
    omoe.combine(Y, np.arange(sub * shape.k), rw[:sub])
    t_comb = (time.perf_counter() - t2) * shape.T / sub
    measured = len(samples) == len(hit)
    return t_rp + t_exp + t_comb, measured, (f"route+permute over all {shape.T} tokens ({t_rp:.2f}s); expert "
                                             f"body: {how}; combine " + ("timed on all tokens" if sub == shape.T
                                             else f"timed on {sub} tokens and scaled to {shape.T}"))


def cpu_baseline(shape, li, budget_s=20.0):
    """The oracle as it stands, timed on this host's cores on a bounded piece of the workload
    (about budget_s seconds of CPU work), reported as whole-layer tokens/s."""
    host = host_info()
    total, measured, how = _time_experts(shape, li, 0, budget_s)
    reps = 1
    if measured and total < 0.2:
        # a layer of a few milliseconds: repeat it (weights regenerated untimed each time) and average
        reps = int(min(200, max(1, 0.5 // max(total, 1e-4))))
        total = float(np.mean([total] + [_time_experts(shape, li, 0, budget_s)[0] for _ in range(reps - 1)]))
        how += f"; mean of {reps} repetitions"
    return {"value": shape.T / total, "unit": "tokens/s", "cores": _blas_threads(host), "kind": "oracle",
            "method": "whole layer timed" if measured else "extrapolated from a stratified sample of experts",
            "sample": f"{how}; whole-layer oracle time {total * 1e3:.1f} ms", "host": host}


def cpu_baseline_streamed(shape, budget_s=5.0, layers=(0, 1, 21, 42)):
    """The oracle on layers {0, 1, 21, 42} of the stacked workload (each layer on the input it would get
    if the previous one produced N(0,1) bf16 rows: the layer's cost does not depend on its input values),
    plus the RMS rescale, scaled by num_layers / 4: an extrapolation, labelled as such."""
    from oracle import moe as omoe
    host = host_info()
    L = shape.layers
    per = []
    notes = []
    for l in layers:
        if l >= L:
            continue
        li = gen.LayerInputs(shape, gen.activations_bf16(shape), gen.router_logits(shape, l))
        t, measured, how = _time_experts(shape, li, l, budget_s)
        y = np.random.default_rng(l).standard_normal((min(shape.T, 1024), shape.H))
        t1 = time.perf_counter()
        omoe.to_bf16_bits(omoe.rms_rescale(y))
        t += (time.perf_counter() - t1) * shape.T / y.shape[0]
        per.append(t)
        notes.append(f"layer {l}: {t:.1f}s ({'all experts timed' if measured else 'expert sample'})")
    total = float(np.mean(per)) * L
    return {"value": shape.T / total, "unit": "tokens/s", "cores": _blas_threads(host), "kind": "oracle",
            "method": f"extrapolated: mean of layers {list(layers)} x {L}",
            "sample": "; ".join(notes) + f"; est. {L}-layer oracle time {total:.0f}s", "host": host}


def hbm_read_peak(nbytes=4 << 30):
    """Measured HBM stream-read bandwidth (libmxmoe_probe.so), best of a small launch-shape sweep over a
    4 GiB buffer: the denominator beside the published 8 TB/s for weight-streaming shapes."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "mxfp4_weight_mixture_amd", "libmxmoe_probe.so"))
    fn = lib.mxmoe_probe_stream_read
    fn.restype = ctypes.c_float
    fn.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(0x3C)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(cus * 32 * 256, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    best, sweep = 0.0, {}
    for per_cu in (4, 8, 16, 32):
        ms = min(fn(buf.data_ptr(), nbytes, cus * per_cu, out.data_ptr(), stream) for _ in range(3))
        if ms <= 0:
            raise RuntimeError("stream-read probe failed")
        gbps = nbytes / (ms * 1e-3) / 1e9
        sweep[f"{per_cu}_blocks_per_cu"] = gbps
        best = max(best, gbps)
    del buf, out
    torch.cuda.empty_cache()
    return {"GBps": best, "bytes": nbytes, "sweep_GBps": sweep,
            "kernel": "mxmoe_probe_stream_read (16-byte nontemporal loads, 8 in flight per thread)"}


# --------------------------------------------------------------- workloads

def bench_layer(args):
    name = args.workload
    over = {"T": args.tokens} if args.tokens else {}
    shape = gen.preset(name, **over)
    dev = "cuda"
    t0 = time.time()
    li = gen.layer_inputs(shape) if shape.act != "mxfp8" else gen.LayerInputs(
        shape, gen.activations_bf16(shape), gen.router_logits(shape))
    x_bf16 = li.x_bf16.to(dev)
    if shape.act == "mxfp8":
        x, xs = gen.quantize_mxfp8(x_bf16.float())      # input preparation, on the device
        li.x_codes, li.x_scales = x.cpu(), xs.cpu()     # the same bytes for the CPU baseline
    else:
        x, xs = x_bf16, None
    logits = torch.from_numpy(li.logits).to(dev)
    w = gen.all_expert_weights(shape, 0, dev)
    torch.cuda.synchronize()
    log(f"[bench] {name}: inputs ready in {time.time() - t0:.1f}s")

    inter = args.inter or ("mxfp8" if shape.act == "mxfp8" and shape.H % 512 == 0 else "bf16")
    w_format = args.w_format or ("tiled" if shape.H % 512 == 0 and shape.I % 512 == 0 else "canonical")
    if w_format == "tiled":
        # load-time reorder of both weight matrices (one resident copy), not timed
        t1 = mx.tile_weights(w[0], w[1], shape.layout)
        t2 = mx.tile_weights(w[2], w[3], "none")
        w = (*t1, *t2)
        del t1, t2
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        log(f"[bench] weights tiled at load in {time.time() - t0:.1f}s (cumulative)")
    hbm = hbm_read_peak()
    log(f"[bench] HBM stream read: {hbm['GBps']:.0f} GB/s (best of {hbm['sweep_GBps']})")
    steps = Steps(shape, w, x, xs, logits, inter, w_format)
    steps.run()
    torch.cuda.synchronize()
    ids = steps.ids.cpu().numpy()
    counts, n_hit = hit_stats(ids, shape.E)
    parity = None
    if not args.no_parity:
        parity = sanity_gate(shape, steps)
        log(f"[bench] checks: {parity}")
        if not parity["passed"]:
            print(json.dumps({"metric": METRIC, "value": None, "error": "output checks failed", "checks": parity}))
            sys.exit(1)

    for _ in range(args.warmup):
        steps.run()
    torch.cuda.synchronize()
    split = np.zeros(5)
    t_start = time.perf_counter()
    for _ in range(args.steps):
        steps.run(timed=True)
        torch.cuda.synchronize()   # per step: so that the events of this step can be read
        split += np.array(steps.split_ms())
    t_wall = time.perf_counter() - t_start
    split /= args.steps
    ms = float(split.sum())
    log(f"[bench] per step ms: " + ", ".join(f"{n} {v:.3f}" for n, v in zip(Steps.NAMES, split)))

    graph = None
    if name in ("decode", "tiny"):
        graph = bench_graph(shape, w, x, xs, logits, inter, args, w_format)
        log(f"[bench] graph replay {graph['replay_ms']:.4f} ms vs eager layer call {graph['eager_forward_ms']:.4f} ms")

    T, H, I, k, E = shape.T, shape.H, shape.I, shape.k, shape.E
    rows = T * k
    flops = gen.flops(shape)
    fc1_flops = 2.0 * rows * 2 * I * H
    fc2_flops = 2.0 * rows * H * I
    eb = gen.expert_bytes(shape)
    act_bytes = T * H * (1 + 1 / 32) if shape.act == "mxfp8" else T * H * 2
    alg_bytes = n_hit * eb + act_bytes + T * E * 4 + T * H * 4
    fc1_w = n_hit * (2 * I * H) * 17 / 32
    fc2_w = n_hit * (H * I) * 17 / 32
    tflops = flops / (ms * 1e-3) / 1e12
    fc1_ms, fc2_ms = split[2], split[3]
    fc1_peak = PEAK["fp8_TFLOPs"] if shape.act == "mxfp8" else PEAK["bf16_TFLOPs"]
    dom = "fc1" if fc1_ms >= fc2_ms else "fc2"
    if name in ("decode", "tiny"):
        # weight-streaming (HBM) bound shapes: dominant GEMM against HBM bandwidth
        dm = fc1_ms if dom == "fc1" else fc2_ms
        dbytes = fc1_w if dom == "fc1" else fc2_w
        roof = {"bound": "hbm", "achieved": dbytes / (dm * 1e-3) / 1e9, "peak": PEAK["hbm_GBps"], "unit": "GB/s",
                "traffic": None, "kernel": f"{dom} grouped GEMM", "per_launch_ms": dm,
                "algorithmic_per_launch": dbytes,
                "measured_read_peak": hbm["GBps"], "frac_of_measured_read_peak": dbytes / (dm * 1e-3) / 1e9 / hbm["GBps"]}
    else:
        dm = fc1_ms if dom == "fc1" else fc2_ms
        dfl = fc1_flops if dom == "fc1" else fc2_flops
        fc2_peak = PEAK["fp8_TFLOPs"] if inter == "mxfp8" else PEAK["bf16_TFLOPs"]
        pk = fc1_peak if dom == "fc1" else fc2_peak
        roof = {"bound": "mfma", "achieved": dfl / (dm * 1e-3) / 1e12, "peak": pk, "unit": "TFLOP/s",
                "traffic": None, "kernel": f"{dom} grouped GEMM", "per_launch_ms": dm,
                "algorithmic_per_launch": dfl}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"], roof["traffic_source"] = measured_traffic(shape, inter, dom, w_format)
    rec = {
        "metric": METRIC,
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8xmxfp4" if shape.act == "mxfp8" else "bf16xmxfp4",
        "data": "synthetic",
        "config": {"workload": name, "T": T, "hidden": H, "intermediate": I, "experts": E, "top_k": k,
                   "activations": shape.act, "intermediate_dtype": inter, "gate_up": shape.layout,
                   "weight_format": w_format,
                   "router_bias": shape.bias,
                   "experts_hit": n_hit, "parallelism": "none (1 GPU)"},
        "tflops": tflops,
        "pct_mxfp4_peak": tflops / PEAK["mxfp4_TFLOPs"],
        "hbm_algorithmic_GBps": alg_bytes / (ms * 1e-3) / 1e9,
        "hbm_algorithmic_frac_of_8TBps": alg_bytes / (ms * 1e-3) / 1e9 / PEAK["hbm_GBps"],
        "hbm_read_peak": hbm,
        "step_split_ms": dict(zip(Steps.NAMES, [float(v) for v in split])),
        "wall_ms_per_step": t_wall / args.steps * 1e3,
        "roofline": roof,
        "checks": parity,
    }
    if graph is not None:
        rec["graph"] = graph
    return rec, shape, li, ids


def _counter_rows(d):
    """{kernel name: [counter value per dispatch]} of a rocprofv3 csv counter collection with one counter."""
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {d}")
    per = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return per


def _gemm_call(kernel_name):
    """'fc1' / 'fc2' for a grouped-GEMM kernel (its epilogue template argument: SwiGLU 1 / plain 0), else None.
    gemm_dma_kernel / gemm_kernel take <BM, FP8, EPI, ...>, gemm_mixed_kernel <FP8, EPI, OUT>."""
    for tag, epi_arg in (("gemm_dma_kernel<", 2), ("gemm_kernel<", 2), ("gemm_mixed_kernel<", 1)):
        if tag in kernel_name:
            targs = kernel_name.split(tag, 1)[1].split(">", 1)[0].split(",")
            return "fc1" if int(targs[epi_arg]) != 0 else "fc2"
    return None


def _traffic_key(shape, inter, w_format):
    """What a traffic record must match to describe this run: the sources of the kernels that decide the
    grouped GEMM's work (the GEMM itself, routing and permutation), the input generator, and the workload."""
    srcs = {}
    for rel in ("mxfp4_weight_mixture_amd/csrc/gemm.hip", "mxfp4_weight_mixture_amd/csrc/route.hip",
                "mxfp4_weight_mixture_amd/csrc/permute.hip", "workloads/gen.py"):
        srcs[rel] = hashlib.sha256(open(os.path.join(ROOT, rel), "rb").read()).hexdigest()[:16]
    return {"sources_sha256_16": srcs, "workload": dataclasses.asdict(shape), "intermediate_dtype": inter,
            "weight_format": w_format}


def _traffic_path(shape, name):
    return os.path.join(ROOT, "profiles", f"gemm_traffic_{name}" + (f"_t{shape.T}" if name == "decode" else "")
                        + ".json")


def write_traffic_record(args):
    """HBM bytes per FC1 / FC2 call from FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by
    what the same counter reads for a device add of 1 GiB in and 1 GiB out (bench.py --copy-calibration).
    A call is one launch per row-tile class, so a call's bytes are the sum of the class kernels' means."""
    import subprocess
    name = args.workload
    shape = gen.preset(name, **({"T": args.tokens} if args.tokens else {}))
    inter = args.inter or ("mxfp8" if shape.act == "mxfp8" and shape.H % 512 == 0 else "bf16")
    w_format = args.w_format or ("tiled" if shape.H % 512 == 0 and shape.I % 512 == 0 else "canonical")
    d = args.traffic_record
    scale = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        # the add dispatches only (the fill that makes the source reads nothing)
        cal = [v for k, vals in _counter_rows(os.path.join(d, f"cal_{ctr}")).items()
               if "elementwise" in k and "_add" in k for v in vals]
        scale[ctr] = (1 << 30) / 1024 / float(np.mean(cal))
    try:
        head = subprocess.run(["git", "-C", ROOT, "rev-parse", "--short=12", "HEAD"], capture_output=True,
                              text=True).stdout.strip() or None
    except OSError:
        head = None
    rec = {"workload": name, "T": shape.T, "key": _traffic_key(shape, inter, w_format),
           "counters_dir": os.path.relpath(os.path.abspath(d), ROOT), "head_when_recorded": head}
    per_kernel = {}
    for ctr, key in (("FETCH_SIZE", "read"), ("WRITE_SIZE", "write")):
        for kname, vals in _counter_rows(os.path.join(d, f"pmc_{ctr}")).items():
            call = _gemm_call(kname)
            if call is None:
                continue
            b = float(np.mean(vals)) * 1024 * scale[ctr]
            rec[f"{call}_{key}_bytes"] = rec.get(f"{call}_{key}_bytes", 0.0) + b
            short = re.search(r"gemm\w*<[^>]*>", kname).group(0)
            per_kernel.setdefault(short, {})[key + "_bytes"] = b
            per_kernel[short]["dispatches"] = len(vals)
    for call in ("fc1", "fc2"):
        rec[f"{call}_bytes"] = rec.get(f"{call}_read_bytes", 0.0) + rec.get(f"{call}_write_bytes", 0.0)
    rec["scale"] = scale
    rec["per_kernel"] = per_kernel
    out = _traffic_path(shape, name)
    json.dump(rec, open(out, "w"), indent=1)
    print(json.dumps({k: v for k, v in rec.items() if k != "per_kernel"}))


def measured_traffic(shape, inter, call, w_format):
    """(HBM bytes of one `call` ("fc1"/"fc2") from the rocprofv3 counter record under profiles/, source)
    or (None, reason) when there is no record for this workload or anything in its key -- the GEMM,
    routing and permutation sources, the input generator, the workload, the intermediate precision or
    the weight format -- differs from this run."""
    name = next((n for n, s in gen.PRESETS.items() if dataclasses.replace(s, T=shape.T) == shape), None)
    if name is None:
        return None, "no record for this workload"
    path = _traffic_path(shape, name)
    if not os.path.exists(path):
        return None, f"no record ({os.path.relpath(path, ROOT)})"
    rec = json.load(open(path))
    if rec.get("key") != _traffic_key(shape, inter, w_format):
        return None, f"{os.path.relpath(path, ROOT)} was taken on other sources or another workload"
    return rec.get(f"{call}_bytes"), {"record": os.path.relpath(path, ROOT),
                                      "head_when_recorded": rec.get("head_when_recorded"),
                                      "counters_dir": rec.get("counters_dir")}


def bench_graph(shape, w, x, xs, logits, inter, args, w_format="canonical"):
    """The resident layer as one eager moe_layer_forward call vs one replay of its
    captured graph (moe_layer_graph_*), each timed over the same step count; the
    replay must equal the eager output bitwise."""
    layer = mx.Layer(*w, k=shape.k, layout=shape.layout, inter=inter, w_format=w_format)
    eager = layer.forward(logits, x, xs).clone()
    g = layer.capture(logits, x, xs)
    try:
        torch.cuda.synchronize()
        same = bool(torch.equal(g.replay(), eager))
        torch.cuda.synchronize()

        def timed(fn):
            for _ in range(args.warmup):
                fn()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record()
            for _ in range(args.steps):
                fn()
            b.record()
            torch.cuda.synchronize()
            return a.elapsed_time(b) / args.steps

        eager_ms = timed(lambda: layer.forward(logits, x, xs))
        replay_ms = timed(g.replay)
    finally:
        g.close()
    return {"replay_ms": replay_ms, "eager_forward_ms": eager_ms, "replay_equals_eager": same,
            "note": "back-to-back steps on one stream, no per-step sync"}


# NUMA placement of the pinned weight blobs (Linux syscalls on x86-64; the
# pages' node is read back, so the record says where they really are)
_SYS_SET_MEMPOLICY, _SYS_GET_MEMPOLICY = 238, 239
_MPOL_DEFAULT, _MPOL_PREFERRED = 0, 1
_MPOL_F_NODE, _MPOL_F_ADDR = 1, 2


def gpu_numa_node():
    """NUMA node of GPU 0 from sysfs (its PCI function), or -1 when the host does not say."""
    try:
        pr = torch.cuda.get_device_properties(0)
        bdf = f"{pr.pci_domain_id:04x}:{pr.pci_bus_id:02x}:{pr.pci_device_id:02x}.0"
        return int(open(f"/sys/bus/pci/devices/{bdf}/numa_node").read())
    except Exception:
        return -1


def _libc():
    import ctypes
    return ctypes.CDLL(None, use_errno=True)


def prefer_numa_node(node):
    """Make this thread's new pages come from `node` (MPOL_PREFERRED); node < 0 restores the default.
    Returns True when the policy was set.  A pinned allocation made meanwhile is placed there (the
    lesson of ktransformers issue #2172, second comment: weight pools bound to the wrong node)."""
    import ctypes
    libc = _libc()
    if node < 0:
        return libc.syscall(_SYS_SET_MEMPOLICY, _MPOL_DEFAULT, None, ctypes.c_ulong(0)) == 0
    mask = (ctypes.c_ulong * 16)()
    mask[node // 64] = 1 << (node % 64)
    return libc.syscall(_SYS_SET_MEMPOLICY, _MPOL_PREFERRED, mask, ctypes.c_ulong(16 * 64)) == 0


def page_numa_nodes(t, samples=16):
    """NUMA nodes holding `samples` evenly spaced pages of host tensor t (-1 where unknown)."""
    import ctypes
    libc = _libc()
    out = []
    base, n = t.data_ptr(), t.numel() * t.element_size()
    for i in range(samples):
        node = ctypes.c_int(-1)
        addr = ctypes.c_void_p(base + (n - 1) * i // max(1, samples - 1))
        rc = libc.syscall(_SYS_GET_MEMPOLICY, ctypes.byref(node), None, ctypes.c_ulong(0), addr,
                          ctypes.c_ulong(_MPOL_F_NODE | _MPOL_F_ADDR))
        out.append(node.value if rc == 0 else -1)
    return out


def bench_streamed(args):
    shape = gen.preset("streamed")
    if args.tokens:
        shape = dataclasses.replace(shape, T=args.tokens)
    T, H, I, E, k, L = shape.T, shape.H, shape.I, shape.E, shape.k, shape.layers
    dev = "cuda"
    nbytes = mx.blob_bytes(H, I, E)
    # distinct pinned blobs: all 43 if host memory allows, else layer L uses blob L % n
    try:
        import psutil
        avail = psutil.virtual_memory().available
    except Exception:
        avail = 64 << 30
    n_blobs = int(max(2, min(L, (0.5 * avail) // nbytes)))
    t0 = time.time()
    # pinned blobs on the GPU's NUMA node when the host has several
    import glob as _glob
    host_nodes = len(_glob.glob("/sys/devices/system/node/node[0-9]*")) or 1
    gnode = gpu_numa_node()
    numa_bound = host_nodes > 1 and gnode >= 0 and prefer_numa_node(gnode)
    blobs = []
    for b in range(n_blobs):
        try:
            blob = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
        except RuntimeError as e:          # the host's pinned-memory limit
            if b < 2:
                raise
            log(f"[bench] streamed: pinned allocation {b + 1} failed ({str(e).splitlines()[0]}); "
                f"layers reuse {b} blobs")
            n_blobs = b
            break
        w = gen.all_expert_weights(shape, b, dev)
        for which, t in enumerate(w):
            o = mx.blob_section_offset(H, I, E, which)
            blob[o:o + t.numel()].copy_(t.reshape(-1))
        del w
        blobs.append(blob)
        if b % 4 == 3 or b == n_blobs - 1:
            log(f"[bench] streamed: {b + 1}/{n_blobs} pinned blobs filled ({time.time() - t0:.1f}s)")
    torch.cuda.synchronize()
    if numa_bound:
        prefer_numa_node(-1)
    page_nodes = sorted(set(n for b in blobs for n in page_numa_nodes(b)))
    numa = {"host_nodes": host_nodes, "gpu_node": gnode, "policy": "preferred gpu node" if numa_bound else
            ("single node: every page is local" if host_nodes == 1 else "gpu node unknown: default policy"),
            "blob_page_nodes": page_nodes}
    log(f"[bench] streamed: {n_blobs} pinned blobs of {nbytes / 1e9:.3f} GB in {time.time() - t0:.1f}s; numa {numa}")
    slots = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(2)]
    logits = torch.from_numpy(np.stack([gen.router_logits(shape, l) for l in range(L)])).to(dev)
    x = gen.activations_bf16(shape).to(dev)
    out = torch.empty((T, H), dtype=torch.float32, device=dev)
    copy = torch.cuda.Stream()
    ws = None
    # measured pinned H2D peak on the same buffers (copy engine): whole blobs on one stream, and
    # 16 MB .. 1 GB pieces on one and on two streams; the best is the denominator
    h2d = {}
    for b in range(min(2, n_blobs)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(copy):
            e0.record()
            slots[b % 2].copy_(blobs[b], non_blocking=True)
            e1.record()
        copy.synchronize()
        h2d[f"blob_1stream_{b}"] = nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9
    copy2 = torch.cuda.Stream()
    for size in (16 << 20, 256 << 20, 1 << 30):
        reps = max(1, (2 << 30) // size)
        for nstreams in (1, 2):
            streams = [copy, copy2][:nstreams]
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for st in streams:
                st.wait_event(e0)
            for r in range(reps):
                st = streams[r % nstreams]
                off = (r * size) % (nbytes - size)
                with torch.cuda.stream(st):
                    slots[r % 2][off:off + size].copy_(blobs[r % n_blobs][off:off + size], non_blocking=True)
            cur = torch.cuda.current_stream()
            for st in streams:
                cur.wait_stream(st)
            e1.record()
            torch.cuda.synchronize()
            h2d[f"{size >> 20}MB_{nstreams}stream"] = reps * size / (e0.elapsed_time(e1) * 1e-3) / 1e9
    h2d_peak = max(h2d.values())
    log("[bench] pinned H2D GB/s: " + ", ".join(f"{k} {v:.1f}" for k, v in h2d.items()))

    def run(depth, events=None, expert_copy=args.expert_copy):
        nonlocal ws
        ws = mx.prefill_streamed(blobs, slots, logits, x, out, T=T, H=H, I=I, E=E, k=k, num_layers=L,
                                 layout=shape.layout, chain="rms", depth=depth, workspace=ws, events=events,
                                 copy_stream=copy, expert_copy=expert_copy)

    # experts each layer's routing hits (torch top-k over the logits: bytes accounting only)
    hits = [int(torch.topk(logits[l], k, dim=1).indices.unique().numel()) if T else 0 for l in range(L)]
    per_expert = 3 * H * I * 17 // 32

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4 * L)]
    for e in ev:
        e.record()
    torch.cuda.synchronize()
    for _ in range(max(1, args.warmup)):
        run(2)
    torch.cuda.synchronize()
    times = []
    for _ in range(args.steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        run(2, ev)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    ms = float(np.mean(times))
    copy_ms = [ev[4 * l].elapsed_time(ev[4 * l + 1]) for l in range(L)]
    comp_ms = [ev[4 * l + 2].elapsed_time(ev[4 * l + 3]) for l in range(L)]
    # overlap of the last timed pass: 1 - (time the compute stream sits idle) / wall, from the
    # first copy's start to the last layer's end
    span = ev[0].elapsed_time(ev[4 * (L - 1) + 3])
    overlap = 1.0 - (span - sum(comp_ms)) / span
    # serialized comparison (depth 1: copy, compute, copy, ...)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    run(1)
    b.record()
    torch.cuda.synchronize()
    ms1 = a.elapsed_time(b)
    routed = args.expert_copy == "routed"
    h2d_bytes = sum(hits) * per_expert if routed else L * nbytes
    achieved = h2d_bytes / (ms * 1e-3) / 1e9
    all_ms = None
    if routed:
        # the all-experts stream at the same T, for comparison
        run(2, expert_copy="all")
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        run(2, expert_copy="all")
        b.record()
        torch.cuda.synchronize()
        all_ms = a.elapsed_time(b)
    flops = gen.flops(shape) * L
    rec = {
        "metric": METRIC, "value": T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16xmxfp4", "data": "synthetic",
        "config": {"workload": "streamed", "layers": L, "T": T, "hidden": H, "intermediate": I, "experts": E,
                   "top_k": k, "distinct_host_blobs": n_blobs, "blob_GB": nbytes / 1e9, "numa": numa,
                   "expert_copy": args.expert_copy, "parallelism": "none (1 GPU)"},
        "experts_hit_per_layer_mean": float(np.mean(hits)), "h2d_bytes_per_pass": h2d_bytes,
        "all_experts_ms": all_ms,
        "tflops": flops / (ms * 1e-3) / 1e12,
        "h2d_GBps": achieved, "h2d_measured_peak_GBps": h2d_peak, "h2d_frac_of_measured": achieved / h2d_peak,
        "h2d_sweep_GBps": h2d,
        "serialized_ms": ms1, "serialized_tokens_per_s": T / (ms1 * 1e-3),
        "per_layer_copy_ms_mean": float(np.mean(copy_ms)), "per_layer_compute_ms_mean": float(np.mean(comp_ms)),
        "compute_busy_fraction": overlap,
        "copy_busy_fraction": sum(copy_ms) / span,
        "roofline": {"bound": "h2d", "achieved": achieved, "peak": h2d_peak, "unit": "GB/s",
                     "frac": achieved / h2d_peak, "traffic": None, "kernel": "host->device weight stream"},
    }
    if args.expert_copy != "all":
        rec["routed_copy_note"] = (
            "the copy stream routes each layer from that layer's router logits before the previous layer's "
            "compute ends, which works because this call receives every layer's logits up front; in a stacked "
            "model a layer's router input is the previous layer's output, so there the hit set is known only "
            "after that layer, and the pass without routing (all_experts_ms) is the one that applies")
    return rec


def mfma_rates():
    """Sustained rate of each matrix instruction the grouped GEMM issues, over the whole chip (two blocks of
    four waves per CU, eight independent accumulators per wave), with constant operands and with operand bits
    that change every round.  The ceilings FC1 / FC2 are read against."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "mxfp4_weight_mixture_amd", "libmxmoe_probe.so"))
    fn = lib.mxmoe_probe_mfma_rate
    fn.restype = ctypes.c_float
    fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = 2 * cus
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    rec = {"probe": "mfma issue rate", "cus": cus, "blocks": blocks, "waves_per_cu": 8,
           "command": "python bench.py --mfma-rate"}
    for kind, name, fl in ((0, "fp8xfp4_scaled_32x32x64", 2 * 32 * 32 * 64), (1, "fp4xfp4_scaled_32x32x64", 2 * 32 * 32 * 64),
                           (2, "bf16_32x32x16", 2 * 32 * 32 * 16)):
        for vary in (0, 1):
            fn(kind, blocks, 2000, vary, out.data_ptr(), stream)          # warm-up (clocks, code load)
            iters = 100000 if kind != 2 else 200000
            ms = fn(kind, blocks, iters, vary, out.data_ptr(), stream)
            if ms <= 0:
                raise RuntimeError("probe launch failed")
            flops = 8.0 * iters * blocks * 4 * fl
            rec[f"{name}_{'random' if vary else 'constant'}_PFLOPs"] = flops / (ms * 1e-3) / 1e15
            log(f"[probe] {name} {'changing' if vary else 'constant'} operands: {flops / (ms * 1e-3) / 1e15:.2f} PF "
                f"({ms:.1f} ms)")
    return rec


def chunk_stream_rates():
    """The grouped GEMM's weight-stream access pattern on its own: each block reads its own run of 16 KB
    chunks (a unit's tiled weight stages), into LDS with the DMA the GEMM uses or into registers, for a few
    block counts (32 / 64: a few CUs streaming beside idle ones; 256: one block per CU; 448: the decode T=1
    FC1 shape, 16 experts x 28 n-tiles of 56 stages) and chunks in flight per block."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "mxfp4_weight_mixture_amd", "libmxmoe_probe.so"))
    fn = lib.mxmoe_probe_chunk_stream
    fn.restype = ctypes.c_float
    fn.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                   ctypes.c_void_p, ctypes.c_void_p]
    nbytes = 1 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    out = torch.empty(448 * 256, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    rec = {"probe": "16 KB chunk stream", "command": "python bench.py --chunk-stream", "runs": []}
    cases = [(b, ch, 0, d) for b, ch in ((32, 448), (64, 448), (256, 224), (448, 56)) for d in (1, 2, 3, 4, 6, 7)]
    cases += [(448, 56, 1, d) for d in (1, 2, 4)]
    for blocks, chunks, mode, depth in cases:
        fn(buf.data_ptr(), nbytes, blocks, chunks, mode, depth, out.data_ptr(), stream)   # warm-up
        ms = min(fn(buf.data_ptr(), nbytes, blocks, chunks, mode, depth, out.data_ptr(), stream) for _ in range(3))
        if ms <= 0:
            raise RuntimeError("probe launch failed")
        tot = blocks * chunks * 16384
        run = {"blocks": blocks, "chunks_per_block": chunks, "path": "global->LDS DMA" if mode == 0 else
               "global->registers", "chunks_in_flight": depth, "ms": ms, "GBps": tot / (ms * 1e-3) / 1e9,
               "GBps_per_block": tot / blocks / (ms * 1e-3) / 1e9}
        rec["runs"].append(run)
        log(f"[probe] {blocks:3d} blocks, {run['path']:17s}, {depth} x 16 KB in flight: {run['GBps']:6.0f} GB/s "
            f"({run['GBps_per_block']:5.1f} per block)")
    del buf, out
    torch.cuda.empty_cache()
    return rec


PHASE_NAMES = ["k_loop", "barrier_and_draw", "epilogue_to_last_staging_write", "next_setup_first_dma_barrier",
               "readback_and_stores", "barrier", "rest"]


def gemm_phases(args):
    """Runs the workload's route and permute with libmxmoe.so, then its FC1 and FC2 grouped-GEMM calls with
    libmxmoe_phases.so (the same kernels with wave 0 of each unit loop reading the 100 MHz s_memrealtime clock
    at the boundaries of a unit's phases; the timers change the kernels' register allocation, so their times
    are a close, not an exact, image of the library's).  Per call and row-tile class: units, mean time per
    unit of each phase, the blocks' summed time, and the spread of the loops' starts and ends."""
    import ctypes
    ph = ctypes.CDLL(os.path.join(ROOT, "mxfp4_weight_mixture_amd", "libmxmoe_phases.so"))
    ph.moe_mxfp4_grouped_gemm.restype = ctypes.c_int
    ph.moe_mxfp4_grouped_gemm.argtypes = [ctypes.POINTER(mx.GemmArgs), ctypes.c_void_p, ctypes.c_size_t,
                                          ctypes.c_void_p]
    name = args.workload
    shape = gen.preset(name, **({"T": args.tokens} if args.tokens else {}))
    li = gen.layer_inputs(shape) if shape.act != "mxfp8" else gen.LayerInputs(
        shape, gen.activations_bf16(shape), gen.router_logits(shape))
    x_bf16 = li.x_bf16.to("cuda")
    x, xs = gen.quantize_mxfp8(x_bf16.float()) if shape.act == "mxfp8" else (x_bf16, None)
    logits = torch.from_numpy(li.logits).to("cuda")
    w = gen.all_expert_weights(shape, 0, "cuda")
    inter = args.inter or ("mxfp8" if shape.act == "mxfp8" and shape.H % 512 == 0 else "bf16")
    w_format = args.w_format or ("tiled" if shape.H % 512 == 0 and shape.I % 512 == 0 else "canonical")
    if w_format == "tiled":
        t1 = mx.tile_weights(w[0], w[1], shape.layout)
        t2 = mx.tile_weights(w[2], w[3], "none")
        w = (*t1, *t2)
        del t1, t2
        torch.cuda.empty_cache()
    steps = Steps(shape, w, x, xs, logits, inter, w_format)
    for _ in range(3):
        steps.run()
    torch.cuda.synchronize()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    buf = np.zeros(2048 * 4 * 12, dtype=np.uint64)
    rec = {"probe": "grouped-GEMM phase timers", "workload": name, "T": shape.T, "inter": inter,
           "command": f"python bench.py --phases --workload {name}" + (f" --tokens {args.tokens}" if args.tokens else ""),
           "calls": {}}
    for which, g in (("fc1", steps.g1), ("fc2", steps.g2)):
        for _ in range(3):
            mx._check(ph.moe_mxfp4_grouped_gemm(ctypes.byref(g), ctypes.c_void_p(steps.gws.data_ptr()), steps.gws_n, stream))
        torch.cuda.synchronize()
        if ph.mxmoe_phase_timers_reset() != 0:
            raise RuntimeError("phase timer reset failed")
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        mx._check(ph.moe_mxfp4_grouped_gemm(ctypes.byref(g), ctypes.c_void_p(steps.gws.data_ptr()), steps.gws_n, stream))
        ev[1].record()
        torch.cuda.synchronize()
        if ph.mxmoe_phase_timers_read(ctypes.c_void_p(buf.ctypes.data)) != 0:
            raise RuntimeError("phase timer read failed")
        d = buf.reshape(2048, 4, 12)
        call = {"call_ms": ev[0].elapsed_time(ev[1]), "classes": {}}
        starts = [int(~np.uint64(v)) for v in d[:, :, 10].max(axis=1) if v]
        ends = [int(v) for v in d[:, :, 11].max(axis=1) if v]
        if starts:
            t0 = min(starts)
            call["loop_start_spread_us"] = (max(starts) - t0) * 10 / 1e3
            call["first_loop_end_us"] = (min(ends) - t0) * 10 / 1e3
            call["last_loop_end_us"] = (max(ends) - t0) * 10 / 1e3
        for ci, bm in enumerate((32, 64, 128, 256)):
            n = int(d[:, ci, 7].sum())
            if n == 0:
                continue
            per = {PHASE_NAMES[j]: float(d[:, ci, j].sum()) * 10 / 1e3 / n for j in range(7)}
            runs = int(d[:, ci, 9].sum())
            call["classes"][f"{bm}_rows"] = {
                "units": n, "us_per_unit": per,
                "block_ms": float(d[:, ci, :7].sum()) * 10 / 1e6,
                "first_setup_us": float(d[:, ci, 8].sum()) * 10 / 1e3 / max(runs, 1), "loops": runs}
            log(f"[phases] {which} {bm:3d}-row units {n:6d}: " +
                ", ".join(f"{k} {v:.2f}" for k, v in per.items()) + f" us; block-ms {call['classes'][f'{bm}_rows']['block_ms']:.1f}")
        rec["calls"][which] = call
        log(f"[phases] {which}: call {call['call_ms']:.3f} ms, loops start within "
            f"{call.get('loop_start_spread_us', 0):.1f} us, end {call.get('first_loop_end_us', 0):.1f}-"
            f"{call.get('last_loop_end_us', 0):.1f} us after the first start")
    return rec


def main():
    args = parse()
    if args.traffic_record:
        write_traffic_record(args)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the layer is not sharded "
              f"across GPUs in this build.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available() or not mx.device_supported():
        print("bench.py needs an MI355X (gfx950) GPU", file=sys.stderr)
        sys.exit(1)

    if args.mfma_rate:
        print(json.dumps(mfma_rates()))
        return
    if args.chunk_stream:
        print(json.dumps(chunk_stream_rates()))
        return
    if args.phases:
        if args.workload == "streamed":
            print("--phases times a resident layer's GEMM calls, not the streamed pass", file=sys.stderr)
            sys.exit(2)
        print(json.dumps(gemm_phases(args)))
        return
    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.add(src, 0.0, out=dst)    # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "launches": 3}))
        return
    if args.workload == "streamed":
        rec = bench_streamed(args)
        if not args.no_cpu_baseline:
            shape = gen.preset("streamed", **({"T": args.tokens} if args.tokens else {}))
            rec["cpu_baseline"] = cpu_baseline_streamed(shape)
            log(f"[bench] cpu baseline: {rec['cpu_baseline']}")
    else:
        rec, shape, li, ids = bench_layer(args)
        if not args.no_cpu_baseline:
            rec["cpu_baseline"] = cpu_baseline(shape, li)
            log(f"[bench] cpu baseline: {rec['cpu_baseline']}")
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
