#!/usr/bin/env python3
"""Benchmark of one routed-MoE layer over block-quantized experts on MI355X.

Metric: MoE-layer decode tokens/s (verify columns per second through one
layer) and the packed expert bytes streamed per step as HBM GB/s, at q = 1,
4 and 5 verify columns.

Workloads (synthetic, seeded; shapes of DeepSeek-V4-Flash-class layers):
  decode-q1-d4096-e256-top6  q=1: d=4096, f=2048, 256 experts top-6 + 1
      shared; gate/up FP2, down FP3, shared FP4; bf16 activations
  verify-q4-zipf  q=4 verify columns, Zipf(1.1) routing per column
  verify-q5-zipf-hot32fp4-43layers  q=5 verify columns, Zipf(1.1), the 32
      hottest experts FP4, 43 layers; also timed as a 43-layer step, eager
      and as one captured HIP graph
  prefill-t2048-zipf  a 2048-token prefill chunk through one layer
The default run times all four, one after the other, and prints one JSON
line whose headline (value, ms_per_step, roofline, cpu_baseline) is the q=1
decode step; q=4, q=5 and prefill are under "workloads".  --workload runs
one of them alone (its line then carries that workload's headline).

A decode step is one moe_layer_forward call (router, top-k, batching,
gate/up, down, combine) on one batch of q columns.  Steps rotate over the
workload's layer instances (synth.ROTATION), each with its own router,
experts and activation batches, so that no weight is re-read from the 256 MB
last-level cache within a rotation.

Timing: W warm-up steps, then 5 batches of exactly K steps, each between two
synchronizations and timed with events on the stream the kernels run on;
value and ms_per_step are the median batch, with min and max beside them.  A
further pass of K steps (moe_layer_forward_timed / moe_prefill_forward_timed)
has every kernel launched through hipExtLaunchKernel with a start and an end
event, stamped when that kernel itself starts and ends: the kernel with the
longest mean duration is the roofline entry ("dominant kernel"), its
achieved rate = its algorithmic bytes (or flops) per launch / that duration.
Stamped launches leave wider gaps between kernels, so that pass gives kernel
durations only.  The CPU oracle is timed on a bounded sample on the host,
single-threaded and on every available core.
"""
from __future__ import annotations

import argparse
import ctypes as C
import json
import os
import platform
import statistics
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer decode tokens/s and packed-weight HBM GB/s (% of peak) at q=1,4,5"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
HIP_EVENT_RELEASE_TO_DEVICE = 0x40000000  # hipEventReleaseToDevice
BATCHES = 5

DECODE_WORKLOADS = ("decode-q1-d4096-e256-top6", "verify-q4-zipf",
                    "verify-q5-zipf-hot32fp4-43layers")
PREFILL_WORKLOAD = "prefill-t2048-zipf"


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t handles through the HIP runtime torch already loaded."""

    def __init__(self):
        path = None
        with open("/proc/self/maps") as fh:
            for line in fh:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("HIP runtime not loaded")
        self.lib = C.CDLL(path)
        self.lib.hipEventCreateWithFlags.argtypes = [C.POINTER(C.c_void_p), C.c_uint]
        self.lib.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.lib.hipEventDestroy.argtypes = [C.c_void_p]

    def create(self, n):
        arr = (C.c_void_p * n)()
        for i in range(n):
            h = C.c_void_p()
            # device-scope release: a timing event then costs no write-back
            # of the caches to system scope between the kernels it separates
            if self.lib.hipEventCreateWithFlags(C.byref(h), HIP_EVENT_RELEASE_TO_DEVICE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            arr[i] = h
        return arr

    def elapsed_ms(self, a, b) -> float:
        ms = C.c_float()
        if self.lib.hipEventElapsedTime(C.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, arr):
        for h in arr:
            self.lib.hipEventDestroy(h)


def expert_bytes(lay, e):
    """(all packed bytes, gate + up bytes) of expert e."""
    import synth
    tot = 0
    gu = 0
    for m in range(3):
        rows, cols = lay.matrix_shape(m)
        b = synth.matrix_bytes(int(lay.fmts[e][m]), rows, cols)
        tot += b
        if m < 2:
            gu += b
    return tot, gu


# The sources that define each product kernel's code and launch (the files
# its code and its launch set-up are built from): a counter summary stays
# valid while these are unchanged.
_DECODE_SOURCES = ("expert.hip", "route.hip", "rfpx_impl.hpp", "rfpx_route.hpp", "abi.hip")
_PREFILL_SOURCES = ("prefill.hip", "rfpx_impl.hpp", "rfpx_route.hpp", "abi.hip")
KERNEL_SOURCES = {"k_gateup": _DECODE_SOURCES, "k_down": _DECODE_SOURCES,
                  "k_pf_gateup": _PREFILL_SOURCES, "k_pf_down": _PREFILL_SOURCES}


def kernel_source_hash(kernel: str, root: str = ROOT) -> str:
    """sha256 over the sources that define `kernel` and its launch."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        path = os.path.join(root, "block_quantized_expert_amd", "csrc", name)
        if os.path.exists(path):
            with open(path, "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary of `kernel` on
    `workload` (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy), or None when
    there is none or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kernel not in KERNEL_SOURCES or kv.get("source_sha256") != kernel_source_hash(kernel):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def host_description() -> dict:
    """CPU model and core counts of this host."""
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return {"cpu_model": model, "nproc": avail, "cpu_count": os.cpu_count()}


def oracle_threads() -> int:
    """Threads for the multi-core oracle leg: every core this process may
    use, at most 16 (the host share of one GPU on a shared node)."""
    return max(1, min(16, host_description()["nproc"]))


def calibration_copy(dev, mib):
    """One plain fp32 copy kernel (torch.neg) of `mib` MiB, for scaling the
    HBM byte counters of a profiled run."""
    import torch
    n = mib * (1 << 18)
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log(f"# calibration copy: {4 * n} bytes read, {4 * n} bytes written")


def timed_batches(run_batch, batches: int):
    """ms of each of `batches` calls of run_batch(), each bracketed by a
    synchronization and timed with events on the current stream."""
    import torch
    out = []
    for _ in range(batches):
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        run_batch()
        t1.record()
        torch.cuda.synchronize()
        out.append(t0.elapsed_time(t1))
    return out


def spread(values):
    return {"median": statistics.median(values), "min": min(values), "max": max(values)}


def cpu_oracle_rate(fn, units_per_call: int, seconds: float, threads: int):
    """Calls of fn() (one oracle job of units_per_call units) on `threads`
    host threads for about `seconds`; returns (units/s, units done, wall s).
    The oracle's ctypes calls release the GIL, so threads run in parallel."""
    if seconds <= 0:
        return None
    done = [0] * threads
    stop = time.time() + seconds

    def worker(i):
        while time.time() < stop:
            fn()
            done[i] += units_per_call

    t = time.time()
    ts = [threading.Thread(target=worker, args=(i,)) for i in range(threads)]
    for th in ts:
        th.start()
    for th in ts:
        th.join()
    dt = time.time() - t
    return sum(done) / dt, sum(done), dt


def cpu_baseline(fn, units_per_call: int, unit: str, what: str, seconds: float):
    """The oracle, single-threaded and on every available core (threads
    over independent columns or tokens), on a bounded sample."""
    if seconds <= 0:
        return None
    host = host_description()
    n = oracle_threads()
    one = cpu_oracle_rate(fn, units_per_call, seconds / 2, 1)
    many = cpu_oracle_rate(fn, units_per_call, seconds / 2, n)
    return {
        "value": many[0], "unit": unit, "cores": n, "kind": "oracle",
        "sample": (f"{what}; plain C oracle in double; {many[1]} {unit.split('/')[0]} on "
                   f"{n} threads in {many[2]:.1f} s"),
        "single_thread": {"value": one[0], "unit": unit, "cores": 1,
                          "sample": f"{one[1]} {unit.split('/')[0]} in {one[2]:.1f} s"},
        "host": host,
    }


# ------------------------------------------------------------------ decode

def bench_decode(args, name: str, steps: int, warmup: int) -> dict:
    """One decode workload: whole-step timing over the layer rotation, the
    stamped kernel pass, the roofline entry; for the 43-layer workload also
    the 43-layer step, eager and as one captured graph."""
    import numpy as np
    import torch

    import block_quantized_expert_amd as bqe
    import synth

    cfg = synth.WORKLOADS[name]
    n_layers = args.layers or synth.ROTATION[name]
    n_var = args.variants or synth.ACTIVATION_BATCHES
    q = cfg.q
    dev = torch.device("cuda:0")

    t_setup = time.time()
    layers, xs = [], []
    lay0 = x0_host = None
    for l in range(n_layers):
        lay = synth.gen_layer(cfg, l)
        L = bqe.upload_layer(lay)
        ws = bqe.workspace(L, q)
        per = []
        for v in range(n_var):
            cols = synth.gen_columns(cfg, lay, q, variant=v, layer=l)
            x = torch.from_numpy(cols.x.view(np.int16)).view(torch.bfloat16).to(dev)
            ids, _ = bqe.moe_route_topk(L, x, ws=ws)
            ids = ids.cpu().numpy()
            if cols.drawn is not None and not np.array_equal(ids, cols.drawn):
                raise RuntimeError("routing differs from the prescribed expert sets")
            uniq = sorted(set(int(e) for e in ids.reshape(-1))) + [lay.E]
            eb = [expert_bytes(lay, e) for e in uniq]
            tot, gu = sum(b[0] for b in eb), sum(b[1] for b in eb)
            per.append({"x": x, "bytes": tot, "gu": gu, "down": tot - gu,
                        "unique": len(uniq) - 1})
            if l == 0 and v == 0:
                x0_host = cols.x.copy()
        layers.append((L, ws))
        xs.append(per)
        if l == 0:
            lay0 = lay
        del lay
        log(f"# {name}: layer {l + 1}/{n_layers} ready ({time.time() - t_setup:.1f}s)")
    y = torch.empty((q, cfg.d), dtype=torch.float32, device=dev)

    order = [(s % n_layers, (s // n_layers) % n_var) for s in range(steps)]

    def step(li, vi, events=None):
        L, ws = layers[li]
        x = xs[li][vi]["x"]
        if events is None:
            bqe.moe_layer_forward(L, x, y=y, ws=ws)
        else:
            bqe.moe_layer_forward_timed(L, x, y, ws, events)

    if args.calibrate_copy_mib > 0:
        calibration_copy(dev, args.calibrate_copy_mib)
    for s in range(warmup):
        step(s % n_layers, (s // n_layers) % n_var)
    torch.cuda.synchronize()

    def batch():
        for li, vi in order:
            step(li, vi)

    batch_ms = timed_batches(batch, BATCHES)
    ms_step = [b / steps for b in batch_ms]
    med = statistics.median(ms_step)
    mean_of = lambda key: float(np.mean([xs[li][vi][key] for li, vi in order]))  # noqa: E731
    bytes_step, gu_bytes, dn_bytes = mean_of("bytes"), mean_of("gu"), mean_of("down")
    uniq_mean = mean_of("unique")

    # stamped kernel pass
    he = HipEvents()
    evs = [he.create(6) for _ in order]
    torch.cuda.synchronize()
    for (li, vi), ev in zip(order, evs):
        step(li, vi, ev)
    torch.cuda.synchronize()
    mean_us = lambda a, b: 1e3 * float(np.mean([he.elapsed_ms(ev[a], ev[b]) for ev in evs]))  # noqa: E731
    k_route, k_gu, k_dn, span = mean_us(0, 1), mean_us(2, 3), mean_us(4, 5), mean_us(0, 5)
    for ev in evs:
        he.destroy(ev)
    route_name = "k_route" if q == 1 else "k_route+k_topk"
    router_bytes = cfg.E * cfg.d * 4 + q * cfg.d * 2
    kernels = {  # name -> (mean us, algorithmic bytes per launch, what)
        route_name: (k_route, router_bytes,
                     "router scores + prepared activations" + ("" if q == 1 else
                                                              ", then the route table")),
        "k_gateup": (k_gu, gu_bytes, ("routing + " if q == 1 else "")
                     + "gate/up dequant-GEMV + SiLU of the shared and routed experts"),
        "k_down": (k_dn, dn_bytes, "down dequant-GEMV of every slot + weighted combine"),
    }
    dom = max(kernels, key=lambda k: kernels[k][0])
    dus, dbytes, dwhat = kernels[dom]
    achieved = dbytes / (dus * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS,
                "traffic": measured_traffic(dom, name),
                "kernel": f"{dom} ({dwhat})", "bytes_per_launch": dbytes,
                "kernel_us": dus}

    out = {
        "workload": name, "q": q, "steps": steps, "warmup": warmup,
        "tokens_per_s": q / (med * 1e-3),
        "layer_steps_per_s": 1.0 / (med * 1e-3),
        "ms_per_step": med,
        "ms_per_step_batches": {"n": BATCHES, "steps_each": steps, **spread(ms_step)},
        "config": {
            "workload": cfg.name, "q": q, "d": cfg.d, "f": cfg.f, "experts": cfg.E,
            "top_k": cfg.k, "shared": 1,
            "formats": ("gate/up FP2, down FP3, shared FP4"
                        + (", 32 hottest experts FP4" if cfg.hot_fp4 else "")),
            "activations": "bf16", "accumulate": "fp32", "layers_rotated": n_layers,
            "activation_batches_per_layer": n_var, "graph_captured": False,
            "seed_master": cfg.master,
        },
        "step_hbm": {
            "packed_expert_bytes_per_step": bytes_step,
            "unique_routed_experts_per_step": uniq_mean,
            "GB_per_s": bytes_step / (med * 1e-3) / 1e9,
            "frac_of_peak": bytes_step / (med * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "router_bytes_per_step": cfg.E * cfg.d * 4,
        },
        "kernels_us": {k: v[0] for k, v in kernels.items()},
        "kernels_GB_per_s": {k: v[1] / (v[0] * 1e-6) / 1e9 for k, v in kernels.items()},
        "first_start_to_last_end_us": span,
        "roofline": roofline,
    }

    if n_layers >= 43 and q > 1:
        out["layers43_step"] = bench_layers43(bqe, layers, xs, y, steps)

    if args.cpu_seconds > 0:
        import oracle
        out["cpu_baseline"] = cpu_baseline(
            lambda: oracle.layer_forward_synth(lay0, x0_host[:1], "bf16"), 1, "tokens/s",
            f"decode columns of layer 0 of {name} (d={cfg.d}, f={cfg.f}, E={cfg.E}, "
            f"top-{cfg.k} + shared), one column per call", args.cpu_seconds)
    del layers, xs, lay0
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def bench_layers43(bqe, layers, xs, y, steps: int) -> dict:
    """The 43-layer verify step: every layer once (activation batch 0 of
    each; outputs are not chained, the layers are independent), eager and
    captured once into a HIP graph and replayed.  Timed as 5 batches of
    max(1, steps // 4) 43-layer steps each."""
    import torch
    reps = max(1, steps // 4)
    n = len(layers)

    def one_step():
        for li in range(n):
            L, ws = layers[li]
            bqe.moe_layer_forward(L, xs[li][0]["x"], y=y, ws=ws)

    def eager():
        for _ in range(reps):
            one_step()

    eager_ms = [b / reps for b in timed_batches(eager, BATCHES)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        one_step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        one_step()
    torch.cuda.synchronize()

    def graph():
        for _ in range(reps):
            g.replay()

    graph_ms = [b / reps for b in timed_batches(graph, BATCHES)]
    del g
    tokens = y.shape[0]
    return {
        "layers": n, "columns": tokens, "steps_per_batch": reps,
        "eager_ms": spread(eager_ms),
        "graph_ms": spread(graph_ms),
        "graph_tokens_per_s": tokens / (statistics.median(graph_ms) * 1e-3),
        "target_ms_at_70pct_of_8TBps": 2.02,
    }


# ----------------------------------------------------------------- prefill

def bench_prefill(args, steps: int, warmup: int) -> dict:
    """The 2048-token prefill chunk: moe_prefill_forward over layer images
    rotated so that no weight is re-read from the last-level cache."""
    import numpy as np
    import torch

    import block_quantized_expert_amd as bqe
    import synth

    name = PREFILL_WORKLOAD
    cfg = synth.WORKLOADS[name]
    dev = torch.device("cuda:0")
    n_layers = args.layers or synth.ROTATION[name]
    layers, gu_bytes, dn_bytes = [], [], []
    lay0 = x0_host = None
    rows = cfg.q * (cfg.k + 1)
    t_setup = time.time()
    for l in range(n_layers):
        lay = synth.gen_layer(cfg, l)
        L = bqe.upload_layer(lay)
        cols = synth.gen_columns(cfg, lay, cfg.q, layer=l)
        x = torch.from_numpy(cols.x.view(np.int16)).view(torch.bfloat16).to(dev)
        ws = bqe.workspace(L, cfg.q, prefill=True)
        # the routing the chunk will take (8 columns per moe_route_topk call)
        # must be the prescribed expert sets
        rws = bqe.workspace(L, 8)
        ids = np.concatenate([bqe.moe_route_topk(L, x[i:i + 8], ws=rws)[0].cpu().numpy()
                              for i in range(0, cfg.q, 8)])
        del rws
        if cols.drawn is not None and not np.array_equal(ids, cols.drawn):
            raise RuntimeError("routing differs from the prescribed expert sets")
        # algorithmic bytes of the gate/up kernel: the packed gate/up blocks of
        # every expert the chunk touches, the bf16 activations once, and h
        # written once per (token, expert) row as bf16 hi + lo
        touched = set(int(e) for e in ids.reshape(-1)) | {lay.E}
        gu_bytes.append(sum(expert_bytes(lay, e)[1] for e in touched)
                        + cfg.q * cfg.d * 2 + rows * cfg.f * 4)
        dn_bytes.append(sum(expert_bytes(lay, e)[0] - expert_bytes(lay, e)[1] for e in touched)
                        + rows * cfg.f * 4 + rows * cfg.d * 4)
        layers.append((L, x, ws))
        weight_bytes = int(lay.blob.size)
        if l == 0:
            lay0, x0_host = lay, cols.x
        del lay
        log(f"# {name}: layer {l + 1}/{n_layers} ready ({time.time() - t_setup:.1f}s)")
    y = torch.empty((cfg.q, cfg.d), dtype=torch.float32, device=dev)
    if args.calibrate_copy_mib > 0:
        calibration_copy(dev, args.calibrate_copy_mib)
    for s in range(warmup):
        L, x, ws = layers[s % n_layers]
        bqe.moe_prefill_forward(L, x, y=y, ws=ws)
    torch.cuda.synchronize()

    def batch():
        for s in range(steps):
            L, x, ws = layers[s % n_layers]
            bqe.moe_prefill_forward(L, x, y=y, ws=ws)

    ms_step = [b / steps for b in timed_batches(batch, BATCHES)]
    ms = statistics.median(ms_step)
    flops = 2.0 * rows * 3 * cfg.f * cfg.d  # gate, up and down of every (token, expert) row
    gu_flops = 2.0 * rows * 2 * cfg.f * cfg.d  # gate and up only
    dn_flops = 2.0 * rows * cfg.f * cfg.d

    he = HipEvents()
    evs = [he.create(6) for _ in range(steps)]
    torch.cuda.synchronize()
    for s, ev in enumerate(evs):
        L, x, ws = layers[s % n_layers]
        bqe.moe_prefill_forward_timed(L, x, y, ws, ev)
    torch.cuda.synchronize()
    st = {k: 1e3 * float(np.mean([he.elapsed_ms(ev[a], ev[b]) for ev in evs]))
          for k, (a, b) in {"routing_and_grouping": (0, 1), "k_pf_gateup": (2, 3),
                            "k_pf_down_and_combine": (4, 5),
                            "first_start_to_last_end": (0, 5)}.items()}
    for ev in evs:
        he.destroy(ev)
    products = {"k_pf_gateup": (st["k_pf_gateup"], gu_flops, float(np.mean(gu_bytes)),
                                "grouped gate/up product + SiLU gating"),
                "k_pf_down": (st["k_pf_down_and_combine"], dn_flops, float(np.mean(dn_bytes)),
                              "grouped down product (stamped with the combine)")}
    dom = max(products, key=lambda k: products[k][0])
    dus, dfl, dby, dwhat = products[dom]
    tfl = dfl / (dus * 1e-6) / 1e12
    out = {
        "workload": name, "tokens": cfg.q, "steps": steps, "warmup": warmup,
        "tokens_per_s": cfg.q / (ms * 1e-3),
        "ms_per_step": ms,
        "ms_per_step_batches": {"n": BATCHES, "steps_each": steps, **spread(ms_step)},
        "config": {"workload": cfg.name, "tokens": cfg.q, "d": cfg.d, "f": cfg.f,
                   "experts": cfg.E, "top_k": cfg.k, "shared": 1,
                   "formats": "gate/up FP2, down FP3, shared FP4", "activations": "bf16",
                   "layers_rotated": n_layers, "seed_master": cfg.master},
        "useful_gflop": flops / 1e9,
        "mfma_utilization": flops / (ms * 1e-3) / (MFMA_BF16_PEAK_TFLOPS * 1e12),
        "kernels_us": st,
        "kernels_bytes": {k: v[2] for k, v in products.items()},
        "roofline": {"bound": "mfma", "achieved": tfl, "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": tfl / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": measured_traffic(dom, name),
                     "kernel": f"{dom} ({dwhat})", "flops_per_launch": dfl,
                     "bytes_per_launch": dby, "kernel_us": dus},
        "weight_GB_per_s": weight_bytes / (ms * 1e-3) / 1e9,
    }
    if args.cpu_seconds > 0:
        import oracle
        out["cpu_baseline"] = cpu_baseline(
            lambda: oracle.layer_forward_synth(lay0, x0_host[:4], "bf16"), 4, "tokens/s",
            f"prefill tokens of layer 0 of {name} (d={cfg.d}, f={cfg.f}, E={cfg.E}, "
            f"top-{cfg.k} + shared), four tokens per call", args.cpu_seconds)
    del layers, lay0
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


# -------------------------------------------------------------- plain read

PLAIN_READ = "plain-read"
# the packed bytes of one q=1 decode step: its down matrices, its gate/up
# matrices, and all of them
PLAIN_READ_SIZES = {"down_q1": 26476544, "gate_up_q1": 40370176, "step_q1": 66846720}


def bench_plain_read(args, steps: int, warmup: int) -> dict:
    """rfpx_stream_read (a plain streaming read, launch included) of the
    byte counts the q=1 decode kernels stream, rotating over buffers that
    total at least 512 MiB so that no read is served by the last-level
    cache: the achievable ceiling each kernel is compared with."""
    import torch

    import block_quantized_expert_amd as bqe

    dev = torch.device("cuda:0")
    out = {"workload": PLAIN_READ, "steps": steps, "sizes": {}}
    sink = torch.zeros(bqe.lib().rfpx_stream_read_sink_words(), dtype=torch.int32, device=dev)
    for name, nbytes in PLAIN_READ_SIZES.items():
        nbuf = max(2, -(-(512 << 20) // nbytes))
        bufs = [torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device=dev) for _ in range(nbuf)]
        for s in range(warmup):
            bqe.rfpx_stream_read(bufs[s % nbuf], sink=sink)

        def batch():
            for s in range(steps):
                bqe.rfpx_stream_read(bufs[s % nbuf], sink=sink)

        us = [1e3 * b / steps for b in timed_batches(batch, BATCHES)]
        med = statistics.median(us)
        out["sizes"][name] = {"bytes": nbytes, "buffers_rotated": nbuf, "us_per_read": spread(us),
                              "GB_per_s": nbytes / (med * 1e-6) / 1e9,
                              "frac_of_peak": nbytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBS}
        del bufs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------------- dense

DENSE_WORKLOAD = "dense-fp4-16384x4096"


def bench_dense(args, steps: int, warmup: int) -> dict:
    """A dense FP4 projection of 16384 x 4096 weights (35.7 MB packed)
    applied to q = 1, 4, 5 columns: one rfpx_dense_forward call per step
    (activation preparation, the product, and the sum of split partials),
    rotating over 8 independently drawn matrices (285 MB, beyond the
    last-level cache)."""
    import numpy as np
    import torch

    import block_quantized_expert_amd as bqe
    import synth

    fmt, rows, cols, n_mat = 4, 16384, 4096, 8
    dev = torch.device("cuda:0")
    mats = []
    for i in range(n_mat):
        data = synth.random_matrix(9000 + i, fmt, rows, cols)
        mats.append(bqe.DenseMatrix(fmt, rows, cols, torch.from_numpy(data).to(dev)))
    packed = synth.matrix_bytes(fmt, rows, cols)
    out = {"workload": DENSE_WORKLOAD, "format": "FP4", "rows": rows, "cols": cols,
           "matrices_rotated": n_mat, "packed_bytes": packed, "steps": steps, "q": {}}
    rng = np.random.default_rng(1)
    for q in (1, 4, 5):
        xs = [torch.from_numpy(synth.to_bf16_bits(rng.standard_normal((q, cols))).view(np.int16))
              .view(torch.bfloat16).to(dev) for _ in range(n_mat)]
        ws = mats[0].workspace(q)
        y = torch.empty((q, rows), dtype=torch.float32, device=dev)
        for s in range(warmup):
            bqe.rfpx_dense_forward(mats[s % n_mat], xs[s % n_mat], y=y, ws=ws)

        def batch():
            for s in range(steps):
                bqe.rfpx_dense_forward(mats[s % n_mat], xs[s % n_mat], y=y, ws=ws)

        ms = [b / steps for b in timed_batches(batch, BATCHES)]
        med = statistics.median(ms)
        gbs = packed / (med * 1e-3) / 1e9
        out["q"][str(q)] = {"us_per_call": spread([1e3 * v for v in ms]),
                            "columns_per_s": q / (med * 1e-3),
                            "GB_per_s": gbs, "frac_of_peak": gbs / HBM_PEAK_GBS}
    del mats
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


# -------------------------------------------------------------------- main

def headline(w: dict, args, metric: str) -> dict:
    """The contract's fields for one workload's result."""
    return {
        "metric": metric,
        "value": w["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": w["steps"],
        "warmup": w["warmup"],
        "ms_per_step": w["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": w["config"],
        "ms_per_step_batches": w["ms_per_step_batches"],
        "roofline": w["roofline"],
        "cpu_baseline": w.get("cpu_baseline"),
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="all",
                    choices=("all",) + DECODE_WORKLOADS + (PREFILL_WORKLOAD, DENSE_WORKLOAD,
                                                          PLAIN_READ))
    ap.add_argument("--layers", type=int, default=0,
                    help="layer instances to rotate over (default: the workload's rotation)")
    ap.add_argument("--variants", type=int, default=0,
                    help="activation batches per layer instance (default 4)")
    ap.add_argument("--cpu-seconds", type=float, default=16.0,
                    help="wall time of the CPU oracle sample, split between the "
                         "single-thread and the all-core leg (0: skip)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="run one plain fp32 copy kernel (torch.neg) of this many MiB "
                         "before the timed region, to scale HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this path has no multi-GPU mode "
              f"(asked for --gpus {args.gpus}); run with --gpus 1.", file=sys.stderr)
        return 2

    import torch

    import block_quantized_expert_amd as bqe

    torch.cuda.set_device(torch.device("cuda:0"))
    bqe.lib()
    pf_steps, pf_warm = max(1, min(args.steps, 20)), min(args.warmup, 4)

    if args.workload == PREFILL_WORKLOAD:
        w = bench_prefill(args, pf_steps, pf_warm)
        out = headline(w, args, "MoE-layer prefill tokens/s (2048-token chunk) and MFMA "
                                "utilization")
        out.update({k: w[k] for k in ("useful_gflop", "mfma_utilization", "kernels_us",
                                      "kernels_bytes", "weight_GB_per_s")})
        print(json.dumps(out))
        return 0
    if args.workload == PLAIN_READ:
        print(json.dumps(bench_plain_read(args, args.steps, args.warmup)))
        return 0
    if args.workload == DENSE_WORKLOAD:
        print(json.dumps(bench_dense(args, args.steps, args.warmup)))
        return 0
    if args.workload != "all":
        w = bench_decode(args, args.workload, args.steps, args.warmup)
        out = headline(w, args, METRIC)
        out.update({k: w[k] for k in w if k not in out and k not in ("workload",)})
        print(json.dumps(out))
        return 0

    # every workload, the q=1 decode step as the headline; the CPU oracle
    # gets the full sample time on the headline workload and a shorter one
    # on the others
    res = {}
    full_cpu = args.cpu_seconds
    for name in DECODE_WORKLOADS:
        args.cpu_seconds = full_cpu if name == DECODE_WORKLOADS[0] else full_cpu / 3
        res[name] = bench_decode(args, name, args.steps, args.warmup)
        log(f"# {name}: {res[name]['ms_per_step'] * 1e3:.2f} us per step")
    args.cpu_seconds = full_cpu / 3
    res[PREFILL_WORKLOAD] = bench_prefill(args, pf_steps, pf_warm)
    log(f"# {PREFILL_WORKLOAD}: {res[PREFILL_WORKLOAD]['ms_per_step']:.3f} ms per chunk")
    dense = bench_dense(args, args.steps, args.warmup)
    log(f"# {DENSE_WORKLOAD}: " + ", ".join(
        f"q={q} {v['us_per_call']['median']:.2f} us" for q, v in dense["q"].items()))
    plain = bench_plain_read(args, args.steps, args.warmup)
    log(f"# {PLAIN_READ}: " + ", ".join(
        f"{k} {v['us_per_read']['median']:.2f} us" for k, v in plain["sizes"].items()))
    head = res[DECODE_WORKLOADS[0]]
    out = headline(head, args, METRIC)
    out["step_hbm"] = head["step_hbm"]
    out["kernels_us"] = head["kernels_us"]
    out["workloads"] = {}
    for name, w in res.items():
        slim = {k: v for k, v in w.items() if k not in ("config", "workload")}
        out["workloads"][name] = slim
    out["workloads"][DENSE_WORKLOAD] = dense
    out["workloads"][PLAIN_READ] = plain
    # each q=1 kernel against a plain read of the same bytes (launch included
    # in both): the share of the achievable ceiling it reaches
    ku = head["kernels_us"]
    out["vs_plain_read"] = {
        "k_gateup": plain["sizes"]["gate_up_q1"]["us_per_read"]["median"] / ku["k_gateup"],
        "k_down": plain["sizes"]["down_q1"]["us_per_read"]["median"] / ku["k_down"],
        "step": plain["sizes"]["step_q1"]["us_per_read"]["median"] / (head["ms_per_step"] * 1e3),
    }
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
