#!/usr/bin/env python3
"""Benchmark of one routed-MoE layer over block-quantized experts on MI355X.

Metric: MoE-layer decode tokens/s (verify columns per second through one
layer) and the packed expert bytes streamed per step as HBM GB/s.

Workloads (synthetic, seeded; shapes of DeepSeek-V4-Flash-class layers),
chosen with --workload:
  decode-q1-d4096-e256-top6 (default)  q=1 decode: d=4096, f=2048, 256
      experts top-6 + 1 shared; gate/up FP2, down FP3, shared FP4; bf16
      activations
  verify-q4-zipf  q=4 verify columns, Zipf(1.1) routing per column
  verify-q5-zipf-hot32fp4-43layers  q=5 verify columns, Zipf(1.1), the 32
      hottest experts FP4, 43 layers
  prefill-t2048-zipf  a 2048-token prefill chunk through one layer
A step is one moe_layer_forward call (router, top-k, batching, gate/up,
down, combine) on one batch of q columns.  Steps rotate over --layers layer
instances, each with its own router, experts and activations, so that no
weight is re-read from the 256 MB last-level cache within a rotation.

Timing: W warm-up steps, then K steps between two synchronizations, timed
with events on the stream the kernels run on.  A second pass of K steps
(moe_layer_forward_timed / moe_prefill_forward_timed) has every kernel of
interest launched through hipExtLaunchKernel with a start and an end event,
which the runtime stamps when that kernel starts and ends: the mean
duration of the dominant kernel (the gate/up kernel) is the time of the
roofline entry.  Stamped launches leave wider gaps between the kernels, so
that pass gives kernel durations only ("kernels_us"; its whole-step figures
are longer than a step); value and ms_per_step come from the first pass.
The CPU oracle is timed on a bounded sample on the host.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes as C
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer decode tokens/s and packed-weight HBM GB/s (% of peak) at q=1,4,5"
HBM_PEAK_GBS = 8000.0
HIP_EVENT_RELEASE_TO_DEVICE = 0x40000000  # hipEventReleaseToDevice


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


KERNEL_SOURCES = ("expert.hip", "prefill.hip", "route.hip", "rfpx_impl.hpp", "rfpx_route.hpp",
                  "abi.hip")


def kernel_source_hash() -> str:
    """sha256 over the sources that define the layer kernels and their launch."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "block_quantized_expert_amd", "csrc", name), "rb") as fh:
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
    if kv.get("source_sha256") != kernel_source_hash():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


MFMA_BF16_PEAK_TFLOPS = 2500.0


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
    print(f"# calibration copy: {4 * n} bytes read, {4 * n} bytes written",
          file=sys.stderr, flush=True)


def bench_prefill(args, cfg) -> int:
    """The 2048-token prefill chunk: moe_prefill_forward over layer images
    rotated so that no weight is re-read from the last-level cache."""
    import numpy as np
    import torch

    import block_quantized_expert_amd as bqe
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bqe.lib()
    n_layers = args.layers or 2
    steps = min(args.steps, 40)
    warm = min(args.warmup, 4)
    layers, gu_bytes = [], []
    lay0 = x0_host = None
    rows = cfg.q * (cfg.k + 1)
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
        layers.append((L, x, ws))
        weight_bytes = int(lay.blob.size)
        if l == 0 and args.cpu_seconds > 0:
            lay0, x0_host = lay, cols.x
        del lay
        print(f"# layer {l + 1}/{n_layers} ready", file=sys.stderr, flush=True)
    y = torch.empty((cfg.q, cfg.d), dtype=torch.float32, device=dev)
    if args.calibrate_copy_mib > 0:
        calibration_copy(dev, args.calibrate_copy_mib)
    for s in range(warm):
        L, x, ws = layers[s % n_layers]
        bqe.moe_prefill_forward(L, x, y=y, ws=ws)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for s in range(steps):
        L, x, ws = layers[s % n_layers]
        bqe.moe_prefill_forward(L, x, y=y, ws=ws)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    flops = 2.0 * rows * 3 * cfg.f * cfg.d  # gate, up and down of every (token, expert) row
    gu_flops = 2.0 * rows * 2 * cfg.f * cfg.d  # gate and up only

    # ---- timed pass: each stage's own kernel times
    he = HipEvents()
    evs = [he.create(6) for _ in range(steps)]
    torch.cuda.synchronize()
    for s, ev in enumerate(evs):
        L, x, ws = layers[s % n_layers]
        bqe.moe_prefill_forward_timed(L, x, y, ws, ev)
    torch.cuda.synchronize()
    st = {name: 1e3 * float(np.mean([he.elapsed_ms(ev[a], ev[b]) for ev in evs]))
          for name, (a, b) in {"routing_and_grouping": (0, 1), "k_pf_gateup": (2, 3),
                               "k_pf_down_and_combine": (4, 5),
                               "first_start_to_last_end": (0, 5)}.items()}
    for ev in evs:
        he.destroy(ev)
    gu_tflops = gu_flops / (st["k_pf_gateup"] * 1e-6) / 1e12

    # ---- CPU oracle on a bounded sample of the chunk: its first tokens, a
    # few at a time (each token is routed and computed on its own)
    cpu = None
    if lay0 is not None:
        import oracle
        per, n_tok = 4, 0
        t = time.time()
        while n_tok + per <= cfg.q:
            oracle.layer_forward_synth(lay0, x0_host[n_tok:n_tok + per], "bf16")
            n_tok += per
            if time.time() - t >= args.cpu_seconds:
                break
        dt = time.time() - t
        cpu = {"value": n_tok / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": (f"the first {n_tok} of the {cfg.q} tokens of layer 0 "
                          f"(d={cfg.d}, f={cfg.f}, E={cfg.E}, top-{cfg.k} + shared), plain C "
                          f"oracle in double, single thread, {dt:.1f} s")}
        del lay0
    out = {
        "metric": "MoE-layer prefill tokens/s (2048-token chunk) and MFMA utilization",
        "value": cfg.q / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "tokens": cfg.q, "d": cfg.d,
                   "f": cfg.f, "experts": cfg.E, "top_k": cfg.k, "shared": 1,
                   "formats": "gate/up FP2, down FP3, shared FP4", "activations": "bf16",
                   "layers_rotated": n_layers, "seed_master": cfg.master},
        "useful_gflop": flops / 1e9,
        "mfma_utilization": flops / (ms * 1e-3) / (MFMA_BF16_PEAK_TFLOPS * 1e12),
        "kernels_us": st,
        "roofline": {"bound": "mfma", "achieved": gu_tflops,
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": gu_tflops / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": measured_traffic("k_pf_gateup", cfg.name),
                     "kernel": "k_pf_gateup (grouped gate/up product + SiLU gating)",
                     "flops_per_launch": gu_flops,
                     "bytes_per_launch": float(np.mean(gu_bytes))},
        "weight_GB_per_s": weight_bytes / (ms * 1e-3) / 1e9,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="decode-q1-d4096-e256-top6",
                    choices=("decode-q1-d4096-e256-top6", "verify-q4-zipf",
                             "verify-q5-zipf-hot32fp4-43layers", "prefill-t2048-zipf"))
    ap.add_argument("--layers", type=int, default=0,
                    help="layer instances to rotate over (default 8; the workload's "
                         "layer count when it names one, 43 for the q=5 workload)")
    ap.add_argument("--variants", type=int, default=4,
                    help="activation batches per layer instance")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="wall time budget of the CPU oracle sample (0: skip)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="run one plain fp32 copy kernel (torch.neg) of this many MiB "
                         "before the timed region, to scale HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this path has no multi-GPU mode "
              f"(asked for --gpus {args.gpus}); run with --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import block_quantized_expert_amd as bqe
    import synth

    cfg = synth.WORKLOADS[args.workload]
    if cfg.prefill:
        return bench_prefill(args, cfg)
    n_layers = args.layers or (cfg.layers if cfg.layers > 1 else 8)
    q = cfg.q
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bqe.lib()

    # ---- setup (untimed): images, activations, expected routing
    t_setup = time.time()
    layers, xs, step_bytes, step_gu = [], [], [], []
    lay0 = None
    x0_host = None
    for l in range(n_layers):
        lay = synth.gen_layer(cfg, l)
        L = bqe.upload_layer(lay)
        ws = bqe.workspace(L, q)
        per = []
        for v in range(args.variants):
            cols = synth.gen_columns(cfg, lay, q, variant=v, layer=l)
            x = torch.from_numpy(cols.x.view(np.int16)).view(torch.bfloat16).to(dev)
            ids, _ = bqe.moe_route_topk(L, x, ws=ws)
            ids = ids.cpu().numpy()
            if cols.drawn is not None and not np.array_equal(ids, cols.drawn):
                raise RuntimeError("routing differs from the prescribed expert sets")
            uniq = sorted(set(int(e) for e in ids.reshape(-1)))
            b = sum(expert_bytes(lay, e)[0] for e in uniq) + expert_bytes(lay, lay.E)[0]
            g = sum(expert_bytes(lay, e)[1] for e in uniq) + expert_bytes(lay, lay.E)[1]
            per.append((x, b, g, len(uniq)))
            if l == 0 and v == 0:
                x0_host = cols.x.copy()
        layers.append((L, ws))
        xs.append(per)
        if l == 0:
            lay0 = lay
        else:
            del lay
        print(f"# layer {l + 1}/{n_layers} ready ({time.time() - t_setup:.1f}s)",
              file=sys.stderr, flush=True)
    y = torch.empty((q, cfg.d), dtype=torch.float32, device=dev)

    order = [(s % n_layers, (s // n_layers) % args.variants) for s in range(args.steps)]
    warm = [(s % n_layers, (s // n_layers) % args.variants) for s in range(args.warmup)]

    def step(li, vi, events=None):
        L, ws = layers[li]
        x = xs[li][vi][0]
        if events is None:
            bqe.moe_layer_forward(L, x, y=y, ws=ws)
        else:
            bqe.moe_layer_forward_timed(L, x, y, ws, events)

    if args.calibrate_copy_mib > 0:
        calibration_copy(dev, args.calibrate_copy_mib)

    for li, vi in warm:
        step(li, vi)
    torch.cuda.synchronize()

    # ---- timed pass: whole steps
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for li, vi in order:
        step(li, vi)
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ms_per_step = total_ms / args.steps
    tokens_per_s = q * args.steps / (total_ms / 1e3)
    bytes_per_step = float(np.mean([xs[li][vi][1] for li, vi in order]))
    gu_bytes = float(np.mean([xs[li][vi][2] for li, vi in order]))
    uniq_mean = float(np.mean([xs[li][vi][3] for li, vi in order]))

    # ---- timed pass: kernels of each step
    he = HipEvents()
    evs = [he.create(6) for _ in order]
    torch.cuda.synchronize()
    t0.record()
    for (li, vi), ev in zip(order, evs):
        step(li, vi, ev)
    t1.record()
    torch.cuda.synchronize()
    total_ev_ms = t0.elapsed_time(t1)
    k_route = [he.elapsed_ms(ev[0], ev[1]) for ev in evs]
    k_gu = [he.elapsed_ms(ev[2], ev[3]) for ev in evs]
    k_dn = [he.elapsed_ms(ev[4], ev[5]) for ev in evs]
    span = [he.elapsed_ms(ev[0], ev[5]) for ev in evs]
    for ev in evs:
        he.destroy(ev)
    gu_us = 1e3 * float(np.mean(k_gu))
    gu_gbs = gu_bytes / (gu_us * 1e-6) / 1e9

    # ---- CPU oracle on a bounded sample of the same workload
    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        n_steps = 0
        t = time.time()
        while True:
            oracle.layer_forward_synth(lay0, x0_host[:cfg.q], "bf16")
            n_steps += 1
            if time.time() - t >= args.cpu_seconds:
                break
        dt = time.time() - t
        cpu = {"value": n_steps * cfg.q / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": (f"{n_steps} decode steps of {cfg.q} column(s) of layer 0 "
                          f"(d={cfg.d}, f={cfg.f}, E={cfg.E}, top-{cfg.k} + shared), plain C "
                          f"oracle in double, single thread, {dt:.1f} s")}

    out = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": cfg.name, "q": q, "d": cfg.d,
            "f": cfg.f, "experts": cfg.E, "top_k": cfg.k, "shared": 1,
            "formats": ("gate/up FP2, down FP3, shared FP4"
                        + (", 32 hottest experts FP4" if cfg.hot_fp4 else "")),
            "activations": "bf16", "accumulate": "fp32",
            "layers_rotated": n_layers, "activation_batches_per_layer": args.variants,
            "graph_captured": False, "seed_master": cfg.master,
        },
        "step_hbm": {
            "packed_expert_bytes_per_step": bytes_per_step,
            "unique_routed_experts_per_step": uniq_mean,
            "GB_per_s": bytes_per_step / (ms_per_step * 1e-3) / 1e9,
            "frac_of_peak": bytes_per_step / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "router_bytes_per_step": cfg.E * cfg.d * 4,
        },
        "kernels_us": {
            ("k_route (router scores + prepared activations)" if cfg.q == 1 else
             "k_route + k_topk (router scores, prepared activations, route table)"):
                1e3 * float(np.mean(k_route)),
            ("k_gateup (routing + gate/up of the shared and routed experts)" if cfg.q == 1 else
             "k_gateup (gate/up of the shared and routed experts)"): gu_us,
            "k_down (down of all slots + combine)": 1e3 * float(np.mean(k_dn)),
            "first_start_to_last_end": 1e3 * float(np.mean(span)),
            "step_with_events": total_ev_ms * 1e3 / args.steps,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": ("k_gateup (routing + gate/up dequant-GEMV + SiLU, shared and routed)"
                       if cfg.q == 1 else
                       "k_gateup (gate/up dequant-GEMV + SiLU, shared and routed)"),
            "achieved": gu_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": gu_gbs / HBM_PEAK_GBS,
            "traffic": measured_traffic("k_gateup", cfg.name),
            "bytes_per_launch": gu_bytes,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
