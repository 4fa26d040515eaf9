#!/usr/bin/env python3
"""Throughput of the routed-expert forward of one MXFP4 Stable LatentMoE layer on one MI355X.

One step = moe_route_forward over one batch of seeded synthetic tokens (router, top-K, grouping by
expert, latent down-projection and shared gate/up, MXFP4 gate/up and down expert products,
gate-weighted combine, up-projection plus shared down-projection) with the inputs already resident
in HBM; the router and the x-side products run as one product over a combined weight copy, and
the step is timed on the caller's stream. The same work as two calls (moe_route, then moe_forward,
one stream) is timed too and reported beside it. Prints one JSON line.

Default workload: one GPU's TP8 share of a Kimi K3 layer at decode size (64 tokens, hidden 7168,
latent 3584, 896 experts top-16, expert intermediate 384, 2 shared experts). `--stage2 fp8` times
the layer with its FP8 second stage (h quantised to MX FP8 for the down product) instead.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed-MoE tokens/s per MI355X; HBM GB/s (decode), MFMA TFLOPS (prefill)"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense BF16 matrix cores
FP8_PEAK_TFLOPS = 5000.0        # MI355X dense FP8 matrix cores (the FP8 x FP4 down product's rate)
FP4_PEAK_TFLOPS = 10100.0       # MI355X dense MXFP4 matrix cores (the A4W4 gate/up product's rate)
MX_BYTES_PER_VALUE = 17 / 32    # E2M1 nibble + one E8M0 byte per 32 values
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CPU_MIN_SECONDS = 10.0


# Headers every kernel source includes: a change there changes the compiled kernel too.
SHARED_HEADERS = ("common.hpp", "kernels.hpp", "wave.hpp", "partials.hpp")


def source_hash(rel: str) -> str:
    """Hash of a kernel source file together with the shared headers beside it."""
    h = hashlib.sha256()
    path = os.path.join(ROOT, rel)
    for p in [path] + [os.path.join(os.path.dirname(path), n) for n in SHARED_HEADERS]:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic(shape, n_active: int) -> dict:
    """Bytes and FLOPs the layer must move / compute for one batch (intermediates excluded)."""
    s = shape
    T, K, E, Lt, I = s.T, s.K, s.E, s.Lt, s.I
    Hin = s.Hin
    expert_mx = 3 * Lt * I * MX_BYTES_PER_VALUE
    gateup_w = 2 * I * Lt * MX_BYTES_PER_VALUE
    dense_w = E * Hin * 2
    if s.has_latent:
        dense_w += 2 * Lt * s.H * 2 + 3 * s.S * s.Is * s.H * 2
    step_bytes = dense_w + n_active * expert_mx + T * Hin * 2 + T * (s.H if s.has_latent else Lt) * 2
    flops = 2 * T * E * Hin + 2 * T * K * 3 * I * Lt
    if s.has_latent:
        flops += 2 * 2 * T * s.H * Lt + 2 * 3 * T * s.S * s.Is * s.H
    return dict(
        step_bytes=step_bytes, step_flops=flops,
        # gate/up product: weights of active experts + z rows in + h rows out
        gateup_bytes=n_active * gateup_w + T * Lt * 2 + T * K * I * 2,
        gateup_flops=2 * T * K * 2 * I * Lt,
    )


def read_traffic(workload: str, kernel: str):
    """HBM bytes per launch from committed PMC counters (FETCH_SIZE + WRITE_SIZE, each scaled by the
    counter's reading for a copy of known size), or None once that kernel's source has changed."""
    try:
        with open(TRAFFIC_FILE) as f:
            d = json.load(f)
        e = d[workload][kernel]
        if e.get("source_sha256_16") != source_hash(e["source"]):
            return None
        return float(e["bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def calibrate_copy(nbytes: int) -> None:
    """A plain device copy of known size, for scaling HBM counters (run under rocprofv3 --pmc)."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reads": nbytes, "writes": nbytes}), flush=True)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="tp8_decode_t64")
    ap.add_argument("--cpu-sample", type=int, default=256,
                    help="tokens the CPU oracle evaluates (seeded sample; the whole batch if it is smaller)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES")
    ap.add_argument("--stage2", choices=("bf16", "fp8"), default="bf16",
                    help="arithmetic of the experts' down product: BF16 h (the layer as defined), or h "
                         "quantised to MX FP8 on the scaled FP8 x FP4 matrix-core instruction")
    ap.add_argument("--flush-steps", type=int, default=20,
                    help="steps timed one by one after a 1 GiB scratch write each (cache-cold distribution)")
    ap.add_argument("--stage1", choices=("bf16", "mxfp4"), default="bf16",
                    help="arithmetic of the experts' gate/up product: BF16 z (the layer as defined), or z "
                         "quantised to MX FP4 on the scaled FP4 x FP4 matrix-core instruction (A4W4)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the layer's TP8 share is measured on a single MI355X", file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return 0

    from mxfp4_latent_mixture_sigmoid_amd import abi
    if not os.path.exists(abi.LIB_PATH):
        from mxfp4_latent_mixture_sigmoid_amd import build
        build.build()
    from mxfp4_latent_mixture_sigmoid_amd import MoELayer
    from workload import SHAPES, make_inputs, sample_tokens

    shape = SHAPES[args.workload]
    T = shape.T
    print(f"[bench] workload {shape.name}: generating inputs", file=sys.stderr, flush=True)
    inp = make_inputs(shape)

    def dev(a):
        import numpy as np
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).cuda()

    weights = {k: dev(v) for k, v in inp.items() if k in abi.WEIGHT_FIELDS and v is not None}
    fp8 = args.stage2 == "fp8"
    a4 = args.stage1 == "mxfp4"
    layer = MoELayer(shape.H, shape.Lt, shape.E, shape.K, shape.I, shape.S, shape.Is, shape.has_latent,
                     weights, T_max=T, stage2_fp8=fp8, stage1_a4=a4)
    torch.cuda.synchronize()
    del weights
    x = dev(inp["x"])
    bias = dev(inp["router_bias"]) if inp.get("router_bias") is not None else None
    routing = layer.alloc_routing(T)
    out = torch.empty(T, layer.H, dtype=torch.bfloat16, device="cuda")

    def step():
        layer.route_forward(x, T, routing, out=out, logit_bias=bias)

    def step_separate():
        layer.route(x, T, routing, logit_bias=bias)
        layer.forward(x, T, routing, out=out)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = wall * 1e3 / args.steps
    print(f"[bench] timed {args.steps} steps: {ms_per_step:.4f} ms/step", file=sys.stderr, flush=True)

    # Per-step distribution: events between back-to-back steps, then steps timed one by one, each
    # after a 1 GiB scratch write outside the timed region (nothing of the layer left in the caches).
    def pct(v):
        v = sorted(v)
        q = lambda f: v[min(len(v) - 1, int(round(f * (len(v) - 1))))]   # noqa: E731
        return {"p10": round(q(0.1), 5), "p50": round(q(0.5), 5), "p90": round(q(0.9), 5), "n": len(v)}

    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    step_pct = pct([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])
    flushed_pct = None
    if args.flush_steps > 0:
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        fl = []
        for i in range(args.flush_steps):
            scratch.fill_(i & 0xFF)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            step()
            b.record(stream)
            torch.cuda.synchronize()
            fl.append(a.elapsed_time(b))
        flushed_pct = pct(fl)
        del scratch

    # The same work as two calls (moe_route, then moe_forward) on the one stream, for reference.
    for _ in range(args.warmup):
        step_separate()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step_separate()
    torch.cuda.synchronize()
    ms_separate = (time.perf_counter() - t0) * 1e3 / args.steps

    # Per-kernel durations from HIP events recorded around each launch on the same stream.
    n_launch = 16 * args.steps
    abi.profile_begin(layer.handle, n_launch)
    for _ in range(args.steps):
        step()
    prof = abi.profile_end(layer.handle, n_launch)
    per_kernel = {}
    for name, ms in prof:
        per_kernel.setdefault(name, []).append(ms)
    kernels_us = {k: round(1e3 * sum(v) / len(v), 3) for k, v in per_kernel.items()}

    counts = routing["counts"].cpu()
    n_active = int((counts > 0).sum())
    alg = algorithmic(shape, n_active)
    decode = T * shape.K <= 4 * shape.E    # few tokens per expert: weight streaming bound
    gateup_s = kernels_us["gateup"] * 1e-6
    if decode:
        gb = alg["gateup_bytes"]
        if a4:   # the gate/up product reads MX FP4 z (17/32 bytes per value) instead of BF16 z
            gb += T * shape.Lt * (MX_BYTES_PER_VALUE - 2)
        achieved = gb / gateup_s / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBPS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBPS, 4))
    else:   # a contraction against the peak of its own operand type
        peak = FP4_PEAK_TFLOPS if a4 else BF16_PEAK_TFLOPS
        achieved = alg["gateup_flops"] / gateup_s / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 2), peak=peak, unit="TFLOP/s",
                    frac=round(achieved / peak, 4))
    roof["kernel"] = "gateup"
    roof["traffic"] = None if a4 else read_traffic(shape.name, "gateup")
    down_roof = None
    if fp8:   # the FP8 x FP4 down product against its own roof
        down_s = kernels_us["down"] * 1e-6
        P = T * shape.K
        if decode:
            b = n_active * shape.Lt * shape.I * MX_BYTES_PER_VALUE + P * shape.I * 33 / 32 + P * shape.Lt * 2
            down_roof = dict(bound="hbm", achieved=round(b / down_s / 1e9, 1), peak=HBM_PEAK_GBPS, unit="GB/s")
        else:
            f = 2 * P * shape.I * shape.Lt
            down_roof = dict(bound="mfma", achieved=round(f / down_s / 1e12, 2), peak=FP8_PEAK_TFLOPS,
                             unit="TFLOP/s")
        down_roof["frac"] = round(down_roof["achieved"] / down_roof["peak"], 4)
        down_roof["kernel"] = "down"

    cpu = None
    if not args.no_cpu_baseline:
        from oracle import oracle as O
        tok = sample_tokens(shape, args.cpu_sample)
        sub = dict(inp, x=inp["x"][tok])
        print(f"[bench] CPU oracle on {len(tok)} tokens", file=sys.stderr, flush=True)
        # the sample's forward is repeated until at least CPU_MIN_SECONDS of work are timed (a small
        # batch alone is over too quickly to time the host steadily)
        passes, c0 = 0, time.perf_counter()
        while True:
            O.forward(sub, shape.K, want_intermediates=False, stage2_fp8=fp8, stage1_a4=a4)
            passes += 1
            csec = time.perf_counter() - c0
            if csec >= CPU_MIN_SECONDS:
                break
        cpu = dict(value=round(passes * len(tok) / csec, 3), unit="tokens/s", cores=O.num_threads(), kind="oracle",
                   sample=f"{len(tok)} seeded tokens of {shape.name}, full forward in FP64, {passes} pass(es) "
                          f"in {csec:.1f} s")

    step_s = ms_per_step * 1e-3
    line = {
        "metric": METRIC,
        "value": round(T / step_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "+".join(["bf16"] + (["mxfp4"] if a4 else []) + (["fp8"] if fp8 else [])),
        "data": "synthetic",
        "config": {"workload": shape.name, "tokens": T, "hidden": shape.H, "latent": shape.Lt,
                   "experts": shape.E, "top_k": shape.K, "inter": shape.I, "shared_experts": shape.S,
                   "shared_inter": shape.Is, "routing": shape.routing, "active_experts": n_active,
                   "stage1": args.stage1, "stage2": args.stage2},
        "roofline": roof,
        "cpu_baseline": cpu,
        "gpu_ms_per_step": round(gpu_ms / args.steps, 5),
        "step_ms_percentiles": step_pct,
        "step_ms_percentiles_cache_flushed": flushed_pct,
        "ms_per_step_route_then_forward": round(ms_separate, 5),
        "step_hbm_gbps": round(alg["step_bytes"] / step_s / 1e9, 1),
        "step_tflops": round(alg["step_flops"] / step_s / 1e12, 2),
        # the whole step against both roofs (the full unsharded experts sit at the ridge between them)
        "step_fracs": {"hbm": round(alg["step_bytes"] / step_s / 1e9 / HBM_PEAK_GBPS, 4),
                       "mfma": round(alg["step_flops"] / step_s / 1e12 / BF16_PEAK_TFLOPS, 4)},
        # the whole step against the roof of its regime (HBM for decode, dense BF16 for prefill)
        "step_roofline": (dict(bound="hbm", achieved=round(alg["step_bytes"] / step_s / 1e9, 1),
                               peak=HBM_PEAK_GBPS, unit="GB/s",
                               frac=round(alg["step_bytes"] / step_s / 1e9 / HBM_PEAK_GBPS, 4)) if decode else
                          dict(bound="mfma", achieved=round(alg["step_flops"] / step_s / 1e12, 2),
                               peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                               frac=round(alg["step_flops"] / step_s / 1e12 / BF16_PEAK_TFLOPS, 4))),
        "kernels_us": kernels_us,
    }
    if down_roof:
        line["roofline_down"] = down_roof
    print(json.dumps(line), flush=True)
    layer.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
