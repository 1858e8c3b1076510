#!/usr/bin/env python3
"""Throughput of the routed LoRA delta on one MI355X.

A step is one batch through the whole hot path: the batch's routing is built
once (admission, slots, segments, copied to the device) and the delta is then
applied on every lane of the workload for each of --layers independent layer
buffers (pool, x, y), as a decode step of a model with that many layers would.
The layer buffers together exceed the 256 MB last-level cache several times,
so every layer's factors and activations come from HBM.

Printed: one JSON line with the step throughput (delta tokens/s: active rows x
lanes x layers per second), the roofline of the delta kernels measured with
HIP events on a replayed graph of the layer launches, and the fp64 CPU oracle's
rate on a bounded sample of the same batch.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic(w, lane_name, admitted):
    """Bytes and flops the delta of one lane must move / compute for a batch:
    x of active rows, read+write of their fp32 y, A and B once per distinct
    adapter, one 4-byte slot id per token row."""
    import oracle
    L = w.lanes[lane_name].spec
    tok = oracle.token_adapters(w.seq_adapter, w.seq_len, admitted)
    act = int((tok != 0).sum())
    bx = 2
    H = L.h_out_total
    nbytes = act * (L.h_in * bx + 8 * H) + 4 * len(tok)
    flops = 0
    for aid in set(tok.tolist()) - {0}:
        n = int((tok == aid).sum())
        for sf, hj in zip(w.adapters[aid].lanes[lane_name], L.h_out):
            nbytes += 2 * sf.rank * (L.h_in + hj)
            flops += n * 2 * sf.rank * (L.h_in + hj)
    return nbytes, flops, act


def cpu_baseline(w, lanes, seconds):
    """The fp64 oracle, as it is, on the same batch, repeated for ~seconds."""
    import oracle
    t0 = time.perf_counter()
    rows = 0
    reps = 0
    while True:
        for ln in lanes:
            d, tok, _ = oracle.workload_lane_delta(w, ln)
            rows += int((tok != 0).sum())
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return rows / dt, dt, reps


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="decode_mix")
    ap.add_argument("--layers", type=int, default=64)
    ap.add_argument("--graph-reps", type=int, default=50)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--prefill-min-len", type=int, default=64)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              "(each GPU applies the delta to its own rows or its own column share "
              "independently); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import adapter_deltas_amd as m
    from workloads import config_by_name, generate
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from harness import to_device_x, to_device_y

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    spec = config_by_name(args.config)
    log(f"generating {spec.name}")
    w = generate(spec)
    lanes = [l.name for l in spec.lanes]
    T = w.n_tokens
    n_seq = len(w.seq_len)

    # layer buffers: each layer has its own pool, x and y per lane
    log(f"building {args.layers} layers x {len(lanes)} lanes")
    fac = {}
    for ln in lanes:
        fac[ln] = {aid: ([torch.from_numpy(s.A.view(np.int16)).to(dev) for s in ad.lanes[ln]],
                         [torch.from_numpy(s.B.view(np.int16)).to(dev) for s in ad.lanes[ln]],
                         [s.rank for s in ad.lanes[ln]], [s.scale for s in ad.lanes[ln]])
                   for aid, ad in w.adapters.items()}
    layers = []
    for li in range(args.layers):
        per = {}
        for ln in lanes:
            L = w.lanes[ln].spec
            pool = m.Pool(L.h_in, L.h_out, spec.n_adapters, spec.max_rank, L.x_dtype, device=dev)
            for aid, (A, B, rk, sc) in fac[ln].items():
                pool.load(aid, A, B, rk, sc, a_col0=L.a_col0)
            per[ln] = (pool, to_device_x(w.lanes[ln].x, dev), to_device_y(w.lanes[ln].y0, dev))
        layers.append(per)
    torch.cuda.synchronize()
    layer_bytes = sum(p.nbytes + x.numel() * 2 + y.numel() * 4
                      for per in layers[:1] for (p, x, y) in per.values())

    # one routing serves every lane: it is built against the pool with the most
    # slices (the others hold the same ranks on their slices)
    build_lane = max(lanes, key=lambda ln: len(w.lanes[ln].spec.h_out))
    routing = m.Routing(T, n_seq, device=dev)
    adm, nd = routing.build(layers[0][build_lane][0], w.seq_adapter, w.seq_len,
                            spec.max_loras, args.prefill_min_len)
    info = routing.info()
    ws = {ln: m.workspace_for(layers[0][ln][0], routing, dev) for ln in lanes}
    torch.cuda.synchronize()

    def step():
        routing.build(layers[0][build_lane][0], w.seq_adapter, w.seq_len, spec.max_loras,
                      args.prefill_min_len)
        for per in layers:
            for ln in lanes:
                pool, x, y = per[ln]
                m.delta_apply(pool, routing, x, y, ws[ln])

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = e0.elapsed_time(e1)
    ms_per_step = wall * 1e3 / args.steps
    delta_rows = info["n_active"] * len(lanes) * args.layers
    value = delta_rows / (ms_per_step * 1e-3)

    # kernel timing: the layer launches captured once and replayed
    log("graph replay timing")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for per in layers:
            for ln in lanes:
                pool, x, y = per[ln]
                m.delta_apply(pool, routing, x, y, ws[ln])
    stream.wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for per in layers:
            for ln in lanes:
                pool, x, y = per[ln]
                m.delta_apply(pool, routing, x, y, ws[ln])
    g.replay()
    torch.cuda.synchronize()
    g0 = torch.cuda.Event(enable_timing=True)
    g1 = torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    for _ in range(args.graph_reps):
        g.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    per_apply_us = g0.elapsed_time(g1) * 1e3 / (args.graph_reps * args.layers * len(lanes))

    nbytes = flops = 0
    for ln in lanes:
        b, f, _ = algorithmic(w, ln, adm)
        nbytes += b
        flops += f
    nbytes /= len(lanes)
    flops /= len(lanes)
    achieved_gbs = nbytes / (per_apply_us * 1e-6) / 1e9

    log(f"cpu baseline ~{args.cpu_seconds}s")
    cpu_rate, cpu_dt, cpu_reps = cpu_baseline(w, lanes, args.cpu_seconds)

    out = {
        "metric": "LoRA-delta tokens/s + achieved HBM GB/s fraction of peak, mixed-adapter decode",
        "value": round(value, 1),
        "unit": "delta tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 x/A/B, fp32 sums",
        "data": "synthetic (seeded numpy PCG64, values and batch structure of the workload)",
        "config": {
            "workload": f"{spec.name}: {spec.description}",
            "lanes": {ln: [w.lanes[ln].spec.h_in, list(w.lanes[ln].spec.h_out)] for ln in lanes},
            "tokens": T, "active_rows": info["n_active"], "distinct_adapters": nd,
            "decode_segments": info["n_decode_segments"],
            "prefill_segments": info["n_prefill_segments"],
            "layers_per_step": args.layers,
            "layer_buffer_bytes": layer_bytes,
            "step": "routing build + delta_apply on every lane of every layer",
        },
        "gpu_ms_per_step": round(gpu_ms / args.steps, 4),
        "kernel_us_per_lane_layer": round(per_apply_us, 3),
        "roofline": {
            "kernel": "delta_apply (all launches of one lane-layer)",
            "bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
            "traffic": None,
            "algorithmic_bytes_per_launch": int(nbytes),
            "algorithmic_flops_per_launch": int(flops),
        },
        "cpu_baseline": {
            "value": round(cpu_rate, 1), "unit": "delta tokens/s", "cores": 1,
            "kind": "oracle",
            "sample": f"fp64 C oracle over the whole {spec.name} batch "
                      f"({info['n_active']} active rows x {len(lanes)} lanes), "
                      f"{cpu_reps} repetitions in {cpu_dt:.1f} s",
        },
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
