#!/usr/bin/env python3
"""Throughput of the routed LoRA delta on one MI355X.

A step is one batch through the whole hot path: the batch's routing is built
once (admission, slots, segments, copied to the device) and the delta is then
applied on every lane of the workload for each of --layers independent layer
buffers (pool, x, y), as a decode step of a model with that many layers would.
By default there are enough layers for the buffers to total at least 1 GiB,
four times the 256 MB last-level cache, so every layer's factors and
activations come from HBM.

Printed: one JSON line with the step throughput (delta tokens/s: active rows x
lanes x layers per second), the roofline of the delta kernels measured with
HIP events on a replayed graph of the layer launches, and the fp64 CPU oracle's
rate on a bounded sample of the same batch.
"""
from __future__ import annotations

import argparse
import json
import os
import re
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
    """Bytes and flops the delta of one lane must move / compute for a batch,
    split by step.  Shrink: x of active rows, A once per distinct (adapter,
    slice), one 4-byte slot id per token row.  Expand: read + write of the
    active rows' fp32 y, B once per distinct (adapter, slice)."""
    L = w.lanes[lane_name].spec
    tok = np.repeat(np.where(admitted, w.seq_adapter, 0), w.seq_len)
    act = int((tok != 0).sum())
    sb = act * L.h_in * 2 + 4 * len(tok)
    eb = act * 8 * L.h_out_total
    sf_ = ef = 0
    for aid in set(tok.tolist()) - {0}:
        n = int((tok == aid).sum())
        for sf, hj in zip(w.adapters[aid].lanes[lane_name], L.h_out):
            sb += 2 * sf.rank * L.h_in
            eb += 2 * sf.rank * hj
            sf_ += n * 2 * sf.rank * L.h_in
            ef += n * 2 * sf.rank * hj
    return {"shrink": (sb, sf_), "expand": (eb, ef), "active": act}


KERNEL_SOURCES = ("include/lora.h", "adapter_deltas_amd/csrc")
# the base projection's kernel is not among the counted ones (delta_apply's)
NOT_COUNTED_SOURCES = ("kernels_linear.hip",)
COPY_CALIBRATION_BYTES = 268435456


def call_kernels(call: str, info) -> str:
    """The kernels one lora_shrink / lora_expand / lora_delta_apply call
    launches, by the kinds of segment in the batch."""
    steps = ("shrink", "expand") if call == "delta_apply" else (call,)
    ks = []
    for st in steps:
        if info["n_decode_segments"]:
            ks.append(f"k_{st}_gemv")
        if info["n_prefill_segments"] or info["n_gather_segments"]:
            ks.append(f"k_{st}_mfma")
    return f"lora_{call}: " + " + ".join(ks)


PMC_STEPS, PMC_WARMUP, PMC_LAYERS = 2, 1, 8
PMC_RUN = (f"--steps {PMC_STEPS} --warmup {PMC_WARMUP} --layers {PMC_LAYERS} --only-apply")


def kernel_step(name: str) -> str:
    """Which step of the delta a library kernel belongs to, from its name
    (k_shrink_*, k_expand_*, k_delta_* -- the last is both in one launch)."""
    m = re.search(r"\bk_(shrink|expand|delta)_\w+", name)
    return m.group(1) if m else ""


def summarize_pmc(pmc_dir: str, configs):
    """profiles/traffic.json from rocprofv3 --pmc runs of `bench.py --config
    <cfg> {PMC_RUN}`, whose only library work is lora_delta_apply on every lane
    of every layer, (warmup + steps) x layers times per lane: per workload, the
    mean HBM bytes per delta_apply call and per step of it (shrink kernels,
    expand kernels), FETCH_SIZE and WRITE_SIZE each scaled by what the same
    counter reads for a plain copy of COPY_CALIBRATION_BYTES."""
    import csv
    import statistics

    from workloads import CONFIGS, MOE_CONFIGS
    lanes_of = {c.name: len(c.lanes) for c in (*CONFIGS, *MOE_CONFIGS)}

    def per_kernel(run):
        out = {}
        with open(os.path.join(pmc_dir, run, "run_counter_collection.csv")) as f:
            for r in csv.DictReader(f):
                out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return out

    def copy_kib(run):
        vals = [statistics.median(v) for k, v in per_kernel(run).items() if "copyBuffer" in k]
        return vals[0]
    fetch_scale = COPY_CALIBRATION_BYTES / (copy_kib("copy_fetch") * 1024)
    write_scale = COPY_CALIBRATION_BYTES / (copy_kib("copy_write") * 1024)
    path = os.path.join(ROOT, "profiles", "traffic.json")
    doc = json.load(open(path)) if os.path.exists(path) else {}
    for cfg in configs:
        fetch = per_kernel(f"{cfg}_fetch")
        write = per_kernel(f"{cfg}_write")
        calls = (PMC_STEPS + PMC_WARMUP) * PMC_LAYERS * lanes_of[cfg]
        entry = {}
        for part, steps in (("delta_apply", ("shrink", "expand", "delta")),
                            ("shrink", ("shrink",)), ("expand", ("expand",))):
            names = [k for k in fetch if kernel_step(k) in steps]
            if not names:
                continue
            f_kib = sum(sum(fetch[k]) for k in names) / calls
            w_kib = sum(sum(write[k]) for k in names) / calls
            entry[part] = {
                "kernels": sorted({re.search(r"k_\w+", k).group(0) for k in names}),
                "calls": calls,
                "fetch_kib_per_call": f_kib, "write_kib_per_call": w_kib,
                "fetch_scale": round(fetch_scale, 4), "write_scale": round(write_scale, 4),
                "hbm_bytes_per_call": int(f_kib * 1024 * fetch_scale +
                                          w_kib * 1024 * write_scale),
                "sources_sha256": sources_digest(),
                "commands": [
                    f"rocprofv3 --pmc FETCH_SIZE --output-format csv -- python3 bench.py "
                    f"--copy-calibration {COPY_CALIBRATION_BYTES}",
                    f"rocprofv3 --pmc WRITE_SIZE --output-format csv -- python3 bench.py "
                    f"--copy-calibration {COPY_CALIBRATION_BYTES}",
                    f"rocprofv3 --pmc FETCH_SIZE --output-format csv -- python3 bench.py "
                    f"--config {cfg} {PMC_RUN}",
                    f"rocprofv3 --pmc WRITE_SIZE --output-format csv -- python3 bench.py "
                    f"--config {cfg} {PMC_RUN}"],
            }
        doc[cfg] = entry
    with open(path, "w") as f:
        json.dump(doc, f, indent=1, sort_keys=True)
    print(json.dumps(doc, indent=1))


def sources_digest() -> str:
    """sha256 over the library's code: a counter summary taken from other code
    no longer describes the kernels that run.  Comments and whitespace are
    left out, so edits to the documentation keep the summary valid, and so is
    the base projection's kernel source, whose kernel the counters do not
    cover."""
    import hashlib
    h = hashlib.sha256()
    comment = re.compile(r"//[^\n]*|/\*.*?\*/", re.S)
    for top in KERNEL_SOURCES:
        path = os.path.join(ROOT, top)
        files = [path] if os.path.isfile(path) else sorted(
            os.path.join(path, f) for f in os.listdir(path)
            if f.endswith((".h", ".hip", ".cpp")) and f not in NOT_COUNTED_SOURCES)
        for f in files:
            h.update(os.path.relpath(f, ROOT).encode())
            with open(f, encoding="utf-8") as fh:
                code = comment.sub(" ", fh.read())
            h.update(" ".join(code.split()).encode())
    return h.hexdigest()


def recorded_traffic(config: str, kernel: str):
    """HBM bytes per launch of `kernel` from profiles/traffic.json, if that
    summary was taken from the current sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(config, {}).get(kernel)
    if not rec or rec.get("sources_sha256") != sources_digest():
        return None
    return rec.get("hbm_bytes_per_call")


def cpu_baseline(w, lanes, seconds, threads=1):
    """The fp64 oracle, as it is, on the same batch, repeated for ~seconds.
    With threads > 1 the batch's active rows are split into chunks that the
    oracle computes on that many threads at once (its C loop runs without the
    interpreter lock)."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    chunks = {}
    for ln in lanes:
        _, tok, _ = oracle.workload_lane_delta(w, ln, rows=np.zeros(0, dtype=np.int64))
        act = np.nonzero(tok)[0]
        chunks[ln] = (len(act), [c for c in np.array_split(act, 4 * threads) if len(c)])
    t0 = time.perf_counter()
    rows = 0
    reps = 0
    with ThreadPoolExecutor(max_workers=threads) as ex:
        while True:
            for ln in lanes:
                n, parts = chunks[ln]
                if threads == 1:
                    oracle.workload_lane_delta(w, ln)
                else:
                    list(ex.map(lambda r: oracle.workload_lane_delta(w, ln, rows=r), parts))
                rows += n
            reps += 1
            if time.perf_counter() - t0 >= seconds:
                break
    dt = time.perf_counter() - t0
    return rows / dt, dt, reps


def stream_copy_gbs(dev, nbytes=1 << 30, reps=10):
    """Read + write bandwidth of a plain device copy of nbytes (context for the
    achievable fraction of the 8 TB/s peak)."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return gbs


def moe_algorithmic(w, lane_name):
    """algorithmic() for one expert projection of a MoE workload: the rows are
    the dispatched (token, expert) rows, the factors those of each distinct
    (adapter, expert) pair the batch uses."""
    L = w.lanes[lane_name].spec
    aid = w.tok_adapter[w.row_token]
    pairs = {}
    for a, e in zip(aid.tolist(), w.row_expert.tolist()):
        if a and (a, e) in w.factors:
            pairs[(a, e)] = pairs.get((a, e), 0) + 1
    act = sum(pairs.values())
    sb = act * L.h_in * 2 + 4 * w.n_rows
    eb = act * 8 * L.h_out_total
    sf_ = ef = 0
    for pair, n in pairs.items():
        for sf, hj in zip(w.factors[pair][lane_name], L.h_out):
            sb += 2 * sf.rank * L.h_in
            eb += 2 * sf.rank * hj
            sf_ += n * 2 * sf.rank * L.h_in
            ef += n * 2 * sf.rank * hj
    return {"shrink": (sb, sf_), "expand": (eb, ef), "active": act, "pairs": len(pairs)}


def linear_leg(args, spec, w, layers, routing, ws, replay_us, dev, adm):
    """The base projection with the delta in its partial sum (lora_linear_delta)
    on each bf16 lane of the workload: the fused call, the same kernel with the
    delta off (no routing), and torch.mm (bf16 in, fp32 out) followed by
    lora_delta_apply as context, each captured for enough layers to pass the
    last-level cache and replayed.  Priced against W + x + A + B + the y write
    (HBM) and against the product's flops (matrix cores)."""
    import torch
    import adapter_deltas_amd as m
    from workloads import draw_base_weight
    out = {}
    for li, L in enumerate(spec.lanes):
        if L.x_dtype != "bf16":
            continue
        W = torch.from_numpy(draw_base_weight(spec, li, L).view(np.int16)).to(dev)
        per_layer = W.numel() * 2 + layers[0][L.name][1].numel() * 2 + \
            layers[0][L.name][2].numel() * 4 + layers[0][L.name][0].nbytes
        n = min(len(layers), max(8, -(-(1 << 30) // per_layer)))
        Ws = [W] + [W.clone() for _ in range(n - 1)]
        lws = m.lora_linear_workspace_bytes(layers[0][L.name][0].handle, routing.handle)
        lw = torch.empty(max(lws, 256), dtype=torch.uint8, device=dev)

        def body(call):
            def f():
                for i in range(n):
                    pool, x, y = layers[i][L.name]
                    call(pool, x, y, Ws[i])
            return f
        fused = replay_us(body(lambda pool, x, y, Wi: m.linear_delta(pool, routing, Wi, x, y,
                                                                      lw))) / n
        base = replay_us(body(lambda pool, x, y, Wi: m.linear_delta(pool, None, Wi, x, y))) / n
        mm_note = "torch.mm(x, W^T, out_dtype=float32)"
        try:
            def tmm(pool, x, y, Wi):
                torch.mm(x.view(torch.bfloat16), Wi.view(torch.bfloat16).t(),
                         out_dtype=torch.float32, out=y)
            tmm(*layers[0][L.name], Ws[0])
        except Exception as e:       # context only: a bf16 product copied into y
            mm_note = f"torch.mm in bf16, copied to fp32 y (out_dtype failed: {e})"

            def tmm(pool, x, y, Wi):
                y.copy_(torch.mm(x.view(torch.bfloat16), Wi.view(torch.bfloat16).t()))
        torch.cuda.synchronize()
        mm_us = replay_us(body(tmm)) / n
        mm_apply = replay_us(body(lambda pool, x, y, Wi: (
            tmm(pool, x, y, Wi), m.delta_apply(pool, routing, x, y, ws[L.name])))) / n
        a = algorithmic(w, L.name, adm)
        T = w.n_tokens
        nbytes = (W.numel() * 2 + T * L.h_in * 2 + T * L.h_out_total * 4 +
                  (a["shrink"][0] - a["active"] * L.h_in * 2 - 4 * T) +
                  (a["expand"][0] - a["active"] * 8 * L.h_out_total))
        flops = 2 * T * L.h_out_total * L.h_in + a["shrink"][1] + a["expand"][1]
        gbs = nbytes / (fused * 1e-6) / 1e9
        out[L.name] = {
            "layers": n,
            "fused_us": round(fused, 3), "base_only_us": round(base, 3),
            "delta_marginal_us": round(fused - base, 3),
            "torch_mm_us": round(mm_us, 3), "torch_mm_plus_delta_apply_us": round(mm_apply, 3),
            "torch_mm": mm_note,
            "algorithmic_bytes": int(nbytes), "flops": int(flops),
            "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "mfma_frac": round(flops / (fused * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "base_only_hbm_frac": round((W.numel() * 2 + T * L.h_in * 2 + T * L.h_out_total * 4)
                                        / (base * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        }
        del Ws
    return out


def main_moe(args, spec):
    """The expert LoRA delta of MoE layers: per layer, the dispatched rows are
    routed on the device to their (adapter, expert) pool slots, then the delta
    is applied on every expert projection of the layer."""
    import torch
    import adapter_deltas_amd as m
    from workloads import generate_moe
    from workloads.device import to_device_x, to_device_y

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"generating {spec.name}")
    w = generate_moe(spec)
    # decode batches that fit are routed on the device; prefill chunks are
    # planned on the host from each row's (adapter, expert) slot
    on_device = not w.row_prefill.any() and w.n_rows <= m.DEVICE_ROUTING_MAX_TOKENS
    lanes = [l.name for l in spec.lanes]
    E = spec.n_experts
    aslot = {aid: i + 1 for i, aid in enumerate(w.adapter_ids)}
    fac = {ln: [(aid * E + e + 1, m.moe_slot(aslot[aid], e, E),
                 [torch.from_numpy(sf.A.view(np.int16)).to(dev) for sf in per[ln]],
                 [torch.from_numpy(sf.B.view(np.int16)).to(dev) for sf in per[ln]],
                 [sf.rank for sf in per[ln]], [sf.scale for sf in per[ln]])
                for (aid, e), per in w.factors.items()] for ln in lanes}

    def make_layer():
        per = {}
        for ln in lanes:
            L = w.lanes[ln].spec
            pool = m.Pool(L.h_in, L.h_out, spec.n_adapters * E, spec.max_rank, L.x_dtype,
                          device=dev)
            for pid, slot, A, B, rk, sc in fac[ln]:
                pool.load(pid, A, B, rk, sc, a_col0=L.a_col0, slot=slot)
            per[ln] = (pool, to_device_x(w.lanes[ln].x, dev), to_device_y(w.lanes[ln].y0, dev))
        return per
    layers = [make_layer()]
    layer_bytes = sum(p.nbytes + x.numel() * 2 + y.numel() * 4
                      for (p, x, y) in layers[0].values())
    if args.layers <= 0:
        args.layers = max(4, -(-(1 << 30) // layer_bytes))
    log(f"building {args.layers} layers x {len(lanes)} lanes, {layer_bytes} bytes each")
    while len(layers) < args.layers:
        layers.append(make_layer())
    del fac
    d32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    tok_slot = d32([aslot[int(a)] if a else 0 for a in w.tok_adapter])
    row_token, row_expert = d32(w.row_token), d32(w.row_expert)
    R = w.n_rows
    first = lanes[0]
    routing = m.Routing(R, R, device=dev)
    edited = np.array([bool(a) and (int(a), int(e)) in w.factors
                       for a, e in zip(w.tok_adapter[w.row_token], w.row_expert)], dtype=bool)
    row_slot = m.moe_row_slots([aslot[int(a)] if a else 0 for a in w.tok_adapter],
                               w.row_token, w.row_expert, E, edited)
    row_prefill = w.row_prefill.astype(np.uint8)

    def route(pool):
        if on_device:
            routing.build_moe(pool, tok_slot, row_token, row_expert, E)
        else:
            routing.build_rows(pool, row_slot, row_prefill)
    route(layers[0][first][0])
    ws = {ln: m.workspace_for(layers[0][ln][0], routing, dev) for ln in lanes}
    torch.cuda.synchronize()
    act_rows = int(routing.device_counts().cpu().numpy()[0]) if on_device else \
        routing.info()["n_active"]

    def step():
        for per in layers:
            route(per[first][0])
            for ln in lanes:
                pool, x, y = per[ln]
                m.delta_apply(pool, routing, x, y, ws[ln])

    warmup(args, step)
    if args.only_apply:
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        print(json.dumps({"only_apply": spec.name, "calls_per_lane":
                          (args.warmup + args.steps) * args.layers, "lanes": len(lanes)}))
        return
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = e0.elapsed_time(e1)
    ms_per_step = wall * 1e3 / args.steps
    delta_rows = act_rows * len(lanes) * args.layers
    value = delta_rows / (ms_per_step * 1e-3)

    side = torch.cuda.Stream()

    def replay_us(body):
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            body()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            body()
        g.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(args.graph_reps):
            g.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        return g0.elapsed_time(g1) * 1e3 / args.graph_reps

    vbuf = {ln: torch.empty(R * layers[0][ln][0].v_stride, dtype=torch.float32, device=dev)
            for ln in lanes}

    def per_call_us(call):
        def body():
            for per in layers:
                for ln in lanes:
                    pool, x, y = per[ln]
                    call(ln, pool, x, y)
        return replay_us(body) / (args.layers * len(lanes))

    log("graph replay timing")
    route(layers[0][first][0])
    apply_us = per_call_us(lambda ln, pool, x, y: m.delta_apply(pool, routing, x, y, ws[ln]))
    shrink_us = per_call_us(lambda ln, pool, x, y: m.shrink(pool, routing, x, vbuf[ln]))
    expand_us = per_call_us(lambda ln, pool, x, y: m.expand(pool, routing, vbuf[ln], y))
    # a host-planned routing is copied from pinned staging: no graph of the step
    step_us = replay_us(step) if on_device else None

    alg = {"shrink": [0, 0], "expand": [0, 0]}
    pairs = 0
    for ln in lanes:
        a = moe_algorithmic(w, ln)
        pairs = a["pairs"]
        for k in ("shrink", "expand"):
            alg[k][0] += a[k][0] / len(lanes)
            alg[k][1] += a[k][1] / len(lanes)
    total_bytes = alg["shrink"][0] + alg["expand"][0]
    achieved_gbs = total_bytes / (apply_us * 1e-6) / 1e9
    info = routing.info()

    log(f"cpu baseline ~{args.cpu_seconds}s")
    import oracle
    t0 = time.perf_counter()
    reps = 0
    while True:
        for ln in lanes:
            oracle.moe_lane_delta(w, ln)
        reps += 1
        if time.perf_counter() - t0 >= args.cpu_seconds:
            break
    cpu_dt = time.perf_counter() - t0
    cpu_rate = act_rows * len(lanes) * reps / cpu_dt

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
        "data": "synthetic (seeded numpy PCG64, values and dispatch structure of the workload)",
        "config": {
            "workload": f"{spec.name}: {spec.description}",
            "lanes": {ln: [w.lanes[ln].spec.h_in, list(w.lanes[ln].spec.h_out)] for ln in lanes},
            "tokens": spec.n_tokens, "dispatched_rows": R, "active_rows": act_rows,
            "distinct_adapter_expert_pairs": pairs,
            "layers_per_step": args.layers, "layer_buffer_bytes": layer_bytes,
            "step": ("per layer: MoE routing on the device" if on_device else
                     "per layer: MoE routing planned on the host from the rows' "
                     "(adapter, expert) slots, copied") +
                    ", then delta_apply on each expert projection",
            "decode_segments": routing.info()["n_decode_segments"] if not on_device else None,
            "gather_segments": routing.info()["n_gather_segments"] if not on_device else None,
        },
        "gpu_ms_per_step": round(gpu_ms / args.steps, 4),
        "graph_step_ms": round(step_us * 1e-3, 4) if step_us is not None else None,
        "roofline": {
            "kernel": call_kernels("delta_apply", info),
            "bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
            "traffic": recorded_traffic(spec.name, "delta_apply"),
            "algorithmic_bytes_per_launch": int(total_bytes),
            "us_per_launch": round(apply_us, 3),
            "note": "one lora_delta_apply call of one expert projection, its kernels "
                    "back to back in a replayed graph, HIP events on the launching stream",
        },
        "per_lane_layer": {
            "delta_apply_us": round(apply_us, 3),
            "shrink_us": round(shrink_us, 3), "expand_us": round(expand_us, 3),
            "algorithmic_bytes": int(total_bytes),
            "delta_apply_gbs": round(total_bytes / (apply_us * 1e-6) / 1e9, 1),
            "shrink_gbs": round(alg["shrink"][0] / (shrink_us * 1e-6) / 1e9, 1),
            "expand_gbs": round(alg["expand"][0] / (expand_us * 1e-6) / 1e9, 1),
            "flops": int(alg["shrink"][1] + alg["expand"][1]),
        },
        "cpu_baseline": {
            "value": round(cpu_rate, 1), "unit": "delta tokens/s", "cores": 1,
            "kind": "oracle",
            "sample": f"fp64 oracle over the whole batch ({act_rows} active dispatched rows "
                      f"x {len(lanes)} lanes), {reps} repetitions in {cpu_dt:.1f} s",
        },
    }
    print(json.dumps(out), flush=True)


# Default warmup: a step count alone left the first timed steps of a fresh
# process up to twice as slow as later ones (decode_mix: 1.64 against 0.87 ms
# per step after 10 warmup steps), so it also runs for a minimum time.
WARMUP_MIN_STEPS = 10
WARMUP_MIN_S = 0.5


def warmup(args, step):
    """Untimed warmup steps: args.warmup of them, or when not given at least
    WARMUP_MIN_STEPS and WARMUP_MIN_S seconds' worth (args.warmup is then set
    to the count run, which the JSON line reports)."""
    import torch
    if args.warmup is not None:
        log(f"warmup {args.warmup}")
        for _ in range(args.warmup):
            step()
    else:
        n, t0 = 0, time.perf_counter()
        while n < WARMUP_MIN_STEPS or time.perf_counter() - t0 < WARMUP_MIN_S:
            step()
            n += 1
            if n % WARMUP_MIN_STEPS == 0:
                torch.cuda.synchronize()     # time what the device has done
        args.warmup = n
        log(f"warmup {n} steps")
    torch.cuda.synchronize()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warmup steps (default: at least %d steps and %.1f s of "
                         "them, so that clocks and first-touch costs have settled)"
                         % (WARMUP_MIN_STEPS, WARMUP_MIN_S))
    ap.add_argument("--config", default="decode_mix")
    ap.add_argument("--layers", type=int, default=0,
                    help="layer buffer sets (default: enough for 1 GiB, at least 16)")
    ap.add_argument("--graph-reps", type=int, default=50)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--prefill-min-len", type=int, default=64)
    ap.add_argument("--no-linear", action="store_true",
                    help="skip the base projection with the delta in its epilogue")
    ap.add_argument("--only-apply", action="store_true",
                    help="only run the steps (routing + delta_apply per lane and layer), "
                         "for counter passes: no graph timing, no CPU baseline")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes 10 times (the "
                         "reference kernel that scales HBM byte counters)")
    ap.add_argument("--summarize-pmc", default="", metavar="DIR",
                    help="only write profiles/traffic.json from rocprofv3 --pmc output "
                         "in DIR for the workloads given with --config (comma list)")
    args = ap.parse_args()

    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc, args.config.split(","))
        return

    if args.copy_calibration:
        import torch
        n = args.copy_calibration // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n * 4, "launches": 10}))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              "(each GPU applies the delta to its own rows or its own column share "
              "independently); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    from workloads import MOE_CONFIGS
    moe = {c.name: c for c in MOE_CONFIGS}
    if args.config in moe:
        main_moe(args, moe[args.config])
        return

    import torch
    import adapter_deltas_amd as m
    from workloads import config_by_name, generate
    from workloads.device import to_device_x, to_device_y

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
    fac = {}
    for ln in lanes:
        fac[ln] = {aid: ([torch.from_numpy(s.A.view(np.int16)).to(dev) for s in ad.lanes[ln]],
                         [torch.from_numpy(s.B.view(np.int16)).to(dev) for s in ad.lanes[ln]],
                         [s.rank for s in ad.lanes[ln]], [s.scale for s in ad.lanes[ln]])
                   for aid, ad in w.adapters.items()}
    def make_layer():
        per = {}
        for ln in lanes:
            L = w.lanes[ln].spec
            pool = m.Pool(L.h_in, L.h_out, spec.n_adapters, spec.max_rank, L.x_dtype, device=dev)
            for aid, (A, B, rk, sc) in fac[ln].items():
                pool.load(aid, A, B, rk, sc, a_col0=L.a_col0)
            per[ln] = (pool, to_device_x(w.lanes[ln].x, dev), to_device_y(w.lanes[ln].y0, dev))
        return per
    layers = [make_layer()]
    layer_bytes = sum(p.nbytes + x.numel() * 2 + y.numel() * 4
                      for (p, x, y) in layers[0].values())
    if args.layers <= 0:
        args.layers = max(16, -(-(1 << 30) // layer_bytes))
    log(f"building {args.layers} layers x {len(lanes)} lanes, {layer_bytes} bytes each")
    while len(layers) < args.layers:
        layers.append(make_layer())
    torch.cuda.synchronize()

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

    warmup(args, step)
    if args.only_apply:
        # a counter pass: the library's only work is delta_apply on every lane
        # of every layer, (warmup + steps) x layers times per lane
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        print(json.dumps({"only_apply": spec.name, "calls_per_lane":
                          (args.warmup + args.steps) * args.layers, "lanes": len(lanes)}))
        return

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

    # Kernel timing: each call's launches for every layer and lane captured
    # once as a graph and replayed; HIP events on the launching stream.
    side = torch.cuda.Stream()
    vbuf = {ln: torch.empty(max(info["n_active"], 1) * layers[0][ln][0].v_stride,
                            dtype=torch.float32, device=dev) for ln in lanes}

    def graph_us(call):
        def body():
            for per in layers:
                for ln in lanes:
                    pool, x, y = per[ln]
                    call(ln, pool, x, y)
        return replay_us(body) / (args.layers * len(lanes))

    def replay_us(body):
        """Microseconds per replay of one graph of body's launches."""
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            body()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            body()
        g.replay()
        torch.cuda.synchronize()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(args.graph_reps):
            g.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        return g0.elapsed_time(g1) * 1e3 / args.graph_reps

    # The host half of the step alone: admission, segments, pinned staging and
    # the enqueue of the copy (the copy itself runs on the device).
    log("host routing timing")
    n_route = 200
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n_route):
        routing.build(layers[0][build_lane][0], w.seq_adapter, w.seq_len, spec.max_loras,
                      args.prefill_min_len)
    route_host_us = (time.perf_counter() - t0) * 1e6 / n_route
    torch.cuda.synchronize()

    log("graph replay timing")
    per_apply_us = graph_us(lambda ln, pool, x, y: m.delta_apply(pool, routing, x, y, ws[ln]))
    shrink_us = graph_us(lambda ln, pool, x, y: m.shrink(pool, routing, x, vbuf[ln]))
    expand_us = graph_us(lambda ln, pool, x, y: m.expand(pool, routing, vbuf[ln], y))

    # A decode-only batch can also be routed on the device: one graph then
    # holds the routing kernel and every layer's delta, with no host work.
    device_routing = None
    if np.all(w.seq_len == 1) and T <= m.DEVICE_ROUTING_MAX_TOKENS:
        log("device routing timing")
        tok = routing.token_slots().clone()
        pool0 = layers[0][build_lane][0]
        droute = m.Routing(T, T, device=dev)
        droute.build_device(pool0, tok)
        dws = {ln: m.workspace_for(layers[0][ln][0], droute, dev) for ln in lanes}

        def dstep():
            droute.build_device(pool0, tok)
            for per in layers:
                for ln in lanes:
                    pool, x, y = per[ln]
                    m.delta_apply(pool, droute, x, y, dws[ln])
        def route32():
            for _ in range(32):
                droute.build_device(pool0, tok)
        route_us = replay_us(route32) / 32
        dstep_us = replay_us(dstep)
        device_routing = {
            "route_us": round(route_us, 3),
            "graph_step_ms": round(dstep_us * 1e-3, 4),
            "graph_value": round(delta_rows / (dstep_us * 1e-6), 1),
            "note": "the same step as one graph replay: the routing kernel on the "
                    "per-row slots, then delta_apply on every lane of every layer",
        }

    linear = None
    if not args.no_linear and any(l.x_dtype == "bf16" for l in spec.lanes):
        log("base projection with the delta in its epilogue")
        linear = linear_leg(args, spec, w, layers, routing, ws, replay_us, dev, adm)

    alg = {"shrink": [0, 0], "expand": [0, 0]}
    for ln in lanes:
        a = algorithmic(w, ln, adm)
        for k in ("shrink", "expand"):
            alg[k][0] += a[k][0] / len(lanes)
            alg[k][1] += a[k][1] / len(lanes)
    total_bytes = alg["shrink"][0] + alg["expand"][0]
    # The headline is the whole delta of a lane: lora_delta_apply (shrink and
    # expand) priced with all its algorithmic bytes over the time per call.
    achieved_gbs = total_bytes / (per_apply_us * 1e-6) / 1e9
    traffic = recorded_traffic(spec.name, "delta_apply")

    log(f"cpu baseline ~{args.cpu_seconds}s")
    cpu_rate, cpu_dt, cpu_reps = cpu_baseline(w, lanes, args.cpu_seconds)
    host_cpus = os.cpu_count() or 1
    n_thr = max(1, min(16, host_cpus))
    log(f"cpu baseline on {n_thr} threads ~{args.cpu_seconds / 2}s")
    par_rate, par_dt, par_reps = cpu_baseline(w, lanes, args.cpu_seconds / 2, n_thr)
    log("stream copy context")
    copy_gbs = stream_copy_gbs(dev)

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
            "gather_segments": info["n_gather_segments"],
            "layers_per_step": args.layers,
            "layer_buffer_bytes": layer_bytes,
            "step": "routing build + delta_apply on every lane of every layer",
        },
        "gpu_ms_per_step": round(gpu_ms / args.steps, 4),
        "routing_host_us": round(route_host_us, 2),
        "roofline": {
            "kernel": call_kernels("delta_apply", info),
            "bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": int(total_bytes),
            "us_per_launch": round(per_apply_us, 3),
            "note": "one lora_delta_apply call of one lane: its kernels back to back "
                    "in a replayed graph of every layer's call, HIP events on the "
                    "launching stream",
        },
        "per_launch": {
            "shrink": {"kernel": call_kernels("shrink", info), "us": round(shrink_us, 3),
                       "algorithmic_bytes": int(alg["shrink"][0]),
                       "frac": round(alg["shrink"][0] / (shrink_us * 1e-6) / 1e9 /
                                     HBM_PEAK_GBS, 4),
                       "traffic": recorded_traffic(spec.name, "shrink")},
            "expand": {"kernel": call_kernels("expand", info), "us": round(expand_us, 3),
                       "algorithmic_bytes": int(alg["expand"][0]),
                       "frac": round(alg["expand"][0] / (expand_us * 1e-6) / 1e9 /
                                     HBM_PEAK_GBS, 4),
                       "traffic": recorded_traffic(spec.name, "expand")},
        },
        "per_lane_layer": {
            "delta_apply_us": round(per_apply_us, 3),
            "shrink_us": round(shrink_us, 3), "expand_us": round(expand_us, 3),
            "algorithmic_bytes": int(total_bytes),
            "delta_apply_gbs": round(total_bytes / (per_apply_us * 1e-6) / 1e9, 1),
            "shrink_gbs": round(alg["shrink"][0] / (shrink_us * 1e-6) / 1e9, 1),
            "expand_gbs": round(alg["expand"][0] / (expand_us * 1e-6) / 1e9, 1),
            "flops": int(alg["shrink"][1] + alg["expand"][1]),
        },
        "cpu_baseline": {
            "value": round(cpu_rate, 1), "unit": "delta tokens/s", "cores": 1,
            "kind": "oracle", "host_cpus": host_cpus,
            "sample": f"fp64 C oracle over the whole {spec.name} batch "
                      f"({info['n_active']} active rows x {len(lanes)} lanes), "
                      f"{cpu_reps} repetitions in {cpu_dt:.1f} s, one thread",
        },
        "cpu_baseline_threads": {
            "value": round(par_rate, 1), "unit": "delta tokens/s", "cores": n_thr,
            "kind": "oracle", "host_cpus": host_cpus,
            "sample": f"the same oracle on row chunks of the batch over {n_thr} threads "
                      f"(the host reports {host_cpus} CPUs; at most 16 are used, the "
                      f"CPU share of one GPU), {par_reps} repetitions in {par_dt:.1f} s",
        },
        "device_routing": device_routing,
        "linear_delta": linear,
        "context": {
            "stream_copy_gbs": round(copy_gbs, 1),
            "stream_copy": "torch copy of 1 GiB, read + write bytes per second",
        },
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
