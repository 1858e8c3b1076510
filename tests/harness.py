"""Test helpers: run a workload lane through the C ABI and compare it with the
fp64 oracle.

Tolerance rule for real-valued inputs (bf16 or fp16 inputs, fp32 sums): per
element, with d_gpu = y_gpu - y0 and d_ref the oracle's delta,
    |d_gpu - d_ref| <= 1e-2 * |d_ref|   or   |d_gpu - d_ref| <= 2e-3 * N
where N is the largest |d_ref| over the same row and output slice.  Rows the
routing leaves alone (base model, deferred, outside the batch) must keep the
exact bits of y0, and integer-mode inputs must give exact results.
"""
from __future__ import annotations

import numpy as np

from workloads.device import to_device_x, to_device_y  # noqa: F401  (re-exported)

REL_TOL = 1e-2
NORM_ABS_TOL = 2e-3


def seq_starts(lens):
    lens = np.asarray(lens, dtype=np.int64)
    return np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)


def compare(y_gpu, y0, d_ref, h_out, rows=None):
    """Tolerance check of active rows.  Returns a stats dict with 'ok'."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    y0 = np.asarray(y0, dtype=np.float64)
    if rows is not None:
        y_gpu, y0 = y_gpu[rows], y0[rows]
    d_gpu = y_gpu - y0
    err = np.abs(d_gpu - d_ref)
    ok = np.ones_like(err, dtype=bool)
    abs_branch = 0
    max_rel = 0.0     # over elements with |d_ref| >= 1e-3 N
    max_nabs = 0.0
    col = 0
    for hj in h_out:
        ref = d_ref[:, col:col + hj]
        e = err[:, col:col + hj]
        N = np.abs(ref).max(axis=1, keepdims=True)
        rel_ok = e <= REL_TOL * np.abs(ref)
        abs_ok = e <= NORM_ABS_TOL * N
        ok[:, col:col + hj] = rel_ok | abs_ok
        abs_branch += int((~rel_ok & abs_ok).sum())
        with np.errstate(divide="ignore", invalid="ignore"):
            big = np.abs(ref) >= 1e-3 * N
            rel = np.where(big, e / np.where(big, np.abs(ref), 1.0), 0.0)
            nabs = np.where(N > 0, e / np.where(N > 0, N, 1.0), np.where(e > 0, np.inf, 0.0))
        if rel.size:
            max_rel = max(max_rel, float(rel.max()))
            max_nabs = max(max_nabs, float(nabs.max()))
        col += hj
    return dict(ok=bool(ok.all()), n_bad=int((~ok).sum()), n=int(ok.size),
                max_rel=max_rel, max_norm_abs=max_nabs, abs_branch=abs_branch)


def load_lane_pool(Pool, workload, lane_name, max_slots=None, max_rank=None,
                   slot_of=None, device="cuda", on_device=False):
    """Pool for one lane with every adapter of the workload loaded.

    slot_of: optional dict registry id -> slot (default: lowest free slot)."""
    import torch
    spec = workload.spec
    lane = workload.lanes[lane_name].spec
    ms = max_slots or spec.n_adapters
    mr = max_rank or spec.max_rank
    pool = Pool(lane.h_in, lane.h_out, ms, mr, lane.x_dtype, device=device)
    for aid, ad in workload.adapters.items():
        sl = ad.lanes[lane_name]
        A = [s.A for s in sl]
        B = [s.B for s in sl]
        if on_device:
            A = [torch.from_numpy(a.view(np.int16)).to(device) for a in A]
            B = [torch.from_numpy(b.view(np.int16)).to(device) for b in B]
        pool.load(aid, A, B, [s.rank for s in sl], [s.scale for s in sl],
                  a_col0=lane.a_col0, slot=(slot_of or {}).get(aid, -1))
    return pool


def load_moe_pool(Pool, workload, lane_name, adapter_slot=None, device="cuda"):
    """Pool of one expert projection of a MoE workload: the pair of (adapter,
    expert) in slot moe_slot(adapter slot, expert, n_experts).

    adapter_slot: registry id -> adapter slot (default: 1 + adapter index).
    Returns (pool, tok_slot int32 [n_tokens] of adapter slots, 0 = base)."""
    from adapter_deltas_amd import moe_slot
    spec = workload.spec
    E = spec.n_experts
    ids = workload.adapter_ids
    if adapter_slot is None:
        adapter_slot = {aid: i + 1 for i, aid in enumerate(ids)}
    n_slots = max(adapter_slot.values())
    lane = workload.lanes[lane_name].spec
    pool = Pool(lane.h_in, lane.h_out, n_slots * E, spec.max_rank, lane.x_dtype, device=device)
    for (aid, e), per_lane in workload.factors.items():
        sl = per_lane[lane_name]
        pool.load(aid * E + e + 1, [s.A for s in sl], [s.B for s in sl], [s.rank for s in sl],
                  [s.scale for s in sl], a_col0=lane.a_col0,
                  slot=moe_slot(adapter_slot[aid], e, E))
    tok_slot = np.array([adapter_slot[int(a)] if a else 0 for a in workload.tok_adapter],
                        dtype=np.int32)
    return pool, tok_slot


def moe_row_slots(workload, tok_slot):
    """Pool slot of every dispatched row of a MoE workload (0 for rows of base
    tokens and of experts the token's adapter does not edit), for
    lora_build_routing_rows."""
    from adapter_deltas_amd import moe_row_slots as slots
    return slots(tok_slot, workload.row_token, workload.row_expert, workload.spec.n_experts,
                 moe_rows_edited(workload))


def moe_rows_edited(workload):
    """Whether each dispatched row's token runs an adapter that edits the row's
    expert (has factors for it)."""
    ids = workload.tok_adapter[workload.row_token]
    return np.array([bool(a) and (int(a), int(e)) in workload.factors
                     for a, e in zip(ids, workload.row_expert)], dtype=bool)


def oracle_row_chunks(workload, lane_name, rows, chunk=256, threads=None):
    """Yields (row indices, oracle delta float64 [len, H_out]) over `rows` in
    chunks, the chunks computed by the fp64 oracle on host threads (its C loop
    runs without the interpreter lock), in order."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    rows = np.asarray(rows, dtype=np.int64)
    parts = [rows[i:i + chunk] for i in range(0, len(rows), chunk)]
    n = threads or max(1, min(16, os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=n) as ex:
        futs = [ex.submit(lambda r: oracle.workload_lane_delta(workload, lane_name, rows=r)[0], r)
                for r in parts]
        for r, f in zip(parts, futs):
            yield r, f.result()


def check_rows_against_oracle(workload, lane_name, tok_adapter, x_bits, y0, y):
    """Rows of a batch given per row as registry ids (0 = base): base rows keep
    the bits of y0, the others hold y0 + delta, exactly for integer inputs and
    within the tolerance rule otherwise.  x_bits, y0 and y are the batch's own
    rows (host arrays)."""
    import oracle
    L = workload.lanes[lane_name]
    tok = np.asarray(tok_adapter, dtype=np.int64)
    factors = {aid: [(s.A, s.B, s.rank, s.scale) for s in ad.lanes[lane_name]]
               for aid, ad in workload.adapters.items()}
    off = tok == 0
    y = np.asarray(y)
    assert np.array_equal(y[off].view(np.uint32), np.asarray(y0)[off].view(np.uint32))
    act = np.nonzero(~off)[0]
    if len(act) == 0:
        return
    d = oracle.lane_delta(x_bits, L.spec.x_dtype, tok, factors, L.spec.h_out, L.spec.a_col0,
                          L.spec.h_in, rows=act)
    if workload.mode == "int":
        assert np.array_equal(y[act].astype(np.float64),
                              np.asarray(y0)[act].astype(np.float64) + d)
    else:
        st = compare(y, y0, d, L.spec.h_out, rows=act)
        assert st["ok"], st
