"""GPU parity of the expert LoRA delta of a mixture-of-experts layer against
the fp64 oracle: dispatched (token, expert) rows routed on the device to the
pool slot of (adapter, expert)."""
import numpy as np
import pytest

import oracle
from workloads import LaneSpec, MoeSpec, generate_moe, moe_config_by_name

from harness import compare, load_moe_pool, moe_row_slots, to_device_x, to_device_y

pytestmark = pytest.mark.gpu

# 16 experts, top 4, 100 tokens (400 dispatched rows); ragged widths; ranks
# 4, 16 and 130 (the last on the matrix-core gather path); 75% of the
# (adapter, expert) pairs carry factors.
SMALL_MOE = MoeSpec(
    name="small_moe_gpu", seed=32,
    lanes=(LaneSpec("gate_up", 520, (136, 136)), LaneSpec("down", 136, (520,))),
    n_experts=16, top_k=4, n_tokens=100, n_adapters=3, ranks=(4, 16, 130), max_rank=130,
    token_input=("gate_up",), scale_mode="uniform", scale_range=(0.5, 3.0),
    base_prob=0.2, expert_coverage=0.75)


@pytest.fixture(scope="module")
def lib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import adapter_deltas_amd as m
    return m


def run_moe(m, w, lane, pool, tok_slot, path="apply", row_token=None, row_expert=None,
            x=None, y0=None):
    import torch
    L = w.lanes[lane]
    rt = w.row_token if row_token is None else row_token
    re = w.row_expert if row_expert is None else row_expert
    n = len(rt)
    routing = m.Routing(max(n, 1), max(n, 1))
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    routing.build_moe(pool, d(tok_slot), d(rt), d(re), w.spec.n_experts)
    xd = to_device_x(L.x if x is None else x)
    yd = to_device_y(L.y0 if y0 is None else y0)
    if path == "apply":
        m.delta_apply(pool, routing, xd, yd)
    else:
        v = torch.zeros(max(n, 1) * pool.v_stride, dtype=torch.float32, device="cuda")
        m.shrink(pool, routing, xd, v)
        m.expand(pool, routing, v, yd)
    torch.cuda.synchronize()
    return yd.cpu().numpy(), routing.device_counts().cpu().numpy()


def check_moe(w, lane, y, counts):
    L = w.lanes[lane]
    d_ref, row_pair = oracle.moe_lane_delta(w, lane)
    on = np.array([p is not None for p in row_pair])
    assert counts[0] == on.sum() and counts[4] == 0
    has_adapter = w.tok_adapter[w.row_token] != 0
    assert counts[5] == int((has_adapter & ~on).sum())
    assert np.array_equal(y[~on].view(np.uint32), L.y0[~on].view(np.uint32))
    if w.mode == "int":
        assert np.array_equal(y[on].astype(np.float64), L.y0[on].astype(np.float64) + d_ref[on])
        return
    st = compare(y, L.y0, d_ref[on], L.spec.h_out, rows=np.nonzero(on)[0])
    assert st["ok"], st


@pytest.mark.parametrize("mode", ["real", "int"])
@pytest.mark.parametrize("lane", ["gate_up", "down"])
@pytest.mark.parametrize("path", ["apply", "split"])
def test_small_moe_full_parity(lib, lane, mode, path):
    w = generate_moe(SMALL_MOE, mode=mode)
    pool, tok_slot = load_moe_pool(lib.Pool, w, lane)
    y, c = run_moe(lib, w, lane, pool, tok_slot, path)
    assert c[1] > 0 and c[3] > 0 and c[5] > 0      # GEMV, gather, unedited rows
    check_moe(w, lane, y, c)


@pytest.mark.parametrize("lane", ["expert_gate_up", "expert_down"])
def test_moe_decode_full_parity(lib, lane):
    """The Qwen3-30B-A3B-sized layer: 2048 dispatched rows, 128 experts."""
    w = generate_moe(moe_config_by_name("moe_decode"))
    pool, tok_slot = load_moe_pool(lib.Pool, w, lane)
    y, c = run_moe(lib, w, lane, pool, tok_slot)
    check_moe(w, lane, y, c)


def test_moe_bits_independent_of_slots_and_other_rows(lib):
    """Other adapter slots (so other pool slots), and half of the rows
    dispatched alone: every row keeps its bits."""
    w = generate_moe(SMALL_MOE)
    lane = "gate_up"
    pool, tok_slot = load_moe_pool(lib.Pool, w, lane)
    y, _ = run_moe(lib, w, lane, pool, tok_slot)
    ids = w.adapter_ids
    pool2, tok_slot2 = load_moe_pool(lib.Pool, w, lane,
                                     adapter_slot={ids[0]: 3, ids[1]: 1, ids[2]: 4})
    y2, _ = run_moe(lib, w, lane, pool2, tok_slot2)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))
    half = np.random.default_rng(4).permutation(w.n_rows)[: w.n_rows // 2]
    L = w.lanes[lane]
    y3, _ = run_moe(lib, w, lane, pool, tok_slot, row_token=w.row_token[half],
                    row_expert=w.row_expert[half], x=L.x[half], y0=L.y0[half])
    assert np.array_equal(y3.view(np.uint32), y[half].view(np.uint32))


def test_moe_invalid_rows_untouched(lib):
    w = generate_moe(SMALL_MOE)
    lane = "down"
    pool, tok_slot = load_moe_pool(lib.Pool, w, lane)
    y_ok, _ = run_moe(lib, w, lane, pool, tok_slot)
    rt, re = w.row_token.copy(), w.row_expert.copy()
    ts = tok_slot.copy()
    rng = np.random.default_rng(6)
    rows = rng.choice(w.n_rows, 9, replace=False)
    re[rows[:3]] = SMALL_MOE.n_experts            # expert out of range
    rt[rows[3:6]] = -1                            # token out of range
    # an adapter slot past the pool's adapter slots, on tokens of none of the rows above
    free = np.setdiff1d(np.arange(SMALL_MOE.n_tokens), rt[rows[:6]])
    t_bad = free[ts[free] != 0][0]
    ts[t_bad] = 7
    bad_rows = np.union1d(rows[:6], np.nonzero(rt == t_bad)[0])
    y, c = run_moe(lib, w, lane, pool, ts, row_token=rt, row_expert=re)
    assert c[4] == len(bad_rows)
    L = w.lanes[lane]
    assert np.array_equal(y[bad_rows].view(np.uint32), L.y0[bad_rows].view(np.uint32))
    keep = np.setdiff1d(np.arange(w.n_rows), bad_rows)
    assert np.array_equal(y[keep].view(np.uint32), y_ok[keep].view(np.uint32))


def test_moe_errors(lib):
    import torch
    w = generate_moe(SMALL_MOE)
    pool, tok_slot = load_moe_pool(lib.Pool, w, "down")
    z = torch.zeros(8, dtype=torch.int32, device="cuda")
    r = lib.Routing(8, 8)
    with pytest.raises(lib.LoraError):      # n_experts does not divide max_slots
        r.build_moe(pool, z, z, z, 5)
    with pytest.raises(lib.LoraError):
        r.build_moe(pool, z, z, z, 0)


def test_moe_graph_replays_any_dispatch(lib):
    """One graph of the reset of y, the MoE routing and delta_apply, replayed
    for different dispatch tables written into the same buffers."""
    import torch
    w = generate_moe(SMALL_MOE)
    lane = "gate_up"
    L = w.lanes[lane]
    pool, tok_slot = load_moe_pool(lib.Pool, w, lane)
    n = w.n_rows
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    ts_d, rt_d, re_d = d(tok_slot), d(w.row_token), d(w.row_expert)
    x, y0 = to_device_x(L.x), to_device_y(L.y0)
    routing = lib.Routing(n, n)
    routing.build_moe(pool, ts_d, rt_d, re_d, SMALL_MOE.n_experts)
    ws = lib.workspace_for(pool, routing)
    y = torch.empty_like(y0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        y.copy_(y0)
        routing.build_moe(pool, ts_d, rt_d, re_d, SMALL_MOE.n_experts)
        lib.delta_apply(pool, routing, x, y, ws)
    rng = np.random.default_rng(8)
    for i in range(3):
        re = rng.integers(0, SMALL_MOE.n_experts, n).astype(np.int32)
        ts = rng.integers(0, 4, SMALL_MOE.n_tokens).astype(np.int32)
        if i == 2:
            ts[:] = 0
        re_d.copy_(d(re))
        ts_d.copy_(d(ts))
        y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        ye, _ = run_moe(lib, w, lane, pool, ts, row_expert=re)
        assert np.array_equal(y.cpu().numpy().view(np.uint32), ye.view(np.uint32)), i



# ------------------------------------------- host routing from per-row slots

import dataclasses

# The small layer with half of its tokens in prefill chunks.
SMALL_MOE_MIXED = dataclasses.replace(SMALL_MOE, name="small_moe_mixed", prefill_frac=0.5)


def run_rows(m, w, lane, pool, row_slot, row_prefill, path="apply", rows=None):
    import torch
    L = w.lanes[lane]
    sel = np.arange(w.n_rows) if rows is None else rows
    n = len(sel)
    r = m.Routing(max(n, 1), max(n, 1))
    r.build_rows(pool, row_slot[sel], None if row_prefill is None else row_prefill[sel])
    xd, yd = to_device_x(L.x[sel]), to_device_y(L.y0[sel])
    if path == "apply":
        m.delta_apply(pool, r, xd, yd)
    else:
        v = torch.zeros(max(n, 1) * pool.v_stride, dtype=torch.float32, device="cuda")
        m.shrink(pool, r, xd, v)
        m.expand(pool, r, v, yd)
    torch.cuda.synchronize()
    return yd.cpu().numpy(), r.info()


@pytest.mark.parametrize("mode", ["real", "int"])
@pytest.mark.parametrize("lane", ["gate_up", "down"])
@pytest.mark.parametrize("path", ["apply", "split"])
def test_host_rows_mixed_prefill_parity(lib, lane, mode, path):
    """Prefill rows grouped per (adapter, expert) on the matrix cores, decode
    rows on the GEMV path (the rank-130 adapter's on the matrix cores)."""
    w = generate_moe(SMALL_MOE_MIXED, mode=mode)
    pool, tok_slot = load_moe_pool(lib.Pool, w, lane)
    rs = moe_row_slots(w, tok_slot)
    y, info = run_rows(lib, w, lane, pool, rs, w.row_prefill, path)
    assert info["n_decode_segments"] > 0 and info["n_gather_segments"] > 0
    assert info["n_active"] == int((rs != 0).sum())
    L = w.lanes[lane]
    d_ref, row_pair = oracle.moe_lane_delta(w, lane)
    on = np.array([p is not None for p in row_pair])
    assert np.array_equal(on, rs != 0)
    assert np.array_equal(y[~on].view(np.uint32), L.y0[~on].view(np.uint32))
    if mode == "int":
        assert np.array_equal(y[on].astype(np.float64), L.y0[on].astype(np.float64) + d_ref[on])
    else:
        st = compare(y, L.y0, d_ref[on], L.spec.h_out, rows=np.nonzero(on)[0])
        assert st["ok"], st


def test_host_rows_decode_equal_device_routing(lib):
    """All rows decode: the host plan and the device routing give the same
    bits; prefill rows keep their bits when dispatched alone."""
    w = generate_moe(SMALL_MOE_MIXED)
    lane = "gate_up"
    pool, tok_slot = load_moe_pool(lib.Pool, w, lane)
    rs = moe_row_slots(w, tok_slot)
    yh, _ = run_rows(lib, w, lane, pool, rs, None)
    yd, _ = run_moe(lib, w, lane, pool, tok_slot)
    assert np.array_equal(yh.view(np.uint32), yd.view(np.uint32))
    ym, _ = run_rows(lib, w, lane, pool, rs, w.row_prefill)
    sub = np.sort(np.random.default_rng(9).permutation(w.n_rows)[: w.n_rows // 3])
    ys, _ = run_rows(lib, w, lane, pool, rs, w.row_prefill, rows=sub)
    assert np.array_equal(ys.view(np.uint32), ym[sub].view(np.uint32))


def test_host_rows_errors(lib):
    """A row naming a slot that holds no pair, or a slot out of range, is an
    error before anything is copied; so is a batch past max_tokens."""
    w = generate_moe(SMALL_MOE)
    E = SMALL_MOE.n_experts
    pool, tok_slot = load_moe_pool(lib.Pool, w, "down")
    rs = moe_row_slots(w, tok_slot)
    ids = w.adapter_ids
    held = {lib.moe_slot(ids.index(aid) + 1, e, E) for (aid, e) in w.factors}
    empty = next(s for s in range(1, pool.max_slots + 1) if s not in held)
    r = lib.Routing(w.n_rows, w.n_rows)
    for s_bad in (empty, pool.max_slots + 1, -2):
        bad = rs.copy()
        bad[5] = s_bad
        with pytest.raises(lib.LoraError) as e:
            r.build_rows(pool, bad)
        assert e.value.status == "LORA_ERR_SLOT"
    with pytest.raises(lib.LoraError) as e:
        lib.Routing(8, 8).build_rows(pool, rs)
    assert e.value.status == "LORA_ERR_CAPACITY"


def test_moe_prefill_layer_parity(lib):
    """The Qwen3-30B-A3B-sized layer on a 2048-token prefill chunk (16384
    dispatched rows), expert down projection."""
    w = generate_moe(moe_config_by_name("moe_prefill"))
    lane = "expert_down"
    pool, tok_slot = load_moe_pool(lib.Pool, w, lane)
    rs = moe_row_slots(w, tok_slot)
    y, info = run_rows(lib, w, lane, pool, rs, w.row_prefill)
    assert info["n_decode_segments"] == 0 and info["n_gather_segments"] > 0
    L = w.lanes[lane]
    d_ref, row_pair = oracle.moe_lane_delta(w, lane)
    on = rs != 0
    assert np.array_equal(y[~on].view(np.uint32), L.y0[~on].view(np.uint32))
    st = compare(y, L.y0, d_ref[on], L.spec.h_out, rows=np.nonzero(on)[0])
    assert st["ok"], st


# Prefill rows only and ranks up to 32: the one-wave gather expand with its
# B tiles prefetched across segments of different (adapter, expert) pairs.
SMALL_MOE_PREFILL = dataclasses.replace(SMALL_MOE, name="small_moe_prefill", ranks=(4, 16, 32),
                                        max_rank=32, prefill_frac=1.0)


@pytest.mark.parametrize("mode", ["real", "int"])
@pytest.mark.parametrize("lane", ["gate_up", "down"])
def test_host_rows_small_groups_parity(lib, lane, mode):
    w = generate_moe(SMALL_MOE_PREFILL, mode=mode)
    pool, tok_slot = load_moe_pool(lib.Pool, w, lane)
    rs = moe_row_slots(w, tok_slot)
    y, info = run_rows(lib, w, lane, pool, rs, w.row_prefill)
    assert info["n_decode_segments"] == 0 and info["n_gather_segments"] > 0
    L = w.lanes[lane]
    d_ref, row_pair = oracle.moe_lane_delta(w, lane)
    on = rs != 0
    assert np.array_equal(y[~on].view(np.uint32), L.y0[~on].view(np.uint32))
    if mode == "int":
        assert np.array_equal(y[on].astype(np.float64), L.y0[on].astype(np.float64) + d_ref[on])
    else:
        st = compare(y, L.y0, d_ref[on], L.spec.h_out, rows=np.nonzero(on)[0])
        assert st["ok"], st
    # every third row alone: other segments, other neighbours, same bits
    sub = np.arange(0, w.n_rows, 3)
    ys, _ = run_rows(lib, w, lane, pool, rs, w.row_prefill, rows=sub)
    assert np.array_equal(ys.view(np.uint32), y[sub].view(np.uint32))


def test_moe_device_routing_at_the_row_limit(lib):
    """1024 tokens x top 8 = 8192 dispatched rows, the most the device
    routing takes (its 1024-thread, 8-key form), against the oracle."""
    spec = dataclasses.replace(SMALL_MOE, name="moe_8192", n_tokens=1024, top_k=8,
                               lanes=(LaneSpec("down", 136, (264,)),), token_input=())
    w = generate_moe(spec)
    assert w.n_rows == lib.DEVICE_ROUTING_MAX_TOKENS
    pool, tok_slot = load_moe_pool(lib.Pool, w, "down")
    y, c = run_moe(lib, w, "down", pool, tok_slot)
    check_moe(w, "down", y, c)
