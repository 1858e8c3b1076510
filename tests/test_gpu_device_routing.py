"""Routing of decode batches built on the device (lora_build_routing_device):
the delta matches the fp64 oracle and is bit-identical to the one a host-built
routing gives, rows whose slot holds no adapter are counted and left
untouched, and one captured graph of the routing and the delta serves any mix
of adapters."""
import numpy as np
import pytest

from workloads import LaneSpec, WorkloadSpec, config_by_name, generate
from harness import check_rows_against_oracle, load_lane_pool, to_device_x, to_device_y

pytestmark = pytest.mark.gpu

# Decode rows only; ranks 1..130, so both the GEMV path (decode segments) and
# the matrix-core path (gather segments) run; ragged widths, bf16 and fp16 x.
DEVICE_MIX = WorkloadSpec(
    name="device_mix", seed=23,
    lanes=(LaneSpec("qkv_like", 1544, (520, 136, 8)),
           LaneSpec("fp16_share", 4616, (264,), "fp16", tp_size=2, tp_rank=1)),
    n_adapters=6, ranks=(3, 12, 130, 1, 64, 16), rank_mode="list",
    scale_mode="uniform", scale_range=(0.25, 3.0), max_rank=130,
    decode_rows=300, base_prob=0.2, prefill_seqs=0, prefill_len=(1, 1))


@pytest.fixture(scope="module")
def lib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import adapter_deltas_amd as m
    return m


def host_apply(m, pool, x, y0, ids):
    """delta_apply with a host-built routing, one decode row per token."""
    import torch
    T = len(ids)
    routing = m.Routing(T, T)
    routing.build(pool, np.asarray(ids, np.int32), np.ones(T, np.int32), 0, m.NO_PREFILL)
    y = y0.clone()
    m.delta_apply(pool, routing, x, y)
    torch.cuda.synchronize()
    return y, routing


def device_apply(m, pool, x, y0, slots, path="apply"):
    import torch
    tok = torch.from_numpy(np.ascontiguousarray(slots, np.int32)).cuda()
    routing = m.Routing(max(len(slots), 1), max(len(slots), 1))
    routing.build_device(pool, tok)
    y = y0.clone()
    if path == "apply":
        m.delta_apply(pool, routing, x, y)
    else:
        v = torch.zeros(max(len(slots), 1) * pool.v_stride, dtype=torch.float32, device="cuda")
        m.shrink(pool, routing, x, v)
        m.expand(pool, routing, v, y)
    torch.cuda.synchronize()
    return y, routing


def slots_of(pool, ids):
    return np.array([pool.slot_of(int(a)) if a else 0 for a in ids], dtype=np.int32)


def bits(t):
    return t.cpu().numpy().view(np.uint32)


def lane_setup(lib, w, lane):
    L = w.lanes[lane]
    pool = load_lane_pool(lib.Pool, w, lane)
    return pool, to_device_x(L.x), to_device_y(L.y0)


@pytest.mark.parametrize("mode", ["real", "int"])
@pytest.mark.parametrize("cfg,lane,path", [("decode_mix", "qkv", "apply"),
                                           ("decode_mix", "qkv", "split"),
                                           ("device_mix", "qkv_like", "apply"),
                                           ("device_mix", "qkv_like", "split"),
                                           ("device_mix", "fp16_share", "apply")])
def test_device_routing_matches_host(lib, cfg, lane, path, mode):
    spec = DEVICE_MIX if cfg == "device_mix" else config_by_name(cfg)
    w = generate(spec, mode=mode)
    pool, x, y0 = lane_setup(lib, w, lane)
    ids = np.repeat(w.seq_adapter, w.seq_len)
    yh, rh = host_apply(lib, pool, x, y0, ids)
    yd, rd = device_apply(lib, pool, x, y0, slots_of(pool, ids), path)
    L = w.lanes[lane]
    check_rows_against_oracle(w, lane, ids, L.x, L.y0, yd.cpu().numpy())
    assert np.array_equal(bits(yd), bits(yh))
    c = rd.device_counts().cpu().numpy()
    hi, di = rh.info(), rd.info()
    assert c[0] == hi["n_active"] and c[2] == 0 and c[4] == 0
    assert c[1] == hi["n_decode_segments"] and c[3] == hi["n_gather_segments"]
    # the host's figures for a device-built routing are bounds
    assert di["n_active"] == len(ids)
    assert di["n_decode_segments"] >= c[1] and di["n_gather_segments"] >= c[3]
    if cfg == "device_mix":
        assert c[1] > 0 and c[3] > 0
    # the per-row slot table: the slot of every row (0 for base rows)
    assert np.array_equal(rd.token_slots().cpu().numpy(), slots_of(pool, ids))


@pytest.mark.parametrize("n", [0, 1, 7, 8, 9, 64, 65, 256, 257, 1000, 1024, 1025, 4096, 4097, 8192])
def test_device_routing_sizes(lib, n):
    """Empty, single-row, segment-edge and maximum batch sizes, and the edges
    of the routing kernel's forms (64, 256 and 1024 threads with 4 keys each,
    1024 threads with 8); adapters of both paths plus base rows."""
    w = generate(DEVICE_MIX)
    pool, x, y0 = lane_setup(lib, w, "qkv_like")
    T = x.shape[0]
    rng = np.random.default_rng(n)
    reps = -(-max(n, 1) // T)
    x = x.repeat(reps, 1)[:max(n, 1)].contiguous()
    y0 = y0.repeat(reps, 1)[:max(n, 1)].contiguous()
    ids = rng.choice(np.array([0] + list(w.adapter_ids)), n) if n else np.zeros(0, np.int32)
    yd, rd = device_apply(lib, pool, x, y0, slots_of(pool, ids))
    c = rd.device_counts().cpu().numpy()
    assert c[0] == int(np.count_nonzero(ids)) and c[4] == 0
    if n == 0:
        assert np.array_equal(bits(yd), bits(y0))
        return
    check_rows_against_oracle(w, "qkv_like", ids, x.cpu().numpy().view(np.uint16),
                              y0.cpu().numpy(), yd.cpu().numpy())
    yh, _ = host_apply(lib, pool, x, y0, ids)
    assert np.array_equal(bits(yd), bits(yh))


def test_device_routing_capacity_errors(lib):
    import torch
    w = generate(DEVICE_MIX)
    pool, _, _ = lane_setup(lib, w, "qkv_like")
    tok = torch.zeros(lib.DEVICE_ROUTING_MAX_TOKENS + 1, dtype=torch.int32, device="cuda")
    r = lib.Routing(len(tok), 1)
    with pytest.raises(lib.LoraError):
        r.build_device(pool, tok)
    r2 = lib.Routing(8, 1)
    with pytest.raises(lib.LoraError):
        r2.build_device(pool, tok[:9])
    with pytest.raises(lib.LoraError):       # built on the host: no device counts
        lib.lora_routing_device_counts(r2.handle)


def test_device_routing_invalid_slots_untouched(lib):
    w = generate(DEVICE_MIX)
    pool, x, y0 = lane_setup(lib, w, "qkv_like")        # slots 1..6 hold adapters
    ids = np.repeat(w.seq_adapter, w.seq_len)
    yh, _ = host_apply(lib, pool, x, y0, ids)
    slots = slots_of(pool, ids)
    bad = np.random.default_rng(5).choice(len(slots), 12, replace=False)
    slots[bad[:6]] = -3
    slots[bad[6:]] = pool.max_slots + 1
    yd, rd = device_apply(lib, pool, x, y0, slots)
    assert rd.device_counts().cpu().numpy()[4] == 12
    ydn, yhn, y0n = bits(yd), bits(yh), bits(y0)
    assert np.array_equal(ydn[bad], y0n[bad])
    keep = np.ones(len(slots), bool)
    keep[bad] = False
    assert np.array_equal(ydn[keep], yhn[keep])


def test_device_routing_after_unload(lib):
    """An unloaded slot holds no adapter for the device routing; a routing
    built before the unload no longer matches the pool; a reload restores
    the delta bit for bit."""
    w = generate(DEVICE_MIX)
    lane = "qkv_like"
    pool, x, y0 = lane_setup(lib, w, lane)
    ids = np.repeat(w.seq_adapter, w.seq_len)
    slots = slots_of(pool, ids)
    yh, _ = host_apply(lib, pool, x, y0, ids)
    gone = int(w.adapter_ids[2])                          # the rank-130 adapter
    s_gone = pool.slot_of(gone)
    before = lib.Routing(len(slots), len(slots))
    import torch
    before.build_device(pool, torch.from_numpy(slots).cuda())
    pool.unload(gone)
    with pytest.raises(lib.LoraError):
        lib.delta_apply(pool, before, x, y0.clone())
    yd, rd = device_apply(lib, pool, x, y0, slots)
    hit = slots == s_gone
    assert hit.any()
    assert rd.device_counts().cpu().numpy()[4] == int(hit.sum())
    assert np.array_equal(bits(yd)[hit], bits(y0)[hit])
    assert np.array_equal(bits(yd)[~hit], bits(yh)[~hit])
    ad = w.adapters[gone].lanes[lane]
    pool.load(gone, [s.A for s in ad], [s.B for s in ad], [s.rank for s in ad],
              [s.scale for s in ad], a_col0=w.lanes[lane].spec.a_col0, slot=s_gone)
    yd2, _ = device_apply(lib, pool, x, y0, slots)
    assert np.array_equal(bits(yd2), bits(yh))


def test_device_routing_graph_serves_any_mixture(lib):
    """One graph of the reset of y, the device routing and delta_apply,
    replayed for different mixes written into the same slot buffer, with
    eager work between the replays."""
    import torch
    w = generate(DEVICE_MIX)
    pool, x, y0 = lane_setup(lib, w, "qkv_like")
    T = x.shape[0]
    tok = torch.zeros(T, dtype=torch.int32, device="cuda")
    routing = lib.Routing(T, T)
    routing.build_device(pool, tok)                       # sizes the workspace
    ws = lib.workspace_for(pool, routing)
    y = torch.empty_like(y0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        y.copy_(y0)
        routing.build_device(pool, tok)
        lib.delta_apply(pool, routing, x, y, ws)
    rng = np.random.default_rng(7)
    for i in range(4):
        ids = np.where(rng.random(T) < 0.25, 0, rng.choice(w.adapter_ids, T))
        if i == 2:
            ids[:] = 0                                    # an all-base batch
        if i == 3:
            ids[:] = w.adapter_ids[2]                     # one adapter, gather path only
        tok.copy_(torch.from_numpy(slots_of(pool, ids)))
        y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        L = w.lanes["qkv_like"]
        check_rows_against_oracle(w, "qkv_like", ids, L.x, L.y0, y.cpu().numpy())
        yh, _ = host_apply(lib, pool, x, y0, ids)
        assert np.array_equal(bits(y), bits(yh)), i


def test_device_routing_padded_rows_copy_their_original(lib):
    """A batch padded to a captured size: each padded row repeats an original
    row's x, y0 and slot, and gets exactly that row's result (a row's bits
    depend only on its own row and adapter); the originals are unchanged."""
    import torch
    w = generate(DEVICE_MIX)
    pool, x, y0 = lane_setup(lib, w, "qkv_like")
    ids = np.repeat(w.seq_adapter, w.seq_len)
    n = len(ids)
    N = 512                                               # the captured size
    src = np.random.default_rng(9).integers(0, n, N - n)
    xp = torch.cat([x, x[torch.from_numpy(src).cuda()]]).contiguous()
    y0p = torch.cat([y0, y0[torch.from_numpy(src).cuda()]]).contiguous()
    slots = slots_of(pool, ids)
    yd, _ = device_apply(lib, pool, xp, y0p, np.concatenate([slots, slots[src]]))
    yh, _ = host_apply(lib, pool, x, y0, ids)
    yb = bits(yd)
    assert np.array_equal(yb[:n], bits(yh))
    assert np.array_equal(yb[n:], yb[src])


def test_relocated_adapter_leaves_its_old_slot_empty(lib):
    """Loading a resident id into another slot moves it: the old slot holds no
    adapter for the device routing (rows naming it are counted invalid and
    left untouched) nor for a plan from per-row slots (an error), and rows
    naming the new slot get the adapter's exact bits."""
    import torch
    w = generate(DEVICE_MIX)
    lane = "qkv_like"
    L = w.lanes[lane]
    pool = load_lane_pool(lib.Pool, w, lane, max_slots=8)   # slots 7 and 8 free
    x, y0 = to_device_x(L.x), to_device_y(L.y0)
    ids = np.repeat(w.seq_adapter, w.seq_len)
    yh, _ = host_apply(lib, pool, x, y0, ids)
    moved = int(w.adapter_ids[1])
    s_old = pool.slot_of(moved)
    before = slots_of(pool, ids)
    ad = w.adapters[moved].lanes[lane]
    pool.load(moved, [s.A for s in ad], [s.B for s in ad], [s.rank for s in ad],
              [s.scale for s in ad], a_col0=L.spec.a_col0, slot=8)
    assert pool.slot_of(moved) == 8
    hit = before == s_old
    assert hit.any()
    # the old slot number, as a stale caller might still write it
    yd, rd = device_apply(lib, pool, x, y0, before)
    assert rd.device_counts().cpu().numpy()[4] == int(hit.sum())
    assert np.array_equal(bits(yd)[hit], bits(y0)[hit])
    assert np.array_equal(bits(yd)[~hit], bits(yh)[~hit])
    r = lib.Routing(len(before), len(before))
    with pytest.raises(lib.LoraError) as e:
        r.build_rows(pool, before)
    assert e.value.status == "LORA_ERR_SLOT"
    # the new slot gives the adapter's bits
    yd2, _ = device_apply(lib, pool, x, y0, slots_of(pool, ids))
    assert np.array_equal(bits(yd2), bits(yh))
    check_rows_against_oracle(w, lane, ids, L.x, L.y0, yd2.cpu().numpy())
