"""GPU parity of the base projection with the delta in its partial sum
(lora_linear_delta) against the fp64 oracle, through the C ABI.

y = x W^T for every row, plus the delta of each adapter row added to the
accumulator before the one store.  Real inputs are held to the tolerance rule
of tests/harness.py (with y0 = 0, so the rule applies to y itself), integer
inputs must be exact; base rows must equal the same kernel's base product bit
for bit, and with W = 0 the result is the delta alone, held to the same rule
(so a wrong delta cannot hide under a large base product).
"""
import numpy as np
import pytest

import oracle
from workloads import LaneSpec, WorkloadSpec, config_by_name, draw_base_weight, generate
from workloads.device import to_device_x, to_device_y

from harness import compare, load_lane_pool

pytestmark = pytest.mark.gpu

# decode, prefill and gather rows; h_in = 24 K-tiles + 8 (a ragged K tail),
# 664 outputs over three slices (tiles straddle slice edges), 190-ish rows
RAGGED = WorkloadSpec(
    name="linear_ragged", seed=51,
    lanes=(LaneSpec("qkv_like", 1544, (520, 136, 8)),),
    n_adapters=5, ranks=(3, 12, 17, 1, 130), rank_mode="list",
    scale_mode="uniform", scale_range=(0.25, 3.0), max_rank=130,
    decode_rows=90, base_prob=0.2, prefill_seqs=4, prefill_len=(1, 150))


# ranks up to 256 on one 1024-wide slice (no 16-column group straddles an edge)
HIGH_RANK = WorkloadSpec(
    name="linear_high_rank", seed=52,
    lanes=(LaneSpec("wide", 1032, (1024,)),),
    n_adapters=4, ranks=(256, 130, 40, 7), rank_mode="list",
    scale_mode="uniform", scale_range=(0.25, 3.0), max_rank=256,
    decode_rows=60, base_prob=0.2, prefill_seqs=3, prefill_len=(1, 90))


# large enough for the 256 x 128 tile (at least 512 of them): 4104 outputs
# over three slices (tiles straddle the slice edges; the last tile is 8
# wide), about 3900 rows of decode and prefill sequences, K = 520 (8 K-tiles
# and a tail)
LARGE_RAGGED = WorkloadSpec(
    name="linear_large_ragged", seed=54,
    lanes=(LaneSpec("wide_out", 520, (2056, 1024, 1024)),),
    n_adapters=12, ranks=(8, 16, 32, 64, 128, 3, 17, 40, 100, 8, 16, 64), rank_mode="list",
    scale_mode="uniform", scale_range=(0.25, 3.0), max_rank=128,
    decode_rows=3000, base_prob=0.2, prefill_seqs=6, prefill_len=(100, 200))


# every decode row its own adapter of rank 256 on two slices: about 60
# distinct slots in a 64-row tile, 32 delta steps each, past what one tile
# holds, so the call takes the base product and then lora_delta_apply
STEP_OVERFLOW = WorkloadSpec(
    name="linear_step_overflow", seed=53,
    lanes=(LaneSpec("two", 136, (72, 64)),),
    n_adapters=96, ranks=(256,) * 96, rank_mode="list",
    scale_mode="uniform", scale_range=(0.25, 2.0), max_rank=256,
    decode_rows=128, base_prob=0.0, popularity="uniform")


@pytest.fixture(scope="module")
def lib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import adapter_deltas_amd as m
    return m


def w_device(W):
    import torch
    return torch.from_numpy(np.ascontiguousarray(W).view(np.int16)).cuda()


def run_linear(m, w, lane, W, with_routing=True, prefill_min_len=64, pool=None, rows=None,
               seq=None):
    """(y, routing info or None) of lora_linear_delta on the workload's batch
    (or on the sequences `seq` = (ids, lens) with x rows `rows`)."""
    import torch
    L = w.lanes[lane]
    pool = pool or load_lane_pool(m.Pool, w, lane)
    ids, lens = seq if seq is not None else (w.seq_adapter, w.seq_len)
    x = L.x if rows is None else L.x[rows]
    T = int(np.sum(lens))
    xd = to_device_x(x)
    yd = torch.full((T, L.spec.h_out_total), float("nan"), device="cuda")
    routing = None
    if with_routing:
        routing = m.Routing(max(T, 1), max(len(ids), 1))
        routing.build(pool, ids, lens, w.spec.max_loras, prefill_min_len)
    m.linear_delta(pool, routing, w_device(W), xd, yd)
    torch.cuda.synchronize()
    return yd.cpu().numpy(), (routing.info() if routing else None), pool, routing


def check_against_oracle(w, lane, W, y, rows=None):
    L = w.lanes[lane]
    ref, tok, _ = oracle.workload_linear_lane(w, lane, W, rows=rows)
    yy = y if rows is None else y[rows]
    if w.mode == "int":
        assert np.array_equal(yy.astype(np.float64), ref)
    else:
        st = compare(yy, np.zeros_like(yy), ref, L.spec.h_out)
        assert st["ok"], st
    return tok


@pytest.mark.parametrize("mode", ["real", "int"])
@pytest.mark.parametrize("cfg,lane", [("decode_mix", "qkv"), ("ragged", "qkv_like"),
                                      ("high_rank", "wide"), ("large", "wide_out")])
def test_linear_matches_oracle(lib, cfg, lane, mode):
    spec = {"ragged": RAGGED, "high_rank": HIGH_RANK,
            "large": LARGE_RAGGED}.get(cfg) or config_by_name(cfg)
    w = generate(spec, mode=mode, lanes=(lane,))
    li = [l.name for l in spec.lanes].index(lane)
    W = draw_base_weight(spec, li, spec.lanes[li], mode=mode)
    y, info, pool, _ = run_linear(lib, w, lane, W)
    if cfg != "decode_mix":
        assert info["n_decode_segments"] and info["n_prefill_segments"]
        assert info["n_gather_segments"]
    tok = check_against_oracle(w, lane, W, y)
    # base rows: the base product of the same kernel without a routing
    yb, _, _, _ = run_linear(lib, w, lane, W, with_routing=False, pool=pool)
    off = tok == 0
    assert off.any()
    assert np.array_equal(y[off].view(np.uint32), yb[off].view(np.uint32))
    base = oracle.base_product(w.lanes[lane].x, "bf16", W, spec.lanes[li].h_in)
    if mode == "int":
        assert np.array_equal(yb.astype(np.float64), base)
    else:
        st = compare(yb, np.zeros_like(yb), base, spec.lanes[li].h_out)
        assert st["ok"], st


@pytest.mark.parametrize("mode", ["real", "int"])
@pytest.mark.parametrize("cfg,lane,pml", [("decode_mix", "qkv", 64), ("high_rank", "wide", 1),
                                          ("ragged", "qkv_like", 64)])
def test_linear_zero_weight_gives_the_delta(lib, cfg, lane, pml, mode):
    """W = 0: every row is its delta alone (zero on base rows), against the
    oracle's delta on every row; prefill_min_len = 1 sends every sequence to
    the matrix-core shrink."""
    spec = {"ragged": RAGGED, "high_rank": HIGH_RANK}.get(cfg) or config_by_name(cfg)
    w = generate(spec, mode=mode, lanes=(lane,))
    li = [l.name for l in spec.lanes].index(lane)
    W = np.zeros((spec.lanes[li].h_out_total, spec.lanes[li].h_in), dtype=np.uint16)
    y, info, _, _ = run_linear(lib, w, lane, W, prefill_min_len=pml)
    if pml == 1:
        assert info["n_decode_segments"] == 0 and info["n_prefill_segments"] > 0
    tok = check_against_oracle(w, lane, W, y)
    assert np.all(y[tok == 0] == 0)


@pytest.mark.parametrize("mode", ["real", "int"])
def test_linear_more_steps_than_a_tile_holds(lib, mode):
    """A batch whose row tiles need more delta steps than the kernel keeps
    (the two-pass form: base product, then lora_delta_apply) still matches
    the oracle, and its base product is the one of a call with no routing."""
    w = generate(STEP_OVERFLOW, mode=mode)
    W = draw_base_weight(STEP_OVERFLOW, 0, STEP_OVERFLOW.lanes[0], mode=mode)
    y, info, pool, _ = run_linear(lib, w, "two", W)
    assert info["n_distinct"] > 60
    check_against_oracle(w, "two", W, y)


def test_linear_permutation_and_solo_bit_exact(lib):
    w = generate(RAGGED)
    W = draw_base_weight(RAGGED, 0, RAGGED.lanes[0])
    y, _, pool, _ = run_linear(lib, w, "qkv_like", W)
    starts = np.concatenate([[0], np.cumsum(w.seq_len)[:-1]])
    perm = np.random.default_rng(3).permutation(len(w.seq_len))
    rows = np.concatenate([np.arange(starts[i], starts[i] + w.seq_len[i]) for i in perm])
    yp, _, _, _ = run_linear(lib, w, "qkv_like", W, pool=pool, rows=rows,
                             seq=(w.seq_adapter[perm], w.seq_len[perm]))
    assert np.array_equal(yp.view(np.uint32), y[rows].view(np.uint32))
    for i in np.random.default_rng(4).choice(len(w.seq_len), 5, replace=False):
        r = np.arange(starts[i], starts[i] + w.seq_len[i])
        ys, _, _, _ = run_linear(lib, w, "qkv_like", W, pool=pool, rows=r,
                                 seq=(w.seq_adapter[i:i + 1], w.seq_len[i:i + 1]))
        assert np.array_equal(ys.view(np.uint32), y[r].view(np.uint32)), i


@pytest.mark.slow
@pytest.mark.parametrize("mode", ["real", "int"])
def test_linear_tp_share_attn_out_every_row(lib, mode):
    """One GPU's share of the row-parallel attention output (2048 -> 7168,
    4096 rows: decode, prefill and gather rows) against the oracle on every
    row, in row chunks on host threads."""
    from harness import oracle_row_chunks  # noqa: F401  (same threading as the delta tests)
    from concurrent.futures import ThreadPoolExecutor
    import os
    spec = config_by_name("tp_share")
    w = generate(spec, mode=mode, lanes=("attn_out",))
    W = draw_base_weight(spec, 0, spec.lanes[0], mode=mode)
    y, info, pool, _ = run_linear(lib, w, "attn_out", W)
    assert info["n_decode_segments"] and info["n_prefill_segments"]
    T = y.shape[0]
    parts = [np.arange(i, min(i + 256, T)) for i in range(0, T, 256)]
    with ThreadPoolExecutor(max_workers=max(1, min(16, os.cpu_count() or 1))) as ex:
        refs = list(ex.map(lambda r: oracle.workload_linear_lane(w, "attn_out", W, rows=r)[0],
                           parts))
    for r, ref in zip(parts, refs):
        if mode == "int":
            assert np.array_equal(y[r].astype(np.float64), ref)
        else:
            st = compare(y[r], np.zeros_like(y[r]), ref, (7168,))
            assert st["ok"], st


def test_linear_errors(lib):
    import torch
    w = generate(RAGGED)
    W = w_device(draw_base_weight(RAGGED, 0, RAGGED.lanes[0]))
    pool = load_lane_pool(lib.Pool, w, "qkv_like")
    T = w.n_tokens
    x = to_device_x(w.lanes["qkv_like"].x)
    y = torch.zeros((T, 664), device="cuda")
    r = lib.Routing(T, len(w.seq_len))
    r.build(pool, w.seq_adapter, w.seq_len)
    with pytest.raises(lib.LoraError) as e:       # rows differ from the routing's
        lib.lora_linear_delta(pool.handle, r.handle, T - 1, W, W.stride(0), x, x.stride(0), y,
                              y.stride(0), None, 0)
    assert e.value.status == "LORA_ERR_SHAPE"
    with pytest.raises(lib.LoraError) as e:       # no workspace for the active rows
        lib.lora_linear_delta(pool.handle, r.handle, T, W, W.stride(0), x, x.stride(0), y,
                              y.stride(0), None, 0)
    assert e.value.status == "LORA_ERR_ARG"
    rd = lib.Routing(T, T)
    rd.build_device(pool, torch.zeros(T, dtype=torch.int32, device="cuda"))
    with pytest.raises(lib.LoraError) as e:       # built on the device
        lib.linear_delta(pool, rd, W, x, y)
    assert e.value.status == "LORA_ERR_ARG"
    fp16 = lib.Pool(1544, (264,), 2, 16, "fp16")
    with pytest.raises(lib.LoraError) as e:
        lib.linear_delta(fp16, None, W, x, torch.zeros((T, 264), device="cuda"))
    assert e.value.status == "LORA_ERR_DTYPE"
    torch.cuda.synchronize()
    assert bool((y == 0).all())
