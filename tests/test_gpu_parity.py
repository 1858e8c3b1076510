"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Real-valued inputs are held to the tolerance rule in tests/harness.py;
integer-mode inputs (every partial sum exact in binary32) must match exactly;
rows the routing leaves alone must keep the exact bits of y0.
"""
import numpy as np
import pytest

import oracle
from workloads import (LaneSpec, WorkloadSpec, config_by_name, generate)

from harness import (compare, load_lane_pool, oracle_row_chunks, seq_starts, to_device_x,
                     to_device_y)

pytestmark = pytest.mark.gpu

MID = WorkloadSpec(
    name="mid_ragged", seed=21,
    lanes=(LaneSpec("qkv_like", 1544, (520, 136, 8)),
           LaneSpec("fp16_share", 1544, (264,), "fp16", tp_size=2, tp_rank=1),
           LaneSpec("wide_in", 4616, (136,))),
    n_adapters=5, ranks=(3, 12, 17, 1, 130), rank_mode="list",
    scale_mode="uniform", scale_range=(0.25, 3.0), max_rank=130,
    decode_rows=90, base_prob=0.2, prefill_seqs=6, prefill_len=(1, 200))


@pytest.fixture(scope="module")
def lib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import adapter_deltas_amd as m
    return m


def run_lane(m, w, lane_name, *, max_loras=None, prefill_min_len=64, path="apply",
             pool=None, x=None, y0=None, seq_ids=None, seq_lens=None):
    import torch
    lane = w.lanes[lane_name]
    if pool is None:
        pool = load_lane_pool(m.Pool, w, lane_name)
    ids = w.seq_adapter if seq_ids is None else seq_ids
    lens = w.seq_len if seq_lens is None else seq_lens
    T = int(np.sum(lens))
    cap = w.spec.max_loras if max_loras is None else max_loras
    routing = m.Routing(max(T, 1), max(len(ids), 1))
    adm, nd = routing.build(pool, ids, lens, cap, prefill_min_len)
    xd = to_device_x(lane.x if x is None else x)
    yd = to_device_y(lane.y0 if y0 is None else y0)
    if path == "apply":
        m.delta_apply(pool, routing, xd, yd)
    else:
        info = routing.info()
        v = torch.zeros(max(info["n_active"], 1) * pool.v_stride, dtype=torch.float32,
                        device="cuda")
        m.shrink(pool, routing, xd, v)
        m.expand(pool, routing, v, yd)
    torch.cuda.synchronize()
    return yd.cpu().numpy(), adm, routing.info()


def inactive_rows(w, admitted, seq_ids=None, seq_lens=None):
    ids = w.seq_adapter if seq_ids is None else seq_ids
    lens = w.seq_len if seq_lens is None else seq_lens
    mask = np.zeros(int(np.sum(lens)), dtype=bool)
    for s0, n, aid, ok in zip(seq_starts(lens), lens, ids, admitted):
        if aid == 0 or not ok:
            mask[s0:s0 + n] = True
    return mask


def check_full(w, lane_name, y, adm, max_loras=None, prefill_min_len=64):
    lane = w.lanes[lane_name]
    d_ref, tok, adm_ref = oracle.workload_lane_delta(w, lane_name, max_loras)
    assert list(adm) == list(adm_ref)
    off = tok == 0
    assert np.array_equal(y[off].view(np.uint32), lane.y0[off].view(np.uint32))
    act = ~off
    if w.mode == "int":
        assert np.array_equal(y[act].astype(np.float64),
                              lane.y0[act].astype(np.float64) + d_ref[act])
        return None
    st = compare(y, lane.y0, d_ref[act], lane.spec.h_out, rows=np.nonzero(act)[0])
    assert st["ok"], st
    return st


# ------------------------------------------------------------- full parity

@pytest.mark.parametrize("mode", ["real", "int"])
@pytest.mark.parametrize("cfg,lane", [("tiny", "proj"), ("decode_mix", "qkv")])
def test_small_configs_full_parity(lib, cfg, lane, mode):
    w = generate(config_by_name(cfg), mode=mode)
    y, adm, info = run_lane(lib, w, lane)
    check_full(w, lane, y, adm)


@pytest.mark.parametrize("mode", ["real", "int"])
@pytest.mark.parametrize("lane", ["qkv_like", "fp16_share", "wide_in"])
@pytest.mark.parametrize("prefill_min_len", [64, 1, 2**31 - 1])
def test_ragged_full_parity(lib, lane, mode, prefill_min_len):
    """h_in = 3 sub-chunks + 8 (wide_in: 9 + 8, so a GEMV part holds two
    sub-chunks), slices 520|136|8, ranks 1..130, sequences of length 1..200
    around the 64-row segment edges, both paths forced."""
    w = generate(MID, mode=mode)
    y, adm, info = run_lane(lib, w, lane, prefill_min_len=prefill_min_len)
    if prefill_min_len == 1:
        assert info["n_decode_segments"] == 0 and info["n_prefill_segments"] > 0
        assert info["n_gather_segments"] == 0
    else:
        # the rank-130 adapter's decode rows take the gather (matrix-core) path
        assert info["n_gather_segments"] > 0 and info["n_decode_segments"] > 0
    if prefill_min_len == 2**31 - 1:
        assert info["n_prefill_segments"] == 0
    check_full(w, lane, y, adm, prefill_min_len=prefill_min_len)


def test_y0_zero_and_split_path_parity(lib):
    w = generate(config_by_name("decode_mix"), y0="zeros")
    y, adm, _ = run_lane(lib, w, "qkv", path="split")
    check_full(w, "qkv", y, adm)
    ya, _, _ = run_lane(lib, w, "qkv")
    assert np.array_equal(ya.view(np.uint32), y.view(np.uint32))


# Decode rows only, ranks up to 16 and slices of at most 1024 columns (the
# one-launch decode delta of delta_apply), ragged widths, bf16 and fp16 x,
# some parts of h_in empty or holding two sub-chunks.
SMALL_RANK = WorkloadSpec(
    name="small_rank_ragged", seed=22,
    lanes=(LaneSpec("qkv_like", 1544, (520, 136, 8)),
           LaneSpec("fp16_share", 4616, (264,), "fp16", tp_size=2, tp_rank=1)),
    n_adapters=5, ranks=(3, 12, 16, 1, 9), rank_mode="list",
    scale_mode="uniform", scale_range=(0.25, 3.0), max_rank=16,
    decode_rows=150, base_prob=0.2, prefill_seqs=0, prefill_len=(1, 1))


# Decode rows over a wide input (parts of h_in holding one or two
# sub-chunks) with ranks past 16, for bf16 and fp16 x: delta_apply matches
# the oracle and, bit for bit, lora_shrink then lora_expand.
WIDE_DECODE = WorkloadSpec(
    name="wide_decode", seed=31,
    lanes=(LaneSpec("fp16_wide", 4616, (264, 72), "fp16"),
           LaneSpec("bf16_wide", 5128, (520,))),
    n_adapters=4, ranks=(24, 40, 8, 33), rank_mode="list",
    scale_mode="uniform", scale_range=(0.5, 2.0), max_rank=48,
    decode_rows=90, base_prob=0.2, prefill_seqs=0, prefill_len=(1, 1))


@pytest.mark.parametrize("mode", ["real", "int"])
@pytest.mark.parametrize("lane", ["fp16_wide", "bf16_wide"])
def test_wide_decode_apply_matches_two_calls(lib, lane, mode):
    w = generate(WIDE_DECODE, mode=mode)
    y, adm, info = run_lane(lib, w, lane)
    assert info["n_decode_segments"] and not info["n_prefill_segments"]
    check_full(w, lane, y, adm)
    ys, _, _ = run_lane(lib, w, lane, path="split")
    assert np.array_equal(y.view(np.uint32), ys.view(np.uint32))


@pytest.mark.parametrize("mode", ["real", "int"])
@pytest.mark.parametrize("lane", ["qkv_like", "fp16_share"])
def test_one_launch_decode_delta_matches_split(lib, lane, mode):
    """delta_apply (shrink and expand in one launch) is bit-identical to
    lora_shrink then lora_expand, and both match the oracle."""
    w = generate(SMALL_RANK, mode=mode)
    ya, adm, info = run_lane(lib, w, lane)
    assert info["n_decode_segments"] > 0 and info["n_prefill_segments"] == 0
    ys, _, _ = run_lane(lib, w, lane, path="split")
    assert np.array_equal(ya.view(np.uint32), ys.view(np.uint32))
    check_full(w, lane, ya, adm)


# Fused QKV with an attention output gate (xLLM #2014, LoRAQKVParallelLinear,
# q_has_gate): the q lane holds query and gate rows of 16 heads x 256, so the q
# slice is 8192 wide next to 512-wide k and v slices (2 kv heads x 256).
GATED_QKV = WorkloadSpec(
    name="gated_qkv", seed=24,
    lanes=(LaneSpec("qkv_gate", 2048, (8192, 512, 512)),),
    n_adapters=4, ranks=(8, 16, 64, 5), rank_mode="list",
    scale_mode="alpha", alpha=32.0, max_rank=64,
    decode_rows=40, base_prob=0.25, prefill_seqs=2, prefill_len=(65, 140))


@pytest.mark.parametrize("mode", ["real", "int"])
@pytest.mark.parametrize("path", ["apply", "split"])
def test_gated_q_lane_full_parity(lib, mode, path):
    w = generate(GATED_QKV, mode=mode)
    y, adm, info = run_lane(lib, w, "qkv_gate", path=path)
    assert info["n_decode_segments"] > 0 and info["n_prefill_segments"] > 0
    check_full(w, "qkv_gate", y, adm)


# ------------------------------------------- ranks the ABI accepts, all paths

# Decode rows of ranks 65..127 on the GEMV path (shrink tasks of rank blocks
# 9..16, the expand's rank loop past 64) next to ranks 8 and 64 in one batch,
# so some rank-block tasks of the launch end early.
HIGH_RANK_GEMV = WorkloadSpec(
    name="high_rank_gemv", seed=25,
    lanes=(LaneSpec("qkv_like", 1544, (520, 136, 8)),
           LaneSpec("fp16_share", 4616, (264,), "fp16", tp_size=2, tp_rank=1)),
    n_adapters=5, ranks=(65, 100, 127, 8, 64), rank_mode="list",
    scale_mode="uniform", scale_range=(0.25, 3.0), max_rank=127,
    decode_rows=120, base_prob=0.2, prefill_seqs=0, prefill_len=(1, 1))

# Ranks up to LORA_MAX_RANK on the matrix cores: prefill segments and gather
# rows of ranks 192 and 256 (the 8-step MFMA expand tile with data in every
# step), rank 130, and a rank-8 adapter whose decode rows take the GEMV path.
HIGH_RANK_MFMA = WorkloadSpec(
    name="high_rank_mfma", seed=26,
    lanes=(LaneSpec("qkv_like", 1544, (520, 136, 8)),
           LaneSpec("fp16_share", 4616, (264,), "fp16", tp_size=2, tp_rank=1)),
    n_adapters=4, ranks=(192, 256, 130, 8), rank_mode="list",
    scale_mode="uniform", scale_range=(0.25, 3.0), max_rank=256,
    decode_rows=100, base_prob=0.2, prefill_seqs=5, prefill_len=(1, 200))


@pytest.mark.parametrize("mode", ["real", "int"])
@pytest.mark.parametrize("path", ["apply", "split"])
@pytest.mark.parametrize("lane", ["qkv_like", "fp16_share"])
def test_gemv_ranks_65_to_127(lib, lane, path, mode):
    w = generate(HIGH_RANK_GEMV, mode=mode)
    y, adm, info = run_lane(lib, w, lane, path=path)
    assert info["n_decode_segments"] > 0
    assert info["n_prefill_segments"] == 0 and info["n_gather_segments"] == 0
    check_full(w, lane, y, adm)


@pytest.mark.parametrize("mode", ["real", "int"])
@pytest.mark.parametrize("path", ["apply", "split"])
@pytest.mark.parametrize("lane", ["qkv_like", "fp16_share"])
@pytest.mark.parametrize("prefill_min_len", [64, 1])
def test_matrix_core_ranks_to_256(lib, lane, path, mode, prefill_min_len):
    w = generate(HIGH_RANK_MFMA, mode=mode)
    y, adm, info = run_lane(lib, w, lane, path=path, prefill_min_len=prefill_min_len)
    assert info["n_prefill_segments"] > 0
    if prefill_min_len == 64:
        # decode rows of ranks 130, 192 and 256 gathered, rank 8 on the GEMV path
        assert info["n_gather_segments"] > 0 and info["n_decode_segments"] > 0
    check_full(w, lane, y, adm, prefill_min_len=prefill_min_len)


# Many short prompts: 200 prefill segments of 24 rows, so a host plan carries
# matrix-core shrink task tables (at least 128 tasks; the 32-row template
# covers them) and, on the two-slice lane, tasks that take a short segment's
# tile of both slices; ranks 8..100 (a rank-100 segment is cut into several
# tasks), h_in with a ragged last K-step pair, decode rows beside them.
SHORT_PROMPTS = WorkloadSpec(
    name="short_prompts", seed=27,
    lanes=(LaneSpec("one", 520, (264,)), LaneSpec("two", 520, (264, 136))),
    n_adapters=4, ranks=(8, 16, 64, 100), rank_mode="list",
    scale_mode="uniform", scale_range=(0.25, 3.0), max_rank=100,
    decode_rows=40, base_prob=0.2, prefill_seqs=200, prefill_len=(24, 24))


def short_prompt_tables(lib, w):
    """The matrix-core task tables a host plan of SHORT_PROMPTS carries (the
    pool loads its adapters into slots 1.. in order)."""
    resident = {aid: i + 1 for i, aid in enumerate(w.adapters)}
    ranks = {aid: [ad.lanes["two"][0].rank] * 2 for aid, ad in w.adapters.items()}
    p = lib.lora_plan_routing(w.seq_adapter, w.seq_len, w.spec.max_loras, 16, resident,
                              w.spec.n_adapters, int(np.sum(w.seq_len)), resident_rank=ranks)
    return p["mfma_tasks"]


@pytest.mark.parametrize("mode", ["real", "int"])
@pytest.mark.parametrize("path", ["apply", "split"])
@pytest.mark.parametrize("lane", ["one", "two"])
def test_short_prompts_task_tables_parity(lib, lane, path, mode):
    w = generate(SHORT_PROMPTS, mode=mode)
    assert sorted(short_prompt_tables(lib, w)) == [1, 2]
    y, adm, info = run_lane(lib, w, lane, path=path, prefill_min_len=16)
    assert info["n_prefill_segments"] >= 128 and info["n_decode_segments"] > 0
    check_full(w, lane, y, adm, prefill_min_len=16)


def test_routing_serves_a_lane_with_fewer_slices(lib):
    """A routing built against the two-slice lane's pool serves the one-slice
    lane (their slice-0 ranks agree) from its one-slice task table: every
    row's bits equal those of the lane's own routing."""
    import torch
    w = generate(SHORT_PROMPTS)
    T = int(np.sum(w.seq_len))
    p1 = load_lane_pool(lib.Pool, w, "one")
    p2 = load_lane_pool(lib.Pool, w, "two")
    shared = lib.Routing(T, len(w.seq_len))
    shared.build(p2, w.seq_adapter, w.seq_len, w.spec.max_loras, 16)
    L = w.lanes["one"]
    xd, yd = to_device_x(L.x), to_device_y(L.y0)
    lib.delta_apply(p1, shared, xd, yd)
    torch.cuda.synchronize()
    y_own, adm, _ = run_lane(lib, w, "one", prefill_min_len=16)
    assert np.array_equal(yd.cpu().numpy().view(np.uint32), y_own.view(np.uint32))
    check_full(w, "one", y_own, adm, prefill_min_len=16)


# ------------------------------------------------- full-size configs, every row

@pytest.mark.slow
@pytest.mark.parametrize("mode", ["real", "int"])
@pytest.mark.parametrize("cfg,lane", [("prefill", "o_proj"), ("prefill", "gate_up"),
                                      ("many_tenants", "down_proj"),
                                      ("many_tenants", "o_proj"),
                                      ("tp_share", "attn_out"), ("tp_share", "shexp_w2")])
def test_full_size_every_row(lib, cfg, lane, mode):
    """Full-size workloads in the launch configuration the benchmark times:
    every active row against the oracle (computed on host threads in row
    chunks), every other row bit-identical to y0."""
    w = generate(config_by_name(cfg), mode=mode, lanes=(lane,))
    y, adm, info = run_lane(lib, w, lane)
    L = w.lanes[lane]
    _, tok, adm_ref = oracle.workload_lane_delta(w, lane, rows=np.zeros(0, np.int64))
    assert list(adm) == list(adm_ref)
    off = tok == 0
    assert np.array_equal(y[off].view(np.uint32), L.y0[off].view(np.uint32))
    act = np.nonzero(~off)[0]
    for rows, d_ref in oracle_row_chunks(w, lane, act):
        if mode == "int":
            assert np.array_equal(y[rows].astype(np.float64),
                                  L.y0[rows].astype(np.float64) + d_ref)
        else:
            st = compare(y, L.y0, d_ref, L.spec.h_out, rows=rows)
            assert st["ok"], st


# ---------------------------------------------------------------- invariants

def test_base_rows_not_read_or_written(lib):
    """NaN in x and y of base rows: base rows keep their NaN payload bits and
    nothing leaks into adapter rows."""
    w = generate(config_by_name("decode_mix"))
    L = w.lanes["qkv"]
    y_ref, adm, _ = run_lane(lib, w, "qkv")
    tok = oracle.token_adapters(w.seq_adapter, w.seq_len, adm)
    x = L.x.copy()
    y0 = L.y0.copy()
    x[tok == 0] = 0x7FC1                                    # bf16 quiet NaN
    y0.view(np.uint32)[tok == 0] = 0x7FC01234               # NaN with payload
    y, _, _ = run_lane(lib, w, "qkv", x=x, y0=y0)
    assert np.array_equal(y.view(np.uint32)[tok == 0], y0.view(np.uint32)[tok == 0])
    assert np.array_equal(y.view(np.uint32)[tok != 0], y_ref.view(np.uint32)[tok != 0])


@pytest.mark.parametrize("cfg,lane", [("decode_mix", "qkv"), ("mid", "qkv_like"),
                                      ("mid", "fp16_share"), ("mid", "wide_in")])
def test_permutation_and_solo_bit_exact(lib, cfg, lane):
    w = generate(MID) if cfg == "mid" else generate(config_by_name(cfg))
    L = w.lanes[lane]
    pool = load_lane_pool(lib.Pool, w, lane)
    y, adm, _ = run_lane(lib, w, lane, pool=pool)
    # sequences in a shuffled order, rows moved with them
    perm = np.random.default_rng(1).permutation(len(w.seq_len))
    starts = seq_starts(w.seq_len)
    rows = np.concatenate([np.arange(starts[i], starts[i] + w.seq_len[i]) for i in perm])
    yp, _, _ = run_lane(lib, w, lane, pool=pool, x=L.x[rows], y0=L.y0[rows],
                        seq_ids=w.seq_adapter[perm], seq_lens=w.seq_len[perm])
    assert np.array_equal(yp.view(np.uint32), y[rows].view(np.uint32))
    # a few sequences alone
    for i in np.random.default_rng(2).choice(len(w.seq_len), 6, replace=False):
        r = np.arange(starts[i], starts[i] + w.seq_len[i])
        ys, _, _ = run_lane(lib, w, lane, pool=pool, x=L.x[r], y0=L.y0[r],
                            seq_ids=w.seq_adapter[i:i + 1], seq_lens=w.seq_len[i:i + 1])
        assert np.array_equal(ys.view(np.uint32), y[r].view(np.uint32)), i


@pytest.mark.parametrize("cfg,lane", [("many_tenants", "down_proj"), ("tp_share", "attn_out")])
def test_solo_matches_large_batch_bit_exact(lib, cfg, lane):
    """The launch shape follows the batch (waves per shrink task by grid size,
    rows per expand wave by how full the decode segments are); a row's bits
    must not: sequences of a full-size batch, run alone, give the same bits."""
    w = generate(config_by_name(cfg), lanes=(lane,))
    L = w.lanes[lane]
    pool = load_lane_pool(lib.Pool, w, lane)
    y, adm, info = run_lane(lib, w, lane, pool=pool)
    kmax = max(s.rank for ad in w.adapters.values() for s in ad.lanes[lane])
    tasks = info["n_decode_segments"] * len(L.spec.h_out) * -(-kmax // 8)
    assert tasks >= 512                    # the large-grid shrink form runs for the batch
    starts = seq_starts(w.seq_len)
    active = [i for i in range(len(w.seq_len)) if w.seq_adapter[i] != 0 and adm[i]]
    for i in np.random.default_rng(3).choice(active, 6, replace=False):
        r = np.arange(starts[i], starts[i] + w.seq_len[i])
        ys, _, _ = run_lane(lib, w, lane, pool=pool, x=L.x[r], y0=L.y0[r],
                            seq_ids=w.seq_adapter[i:i + 1], seq_lens=w.seq_len[i:i + 1])
        assert np.array_equal(ys.view(np.uint32), y[r].view(np.uint32)), i


def test_run_to_run_relocation_and_split_bit_exact(lib):
    w = generate(MID)
    lane = "qkv_like"
    y1, _, _ = run_lane(lib, w, lane)
    y2, _, _ = run_lane(lib, w, lane)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    # other slots, more slots, larger max_rank, device-side packing
    ids = w.adapter_ids
    slot_of = {aid: 9 - i for i, aid in enumerate(ids)}
    pool = load_lane_pool(lib.Pool, w, lane, max_slots=9, max_rank=160, slot_of=slot_of,
                          on_device=True)
    y3, _, _ = run_lane(lib, w, lane, pool=pool)
    assert np.array_equal(y1.view(np.uint32), y3.view(np.uint32))
    y4, _, _ = run_lane(lib, w, lane, path="split")
    assert np.array_equal(y1.view(np.uint32), y4.view(np.uint32))


def test_scale_zero_gives_y0(lib):
    w = generate(MID)
    lane = "qkv_like"
    for ad in w.adapters.values():
        for s in ad.lanes[lane]:
            s.scale = 0.0
    y, adm, _ = run_lane(lib, w, lane)
    assert np.array_equal(y, w.lanes[lane].y0)   # numeric ==, -0.0 == +0.0


# ------------------------------------------------------ admission and errors

def test_max_loras_deferral(lib):
    w = generate(config_by_name("decode_mix"))
    y, adm, info = run_lane(lib, w, "qkv", max_loras=3)
    assert info["n_distinct"] == 3 and not all(adm)
    check_full(w, "qkv", y, adm, max_loras=3)


def test_empty_and_all_base_batches_touch_nothing(lib):
    import torch
    w = generate(config_by_name("tiny"))
    L = w.lanes["proj"]
    pool = load_lane_pool(lib.Pool, w, "proj")
    for ids, lens in [([], []), ([0, 0, 0], [1, 5, 2]), ([1037, 0], [0, 3])]:
        T = int(sum(lens))
        routing = lib.Routing(max(T, 1), 4)
        routing.build(pool, ids, lens, 0, 64)
        assert routing.info()["n_active"] == 0
        yd = torch.full((max(T, 1), 64), 3.5, device="cuda")
        xd = torch.zeros((max(T, 1), 64), dtype=torch.int16, device="cuda")
        lib.delta_apply(pool, routing, xd, yd)
        torch.cuda.synchronize()
        assert bool((yd == 3.5).all())


def test_unknown_adapter_is_an_error(lib):
    w = generate(config_by_name("tiny"))
    pool = load_lane_pool(lib.Pool, w, "proj")
    routing = lib.Routing(8, 8)
    with pytest.raises(lib.LoraError) as e:
        routing.build(pool, [1037, 999], [1, 1], 0, 64)
    assert e.value.status == "LORA_ERR_UNKNOWN_ADAPTER"
    # a deferred unknown id is not an error: it is never admitted
    adm, _ = routing.build(pool, [1037, 999], [1, 1], 1, 64)
    assert list(adm) == [True, False]


def test_load_errors(lib):
    w = generate(config_by_name("tiny"))
    pool = load_lane_pool(lib.Pool, w, "proj")
    ad = next(iter(w.adapters.values()))
    s = ad.lanes["proj"][0]
    cases = [
        (dict(adapter_id=0), "LORA_ERR_ARG"),
        (dict(slot=0), "LORA_ERR_SLOT"),
        (dict(slot=3), "LORA_ERR_SLOT"),
        (dict(ranks=[5]), "LORA_ERR_RANK"),
        (dict(scales=[float("nan")]), "LORA_ERR_ARG"),
        (dict(a_col0=8), "LORA_ERR_SHAPE"),
    ]
    for kw, status in cases:
        args = dict(adapter_id=77, A=[s.A], B=[s.B], ranks=[s.rank], scales=[s.scale],
                    a_col0=0, slot=-1)
        args.update(kw)
        if "ranks" in kw:
            args["A"] = [np.zeros((5, 64), np.uint16)]
            args["B"] = [np.zeros((64, 5), np.uint16)]
        with pytest.raises(lib.LoraError) as e:
            pool.load(**args)
        assert e.value.status == status, kw
    # both slots are taken: a third id has no free slot
    with pytest.raises(lib.LoraError) as e:
        pool.load(77, [s.A], [s.B], [s.rank], [s.scale])
    assert e.value.status == "LORA_ERR_CAPACITY"


def test_graph_replays_match_eager(lib):
    """delta_apply captured in a HIP graph, together with the reset of y, gives
    the eager bits on every replay, with other device work run in between.
    MID routes rows through the decode GEMV, prefill and gather kernels."""
    import torch
    w = generate(MID)
    for lane in ("qkv_like", "wide_in"):
        L = w.lanes[lane]
        pool = load_lane_pool(lib.Pool, w, lane)
        routing = lib.Routing(int(np.sum(w.seq_len)), len(w.seq_len))
        routing.build(pool, w.seq_adapter, w.seq_len, w.spec.max_loras)
        info = routing.info()
        assert info["n_decode_segments"] and info["n_prefill_segments"]
        assert info["n_gather_segments"]
        xd, y0 = to_device_x(L.x), to_device_y(L.y0)
        ws = lib.workspace_for(pool, routing)
        ye = y0.clone()
        lib.delta_apply(pool, routing, xd, ye, ws)
        torch.cuda.synchronize()
        ref = ye.cpu().numpy().view(np.uint32)
        yg = torch.empty_like(y0)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            yg.copy_(y0)
            lib.delta_apply(pool, routing, xd, yg, ws)
        for i in range(4):
            yg.fill_(float("nan"))
            torch.randn(1 << 20, device="cuda").sum().item()
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(yg.cpu().numpy().view(np.uint32), ref), (lane, i)


def test_graph_replays_of_split_calls_on_a_mixed_batch(lib):
    """lora_shrink and lora_expand captured separately on a batch with decode,
    prefill and gather segments (each call forks its decode kernels to the
    routing's second stream and joins them back): every replay gives the
    bits of an eager delta_apply."""
    import torch
    w = generate(MID)
    lane = "qkv_like"
    L = w.lanes[lane]
    pool = load_lane_pool(lib.Pool, w, lane)
    routing = lib.Routing(int(np.sum(w.seq_len)), len(w.seq_len))
    routing.build(pool, w.seq_adapter, w.seq_len, w.spec.max_loras)
    info = routing.info()
    assert info["n_decode_segments"] and (info["n_prefill_segments"] or info["n_gather_segments"])
    xd, y0 = to_device_x(L.x), to_device_y(L.y0)
    ye = y0.clone()
    lib.delta_apply(pool, routing, xd, ye)
    torch.cuda.synchronize()
    ref = ye.cpu().numpy().view(np.uint32)
    v = torch.zeros(max(info["n_active"], 1) * pool.v_stride, dtype=torch.float32, device="cuda")
    yg = torch.empty_like(y0)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        yg.copy_(y0)
        lib.shrink(pool, routing, xd, v)
        lib.expand(pool, routing, v, yg)
    for i in range(3):
        yg.fill_(float("nan"))
        v.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(yg.cpu().numpy().view(np.uint32), ref), i
