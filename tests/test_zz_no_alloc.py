"""lora_delta_apply_noalloc (v in the library's static scratch) gives the bits
of lora_delta_apply (v in a caller workspace) and the oracle's values, on two
calls in a row, the second with a smaller batch; a batch whose v does not fit
the scratch is refused before anything runs."""
import numpy as np
import pytest

import oracle
from workloads import LaneSpec, WorkloadSpec, config_by_name, generate
from workloads.device import to_device_x, to_device_y

from harness import compare, load_lane_pool, seq_starts

pytestmark = pytest.mark.gpu

# decode (GEMV), prefill and gather (matrix-core) segments in one batch
MIXED = WorkloadSpec(
    name="noalloc_mixed", seed=41,
    lanes=(LaneSpec("qkv_like", 1544, (520, 136, 8)),),
    n_adapters=5, ranks=(3, 12, 17, 1, 130), rank_mode="list",
    scale_mode="uniform", scale_range=(0.25, 3.0), max_rank=130,
    decode_rows=90, base_prob=0.2, prefill_seqs=6, prefill_len=(1, 200))


@pytest.fixture(scope="module")
def lib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import adapter_deltas_amd as m
    return m


def both_paths(m, pool, ids, lens, x, y0):
    """(y from lora_delta_apply, y from lora_delta_apply_noalloc) for one batch."""
    import torch
    T = int(np.sum(lens))
    routing = m.Routing(max(T, 1), max(len(ids), 1))
    routing.build(pool, ids, lens, 0, m.DEFAULT_PREFILL_MIN_LEN)
    xd, yw, yn = to_device_x(x), to_device_y(y0), to_device_y(y0)
    m.delta_apply(pool, routing, xd, yw)
    m.delta_apply_noalloc(pool, routing, xd, yn)
    torch.cuda.synchronize()
    return yw.cpu().numpy(), yn.cpu().numpy(), routing.info()


def check_oracle(w, lane, ids, lens, x, y0, y):
    L = w.lanes[lane]
    adm, _ = oracle.admit(ids, 0)
    tok = oracle.token_adapters(ids, lens, adm)
    factors = {aid: [(s.A, s.B, s.rank, s.scale) for s in ad.lanes[lane]]
               for aid, ad in w.adapters.items()}
    d = oracle.lane_delta(x, L.spec.x_dtype, tok, factors, L.spec.h_out, L.spec.a_col0,
                          L.spec.h_in)
    off = tok == 0
    assert np.array_equal(y[off].view(np.uint32), y0[off].view(np.uint32))
    if w.mode == "int":
        assert np.array_equal(y[~off].astype(np.float64), y0[~off].astype(np.float64) + d[~off])
    else:
        st = compare(y, y0, d[~off], L.spec.h_out, rows=np.nonzero(~off)[0])
        assert st["ok"], st


@pytest.mark.parametrize("mode", ["real", "int"])
def test_noalloc_matches_workspace_path_twice(lib, mode):
    w = generate(MIXED, mode=mode)
    lane = "qkv_like"
    L = w.lanes[lane]
    pool = load_lane_pool(lib.Pool, w, lane)
    # first call: the whole batch (decode, prefill and gather segments)
    yw, yn, info = both_paths(lib, pool, w.seq_adapter, w.seq_len, L.x, L.y0)
    assert info["n_decode_segments"] and info["n_prefill_segments"]
    assert info["n_gather_segments"]
    assert np.array_equal(yn.view(np.uint32), yw.view(np.uint32))
    check_oracle(w, lane, w.seq_adapter, w.seq_len, L.x, L.y0, yn)
    # second call: a smaller batch (the first third of the sequences); the
    # scratch still holds the first call's v
    n = len(w.seq_len) // 3
    rows = np.arange(int(np.sum(w.seq_len[:n])))
    ids, lens = w.seq_adapter[:n], w.seq_len[:n]
    yw2, yn2, info2 = both_paths(lib, pool, ids, lens, L.x[rows], L.y0[rows])
    assert 0 < info2["n_active"] < info["n_active"]
    assert np.array_equal(yn2.view(np.uint32), yw2.view(np.uint32))
    check_oracle(w, lane, ids, lens, L.x[rows], L.y0[rows], yn2)


def test_noalloc_decode_mix_and_device_routing(lib):
    """The headline decode batch (host routing) and then a smaller device-built
    routing of part of it, each against lora_delta_apply's bits."""
    import torch
    w = generate(config_by_name("decode_mix"))
    L = w.lanes["qkv"]
    pool = load_lane_pool(lib.Pool, w, "qkv")
    yw, yn, _ = both_paths(lib, pool, w.seq_adapter, w.seq_len, L.x, L.y0)
    assert np.array_equal(yn.view(np.uint32), yw.view(np.uint32))
    n = 100
    ids = w.seq_adapter[:n]
    tok = torch.from_numpy(np.array([pool.slot_of(int(a)) if a else 0 for a in ids],
                                    np.int32)).cuda()
    routing = lib.Routing(n, n)
    routing.build_device(pool, tok)
    xd, yw2, yn2 = to_device_x(L.x[:n]), to_device_y(L.y0[:n]), to_device_y(L.y0[:n])
    lib.delta_apply(pool, routing, xd, yw2)
    lib.delta_apply_noalloc(pool, routing, xd, yn2)
    torch.cuda.synchronize()
    assert np.array_equal(yn2.cpu().numpy().view(np.uint32), yw2.cpu().numpy().view(np.uint32))
    check_oracle(w, "qkv", ids, np.ones(n, np.int32), L.x[:n], L.y0[:n], yn2.cpu().numpy())


def test_noalloc_refuses_a_batch_beyond_the_scratch(lib):
    import torch
    from adapter_deltas_amd import _lib
    # four slices padded to rank 256: 4 KiB of v per active row
    pool = lib.Pool(64, (64, 64, 64, 64), 1, 256)
    A = [np.zeros((4, 64), np.uint16)] * 4
    B = [np.zeros((64, 4), np.uint16)] * 4
    pool.load(7, A, B, [4] * 4, [1.0] * 4)
    T = _lib.NOALLOC_SCRATCH_BYTES // (4 * 256 * 4) + 1
    routing = lib.Routing(T, T)
    routing.build(pool, np.full(T, 7, np.int32), np.ones(T, np.int32), 0, lib.NO_PREFILL)
    assert lib.lora_workspace_bytes(pool.handle, routing.handle) > _lib.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((T, 64), dtype=torch.int16, device="cuda")
    y = torch.full((T, 256), 2.5, device="cuda")
    with pytest.raises(lib.LoraError) as e:
        lib.delta_apply_noalloc(pool, routing, x, y)
    assert e.value.status == "LORA_ERR_CAPACITY"
    torch.cuda.synchronize()
    assert bool((y == 2.5).all())
