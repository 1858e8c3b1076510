"""GPU parity of adapters loaded with A folded onto a transformed input
(lora_pool_load_folded): the shared expert's down projection reading a
rotated, scaled fp16 hidden state, on one GPU's column share."""
import numpy as np
import pytest

import oracle
from workloads import LaneSpec, WorkloadSpec, draw_fold, generate

from harness import compare, to_device_x, to_device_y

pytestmark = pytest.mark.gpu

# Second of two column shares of a 4096-wide input (a_col0 = 2048); x is the
# transformed fp16 state; ranks 8, 64 and 128 (the last on the gather path),
# decode rows and prefill sequences.
FOLDED = WorkloadSpec(
    name="folded_shexp", seed=25,
    lanes=(LaneSpec("shexp_w2", 2048, (1024,), "fp16", tp_size=2, tp_rank=1),),
    n_adapters=3, ranks=(8, 64, 128), rank_mode="list", scale_mode="alpha", alpha=32.0,
    max_rank=128, decode_rows=48, base_prob=0.2, prefill_seqs=2, prefill_len=(65, 100))


@pytest.fixture(scope="module")
def lib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import adapter_deltas_amd as m
    return m


def folded_pool(m, w, lane, fold_d):
    import torch
    L = w.lanes[lane].spec
    pool = m.Pool(L.h_in, L.h_out, w.spec.n_adapters, w.spec.max_rank, L.x_dtype)
    dev = lambda a: torch.from_numpy(a.view(np.int16)).cuda()
    for aid, ad in w.adapters.items():
        sl = ad.lanes[lane]
        pool.load_folded(aid, [dev(s.A) for s in sl], [dev(s.B) for s in sl],
                         [s.rank for s in sl], [s.scale for s in sl], fold_d, a_col0=L.a_col0)
    return pool


def apply(m, w, lane, pool):
    import torch
    T = w.n_tokens
    r = m.Routing(T, len(w.seq_len))
    r.build(pool, w.seq_adapter, w.seq_len)
    x, y = to_device_x(w.lanes[lane].x), to_device_y(w.lanes[lane].y0)
    m.delta_apply(pool, r, x, y)
    torch.cuda.synchronize()
    return y.cpu().numpy(), r.info()


@pytest.mark.parametrize("mode", ["real", "int"])
def test_folded_load_parity(lib, mode):
    import torch
    w = generate(FOLDED, mode=mode)
    lane = "shexp_w2"
    L = w.lanes[lane]
    _, fold = draw_fold(FOLDED.seed, L.spec.h_in)
    pool = folded_pool(lib, w, lane, torch.from_numpy(fold).cuda())
    y, info = apply(lib, w, lane, pool)
    assert info["n_decode_segments"] > 0 and info["n_prefill_segments"] > 0
    assert info["n_gather_segments"] > 0
    tok = np.repeat(w.seq_adapter, w.seq_len)
    factors = {}
    for aid, ad in w.adapters.items():
        s = ad.lanes[lane][0]
        Af = oracle.fold_a(s.A, L.spec.a_col0, L.spec.h_in, fold, s.rank)
        factors[aid] = [(Af, s.B, s.rank, s.scale)]
    act = np.nonzero(tok)[0]
    d_ref = oracle.lane_delta(L.x, "fp16", tok, factors, L.spec.h_out, 0, L.spec.h_in, rows=act)
    off = tok == 0
    assert np.array_equal(y[off].view(np.uint32), L.y0[off].view(np.uint32))
    # the device folds in fp32 and the oracle in fp64 before rounding to bf16,
    # so single factors may differ by a bf16 unit: compared to tolerance in
    # both value modes
    st = compare(y, L.y0, d_ref, L.spec.h_out, rows=act)
    assert st["ok"], st


def test_signed_permutation_fold_equals_permuted_load(lib):
    """A fold that permutes and negates columns is exact: the pool then holds
    the same factors as a plain load of the permuted A, bit for bit."""
    import torch
    w = generate(FOLDED)
    lane = "shexp_w2"
    L = w.lanes[lane].spec
    n = L.h_in
    rng = np.random.default_rng(12)
    perm = rng.permutation(n)
    sign = rng.choice([-1.0, 1.0], n).astype(np.float32)
    P = np.zeros((n, n + 8), np.float32)                 # ld_fold > h_in
    P[perm, np.arange(n)] = sign
    pool_f = folded_pool(lib, w, lane, torch.from_numpy(P).cuda())
    pool_p = lib.Pool(L.h_in, L.h_out, FOLDED.n_adapters, FOLDED.max_rank, L.x_dtype)
    for aid, ad in w.adapters.items():
        s = ad.lanes[lane][0]
        Ash = (s.A[:, L.a_col0:L.a_col0 + n].astype(np.uint32) << 16).view(np.float32)
        Ap = (Ash[:, perm] * sign).astype(np.float32)
        Ap_bits = (Ap.view(np.uint32) >> 16).astype(np.uint16)   # exact: values are bf16
        pool_p.load(aid, [Ap_bits], [s.B], [s.rank], [s.scale], a_col0=0,
                    slot=pool_f.slot_of(aid))
    yf, _ = apply(lib, w, lane, pool_f)
    yp, _ = apply(lib, w, lane, pool_p)
    assert np.array_equal(yf.view(np.uint32), yp.view(np.uint32))


def test_folded_load_errors(lib):
    import torch
    w = generate(FOLDED)
    lane = "shexp_w2"
    L = w.lanes[lane].spec
    s = w.adapters[w.adapter_ids[0]].lanes[lane][0]
    dev = lambda a: torch.from_numpy(a.view(np.int16)).cuda()
    pool = lib.Pool(L.h_in, L.h_out, 2, FOLDED.max_rank, L.x_dtype)
    narrow = torch.zeros((L.h_in, L.h_in - 8), dtype=torch.float32, device="cuda")
    with pytest.raises(lib.LoraError):
        pool.load_folded(1, [dev(s.A)], [dev(s.B)], [s.rank], [s.scale], narrow,
                         a_col0=L.a_col0)
    with pytest.raises(lib.LoraError):
        lib.lora_pool_load_folded(pool.handle, 1, -1, [dev(s.A)], [s.A.shape[1]], L.a_col0,
                                  [dev(s.B)], [s.B.shape[1]], [s.rank], [s.scale], 0, L.h_in)
