"""Pins of the fp64 oracle against facts other than itself.

Each test checks the oracle against something the pages or the mathematics
fix: hand-derived worked examples (tests/golden), library decoders, the dense
product B @ A computed by numpy, exact integer brute force, and invariants
(slot 0, permutation, scale 0, linearity, slices, column shares).
"""
import json
import os

import numpy as np
import pytest

import oracle
from workloads import (CONFIGS, WorkloadSpec, LaneSpec, generate, config_by_name,
                       f32_to_bf16_bits, bf16_bits_to_f32, MoeSpec, generate_moe,
                       draw_base_weight)
from workloads.gen import f32_to_fp16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(vals, dtype="bf16"):
    a = np.asarray(vals, dtype=np.float32)
    return f32_to_fp16_bits(a) if dtype == "fp16" else f32_to_bf16_bits(a)


# ---------------------------------------------------------------- decoders

def test_bf16_decode_matches_torch_for_every_pattern():
    torch = pytest.importorskip("torch")
    bits = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    got = np.array([oracle.bf16_value(b) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_fp16_decode_matches_numpy_for_every_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.fp16_value(b) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


# ---------------------------------------------------------- worked examples

def test_worked_examples():
    with open(os.path.join(GOLDEN, "worked_examples.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        dt = c["x_dtype"]
        if "x_bits" in c:
            x = np.array([c["x_bits"]], dtype=np.uint16)
        else:
            x = _bits([c["x"]], dt)
        h_in = x.shape[1]
        factors = {5: []}
        h_out = []
        for s in c["slices"]:
            A = _bits(s["A"])
            B = _bits(s["B"])
            factors[5].append((A, B, A.shape[0], s["scale"]))
            h_out.append(B.shape[0])
        d = oracle.lane_delta(x, dt, [5], factors, h_out, c["a_col0"], h_in)
        assert d.tolist() == [c["delta"]], c["name"]


# ----------------------------------------------------------------- admission

def test_admission_cases():
    with open(os.path.join(GOLDEN, "admission_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        adm, distinct = oracle.admit(c["ids"], c["max_loras"])
        assert adm == c["admitted"], c["name"]
        assert distinct == c["distinct"], c["name"]


def test_token_adapters_is_repeat_interleave():
    rng = np.random.default_rng(5)
    ids = rng.integers(0, 4, size=50) * 11
    lens = rng.integers(1, 9, size=50)
    adm = rng.random(50) < 0.8
    got = oracle.token_adapters(ids, lens, adm)
    ref = np.repeat(np.where(adm, ids, 0), lens)
    assert np.array_equal(got, ref)


# -------------------------------------------------- dense identity, brute force

def _single_adapter_lane(seed, h_in, h_out, rank, T, x_dtype="bf16", mode="real",
                         tp_size=1, tp_rank=0):
    spec = WorkloadSpec(
        name="pin", seed=seed,
        lanes=(LaneSpec("l", h_in, tuple(h_out), x_dtype, tp_size, tp_rank),),
        n_adapters=1, ranks=(rank,), rank_mode="list", scale_mode="fixed",
        scale=1.75, max_rank=rank, decode_rows=T, base_prob=0.0)
    return generate(spec, mode=mode)


@pytest.mark.parametrize("x_dtype", ["bf16", "fp16"])
def test_dense_identity(x_dtype):
    """Single adapter: the factored delta equals scale * (B A) x with the dense
    [h_out, h_in] matrix formed by numpy's fp64 matmul."""
    w = _single_adapter_lane(11, 96, [40, 24], 7, 13, x_dtype)
    lane = w.lanes["l"]
    d, tok, _ = oracle.workload_lane_delta(w, "l")
    xf = (lane.x.view(np.float16).astype(np.float64) if x_dtype == "fp16"
          else bf16_bits_to_f32(lane.x).astype(np.float64))
    (aid, ad), = w.adapters.items()
    col = 0
    for sf in ad.lanes["l"]:
        A = bf16_bits_to_f32(sf.A).astype(np.float64)
        B = bf16_bits_to_f32(sf.B).astype(np.float64)
        M = np.matmul(B, A)                               # [h_out_j, h_in]
        ref = np.float64(sf.scale) * np.matmul(xf, M.T)   # [T, h_out_j]
        got = d[:, col:col + sf.B.shape[0]]
        err = np.abs(got - ref).max() / np.abs(ref).max()
        assert err <= 1e-12, err
        col += sf.B.shape[0]


def test_integer_brute_force_exact():
    """Integer mode: exact rational brute force through B @ A first."""
    w = _single_adapter_lane(12, 40, [9, 5], 3, 6, mode="int")
    lane = w.lanes["l"]
    d, _, _ = oracle.workload_lane_delta(w, "l")
    x = bf16_bits_to_f32(lane.x).astype(np.int64)
    (aid, ad), = w.adapters.items()
    col = 0
    for sf in ad.lanes["l"]:
        A = bf16_bits_to_f32(sf.A).astype(np.int64).tolist()
        B = bf16_bits_to_f32(sf.B).astype(np.int64).tolist()
        M = [[sum(B[o][k] * A[k][i] for k in range(sf.rank)) for i in range(40)]
             for o in range(len(B))]
        for t in range(x.shape[0]):
            for o in range(len(B)):
                exact = sum(M[o][i] * int(x[t, i]) for i in range(40)) * sf.scale
                assert d[t, col + o] == exact
        col += len(B)


# ---------------------------------------------------------------- invariants

def test_base_rows_get_zero_delta_and_scale_zero():
    w = generate(config_by_name("tiny"))
    d, tok, _ = oracle.workload_lane_delta(w, "proj")
    assert (tok == 0).any() and (tok != 0).any()
    assert np.all(d[tok == 0] == 0.0)
    assert np.all(np.abs(d[tok != 0]).max(axis=1) > 0)
    lane = w.lanes["proj"]
    factors = {aid: [(sf.A, sf.B, sf.rank, 0.0) for sf in ad.lanes["proj"]]
               for aid, ad in w.adapters.items()}
    d0 = oracle.lane_delta(lane.x, "bf16", tok, factors, lane.spec.h_out, 0, 64)
    assert np.all(d0 == 0.0)


def test_permutation_invariance():
    w = generate(config_by_name("decode_mix"))
    d, tok, _ = oracle.workload_lane_delta(w, "qkv")
    perm = np.random.default_rng(3).permutation(len(tok))
    lane = w.lanes["qkv"]
    factors = {aid: [(sf.A, sf.B, sf.rank, sf.scale) for sf in ad.lanes["qkv"]]
               for aid, ad in w.adapters.items()}
    dp = oracle.lane_delta(lane.x[perm], "bf16", tok[perm], factors,
                           lane.spec.h_out, 0, 4096)
    assert np.array_equal(dp, d[perm])


def test_linearity_exact_in_integer_mode():
    w = _single_adapter_lane(13, 64, [16], 4, 8, mode="int")
    lane = w.lanes["l"]
    x = bf16_bits_to_f32(lane.x)
    x1 = np.where(np.arange(64) < 32, x, 0).astype(np.float32)
    x2 = (x - x1).astype(np.float32)
    (aid, ad), = w.adapters.items()
    f = {aid: [(sf.A, sf.B, sf.rank, sf.scale) for sf in ad.lanes["l"]]}
    tok = np.full(8, aid)
    d = oracle.lane_delta(lane.x, "bf16", tok, f, [16], 0, 64)
    d1 = oracle.lane_delta(f32_to_bf16_bits(x1), "bf16", tok, f, [16], 0, 64)
    d2 = oracle.lane_delta(f32_to_bf16_bits(x2), "bf16", tok, f, [16], 0, 64)
    assert np.array_equal(d, d1 + d2)
    assert np.abs(d).max() > 0


def test_fused_slices_equal_separate_lanes():
    w = generate(config_by_name("decode_mix"))
    d, tok, _ = oracle.workload_lane_delta(w, "qkv")
    lane = w.lanes["qkv"]
    col = 0
    for j, hj in enumerate(lane.spec.h_out):
        f = {aid: [tuple((sf.A, sf.B, sf.rank, sf.scale))
                   for sf in ad.lanes["qkv"][j:j + 1]]
             for aid, ad in w.adapters.items()}
        dj = oracle.lane_delta(lane.x, "bf16", tok, f, [hj], 0, 4096)
        assert np.array_equal(dj, d[:, col:col + hj])
        col += hj


@pytest.mark.parametrize("mode", ["real", "int"])
def test_column_shares_sum_to_unsharded(mode):
    """A cut by input columns: the shares' deltas sum to the full delta."""
    tp = 8
    w = _single_adapter_lane(14, 8 * 24, [33], 5, 7, mode=mode)
    lane = w.lanes["l"]
    (aid, ad), = w.adapters.items()
    f = {aid: [(sf.A, sf.B, sf.rank, sf.scale) for sf in ad.lanes["l"]]}
    tok = np.full(7, aid)
    full = oracle.lane_delta(lane.x, "bf16", tok, f, [33], 0, 8 * 24)
    parts = np.zeros_like(full)
    for r in range(tp):
        xs = np.ascontiguousarray(lane.x[:, r * 24:(r + 1) * 24])
        parts += oracle.lane_delta(xs, "bf16", tok, f, [33], r * 24, 24)
    if mode == "int":
        assert np.array_equal(parts, full)
    else:
        assert np.abs(parts - full).max() <= 1e-12 * np.abs(full).max()


def test_deferred_rows_untouched():
    spec = config_by_name("many_tenants")
    w = generate(spec, lanes=("o_proj",))
    d, tok, adm = oracle.workload_lane_delta(w, "o_proj", max_loras=8)
    assert not all(adm)
    lens = w.seq_len
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    for s, ok in enumerate(adm):
        if not ok:
            assert np.all(d[starts[s]:starts[s] + lens[s]] == 0.0)
    assert len(set(tok.tolist()) - {0}) == 8


# ----------------------------------------------------- mixture-of-experts

SMALL_MOE = MoeSpec(
    name="small_moe", seed=31,
    lanes=(LaneSpec("gate_up", 64, (48, 40)), LaneSpec("down", 48, (64,))),
    n_experts=6, top_k=2, n_tokens=30, n_adapters=3, ranks=(4, 8, 3), max_rank=8,
    token_input=("gate_up",), scale_mode="uniform", scale_range=(0.5, 3.0),
    base_prob=0.2, expert_coverage=0.7)


def _dense_row(w, lane, p, pair):
    """scale * (B @ A) @ x of one dispatched row, as a dense product."""
    L = w.lanes[lane]
    x = bf16_bits_to_f32(L.x[p]).astype(np.float64)
    out = []
    for sf in w.factors[pair][lane]:
        A = bf16_bits_to_f32(sf.A).astype(np.float64)[:sf.rank]
        B = bf16_bits_to_f32(sf.B).astype(np.float64)[:, :sf.rank]
        out.append(sf.scale * (np.matmul(B, A) @ x))
    return np.concatenate(out)


@pytest.mark.parametrize("mode", ["real", "int"])
@pytest.mark.parametrize("lane", ["gate_up", "down"])
def test_moe_rows_match_dense_expert_product(lane, mode):
    """Every dispatched row equals the dense product of its (adapter, expert)
    factors, found here from the dispatch table directly; rows of base tokens
    and of experts the adapter does not edit are exactly zero."""
    w = generate_moe(SMALL_MOE, mode=mode)
    d, row_pair = oracle.moe_lane_delta(w, lane)
    n_edit = n_base = n_unedited = 0
    for p in range(w.n_rows):
        aid = int(w.tok_adapter[w.row_token[p]])
        e = int(w.row_expert[p])
        if aid == 0 or (aid, e) not in w.factors:
            assert row_pair[p] is None and not d[p].any()
            n_base += aid == 0
            n_unedited += aid != 0
            continue
        assert row_pair[p] == (aid, e)
        ref = _dense_row(w, lane, p, (aid, e))
        if mode == "int":
            assert np.array_equal(d[p], ref)
        else:
            assert np.allclose(d[p], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
        n_edit += 1
    assert n_edit > 0 and n_base > 0 and n_unedited > 0


def test_moe_dispatch_structure():
    """top_k distinct experts per token, rows grouped by expert then token,
    and the gate_up input of every row of a token is that token's row."""
    w = generate_moe(SMALL_MOE)
    k = SMALL_MOE.top_k
    assert w.n_rows == SMALL_MOE.n_tokens * k
    key = w.row_expert.astype(np.int64) * SMALL_MOE.n_tokens + w.row_token
    assert np.all(np.diff(key) > 0)
    for t in range(SMALL_MOE.n_tokens):
        rows = np.nonzero(w.row_token == t)[0]
        assert len(rows) == k and len(set(w.row_expert[rows].tolist())) == k
        x = w.lanes["gate_up"].x
        assert all(np.array_equal(x[rows[0]], x[r]) for r in rows)


def test_moe_row_order_does_not_matter():
    """Permuting the dispatched rows permutes the oracle's delta exactly."""
    w = generate_moe(SMALL_MOE)
    d, _ = oracle.moe_lane_delta(w, "down")
    perm = np.random.default_rng(3).permutation(w.n_rows)
    w.row_token, w.row_expert = w.row_token[perm], w.row_expert[perm]
    L = w.lanes["down"]
    L.x, L.y0 = L.x[perm], L.y0[perm]
    dp, _ = oracle.moe_lane_delta(w, "down")
    assert np.array_equal(dp, d[perm])


# ------------------------------------------------------------ folded A

from workloads import hadamard, draw_fold


def test_bf16_nearest_matches_torch_on_binary32_values():
    """For values that are exact in binary32, rounding to bf16 must agree
    with torch's binary32 -> bfloat16 conversion (nearest, ties to even)."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(41)
    hi = np.arange(0, 1 << 16, dtype=np.uint32)
    hi = hi[(hi & 0x7f80) != 0x7f80]                     # finite patterns only
    lo = np.concatenate([[0, 0x8000, 0x7fff, 0x8001, 0xffff],
                         rng.integers(0, 1 << 16, 11)]).astype(np.uint32)
    u = (hi[:, None] << 16 | lo[None, :]).reshape(-1)
    f = u.view(np.float32)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_nearest_bits(f.astype(np.float64)), ref)


def test_fold_identity_and_signed_permutation_are_exact():
    rng = np.random.default_rng(42)
    r, n, c0 = 5, 64, 32
    A = _bits(rng.standard_normal((r, c0 + n)) * 0.02)
    assert np.array_equal(oracle.fold_a(A, c0, n, np.eye(n, dtype=np.float32), r), A[:, c0:])
    perm = rng.permutation(n)
    sign = rng.choice([-1.0, 1.0], n)
    P = np.zeros((n, n), np.float32)
    P[perm, np.arange(n)] = sign                          # column c takes column perm[c]
    ref = bf16_bits_to_f32(A[:, c0:])[:, perm] * sign
    assert np.array_equal(oracle.fold_a(A, c0, n, P, r), _bits(ref))


def test_fold_reads_the_transformed_input():
    """With fold = M^-1 the exact folded factor applied to M x gives A x;
    M = diag(d) H / 8 with d powers of two, so every product is exact."""
    rng = np.random.default_rng(43)
    r, n = 6, 64
    A = _bits(rng.standard_normal((r, n)) * 0.02)
    d = 2.0 ** rng.integers(-2, 3, n)
    H = hadamard(n) / 8.0
    M = d[:, None] * H
    fold = (H.T / d[None, :]).astype(np.float32)
    x = bf16_bits_to_f32(_bits(rng.standard_normal((n, 3)))).astype(np.float64)
    Af = oracle.fold_a(A, 0, n, fold, r, rounded=False)
    ref = bf16_bits_to_f32(A).astype(np.float64) @ x
    assert np.allclose(Af @ (M @ x), ref, rtol=1e-12, atol=1e-15)
    # the stored factor is within half a bf16 unit of the exact one
    Ab = bf16_bits_to_f32(oracle.fold_a(A, 0, n, fold, r)).astype(np.float64)
    assert np.all(np.abs(Ab - Af) <= 2.0 ** -8 * np.abs(Af) + 2.0 ** -134)


def test_draw_fold_is_an_inverse():
    M, fold = draw_fold(7, 256)
    assert np.allclose(M @ fold.astype(np.float64), np.eye(256), atol=1e-6)


# ------------------------------------------- base projection + delta (fused)

def test_linear_worked_examples():
    with open(os.path.join(GOLDEN, "worked_examples.json")) as f:
        cases = json.load(f)["linear_cases"]
    for c in cases:
        x = _bits([c["x"], c["x"]])                 # row 0 runs the adapter, row 1 base
        W = _bits(c["W"])
        A, B = _bits(c["A"]), _bits(c["B"])
        h_in = x.shape[1]
        f = {5: [(A, B, A.shape[0], c["scale"])]}
        y = oracle.linear_lane(x, "bf16", W, [5, 0], f, [B.shape[0]], c.get("a_col0", 0), h_in)
        assert y.tolist() == [c["y_adapter"], c["y_base"]], c["name"]


def _decoded(bits, dtype="bf16"):
    return (bits.view(np.float16).astype(np.float64) if dtype == "fp16"
            else bf16_bits_to_f32(bits).astype(np.float64))


@pytest.mark.parametrize("x_dtype", ["bf16", "fp16"])
def test_linear_merged_weight_identity(x_dtype):
    """One adapter on every row: x W^T + scale B (A x) equals x (W + scale B A)^T
    with the merged [h_out, h_in] weight formed by numpy's fp64 matmul (the
    usual LoRA merge); base rows equal x W^T from numpy's matmul."""
    w = _single_adapter_lane(15, 96, [40, 24], 7, 13, x_dtype)
    lane = w.lanes["l"]
    W = draw_base_weight(w.spec, 0, lane.spec)
    y, tok, _ = oracle.workload_linear_lane(w, "l", W)
    xf = _decoded(lane.x, x_dtype)
    (aid, ad), = w.adapters.items()
    merged = []
    for sf in ad.lanes["l"]:
        M = np.matmul(bf16_bits_to_f32(sf.B).astype(np.float64),
                      bf16_bits_to_f32(sf.A).astype(np.float64))
        merged.append(np.float64(sf.scale) * M)
    Wm = _decoded(W) + np.concatenate(merged, axis=0)
    ref = np.matmul(xf, Wm.T)
    assert np.abs(y - ref).max() <= 1e-12 * np.abs(ref).max()
    base = oracle.base_product(lane.x, x_dtype, W, 96)
    ref_b = np.matmul(xf, _decoded(W).T)
    assert np.abs(base - ref_b).max() <= 1e-12 * np.abs(ref_b).max()


def test_linear_integer_brute_force_and_base_rows():
    """Integer inputs: every row against exact integer sums written out; rows
    of the base model get the base product alone, bit for bit."""
    spec = WorkloadSpec(
        name="lin_int", seed=16, lanes=(LaneSpec("l", 40, (9, 5)),), n_adapters=2,
        ranks=(3, 6), rank_mode="list", scale_mode="fixed", scale=2.0, max_rank=6,
        decode_rows=12, base_prob=0.3)
    w = generate(spec, mode="int")
    lane = w.lanes["l"]
    W = draw_base_weight(spec, 0, lane.spec, mode="int")
    y, tok, _ = oracle.workload_linear_lane(w, "l", W)
    x = bf16_bits_to_f32(lane.x).astype(np.int64).tolist()
    Wi = bf16_bits_to_f32(W).astype(np.int64).tolist()
    for t in range(len(x)):
        base = [sum(Wi[o][i] * x[t][i] for i in range(40)) for o in range(14)]
        want = list(base)
        if tok[t]:
            col = 0
            for sf in w.adapters[int(tok[t])].lanes["l"]:
                A = bf16_bits_to_f32(sf.A).astype(np.int64).tolist()
                B = bf16_bits_to_f32(sf.B).astype(np.int64).tolist()
                u = [sum(A[k][i] * x[t][i] for i in range(40)) for k in range(sf.rank)]
                for o in range(len(B)):
                    want[col + o] += sf.scale * sum(B[o][k] * u[k] for k in range(sf.rank))
                col += len(B)
        assert y[t].tolist() == want, t
    assert (tok == 0).any() and (tok != 0).any()
    base = oracle.base_product(lane.x, "bf16", W, 40)
    off = tok == 0
    assert np.array_equal(y[off].view(np.uint64), base[off].view(np.uint64))


@pytest.mark.parametrize("mode", ["real", "int"])
def test_linear_column_shares_sum_to_unsharded(mode):
    """A row-parallel layer cut in 8 input-column shares (W and A cut by
    columns, B whole): the shares' outputs sum to the unsharded output, the
    sum the cross-rank reduction forms."""
    tp, hs = 8, 24
    w = _single_adapter_lane(17, tp * hs, [33], 5, 7, mode=mode)
    lane = w.lanes["l"]
    W = draw_base_weight(w.spec, 0, lane.spec, mode=mode)
    (aid, ad), = w.adapters.items()
    f = {aid: [(sf.A, sf.B, sf.rank, sf.scale) for sf in ad.lanes["l"]]}
    tok = np.full(7, aid)
    full = oracle.linear_lane(lane.x, "bf16", W, tok, f, [33], 0, tp * hs)
    parts = np.zeros_like(full)
    for r in range(tp):
        xs = np.ascontiguousarray(lane.x[:, r * hs:(r + 1) * hs])
        Ws = np.ascontiguousarray(W[:, r * hs:(r + 1) * hs])
        parts += oracle.linear_lane(xs, "bf16", Ws, tok, f, [33], r * hs, hs)
    if mode == "int":
        assert np.array_equal(parts, full)
    else:
        assert np.abs(parts - full).max() <= 1e-12 * np.abs(full).max()
