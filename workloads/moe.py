"""Seeded draws for mixture-of-experts workloads (numpy PCG64).

A MoE layer sends every token to `top_k` distinct experts; each (token,
expert) pair is one dispatched row of the expert projections, and the rows are
laid out grouped by expert, then by token (the order a grouped GEMM reads
them in).  An adapter that edits the experts carries its own factors per
expert; `expert_coverage` < 1 leaves some (adapter, expert) pairs without
factors (the adapter does not edit that expert).

Like the dense generator this module only draws numbers and holds none of the
delta's arithmetic.  Value modes are those of the dense generator ("real" and
"int").
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .configs import LaneSpec
from .gen import (SliceFactors, Lane, _factor, _stream, adapter_registry_id,
                  f32_to_bf16_bits, f32_to_fp16_bits, INT_MODE_NNZ)


@dataclass(frozen=True)
class MoeSpec:
    name: str
    seed: int
    lanes: tuple                   # LaneSpec per expert projection
    n_experts: int
    top_k: int
    n_tokens: int
    n_adapters: int
    ranks: tuple                   # rank per adapter (all experts of an adapter)
    max_rank: int
    token_input: tuple = ()        # lanes whose input row is the token's hidden state
    alpha: float = 32.0
    scale_mode: str = "alpha"      # "alpha" (alpha / r) or "uniform"
    scale_range: tuple = (0.5, 4.0)
    base_prob: float = 0.25
    expert_coverage: float = 1.0
    prefill_frac: float = 0.0      # fraction of tokens that are prefill tokens
    description: str = ""


@dataclass
class MoeWorkload:
    spec: MoeSpec
    mode: str
    tok_adapter: np.ndarray    # int32 [T], registry ids, 0 = base model
    row_token: np.ndarray      # int32 [R], token of each dispatched row
    row_expert: np.ndarray     # int32 [R], expert of each dispatched row
    factors: dict              # (registry id, expert) -> {lane name: [SliceFactors]}
    lanes: dict                # lane name -> Lane (x [R, h_in], y0 [R, H_out])
    tok_prefill: np.ndarray    # bool [T], the token belongs to a prefill chunk

    @property
    def adapter_ids(self) -> list:
        return [adapter_registry_id(i) for i in range(self.spec.n_adapters)]

    @property
    def n_rows(self) -> int:
        return len(self.row_token)

    @property
    def row_prefill(self) -> np.ndarray:
        return self.tok_prefill[self.row_token]


def draw_dispatch(spec: MoeSpec):
    """Per-token adapter ids, and the dispatched rows grouped by expert."""
    rng = _stream(spec.seed, 10)
    T, E, k = spec.n_tokens, spec.n_experts, spec.top_k
    ids = np.array([adapter_registry_id(i) for i in range(spec.n_adapters)], dtype=np.int64)
    is_base = rng.random(T) < spec.base_prob
    tok_adapter = np.where(is_base, 0, ids[rng.integers(0, spec.n_adapters, size=T)])
    # top_k distinct experts per token: the k smallest of E uniform scores
    experts = np.argsort(rng.random((T, E)), axis=1)[:, :k]
    token = np.repeat(np.arange(T), k)
    expert = experts.reshape(-1)
    order = np.lexsort((token, expert))
    return (tok_adapter.astype(np.int32), token[order].astype(np.int32),
            expert[order].astype(np.int32))


def draw_coverage(spec: MoeSpec):
    """Boolean [n_adapters, n_experts]: which experts each adapter edits."""
    rng = _stream(spec.seed, 11)
    if spec.expert_coverage >= 1.0:
        return np.ones((spec.n_adapters, spec.n_experts), dtype=bool)
    return rng.random((spec.n_adapters, spec.n_experts)) < spec.expert_coverage


def draw_moe_scales(spec: MoeSpec, mode: str):
    rng = _stream(spec.seed, 12)
    n = spec.n_adapters
    ranks = np.array(spec.ranks[:n], dtype=np.int64)
    if mode == "int":
        return ranks, rng.choice(np.array([0.5, 1.0, 2.0, 4.0], np.float32), size=n)
    if spec.scale_mode == "alpha":
        return ranks, (np.float32(spec.alpha) / ranks.astype(np.float32)).astype(np.float32)
    lo, hi = spec.scale_range
    return ranks, rng.uniform(lo, hi, size=n).astype(np.float32)


def _activations(rng, lane: LaneSpec, n: int, mode: str):
    """n rows of lane inputs, drawn as the dense generator draws x."""
    h = lane.h_in
    if mode == "int":
        nnz = min(h, INT_MODE_NNZ)
        x = np.zeros((n, h), dtype=np.float32)
        if n:
            pos = np.argpartition(rng.random((n, h)), nnz - 1, axis=1)[:, :nnz]
            sgn = rng.integers(0, 2, size=(n, nnz)).astype(np.float32) * 2 - 1
            np.put_along_axis(x, pos, sgn, axis=1)
    else:
        x = rng.standard_normal((n, h), dtype=np.float32)
    return f32_to_fp16_bits(x) if lane.x_dtype == "fp16" else f32_to_bf16_bits(x)


def _partial_sums(rng, lane: LaneSpec, n: int, mode: str, y0: str):
    shape = (n, lane.h_out_total)
    if y0 == "zeros":
        return np.zeros(shape, dtype=np.float32)
    if mode == "int":
        return rng.integers(-8, 9, size=shape).astype(np.float32)
    return rng.standard_normal(shape, dtype=np.float32)


def generate_moe(spec: MoeSpec, mode: str = "real", y0: str = "normal") -> MoeWorkload:
    if mode not in ("real", "int"):
        raise ValueError(mode)
    tok_adapter, row_token, row_expert = draw_dispatch(spec)
    cover = draw_coverage(spec)
    ranks, scales = draw_moe_scales(spec, mode)
    factors = {}
    for i in range(spec.n_adapters):
        aid = adapter_registry_id(i)
        r = int(ranks[i])
        for e in range(spec.n_experts):
            if not cover[i, e]:
                continue
            per_lane = {}
            for li, l in enumerate(spec.lanes):
                sl = []
                for j, hj in enumerate(l.h_out):
                    A = _factor(_stream(spec.seed, 14, i, e, li, j), (r, l.h_in_full), mode)
                    B = _factor(_stream(spec.seed, 15, i, e, li, j), (hj, r), mode)
                    sl.append(SliceFactors(r, float(scales[i]), A, B))
                per_lane[l.name] = sl
            factors[(aid, e)] = per_lane
    R = len(row_token)
    lanes = {}
    for li, l in enumerate(spec.lanes):
        if l.name in spec.token_input:
            # every dispatched row of a token carries the token's hidden state
            x = _activations(_stream(spec.seed, 16, li), l, spec.n_tokens, mode)[row_token]
        else:
            x = _activations(_stream(spec.seed, 16, li), l, R, mode)
        y = _partial_sums(_stream(spec.seed, 17, li), l, R, mode, y0)
        lanes[l.name] = Lane(l, np.ascontiguousarray(x), y)
    if spec.prefill_frac >= 1.0:
        tok_prefill = np.ones(spec.n_tokens, dtype=bool)
    elif spec.prefill_frac <= 0.0:
        tok_prefill = np.zeros(spec.n_tokens, dtype=bool)
    else:
        tok_prefill = _stream(spec.seed, 18).random(spec.n_tokens) < spec.prefill_frac
    return MoeWorkload(spec, mode, tok_adapter, row_token, row_expert, factors, lanes,
                       tok_prefill)


# Expert projections of a Qwen3-30B-A3B-sized MoE layer (hidden 2048, 128
# experts of intermediate size 768, top 8), the model the multi-tenant LoRA
# framework page validates on; 256 decode tokens, 8 adapters of rank 16.
MOE_DECODE = MoeSpec(
    name="moe_decode", seed=6,
    lanes=(LaneSpec("expert_gate_up", 2048, (768, 768)),
           LaneSpec("expert_down", 768, (2048,))),
    n_experts=128, top_k=8, n_tokens=256, n_adapters=8, ranks=(16,) * 8, max_rank=16,
    token_input=("expert_gate_up",), base_prob=0.25,
    description="T=256 decode tokens x top-8 of 128 experts = 2048 dispatched rows; "
                "expert gate_up 2048->768|768 and down 768->2048; 8 adapters r=16 "
                "alpha=32 on every expert, 25% base")

# The same layer on a 2048-token prefill chunk: 16384 dispatched rows, about
# 12 per (adapter, expert) pair.
MOE_PREFILL = MoeSpec(
    name="moe_prefill", seed=7,
    lanes=(LaneSpec("expert_gate_up", 2048, (768, 768)),
           LaneSpec("expert_down", 768, (2048,))),
    n_experts=128, top_k=8, n_tokens=2048, n_adapters=8, ranks=(16,) * 8, max_rank=16,
    token_input=("expert_gate_up",), base_prob=0.25, prefill_frac=1.0,
    description="T=2048 prefill tokens x top-8 of 128 experts = 16384 dispatched rows; "
                "expert gate_up 2048->768|768 and down 768->2048; 8 adapters r=16 "
                "alpha=32 on every expert, 25% base")

MOE_CONFIGS = (MOE_DECODE, MOE_PREFILL)


def moe_config_by_name(name: str) -> MoeSpec:
    for c in MOE_CONFIGS:
        if c.name == name:
            return c
    raise KeyError(name)
