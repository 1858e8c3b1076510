"""Seeded draws for the synthetic workloads (numpy PCG64).

Every component is drawn from its own stream, keyed by (seed, component, ...),
so a lane or an adapter can be generated alone and still get the same bits.

Two value modes:
  "real"  x ~ N(0,1), A and B ~ N(0, 0.02^2) (0.02 is the standard
          deviation), rounded to bf16 (fp16 for an fp16 lane) with
          round-to-nearest-even; y0 ~ N(0,1) or zeros.
  "int"   x has +-1 at min(h_in, 128) random positions per row and 0
          elsewhere, A and B take values in {-1, 0, 1}, each adapter's scale
          is one of {0.5, 1, 2, 4} and y0 holds integers in [-8, 8].  Every
          product and partial sum of the delta is then an exactly
          representable binary32 value (|A.x| <= 128, |delta| <= 128*512),
          whatever the summation order.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .configs import LaneSpec, WorkloadSpec

ID_BASE = 1000
ID_STRIDE = 37
INT_MODE_NNZ = 128


def adapter_registry_id(index: int) -> int:
    """Registry id of the adapter at 0-based position `index` (never 0)."""
    return ID_BASE + ID_STRIDE * (index + 1)


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round binary32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    out = ((u + r) >> 16).astype(np.uint16)
    if nan.any():
        out[nan] = ((u[nan] >> 16) | 0x0040).astype(np.uint16)
    return out


def bf16_bits_to_f32(b) -> np.ndarray:
    """Widen bf16 bits to binary32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def f32_to_fp16_bits(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def _stream(seed: int, *key: int) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy=int(seed), spawn_key=tuple(int(k) for k in key))
    return np.random.Generator(np.random.PCG64(ss))


@dataclass
class SliceFactors:
    """One adapter's factors for one output slice, in PEFT orientation.

    A: bf16 bits [rank, h_in_full]   (lora_A weight: rank x input features)
    B: bf16 bits [h_out_j, rank]     (lora_B weight: output features x rank)
    scale: the binary32 factor the product is multiplied by
    """
    rank: int
    scale: float
    A: np.ndarray
    B: np.ndarray


@dataclass
class Adapter:
    adapter_id: int
    index: int
    lanes: dict = field(default_factory=dict)   # lane name -> [SliceFactors]


@dataclass
class Lane:
    spec: LaneSpec
    x: np.ndarray    # uint16 bits [T, h_in], bf16 or fp16 per spec.x_dtype
    y0: np.ndarray   # float32 [T, sum(h_out)]

    @property
    def name(self) -> str:
        return self.spec.name


@dataclass
class Workload:
    spec: WorkloadSpec
    mode: str
    seq_adapter: np.ndarray   # int32 [n_seq], registry ids, 0 = base model
    seq_len: np.ndarray       # int32 [n_seq]
    adapters: dict            # registry id -> Adapter, in index order
    lanes: dict               # lane name -> Lane

    @property
    def n_tokens(self) -> int:
        return int(self.seq_len.sum())

    @property
    def adapter_ids(self) -> list:
        return list(self.adapters.keys())


def draw_structure(spec: WorkloadSpec):
    """Per-sequence registry ids (0 = base) and lengths."""
    rng = _stream(spec.seed, 0)
    n = spec.n_adapters
    ids = np.array([adapter_registry_id(i) for i in range(n)], dtype=np.int64)

    d = spec.decode_rows
    dec_ids = np.zeros(d, dtype=np.int64)
    if d:
        is_base = rng.random(d) < spec.base_prob
        if spec.popularity == "uniform":
            pick = rng.integers(0, n, size=d)
        elif spec.popularity == "zipf":
            w = np.arange(1, n + 1, dtype=np.float64) ** (-spec.zipf_s)
            pick = rng.choice(n, size=d, p=w / w.sum())
        else:
            raise ValueError(spec.popularity)
        dec_ids = np.where(is_base, 0, ids[pick])
    dec_len = np.ones(d, dtype=np.int64)

    p = spec.prefill_seqs
    pre_len = rng.integers(spec.prefill_len[0], spec.prefill_len[1] + 1, size=p)
    pre_ids = ids[rng.integers(0, n, size=p)] if p else np.zeros(0, np.int64)

    seq_ids = np.concatenate([dec_ids, pre_ids])
    seq_len = np.concatenate([dec_len, pre_len])
    if d and p:
        perm = rng.permutation(d + p)
        seq_ids, seq_len = seq_ids[perm], seq_len[perm]
    return seq_ids.astype(np.int32), seq_len.astype(np.int32)


def draw_ranks_scales(spec: WorkloadSpec, mode: str):
    rng = _stream(spec.seed, 1)
    n = spec.n_adapters
    if spec.rank_mode == "list":
        ranks = np.array(spec.ranks[:n], dtype=np.int64)
    elif spec.rank_mode == "choice":
        ranks = rng.choice(np.array(spec.ranks, dtype=np.int64), size=n)
    else:
        raise ValueError(spec.rank_mode)
    if mode == "int":
        scales = rng.choice(np.array([0.5, 1.0, 2.0, 4.0], np.float32), size=n)
    elif spec.scale_mode == "alpha":
        scales = (np.float32(spec.alpha) / ranks.astype(np.float32)).astype(np.float32)
    elif spec.scale_mode == "fixed":
        scales = np.full(n, spec.scale, dtype=np.float32)
    elif spec.scale_mode == "uniform":
        lo, hi = spec.scale_range
        scales = rng.uniform(lo, hi, size=n).astype(np.float32)
    else:
        raise ValueError(spec.scale_mode)
    return ranks, scales


def _factor(rng, shape, mode):
    if mode == "int":
        return f32_to_bf16_bits(rng.integers(-1, 2, size=shape).astype(np.float32))
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(0.02))


def draw_x(spec: WorkloadSpec, lane_index: int, lane: LaneSpec, T: int, mode: str):
    rng = _stream(spec.seed, 4, lane_index)
    h = lane.h_in
    if mode == "int":
        nnz = min(h, INT_MODE_NNZ)
        x = np.zeros((T, h), dtype=np.float32)
        if T:
            pos = np.argpartition(rng.random((T, h)), nnz - 1, axis=1)[:, :nnz]
            sgn = rng.integers(0, 2, size=(T, nnz)).astype(np.float32) * 2 - 1
            np.put_along_axis(x, pos, sgn, axis=1)
    else:
        x = rng.standard_normal((T, h), dtype=np.float32)
    return f32_to_fp16_bits(x) if lane.x_dtype == "fp16" else f32_to_bf16_bits(x)


def draw_y0(spec: WorkloadSpec, lane_index: int, lane: LaneSpec, T: int, mode: str,
            y0: str):
    rng = _stream(spec.seed, 5, lane_index)
    shape = (T, lane.h_out_total)
    if y0 == "zeros":
        return np.zeros(shape, dtype=np.float32)
    if mode == "int":
        return rng.integers(-8, 9, size=shape).astype(np.float32)
    return rng.standard_normal(shape, dtype=np.float32)


def generate(spec: WorkloadSpec, mode: str = "real", y0: str = "normal",
             lanes=None, with_activations: bool = True) -> Workload:
    """Draw a workload.  `lanes` restricts to a subset of lane names."""
    if mode not in ("real", "int"):
        raise ValueError(mode)
    seq_ids, seq_len = draw_structure(spec)
    T = int(seq_len.sum())
    ranks, scales = draw_ranks_scales(spec, mode)
    lane_list = [(li, l) for li, l in enumerate(spec.lanes)
                 if lanes is None or l.name in lanes]

    adapters = {}
    for i in range(spec.n_adapters):
        ad = Adapter(adapter_registry_id(i), i)
        r = int(ranks[i])
        for li, l in lane_list:
            sl = []
            for j, hj in enumerate(l.h_out):
                A = _factor(_stream(spec.seed, 2, i, li, j), (r, l.h_in_full), mode)
                B = _factor(_stream(spec.seed, 3, i, li, j), (hj, r), mode)
                sl.append(SliceFactors(r, float(scales[i]), A, B))
            ad.lanes[l.name] = sl
        adapters[ad.adapter_id] = ad

    lane_objs = {}
    for li, l in lane_list:
        if with_activations:
            x = draw_x(spec, li, l, T, mode)
            y = draw_y0(spec, li, l, T, mode, y0)
        else:
            x = np.zeros((0, l.h_in), np.uint16)
            y = np.zeros((0, l.h_out_total), np.float32)
        lane_objs[l.name] = Lane(l, x, y)
    return Workload(spec, mode, seq_ids, seq_len, adapters, lane_objs)


def hadamard(n: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order n (a power of two), entries +-1."""
    if n < 1 or n & (n - 1):
        raise ValueError("n must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def draw_fold(seed: int, n: int):
    """An input transform of n features and its inverse, as a projection that
    reads a rotated, scaled hidden state would see it: M = diag(d) H / sqrt(n)
    with H the Hadamard matrix and d ~ U[0.5, 2] per feature.

    Returns (M float64 [n, n], fold float32 [n, n]) with fold = M^-1 =
    H^T diag(1/d) / sqrt(n), rounded to binary32 (the fold a loader is given)."""
    rng = _stream(seed, 20, n)
    d = rng.uniform(0.5, 2.0, size=n)
    h = hadamard(n) / np.sqrt(n)
    M = d[:, None] * h
    fold = np.ascontiguousarray((h.T / d[None, :]).astype(np.float32))
    return M, fold


def draw_base_weight(spec: WorkloadSpec, lane_index: int, lane: LaneSpec, mode: str = "real"):
    """The base projection's weight of a lane as this GPU holds it: bf16 bits
    [sum(h_out), h_in] (out_features x this GPU's input columns), drawn from
    its own stream.  "real": N(0, 0.02^2) like the factors; "int": values in
    {-1, 0, 1}, so x W^T of an integer-mode x is exact (|.| <= 128)."""
    return _factor(_stream(spec.seed, 6, lane_index), (lane.h_out_total, lane.h_in), mode)
