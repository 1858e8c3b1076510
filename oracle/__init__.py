"""fp64 CPU oracle for the routed LoRA delta.  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package; the product library never does.  It shares no code with the HIP
path: admission and per-token routing are plain Python loops written from the
pages, the delta is the plain C loop in lora_oracle.c.

What it follows:
  * admission under max_loras -- tokenspeed PR #976, first commit message
    ("max_loras batch cap"): walk the candidate requests in order; a base-model
    request is never charged; a request whose adapter is already in the batch
    costs nothing; a request that would bring a new adapter past the cap is
    deferred and the walk goes on; max_loras == 0 means no cap at all.
  * per-token adapter ids -- xLLM PR #2014, "Wire-up": one adapter id per
    sequence, aligned with the sequences' query lengths, expanded to one id
    per token with repeat_interleave; id 0 is the base model (tokenspeed PR
    #976, third commit message).
  * the delta -- TensorFold PR #47, third commit message: scale * B @ (A @ x)
    added to the fp32 partial sum of the projection; a row of slot 0 is not
    read or written.

  * expert LoRA of a mixture-of-experts layer -- xLLM PR #2014, "Not in this
    PR" (the fused MoE expert LoRA delta, injected as a grouped GEMM): each
    dispatched (token, expert) row of an expert projection takes the factors
    of its token's adapter for that expert; the reading taken is that an
    adapter carries one LoRA pair per expert it edits, and a row whose token
    runs the base model, or whose adapter does not edit that expert, gets no
    delta.

  * the base projection with the delta in its partial sum -- TensorFold PR
    #47, third commit message and PR body "What this changes": the delta is
    added in fp32 to the partial sum the base projection produces, before the
    cross-rank reduction.  The reading taken: the projection's output is
    y = x W^T + delta, with W the linear layer's bf16 weight in its usual
    [out_features, in_features] orientation (this GPU's input columns for a
    row-parallel share), and a base-model row gets x W^T alone.

  * A folded onto a transformed input -- TensorFold PR #47, first and third
    commit messages: the packed shared expert's down projection reads a
    rotated, scaled fp16 hidden state x' = M x, and its adapter's A is
    rewritten once at load to read it.  The reading taken: the stored factor
    is A' = A M^-1 (the loader is given fold = M^-1), computed exactly and
    rounded to bf16, the factors' type, to nearest with ties to even.

Rows of deferred sequences are outside this batch: the oracle leaves them
exactly as they were, like base-model rows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lora_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

X_KIND = {"bf16": 1, "fp16": 2}


def build(force: bool = True) -> str:
    """Compile lora_oracle.c with gcc into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared",
               "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        lib.oracle_bf16_value.restype = ctypes.c_double
        lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
        lib.oracle_fp16_value.restype = ctypes.c_double
        lib.oracle_fp16_value.argtypes = [ctypes.c_uint16]
        P = ctypes.c_void_p
        I = ctypes.c_int64
        lib.oracle_slice_delta.restype = ctypes.c_int
        lib.oracle_slice_delta.argtypes = [
            I, P, I, P, I, ctypes.c_int32, I, P, I, I, I, P, I,
            ctypes.c_double, P, I, I]
        lib.oracle_linear_rows.restype = ctypes.c_int
        lib.oracle_linear_rows.argtypes = [I, P, I, P, I, ctypes.c_int32, I, P, I, P, I]
        _lib = lib
    return _lib


def bf16_value(bits: int) -> float:
    return _load().oracle_bf16_value(int(bits))


def fp16_value(bits: int) -> float:
    return _load().oracle_fp16_value(int(bits))


# --------------------------------------------------------------------------
# Admission and routing (tokenspeed PR #976; xLLM PR #2014 "Wire-up")
# --------------------------------------------------------------------------

def admit(seq_adapter_ids, max_loras: int):
    """Admission of candidate sequences under the distinct-adapter cap.

    Returns (admitted: list[bool], distinct: list[int] in order of admission).
    """
    admitted = []
    in_batch = []
    for aid in seq_adapter_ids:
        aid = int(aid)
        if aid == 0:
            admitted.append(True)             # base model: never charged
        elif aid in in_batch:
            admitted.append(True)             # reuse: no extra slot
        elif max_loras == 0 or len(in_batch) < max_loras:
            in_batch.append(aid)              # new adapter within the cap
            admitted.append(True)
        else:
            admitted.append(False)            # defer, keep scanning
    return admitted, in_batch


def token_adapters(seq_adapter_ids, seq_lens, admitted):
    """Per-token adapter id: repeat each sequence's id over its query length.

    Rows of a deferred sequence get id 0: they are not part of this batch and
    nothing reads or writes them.
    """
    out = []
    for aid, n, ok in zip(seq_adapter_ids, seq_lens, admitted):
        out.extend([int(aid) if ok else 0] * int(n))
    return np.array(out, dtype=np.int64)


# --------------------------------------------------------------------------
# The delta
# --------------------------------------------------------------------------

def slice_delta(rows, x_bits, x_dtype, A_bits, a_col0, h_in, B_bits, rank, scale):
    """fp64 delta of one adapter on one slice for the given rows of x.

    Returns float64 [len(rows), h_out_j].
    """
    lib = _load()
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    A_bits = np.ascontiguousarray(A_bits, dtype=np.uint16)
    B_bits = np.ascontiguousarray(B_bits, dtype=np.uint16)
    h_out = B_bits.shape[0]
    out = np.zeros((len(rows), h_out), dtype=np.float64)
    if len(rows) == 0 or h_out == 0:
        return out
    assert A_bits.shape[0] >= rank and B_bits.shape[1] >= rank
    assert a_col0 + h_in <= A_bits.shape[1] and x_bits.shape[1] >= h_in
    rc = lib.oracle_slice_delta(
        len(rows), rows.ctypes.data, h_in, x_bits.ctypes.data, x_bits.shape[1],
        X_KIND[x_dtype], rank, A_bits.ctypes.data, A_bits.shape[1], a_col0,
        h_out, B_bits.ctypes.data, B_bits.shape[1], float(scale),
        out.ctypes.data, h_out, 0)
    if rc != 0:
        raise MemoryError("oracle_slice_delta")
    return out


def lane_delta(x_bits, x_dtype, tok_adapter, factors, h_out, a_col0, h_in,
               rows=None):
    """fp64 delta of a lane for the rows `rows` (default: all rows of x).

    tok_adapter  per-token adapter id (0 = base, or deferred)
    factors      adapter id -> list over slices of (A_bits, B_bits, rank, scale)
    h_out        per-slice output widths; slice j sits at column sum(h_out[:j])

    Returns float64 [len(rows), sum(h_out)]; rows with adapter 0 are all zero.
    """
    tok_adapter = np.asarray(tok_adapter, dtype=np.int64)
    if rows is None:
        rows = np.arange(len(tok_adapter), dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    H = int(sum(h_out))
    delta = np.zeros((len(rows), H), dtype=np.float64)
    ids = tok_adapter[rows]
    for aid in sorted(set(ids.tolist()) - {0}):
        sel = np.nonzero(ids == aid)[0]
        col = 0
        for j, hj in enumerate(h_out):
            A, B, r, s = factors[aid][j]
            delta[sel, col:col + hj] = slice_delta(
                rows[sel], x_bits, x_dtype, A, a_col0, h_in, B, r, s)
            col += hj
    return delta


def workload_lane_delta(workload, lane_name, max_loras=None, rows=None):
    """Routing + delta for one lane of a generated workload.

    Returns (delta float64 [n_rows, H_out], tok_adapter int64 [T], admitted).
    """
    spec = workload.spec
    cap = spec.max_loras if max_loras is None else max_loras
    admitted, _ = admit(workload.seq_adapter, cap)
    tok = token_adapters(workload.seq_adapter, workload.seq_len, admitted)
    lane = workload.lanes[lane_name]
    factors = {aid: [(sf.A, sf.B, sf.rank, sf.scale) for sf in ad.lanes[lane_name]]
               for aid, ad in workload.adapters.items()}
    d = lane_delta(lane.x, lane.spec.x_dtype, tok, factors, lane.spec.h_out,
                   lane.spec.a_col0, lane.spec.h_in, rows)
    return d, tok, admitted


def moe_lane_delta(workload, lane_name, rows=None):
    """fp64 delta of one expert projection of a MoE layer.

    Dispatched row p is token row_token[p] sent to expert row_expert[p]; it
    takes the factors of (that token's adapter, that expert) when the adapter
    edits the expert, and no delta otherwise.

    Returns (delta float64 [len(rows), H_out], row_pair) where row_pair[p] is
    the (adapter id, expert) whose factors row p takes, or None.
    """
    lane = workload.lanes[lane_name]
    n = len(workload.row_token)
    pair_key = {}
    row_key = np.zeros(n, dtype=np.int64)
    row_pair = [None] * n
    for p in range(n):
        aid = int(workload.tok_adapter[workload.row_token[p]])
        pair = (aid, int(workload.row_expert[p]))
        if aid != 0 and pair in workload.factors:
            row_key[p] = pair_key.setdefault(pair, len(pair_key) + 1)
            row_pair[p] = pair
    factors = {key: [(sf.A, sf.B, sf.rank, sf.scale) for sf in workload.factors[pair][lane_name]]
               for pair, key in pair_key.items()}
    d = lane_delta(lane.x, lane.spec.x_dtype, row_key, factors, lane.spec.h_out,
                   lane.spec.a_col0, lane.spec.h_in, rows)
    return d, row_pair


def base_product(x_bits, x_dtype, W_bits, h_in, rows=None):
    """fp64 base projection x W^T of the given rows (default: all rows of x).

    x_bits [T, >= h_in] (bf16 or fp16 bits), W_bits [h_out, >= h_in] bf16
    bits.  Returns float64 [len(rows), h_out]."""
    lib = _load()
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    W_bits = np.ascontiguousarray(W_bits, dtype=np.uint16)
    if rows is None:
        rows = np.arange(x_bits.shape[0], dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    h_out = W_bits.shape[0]
    out = np.zeros((len(rows), h_out), dtype=np.float64)
    if len(rows) == 0 or h_out == 0:
        return out
    assert W_bits.shape[1] >= h_in and x_bits.shape[1] >= h_in
    rc = lib.oracle_linear_rows(len(rows), rows.ctypes.data, h_in, x_bits.ctypes.data,
                                x_bits.shape[1], X_KIND[x_dtype], h_out, W_bits.ctypes.data,
                                W_bits.shape[1], out.ctypes.data, h_out)
    if rc != 0:
        raise MemoryError("oracle_linear_rows")
    return out


def linear_lane(x_bits, x_dtype, W_bits, tok_adapter, factors, h_out, a_col0, h_in,
                rows=None):
    """fp64 output of a lane's projection with the delta in its partial sum:
    x W^T for every row, plus the delta for rows with an adapter (lane_delta's
    arguments).  Returns float64 [len(rows), sum(h_out)]."""
    base = base_product(x_bits, x_dtype, W_bits, h_in, rows)
    return base + lane_delta(x_bits, x_dtype, tok_adapter, factors, h_out, a_col0, h_in, rows)


def workload_linear_lane(workload, lane_name, W_bits, max_loras=None, rows=None):
    """Routing, base projection and delta for one lane of a generated
    workload.  Returns (y float64 [n_rows, H_out], tok_adapter, admitted)."""
    d, tok, admitted = workload_lane_delta(workload, lane_name, max_loras, rows)
    lane = workload.lanes[lane_name]
    base = base_product(lane.x, lane.spec.x_dtype, W_bits, lane.spec.h_in, rows)
    return base + d, tok, admitted


def bf16_nearest_bits(v):
    """bf16 bits of the nearest bf16 value to each float64 in v, ties to
    even (finite inputs): the significand is cut to 8 bits with rint, which
    rounds halves to even; below the smallest normal the spacing is 2^-133."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)                       # v = m * 2^e, 0.5 <= |m| < 1
    r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    tiny = np.abs(v) < 2.0 ** -126
    r = np.where(tiny, np.ldexp(np.rint(np.ldexp(v, 133)), -133), r)
    # r is a bf16 value, so its binary32 form is exact; keep its upper half
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def fold_a(A_bits, a_col0, h_in, fold, rank, rounded=True):
    """A' = A[:rank, a_col0:a_col0 + h_in] @ fold in fp64 (fold [h_in, >= h_in]
    is read as [h_in, h_in]); returned as bf16 bits [rank, h_in] when
    `rounded`, else the exact float64 product."""
    A = (np.asarray(A_bits, dtype=np.uint16)[:rank, a_col0:a_col0 + h_in]
         .astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    F = np.asarray(fold, dtype=np.float64)[:h_in, :h_in]
    P = np.matmul(A, F)
    return bf16_nearest_bits(P) if rounded else P
