"""Python binding of the C ABI in include/lora.h.

The functions carry the C names and only marshal arguments (torch tensors and
numpy arrays to raw pointers, the current torch stream to a hipStream_t).
PyTorch provides device memory and streams; every step of the delta runs in
the library's HIP kernels.  `Pool` and `Routing` bundle a handle with the
torch buffer that backs it.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import numpy as np

from . import _lib as L

DEFAULT_PREFILL_MIN_LEN = 64
NO_PREFILL = 2**31 - 1
DEVICE_ROUTING_MAX_TOKENS = L.DEVICE_ROUTING_MAX_TOKENS


class LoraError(RuntimeError):
    def __init__(self, code: int, message: str):
        self.code = code
        self.status = L.STATUS.get(code, str(code))
        super().__init__(f"{self.status}: {message}")


def _lib():
    return L.load()


def lora_last_error() -> str:
    return _lib().lora_last_error().decode()


def lora_version() -> str:
    return _lib().lora_version().decode()


def _check(rc: int):
    if rc != L.LORA_OK:
        raise LoraError(rc, lora_last_error())


_current_stream = None


def _stream(stream) -> Optional[int]:
    """A stream argument as a raw handle; None is torch's current stream on the
    current device (looked up without building a Stream object: this runs on
    every call, and the object costs a few microseconds)."""
    global _current_stream
    if stream is None:
        if _current_stream is None:
            import torch
            raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
            dev = torch.cuda.current_device
            _current_stream = ((lambda: raw(dev())) if raw is not None else
                               (lambda: torch.cuda.current_stream().cuda_stream))
        return _current_stream()
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr(a) -> int:
    if a is None:
        return 0
    if isinstance(a, int):
        return a
    if isinstance(a, np.ndarray):
        return a.ctypes.data
    return a.data_ptr()


def make_desc(h_in: int, h_out: Sequence[int], max_slots: int, max_rank: int,
              x_dtype: str = "bf16") -> L.LaneDesc:
    d = L.LaneDesc()
    d.h_in = h_in
    d.n_slices = len(h_out)
    for j, h in enumerate(h_out):
        d.h_out[j] = h
    d.max_slots = max_slots
    d.max_rank = max_rank
    d.x_dtype = L.DTYPE[x_dtype]
    return d


# ---------------------------------------------------------------- raw calls

def lora_pool_bytes(desc: L.LaneDesc) -> int:
    n = ctypes.c_int64()
    _check(_lib().lora_pool_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def lora_pool_create(desc, dev_mem, dev_bytes, stream=None) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check(_lib().lora_pool_create(ctypes.byref(desc), _ptr(dev_mem), dev_bytes,
                                   _stream(stream), ctypes.byref(h)))
    return h


def lora_pool_destroy(pool) -> None:
    _check(_lib().lora_pool_destroy(pool))


def lora_pool_load(pool, adapter_id, slot, A, lda, a_col0, B, ldb, rank, scale,
                   src_on_device, stream=None) -> int:
    n = len(A)
    Ap = (ctypes.c_void_p * n)(*[_ptr(a) for a in A])
    Bp = (ctypes.c_void_p * n)(*[_ptr(b) for b in B])
    la = (ctypes.c_int64 * n)(*lda)
    lb = (ctypes.c_int64 * n)(*ldb)
    rk = (ctypes.c_int32 * n)(*rank)
    sc = (ctypes.c_float * n)(*scale)
    out = ctypes.c_int32(0)
    _check(_lib().lora_pool_load(pool, adapter_id, slot, Ap, la, a_col0, Bp, lb, rk, sc,
                                 int(src_on_device), _stream(stream), ctypes.byref(out)))
    return out.value


def lora_pool_load_folded(pool, adapter_id, slot, A, lda, a_col0, B, ldb, rank, scale, fold,
                          ld_fold, stream=None) -> int:
    """Device A, B and fold (fp32 [h_in][ld_fold]): A is stored as A @ fold."""
    n = len(A)
    Ap = (ctypes.c_void_p * n)(*[_ptr(a) for a in A])
    Bp = (ctypes.c_void_p * n)(*[_ptr(b) for b in B])
    la = (ctypes.c_int64 * n)(*lda)
    lb = (ctypes.c_int64 * n)(*ldb)
    rk = (ctypes.c_int32 * n)(*rank)
    sc = (ctypes.c_float * n)(*scale)
    out = ctypes.c_int32(0)
    _check(_lib().lora_pool_load_folded(pool, adapter_id, slot, Ap, la, a_col0, Bp, lb, rk, sc,
                                        _ptr(fold), ld_fold, _stream(stream), ctypes.byref(out)))
    return out.value


def lora_pool_unload(pool, adapter_id) -> None:
    _check(_lib().lora_pool_unload(pool, adapter_id))


def lora_pool_slot_of(pool, adapter_id) -> int:
    s = ctypes.c_int32()
    _check(_lib().lora_pool_slot_of(pool, adapter_id, ctypes.byref(s)))
    return s.value


def lora_routing_bytes(max_tokens: int) -> int:
    n = ctypes.c_int64()
    _check(_lib().lora_routing_bytes(max_tokens, ctypes.byref(n)))
    return n.value


def lora_routing_create(max_tokens, max_seqs, dev_mem, dev_bytes) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check(_lib().lora_routing_create(max_tokens, max_seqs, _ptr(dev_mem), dev_bytes,
                                      ctypes.byref(h)))
    return h


def lora_routing_destroy(routing) -> None:
    _check(_lib().lora_routing_destroy(routing))


def _seq_ids(seq_adapter_id) -> np.ndarray:
    """int32 registry ids per sequence; a missing id (None) is the base model,
    id 0 (tokenspeed PR #976, first commit message: the front end turns a
    request without a LoRA id into id 0)."""
    return np.ascontiguousarray([0 if a is None else a for a in seq_adapter_id],
                                dtype=np.int32)


def lora_build_routing(pool, seq_adapter_id, seq_len, max_loras, prefill_min_len,
                       routing, stream=None):
    ids = _seq_ids(seq_adapter_id)
    lens = np.ascontiguousarray(seq_len, dtype=np.int32)
    n = len(ids)
    if len(lens) != n:
        raise ValueError("seq_adapter_id and seq_len differ in length")
    adm = np.zeros(max(n, 1), dtype=np.uint8)
    nd = ctypes.c_int32()
    _check(_lib().lora_build_routing(
        pool, n, ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
        lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), max_loras, prefill_min_len,
        routing, adm.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), ctypes.byref(nd),
        _stream(stream)))
    return adm[:n].astype(bool), nd.value


def lora_routing_get_info(routing) -> dict:
    info = L.RoutingInfo()
    _check(_lib().lora_routing_get_info(routing, ctypes.byref(info)))
    return info.as_dict()


def _task_tables(words, offs, n_active, n_tokens):
    """The per-row metadata and shrink task words of a packed plan: 4 words
    per active row {slot, rank0 | rank1 << 16, rank2 | rank3 << 16, 0}, the
    decode (GEMV) tasks, and the matrix-core task table per lane slice count
    (absent: no table)."""
    h = offs[4]
    m0 = (offs[2] + n_tokens + 3) // 4 * 4
    if m0 + 4 * n_active != offs[3]:
        raise LoraError(f"plan words: row metadata at {m0} does not end at the tasks ({offs[3]})")
    meta = words[m0:offs[3]].reshape(-1, 4).copy()
    mfma = {}
    for s in range(1, 5):
        o, n = int(words[h + 2 * (s - 1)]), int(words[h + 2 * (s - 1) + 1])
        if n:
            mfma[s] = words[h + o:h + o + n].view(np.uint32).copy()
    return dict(row_meta=meta, gemv_tasks=words[offs[3]:h].view(np.uint32).copy(),
                mfma_tasks=mfma)


def lora_plan_routing(seq_adapter_id, seq_len, max_loras, prefill_min_len, resident,
                      max_slots, max_tokens, resident_rank=None):
    """Host-only routing plan.  `resident` maps registry id -> slot and
    `resident_rank` (optional) registry id -> per-slice ranks.

    Returns a dict with info counts, admitted (bool array), the tables seg
    (int32 [n_seg, 16]), rows (int32 [n_active]) and tok_slot (int32 [T]),
    the per-row metadata row_meta (int32 [n_active, 4]) and the shrink task
    words gemv_tasks and mfma_tasks ({slice count: words}).
    """
    i32p = ctypes.POINTER(ctypes.c_int32)
    ids = _seq_ids(seq_adapter_id)
    lens = np.ascontiguousarray(seq_len, dtype=np.int32)
    rid = np.ascontiguousarray(list(resident.keys()), dtype=np.int32)
    rsl = np.ascontiguousarray(list(resident.values()), dtype=np.int32)
    rrk = np.zeros((max(len(rid), 1), 4), dtype=np.int32)
    for i, aid in enumerate(resident.keys()):
        rk = (resident_rank or {}).get(aid, ())
        rrk[i, :len(rk)] = rk
    cap = lora_routing_bytes(max_tokens) // 4
    words = np.zeros(cap, dtype=np.int32)
    offs = np.zeros(5, dtype=np.int32)
    info = L.RoutingInfo()
    adm = np.zeros(max(len(ids), 1), dtype=np.uint8)
    _check(_lib().lora_plan_routing(
        len(ids), ids.ctypes.data_as(i32p), lens.ctypes.data_as(i32p), max_loras,
        prefill_min_len, len(rid), rid.ctypes.data_as(i32p), rsl.ctypes.data_as(i32p),
        rrk.ctypes.data_as(i32p), max_slots, max_tokens, words.ctypes.data_as(i32p), cap,
        offs.ctypes.data_as(i32p),
        ctypes.byref(info), adm.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))))
    d = info.as_dict()
    return dict(
        info=d, admitted=adm[:len(ids)].astype(bool),
        seg=words[offs[0]:offs[0] + L.SEG_WORDS * d["n_segments"]].reshape(-1, L.SEG_WORDS).copy(),
        rows=words[offs[1]:offs[1] + d["n_active"]].copy(),
        tok_slot=words[offs[2]:offs[2] + d["n_tokens"]].copy(),
        **_task_tables(words, offs, d["n_active"], d["n_tokens"]))


def lora_routing_token_slots(routing) -> int:
    p = ctypes.c_void_p()
    _check(_lib().lora_routing_token_slots(routing, ctypes.byref(p)))
    return p.value or 0


def lora_build_routing_device(pool, tok_slot, n_tokens, routing, stream=None) -> None:
    """tok_slot: device int32 tensor (or address) of the slot of each row."""
    _check(_lib().lora_build_routing_device(pool, _ptr(tok_slot), n_tokens, routing,
                                            _stream(stream)))


def lora_build_routing_moe(pool, tok_slot, n_tokens, row_token, row_expert, n_rows, n_experts,
                           routing, stream=None) -> None:
    """Device int32 tensors (or addresses): adapter slot per token, and the
    token and expert of each dispatched row."""
    _check(_lib().lora_build_routing_moe(pool, _ptr(tok_slot), n_tokens, _ptr(row_token),
                                         _ptr(row_expert), n_rows, n_experts, routing,
                                         _stream(stream)))


def lora_build_routing_rows(pool, row_slot, row_prefill, routing, stream=None) -> None:
    """Host arrays: int32 slot per row (0 = skip) and optional uint8 prefill flags."""
    slots = np.ascontiguousarray(row_slot, dtype=np.int32)
    pre = None if row_prefill is None else np.ascontiguousarray(row_prefill, dtype=np.uint8)
    if pre is not None and len(pre) != len(slots):
        raise ValueError("row_slot and row_prefill differ in length")
    _check(_lib().lora_build_routing_rows(
        pool, len(slots), slots.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
        None if pre is None else pre.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)),
        routing, _stream(stream)))


def lora_plan_rows(row_slot, row_prefill, max_slots, slot_rank, max_tokens):
    """Host-only plan from per-row slots.  slot_rank: int32 [max_slots + 1, 4].

    Returns a dict with info counts, the tables seg (int32 [n_seg, 16]),
    rows (int32 [n_active]) and tok_slot (int32 [n_rows]), the per-row
    metadata row_meta (int32 [n_active, 4]) and the shrink task words
    gemv_tasks and mfma_tasks ({slice count: words})."""
    i32p = ctypes.POINTER(ctypes.c_int32)
    slots = np.ascontiguousarray(row_slot, dtype=np.int32)
    pre = None if row_prefill is None else np.ascontiguousarray(row_prefill, dtype=np.uint8)
    rk = np.ascontiguousarray(slot_rank, dtype=np.int32)
    if rk.shape != (max_slots + 1, 4):
        raise ValueError("slot_rank must be [max_slots + 1, 4]")
    cap = lora_routing_bytes(max_tokens) // 4
    words = np.zeros(cap, dtype=np.int32)
    offs = np.zeros(5, dtype=np.int32)
    info = L.RoutingInfo()
    _check(_lib().lora_plan_rows(
        len(slots), slots.ctypes.data_as(i32p),
        None if pre is None else pre.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)),
        max_slots, rk.ctypes.data_as(i32p), words.ctypes.data_as(i32p), cap,
        offs.ctypes.data_as(i32p), ctypes.byref(info)))
    d = info.as_dict()
    return dict(
        info=d,
        seg=words[offs[0]:offs[0] + L.SEG_WORDS * d["n_segments"]].reshape(-1, L.SEG_WORDS).copy(),
        rows=words[offs[1]:offs[1] + d["n_active"]].copy(),
        tok_slot=words[offs[2]:offs[2] + d["n_tokens"]].copy(),
        **_task_tables(words, offs, d["n_active"], d["n_tokens"]))


def moe_slot(adapter_slot: int, expert: int, n_experts: int) -> int:
    """Pool slot of (adapter slot, expert) in an expert projection's pool
    (LORA_MOE_SLOT)."""
    return (adapter_slot - 1) * n_experts + expert + 1


def moe_row_slots(tok_slot, row_token, row_expert, n_experts, row_edited=None):
    """Pool slot of every dispatched row of a MoE layer, for
    lora_build_routing_rows: moe_slot(adapter slot of the row's token, the
    row's expert), or 0 for a row of a base token (slot 0) or a row whose
    adapter does not edit its expert (row_edited False)."""
    a = np.asarray(tok_slot, dtype=np.int64)[np.asarray(row_token, dtype=np.int64)]
    e = np.asarray(row_expert, dtype=np.int64)
    s = moe_slot(a, e, n_experts)
    keep = a != 0
    if row_edited is not None:
        keep &= np.asarray(row_edited, dtype=bool)
    return np.where(keep, s, 0).astype(np.int32)


def lora_routing_device_counts(routing) -> int:
    p = ctypes.c_void_p()
    _check(_lib().lora_routing_device_counts(routing, ctypes.byref(p)))
    return p.value or 0


def lora_shrink(pool, routing, x, ldx, v, stream=None) -> None:
    _check(_lib().lora_shrink(pool, routing, _ptr(x), ldx, _ptr(v), _stream(stream)))


def lora_expand(pool, routing, v, y, ldy, stream=None) -> None:
    _check(_lib().lora_expand(pool, routing, _ptr(v), _ptr(y), ldy, _stream(stream)))


def lora_workspace_bytes(pool, routing) -> int:
    n = ctypes.c_int64()
    _check(_lib().lora_workspace_bytes(pool, routing, ctypes.byref(n)))
    return n.value


def lora_delta_apply(pool, routing, x, ldx, y, ldy, workspace, workspace_bytes,
                     stream=None) -> None:
    _check(_lib().lora_delta_apply(pool, routing, _ptr(x), ldx, _ptr(y), ldy,
                                   _ptr(workspace), workspace_bytes, _stream(stream)))


def lora_delta_apply_noalloc(pool, routing, x, ldx, y, ldy, stream=None) -> None:
    _check(_lib().lora_delta_apply_noalloc(pool, routing, _ptr(x), ldx, _ptr(y), ldy,
                                           _stream(stream)))


def lora_linear_workspace_bytes(pool, routing) -> int:
    n = ctypes.c_int64()
    _check(_lib().lora_linear_workspace_bytes(pool, routing, ctypes.byref(n)))
    return n.value


def lora_linear_delta(pool, routing, n_rows, W, ldw, x, ldx, y, ldy, workspace,
                      workspace_bytes, stream=None) -> None:
    _check(_lib().lora_linear_delta(pool, routing, n_rows, _ptr(W), ldw, _ptr(x), ldx, _ptr(y),
                                    ldy, _ptr(workspace), workspace_bytes, _stream(stream)))


# ------------------------------------------------------------ owning wrappers

class Pool:
    """A lane's adapter pool: a handle plus the torch buffer holding it."""

    def __init__(self, h_in, h_out, max_slots, max_rank, x_dtype="bf16",
                 device="cuda", stream=None):
        import torch
        self.desc = make_desc(h_in, h_out, max_slots, max_rank, x_dtype)
        self.h_in, self.h_out = h_in, tuple(h_out)
        self.max_slots, self.max_rank, self.x_dtype = max_slots, max_rank, x_dtype
        self.rank_pad = -(-max_rank // 16) * 16
        self.v_stride = len(h_out) * self.rank_pad
        self.nbytes = lora_pool_bytes(self.desc)
        self.mem = torch.empty(self.nbytes, dtype=torch.uint8, device=device)
        self.handle = lora_pool_create(self.desc, self.mem, self.nbytes, stream)

    def load(self, adapter_id, A, B, ranks, scales, a_col0=0, slot=-1, stream=None):
        """A[j] [rank_j, lda] and B[j] [h_out_j, ldb] bf16 bits or bfloat16
        tensors; numpy arrays are host sources, torch cuda tensors device ones."""
        on_dev = not isinstance(A[0], np.ndarray)
        if on_dev:
            A = [a.contiguous() for a in A]
            B = [b.contiguous() for b in B]
        else:
            A = [np.ascontiguousarray(a, dtype=np.uint16) for a in A]
            B = [np.ascontiguousarray(b, dtype=np.uint16) for b in B]
        lda = [a.shape[1] for a in A]
        ldb = [b.shape[1] for b in B]
        return lora_pool_load(self.handle, adapter_id, slot, A, lda, a_col0, B, ldb,
                              list(ranks), list(scales), on_dev, stream)

    def load_folded(self, adapter_id, A, B, ranks, scales, fold, a_col0=0, slot=-1,
                    stream=None):
        """Like load, for a lane whose input arrives as M x: device factors and
        fold = M^-1 (fp32 cuda tensor [h_in, >= h_in]); A is stored as A @ fold."""
        A = [a.contiguous() for a in A]
        B = [b.contiguous() for b in B]
        if fold.stride(1) != 1:
            fold = fold.contiguous()
        return lora_pool_load_folded(self.handle, adapter_id, slot, A, [a.shape[1] for a in A],
                                     a_col0, B, [b.shape[1] for b in B], list(ranks),
                                     list(scales), fold, fold.stride(0), stream)

    def unload(self, adapter_id):
        lora_pool_unload(self.handle, adapter_id)

    def slot_of(self, adapter_id):
        return lora_pool_slot_of(self.handle, adapter_id)

    def close(self):
        if getattr(self, "handle", None):
            lora_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Routing:
    """Per-batch routing: a handle plus the torch buffer holding its tables."""

    def __init__(self, max_tokens, max_seqs, device="cuda"):
        import torch
        self.max_tokens, self.max_seqs = max_tokens, max_seqs
        self.nbytes = lora_routing_bytes(max_tokens)
        self.mem = torch.empty(self.nbytes, dtype=torch.uint8, device=device)
        self.handle = lora_routing_create(max_tokens, max_seqs, self.mem, self.nbytes)

    def build(self, pool: Pool, seq_adapter_id, seq_len, max_loras=0,
              prefill_min_len=DEFAULT_PREFILL_MIN_LEN, stream=None):
        return lora_build_routing(pool.handle, seq_adapter_id, seq_len, max_loras,
                                  prefill_min_len, self.handle, stream)

    def build_device(self, pool: Pool, tok_slot, stream=None):
        """Routing of a decode batch built on the device from an int32 device
        tensor of per-row slots (0 = base)."""
        lora_build_routing_device(pool.handle, tok_slot, int(tok_slot.numel()), self.handle,
                                  stream)

    def build_moe(self, pool: Pool, tok_slot, row_token, row_expert, n_experts, stream=None):
        """Routing of a MoE layer's dispatched rows built on the device from
        int32 device tensors: adapter slot per token, token and expert per row."""
        lora_build_routing_moe(pool.handle, tok_slot, int(tok_slot.numel()), row_token,
                               row_expert, int(row_token.numel()), n_experts, self.handle,
                               stream)

    def build_rows(self, pool: Pool, row_slot, row_prefill=None, stream=None):
        """Routing planned on the host from the slot of every row (0 = skip)
        and, optionally, which rows belong to prefill tokens."""
        lora_build_routing_rows(pool.handle, row_slot, row_prefill, self.handle, stream)

    def device_counts(self):
        """The int32 [8] device counts of a device-built routing, as a tensor
        viewing the routing's memory."""
        import torch
        off = (lora_routing_device_counts(self.handle) - self.mem.data_ptr()) // 4
        return self.mem.view(torch.int32)[off:off + 8]

    def info(self) -> dict:
        return lora_routing_get_info(self.handle)

    def token_slots(self):
        """int32 [n_tokens] view of the per-token slot array in device memory."""
        import torch
        n = self.info()["n_tokens"]
        off = lora_routing_token_slots(self.handle) - self.mem.data_ptr()
        return self.mem[off:off + 4 * n].view(torch.int32)

    def close(self):
        if getattr(self, "handle", None):
            lora_routing_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def workspace_for(pool: Pool, routing: Routing, device="cuda"):
    import torch
    n = lora_workspace_bytes(pool.handle, routing.handle)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def shrink(pool: Pool, routing: Routing, x, v, stream=None):
    lora_shrink(pool.handle, routing.handle, x, x.stride(0), v, stream)


def expand(pool: Pool, routing: Routing, v, y, stream=None):
    lora_expand(pool.handle, routing.handle, v, y, y.stride(0), stream)


def delta_apply(pool: Pool, routing: Routing, x, y, workspace=None, stream=None):
    if workspace is None:
        workspace = workspace_for(pool, routing, y.device)
    lora_delta_apply(pool.handle, routing.handle, x, x.stride(0), y, y.stride(0),
                     workspace, workspace.numel(), stream)
    return workspace


def delta_apply_noalloc(pool: Pool, routing: Routing, x, y, stream=None):
    """delta_apply with v in the library's static scratch (no workspace)."""
    lora_delta_apply_noalloc(pool.handle, routing.handle, x, x.stride(0), y, y.stride(0), stream)


def linear_delta(pool: Pool, routing, W, x, y, workspace=None, stream=None):
    """y = x W^T (+ the delta of the routing's rows; routing None: no delta).
    W: bf16 bits [sum(h_out), >= h_in] on the device."""
    rh = routing.handle if routing is not None else None
    if workspace is None:
        n = lora_linear_workspace_bytes(pool.handle, rh)
        if n > 0:
            import torch
            workspace = torch.empty(n, dtype=torch.uint8, device=y.device)
    nbytes = workspace.numel() if workspace is not None else 0
    lora_linear_delta(pool.handle, rh, x.shape[0], W, W.stride(0), x, x.stride(0), y,
                      y.stride(0), workspace, nbytes, stream)
    return workspace
