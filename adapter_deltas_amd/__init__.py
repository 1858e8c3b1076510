"""Routed LoRA delta for MI355X (gfx950): y += scale * B @ (A @ x) per token,
with slot 0 the base model.  The compute runs in liblora.so (HIP kernels);
importing this package loads it and fails if it has not been built."""
from . import _lib
from .lora import (
    LoraError, Pool, Routing, make_desc, workspace_for, shrink, expand, delta_apply,
    DEFAULT_PREFILL_MIN_LEN, NO_PREFILL, DEVICE_ROUTING_MAX_TOKENS,
    lora_last_error, lora_version, lora_pool_bytes, lora_pool_create, lora_pool_destroy,
    lora_pool_load, lora_pool_load_folded, lora_pool_unload, lora_pool_slot_of, lora_routing_bytes,
    lora_routing_create, lora_routing_destroy, lora_build_routing, lora_routing_get_info,
    lora_plan_routing,
    lora_routing_token_slots, lora_build_routing_device, lora_build_routing_moe,
    lora_build_routing_rows, lora_plan_rows,
    lora_routing_device_counts, moe_slot, moe_row_slots,
    lora_shrink, lora_expand, lora_workspace_bytes,
    lora_delta_apply, lora_delta_apply_noalloc, delta_apply_noalloc,
    lora_linear_workspace_bytes, lora_linear_delta, linear_delta,
)

_lib.load()

__all__ = [n for n in dir() if n.startswith(("lora_", "Lora")) or n in (
    "Pool", "Routing", "make_desc", "workspace_for", "shrink", "expand", "delta_apply",
    "delta_apply_noalloc", "linear_delta",
    "DEFAULT_PREFILL_MIN_LEN", "NO_PREFILL", "DEVICE_ROUTING_MAX_TOKENS", "moe_slot",
    "moe_row_slots")]
