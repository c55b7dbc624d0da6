"""MI355X-native heterogeneous-batch LoRA linear.

The product is the C-ABI library ``libhrglora.so`` (``include/lora.h``);
``heterogeneous_rank_gemm_amd._lora`` is its ctypes binding with the same
entry-point names, and :class:`LoraPool` a small convenience wrapper over it.
Importing the package fails loudly when the library is not built.
"""
from . import _lora
from ._lora import (LoraError, STATUS_NAMES, EXPORTED, lora_status_string, lora_pool_create,
                    lora_pool_destroy, lora_load_adapter, lora_unload_adapter, lora_pool_query,
                    lora_plan_create, lora_plan_destroy, lora_plan, lora_apply, lora_base_apply,
                    lora_status, lora_debug_read_plan, lora_host_cache_create,
                    lora_host_register, lora_host_unregister, lora_prefetch, lora_pin_adapter,
                    lora_paging_query, lora_paging_stats, lora_q4_pack, lora_apply_q4,
                    lora_base_apply_q4, lora_load_chain, lora_apply_group, lora_base_apply_group,
                    lora_packed_weight_elems, lora_pack_weight, lora_apply_group_packed,
                    lora_base_apply_group_packed, lora_apply_noalloc, lora_apply_group_q4,
                    lora_base_apply_group_q4)
from .pool import LoraPool

__all__ = [
    "LoraError", "STATUS_NAMES", "EXPORTED", "LoraPool", "lora_status_string",
    "lora_pool_create", "lora_pool_destroy", "lora_load_adapter", "lora_unload_adapter",
    "lora_pool_query", "lora_plan_create", "lora_plan_destroy", "lora_plan", "lora_apply",
    "lora_base_apply", "lora_status", "lora_debug_read_plan", "lora_host_cache_create",
    "lora_host_register", "lora_host_unregister", "lora_prefetch", "lora_pin_adapter",
    "lora_paging_query", "lora_paging_stats", "lora_q4_pack", "lora_apply_q4", "lora_base_apply_q4",
    "lora_load_chain", "lora_apply_group", "lora_base_apply_group", "lora_packed_weight_elems",
    "lora_pack_weight", "lora_apply_group_packed", "lora_base_apply_group_packed", "lora_apply_noalloc",
    "lora_apply_group_q4", "lora_base_apply_group_q4",
]
