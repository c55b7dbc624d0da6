"""A small object wrapper over the C ABI (argument marshalling only)."""
from __future__ import annotations

from typing import Optional, Sequence

from . import _lora


class LoraPool:
    """Owns one ``lora_pool_t``.  All methods forward to the C entry points."""

    def __init__(self, max_adapters: int, max_ids: int, max_rank: int, d_in: Sequence[int],
                 d_out: Sequence[int], max_tokens: int, stream=None):
        self.max_tokens = max_tokens
        self.d_in = list(d_in)
        self.d_out = list(d_out)
        self.handle = _lora.lora_pool_create(max_adapters, max_ids, max_rank, d_in, d_out,
                                             max_tokens, stream)
        self._plans = []

    def close(self) -> None:
        if self.handle:
            _lora.lora_pool_destroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def load_adapter(self, adapter_id: int, rank: int, alpha: float, A, B, stream=None):
        _lora.lora_load_adapter(self.handle, adapter_id, rank, alpha, A, B, stream)

    def unload_adapter(self, adapter_id: int, stream=None):
        _lora.lora_unload_adapter(self.handle, adapter_id, stream)

    def query(self, adapter_id: int):
        return _lora.lora_pool_query(self.handle, adapter_id)

    def plan_create(self) -> int:
        p = _lora.lora_plan_create(self.handle)
        self._plans.append(p)
        return p

    def plan(self, ids, T: int, plan: int, stream=None):
        _lora.lora_plan(self.handle, ids, T, plan, stream)

    def apply(self, module: int, X, ids, W, out, plan: Optional[int] = None, stream=None,
              T: Optional[int] = None):
        T = X.shape[0] if T is None else T
        _lora.lora_apply(self.handle, module, X, ids, T, W, out, plan, stream)

    def base_apply(self, module: int, X, W, out, stream=None, T: Optional[int] = None):
        T = X.shape[0] if T is None else T
        _lora.lora_base_apply(self.handle, module, X, T, W, out, stream)

    def status(self, stream=None) -> str:
        return _lora.lora_status(self.handle, stream)

    def debug_read_plan(self, plan: Optional[int] = None, stream=None):
        return _lora.lora_debug_read_plan(self.handle, plan, self.max_tokens, stream)

    # host <-> device paging
    def host_cache_create(self, max_cpu_adapters: int):
        _lora.lora_host_cache_create(self.handle, max_cpu_adapters)

    def host_register(self, adapter_id: int, rank: int, alpha: float, A, B):
        _lora.lora_host_register(self.handle, adapter_id, rank, alpha, A, B)

    def host_unregister(self, adapter_id: int, stream=None):
        _lora.lora_host_unregister(self.handle, adapter_id, stream)

    def prefetch(self, ids, stream=None):
        _lora.lora_prefetch(self.handle, ids, stream)

    def pin(self, adapter_id: int, pin: bool = True, stream=None):
        _lora.lora_pin_adapter(self.handle, adapter_id, pin, stream)

    def paging_query(self, adapter_id: int):
        return _lora.lora_paging_query(self.handle, adapter_id)

    def paging_stats(self):
        return _lora.lora_paging_stats(self.handle)

    # INT4 base weight
    def apply_q4(self, module: int, X, ids, Wq, Wsz, out, W_scratch=None, plan: Optional[int] = None,
                 stream=None, T: Optional[int] = None):
        T = X.shape[0] if T is None else T
        _lora.lora_apply_q4(self.handle, module, X, ids, T, Wq, Wsz, W_scratch, out, plan, stream)

    def base_apply_q4(self, module: int, X, Wq, Wsz, out, W_scratch=None, stream=None,
                      T: Optional[int] = None):
        T = X.shape[0] if T is None else T
        _lora.lora_base_apply_q4(self.handle, module, X, T, Wq, Wsz, W_scratch, out, stream)

    def load_chain(self, chain_id: int, members, stream=None):
        _lora.lora_load_chain(self.handle, chain_id, members, stream)
