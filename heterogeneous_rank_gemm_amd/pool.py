"""A small object wrapper over the C ABI (argument marshalling only).

Before a tensor's address is handed to the library, its dtype, layout,
device and shape are checked here: the C entry points see raw pointers and
cannot tell an int64 id tensor, a transposed view or a short buffer from a
valid one."""
from __future__ import annotations

from typing import Optional, Sequence

from . import _lora
from ._lora import LoraError


def check_tensor(t, name: str, dtype, cols: Optional[int], min_rows: int, where: str,
                 need_cuda: bool = True) -> None:
    """Raises LoraError (INVALID_ARG) unless ``t`` is a contiguous tensor of
    ``dtype`` with at least ``min_rows`` rows of ``cols`` columns (a 1-D
    tensor of at least ``min_rows`` entries when ``cols`` is None) on a GPU."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise LoraError(1, f"{where}: {name} must be a torch tensor")
    if t.dtype != dtype:
        raise LoraError(1, f"{where}: {name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise LoraError(1, f"{where}: {name} is not contiguous")
    if cols is None:
        if t.dim() != 1 or t.shape[0] < min_rows:
            raise LoraError(1, f"{where}: {name} has shape {tuple(t.shape)}, expected ({min_rows},)")
    elif t.dim() != 2 or t.shape[1] != cols or t.shape[0] < min_rows:
        raise LoraError(1, f"{where}: {name} has shape {tuple(t.shape)}, expected (>={min_rows}, {cols})")
    if need_cuda and not t.is_cuda:
        raise LoraError(1, f"{where}: {name} is not on a GPU")


def _bf16():
    import torch
    return torch.bfloat16


def _i32():
    import torch
    return torch.int32


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
        check_tensor(ids, "ids", _i32(), None, T, "lora_plan")
        _lora.lora_plan(self.handle, ids, T, plan, stream)

    def _check_linear(self, where: str, module: int, X, ids, W, out, T: int) -> None:
        if not 0 <= module < len(self.d_in):
            raise LoraError(1, f"{where}: module {module} out of range")
        din, dout = self.d_in[module], self.d_out[module]
        check_tensor(X, "X", _bf16(), din, T, where)
        if ids is not None:
            check_tensor(ids, "ids", _i32(), None, T, where)
        if W is not None:
            check_tensor(W, "W", _bf16(), din, dout, where)
            if W.shape[0] != dout:
                raise LoraError(1, f"{where}: W has {W.shape[0]} rows, expected {dout}")
        check_tensor(out, "out", _bf16(), dout, T, where)

    def apply(self, module: int, X, ids, W, out, plan: Optional[int] = None, stream=None,
              T: Optional[int] = None):
        T = X.shape[0] if T is None else T
        self._check_linear("lora_apply", module, X, ids, W, out, T)
        _lora.lora_apply(self.handle, module, X, ids, T, W, out, plan, stream)

    def base_apply(self, module: int, X, W, out, stream=None, T: Optional[int] = None):
        T = X.shape[0] if T is None else T
        self._check_linear("lora_base_apply", module, X, None, W, out, T)
        _lora.lora_base_apply(self.handle, module, X, T, W, out, stream)

    def apply_group(self, modules: Sequence[int], X, ids, W: Sequence, out: Sequence,
                    plan: Optional[int] = None, stream=None, T: Optional[int] = None):
        """lora_apply_group: the linears ``modules`` (one d_in) on the same X."""
        T = X.shape[0] if T is None else T
        for m, w, o in zip(modules, W, out):
            self._check_linear("lora_apply_group", m, X, ids, w, o, T)
        _lora.lora_apply_group(self.handle, modules, X, ids, T, W, out, plan, stream)

    def base_apply_group(self, modules: Sequence[int], X, W: Sequence, out: Sequence, stream=None,
                         T: Optional[int] = None):
        T = X.shape[0] if T is None else T
        for m, w, o in zip(modules, W, out):
            self._check_linear("lora_base_apply_group", m, X, None, w, o, T)
        _lora.lora_base_apply_group(self.handle, modules, X, T, W, out, stream)

    def pack_weight(self, W, stream=None):
        """A new device tensor holding row-major W (d_out x d_in bf16) in the
        decode kernels' fragment-tile layout (lora_pack_weight)."""
        import torch
        check_tensor(W, "W", _bf16(), W.shape[1] if W.dim() == 2 else -1, 1, "lora_pack_weight")
        N, K = W.shape
        Wp = torch.empty(_lora.lora_packed_weight_elems(N, K), dtype=torch.bfloat16, device=W.device)
        _lora.lora_pack_weight(W, N, K, Wp, stream)
        return Wp

    def _check_packed(self, where: str, modules, X, ids, Wp, out, T: int) -> None:
        import torch
        for m, w, o in zip(modules, Wp, out):
            self._check_linear(where, m, X, ids, None, o, T)
            n = _lora.lora_packed_weight_elems(self.d_out[m], self.d_in[m])
            if not isinstance(w, torch.Tensor) or w.dtype != torch.bfloat16 or not w.is_contiguous() \
                    or w.numel() < n or not w.is_cuda:
                raise LoraError(1, f"{where}: a packed weight of module {m} holds {n} bf16 on a GPU")

    def apply_group_packed(self, modules: Sequence[int], X, ids, Wp: Sequence, out: Sequence, stream=None,
                           T: Optional[int] = None):
        """lora_apply_group_packed: decode batches (T <= 64), weights from pack_weight."""
        T = X.shape[0] if T is None else T
        self._check_packed("lora_apply_group_packed", modules, X, ids, Wp, out, T)
        _lora.lora_apply_group_packed(self.handle, modules, X, ids, T, Wp, out, stream)

    def base_apply_group_packed(self, modules: Sequence[int], X, Wp: Sequence, out: Sequence, stream=None,
                                T: Optional[int] = None):
        T = X.shape[0] if T is None else T
        self._check_packed("lora_base_apply_group_packed", modules, X, None, Wp, out, T)
        _lora.lora_base_apply_group_packed(self.handle, modules, X, T, Wp, out, stream)

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
    def _check_q4(self, where: str, module: int, Wq, Wsz, W_scratch) -> None:
        import torch
        din, dout = self.d_in[module], self.d_out[module]
        if Wq.dtype not in (torch.int32, torch.uint32) or Wsz.dtype not in (torch.int32, torch.uint32):
            raise LoraError(1, f"{where}: Wq and Wsz hold 32-bit words")
        check_tensor(Wq, "Wq", Wq.dtype, din // 8, dout, where)
        check_tensor(Wsz, "Wsz", Wsz.dtype, din // 128, dout, where)
        if W_scratch is not None:
            if W_scratch.dtype != torch.bfloat16 or not W_scratch.is_contiguous() or \
                    W_scratch.numel() < din * dout or not W_scratch.is_cuda:
                raise LoraError(1, f"{where}: W_scratch must hold {dout} x {din} bf16 on a GPU")

    def apply_q4(self, module: int, X, ids, Wq, Wsz, out, W_scratch=None, plan: Optional[int] = None,
                 stream=None, T: Optional[int] = None):
        T = X.shape[0] if T is None else T
        self._check_linear("lora_apply_q4", module, X, ids, None, out, T)
        self._check_q4("lora_apply_q4", module, Wq, Wsz, W_scratch)
        _lora.lora_apply_q4(self.handle, module, X, ids, T, Wq, Wsz, W_scratch, out, plan, stream)

    def base_apply_q4(self, module: int, X, Wq, Wsz, out, W_scratch=None, stream=None,
                      T: Optional[int] = None):
        T = X.shape[0] if T is None else T
        self._check_linear("lora_base_apply_q4", module, X, None, None, out, T)
        self._check_q4("lora_base_apply_q4", module, Wq, Wsz, W_scratch)
        _lora.lora_base_apply_q4(self.handle, module, X, T, Wq, Wsz, W_scratch, out, stream)

    def _check_q4_scratch(self, where: str, modules, W_scratch) -> None:
        import torch
        need = max(self.d_in[m] * self.d_out[m] for m in modules) if len(modules) else 0
        if W_scratch is not None and (W_scratch.dtype != torch.bfloat16 or not W_scratch.is_contiguous()
                                      or W_scratch.numel() < need or not W_scratch.is_cuda):
            raise LoraError(1, f"{where}: W_scratch must hold {need} bf16 on a GPU")

    def apply_group_q4(self, modules: Sequence[int], X, ids, Wq: Sequence, Wsz: Sequence, out: Sequence,
                       W_scratch=None, plan: Optional[int] = None, stream=None, T: Optional[int] = None):
        """lora_apply_group_q4: the linears ``modules`` (one d_in) on the same X, INT4 weights."""
        T = X.shape[0] if T is None else T
        for m, q, z, o in zip(modules, Wq, Wsz, out):
            self._check_linear("lora_apply_group_q4", m, X, ids, None, o, T)
            self._check_q4("lora_apply_group_q4", m, q, z, None)
        self._check_q4_scratch("lora_apply_group_q4", modules, W_scratch)
        _lora.lora_apply_group_q4(self.handle, modules, X, ids, T, Wq, Wsz, W_scratch, out, plan, stream)

    def base_apply_group_q4(self, modules: Sequence[int], X, Wq: Sequence, Wsz: Sequence, out: Sequence,
                            W_scratch=None, stream=None, T: Optional[int] = None):
        T = X.shape[0] if T is None else T
        for m, q, z, o in zip(modules, Wq, Wsz, out):
            self._check_linear("lora_base_apply_group_q4", m, X, None, None, o, T)
            self._check_q4("lora_base_apply_group_q4", m, q, z, None)
        self._check_q4_scratch("lora_base_apply_group_q4", modules, W_scratch)
        _lora.lora_base_apply_group_q4(self.handle, modules, X, T, Wq, Wsz, W_scratch, out, stream)

    def load_chain(self, chain_id: int, members, stream=None):
        _lora.lora_load_chain(self.handle, chain_id, members, stream)
