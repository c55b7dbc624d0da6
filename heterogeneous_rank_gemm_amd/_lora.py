"""ctypes binding of ``include/lora.h``: the same entry points, argument
marshalling only.  Every step of the LoRA linear runs in the HIP library;
nothing here computes.  Tensors are passed as raw device pointers
(``tensor.data_ptr()``), streams as ``torch.cuda.Stream.cuda_stream``.

Importing this module loads ``libhrglora.so`` and raises ``ImportError``
if it is missing -- there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhrglora.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python heterogeneous_rank_gemm_amd/build.py`")
_lib = C.CDLL(LIB_PATH)

STATUS_NAMES = {
    0: "OK", 1: "INVALID_ARG", 2: "OOM", 3: "POOL_FULL", 4: "RANK", 5: "EXISTS",
    6: "NOT_LOADED", 7: "ID_RANGE", 8: "HIP",
}
EXPORTED = (
    "lora_status_string", "lora_pool_create", "lora_pool_destroy", "lora_load_adapter",
    "lora_unload_adapter", "lora_pool_query", "lora_plan_create", "lora_plan_destroy",
    "lora_plan", "lora_apply", "lora_base_apply", "lora_status", "lora_debug_read_plan",
    "lora_host_cache_create", "lora_host_register", "lora_host_unregister", "lora_prefetch",
    "lora_pin_adapter", "lora_paging_query", "lora_paging_stats", "lora_q4_pack", "lora_apply_q4",
    "lora_base_apply_q4", "lora_load_chain", "lora_apply_group", "lora_base_apply_group",
    "lora_packed_weight_elems", "lora_pack_weight", "lora_apply_group_packed",
    "lora_base_apply_group_packed", "lora_apply_noalloc", "lora_apply_group_q4", "lora_base_apply_group_q4",
)

_vp = C.c_void_p
_i32 = C.c_int32
_P_i32 = C.POINTER(C.c_int32)

_lib.lora_status_string.restype = C.c_char_p
_lib.lora_status_string.argtypes = [C.c_int]
_sigs = {
    "lora_pool_create": [C.POINTER(_vp), _i32, _i32, _i32, _i32, _P_i32, _P_i32, _i32, _vp],
    "lora_pool_destroy": [_vp],
    "lora_load_adapter": [_vp, _i32, _i32, C.c_float, C.POINTER(_vp), C.POINTER(_vp), _vp],
    "lora_unload_adapter": [_vp, _i32, _vp],
    "lora_pool_query": [_vp, _i32, _P_i32, _P_i32, C.POINTER(C.c_float)],
    "lora_plan_create": [_vp, C.POINTER(_vp)],
    "lora_plan_destroy": [_vp, _vp],
    "lora_plan": [_vp, _vp, _i32, _vp, _vp],
    "lora_apply": [_vp, _i32, _vp, _vp, _i32, _vp, _vp, _vp, _vp],
    "lora_base_apply": [_vp, _i32, _vp, _i32, _vp, _vp, _vp],
    "lora_status": [_vp, _vp],
    "lora_debug_read_plan": [_vp, _vp, _P_i32, _P_i32, _P_i32, _P_i32, _P_i32, _P_i32, _vp],
    "lora_host_cache_create": [_vp, _i32],
    "lora_host_register": [_vp, _i32, _i32, C.c_float, C.POINTER(_vp), C.POINTER(_vp)],
    "lora_host_unregister": [_vp, _i32, _vp],
    "lora_prefetch": [_vp, _P_i32, _i32, _vp],
    "lora_pin_adapter": [_vp, _i32, _i32, _vp],
    "lora_paging_query": [_vp, _i32, _P_i32, _P_i32],
    "lora_paging_stats": [_vp, C.POINTER(C.c_int64), C.POINTER(C.c_int64), C.POINTER(C.c_int64)],
    "lora_q4_pack": [_vp, _vp, _vp, _i32, _i32, _vp, _vp],
    "lora_apply_q4": [_vp, _i32, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp],
    "lora_base_apply_q4": [_vp, _i32, _vp, _i32, _vp, _vp, _vp, _vp, _vp],
    "lora_load_chain": [_vp, _i32, _i32, _P_i32, _vp],
    "lora_apply_group": [_vp, _i32, _P_i32, _vp, _vp, _i32, C.POINTER(_vp), C.POINTER(_vp), _vp, _vp],
    "lora_base_apply_group": [_vp, _i32, _P_i32, _vp, _i32, C.POINTER(_vp), C.POINTER(_vp), _vp],
    "lora_packed_weight_elems": [_i32, _i32, C.POINTER(C.c_int64)],
    "lora_pack_weight": [_vp, _i32, _i32, _vp, _vp],
    "lora_apply_group_packed": [_vp, _i32, _P_i32, _vp, _vp, _i32, C.POINTER(_vp), C.POINTER(_vp), _vp],
    "lora_apply_group_q4": [_vp, _i32, _P_i32, _vp, _vp, _i32, C.POINTER(_vp), C.POINTER(_vp), _vp,
                            C.POINTER(_vp), _vp, _vp],
    "lora_base_apply_group_q4": [_vp, _i32, _P_i32, _vp, _i32, C.POINTER(_vp), C.POINTER(_vp), _vp,
                                 C.POINTER(_vp), _vp],
    "lora_base_apply_group_packed": [_vp, _i32, _P_i32, _vp, _i32, C.POINTER(_vp), C.POINTER(_vp), _vp],
    "lora_apply_noalloc": [_vp, _i32, _vp, _vp, _i32, _vp, _vp, _vp],
}
for _name, _args in _sigs.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = C.c_int


class LoraError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = int(code)
        self.status = STATUS_NAMES.get(self.code, f"UNKNOWN({code})")
        super().__init__(f"{where}: {_lib.lora_status_string(self.code).decode()}")


def _check(code: int, where: str) -> int:
    if code != 0:
        raise LoraError(code, where)
    return code


def _ptr(t) -> Optional[int]:
    """Device/host address of a tensor (or an int address, or None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ---------------------------------------------------------------------------
# entry points, same names as the C ABI
# ---------------------------------------------------------------------------
def lora_status_string(code: int) -> str:
    return _lib.lora_status_string(int(code)).decode()


def lora_pool_create(max_adapters: int, max_ids: int, max_rank: int, d_in: Sequence[int],
                     d_out: Sequence[int], max_tokens: int, stream=None) -> int:
    n = len(d_in)
    if len(d_out) != n:
        raise LoraError(1, "lora_pool_create")
    din = (C.c_int32 * max(n, 1))(*d_in)
    dout = (C.c_int32 * max(n, 1))(*d_out)
    h = _vp()
    _check(_lib.lora_pool_create(C.byref(h), max_adapters, max_ids, max_rank, n, din, dout,
                                 max_tokens, _stream(stream)), "lora_pool_create")
    return h.value


def lora_pool_destroy(pool: int) -> None:
    _check(_lib.lora_pool_destroy(pool), "lora_pool_destroy")


def lora_load_adapter(pool: int, adapter_id: int, rank: int, alpha: float, A: Sequence,
                      B: Sequence, stream=None) -> None:
    n = len(A)
    pa = (_vp * max(n, 1))(*[_ptr(a) for a in A])
    pb = (_vp * max(n, 1))(*[_ptr(b) for b in B])
    _check(_lib.lora_load_adapter(pool, adapter_id, rank, float(alpha), pa, pb, _stream(stream)),
           "lora_load_adapter")


def lora_unload_adapter(pool: int, adapter_id: int, stream=None) -> None:
    _check(_lib.lora_unload_adapter(pool, adapter_id, _stream(stream)), "lora_unload_adapter")


def lora_pool_query(pool: int, adapter_id: int):
    slot, rank, scale = C.c_int32(), C.c_int32(), C.c_float()
    _check(_lib.lora_pool_query(pool, adapter_id, C.byref(slot), C.byref(rank), C.byref(scale)),
           "lora_pool_query")
    return slot.value, rank.value, scale.value


def lora_plan_create(pool: int) -> int:
    h = _vp()
    _check(_lib.lora_plan_create(pool, C.byref(h)), "lora_plan_create")
    return h.value


def lora_plan_destroy(pool: int, plan: int) -> None:
    _check(_lib.lora_plan_destroy(pool, plan), "lora_plan_destroy")


def lora_plan(pool: int, ids, T: int, plan: int, stream=None) -> None:
    _check(_lib.lora_plan(pool, _ptr(ids), T, plan, _stream(stream)), "lora_plan")


def lora_apply(pool: int, module: int, X, ids, T: int, W, out, plan: Optional[int] = None,
               stream=None) -> None:
    _check(_lib.lora_apply(pool, module, _ptr(X), _ptr(ids), T, _ptr(W), _ptr(out), plan,
                           _stream(stream)), "lora_apply")


def _group_arrays(modules: Sequence[int], W: Sequence, out: Sequence):
    n = len(modules)
    mods = (C.c_int32 * max(n, 1))(*[int(m) for m in modules])
    pw = (_vp * max(n, 1))(*[_ptr(w) for w in W])
    po = (_vp * max(n, 1))(*[_ptr(o) for o in out])
    return n, mods, pw, po


def lora_apply_group(pool: int, modules: Sequence[int], X, ids, T: int, W: Sequence, out: Sequence,
                     plan: Optional[int] = None, stream=None) -> None:
    n, mods, pw, po = _group_arrays(modules, W, out)
    _check(_lib.lora_apply_group(pool, n, mods, _ptr(X), _ptr(ids), T, pw, po, plan, _stream(stream)),
           "lora_apply_group")


def lora_base_apply_group(pool: int, modules: Sequence[int], X, T: int, W: Sequence, out: Sequence,
                          stream=None) -> None:
    n, mods, pw, po = _group_arrays(modules, W, out)
    _check(_lib.lora_base_apply_group(pool, n, mods, _ptr(X), T, pw, po, _stream(stream)),
           "lora_base_apply_group")


def lora_packed_weight_elems(N: int, K: int) -> int:
    n = C.c_int64()
    _check(_lib.lora_packed_weight_elems(N, K, C.byref(n)), "lora_packed_weight_elems")
    return n.value


def lora_pack_weight(W, N: int, K: int, Wp, stream=None) -> None:
    _check(_lib.lora_pack_weight(_ptr(W), N, K, _ptr(Wp), _stream(stream)), "lora_pack_weight")


def lora_apply_group_packed(pool: int, modules: Sequence[int], X, ids, T: int, Wp: Sequence,
                            out: Sequence, stream=None) -> None:
    n, mods, pw, po = _group_arrays(modules, Wp, out)
    _check(_lib.lora_apply_group_packed(pool, n, mods, _ptr(X), _ptr(ids), T, pw, po, _stream(stream)),
           "lora_apply_group_packed")


def lora_base_apply_group_packed(pool: int, modules: Sequence[int], X, T: int, Wp: Sequence,
                                 out: Sequence, stream=None) -> None:
    n, mods, pw, po = _group_arrays(modules, Wp, out)
    _check(_lib.lora_base_apply_group_packed(pool, n, mods, _ptr(X), T, pw, po, _stream(stream)),
           "lora_base_apply_group_packed")


def lora_apply_noalloc(pool: int, module: int, X, ids, T: int, W, out, stream=None) -> None:
    _check(_lib.lora_apply_noalloc(pool, module, _ptr(X), _ptr(ids), T, _ptr(W), _ptr(out), _stream(stream)),
           "lora_apply_noalloc")


def lora_base_apply(pool: int, module: int, X, T: int, W, out, stream=None) -> None:
    _check(_lib.lora_base_apply(pool, module, _ptr(X), T, _ptr(W), _ptr(out), _stream(stream)),
           "lora_base_apply")


def lora_status(pool: int, stream=None) -> str:
    """Synchronises, returns and clears the sticky device status (a name)."""
    code = _lib.lora_status(pool, _stream(stream))
    if code == 8:
        raise LoraError(code, "lora_status")
    return STATUS_NAMES.get(code, f"UNKNOWN({code})")


def lora_debug_read_plan(pool: int, plan: Optional[int], max_tokens: int, stream=None):
    """Returns (perm, inv, seg_id, seg_off) as Python lists."""
    perm = (C.c_int32 * max(max_tokens, 1))()
    inv = (C.c_int32 * max(max_tokens, 1))()
    seg_id = (C.c_int32 * (max_tokens + 1))()
    seg_off = (C.c_int32 * (max_tokens + 2))()
    T, S = C.c_int32(), C.c_int32()
    _check(_lib.lora_debug_read_plan(pool, plan, perm, inv, seg_id, seg_off, C.byref(T),
                                     C.byref(S), _stream(stream)), "lora_debug_read_plan")
    t, s = T.value, S.value
    return list(perm[:t]), list(inv[:t]), list(seg_id[:s]), list(seg_off[:s + 1])


# ---------------------------------------------------------------------------
# host <-> device paging
# ---------------------------------------------------------------------------
def lora_host_cache_create(pool: int, max_cpu_adapters: int) -> None:
    _check(_lib.lora_host_cache_create(pool, max_cpu_adapters), "lora_host_cache_create")


def lora_host_register(pool: int, adapter_id: int, rank: int, alpha: float, A: Sequence,
                       B: Sequence) -> None:
    n = len(A)
    pa = (_vp * max(n, 1))(*[_ptr(a) for a in A])
    pb = (_vp * max(n, 1))(*[_ptr(b) for b in B])
    _check(_lib.lora_host_register(pool, adapter_id, rank, float(alpha), pa, pb),
           "lora_host_register")


def lora_host_unregister(pool: int, adapter_id: int, stream=None) -> None:
    _check(_lib.lora_host_unregister(pool, adapter_id, _stream(stream)), "lora_host_unregister")


def lora_prefetch(pool: int, ids: Sequence[int], stream=None) -> None:
    """``ids``: the batch's adapter ids as a host sequence (list, numpy array)."""
    vals = [int(i) for i in ids]
    arr = (C.c_int32 * max(len(vals), 1))(*vals)
    _check(_lib.lora_prefetch(pool, arr, len(vals), _stream(stream)), "lora_prefetch")


def lora_pin_adapter(pool: int, adapter_id: int, pin: bool, stream=None) -> None:
    _check(_lib.lora_pin_adapter(pool, adapter_id, 1 if pin else 0, _stream(stream)),
           "lora_pin_adapter")


def lora_paging_query(pool: int, adapter_id: int):
    """(where, pinned): where 0 unknown, 1 host cache only, 2 device copy not
    addressable, 3 addressable."""
    w, p = C.c_int32(), C.c_int32()
    _check(_lib.lora_paging_query(pool, adapter_id, C.byref(w), C.byref(p)), "lora_paging_query")
    return w.value, p.value


def lora_paging_stats(pool: int):
    """(prefetch calls, slots copied host -> device, bytes per slot copy)."""
    a, b, c = C.c_int64(), C.c_int64(), C.c_int64()
    _check(_lib.lora_paging_stats(pool, C.byref(a), C.byref(b), C.byref(c)), "lora_paging_stats")
    return a.value, b.value, c.value


# ---------------------------------------------------------------------------
# INT4 base weight
# ---------------------------------------------------------------------------
def lora_q4_pack(q, z, s):
    """Packs host arrays q [N, K] and z [N, K/128] (integers 0..15) and the bf16
    scales s [N, K/128] (a bf16 tensor or uint16 bits) into the device layout;
    returns numpy (Wq uint32 [N, K/8], Wsz uint32 [N, K/128]).  The packing runs
    in the library."""
    import numpy as np
    q = np.ascontiguousarray(q, dtype=np.uint8)
    z = np.ascontiguousarray(z, dtype=np.uint8)
    try:
        import torch
        if isinstance(s, torch.Tensor):
            s = s.detach().cpu().contiguous().view(torch.int16).numpy()
    except ImportError:  # pragma: no cover
        pass
    s = np.ascontiguousarray(np.asarray(s).view(np.uint16))
    N, K = q.shape
    Wq = np.empty((N, K // 8), dtype=np.uint32)
    Wsz = np.empty((N, max(K // 128, 1)), dtype=np.uint32)
    _check(_lib.lora_q4_pack(q.ctypes.data, z.ctypes.data, s.ctypes.data, N, K, Wq.ctypes.data,
                             Wsz.ctypes.data), "lora_q4_pack")
    return Wq, Wsz


def lora_apply_q4(pool: int, module: int, X, ids, T: int, Wq, Wsz, W_scratch, out,
                  plan: Optional[int] = None, stream=None) -> None:
    _check(_lib.lora_apply_q4(pool, module, _ptr(X), _ptr(ids), T, _ptr(Wq), _ptr(Wsz),
                              _ptr(W_scratch), _ptr(out), plan, _stream(stream)), "lora_apply_q4")


def lora_base_apply_q4(pool: int, module: int, X, T: int, Wq, Wsz, W_scratch, out,
                       stream=None) -> None:
    _check(_lib.lora_base_apply_q4(pool, module, _ptr(X), T, _ptr(Wq), _ptr(Wsz), _ptr(W_scratch),
                                   _ptr(out), _stream(stream)), "lora_base_apply_q4")


def lora_apply_group_q4(pool: int, modules: Sequence[int], X, ids, T: int, Wq: Sequence, Wsz: Sequence,
                        W_scratch, out: Sequence, plan: Optional[int] = None, stream=None) -> None:
    n, mods, pq, po = _group_arrays(modules, Wq, out)
    pz = (_vp * max(n, 1))(*[_ptr(z) for z in Wsz])
    _check(_lib.lora_apply_group_q4(pool, n, mods, _ptr(X), _ptr(ids), T, pq, pz, _ptr(W_scratch), po, plan,
                                    _stream(stream)), "lora_apply_group_q4")


def lora_base_apply_group_q4(pool: int, modules: Sequence[int], X, T: int, Wq: Sequence, Wsz: Sequence,
                             W_scratch, out: Sequence, stream=None) -> None:
    n, mods, pq, po = _group_arrays(modules, Wq, out)
    pz = (_vp * max(n, 1))(*[_ptr(z) for z in Wsz])
    _check(_lib.lora_base_apply_group_q4(pool, n, mods, _ptr(X), T, pq, pz, _ptr(W_scratch), po,
                                         _stream(stream)), "lora_base_apply_group_q4")


def lora_load_chain(pool: int, chain_id: int, members: Sequence[int], stream=None) -> None:
    vals = [int(i) for i in members]
    arr = (C.c_int32 * max(len(vals), 1))(*vals)
    _check(_lib.lora_load_chain(pool, chain_id, len(vals), arr, _stream(stream)), "lora_load_chain")
