"""CPU-only checks of the C-ABI library: it loads, exports every entry point
that include/lora.h declares, and rejects bad arguments on the host before
touching the GPU (no compute call is made here)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lora.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:lora_status_t|const char\*)\s+(lora_\w+)\s*\(", src,
                                 flags=re.M)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("lora_pool_create", "lora_pool_destroy", "lora_load_adapter",
              "lora_unload_adapter", "lora_apply", "lora_plan", "lora_base_apply",
              "lora_status", "lora_debug_read_plan", "lora_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol():
    import heterogeneous_rank_gemm_amd as hrg
    lib = C.CDLL(hrg._lora.LIB_PATH)
    for n in _declared():
        assert hasattr(lib, n), n
    assert sorted(hrg.EXPORTED) == _declared()


def test_status_strings():
    import heterogeneous_rank_gemm_amd as hrg
    for code, name in hrg.STATUS_NAMES.items():
        assert hrg.lora_status_string(code) == "LORA_" + ("OK" if name == "OK" else "ERR_" + name)


def _raw():
    import heterogeneous_rank_gemm_amd as hrg
    return hrg._lora._lib


@pytest.mark.parametrize("kw,code", [
    (dict(max_rank=0), 1), (dict(max_rank=65), 1), (dict(max_ids=0), 1),
    (dict(max_ids=16385), 1), (dict(max_adapters=0), 1), (dict(max_tokens=0), 1),
    (dict(d_in=[1020]), 1), (dict(d_out=[4]), 1), (dict(n_modules=0), 1),
    (dict(d_in=[65536], d_out=[16384]), 1),       # a 2 GiB base weight
])
def test_pool_create_rejects_bad_arguments_on_host(kw, code):
    args = dict(max_adapters=4, max_ids=4, max_rank=8, d_in=[64], d_out=[64], max_tokens=64,
                n_modules=None)
    args.update(kw)
    n = len(args["d_in"]) if args["n_modules"] is None else args["n_modules"]
    din = (C.c_int32 * 1)(*args["d_in"])
    dout = (C.c_int32 * 1)(*args["d_out"])
    h = C.c_void_p()
    r = _raw().lora_pool_create(C.byref(h), args["max_adapters"], args["max_ids"],
                                args["max_rank"], n, din, dout, args["max_tokens"], None)
    assert r == code
    assert h.value is None


def test_null_handles_are_rejected():
    lib = _raw()
    assert lib.lora_pool_destroy(None) == 1
    assert lib.lora_apply(None, 0, None, None, 0, None, None, None, None) == 1
    assert lib.lora_base_apply(None, 0, None, 0, None, None, None) == 1
    assert lib.lora_unload_adapter(None, 0, None) == 1
    assert lib.lora_status(None, None) == 1
    assert lib.lora_plan(None, None, 0, None, None) == 1
    h = C.c_void_p()
    assert lib.lora_pool_create(None, 1, 1, 8, 1, None, None, 1, None) == 1
    assert lib.lora_plan_create(None, C.byref(h)) == 1


def test_package_fails_loudly_without_library(tmp_path, monkeypatch):
    # the binding refuses to import from a tree without the built library
    import importlib.util
    src = os.path.join(ROOT, "heterogeneous_rank_gemm_amd", "_lora.py")
    pkg = tmp_path / "pkg"
    pkg.mkdir()
    (pkg / "_lora.py").write_text(open(src).read())
    spec = importlib.util.spec_from_file_location("lonely_lora", pkg / "_lora.py")
    mod = importlib.util.module_from_spec(spec)
    with pytest.raises(ImportError):
        spec.loader.exec_module(mod)


def test_q4_pack_layout():
    """The host-side INT4 packer (no GPU call) writes the layout lora.h
    documents: word 16 g + 4 j + st of a row holds k = 128 g + 32 st + 8 j + e
    in nibble e; the group word is the bf16 scale bits | zero point << 16."""
    import numpy as np
    import heterogeneous_rank_gemm_amd as hrg
    g = np.random.default_rng(0)
    N, K = 3, 384
    q = g.integers(0, 16, (N, K))
    z = g.integers(0, 16, (N, K // 128))
    s = g.integers(0, 65535, (N, K // 128)).astype(np.uint16)
    Wq, Wsz = hrg.lora_q4_pack(q, z, s)
    for n in range(N):
        for k in range(K):
            gg, st, j, e = k // 128, (k % 128) // 32, (k % 32) // 8, k % 8
            assert (int(Wq[n, 16 * gg + 4 * j + st]) >> (4 * e)) & 15 == q[n, k]
        for gg in range(K // 128):
            assert int(Wsz[n, gg]) == int(s[n, gg]) | (int(z[n, gg]) << 16)
    with pytest.raises(hrg.LoraError):
        hrg.lora_q4_pack(np.full((1, 128), 16), np.zeros((1, 1)), np.zeros((1, 1), np.uint16))
    with pytest.raises(hrg.LoraError):
        hrg.lora_q4_pack(np.zeros((1, 200)), np.zeros((1, 1)), np.zeros((1, 1), np.uint16))


def test_wrapper_rejects_bad_tensors_before_the_library():
    """The Python wrapper checks dtype, layout, shape and device before it
    passes raw addresses on (an int64 id tensor or a transposed view would
    otherwise be read as something else)."""
    import torch
    from heterogeneous_rank_gemm_amd import LoraError
    from heterogeneous_rank_gemm_amd.pool import check_tensor
    good = torch.zeros((8, 64), dtype=torch.bfloat16)
    check_tensor(good, "X", torch.bfloat16, 64, 8, "t", need_cuda=False)
    cases = [
        (torch.zeros((8, 64), dtype=torch.float32), torch.bfloat16, 64, 8),   # dtype
        (torch.zeros((64, 8), dtype=torch.bfloat16).t(), torch.bfloat16, 64, 8),  # not contiguous
        (torch.zeros((4, 64), dtype=torch.bfloat16), torch.bfloat16, 64, 8),   # too few rows
        (torch.zeros((8, 32), dtype=torch.bfloat16), torch.bfloat16, 64, 8),   # wrong width
        (torch.zeros(8, dtype=torch.int64), torch.int32, None, 8),            # int64 ids
        (torch.zeros((8, 1), dtype=torch.int32), torch.int32, None, 8),       # ids not 1-D
    ]
    for t, dt, cols, rows in cases:
        with pytest.raises(LoraError) as e:
            check_tensor(t, "x", dt, cols, rows, "t", need_cuda=False)
        assert e.value.status == "INVALID_ARG"
    with pytest.raises(LoraError) as e:                                       # host tensor
        check_tensor(good, "X", torch.bfloat16, 64, 8, "t")
    assert e.value.status == "INVALID_ARG"
