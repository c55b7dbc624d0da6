"""GPU test of lora_apply_noalloc, the decode entry point whose scratch is a
fixed device array inside the library (for callers that cannot allocate):
its outputs must equal lora_apply's bit for bit, on calls in a row that
reuse the array with shrinking and growing inputs, and it must refuse sizes
beyond the array with INVALID_ARG."""
from __future__ import annotations

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402

SHAPES = [(4096, 4096), (1032, 520), (11008, 4096), (16384, 16384)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _pool():
    from heterogeneous_rank_gemm_amd import LoraPool
    pool = LoraPool(6, 8, 32, [s[0] for s in SHAPES], [s[1] for s in SHAPES], 64)
    reg = oracle.Registry(6, 8, 32, [s[0] for s in SHAPES[:3]], [s[1] for s in SHAPES[:3]], 64)
    gen = torch.Generator().manual_seed(5)
    for i, r in enumerate([16, 8, 32, 5, 16]):
        A = [(torch.randn((d_in, r), generator=gen) * 0.02).to(torch.bfloat16) for d_in, _ in SHAPES]
        B = [(torch.randn((r, d_out), generator=gen) * 0.02).to(torch.bfloat16) for _, d_out in SHAPES]
        pool.load_adapter(i, r, 2.0 * r, [a.cuda() for a in A], [b.cuda() for b in B])
        reg.load(i, r, 2.0 * r, A[:3], B[:3])
    return pool, reg, gen


def test_noalloc_equals_lora_apply():
    from heterogeneous_rank_gemm_amd import lora_apply, lora_apply_noalloc
    pool, reg, gen = _pool()
    # two calls in a row, the second smaller, then larger ones again
    for m, T in ((0, 64), (1, 17), (2, 64), (0, 9), (1, 64)):
        d_in, d_out = SHAPES[m]
        X = torch.randn((T, d_in), generator=gen).to(torch.bfloat16)
        W = (torch.randn((d_out, d_in), generator=gen) * 0.02).to(torch.bfloat16)
        ids_np = np.random.default_rng(10 * m + T).integers(-1, 5, size=T).astype(np.int32)
        Xd, Wd, ids = X.cuda(), W.cuda(), torch.as_tensor(ids_np, device="cuda")
        ref = torch.full((T, d_out), 5.0, dtype=torch.bfloat16, device="cuda")
        got = torch.full((T, d_out), -5.0, dtype=torch.bfloat16, device="cuda")
        lora_apply(pool.handle, m, Xd, ids, T, Wd, ref, None)
        lora_apply_noalloc(pool.handle, m, Xd, ids, T, Wd, got)
        torch.cuda.synchronize()
        assert pool.status() == "OK"
        assert torch.equal(got, ref), (m, T)
        mx, rl1, _ = oracle.parity_metrics(got.cpu(), oracle.lora_linear(reg, m, X, ids_np, W))
        assert mx <= oracle.MAX_REL_TOL and rl1 <= oracle.RELL1_TOL, (m, T, mx, rl1)
    pool.close()


def test_noalloc_refuses_what_does_not_fit():
    from heterogeneous_rank_gemm_amd import LoraError, lora_apply_noalloc
    pool, _, _ = _pool()
    x = torch.zeros((64, 16384), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((8, 8), dtype=torch.bfloat16, device="cuda")     # never read: refused on the host
    ids = torch.zeros(100, dtype=torch.int32, device="cuda")
    out = torch.zeros((100, 16384), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(LoraError) as e:                                # 16 x 64 x 16384 floats > 4 Mi
        lora_apply_noalloc(pool.handle, 3, x, ids, 64, w, out)
    assert e.value.status == "INVALID_ARG"
    with pytest.raises(LoraError) as e:                                # T > 64
        lora_apply_noalloc(pool.handle, 1, torch.zeros((100, 1032), dtype=torch.bfloat16, device="cuda"),
                           ids, 100, w, out)
    assert e.value.status == "INVALID_ARG"
    torch.cuda.synchronize()
    pool.close()
