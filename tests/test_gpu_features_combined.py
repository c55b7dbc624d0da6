"""One pool exercising the features together through the C ABI: adapters
loaded directly and paged in from the host cache, untargeted modules,
a chain over a paged and a direct adapter, and an INT4 base weight, in
decode and batched batches; against the oracle on the same bf16 bits
(its registry holds the addressable adapters and the chain)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402

SHAPES = [(256, 520), (640, 264)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _ab(i, r, targets, gen):
    A = [(torch.randn((d_in, r), generator=gen) * 0.02).to(torch.bfloat16) if m in targets else None
         for m, (d_in, _) in enumerate(SHAPES)]
    B = [(torch.randn((r, d_out), generator=gen) * 0.02).to(torch.bfloat16) if m in targets else None
         for m, (_, d_out) in enumerate(SHAPES)]
    return A, B


@pytest.mark.parametrize("T", [48, 200])
def test_paging_chains_target_sets_and_int4_together(T):
    import heterogeneous_rank_gemm_amd as hrg
    from heterogeneous_rank_gemm_amd import LoraPool
    gen = torch.Generator().manual_seed(T)
    pool = LoraPool(8, 24, 32, [s[0] for s in SHAPES], [s[1] for s in SHAPES], T)
    pool.host_cache_create(8)
    reg = oracle.Registry(24, 24, 32, [s[0] for s in SHAPES], [s[1] for s in SHAPES], T)
    # direct loads 0, 1 (1 skips module 1); host-cached 10..13 (12 skips module 0)
    for i, r, tg in [(0, 16, (0, 1)), (1, 8, (0,))]:
        A, B = _ab(i, r, tg, gen)
        pool.load_adapter(i, r, 2.0 * r, [a.cuda() if a is not None else None for a in A],
                          [b.cuda() if b is not None else None for b in B])
        reg.load(i, r, 2.0 * r, A, B)
    for i, r, tg in [(10, 16, (0, 1)), (11, 12, (0, 1)), (12, 16, (1,)), (13, 4, (0, 1))]:
        A, B = _ab(i, r, tg, gen)
        pool.host_register(i, r, 24.0, A, B)
        reg.load(i, r, 24.0, A, B)
    ids_np = np.random.default_rng(T).choice([-1, 0, 1, 10, 11, 12, 13, 20], size=T).astype(np.int32)
    named = [10, 11, 12, 13]
    pool.prefetch(named)
    pool.load_chain(20, [10, 1])                      # a paged and a direct member
    reg.load_chain(20, [10, 1])
    ids = torch.as_tensor(ids_np, device="cuda")
    for m, (d_in, d_out) in enumerate(SHAPES):
        g = np.random.default_rng(100 + m)
        q = g.integers(0, 16, (d_out, d_in))
        z = g.integers(4, 12, (d_out, d_in // 128))
        s = torch.as_tensor(np.abs(g.normal(0.0045, 0.001, (d_out, d_in // 128))).astype(np.float32)
                            ).to(torch.bfloat16)
        Wq, Wsz = hrg.lora_q4_pack(q, z, s)
        Wdeq = oracle.dequant_q4(q, z, s)
        X = torch.randn((T, d_in), generator=gen).to(torch.bfloat16)
        out = torch.empty((T, d_out), dtype=torch.bfloat16, device="cuda")
        base = torch.empty_like(out)
        scratch = torch.empty((d_out, d_in), dtype=torch.bfloat16, device="cuda") if T > 64 else None
        Wq_d = torch.as_tensor(Wq.view(np.int32)).cuda()
        Wsz_d = torch.as_tensor(Wsz.view(np.int32)).cuda()
        pool.apply_q4(m, X.cuda(), ids, Wq_d, Wsz_d, out, W_scratch=scratch)
        pool.base_apply_q4(m, X.cuda(), Wq_d, Wsz_d, base, W_scratch=scratch)
        torch.cuda.synchronize()
        assert pool.status() == "OK"
        ref = oracle.lora_linear(reg, m, X, ids_np, Wdeq)
        mx, rl1, _ = oracle.parity_metrics(out.cpu(), ref)
        assert mx <= oracle.MAX_REL_TOL and rl1 <= oracle.RELL1_TOL, (m, mx, rl1)
        skip = {0: [-1, 12], 1: [-1, 1]}[m]           # base only on this module
        mask = torch.as_tensor(np.isin(ids_np, skip), device="cuda")
        assert torch.equal(out[mask], base[mask])
    pool.close()
