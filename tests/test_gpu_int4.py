"""GPU tests of the INT4 base weight ([vLLM-ch7] performance notes: an
AWQ-INT4 base with bf16 adapters) through the C ABI.

The oracle dequantizes the same (q, z, s) to W = bf16((q - z) s) and applies
the definition; the library dequantizes in the decode kernel's registers (T
<= 64) or into a scratch weight before the batched GEMM.  Because the
dequantized weights are the same bf16 values and the GEMMs keep the bf16
path's K order, the INT4 calls must also equal the bf16 calls on the
oracle's dequantized weight bit for bit."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _q4(N, K, seed):
    g = np.random.default_rng(seed)
    q = g.integers(0, 16, (N, K))
    z = g.integers(4, 12, (N, K // 128))
    s = torch.as_tensor(np.abs(g.normal(0.0045, 0.001, (N, K // 128))).astype(np.float32)).to(torch.bfloat16)
    return q, z, s


@pytest.mark.parametrize("T,K,N", [(1, 1024, 200), (17, 640, 1032), (64, 4096, 4096), (40, 11008, 512),
                                   (130, 1024, 520), (300, 4224, 264)])
def test_int4_base_parity(T, K, N):
    import heterogeneous_rank_gemm_amd as hrg
    from heterogeneous_rank_gemm_amd import LoraPool
    seed = T * 7 + K + N
    q, z, s = _q4(N, K, seed)
    Wq, Wsz = hrg.lora_q4_pack(q, z, s)
    Wq_d = torch.as_tensor(Wq.view(np.int32)).cuda()
    Wsz_d = torch.as_tensor(Wsz.view(np.int32)).cuda()
    Wdeq = oracle.dequant_q4(q, z, s)                          # float64 holding bf16 values
    Wdeq_bf = torch.as_tensor(Wdeq.astype(np.float32)).to(torch.bfloat16)
    assert np.array_equal(Wdeq_bf.double().numpy(), Wdeq)
    ranks = [8, 16, 16, 12]
    pool = LoraPool(4, 4, 16, [K], [N], T)
    reg = oracle.Registry(4, 4, 16, [K], [N], T)
    gen = torch.Generator().manual_seed(seed)
    for i, r in enumerate(ranks):
        A = (torch.randn((K, r), generator=gen) * 0.02).to(torch.bfloat16)
        B = (torch.randn((r, N), generator=gen) * 0.02).to(torch.bfloat16)
        pool.load_adapter(i, r, 2.0 * r, [A.cuda()], [B.cuda()])
        reg.load(i, r, 2.0 * r, [A], [B])
    ids_np = np.random.default_rng(seed).integers(-1, 4, T).astype(np.int32)
    ids = torch.as_tensor(ids_np, device="cuda")
    X = torch.randn((T, K), generator=gen).to(torch.bfloat16)
    Xd = X.cuda()
    scratch = torch.empty((N, K), dtype=torch.bfloat16, device="cuda") if T > 64 else None
    out = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    base = torch.empty_like(out)
    out_bf = torch.empty_like(out)
    base_bf = torch.empty_like(out)
    pool.apply_q4(0, Xd, ids, Wq_d, Wsz_d, out, W_scratch=scratch)
    pool.base_apply_q4(0, Xd, Wq_d, Wsz_d, base, W_scratch=scratch)
    Wd = Wdeq_bf.cuda()
    pool.apply(0, Xd, ids, Wd, out_bf)
    pool.base_apply(0, Xd, Wd, base_bf)
    torch.cuda.synchronize()
    assert pool.status() == "OK"
    ref = oracle.lora_linear(reg, 0, X, ids_np, Wdeq)
    mx, rl1, _ = oracle.parity_metrics(out.cpu(), ref)
    assert mx <= oracle.MAX_REL_TOL and rl1 <= oracle.RELL1_TOL, (mx, rl1)
    bref = oracle.base_linear(X, Wdeq)
    mx, rl1, _ = oracle.parity_metrics(base.cpu(), bref)
    assert mx <= oracle.MAX_REL_TOL and rl1 <= oracle.RELL1_TOL, (mx, rl1)
    m = torch.as_tensor(ids_np < 0, device="cuda")
    assert torch.equal(out[m], base[m])                       # id -1 rows: base only, bit for bit
    assert torch.equal(out, out_bf) and torch.equal(base, base_bf)
    pool.close()


def test_int4_argument_errors():
    import heterogeneous_rank_gemm_amd as hrg
    from heterogeneous_rank_gemm_amd import LoraError, LoraPool
    q, z, s = _q4(64, 256, 1)
    Wq, Wsz = hrg.lora_q4_pack(q, z, s)
    Wq_d = torch.as_tensor(Wq.view(np.int32)).cuda()
    Wsz_d = torch.as_tensor(Wsz.view(np.int32)).cuda()
    X = torch.zeros((100, 256), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((100, 64), dtype=torch.bfloat16, device="cuda")
    pool = LoraPool(2, 2, 8, [256, 200], [64, 64], 128)
    with pytest.raises(LoraError) as e:                       # T > 64 needs the scratch weight
        pool.base_apply_q4(0, X, Wq_d, Wsz_d, out)
    assert e.value.status == "INVALID_ARG"
    with pytest.raises(LoraError) as e:                       # d_in not a multiple of 128
        pool.base_apply_q4(1, X[:8, :200].contiguous(), Wq_d, Wsz_d, out[:8])
    assert e.value.status == "INVALID_ARG"
    pool.close()


@pytest.mark.parametrize("T,K", [(64, 4096), (17, 2048), (130, 1024)])
def test_int4_group_equals_single_linears(T, K):
    """lora_apply_group_q4 / lora_base_apply_group_q4 over linears that read
    one X: each output equals the INT4 call on that linear alone and the
    bf16 group call on the dequantized weights, bit for bit, and meets the
    oracle's bar."""
    import heterogeneous_rank_gemm_amd as hrg
    from heterogeneous_rank_gemm_amd import LoraPool
    # (at K = 4096 and 64 tokens the bf16 group is large enough for blocks of
    # two K chunks, the INT4 one always takes one: the sums must still agree)
    d_outs = [4104, 264, 4096]
    n = len(d_outs)
    seed = T + K
    pool = LoraPool(6, 6, 16, [K] * n, d_outs, T)
    reg = oracle.Registry(6, 6, 16, [K] * n, d_outs, T)
    gen = torch.Generator().manual_seed(seed)
    for i, r in enumerate([16, 8, 5, 16, 12, 1]):
        A = [(torch.randn((K, r), generator=gen) * 0.02).to(torch.bfloat16) for _ in d_outs]
        B = [(torch.randn((r, d), generator=gen) * 0.02).to(torch.bfloat16) for d in d_outs]
        pool.load_adapter(i, r, 2.0 * r, [a.cuda() for a in A], [b.cuda() for b in B])
        reg.load(i, r, 2.0 * r, A, B)
    Wq, Wsz, Wdeq = [], [], []
    for m, d in enumerate(d_outs):
        q, z, s = _q4(d, K, seed + m)
        a, b = hrg.lora_q4_pack(q, z, s)
        Wq.append(torch.as_tensor(a.view(np.int32)).cuda())
        Wsz.append(torch.as_tensor(b.view(np.int32)).cuda())
        Wdeq.append(oracle.dequant_q4(q, z, s))
    Wbf = [torch.as_tensor(w.astype(np.float32)).to(torch.bfloat16).cuda() for w in Wdeq]
    ids_np = np.random.default_rng(seed).integers(-1, 6, T).astype(np.int32)
    ids = torch.as_tensor(ids_np, device="cuda")
    X = torch.randn((T, K), generator=gen).to(torch.bfloat16)
    Xd = X.cuda()
    scratch = torch.empty(max(d_outs) * K, dtype=torch.bfloat16, device="cuda") if T > 64 else None
    mods = list(range(n))

    def outs():
        return [torch.empty((T, d), dtype=torch.bfloat16, device="cuda") for d in d_outs]
    g, gb, bf, bfb = outs(), outs(), outs(), outs()
    pool.apply_group_q4(mods, Xd, ids, Wq, Wsz, g, W_scratch=scratch)
    pool.base_apply_group_q4(mods, Xd, Wq, Wsz, gb, W_scratch=scratch)
    pool.apply_group(mods, Xd, ids, Wbf, bf)
    pool.base_apply_group(mods, Xd, Wbf, bfb)
    torch.cuda.synchronize()
    assert pool.status() == "OK"
    for m in mods:
        one = torch.empty((T, d_outs[m]), dtype=torch.bfloat16, device="cuda")
        oneb = torch.empty_like(one)
        pool.apply_q4(m, Xd, ids, Wq[m], Wsz[m], one, W_scratch=scratch)
        pool.base_apply_q4(m, Xd, Wq[m], Wsz[m], oneb, W_scratch=scratch)
        torch.cuda.synchronize()
        assert torch.equal(g[m], one), f"linear {m}: INT4 group differs from lora_apply_q4"
        assert torch.equal(gb[m], oneb), f"linear {m}: INT4 base group differs from lora_base_apply_q4"
        assert torch.equal(g[m], bf[m]) and torch.equal(gb[m], bfb[m]), f"linear {m}: INT4 differs from bf16"
        ref = oracle.lora_linear(reg, m, X, ids_np, Wdeq[m])
        mx, rl1, _ = oracle.parity_metrics(g[m].cpu(), ref)
        assert mx <= oracle.MAX_REL_TOL and rl1 <= oracle.RELL1_TOL, (m, mx, rl1)
    pool.close()


N_RANDOM = int(__import__("os").environ.get("HRG_INT4_RANDOM_CASES", 12))


@pytest.mark.parametrize("k", range(N_RANDOM))
def test_int4_random_shapes(k):
    """Seeded random shapes on both paths (K any multiple of 128, N any
    multiple of 8, pool ranks up to 64, zero points over 0..15): the oracle's
    values, the bf16 call's bits on the dequantized weight, id -1 rows equal
    to the base-only call.  HRG_INT4_RANDOM_CASES scales the count (300
    cases have passed)."""
    import heterogeneous_rank_gemm_amd as hrg
    from heterogeneous_rank_gemm_amd import LoraPool
    g = np.random.default_rng(660000 + k)
    T = int(g.choice([int(g.integers(1, 65)), int(g.integers(65, 1200))]))
    K, N = int(128 * g.integers(1, 40)), int(8 * g.integers(1, 700))
    max_rank, n = int(g.choice([4, 16, 32, 64])), int(g.integers(1, 8))
    ranks = [int(g.integers(1, max_rank + 1)) for _ in range(n)]
    print(f"[int4 random {k}] T={T} K={K} N={N} max_rank={max_rank} ranks={ranks}", flush=True)
    q, z = g.integers(0, 16, (N, K)), g.integers(0, 16, (N, K // 128))
    s = torch.as_tensor(np.abs(g.normal(0.0045, 0.002, (N, K // 128))).astype(np.float32)).to(torch.bfloat16)
    Wq, Wsz = hrg.lora_q4_pack(q, z, s)
    Wq_d, Wsz_d = torch.as_tensor(Wq.view(np.int32)).cuda(), torch.as_tensor(Wsz.view(np.int32)).cuda()
    Wdeq = oracle.dequant_q4(q, z, s)
    Wdeq_bf = torch.as_tensor(Wdeq.astype(np.float32)).to(torch.bfloat16)
    pool, reg = LoraPool(n, n, max_rank, [K], [N], T), oracle.Registry(n, n, max_rank, [K], [N], T)
    gen = torch.Generator().manual_seed(k)
    for i, r in enumerate(ranks):
        A = (torch.randn((K, r), generator=gen) * 0.02).to(torch.bfloat16)
        B = (torch.randn((r, N), generator=gen) * 0.02).to(torch.bfloat16)
        pool.load_adapter(i, r, 2.0 * r, [A.cuda()], [B.cuda()])
        reg.load(i, r, 2.0 * r, [A], [B])
    ids_np = g.integers(-1, n, T).astype(np.int32)
    ids = torch.as_tensor(ids_np, device="cuda")
    X = torch.randn((T, K), generator=gen).to(torch.bfloat16)
    Xd = X.cuda()
    scratch = torch.empty((N, K), dtype=torch.bfloat16, device="cuda") if T > 64 else None
    out = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    out_bf, base = torch.empty_like(out), torch.empty_like(out)
    pool.apply_q4(0, Xd, ids, Wq_d, Wsz_d, out, W_scratch=scratch)
    pool.base_apply_q4(0, Xd, Wq_d, Wsz_d, base, W_scratch=scratch)
    pool.apply(0, Xd, ids, Wdeq_bf.cuda(), out_bf)
    torch.cuda.synchronize()
    assert pool.status() == "OK"
    mx, rl1, _ = oracle.parity_metrics(out.cpu(), oracle.lora_linear(reg, 0, X, ids_np, Wdeq))
    assert mx <= oracle.MAX_REL_TOL and rl1 <= oracle.RELL1_TOL, (mx, rl1)
    assert torch.equal(out, out_bf)
    m = torch.as_tensor(ids_np < 0, device="cuda")
    assert torch.equal(out[m], base[m])
    pool.close()
