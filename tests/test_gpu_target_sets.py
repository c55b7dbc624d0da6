"""GPU tests of per-adapter target sets through the C ABI.

An adapter loaded without pages for a module does not target it: its tokens
take the skip path there ([vLLM-ch7] performance notes: adapters of one batch
with different target_modules send some sequences down a skip path; [icman]
section 2.1: the branch is added on the target linears only).  Checked
against the oracle on the same bf16 bits, and rows of untargeted modules
against lora_base_apply bit for bit."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402

SHAPES = [(264, 520), (520, 264), (264, 200)]
# adapter -> targeted modules
TARGETS = {0: (0, 1, 2), 1: (0, 2), 2: (1,), 3: (2,), 4: (0, 1), 5: (1, 2), 6: (0,), 7: (0, 1, 2)}
RANKS = {0: 8, 1: 16, 2: 13, 3: 4, 4: 16, 5: 8, 6: 12, 7: 16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _weights(i, seed):
    g = torch.Generator()
    g.manual_seed(7919 * seed + i)
    r = RANKS[i]
    A = [(torch.randn((d_in, r), generator=g) * 0.02).to(torch.bfloat16) if m in TARGETS[i] else None
         for m, (d_in, _) in enumerate(SHAPES)]
    B = [(torch.randn((r, d_out), generator=g) * 0.02).to(torch.bfloat16) if m in TARGETS[i] else None
         for m, (_, d_out) in enumerate(SHAPES)]
    return A, B


@pytest.mark.parametrize("T,max_adapters,max_ids,paged", [
    (40, 8, 8, False), (40, 8, 12, False), (40, 4, 12, True), (130, 8, 12, False),
    (130, 8, 8, False), (130, 5, 12, True), (64, 16, 8, False)])
def test_target_sets_match_oracle_and_base(T, max_adapters, max_ids, paged):
    """Direct-mapped (max_ids <= max_adapters) and slot-table pools, loaded
    directly or paged in from the host cache; decode (T <= 64) and batched."""
    from heterogeneous_rank_gemm_amd import LoraPool
    seed = T + max_adapters + max_ids
    pool = LoraPool(max_adapters, max_ids, 16, [s[0] for s in SHAPES], [s[1] for s in SHAPES], T)
    reg = oracle.Registry(max_ids, max_ids, 16, [s[0] for s in SHAPES], [s[1] for s in SHAPES], T)
    g = np.random.default_rng(seed)
    if paged:
        pool.host_cache_create(8)
    for i in range(8):
        A, B = _weights(i, seed)
        alpha = 2.0 * RANKS[i] if i != 4 else 24.0
        if paged:
            pool.host_register(i, RANKS[i], alpha, A, B)
        else:
            pool.load_adapter(i, RANKS[i], alpha, [a.cuda() if a is not None else None for a in A],
                              [b.cuda() if b is not None else None for b in B])
        reg.load(i, RANKS[i], alpha, A, B)
    n_used = max_adapters if paged else 8
    used = [int(x) for x in g.choice(8, size=n_used, replace=False)]
    ids_np = g.choice(used + [-1], size=T).astype(np.int32)
    if paged:
        pool.prefetch(ids_np.tolist())
    ids = torch.as_tensor(ids_np, device="cuda")
    for m, (d_in, d_out) in enumerate(SHAPES):
        X = (torch.randn((T, d_in), generator=torch.Generator().manual_seed(seed + m))).to(torch.bfloat16)
        W = (torch.randn((d_out, d_in), generator=torch.Generator().manual_seed(seed + 10 + m)) * 0.02
             ).to(torch.bfloat16)
        Xd, Wd = X.cuda(), W.cuda()
        out = torch.empty((T, d_out), dtype=torch.bfloat16, device="cuda")
        base = torch.empty_like(out)
        pool.apply(m, Xd, ids, Wd, out)
        pool.base_apply(m, Xd, Wd, base)
        torch.cuda.synchronize()
        assert pool.status() == "OK"
        ref = oracle.lora_linear(reg, m, X, ids_np, W)
        mx, rl1, _ = oracle.parity_metrics(out.cpu(), ref)
        assert mx <= oracle.MAX_REL_TOL and rl1 <= oracle.RELL1_TOL, (m, mx, rl1)
        skip = np.array([i < 0 or m not in TARGETS[int(i)] for i in ids_np])
        assert skip.any()
        mask = torch.as_tensor(skip, device="cuda")
        assert torch.equal(out[mask], base[mask]), f"module {m}: skipped rows differ from base"
        if (~skip).any():
            assert not torch.equal(out[~mask], base[~mask])
    pool.close()


def test_target_set_argument_errors():
    from heterogeneous_rank_gemm_amd import LoraError, LoraPool
    pool = LoraPool(4, 4, 16, [s[0] for s in SHAPES], [s[1] for s in SHAPES], 16)
    A, B = _weights(1, 0)
    A = [a.cuda() if a is not None else None for a in A]
    B = [b.cuda() if b is not None else None for b in B]
    with pytest.raises(LoraError) as e:                      # A without B
        pool.load_adapter(0, RANKS[1], 32.0, A, [B[0], None, None])
    assert e.value.status == "INVALID_ARG"
    with pytest.raises(LoraError) as e:                      # targets nothing
        pool.load_adapter(0, RANKS[1], 32.0, [None] * 3, [None] * 3)
    assert e.value.status == "INVALID_ARG"
    pool.load_adapter(0, RANKS[1], 32.0, A, B)
    pool.close()


@pytest.mark.parametrize("k", range(int(__import__("os").environ.get("HRG_TARGET_RANDOM_CASES", 8))))
def test_random_target_sets(k):
    """Seeded random pools of 2 to 4 linears of one d_in (direct-mapped), each
    adapter targeting a random non-empty subset, both paths: the oracle's
    values, and rows whose adapter skips a linear equal to lora_base_apply
    there bit for bit.  HRG_TARGET_RANDOM_CASES scales the count (200 have
    passed)."""
    from heterogeneous_rank_gemm_amd import LoraPool
    g = np.random.default_rng(730000 + k)
    T = int(g.choice([int(g.integers(1, 65)), int(g.integers(65, 600))]))
    K, nl = int(8 * g.integers(2, 200)), int(g.integers(2, 5))
    d_outs = [int(8 * g.integers(2, 300)) for _ in range(nl)]
    max_rank, n = int(g.choice([8, 16, 32])), int(g.integers(2, 10))
    ranks = [int(g.integers(1, max_rank + 1)) for _ in range(n)]
    targets = []
    for _ in range(n):
        t = [m for m in range(nl) if g.random() < 0.6]
        targets.append(t or [int(g.integers(0, nl))])
    print(f"[targets random {k}] T={T} K={K} d_outs={d_outs} ranks={ranks} targets={targets}", flush=True)
    pool = LoraPool(n, n, max_rank, [K] * nl, d_outs, T)
    reg = oracle.Registry(n, n, max_rank, [K] * nl, d_outs, T)
    gen = torch.Generator().manual_seed(k)
    for i, r in enumerate(ranks):
        A = [(torch.randn((K, r), generator=gen) * 0.02).to(torch.bfloat16) if m in targets[i] else None
             for m in range(nl)]
        B = [(torch.randn((r, d_outs[m]), generator=gen) * 0.02).to(torch.bfloat16) if m in targets[i] else None
             for m in range(nl)]
        pool.load_adapter(i, r, 2.0 * r, [a.cuda() if a is not None else None for a in A],
                          [b.cuda() if b is not None else None for b in B])
        reg.load(i, r, 2.0 * r, A, B)
    ids_np = g.integers(-1, n, T).astype(np.int32)
    ids = torch.as_tensor(ids_np, device="cuda")
    X = torch.randn((T, K), generator=gen).to(torch.bfloat16)
    Xd = X.cuda()
    for m in range(nl):
        W = (torch.randn((d_outs[m], K), generator=gen) * 0.02).to(torch.bfloat16)
        out = torch.empty((T, d_outs[m]), dtype=torch.bfloat16, device="cuda")
        base = torch.empty_like(out)
        pool.apply(m, Xd, ids, W.cuda(), out)
        pool.base_apply(m, Xd, W.cuda(), base)
        torch.cuda.synchronize()
        assert pool.status() == "OK"
        mx, rl1, _ = oracle.parity_metrics(out.cpu(), oracle.lora_linear(reg, m, X, ids_np, W))
        assert mx <= oracle.MAX_REL_TOL and rl1 <= oracle.RELL1_TOL, (m, mx, rl1)
        skip = np.array([i < 0 or m not in targets[i] for i in ids_np])
        keep = torch.as_tensor(skip, device="cuda")
        assert torch.equal(out[keep], base[keep]), f"linear {m}: skipped rows differ from base-only"
    pool.close()
