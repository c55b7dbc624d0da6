"""GPU tests of adapter chains through the C ABI ([LoRA-Land] "technical
approach", item 3, and "3. hot-plug API and composition":
set_adaptive_chain).  A chain id adds every member's update; the oracle
computes the member terms one adapter at a time on the same bf16 bits."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from oracle import OracleError  # noqa: E402

SHAPES = [(264, 520), (520, 264)]
RANKS = [8, 16, 5, 13, 16, 4]
ALPHAS = [16.0, 24.0, 10.0, 26.0, 32.0, 6.0]
CHAINS = {10: [0, 1], 11: [2, 3, 5], 12: [4], 13: [1, 0]}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _setup(max_adapters, max_ids, T, seed):
    from heterogeneous_rank_gemm_amd import LoraPool
    pool = LoraPool(max_adapters, max_ids, 48, [s[0] for s in SHAPES], [s[1] for s in SHAPES], T)
    reg = oracle.Registry(max_adapters, max_ids, 48, [s[0] for s in SHAPES], [s[1] for s in SHAPES], T)
    gen = torch.Generator().manual_seed(seed)
    for i, (r, al) in enumerate(zip(RANKS, ALPHAS)):
        A = [(torch.randn((d_in, r), generator=gen) * 0.02).to(torch.bfloat16) for d_in, _ in SHAPES]
        B = [(torch.randn((r, d_out), generator=gen) * 0.02).to(torch.bfloat16) for _, d_out in SHAPES]
        if i == 5:            # adapter 5 does not target module 1
            A[1] = B[1] = None
        pool.load_adapter(i, r, al, [a.cuda() if a is not None else None for a in A],
                          [b.cuda() if b is not None else None for b in B])
        reg.load(i, r, al, A, B)
    for c, members in CHAINS.items():
        pool.load_chain(c, members)
        reg.load_chain(c, members)
    return pool, reg, gen


def _run(pool, gen, T, ids_np, m):
    d_in, d_out = SHAPES[m]
    X = torch.randn((T, d_in), generator=gen).to(torch.bfloat16)
    W = (torch.randn((d_out, d_in), generator=gen) * 0.02).to(torch.bfloat16)
    out = torch.empty((T, d_out), dtype=torch.bfloat16, device="cuda")
    pool.apply(m, X.cuda(), torch.as_tensor(ids_np, device="cuda"), W.cuda(), out)
    return X, W, out


@pytest.mark.parametrize("T,max_adapters,max_ids", [(40, 16, 16), (64, 16, 20), (130, 16, 16),
                                                    (300, 16, 20)])
def test_chains_match_oracle(T, max_adapters, max_ids):
    seed = T + max_ids
    pool, reg, gen = _setup(max_adapters, max_ids, T, seed)
    g = np.random.default_rng(seed)
    choices = [-1, 0, 1, 2, 3, 4, 5, 10, 11, 12, 13]
    ids_np = g.choice(choices, size=T).astype(np.int32)
    if T >= 130:   # a long chain segment too, so the GEMM walks chain segments
        ids_np[:40] = 11
    outs = {}
    for m in range(len(SHAPES)):
        X, W, out = _run(pool, gen, T, ids_np, m)
        torch.cuda.synchronize()
        assert pool.status() == "OK"
        ref = oracle.lora_linear(reg, m, X, ids_np, W)
        mx, rl1, _ = oracle.parity_metrics(out.cpu(), ref)
        assert mx <= oracle.MAX_REL_TOL and rl1 <= oracle.RELL1_TOL, (m, mx, rl1)
        outs[m] = (X, W, out.clone())
    # chains are snapshots: unloading members changes nothing
    for i in (0, 1, 3):
        pool.unload_adapter(i)
        reg.unload(i)
    ids2 = np.where(np.isin(ids_np, [0, 1, 3]), -1, ids_np).astype(np.int32)
    for m, (X, W, out) in outs.items():
        out2 = torch.empty_like(out)
        pool.apply(m, X.cuda(), torch.as_tensor(ids2, device="cuda"), W.cuda(), out2)
        torch.cuda.synchronize()
        assert pool.status() == "OK"
        keep = torch.as_tensor(ids2 == ids_np, device="cuda")
        assert torch.equal(out2[keep], out[keep])
    pool.close()


def test_chain_errors_match_oracle():
    from heterogeneous_rank_gemm_amd import LoraError
    pool, reg, _ = _setup(16, 16, 16, 3)
    for cid, members in [(14, [1, 4, 0, 3]), (14, [0, 0]), (14, [0, 10]), (14, [7]), (10, [2]),
                         (16, [0]), (14, [0, 99]), (14, [])]:
        try:
            pool.load_chain(cid, members)
            lib = "OK"
        except LoraError as e:
            lib = e.status
        try:
            reg.load_chain(cid, members)
            ora = "OK"
        except OracleError as e:
            ora = e.status
        assert lib == ora and lib != "OK", (cid, members, lib, ora)
    pool.close()


def test_chain_block_layout_limit():
    """The library's own, stricter limit (not the pages' rule, which the oracle
    follows): a chain's pages hold its members side by side in whole 16-rank
    blocks, one scale per block, so every member but the last takes a multiple
    of 16 ranks.  Three rank-5 adapters (15 ranks) therefore fit the oracle's
    rule at a max rank of 16 but need 16 + 16 + 5 page rows and are refused
    with RANK; at a max rank of 48 the library accepts them."""
    from heterogeneous_rank_gemm_amd import LoraError, LoraPool
    for max_rank, lib_ok in ((16, False), (48, True)):
        pool = LoraPool(8, 8, max_rank, [64], [64], 8)
        reg = oracle.Registry(8, 8, max_rank, [64], [64], 8)
        for i in range(3):
            a = (torch.randn((64, 5)) * 0.02).to(torch.bfloat16)
            b = (torch.randn((5, 64)) * 0.02).to(torch.bfloat16)
            pool.load_adapter(i, 5, 10.0, [a.cuda()], [b.cuda()])
            reg.load(i, 5, 10.0, [a], [b])
        reg.load_chain(5, [0, 1, 2])                 # the pages' rule: 15 <= max rank
        if lib_ok:
            pool.load_chain(5, [0, 1, 2])
        else:
            with pytest.raises(LoraError) as e:
                pool.load_chain(5, [0, 1, 2])
            assert e.value.status == "RANK"
        pool.close()


@pytest.mark.parametrize("k", range(int(__import__("os").environ.get("HRG_CHAIN_RANDOM_CASES", 8))))
def test_random_chains_match_oracle(k):
    """Seeded random chains (1 to 3 members of ranks up to 16, pool ranks 32
    to 64, one or two linears, both paths) within the library's page layout
    (each member but the last takes whole 16-rank blocks): the oracle's
    values for a batch over adapters, chains and id -1.
    HRG_CHAIN_RANDOM_CASES scales the count (300 have passed)."""
    from heterogeneous_rank_gemm_amd import LoraPool
    g = np.random.default_rng(700000 + k)
    T = int(g.choice([int(g.integers(1, 65)), int(g.integers(65, 700))]))
    K = int(8 * g.integers(2, 300))
    d_outs = [int(8 * g.integers(2, 300)) for _ in range(int(g.integers(1, 3)))]
    max_rank, n = int(g.choice([32, 48, 64])), int(g.integers(2, 9))
    ranks = [int(g.integers(1, 17)) for _ in range(n)]
    max_ids = n + 6
    print(f"[chain random {k}] T={T} K={K} d_outs={d_outs} max_rank={max_rank} ranks={ranks}", flush=True)
    pool = LoraPool(max_ids, max_ids, max_rank, [K] * len(d_outs), d_outs, T)
    reg = oracle.Registry(max_ids, max_ids, max_rank, [K] * len(d_outs), d_outs, T)
    gen = torch.Generator().manual_seed(k)
    for i, r in enumerate(ranks):
        A = [(torch.randn((K, r), generator=gen) * 0.02).to(torch.bfloat16) for _ in d_outs]
        B = [(torch.randn((r, d), generator=gen) * 0.02).to(torch.bfloat16) for d in d_outs]
        al = float(2 * r if i % 2 else 24)
        pool.load_adapter(i, r, al, [a.cuda() for a in A], [b.cuda() for b in B])
        reg.load(i, r, al, A, B)
    X = torch.randn((T, K), generator=gen).to(torch.bfloat16)
    W = [(torch.randn((d, K), generator=gen) * 0.02).to(torch.bfloat16) for d in d_outs]
    made = []
    for c in range(n, max_ids):
        members = [int(x) for x in g.choice(n, size=min(int(g.integers(1, 4)), n), replace=False)]
        if 16 * sum((ranks[x] + 15) // 16 for x in members[:-1]) + ranks[members[-1]] > max_rank:
            continue
        pool.load_chain(c, members)
        reg.load_chain(c, members)
        made.append(c)
    ids_np = g.choice(np.array([-1] + list(range(n)) + made, np.int32), size=T)
    ids = torch.as_tensor(ids_np, device="cuda")
    for m in range(len(d_outs)):
        out = torch.empty((T, d_outs[m]), dtype=torch.bfloat16, device="cuda")
        pool.apply(m, X.cuda(), ids, W[m].cuda(), out)
        torch.cuda.synchronize()
        assert pool.status() == "OK"
        mx, rl1, _ = oracle.parity_metrics(out.cpu(), oracle.lora_linear(reg, m, X, ids_np, W[m]))
        assert mx <= oracle.MAX_REL_TOL and rl1 <= oracle.RELL1_TOL, (m, mx, rl1)
    pool.close()
