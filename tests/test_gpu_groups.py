"""GPU tests of lora_apply_group / lora_base_apply_group through the C ABI:
linears that read the same X in one call ([LoRA-Land] section "2. multi-LoRA
batch scheduling": one forward serves the grouped batch).

Each output of a group must be bit-identical to lora_apply on that linear
alone (the group only shares the staging of X and the launches), and within
the parity bar of the oracle.  Also: a graph captured while few adapters are
resident, replayed after more are loaded, must match the eager result."""
from __future__ import annotations

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402

D_IN = 520
D_OUTS = [264, 1032, 64, 776, 8, 2056, 520, 136]   # multiples of 8, ragged against 16 and 64


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _setup(max_adapters, max_ids, max_rank, ranks, T, seed, d_outs=D_OUTS, untarget=()):
    from heterogeneous_rank_gemm_amd import LoraPool
    n = len(d_outs)
    pool = LoraPool(max_adapters, max_ids, max_rank, [D_IN] * n, d_outs, max(T, 1))
    reg = oracle.Registry(max_adapters, max_ids, max_rank, [D_IN] * n, d_outs, max(T, 1))
    gen = torch.Generator().manual_seed(seed)
    for i, r in enumerate(ranks):
        A = [(torch.randn((D_IN, r), generator=gen) * 0.02).to(torch.bfloat16) for _ in d_outs]
        B = [(torch.randn((r, d), generator=gen) * 0.02).to(torch.bfloat16) for d in d_outs]
        for (ai, m) in untarget:
            if ai == i:
                A[m] = B[m] = None
        al = 2.0 * r if i % 3 else 1.5 * r
        pool.load_adapter(i, r, al, [a.cuda() if a is not None else None for a in A],
                          [b.cuda() if b is not None else None for b in B])
        reg.load(i, r, al, A, B)
    X = torch.randn((max(T, 1), D_IN), generator=gen).to(torch.bfloat16)[:T].contiguous()
    W = [(torch.randn((d, D_IN), generator=gen) * 0.02).to(torch.bfloat16) for d in d_outs]
    return pool, reg, X, W


def _outs(T, d_outs, fill=0.0):
    return [torch.full((T, d), fill, dtype=torch.bfloat16, device="cuda") for d in d_outs]


@pytest.mark.parametrize("T,max_adapters,max_ids,max_rank", [
    (64, 12, 12, 32), (17, 12, 12, 32), (1, 12, 12, 32), (64, 12, 40, 32), (40, 12, 30, 16),
    (64, 12, 12, 64)])
@pytest.mark.parametrize("group", [(0, 1, 2, 3, 4, 5, 6, 7), (5,), (1, 3), (2, 0, 6, 4, 7)])
def test_group_equals_single_linears_and_oracle(T, max_adapters, max_ids, max_rank, group):
    ranks = [8, 16, 5, min(32, max_rank), 1, 13, 16, 9, 4, 12, 3, 16][:max_adapters]
    ranks = [min(r, max_rank) for r in ranks]
    seed = 7 * T + max_ids + len(group)
    pool, reg, X, W = _setup(max_adapters, max_ids, max_rank, ranks, T, seed,
                             untarget=((2, 1), (4, 6)))
    g = np.random.default_rng(seed)
    ids_np = g.integers(-1, max_adapters, size=T).astype(np.int32)
    ids = torch.as_tensor(ids_np, device="cuda")
    Xd = X.cuda()
    Wd = [W[m].cuda() for m in group]
    d_outs = [D_OUTS[m] for m in group]
    outs = _outs(T, d_outs)
    pool.apply_group(list(group), Xd, ids, Wd, outs)
    base = _outs(T, d_outs)
    pool.base_apply_group(list(group), Xd, Wd, base)
    torch.cuda.synchronize()
    assert pool.status() == "OK"
    for k, m in enumerate(group):
        single = torch.empty_like(outs[k])
        pool.apply(m, Xd, ids, Wd[k], single)
        sbase = torch.empty_like(base[k])
        pool.base_apply(m, Xd, Wd[k], sbase)
        torch.cuda.synchronize()
        assert torch.equal(outs[k], single), f"linear {m}: group differs from lora_apply"
        assert torch.equal(base[k], sbase), f"linear {m}: base group differs from lora_base_apply"
        ref = oracle.lora_linear(reg, m, X, ids_np, W[m])
        mx, rl1, _ = oracle.parity_metrics(outs[k].cpu(), ref)
        assert mx <= oracle.MAX_REL_TOL and rl1 <= oracle.RELL1_TOL, (m, mx, rl1)
        keep = torch.as_tensor(ids_np < 0, device="cuda")
        assert torch.equal(outs[k][keep], base[k][keep])
    assert pool.status() == "OK"
    pool.close()


def test_group_batched_path_equals_single_linears():
    """Above 64 tokens a group runs its linears in turn on one plan."""
    T = 150
    pool, reg, X, W = _setup(6, 6, 16, [16, 8, 4, 16, 2, 11], T, 5)
    ids_np = np.random.default_rng(5).integers(-1, 6, size=T).astype(np.int32)
    ids = torch.as_tensor(ids_np, device="cuda")
    group = [0, 3, 5]
    Wd = [W[m].cuda() for m in group]
    outs = _outs(T, [D_OUTS[m] for m in group])
    pool.apply_group(group, X.cuda(), ids, Wd, outs)
    torch.cuda.synchronize()
    for k, m in enumerate(group):
        single = torch.empty_like(outs[k])
        pool.apply(m, X.cuda(), ids, Wd[k], single)
        torch.cuda.synchronize()
        assert torch.equal(outs[k], single)
        mx, rl1, _ = oracle.parity_metrics(outs[k].cpu(), oracle.lora_linear(reg, m, X, ids_np, W[m]))
        assert mx <= oracle.MAX_REL_TOL and rl1 <= oracle.RELL1_TOL
    assert pool.status() == "OK"
    pool.close()


def test_group_strict_mode_leaves_every_output_untouched():
    T = 48
    pool, _, X, W = _setup(8, 8, 16, [16, 8, 4], T, 3)
    group = [0, 1, 2]
    ids_np = np.zeros(T, np.int32)
    ids_np[9] = 5                                  # not loaded
    outs = _outs(T, [D_OUTS[m] for m in group], fill=3.0)
    pool.apply_group(group, X.cuda(), torch.as_tensor(ids_np, device="cuda"),
                     [W[m].cuda() for m in group], outs)
    torch.cuda.synchronize()
    for o in outs:
        assert bool((o == 3.0).all())
    assert pool.status() == "NOT_LOADED"
    pool.close()


def test_group_argument_errors():
    from heterogeneous_rank_gemm_amd import LoraError, LoraPool, lora_apply_group
    pool = LoraPool(4, 4, 8, [64, 64, 128] + [64] * 7, [64, 32, 64] + [16] * 7, 16)
    X = torch.zeros((16, 64), dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros(16, dtype=torch.int32, device="cuda")
    W = [torch.zeros((pool.d_out[m], pool.d_in[m]), dtype=torch.bfloat16, device="cuda")
         for m in range(10)]
    out = [torch.zeros((16, pool.d_out[m]), dtype=torch.bfloat16, device="cuda") for m in range(10)]
    for mods in ([], [0, 0], [0, 2], list(range(3, 10)) + [0, 1], [10]):
        with pytest.raises(LoraError) as e:
            lora_apply_group(pool.handle, mods, X, ids, 16, [W[m % 10] for m in mods],
                             [out[m % 10] for m in mods])
        assert e.value.status == "INVALID_ARG", mods
    pool.close()


@pytest.mark.parametrize("max_ids", [12, 20], ids=["direct-mapped", "slot-table"])
def test_graph_captured_with_few_adapters_replays_after_more_load(max_ids):
    """Regression: the decode launch covers every adapter the pool could hold,
    not the ones resident at capture.  Capture with 2 adapters loaded, load 10
    more, replay on a batch over all 12: outputs equal the eager call and the
    oracle."""
    from heterogeneous_rank_gemm_amd import LoraPool
    T, n_ad, r = 64, 12, 16
    d_outs = [264, 1032]
    pool = LoraPool(n_ad, max_ids, r, [D_IN] * 2, d_outs, T)
    reg = oracle.Registry(n_ad, max_ids, r, [D_IN] * 2, d_outs, T)
    gen = torch.Generator().manual_seed(11)
    AB = []
    for i in range(n_ad):
        A = [(torch.randn((D_IN, r), generator=gen) * 0.02).to(torch.bfloat16) for _ in d_outs]
        B = [(torch.randn((r, d), generator=gen) * 0.02).to(torch.bfloat16) for d in d_outs]
        AB.append((A, B))
    for i in range(2):
        pool.load_adapter(i, r, 32.0, [a.cuda() for a in AB[i][0]], [b.cuda() for b in AB[i][1]])
        reg.load(i, r, 32.0, *AB[i])
    X = torch.randn((T, D_IN), generator=gen).to(torch.bfloat16)
    W = [(torch.randn((d, D_IN), generator=gen) * 0.02).to(torch.bfloat16) for d in d_outs]
    Xd, Wd = X.cuda(), [w.cuda() for w in W]
    ids = torch.zeros(T, dtype=torch.int32, device="cuda")
    outs = _outs(T, d_outs)

    def step():
        pool.apply_group([0, 1], Xd, ids, Wd, outs)
        pool.apply(1, Xd, ids, Wd[1], outs[1])

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for i in range(2, n_ad):
        pool.load_adapter(i, r, 32.0, [a.cuda() for a in AB[i][0]], [b.cuda() for b in AB[i][1]])
        reg.load(i, r, 32.0, *AB[i])
    ids_np = np.random.default_rng(4).integers(-1, n_ad, size=T).astype(np.int32)
    ids.copy_(torch.as_tensor(ids_np, device="cuda"))
    torch.cuda.synchronize()
    step()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    for rep in range(3):
        for o in outs:
            o.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in range(2):
            assert torch.equal(outs[k], eager[k]), f"replay {rep}, linear {k}"
    assert pool.status() == "OK"
    for k in range(2):
        mx, rl1, _ = oracle.parity_metrics(outs[k].cpu(), oracle.lora_linear(reg, k, X, ids_np, W[k]))
        assert mx <= oracle.MAX_REL_TOL and rl1 <= oracle.RELL1_TOL, (k, mx, rl1)
    pool.close()


def _frag_layout_reference(W):
    """The fragment-tile layout written out with numpy reshapes (not the
    library's index formula): pad to 16 x 32 multiples; for each block of
    1024 columns, cut into 16-row x 32-column tiles ordered by row group,
    then step, and inside a tile order the 8-element pieces by (column
    octet, row)."""
    N, K = W.shape
    Np, Kp = -(-N // 16) * 16, -(-K // 32) * 32
    P = np.zeros((Np, Kp), dtype=W.dtype)
    P[:N, :K] = W
    out = []
    for c0 in range(0, Kp, 1024):
        blk = P[:, c0:min(c0 + 1024, Kp)]
        t = blk.reshape(Np // 16, 16, blk.shape[1] // 32, 4, 8)   # (group, row, step, octet, element)
        out.append(t.transpose(0, 2, 3, 1, 4).reshape(-1))        # (group, step, octet, row, element)
    return np.concatenate(out)


@pytest.mark.parametrize("N,K", [(264, 520), (8, 40), (1032, 4096), (64, 32), (40, 2600)])
def test_pack_weight_layout(N, K):
    import heterogeneous_rank_gemm_amd as hrg
    W = (torch.arange(N * K, dtype=torch.int64) % 30011).to(torch.int16).view(N, K)
    Wd = W.view(torch.bfloat16).cuda()
    Wp = torch.full((hrg.lora_packed_weight_elems(N, K),), -1, dtype=torch.int16, device="cuda")
    hrg.lora_pack_weight(Wd, N, K, Wp.view(torch.bfloat16), None)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(Wp.cpu().numpy(), _frag_layout_reference(W.numpy()))


@pytest.mark.parametrize("T,max_ids", [(64, 12), (17, 30), (1, 12)])
def test_packed_group_equals_row_major(T, max_ids):
    """Fragment-tiled weights give the row-major call's bits (the same
    products in the same order), LoRA and base-only."""
    max_adapters, max_rank = 12, 32
    ranks = [8, 16, 5, 32, 1, 13, 16, 9, 4, 12, 3, 16]
    pool, reg, X, W = _setup(max_adapters, max_ids, max_rank, ranks, T, 31 + T,
                             untarget=((2, 1), (4, 6)))
    ids_np = np.random.default_rng(T).integers(-1, max_adapters, size=T).astype(np.int32)
    ids = torch.as_tensor(ids_np, device="cuda")
    Xd = X.cuda()
    group = [0, 1, 2, 3, 4, 5, 6, 7]
    Wd = [W[m].cuda() for m in group]
    Wp = [pool.pack_weight(w) for w in Wd]
    d_outs = [D_OUTS[m] for m in group]
    ref, got, refb, gotb = _outs(T, d_outs), _outs(T, d_outs), _outs(T, d_outs), _outs(T, d_outs)
    pool.apply_group(group, Xd, ids, Wd, ref)
    pool.apply_group_packed(group, Xd, ids, Wp, got)
    pool.base_apply_group(group, Xd, Wd, refb)
    pool.base_apply_group_packed(group, Xd, Wp, gotb)
    torch.cuda.synchronize()
    assert pool.status() == "OK"
    for k, m in enumerate(group):
        assert torch.equal(got[k], ref[k]), f"linear {m}"
        assert torch.equal(gotb[k], refb[k]), f"base linear {m}"
        mx, rl1, _ = oracle.parity_metrics(got[k].cpu(), oracle.lora_linear(reg, m, X, ids_np, W[m]))
        assert mx <= oracle.MAX_REL_TOL and rl1 <= oracle.RELL1_TOL, (m, mx, rl1)
    pool.close()


def test_packed_rejects_batched_sizes():
    from heterogeneous_rank_gemm_amd import LoraError, LoraPool
    pool = LoraPool(2, 2, 8, [64], [64], 128)
    X = torch.zeros((100, 64), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((100, 64), dtype=torch.bfloat16, device="cuda")
    Wp = pool.pack_weight(W)
    with pytest.raises(LoraError) as e:
        pool.base_apply_group_packed([0], X, [Wp], [out])
    assert e.value.status == "INVALID_ARG"
    pool.close()


@pytest.mark.parametrize("T", [64, 17, 1])
@pytest.mark.parametrize("K", [2048, 3000, 5000, 11008])
def test_deep_group_equals_single_linears(K, T):
    """Deep K (2 to 11 chunks of 1024, ragged tails): a group of eight
    linears fills the chip with blocks that each take two chunks, while each
    linear alone is small enough to take one chunk per block.  Both add the
    chunk sums in pairs, so every output must be the same bits; both must
    meet the oracle's bar."""
    from heterogeneous_rank_gemm_amd import LoraPool
    n_ad, r, n_lin, N = 64, 16, 8, 1024
    pool = LoraPool(n_ad, n_ad, r, [K] * n_lin, [N] * n_lin, 64)
    reg = oracle.Registry(n_ad, n_ad, r, [K] * n_lin, [N] * n_lin, 64)
    gen = torch.Generator().manual_seed(K + T)
    ids_np = np.random.default_rng(K + T).integers(-1, n_ad, size=T).astype(np.int32)
    for i in sorted(set(ids_np[ids_np >= 0].tolist())):
        A = [(torch.randn((K, r), generator=gen) * 0.02).to(torch.bfloat16) for _ in range(n_lin)]
        B = [(torch.randn((r, N), generator=gen) * 0.02).to(torch.bfloat16) for _ in range(n_lin)]
        pool.load_adapter(i, r, 32.0, [a.cuda() for a in A], [b.cuda() for b in B])
        reg.load(i, r, 32.0, A, B)
    X = torch.randn((T, K), generator=gen).to(torch.bfloat16)
    W = [(torch.randn((N, K), generator=gen) * 0.02).to(torch.bfloat16) for _ in range(n_lin)]
    Xd, Wd = X.cuda(), [w.cuda() for w in W]
    ids = torch.as_tensor(ids_np, device="cuda")
    mods = list(range(n_lin))
    outs, base = _outs(T, [N] * n_lin), _outs(T, [N] * n_lin)
    pool.apply_group(mods, Xd, ids, Wd, outs)
    pool.base_apply_group(mods, Xd, Wd, base)
    single, sbase = _outs(T, [N] * n_lin), _outs(T, [N] * n_lin)
    for m in mods:
        pool.apply(m, Xd, ids, Wd[m], single[m])
        pool.base_apply(m, Xd, Wd[m], sbase[m])
    torch.cuda.synchronize()
    assert pool.status() == "OK"
    keep = torch.as_tensor(ids_np < 0, device="cuda")
    for m in mods:
        assert torch.equal(outs[m], single[m]), f"linear {m}: group differs from lora_apply"
        assert torch.equal(base[m], sbase[m]), f"linear {m}: base group differs from lora_base_apply"
        assert torch.equal(outs[m][keep], base[m][keep])
    for m in (0, n_lin - 1):
        mx, rl1, _ = oracle.parity_metrics(outs[m].cpu(), oracle.lora_linear(reg, m, X, ids_np, W[m]))
        assert mx <= oracle.MAX_REL_TOL and rl1 <= oracle.RELL1_TOL, (m, mx, rl1)
    pool.close()


N_RANDOM_GROUPS = int(__import__("os").environ.get("HRG_GROUP_RANDOM_CASES", 12))


@pytest.mark.parametrize("k", range(N_RANDOM_GROUPS))
def test_random_groups_equal_single_linears(k):
    """Seeded random groups: 1 to 8 linears of one d_in (any multiple of 8)
    in random order, T on both paths, pool ranks up to 64.  Every output must
    equal its single call bit for bit and meet the oracle's bar.
    HRG_GROUP_RANDOM_CASES scales the count (400 cases have passed)."""
    from heterogeneous_rank_gemm_amd import LoraPool
    g = np.random.default_rng(670000 + k)
    T = int(g.choice([int(g.integers(1, 65)), int(g.integers(65, 900))]))
    K, nl = int(8 * g.integers(1, 400)), int(g.integers(1, 9))
    d_outs = [int(8 * g.integers(1, 500)) for _ in range(nl)]
    max_rank, n = int(g.choice([1, 8, 16, 24, 48, 64])), int(g.integers(1, 10))
    ranks = [int(g.integers(1, max_rank + 1)) for _ in range(n)]
    print(f"[group random {k}] T={T} K={K} d_outs={d_outs} max_rank={max_rank} ranks={ranks}", flush=True)
    pool = LoraPool(n, n, max_rank, [K] * nl, d_outs, T)
    reg = oracle.Registry(n, n, max_rank, [K] * nl, d_outs, T)
    gen = torch.Generator().manual_seed(k)
    for i, r in enumerate(ranks):
        A = [(torch.randn((K, r), generator=gen) * 0.02).to(torch.bfloat16) for _ in d_outs]
        B = [(torch.randn((r, d), generator=gen) * 0.02).to(torch.bfloat16) for d in d_outs]
        pool.load_adapter(i, r, 2.0 * r, [a.cuda() for a in A], [b.cuda() for b in B])
        reg.load(i, r, 2.0 * r, A, B)
    ids_np = g.integers(-1, n, T).astype(np.int32)
    ids = torch.as_tensor(ids_np, device="cuda")
    X = torch.randn((T, K), generator=gen).to(torch.bfloat16)
    Xd = X.cuda()
    W = [(torch.randn((d, K), generator=gen) * 0.02).to(torch.bfloat16) for d in d_outs]
    Wd = [w.cuda() for w in W]
    group = [int(m) for m in g.permutation(nl)]
    outs = [torch.empty((T, d_outs[m]), dtype=torch.bfloat16, device="cuda") for m in group]
    pool.apply_group(group, Xd, ids, [Wd[m] for m in group], outs)
    torch.cuda.synchronize()
    assert pool.status() == "OK"
    for j, m in enumerate(group):
        single = torch.empty_like(outs[j])
        pool.apply(m, Xd, ids, Wd[m], single)
        torch.cuda.synchronize()
        assert torch.equal(outs[j], single), f"linear {m}: group differs from lora_apply"
        mx, rl1, _ = oracle.parity_metrics(outs[j].cpu(), oracle.lora_linear(reg, m, X, ids_np, W[m]))
        assert mx <= oracle.MAX_REL_TOL and rl1 <= oracle.RELL1_TOL, (m, mx, rl1)
    pool.close()


@pytest.mark.parametrize("k", range(int(__import__("os").environ.get("HRG_PACKED_RANDOM_CASES", 8))))
def test_random_packed_groups_equal_row_major(k):
    """Seeded random decode groups (T <= 64, 1 to 8 linears of any multiple of
    8, in random order) on fragment-tiled weights: bit for bit the row-major
    group call, and the oracle's values.  HRG_PACKED_RANDOM_CASES scales the
    count (300 have passed)."""
    from heterogeneous_rank_gemm_amd import LoraPool
    g = np.random.default_rng(680000 + k)
    T, K, nl = int(g.integers(1, 65)), int(8 * g.integers(1, 600)), int(g.integers(1, 9))
    d_outs = [int(8 * g.integers(1, 700)) for _ in range(nl)]
    max_rank = int(g.choice([1, 8, 16, 32, 64]))
    ranks = [int(g.integers(1, max_rank + 1)) for _ in range(int(g.integers(1, 12)))]
    n = len(ranks)
    print(f"[packed random {k}] T={T} K={K} d_outs={d_outs} max_rank={max_rank} ranks={ranks}", flush=True)
    pool = LoraPool(n, n, max_rank, [K] * nl, d_outs, T)
    reg = oracle.Registry(n, n, max_rank, [K] * nl, d_outs, T)
    gen = torch.Generator().manual_seed(k)
    for i, r in enumerate(ranks):
        A = [(torch.randn((K, r), generator=gen) * 0.02).to(torch.bfloat16) for _ in d_outs]
        B = [(torch.randn((r, d), generator=gen) * 0.02).to(torch.bfloat16) for d in d_outs]
        al = float(2 * r if i % 2 else 24)
        pool.load_adapter(i, r, al, [a.cuda() for a in A], [b.cuda() for b in B])
        reg.load(i, r, al, A, B)
    X = torch.randn((T, K), generator=gen).to(torch.bfloat16)
    W = [(torch.randn((d, K), generator=gen) * 0.02).to(torch.bfloat16) for d in d_outs]
    ids_np = g.integers(-1, n, T).astype(np.int32)
    ids = torch.as_tensor(ids_np, device="cuda")
    Xd, Wd = X.cuda(), [w.cuda() for w in W]
    Wp = [pool.pack_weight(w) for w in Wd]
    group = [int(m) for m in g.permutation(nl)]
    packed = [torch.empty((T, d_outs[m]), dtype=torch.bfloat16, device="cuda") for m in group]
    rowmaj = [torch.empty_like(x) for x in packed]
    pool.apply_group_packed(group, Xd, ids, [Wp[m] for m in group], packed)
    pool.apply_group(group, Xd, ids, [Wd[m] for m in group], rowmaj)
    torch.cuda.synchronize()
    assert pool.status() == "OK"
    for j, m in enumerate(group):
        assert torch.equal(packed[j], rowmaj[j]), f"linear {m}: packed differs from row-major"
        mx, rl1, _ = oracle.parity_metrics(packed[j].cpu(), oracle.lora_linear(reg, m, X, ids_np, W[m]))
        assert mx <= oracle.MAX_REL_TOL and rl1 <= oracle.RELL1_TOL, (m, mx, rl1)
    pool.close()
