"""GPU tests of host <-> device paging through the C ABI, against the
oracle's PagedRegistry on the same calls.

[vLLM-ch7] "starting a multi-LoRA service" (--max-loras on the GPU,
--max-cpu-loras swapped in on demand); [icman] section 2.2 (LRU swap-out,
preload list).  Checked after every prefetch: the outputs of the batch
(parity bar of the linear), and where every id is (host only / cached /
addressable), which must equal the oracle's exactly."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from oracle import OracleError  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _adapter(i, rank, shapes, seed):
    g = torch.Generator()
    g.manual_seed(10007 * seed + i)
    A = [(torch.randn((d_in, rank), generator=g) * 0.02).to(torch.bfloat16) for d_in, _ in shapes]
    B = [(torch.randn((rank, d_out), generator=g) * 0.02).to(torch.bfloat16) for _, d_out in shapes]
    return A, B


class Paged:
    """A paged pool and the oracle model, driven by the same calls."""

    def __init__(self, shapes, max_adapters, max_ids, max_cpu, max_rank, max_tokens, seed):
        from heterogeneous_rank_gemm_amd import LoraPool
        self.shapes = shapes
        d_in = [s[0] for s in shapes]
        d_out = [s[1] for s in shapes]
        self.pool = LoraPool(max_adapters, max_ids, max_rank, d_in, d_out, max_tokens)
        self.pool.host_cache_create(max_cpu)
        self.reg = oracle.PagedRegistry(max_adapters, max_ids, max_rank, d_in, d_out, max_tokens,
                                        max_cpu)
        self.max_ids = max_ids
        self.seed = seed
        g = torch.Generator()
        g.manual_seed(seed)
        self.W = [(torch.randn((o, i), generator=g) * 0.02).to(torch.bfloat16) for i, o in shapes]
        self.Wd = [w.cuda() for w in self.W]

    def register(self, i, rank, alpha):
        A, B = _adapter(i, rank, self.shapes, self.seed)
        self.pool.host_register(i, rank, alpha, A, B)
        self.reg.host_register(i, rank, alpha, A, B)

    def call(self, name, *args):
        """Run one paging call on both sides; both must agree on the status."""
        from heterogeneous_rank_gemm_amd import LoraError
        lib_status = ora_status = "OK"
        try:
            getattr(self.pool, name)(*args)
        except LoraError as e:
            lib_status = e.status
        try:
            getattr(self.reg, {"prefetch": "prefetch", "pin": "pin", "unload_adapter": "unload",
                               "host_unregister": "host_unregister"}[name])(*args)
        except OracleError as e:
            ora_status = e.status
        assert lib_status == ora_status, (name, args, lib_status, ora_status)
        return lib_status

    def check_where(self):
        for i in range(self.max_ids):
            w, p = self.pool.paging_query(i)
            assert w == self.reg.where(i), (i, w, self.reg.where(i))
            assert p == (1 if i in self.reg.pinned else 0), i

    def batch(self, T, ids_np, seed):
        g = torch.Generator()
        g.manual_seed(seed)
        ids = torch.as_tensor(ids_np, dtype=torch.int32, device="cuda")
        res = []
        for m, (d_in, d_out) in enumerate(self.shapes):
            X = torch.randn((T, d_in), generator=g).to(torch.bfloat16)
            out = torch.empty((T, d_out), dtype=torch.bfloat16, device="cuda")
            self.pool.apply(m, X.cuda(), ids, self.Wd[m], out)
            res.append((m, X, out))
        return ids, res

    def check_batch(self, ids_np, res, what):
        for m, X, out in res:
            ref = oracle.lora_linear(self.reg, m, X, ids_np, self.W[m])
            mx, rl1, _ = oracle.parity_metrics(out.cpu(), ref)
            assert mx <= oracle.MAX_REL_TOL and rl1 <= oracle.RELL1_TOL, (what, m, mx, rl1)


@pytest.mark.parametrize("T,max_adapters,max_ids", [(40, 6, 24), (130, 6, 24), (64, 24, 20)])
def test_paging_sequence_matches_oracle(T, max_adapters, max_ids):
    shapes = [(264, 520), (520, 200)]
    pg = Paged(shapes, max_adapters, max_ids, 16, 16, max(T, 8), seed=T + max_ids)
    ranks = [4, 8, 16, 13]
    for i in range(16):
        r = ranks[i % 4]
        pg.register(i, r, 24.0 if i == 5 else 2.0 * r)
    assert pg.call("pin", 3, True) == "OK"
    pg.check_where()
    g = np.random.default_rng(T)
    for k in range(10):
        req = [int(x) for x in g.choice(16, size=int(g.integers(1, 6)), replace=False)]
        ids_np = g.choice(req + [-1], size=T).astype(np.int32)
        if k == 6:
            assert pg.call("pin", 3, False) == "OK"
        st = pg.call("prefetch", ids_np.tolist())
        assert st == "OK"
        pg.check_where()
        _, res = pg.batch(T, ids_np, seed=100 + k)
        torch.cuda.synchronize()
        assert pg.pool.status() == "OK"
        pg.check_batch(ids_np, res, f"batch {k}")
    # an id that is cached but not named by the last prefetch is rejected
    cached_not_named = [i for i in range(16) if pg.reg.where(i) == 2]
    if cached_not_named:
        i = cached_not_named[0]
        ids = torch.full((T,), i, dtype=torch.int32, device="cuda")
        X = torch.zeros((T, shapes[0][0]), dtype=torch.bfloat16, device="cuda")
        out = torch.full((T, shapes[0][1]), 7.0, dtype=torch.bfloat16, device="cuda")
        pg.pool.apply(0, X, ids, pg.Wd[0], out)
        assert pg.pool.status() == "NOT_LOADED"
        assert bool((out == 7.0).all())
    pg.pool.close()


def test_prefetch_overlaps_running_batches():
    """Eight batches enqueued back to back, each evicting adapters of the
    batches before it, with no host synchronisation in between: the copies
    into evicted slots must wait for the batches that read them."""
    shapes = [(4096, 4096)]
    pg = Paged(shapes, 6, 40, 12, 16, 64, seed=5)
    for i in range(12):
        pg.register(i, 16, 32.0)
    g = np.random.default_rng(11)
    pending = []
    evictions = 0
    for k in range(8):
        req = [int(x) for x in g.choice(12, size=3, replace=False)]
        ids_np = g.choice(req, size=64).astype(np.int32)
        before = set(pg.reg.cached)
        assert pg.call("prefetch", ids_np.tolist()) == "OK"
        evictions += len(before - pg.reg.cached)
        _, res = pg.batch(64, ids_np, seed=200 + k)
        # the oracle's view of this batch, taken before the next prefetch
        refs = [oracle.lora_linear(pg.reg, m, X, ids_np, pg.W[m]) for m, X, _ in res]
        pending.append((k, res, refs))
    assert evictions > 0
    torch.cuda.synchronize()
    assert pg.pool.status() == "OK"
    for k, res, refs in pending:
        for (m, X, out), ref in zip(res, refs):
            mx, rl1, _ = oracle.parity_metrics(out.cpu(), ref)
            assert mx <= oracle.MAX_REL_TOL and rl1 <= oracle.RELL1_TOL, (k, mx, rl1)
    pg.pool.close()


def test_paging_errors_match_oracle():
    from heterogeneous_rank_gemm_amd import LoraError, LoraPool
    shapes = [(128, 64)]
    pg = Paged(shapes, 3, 10, 4, 8, 16, seed=3)
    for i in range(4):
        pg.register(i, 8, 16.0)
    # host cache full, duplicate, rank, range
    for args, status in [((4, 8, 16.0), "POOL_FULL"), ((2, 8, 16.0), "EXISTS"),
                         ((9, 9, 18.0), "RANK"), ((10, 8, 16.0), "ID_RANGE")]:
        with pytest.raises(LoraError) as e:
            A, B = _adapter(args[0], min(args[1], 8), shapes, 3)
            pg.pool.host_register(args[0], args[1], args[2], A, B)
        assert e.value.status == status, args
    # a host-cached id cannot also be loaded directly
    A, B = _adapter(1, 8, shapes, 3)
    with pytest.raises(LoraError) as e:
        pg.pool.load_adapter(1, 8, 16.0, [a.cuda() for a in A], [b.cuda() for b in B])
    assert e.value.status == "EXISTS"
    assert pg.call("prefetch", [0, 1, -1]) == "OK"
    pg.check_where()
    assert pg.call("prefetch", [0, 1, 2, 3]) == "POOL_FULL"
    assert pg.call("prefetch", [5]) == "NOT_LOADED"
    assert pg.call("prefetch", [5, 11]) == "ID_RANGE"
    pg.check_where()                                    # failed calls changed nothing
    assert pg.call("pin", 2, True) == "OK"
    assert pg.call("pin", 3, True) == "POOL_FULL"       # 0 and 1 are addressable
    assert pg.call("unload_adapter", 3) == "NOT_LOADED"
    assert pg.call("unload_adapter", 1) == "OK"
    pg.check_where()
    assert pg.call("host_unregister", 0) == "OK"
    assert pg.call("host_unregister", 0) == "NOT_LOADED"
    pg.check_where()
    pg.pool.close()
    p = LoraPool(2, 4, 8, [128], [64], 16)
    with pytest.raises(LoraError) as e:
        p.prefetch([0])
    assert e.value.status == "INVALID_ARG"             # no host cache
    p.host_cache_create(2)
    with pytest.raises(LoraError) as e:
        p.host_cache_create(2)
    assert e.value.status == "INVALID_ARG"
    p.close()


@pytest.mark.parametrize("k", range(int(__import__("os").environ.get("HRG_PAGING_RANDOM_CASES", 6))))
def test_random_paging_sequences_match_oracle(k):
    """Seeded random pools (slots, ids, host cache, ranks, one or two linears)
    driven by random sequences: prefetches of random id sets (some over
    capacity, some naming unregistered ids), pins and unpins,
    unregistrations.  After every call the statuses and every id's place
    equal the oracle's; after every successful prefetch the batch meets the
    oracle's bar.  HRG_PAGING_RANDOM_CASES scales the count (200 have
    passed)."""
    g = np.random.default_rng(720000 + k)
    T = int(g.choice([int(g.integers(1, 65)), int(g.integers(65, 400))]))
    shapes = [(int(8 * g.integers(2, 80)), int(8 * g.integers(2, 80))) for _ in range(int(g.integers(1, 3)))]
    max_adapters = int(g.integers(2, 12))
    max_ids = int(g.integers(max_adapters, 40))
    max_cpu = int(g.integers(2, max_ids + 1))
    max_rank, n_reg = int(g.choice([8, 16, 32])), int(g.integers(1, max_cpu + 1))
    print(f"[paging random {k}] T={T} shapes={shapes} slots={max_adapters} ids={max_ids} cpu={max_cpu}",
          flush=True)
    pg = Paged(shapes, max_adapters, max_ids, max_cpu, max_rank, max(T, 8), seed=k)
    ids_reg = [int(x) for x in g.choice(max_ids, size=n_reg, replace=False)]
    for i in ids_reg:
        r = int(g.integers(1, max_rank + 1))
        pg.register(i, r, 2.0 * r if i % 2 else 24.0)
    pg.check_where()
    for step in range(12):
        op = g.random()
        if op < 0.1 and ids_reg:
            pg.call("pin", int(g.choice(ids_reg)), bool(g.random() < 0.6))
            pg.check_where()
            continue
        if op < 0.15 and ids_reg:
            i = int(g.choice(ids_reg))
            if pg.call("host_unregister", i) == "OK":
                ids_reg.remove(i)
            pg.check_where()
            continue
        pool_ids = ids_reg + [int(x) for x in g.integers(0, max_ids, size=1)]
        n_req = int(g.integers(1, min(len(pool_ids), max_adapters + 2) + 1))
        req = [int(x) for x in g.choice(pool_ids, size=n_req, replace=False)]
        ids_np = g.choice(req + [-1], size=T).astype(np.int32)
        st = pg.call("prefetch", ids_np.tolist())
        pg.check_where()
        if st != "OK":
            continue
        _, res = pg.batch(T, ids_np, seed=1000 * k + step)
        torch.cuda.synchronize()
        assert pg.pool.status() == "OK"
        pg.check_batch(ids_np, res, f"step {step}")
    pg.pool.close()
