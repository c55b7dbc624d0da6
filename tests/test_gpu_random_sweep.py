"""GPU parity over a seeded sweep of random shapes, ranks, pools and id mixes.

The fixed cases pin the workloads' own shapes; these draw the rest of the
space the boundary accepts: d_in and d_out any multiple of 8 (down to 8),
any page rank up to 64 with adapter ranks below it, direct-mapped and
slot-table pools, T on both sides of the decode size, ids uniform with -1
or piled on a few hot adapters beside a tail of single tokens.  Bar as in
the other parity tests: the oracle's tolerance, and id -1 rows bit-equal to
the base-only call ([LoRA-Land] section "2. multi-LoRA batch scheduling":
the shared base product plus each token's own low-rank term)."""
import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import workloads as wk  # noqa: E402

N_CASES = 48


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import heterogeneous_rank_gemm_amd  # noqa: F401  (fails loudly if the library is missing)
    yield


def _draw(k):
    """Case k of the sweep: everything from one seeded generator."""
    g = np.random.default_rng(90210 + k)
    T = int(g.integers(1, 65)) if k % 2 == 0 else int(g.integers(65, 700))
    dims = lambda: int(8 * (g.integers(1, 4) if g.random() < 0.15 else g.integers(2, 258)))  # noqa: E731
    d_in, d_out = dims(), dims()
    max_rank = int(g.choice([1, 4, 8, 13, 16, 24, 32, 48, 64]))
    ranks = tuple(sorted({int(r) for r in g.integers(1, max_rank + 1, size=int(g.integers(1, 4)))}))
    n_ids = int(g.integers(1, 13))
    slot_table = bool(g.random() < 0.4) and n_ids > 2
    resident = sorted(int(i) for i in g.choice(n_ids, size=max(1, n_ids // 2), replace=False)) \
        if slot_table else list(range(n_ids))
    if g.random() < 0.5:
        ids = g.choice(np.array([-1] + resident, np.int32), size=T)
    else:
        hot = g.choice(resident, size=min(2, len(resident)), replace=False)
        tail = g.choice(np.array([-1] + resident, np.int32), size=T)
        ids = np.where(g.random(T) < 0.7, g.choice(hot, size=T), tail).astype(np.int32)
    return dict(T=T, d_in=d_in, d_out=d_out, max_rank=max_rank, ranks=ranks, n_ids=n_ids,
                slot_table=slot_table, resident=resident, ids=ids.astype(np.int32))


def test_sweep_draws_cover_the_space():
    """The sweep reaches both paths, both pool modes, tiny dims and every rank regime."""
    cs = [_draw(k) for k in range(N_CASES)]
    assert any(c["T"] <= 64 for c in cs) and any(c["T"] > 64 for c in cs)
    assert any(c["slot_table"] for c in cs) and any(not c["slot_table"] for c in cs)
    assert any(min(c["d_in"], c["d_out"]) <= 24 for c in cs)
    assert any(c["max_rank"] > 32 for c in cs) and any(c["max_rank"] <= 8 for c in cs)
    assert any((c["ids"] < 0).any() for c in cs)


@pytest.mark.parametrize("k", range(N_CASES))
def test_random_sweep_parity(k):
    from gpu_helpers import Case, assert_parity
    c = _draw(k)
    _say(f"[sweep {k}] T={c['T']} d_in={c['d_in']} d_out={c['d_out']} max_rank={c['max_rank']} "
         f"ranks={c['ranks']} ids={c['n_ids']} slot_table={c['slot_table']}")
    wl = wk.small_workload(c["T"], c["d_in"], c["d_out"], c["n_ids"], c["max_rank"], c["ranks"],
                           key=500 + k)
    case = Case(wl, ids=c["ids"], adapters=c["resident"],
                max_adapters=len(c["resident"]) if c["slot_table"] else None)
    out = case.apply(0)
    torch.cuda.synchronize()
    assert case.pool.status() == "OK"
    assert_parity(out, case.oracle(0), f"sweep {k}")
    base = case.base_apply(0)
    m = torch.as_tensor(c["ids"] < 0, device="cuda")
    if m.any():
        assert torch.equal(out[m], base[m])
    case.close()
