"""GPU parity over a seeded sweep of random shapes, ranks, pools and id mixes.

The fixed cases pin the workloads' own shapes; these draw the rest of the
space the boundary accepts: d_in and d_out any multiple of 8 (down to 8),
any page rank up to 64 with adapter ranks below it, direct-mapped and
slot-table pools, T on both sides of the decode size, ids uniform with -1
or piled on a few hot adapters beside a tail of single tokens.  Bar as in
the other parity tests: the oracle's tolerance, and id -1 rows bit-equal to
the base-only call ([LoRA-Land] section "2. multi-LoRA batch scheduling":
the shared base product plus each token's own low-rank term).

Two more bands: larger batches (700 to 5000 tokens, hot adapters beside a
tail) and batch sizes at the edges of the tiles, the decode size and the
plan's 8192-token staging blocks.  HRG_SWEEP_CASES, HRG_SWEEP_BIG and
HRG_SWEEP_EDGE_ROUNDS scale the number of cases (defaults 48, 8, 1)."""
import os
import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import workloads as wk  # noqa: E402

N_CASES = int(os.environ.get("HRG_SWEEP_CASES", 48))
N_BIG = int(os.environ.get("HRG_SWEEP_BIG", 8))
# batch sizes at the edges: the decode size, 64- to 256-row tiles, the
# 8192-token placement blocks of the plan, the Llama-3-8B layer batch
EDGE_T = [65, 66, 127, 128, 129, 255, 256, 257, 383, 511, 512, 513, 1023, 1024, 1025, 4095, 4096, 4097,
          4352, 8191, 8192, 8193, 9000]
N_EDGE = len(EDGE_T) * int(os.environ.get("HRG_SWEEP_EDGE_ROUNDS", 1))


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


def _draw_big(k):
    """Band 2, case k: 700 to 5000 tokens, hot adapters beside a tail."""
    g = np.random.default_rng(770000 + k)
    T = int(g.integers(700, 5000))
    d_in, d_out = int(8 * g.integers(16, 260)), int(8 * g.integers(8, 520))
    max_rank = int(g.choice([8, 16, 32, 64]))
    ranks = tuple(sorted({int(r) for r in g.integers(1, max_rank + 1, size=int(g.integers(1, 4)))}))
    n_ids = int(g.integers(2, 40))
    resident = list(range(n_ids))
    hot = g.choice(resident, size=min(3, n_ids), replace=False)
    tail = g.choice(np.array([-1] + resident, np.int32), size=T)
    ids = np.where(g.random(T) < 0.7, g.choice(hot, size=T), tail).astype(np.int32)
    return dict(T=T, d_in=d_in, d_out=d_out, max_rank=max_rank, ranks=ranks, n_ids=n_ids,
                slot_table=False, resident=resident, ids=ids)


def _draw_edge(k):
    """Band 3, case k: T = EDGE_T[k mod len]; ids uniform with -1, all one
    adapter, or hot adapters beside single tokens."""
    g = np.random.default_rng(880000 + k)
    T = EDGE_T[k % len(EDGE_T)]
    d_in, d_out = int(8 * g.integers(1, 200)), int(8 * g.integers(1, 600))
    max_rank = int(g.choice([1, 16, 17, 32, 48, 64]))
    ranks = tuple(sorted({int(r) for r in g.integers(1, max_rank + 1, size=int(g.integers(1, 4)))}))
    n_ids = int(g.integers(1, 64))
    resident = list(range(n_ids))
    if k % 3 == 0:
        ids = g.choice(np.array([-1] + resident, np.int32), size=T)
    elif k % 3 == 1:
        ids = np.full(T, resident[0], np.int32)
    else:
        hot = g.choice(resident, size=min(2, n_ids), replace=False)
        tail = g.choice(np.array([-1] + resident, np.int32), size=T)
        ids = np.where(g.random(T) < 0.8, g.choice(hot, size=T), tail)
    return dict(T=T, d_in=d_in, d_out=d_out, max_rank=max_rank, ranks=ranks, n_ids=n_ids,
                slot_table=False, resident=resident, ids=ids.astype(np.int32))


def test_sweep_draws_cover_the_space():
    """The sweep reaches both paths, both pool modes, tiny dims and every rank regime."""
    cs = [_draw(k) for k in range(N_CASES)]
    assert any(c["T"] <= 64 for c in cs) and any(c["T"] > 64 for c in cs)
    assert any(c["slot_table"] for c in cs) and any(not c["slot_table"] for c in cs)
    assert any(min(c["d_in"], c["d_out"]) <= 24 for c in cs)
    assert any(c["max_rank"] > 32 for c in cs) and any(c["max_rank"] <= 8 for c in cs)
    assert any((c["ids"] < 0).any() for c in cs)


def _run(c, tag, key):
    from gpu_helpers import Case, assert_parity
    _say(f"[{tag}] T={c['T']} d_in={c['d_in']} d_out={c['d_out']} max_rank={c['max_rank']} "
         f"ranks={c['ranks']} ids={c['n_ids']} slot_table={c['slot_table']}")
    wl = wk.small_workload(c["T"], c["d_in"], c["d_out"], c["n_ids"], c["max_rank"], c["ranks"], key=key)
    case = Case(wl, ids=c["ids"], adapters=c["resident"],
                max_adapters=len(c["resident"]) if c["slot_table"] else None)
    out = case.apply(0)
    torch.cuda.synchronize()
    assert case.pool.status() == "OK"
    assert_parity(out, case.oracle(0), tag)
    base = case.base_apply(0)
    m = torch.as_tensor(c["ids"] < 0, device="cuda")
    if m.any():
        assert torch.equal(out[m], base[m])
    case.close()


@pytest.mark.parametrize("k", range(N_CASES))
def test_random_sweep_parity(k):
    _run(_draw(k), f"sweep {k}", 500 + k)


@pytest.mark.parametrize("k", range(N_BIG))
def test_random_sweep_large_batches(k):
    _run(_draw_big(k), f"sweep large {k}", 900000 + k)


@pytest.mark.parametrize("k", range(N_EDGE))
def test_random_sweep_edge_batch_sizes(k):
    _run(_draw_edge(k), f"sweep edge {k}", 910000 + k)
