"""GPU tests: the batched path (T > 64: plan, shrink, small-segment expand,
GEMM) captured as a hipGraph and replayed.

The library records kernel launches only on this path (no memsets, no host
synchronisation), so a captured apply must replay to the eager result bit for
bit, every time, with other work on the pool between the replays (the graph
replays of a serving loop).  Cases: a single linear with the library's own
plan inside the graph, and a grouped call on a plan built outside it."""
from __future__ import annotations

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


def _say(msg):
    print(msg, flush=True)


def _setup(d_in, d_outs, ranks, max_rank, T, seed):
    from heterogeneous_rank_gemm_amd import LoraPool
    n = len(d_outs)
    pool = LoraPool(len(ranks), len(ranks), max_rank, [d_in] * n, d_outs, T)
    reg = oracle.Registry(len(ranks), len(ranks), max_rank, [d_in] * n, d_outs, T)
    gen = torch.Generator().manual_seed(seed)
    for i, r in enumerate(ranks):
        A = [(torch.randn((d_in, r), generator=gen) * 0.02).to(torch.bfloat16) for _ in d_outs]
        B = [(torch.randn((r, d), generator=gen) * 0.02).to(torch.bfloat16) for d in d_outs]
        al = 2.0 * r if i % 3 else 24.0
        pool.load_adapter(i, r, al, [a.cuda() for a in A], [b.cuda() for b in B])
        reg.load(i, r, al, A, B)
    X = torch.randn((T, d_in), generator=gen).to(torch.bfloat16)
    W = [(torch.randn((d, d_in), generator=gen) * 0.02).to(torch.bfloat16) for d in d_outs]
    return pool, reg, X, W


def _ids(T, n_adapters, seed):
    """Long segments (hot adapters), short ones (rare adapters) and id -1."""
    g = np.random.default_rng(seed)
    hot = g.choice(n_adapters, size=3, replace=False)
    ids = np.where(g.random(T) < 0.75, hot[g.integers(0, 3, size=T)], g.integers(0, n_adapters, size=T))
    ids[g.random(T) < 0.1] = -1
    return ids.astype(np.int32)


def _capture(fn):
    """fn() captured once after an eager warm-up on the capture stream."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_batched_apply_with_its_own_plan_replays():
    T, d_in, d_out = 600, 1032, 2056
    _say(f"[graph batched] own plan T={T} K={d_in} N={d_out}")
    ranks = [16, 8, 64, 4, 33, 24, 1, 16]
    pool, reg, X, W = _setup(d_in, [d_out], ranks, 64, T, 31)
    ids_np = _ids(T, len(ranks), 31)
    ids = torch.as_tensor(ids_np, device="cuda")
    Xd, Wd = X.cuda(), W[0].cuda()
    eager = torch.empty((T, d_out), dtype=torch.bfloat16, device="cuda")
    pool.apply(0, Xd, ids, Wd, eager)
    torch.cuda.synchronize()
    mx, rl1, _ = oracle.parity_metrics(eager.cpu(), oracle.lora_linear(reg, 0, X, ids_np, W[0]))
    assert mx <= oracle.MAX_REL_TOL and rl1 <= oracle.RELL1_TOL, (mx, rl1)
    out = torch.zeros_like(eager)
    other = torch.empty_like(eager)
    g = _capture(lambda: pool.apply(0, Xd, ids, Wd, out))
    for rep in range(3):
        out.zero_()
        # eager work on the pool between the replays: another batch's apply
        # (its own plan and workspace use) and a base-only call
        pool.apply(0, Xd, torch.flip(ids, [0]), Wd, other)
        pool.base_apply(0, Xd, Wd, other)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs from the eager call"
    assert pool.status() == "OK"
    del g
    pool.close()


def test_grouped_batched_apply_on_an_outside_plan_replays():
    T, d_in, d_outs = 300, 520, [264, 1032, 776]
    _say(f"[graph batched] group T={T} N={d_outs}")
    ranks = [16, 8, 4, 16, 2, 11]
    pool, reg, X, W = _setup(d_in, d_outs, ranks, 16, T, 37)
    ids_np = _ids(T, len(ranks), 37)
    ids = torch.as_tensor(ids_np, device="cuda")
    Xd = X.cuda()
    Wd = [w.cuda() for w in W]
    group = [0, 1, 2]
    plan = pool.plan_create()
    pool.plan(ids, T, plan)
    eager = [torch.empty((T, d), dtype=torch.bfloat16, device="cuda") for d in d_outs]
    pool.apply_group(group, Xd, ids, Wd, eager, plan=plan)
    torch.cuda.synchronize()
    for m in group:
        mx, rl1, _ = oracle.parity_metrics(eager[m].cpu(), oracle.lora_linear(reg, m, X, ids_np, W[m]))
        assert mx <= oracle.MAX_REL_TOL and rl1 <= oracle.RELL1_TOL, (m, mx, rl1)
    outs = [torch.zeros_like(e) for e in eager]
    g = _capture(lambda: pool.apply_group(group, Xd, ids, Wd, outs, plan=plan))
    for rep in range(3):
        for o in outs:
            o.zero_()
        pool.apply(1, Xd, ids, Wd[1], torch.empty_like(eager[1]))   # the pool's own plan and workspace
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for m in group:
            assert torch.equal(outs[m], eager[m]), f"replay {rep}, linear {m} differs from the eager call"
    assert pool.status() == "OK"
    del g
    pool.close()
