"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar: plan tables bit-exact; bf16 outputs with
max|out - Yref| <= 1e-2 * max|Yref| and sum|out - Yref| / sum|Yref| <= 2e-3
(Yref is the oracle's unrounded float64 value).  Id -1 rows must equal the
base-only kernel's rows bit for bit.

Pages cited:
  [LoRA-Land]  "LoRA-Land: turning the LLM into an operating system ..."
  [vLLM-ch7]   "Multi-LoRA hot-plug: one model serving many tenants"
  [icman]      field report on Multi-LoRA in managed inference (news 62580)
"""
import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import workloads as wk  # noqa: E402


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import heterogeneous_rank_gemm_amd  # noqa: F401  (fails loudly if the library is missing)
    yield


def _case(*a, **k):
    from gpu_helpers import Case
    return Case(*a, **k)


def _parity(*a, **k):
    from gpu_helpers import assert_parity
    return assert_parity(*a, **k)


# --------------------------------------------------------------------------
# plan: bit-exact against the oracle's counting sort
# --------------------------------------------------------------------------
PLAN_IDS = {
    "all_base": [-1] * 70,
    "all_one": [3] * 65,
    "all_distinct_desc": list(range(63, -1, -1)),
    "single": [5],
    "ragged_mix": [(t * 37) % 11 - 1 for t in range(131)],
    "dups": [9, 9, 8, 8, 7, -1, -1, 7, 0, 0],
}


@pytest.mark.parametrize("name", sorted(PLAN_IDS))
def test_plan_adversarial_bit_exact(name):
    _say(f"[plan] {name}")
    ids = np.asarray(PLAN_IDS[name], np.int32)
    wl = wk.small_workload(len(ids), 64, 64, max(16, int(ids.max()) + 1), 8, (8,))
    c = _case(wl, ids=ids, max_tokens=256)
    plan = c.pool.plan_create()
    c.pool.plan(c.ids, c.T, plan)
    got = c.pool.debug_read_plan(plan)
    want = oracle.plan(ids, wl.n_adapters)
    for g, w in zip(got, want):
        assert g == w.tolist()
    if c.T > 64:
        # above the decode size an apply without a plan builds the pool's own
        c.apply(0)
        got = c.pool.debug_read_plan()
        for g, w in zip(got, want):
            assert g == w.tolist()
    assert c.pool.status() == "OK"
    c.close()


@pytest.mark.parametrize("key", [1, 2, 3, 4, 5])
def test_plan_workload_ids_bit_exact(key):
    _say(f"[plan] workload {key}")
    wl = wk.WORKLOADS[key]
    from heterogeneous_rank_gemm_amd import LoraPool
    # tables only: a pool of tiny modules with every id loaded
    pool = LoraPool(wl.n_adapters, wl.n_adapters, 8, [64], [64], wl.T)
    A = torch.zeros((64, 8), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((8, 64), dtype=torch.bfloat16, device="cuda")
    for i in range(wl.n_adapters):
        pool.load_adapter(i, 8, 16.0, [A], [B])
    plan = pool.plan_create()
    for seed in (wl.default_seed, 11, 12):
        ids_np = wk.adapter_ids(wl, seed)
        ids = torch.as_tensor(ids_np, device="cuda")
        pool.plan(ids, wl.T, plan)
        got = pool.debug_read_plan(plan)
        want = oracle.plan(ids_np, wl.n_adapters)
        for g, w in zip(got, want):
            assert g == w.tolist()
    assert pool.status() == "OK"
    pool.close()


def test_plan_2000_distinct():
    _say("[plan] 2000 distinct ids")
    from heterogeneous_rank_gemm_amd import LoraPool
    pool = LoraPool(2000, 2000, 8, [64], [64], 2000)
    A = torch.zeros((64, 8), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((8, 64), dtype=torch.bfloat16, device="cuda")
    for i in range(2000):
        pool.load_adapter(i, 8, 16.0, [A], [B])
    ids_np = np.random.default_rng(3).permutation(2000).astype(np.int32)
    plan = pool.plan_create()
    pool.plan(torch.as_tensor(ids_np, device="cuda"), 2000, plan)
    got = pool.debug_read_plan(plan)
    want = oracle.plan(ids_np, 2000)
    for g, w in zip(got, want):
        assert g == w.tolist()
    pool.close()


# the largest batches and id ranges the plan takes: placement over several
# LDS-staged blocks of 8192 tokens (T > 8192), and each cursor layout (16, 8,
# 4 or 1 placement waves for pools of up to 1024, 2048, 4096 or 16384 ids)
PLAN_LIMITS = [(8969, 48), (9000, 1500), (12000, 3000), (4096, 16384), (1, 16384)]


@pytest.mark.parametrize("T,max_ids", PLAN_LIMITS)
def test_plan_size_limits_bit_exact(T, max_ids):
    _say(f"[plan] T={T} max_ids={max_ids}")
    from heterogeneous_rank_gemm_amd import LoraPool
    g = np.random.default_rng(T + max_ids)
    # half uniform over every id (and -1), half on five hot ids: long runs
    # beside single-token segments
    hot = g.choice(max_ids, size=5, replace=False)
    ids_np = np.where(g.random(T) < 0.5, g.integers(-1, max_ids, T), g.choice(hot, T)).astype(np.int32)
    used = sorted(set(int(i) for i in ids_np if i >= 0))
    pool = LoraPool(max(len(used), 1), max_ids, 8, [64], [64], T)
    A = torch.zeros((64, 8), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((8, 64), dtype=torch.bfloat16, device="cuda")
    for i in used:
        pool.load_adapter(i, 8, 16.0, [A], [B])
    plan = pool.plan_create()
    pool.plan(torch.as_tensor(ids_np, device="cuda"), T, plan)
    got = pool.debug_read_plan(plan)
    want = oracle.plan(ids_np, max_ids)
    for g_, w in zip(got, want):
        assert g_ == w.tolist()
    assert pool.status() == "OK"
    pool.close()


# --------------------------------------------------------------------------
# values: small ragged shapes that span several tiles
# --------------------------------------------------------------------------
RAGGED = [
    # (T, d_in, d_out, ranks, max_rank, id_lo); T <= 64 runs the one-launch decode kernel
    (1, 64, 64, (8,), 8, 0),
    (17, 1032, 520, (64, 3, 17), 64, -1),
    (48, 264, 2056, (16, 2), 16, -1),
    (64, 4104, 200, (8, 16, 32, 64), 64, -1),
    (64, 11008, 256, (16,), 16, 0),
    (3, 200, 136, (1, 5, 16), 16, -1),
    (64, 1024, 1024, (8,), 8, -1),
    (65, 520, 264, (16, 3), 16, -1),
    (130, 1032, 200, (8, 16, 32, 64), 64, -1),
    (257, 264, 1160, (4, 64, 17), 64, -1),
    (333, 4104, 136, (16,), 16, 0),
    (9000, 72, 136, (16, 5, 64), 64, -1),  # above one 8192-token placement block
    # 15 rows of 256x256 tiles, then 356 rows (a ragged 64-row tile last) of
    # 64x64 tiles in a second launch; rank-64 pages, ragged K and columns
    (4196, 264, 4104, (8, 16, 32, 64), 64, -1),
]


@pytest.mark.parametrize("T,d_in,d_out,ranks,max_rank,id_lo", RAGGED)
def test_ragged_parity(T, d_in, d_out, ranks, max_rank, id_lo):
    _say(f"[ragged] T={T} d_in={d_in} d_out={d_out} ranks={ranks}")
    n_ad = 7
    wl = wk.small_workload(T, d_in, d_out, n_ad, max_rank, ranks, key=200 + T)
    ids = wk.uniform_ids(T, id_lo, n_ad, T)
    c = _case(wl, ids=ids)
    out = c.apply(0)
    torch.cuda.synchronize()
    assert c.pool.status() == "OK"
    _parity(out, c.oracle(0), f"ragged T={T}")
    # id -1 rows: bit-identical to the base-only kernel
    base = c.base_apply(0)
    m = torch.as_tensor(ids < 0, device="cuda")
    if m.any():
        assert torch.equal(out[m], base[m])
    c.close()


# the largest batches a pool accepts: 65536 tokens, and X of just under
# 2 GiB (the batched path's 32-bit X offsets)
LARGEST = [(65536, 1024, 520, (16, 8, 3), 16, 40), (65536, 16376, 64, (64, 17), 64, 12),
           (32768, 4096, 1032, (8, 16, 32, 64), 64, 2000)]


@pytest.mark.parametrize("T,d_in,d_out,ranks,max_rank,n_ids", LARGEST)
def test_largest_batches_parity(T, d_in, d_out, ranks, max_rank, n_ids):
    _say(f"[largest] T={T} d_in={d_in} d_out={d_out} ranks={ranks} ids={n_ids}")
    assert T * d_in * 2 < 2 ** 31
    g = np.random.default_rng(T + d_in)
    hot = g.choice(n_ids, size=min(5, n_ids), replace=False)
    ids = np.where(g.random(T) < 0.8, g.choice(hot, size=T), g.integers(-1, n_ids, size=T)).astype(np.int32)
    wl = wk.small_workload(T, d_in, d_out, n_ids, max_rank, ranks, key=930000 + d_in)
    c = _case(wl, ids=ids, adapters=list(range(n_ids)))
    out = c.apply(0)
    torch.cuda.synchronize()
    assert c.pool.status() == "OK"
    _parity(out, c.oracle(0), f"largest T={T}")
    base = c.base_apply(0)
    m = torch.as_tensor(ids < 0, device="cuda")
    assert torch.equal(out[m], base[m])
    c.close()


# the largest dims a pool accepts (d_in, d_out up to 65536 with a weight of
# at most 2^31 - 1 bytes, the decode kernels' 32-bit offsets), both paths
LARGEST_DIMS = [(64, 65536, 16376, (16, 5), 16, 6), (17, 8, 65536, (64, 9), 64, 4),
                (64, 16376, 65528, (32, 1), 32, 5), (1, 65536, 8, (8,), 8, 2),
                (200, 65536, 4096, (16, 2), 16, 6), (300, 4096, 65536, (16,), 16, 3)]


@pytest.mark.parametrize("T,d_in,d_out,ranks,max_rank,n_ids", LARGEST_DIMS)
def test_largest_dims_parity(T, d_in, d_out, ranks, max_rank, n_ids):
    _say(f"[largest dims] T={T} d_in={d_in} d_out={d_out} ranks={ranks}")
    assert d_in * d_out * 2 <= 2 ** 31 - 1
    ids = np.random.default_rng(d_in + d_out).integers(-1, n_ids, size=T).astype(np.int32)
    wl = wk.small_workload(T, d_in, d_out, n_ids, max_rank, ranks, key=940000 + T)
    c = _case(wl, ids=ids, adapters=list(range(n_ids)))
    out = c.apply(0)
    torch.cuda.synchronize()
    assert c.pool.status() == "OK"
    _parity(out, c.oracle(0), f"largest dims {d_in}x{d_out}")
    base = c.base_apply(0)
    m = torch.as_tensor(ids < 0, device="cuda")
    assert torch.equal(out[m], base[m])
    c.close()


# a pool with more ids than slots reaches pages through the slot table (slot !=
# id); one with as many slots as ids keeps adapter id in slot id
INDIRECT = [
    (40, 1032, 520, (64, 3, 17), 64),
    (64, 4104, 264, (16,), 16),
    (130, 520, 1160, (8, 16, 32), 32),
]


@pytest.mark.parametrize("T,d_in,d_out,ranks,max_rank", INDIRECT)
def test_slot_table_pool_parity(T, d_in, d_out, ranks, max_rank):
    _say(f"[slot table] T={T} d_in={d_in} d_out={d_out} ranks={ranks}")
    n_ids, resident = 9, [1, 4, 5, 7, 8]   # 5 slots for 9 ids: slots 0..4 hold ids 1, 4, 5, 7, 8
    wl = wk.small_workload(T, d_in, d_out, n_ids, max_rank, ranks, key=300 + T)
    rng = np.random.Generator(np.random.PCG64(T))
    ids = rng.choice(np.array([-1] + resident, np.int32), size=T)
    c = _case(wl, ids=ids, adapters=resident, max_adapters=len(resident))
    assert [c.pool.query(i)[0] for i in resident] == list(range(len(resident)))
    out = c.apply(0)
    torch.cuda.synchronize()
    assert c.pool.status() == "OK"
    _parity(out, c.oracle(0), f"slot table T={T}")
    c.close()


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------
def test_workload1_full():
    _say("[workload 1] full")
    c = _case(wk.WORKLOADS[1])
    out = c.apply(0)
    assert c.pool.status() == "OK"
    mx, rl1, el = _parity(out, c.oracle(0), "workload 1")
    _say(f"  max {mx:.2e} relL1 {rl1:.2e} elem {el:.2e}")
    base = c.base_apply(0)
    m = torch.as_tensor(c.ids_np < 0, device="cuda")
    assert torch.equal(out[m], base[m])
    c.close()


def test_workload2_full():
    _say("[workload 2] full")
    c = _case(wk.WORKLOADS[2])
    out = c.apply(0)
    assert c.pool.status() == "OK"
    mx, rl1, el = _parity(out, c.oracle(0), "workload 2")
    _say(f"  max {mx:.2e} relL1 {rl1:.2e} elem {el:.2e}")
    c.close()


def test_workload3_full():
    """Every row of all seven linears: 8 prefill requests of 512 tokens and
    256 decode tokens span every 256 x 256 tile, every 32-row expand block and
    the small-segment rows."""
    _say("[workload 3] all seven modules, all 4352 rows")
    wl = wk.WORKLOADS[3]
    c = _case(wl)
    plan = c.pool.plan_create()
    c.pool.plan(c.ids, c.T, plan)
    for j in range(wl.n_modules):
        out = c.apply(j, plan=plan)
        ref = c.oracle(j)
        mx, rl1, el = _parity(out, ref, f"workload 3 {wl.modules[j].name}")
        _say(f"  {wl.modules[j].name}: max {mx:.2e} relL1 {rl1:.2e}")
    assert c.pool.status() == "OK"
    c.close()


def test_workload4_full():
    _say("[workload 4] full")
    c = _case(wk.WORKLOADS[4])
    out = c.apply(0)
    assert c.pool.status() == "OK"
    mx, rl1, el = _parity(out, c.oracle(0), "workload 4")
    _say(f"  max {mx:.2e} relL1 {rl1:.2e} elem {el:.2e}")
    base = c.base_apply(0)
    m = torch.as_tensor(c.ids_np < 0, device="cuda")
    assert m.any()
    assert torch.equal(out[m], base[m])
    c.close()


# --------------------------------------------------------------------------
# invariants the definition implies
# --------------------------------------------------------------------------
def test_permutation_invariance_bit_exact():
    _say("[invariant] permutation")
    wl = wk.WORKLOADS[1]
    c = _case(wl)
    out = c.apply(0)
    p = torch.as_tensor(np.random.default_rng(1).permutation(c.T), device="cuda")
    Xp = c.x_for(0)[p].contiguous()
    ids_p = c.ids[p].contiguous()
    outp = c.out_buf(0)
    c.pool.apply(0, Xp, ids_p, c.W[0], outp)
    torch.cuda.synchronize()
    assert torch.equal(outp, out[p])
    c.close()


@pytest.mark.parametrize("key", [2, 4])
def test_determinism_bit_exact(key):
    _say(f"[invariant] determinism, workload {key}")
    c = _case(wk.WORKLOADS[key])
    a = c.apply(0)
    outs = [c.apply(0) for _ in range(3)]
    torch.cuda.synchronize()
    for b in outs:
        assert torch.equal(a, b)
    base = [c.base_apply(0) for _ in range(2)]
    torch.cuda.synchronize()
    assert torch.equal(base[0], base[1])
    c.close()


def test_zero_padding_gives_identical_bits():
    # [vLLM-ch7] performance notes: mixed ranks aligned to the max rank only
    # waste work; the same adapters in a max-rank-64 pool give the same bits
    _say("[invariant] padding")
    wl = wk.small_workload(96, 512, 384, 5, 16, (16,), key=301)
    ids = wk.uniform_ids(96, -1, 5, 4)
    c16 = _case(wl, ids=ids, max_rank=16)
    c64 = _case(wl, ids=ids, max_rank=64)
    a = c16.apply(0)
    b = c64.apply(0)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    c16.close()
    c64.close()


def test_plan_reuse_matches_internal_plan():
    _say("[plan] reuse")
    wl = wk.WORKLOADS[2]
    c = _case(wl)
    plan = c.pool.plan_create()
    c.pool.plan(c.ids, c.T, plan)
    a = c.apply(0, plan=plan)
    b = c.apply(0)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    c.close()
