"""Pins for the oracle's model of host <-> device paging (PagedRegistry).

The policy ([vLLM-ch7] "starting a multi-LoRA service": --max-loras on the
GPU, --max-cpu-loras in a CPU cache swapped in on demand; [icman] section
2.2: least-recently-used adapters are swapped out, a preload list stays) is
checked against things other than itself:
  * a closed form of LRU: after every call the device holds the C most
    recently named ids (recency = (last call that named it, id));
  * a textbook LRU (collections.OrderedDict) on one-id batches, where the
    batch-aware policy and the classic one coincide;
  * invariants: pinned and directly loaded adapters are never evicted, a
    failed call changes nothing, strict mode rejects ids not named by the
    last prefetch, and the values equal those of a plain registry.
"""
from collections import OrderedDict

import numpy as np
import pytest

import oracle
from oracle import OracleError, PagedRegistry, Registry


def _adapter(rank, d_in=6, d_out=5, seed=0):
    g = np.random.default_rng(seed)
    A = np.round(g.standard_normal((d_in, rank)) * 8) / 8
    B = np.round(g.standard_normal((rank, d_out)) * 8) / 8
    return [A], [B]


def _paged(C, n_ids, max_cpu=None, d_in=6, d_out=5, rank=2):
    reg = PagedRegistry(C, n_ids, 4, [d_in], [d_out], 16, max_cpu or n_ids)
    for i in range(n_ids if max_cpu is None else max_cpu):
        reg.host_register(i, rank, 2.0 * rank, *_adapter(rank, d_in, d_out, seed=i))
    return reg


def _top_c(history, C):
    """Closed form: the C most recently named ids by (last call, id)."""
    last = {}
    for c, batch in enumerate(history, start=1):
        for i in batch:
            last[i] = c
    ranked = sorted(last, key=lambda i: (last[i], i), reverse=True)
    return set(ranked[:C])


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_lru_matches_closed_form(seed):
    g = np.random.default_rng(seed)
    C, n_ids = 5, 17
    reg = _paged(C, n_ids)
    history = []
    for _ in range(60):
        size = int(g.integers(1, C + 1))
        batch = [int(x) for x in g.choice(n_ids, size=size, replace=False)]
        ids = batch + [int(x) for x in g.choice(batch, size=3)] + [-1]   # repeats and base rows
        g.shuffle(ids)
        before = set(reg.cached)
        loads = reg.prefetch(ids)
        history.append(batch)
        assert set(loads) == set(batch) - before
        assert reg.cached == _top_c(history, C)
        assert set(reg.adapters) == set(batch)


def test_lru_matches_textbook_lru_on_single_id_batches():
    g = np.random.default_rng(7)
    C, n_ids = 4, 11
    reg = _paged(C, n_ids)
    lru = OrderedDict()
    for _ in range(200):
        i = int(g.integers(0, n_ids))
        loads = reg.prefetch([i])
        if i in lru:
            lru.move_to_end(i)
            assert loads == []
        else:
            if len(lru) == C:
                lru.popitem(last=False)
            lru[i] = True
            assert loads == [i]
        assert reg.cached == set(lru)


def test_pinned_and_direct_adapters_are_never_evicted():
    g = np.random.default_rng(3)
    reg = PagedRegistry(6, 30, 4, [6], [5], 16, 20)
    for i in range(20):
        reg.host_register(i, 2, 4.0, *_adapter(2, seed=i))
    reg.load(25, 3, 6.0, *_adapter(3, seed=25))        # loaded directly
    reg.pin(4, True)
    reg.pin(9, True)
    assert reg.where(4) == 3 and reg.where(9) == 3 and reg.where(25) == 3
    for _ in range(80):
        batch = [int(x) for x in g.choice(20, size=int(g.integers(1, 4)), replace=False)]
        reg.prefetch(batch + [25])
        assert {4, 9} <= reg.cached
        assert 25 in reg.adapters and 4 in reg.adapters and 9 in reg.adapters
        assert len(reg.cached) + len(reg.direct) <= 6
    reg.pin(4, False)
    reg.prefetch([0, 1, 2])
    reg.prefetch([3, 5, 6])                               # 4 is evictable now
    assert 4 not in reg.cached
    assert 9 in reg.cached


def test_failed_prefetch_changes_nothing():
    reg = _paged(3, 8)
    reg.pin(0, True)
    reg.prefetch([1, 2])
    state = (set(reg.cached), dict(reg.last_use), reg.calls, set(reg.adapters))
    for bad, status in [([3, 4, 5], oracle.POOL_FULL), ([1, 99], oracle.ID_RANGE),
                        ([-2], oracle.ID_RANGE)]:
        with pytest.raises(OracleError) as e:
            reg.prefetch(bad)
        assert e.value.status == status
        assert (set(reg.cached), dict(reg.last_use), reg.calls, set(reg.adapters)) == state
    reg2 = _paged(3, 8, max_cpu=5)
    with pytest.raises(OracleError) as e:
        reg2.prefetch([1, 6, 99])                          # out of range beats not loaded
    assert e.value.status == oracle.ID_RANGE
    with pytest.raises(OracleError) as e:
        reg2.prefetch([1, 6])
    assert e.value.status == oracle.NOT_LOADED
    assert reg2.calls == 0 and not reg2.cached


def test_registration_errors():
    reg = PagedRegistry(2, 6, 4, [6], [5], 16, 2)
    reg.host_register(0, 2, 4.0, *_adapter(2))
    for args, status in [((0, 2), oracle.EXISTS), ((6, 2), oracle.ID_RANGE),
                         ((1, 5), oracle.RANK), ((1, 0), oracle.RANK)]:
        with pytest.raises(OracleError) as e:
            reg.host_register(args[0], args[1], 1.0, *_adapter(max(args[1], 1)))
        assert e.value.status == status
    reg.host_register(1, 2, 4.0, *_adapter(2, seed=1))
    with pytest.raises(OracleError) as e:
        reg.host_register(2, 2, 4.0, *_adapter(2, seed=2))
    assert e.value.status == oracle.POOL_FULL               # host cache full
    with pytest.raises(OracleError) as e:
        reg.load(1, 2, 4.0, *_adapter(2))
    assert e.value.status == oracle.EXISTS                  # already host-cached
    with pytest.raises(OracleError) as e:
        reg.pin(3, True)
    assert e.value.status == oracle.NOT_LOADED
    with pytest.raises(OracleError) as e:
        reg.unload(1)                                       # registered, not on the device
    assert e.value.status == oracle.NOT_LOADED
    reg.prefetch([1])
    reg.unload(1)                                           # drops the device copy only
    assert reg.where(1) == 1
    reg.host_unregister(1)
    assert reg.where(1) == 0
    with pytest.raises(OracleError) as e:
        reg.host_unregister(1)
    assert e.value.status == oracle.NOT_LOADED


def test_pin_needs_an_evictable_slot():
    reg = _paged(2, 6)
    reg.prefetch([0, 1])                                    # both addressable: not evictable
    with pytest.raises(OracleError) as e:
        reg.pin(2, True)
    assert e.value.status == oracle.POOL_FULL
    reg.prefetch([0])                                       # 1 stays cached, not addressable
    reg.pin(2, True)
    assert reg.cached == {0, 2} and reg.where(1) == 1


def test_strict_mode_and_values_follow_the_last_prefetch():
    d_in, d_out, T = 6, 5, 4
    reg = _paged(3, 6, d_in=d_in, d_out=d_out, rank=3)
    plain = Registry(6, 6, 4, [d_in], [d_out], 16)
    for i in range(6):
        plain.load(i, 3, 6.0, *_adapter(3, d_in, d_out, seed=i))
    g = np.random.default_rng(0)
    X = np.round(g.standard_normal((T, d_in)) * 4) / 4
    W = np.round(g.standard_normal((d_out, d_in)) * 4) / 4
    reg.prefetch([0, 2])
    ids = np.array([2, -1, 0, 2])
    np.testing.assert_array_equal(oracle.lora_linear(reg, 0, X, ids, W),
                                  oracle.lora_linear(plain, 0, X, ids, W))
    reg.prefetch([1])
    assert reg.where(0) == 2 and reg.where(2) == 2        # cached, no longer named
    with pytest.raises(OracleError) as e:
        oracle.lora_linear(reg, 0, X, ids, W)
    assert e.value.status == oracle.NOT_LOADED
