"""GPU tests of the boundary's error behaviour and the hot-plug life cycle.

Strict mode (icman report, section 4.1): a request whose adapter is not
resident is rejected and the output is left untouched -- never silently
served by the base.  Rank limit (vLLM chapter "Multi-LoRA hot-plug",
--max-lora-rank; icman section 3.3).  Hot-plug load / unload (LoRA-Land
post, section "3. hot-plug API")."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import workloads as wk  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _pool(**kw):
    from heterogeneous_rank_gemm_amd import LoraPool
    args = dict(max_adapters=3, max_ids=8, max_rank=16, d_in=[128], d_out=[64], max_tokens=64)
    args.update(kw)
    return LoraPool(**args)


def _ab(rank, d_in=128, d_out=64, device="cuda"):
    g = torch.Generator(device=device)
    g.manual_seed(rank)
    A = (torch.randn((d_in, rank), generator=g, device=device) * 0.02).to(torch.bfloat16)
    B = (torch.randn((rank, d_out), generator=g, device=device) * 0.02).to(torch.bfloat16)
    return [A], [B]


def test_load_errors():
    from heterogeneous_rank_gemm_amd import LoraError
    p = _pool()
    with pytest.raises(LoraError) as e:
        p.load_adapter(0, 17, 34.0, *_ab(17))
    assert e.value.status == "RANK"
    with pytest.raises(LoraError) as e:
        p.load_adapter(0, 0, 1.0, *_ab(1))
    assert e.value.status == "RANK"
    with pytest.raises(LoraError) as e:
        p.load_adapter(8, 4, 8.0, *_ab(4))
    assert e.value.status == "ID_RANGE"
    p.load_adapter(0, 4, 8.0, *_ab(4))
    with pytest.raises(LoraError) as e:
        p.load_adapter(0, 4, 8.0, *_ab(4))
    assert e.value.status == "EXISTS"
    p.load_adapter(5, 16, 32.0, *_ab(16))
    p.load_adapter(7, 8, 16.0, *_ab(8))
    with pytest.raises(LoraError) as e:
        p.load_adapter(6, 8, 16.0, *_ab(8))
    assert e.value.status == "POOL_FULL"
    # lowest free slot first
    assert p.query(0)[0] == 0 and p.query(5)[0] == 1 and p.query(7)[0] == 2
    p.unload_adapter(5)
    p.load_adapter(6, 8, 16.0, *_ab(8))
    assert p.query(6)[0] == 1
    assert p.query(6)[1:] == (8, 2.0)
    with pytest.raises(LoraError) as e:
        p.unload_adapter(5)
    assert e.value.status == "NOT_LOADED"
    with pytest.raises(LoraError) as e:
        p.query(5)
    assert e.value.status == "NOT_LOADED"
    p.close()


def test_host_adapter_buffers_are_accepted():
    p = _pool()
    A, B = _ab(4, device="cpu")
    p.load_adapter(1, 4, 8.0, A, B)   # host pointers are copied too
    assert p.query(1) == (0, 4, 2.0)
    p.close()


def test_apply_argument_errors():
    from heterogeneous_rank_gemm_amd import LoraError, lora_apply
    p = _pool()
    X = torch.zeros((64, 128), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((64, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros(64, dtype=torch.int32, device="cuda")
    for kw, status in [(dict(module=1), "INVALID_ARG"), (dict(T=65), "INVALID_ARG"),
                       (dict(T=-1), "INVALID_ARG"), (dict(ids=None), "INVALID_ARG")]:
        a = dict(module=0, T=64, ids=ids)
        a.update(kw)
        with pytest.raises(LoraError) as e:
            lora_apply(p.handle, a["module"], X, a["ids"], a["T"], W, out)
        assert e.value.status == status
    # T = 0 is a no-op
    lora_apply(p.handle, 0, X, ids, 0, W, out)
    # a plan must match the ids pointer and T it was built from
    plan = p.plan_create()
    p.plan(ids, 64, plan)
    with pytest.raises(LoraError):
        lora_apply(p.handle, 0, X, ids, 32, W, out, plan)
    p.close()


@pytest.mark.parametrize("slots", [3, 8], ids=["slot-table", "direct-mapped"])
@pytest.mark.parametrize("bad,status", [(3, "NOT_LOADED"), (8, "ID_RANGE"), (-2, "ID_RANGE")])
def test_strict_mode_leaves_output_untouched(bad, status, slots):
    # 8 slots for 8 ids: the pool keeps adapter id in slot id; 3 slots: ids
    # reach their pages through the slot table
    p = _pool(max_adapters=slots)
    p.load_adapter(0, 4, 8.0, *_ab(4))
    T = 40
    X = torch.randn((T, 128), device="cuda").to(torch.bfloat16)
    W = (torch.randn((64, 128), device="cuda") * 0.02).to(torch.bfloat16)
    ids_np = np.zeros(T, np.int32)
    ids_np[::4] = -1
    ids_np[17] = bad
    ids = torch.as_tensor(ids_np, device="cuda")
    sentinel = torch.full((T, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    out = sentinel.clone()
    p.apply(0, X, ids, W, out)
    torch.cuda.synchronize()
    assert torch.equal(out, sentinel)            # nothing written, no base fallback
    # sticky: the next (valid) apply is also a no-op until the status is read
    ok_ids = torch.zeros(T, dtype=torch.int32, device="cuda")
    p.apply(0, X, ok_ids, W, out)
    torch.cuda.synchronize()
    assert torch.equal(out, sentinel)
    assert p.status() == status
    assert p.status() == "OK"                    # cleared
    p.apply(0, X, ok_ids, W, out)
    torch.cuda.synchronize()
    assert not torch.equal(out, sentinel)
    # after the error the pool computes exactly what a fresh pool computes
    q = _pool(max_adapters=slots)
    q.load_adapter(0, 4, 8.0, *_ab(4))
    ref = torch.empty_like(out)
    q.apply(0, X, ok_ids, W, ref)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert q.status() == "OK"
    q.close()
    p.close()


def test_hot_plug_round_trip_bit_exact():
    from gpu_helpers import Case
    wl = wk.WORKLOADS[1]
    c = Case(wl)
    first = c.apply(0)
    torch.cuda.synchronize()
    c.unload(2)
    sentinel = c.out_buf(0, fill=3.0)
    out = sentinel.clone()
    c.pool.apply(0, c.x_for(0), c.ids, c.W[0], out)
    torch.cuda.synchronize()
    assert torch.equal(out, sentinel)
    assert c.pool.status() == "NOT_LOADED"
    c.load(2)
    again = c.apply(0)
    torch.cuda.synchronize()
    assert torch.equal(first, again)
    c.close()
