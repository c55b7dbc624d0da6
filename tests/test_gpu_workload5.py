"""Workload 5 on the GPU: a whole decode step of a 32-layer Llama-2-7B-shaped
stack (7 LoRA-augmented linears per layer, 224 in all), 64 tokens, 200
resident rank-16 adapters in one pool of 224 modules.

The step is captured as one hipGraph (the library records kernel launches
only) and replayed several times with eager work in between; every replay
must reproduce the eager outputs bit for bit.  Parity against the oracle is
checked on sampled rows of every linear of layers 0, 15 and 31, and the
base-only step's id-free rows against the oracle's base product."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import workloads as wk  # noqa: E402

LAYERS = (0, 15, 31)
ROWS = np.array([0, 1, 17, 31, 32, 47, 62, 63])


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def case5():
    from gpu_helpers import Case
    wl = wk.WORKLOADS[5]
    sampled = [7 * L + k for L in LAYERS for k in range(7)]
    _say("[workload 5] loading 200 adapters x 224 modules")
    c = Case(wl, oracle_modules=sampled)
    c.sampled = sampled
    c.outs = [c.out_buf(j) for j in range(len(c.modules))]
    yield c
    c.close()


def _step(c, lora=True):
    for j in range(len(c.modules)):
        if lora:
            c.pool.apply(j, c.x_for(j), c.ids, c.W[j], c.outs[j])
        else:
            c.pool.base_apply(j, c.x_for(j), c.W[j], c.outs[j])


def _snapshot(c):
    return [o.clone() for o in c.outs]


def _capture(c, lora):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _step(c, lora)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(c, lora)
    torch.cuda.synchronize()
    return g


def test_workload5_eager_step_parity_sampled_layers(case5):
    c = case5
    _say("[workload 5] eager step, parity on layers 0, 15, 31")
    _step(c, lora=True)
    torch.cuda.synchronize()
    assert c.pool.status() == "OK"
    for j in c.sampled:
        out = c.outs[j][torch.as_tensor(ROWS, device="cuda")].cpu()
        from gpu_helpers import assert_parity
        mx, rl1, _ = assert_parity(out, c.oracle(j, rows=ROWS), f"module {c.wl.modules[j].name}")
        _say(f"  {c.wl.modules[j].name}: max {mx:.3e} relL1 {rl1:.3e}")


def test_workload5_graph_replays_match_eager(case5):
    c = case5
    _say("[workload 5] eager reference step")
    _step(c, lora=True)
    torch.cuda.synchronize()
    ref = _snapshot(c)
    _say("[workload 5] capture and replay")
    g = _capture(c, lora=True)
    for rep in range(3):
        for o in c.outs:
            o.fill_(0)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for j in range(len(c.outs)):
            assert torch.equal(c.outs[j], ref[j]), f"replay {rep}: module {j} differs from eager"
    assert c.pool.status() == "OK"


def test_workload5_base_step_graph(case5):
    c = case5
    _say("[workload 5] base-only step as a graph")
    _step(c, lora=False)
    torch.cuda.synchronize()
    ref = _snapshot(c)
    g = _capture(c, lora=False)
    g.replay()
    torch.cuda.synchronize()
    for j in range(len(c.outs)):
        assert torch.equal(c.outs[j], ref[j])
    # the base-only product against the oracle's, on the sampled rows of layer 0
    from gpu_helpers import assert_parity
    for j in c.sampled[:7]:
        X = c.x_for(j).cpu()[torch.as_tensor(ROWS)]
        Yb = oracle.base_linear(X, c.W[j].cpu())
        assert_parity(ref[j][torch.as_tensor(ROWS, device="cuda")].cpu(), Yb, f"base {j}")
