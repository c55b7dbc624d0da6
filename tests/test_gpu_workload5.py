"""Workload 5 on the GPU: a whole decode step of a 32-layer Llama-2-7B-shaped
stack (7 LoRA-augmented linears per layer, 224 in all), 64 tokens, 200
resident rank-16 adapters in one pool of 224 modules.

A layer runs as four calls in the order of a Llama decoder layer: one
lora_apply_group over q, k, v (they read the attention block's input), then
o, then one group over gate and up (they read the MLP block's input), then
down.  Checked:
  * every row of every one of the 224 linears against the oracle (a registry
    of one layer at a time, so the host holds one layer's adapters);
  * the per-linear step (224 lora_apply calls) equals the grouped step bit
    for bit;
  * the step captured as one hipGraph and replayed several times, with eager
    work in between, reproduces the eager outputs bit for bit;
  * the base-only step likewise, and against the oracle's base product."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import workloads as wk  # noqa: E402

# positions within a layer: q/k/v, o, gate/up, down
LAYER_GROUPS = ((0, 1, 2), (3,), (4, 5), (6,))
LAYERS = 32


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def case5():
    from gpu_helpers import Case
    wl = wk.WORKLOADS[5]
    _say("[workload 5] loading 200 adapters x 224 modules")
    c = Case(wl, oracle_modules=[0])
    c.outs = [c.out_buf(j) for j in range(len(c.modules))]
    yield c
    c.close()


def _step(c, lora=True, grouped=True, outs=None):
    outs = c.outs if outs is None else outs
    for L in range(LAYERS):
        for grp in LAYER_GROUPS:
            mods = [7 * L + k for k in grp]
            X = c.x_for(mods[0])
            if grouped:
                W = [c.W[m] for m in mods]
                O = [outs[m] for m in mods]
                if lora:
                    c.pool.apply_group(mods, X, c.ids, W, O)
                else:
                    c.pool.base_apply_group(mods, X, W, O)
            else:
                for m in mods:
                    if lora:
                        c.pool.apply(m, X, c.ids, c.W[m], outs[m])
                    else:
                        c.pool.base_apply(m, X, c.W[m], outs[m])


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


def _layer_registry(c, L):
    """The oracle's registry for layer L's seven linears, holding the adapters
    the batch uses (the same bf16 bits the library got, regenerated)."""
    wl = c.wl
    mods = [wl.modules[7 * L + k] for k in range(7)]
    reg = oracle.Registry(wl.n_adapters, wl.n_adapters, wl.max_rank, [m.d_in for m in mods],
                          [m.d_out for m in mods], wl.T)
    for i in sorted(c.used):
        r = int(c.ranks[i])
        A, B = [], []
        for k in range(7):
            a, b = wk.adapter_weights(wl, i, 7 * L + k, r, c.seed, "cuda")
            A.append(a.cpu())
            B.append(b.cpu())
        reg.load(i, r, wk.adapter_alpha(wl, r), A, B)
    return reg


def test_workload5_grouped_step_full_parity(case5):
    c = case5
    _say("[workload 5] grouped eager step, parity on all 64 rows of all 224 linears")
    _step(c, lora=True)
    torch.cuda.synchronize()
    assert c.pool.status() == "OK"
    from gpu_helpers import assert_parity
    for L in range(LAYERS):
        reg = _layer_registry(c, L)
        worst = 0.0
        for k in range(7):
            j = 7 * L + k
            ref = oracle.lora_linear(reg, k, c.x_for(j).cpu(), c.ids_np, c.W[j].cpu())
            mx, rl1, _ = assert_parity(c.outs[j].cpu(), ref, f"module {c.wl.modules[j].name}")
            worst = max(worst, rl1)
        _say(f"  layer {L}: worst relL1 {worst:.3e}")


def test_workload5_per_linear_step_equals_grouped(case5):
    c = case5
    _say("[workload 5] per-linear step against the grouped step")
    _step(c, lora=True)
    other = [torch.empty_like(o) for o in c.outs]
    _step(c, lora=True, grouped=False, outs=other)
    torch.cuda.synchronize()
    assert c.pool.status() == "OK"
    for j in range(len(c.outs)):
        assert torch.equal(other[j], c.outs[j]), f"module {j}"


def test_workload5_graph_replays_match_eager(case5):
    c = case5
    _say("[workload 5] eager reference step")
    _step(c, lora=True)
    torch.cuda.synchronize()
    ref = [o.clone() for o in c.outs]
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
    ref = [o.clone() for o in c.outs]
    g = _capture(c, lora=False)
    g.replay()
    torch.cuda.synchronize()
    for j in range(len(c.outs)):
        assert torch.equal(c.outs[j], ref[j])
    # the base-only product against the oracle's, every row of layers 0 and 31
    from gpu_helpers import assert_parity
    for j in list(range(7)) + list(range(7 * 31, 7 * 32)):
        Yb = oracle.base_linear(c.x_for(j).cpu(), c.W[j].cpu())
        assert_parity(ref[j].cpu(), Yb, f"base {j}")
