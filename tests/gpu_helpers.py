"""Helpers for the GPU tests: build a pool from a seeded workload, run the
HIP path through the C ABI, and compute the oracle on the same bf16 bits.

The oracle receives host copies of exactly the tensors handed to the
library; nothing it sees comes from the HIP path."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads as wk
from heterogeneous_rank_gemm_amd import LoraPool

DEV = "cuda"


class Case:
    """A loaded pool plus inputs for a subset of a workload's modules."""

    def __init__(self, wl: wk.Workload, seed=None, modules=None, max_rank=None,
                 adapters=None, ids=None, max_tokens=None, max_adapters=None,
                 oracle_modules=None):
        self.wl = wl
        self.seed = wl.default_seed if seed is None else seed
        self.modules = list(range(wl.n_modules)) if modules is None else list(modules)
        self.ranks = wk.adapter_ranks(wl, self.seed)
        self.ids_np = wk.adapter_ids(wl, self.seed) if ids is None else np.asarray(ids, np.int32)
        self.T = int(self.ids_np.shape[0])
        self.max_rank = wl.max_rank if max_rank is None else max_rank
        mods = [wl.modules[m] for m in self.modules]
        self.pool = LoraPool(max_adapters or wl.n_adapters, wl.n_adapters, self.max_rank,
                             [m.d_in for m in mods], [m.d_out for m in mods],
                             max(max_tokens or self.T, 1))
        self.adapters = list(range(wl.n_adapters)) if adapters is None else list(adapters)
        # the oracle registry may hold a subset of the modules (positions j)
        self.oj = list(range(len(self.modules))) if oracle_modules is None else list(oracle_modules)
        omods = [mods[j] for j in self.oj]
        self.reg = oracle.Registry(max_adapters or wl.n_adapters, wl.n_adapters, self.max_rank,
                                   [m.d_in for m in omods], [m.d_out for m in omods],
                                   max(max_tokens or self.T, 1))
        # the oracle only needs the adapters this batch uses
        self.used = set(wk.distinct_adapters(self.ids_np))
        for i in self.adapters:
            self.load(i)
        self.ids = torch.as_tensor(self.ids_np, device=DEV)
        self.X = {}
        self.W = {}
        for j, m in enumerate(self.modules):
            mod = wl.modules[m]
            if mod.input_group not in self.X:
                self.X[mod.input_group] = wk.activation(wl, mod.input_group, mod.d_in, self.seed,
                                                        DEV, T=self.T)
            self.W[j] = wk.base_weight(wl, m, self.seed, DEV)
        torch.cuda.synchronize()

    def load(self, i: int):
        r = int(self.ranks[i])
        al = wk.adapter_alpha(self.wl, r)
        A, B = [], []
        for m in self.modules:
            a, b = wk.adapter_weights(self.wl, i, m, r, self.seed, DEV)
            A.append(a)
            B.append(b)
        self.pool.load_adapter(i, r, al, A, B)
        if i in self.used:
            self.reg.load(i, r, al, [A[j].cpu() for j in self.oj], [B[j].cpu() for j in self.oj])

    def unload(self, i: int):
        self.pool.unload_adapter(i)
        if i in self.reg.adapters:
            self.reg.unload(i)

    def x_for(self, j: int):
        return self.X[self.wl.modules[self.modules[j]].input_group]

    def out_buf(self, j: int, fill=None):
        d_out = self.wl.modules[self.modules[j]].d_out
        o = torch.empty((self.T, d_out), dtype=torch.bfloat16, device=DEV)
        if fill is not None:
            o.fill_(fill)
        return o

    def apply(self, j: int, plan=None, ids=None):
        out = self.out_buf(j)
        self.pool.apply(j, self.x_for(j), self.ids if ids is None else ids, self.W[j], out,
                        plan=plan)
        return out

    def base_apply(self, j: int):
        out = self.out_buf(j)
        self.pool.base_apply(j, self.x_for(j), self.W[j], out)
        return out

    def oracle(self, j: int, rows=None):
        X = self.x_for(j).cpu()
        W = self.W[j].cpu()
        k = self.oj.index(j)  # the module's index in the oracle registry
        if rows is None:
            return oracle.lora_linear(self.reg, k, X, self.ids_np, W)
        rows = np.asarray(rows)
        return oracle.lora_linear_sampled(self.reg, k, X[torch.as_tensor(rows)],
                                          self.ids_np[rows], W)

    def close(self):
        self.pool.close()


def assert_parity(out, Yref, what=""):
    mx, rl1, elem = oracle.parity_metrics(out, Yref)
    assert mx <= oracle.MAX_REL_TOL, f"{what}: max|err|/max|Y| = {mx:.3e}"
    assert rl1 <= oracle.RELL1_TOL, f"{what}: relL1 = {rl1:.3e}"
    return mx, rl1, elem
