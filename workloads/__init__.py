"""Seeded synthetic workloads for the heterogeneous-batch LoRA linear.

This module only *draws inputs*: shapes, adapter ids, adapter ranks and
bf16 tensors from seeded generators.  It holds none of the method's
arithmetic, so both the HIP path (through its Python binding) and the CPU
oracle can take their inputs from it without sharing any computation.

Pages cited (all three describe multi-LoRA serving):
  [LoRA-Land]  "LoRA-Land: turning the LLM into an operating system with
               hot-pluggable multi-task fine-tuned serving" (blog.itodd.wang)
  [vLLM-ch7]   "Multi-LoRA hot-plug: one model serving many tenants"
               (gufacode.com, vLLM chapter 7)
  [icman]      field report on Multi-LoRA in managed inference
               (icman.com.cn news 62580)

Recipe (the same for every workload):
  * adapter ids come from ``numpy.random.Generator(PCG64(seed))``;
  * every bf16 tensor is drawn as float32 normals from a ``torch.Generator``
    on the requested device, seeded from a hash of (workload, seed, role,
    indices), scaled by its standard deviation and rounded to bf16 by
    torch's round-to-nearest-even cast.  Seeding per tensor lets any single
    weight or adapter be regenerated on its own, which keeps sampled checks
    of the large workloads cheap;
  * X ~ N(0, 1); W_base, A and B ~ N(0, 0.02).  B is *not* zero-initialised
    (a trained adapter is not), so a dropped or doubled delta is visible.

The five workloads follow the shapes of the pages' deployments: Llama-2-7B
with 200 rank-16 adapters and 64 concurrent requests on random adapters
([LoRA-Land] "running results"), Llama-3-8B with 32 rank-16 adapters and
the seven target modules ([vLLM-ch7] "multi-LoRA hot-plug" and "training a
vLLM-compatible LoRA"), mixed ranks 8..64 aligned to the maximum rank
([vLLM-ch7] "performance notes"), and an S-LoRA-scale pool of 2000 adapters
([LoRA-Land] "technical approach").
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

# Llama shapes used by the workloads: (name, d_in, d_out).
LLAMA2_7B_TARGETS: Tuple[Tuple[str, int, int], ...] = (
    ("q_proj", 4096, 4096), ("k_proj", 4096, 4096), ("v_proj", 4096, 4096),
    ("o_proj", 4096, 4096), ("gate_proj", 4096, 11008), ("up_proj", 4096, 11008),
    ("down_proj", 11008, 4096),
)
LLAMA3_8B_TARGETS: Tuple[Tuple[str, int, int], ...] = (
    ("q_proj", 4096, 4096), ("k_proj", 4096, 1024), ("v_proj", 4096, 1024),
    ("o_proj", 4096, 4096), ("gate_proj", 4096, 14336), ("up_proj", 4096, 14336),
    ("down_proj", 14336, 4096),
)
# Which activation feeds each target in a Llama decoder layer: the attention
# block's normalised input feeds q/k/v, the attention output feeds o, the MLP
# block's normalised input (taken after the attention residual, so a different
# tensor) feeds gate/up, and the gated activation feeds down.  Linears with
# one input can share a launch; the four inputs of a layer come one after
# another in a real forward pass.
TARGET_INPUT = {"q_proj": "attn_in", "k_proj": "attn_in", "v_proj": "attn_in", "o_proj": "attn_out",
                "gate_proj": "mlp_in", "up_proj": "mlp_in", "down_proj": "mlp_act"}

X_STD = 1.0
W_STD = 0.02
AB_STD = 0.02


@dataclasses.dataclass(frozen=True)
class Module:
    """One LoRA-augmented linear: out = in @ W^T, W is d_out x d_in."""
    name: str
    d_in: int
    d_out: int
    input_group: str  # modules with the same (layer, group) read the same X


@dataclasses.dataclass(frozen=True)
class Workload:
    key: int
    name: str
    description: str
    modules: Tuple[Module, ...]
    T: int
    n_adapters: int          # ids valid in [0, n_adapters)
    max_rank: int            # pool pages are padded to this rank
    rank_choices: Tuple[int, ...]
    alpha_per_rank: float    # alpha = alpha_per_rank * r  (alpha is 2r on the pages)
    default_seed: int

    @property
    def n_modules(self) -> int:
        return len(self.modules)


def _llama_modules(targets, layers: int) -> Tuple[Module, ...]:
    mods = []
    for layer in range(layers):
        for name, din, dout in targets:
            mods.append(Module(f"L{layer}.{name}", din, dout, f"L{layer}.{TARGET_INPUT[name]}"))
    return tuple(mods)


WORKLOADS: Dict[int, Workload] = {
    1: Workload(1, "toy-1024-T64-4xr8",
                "single 1024->1024 linear, 64 tokens, 4 adapters of rank 8 (alpha 16), "
                "ids uniform over {-1,0,1,2,3}",
                (Module("linear", 1024, 1024, "x"),), 64, 4, 8, (8,), 2.0, 1),
    2: Workload(2, "llama2-7b-q_proj-decode-T64-200xr16",
                "Llama-2-7B q_proj 4096->4096, decode batch of 64 tokens, 200 resident "
                "adapters of rank 16 (alpha 32), ids uniform over the 200",
                (Module("q_proj", 4096, 4096, "x"),), 64, 200, 16, (16,), 2.0, 2),
    3: Workload(3, "llama3-8b-layer-prefill8x512+decode256-32xr16-zipf1.1",
                "one Llama-3-8B layer's seven targets, 8 prefill requests of 512 tokens "
                "plus 256 decode tokens (T=4352), 32 adapters of rank 16 (alpha 32), "
                "one Zipf(1.1) adapter draw per request",
                _llama_modules(LLAMA3_8B_TARGETS, 1), 4352, 32, 16, (16,), 2.0, 3),
    4: Workload(4, "slora-pool-2000-4096-T1024-r8..64",
                "4096->4096 linear, 1024 decode tokens, 2000 resident adapters with ranks "
                "drawn from {8,16,32,64} padded to 64 (alpha 2r); 10% of tokens id -1, "
                "80% on 5 hot adapters, 10% uniform over the other 1995",
                (Module("linear", 4096, 4096, "x"),), 1024, 2000, 64, (8, 16, 32, 64), 2.0, 4),
    5: Workload(5, "llama2-7b-decode-step-32x7-T64-200xr16",
                "full decode step of a 32-layer Llama-2-7B-shaped stack of the seven "
                "targets (224 linears), 64 tokens, 200 adapters of rank 16 (alpha 32), "
                "ids uniform over the 200, one plan per step",
                _llama_modules(LLAMA2_7B_TARGETS, 32), 64, 200, 16, (16,), 2.0, 5),
}

# Config-3 request structure: prefill requests then single-token decode requests.
CFG3_PREFILL_REQUESTS = 8
CFG3_PREFILL_LEN = 512
CFG3_DECODE_REQUESTS = 256
ZIPF_S = 1.1
# Config-4 popularity mixture (shares of all tokens).
CFG4_BASE_SHARE = 0.10
CFG4_HOT_SHARE = 0.80
CFG4_N_HOT = 5


def derive_seed(*parts) -> int:
    """Stable 63-bit seed from a tuple of ints/strings (platform independent)."""
    h = hashlib.blake2b(repr(parts).encode("utf-8"), digest_size=8).digest()
    return int.from_bytes(h, "little") & ((1 << 63) - 1)


def _rng(*parts) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(derive_seed(*parts)))


# --------------------------------------------------------------------------
# adapter ids and ranks
# --------------------------------------------------------------------------
def adapter_ids(wl: Workload, seed: Optional[int] = None) -> np.ndarray:
    """Per-token adapter ids (int32[T]); -1 means base only."""
    seed = wl.default_seed if seed is None else seed
    rng = _rng(wl.key, seed, "ids")
    if wl.key == 1:
        ids = rng.integers(-1, wl.n_adapters, size=wl.T)
    elif wl.key in (2, 5):
        ids = rng.integers(0, wl.n_adapters, size=wl.T)
    elif wl.key == 3:
        k = np.arange(1, wl.n_adapters + 1, dtype=np.float64)
        p = k ** (-ZIPF_S)
        p /= p.sum()
        n_req = CFG3_PREFILL_REQUESTS + CFG3_DECODE_REQUESTS
        req = rng.choice(wl.n_adapters, size=n_req, p=p)
        ids = np.concatenate([np.repeat(req[:CFG3_PREFILL_REQUESTS], CFG3_PREFILL_LEN),
                              req[CFG3_PREFILL_REQUESTS:]])
    elif wl.key == 4:
        u = rng.random(wl.T)
        hot = rng.integers(0, CFG4_N_HOT, size=wl.T)
        cold = rng.integers(CFG4_N_HOT, wl.n_adapters, size=wl.T)
        ids = np.where(u < CFG4_BASE_SHARE, -1,
                       np.where(u < CFG4_BASE_SHARE + CFG4_HOT_SHARE, hot, cold))
    else:
        raise ValueError(f"unknown workload {wl.key}")
    ids = np.asarray(ids, dtype=np.int32)
    assert ids.shape == (wl.T,)
    return ids


def adapter_ranks(wl: Workload, seed: Optional[int] = None) -> np.ndarray:
    """True rank of every adapter id (int32[n_adapters])."""
    seed = wl.default_seed if seed is None else seed
    if len(wl.rank_choices) == 1:
        return np.full(wl.n_adapters, wl.rank_choices[0], dtype=np.int32)
    rng = _rng(wl.key, seed, "ranks")
    return rng.choice(np.asarray(wl.rank_choices), size=wl.n_adapters).astype(np.int32)


def adapter_alpha(wl: Workload, rank: int) -> float:
    return float(wl.alpha_per_rank * rank)


# --------------------------------------------------------------------------
# bf16 tensors
# --------------------------------------------------------------------------
def normal_bf16(shape: Sequence[int], std: float, key: Tuple, device="cpu"):
    """bf16 tensor of N(0, std^2) draws from a generator seeded by ``key``."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(derive_seed(*key))
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(torch.bfloat16)


def activation(wl: Workload, group: str, d_in: int, seed: Optional[int] = None,
               device="cpu", T: Optional[int] = None):
    seed = wl.default_seed if seed is None else seed
    T = wl.T if T is None else T
    return normal_bf16((T, d_in), X_STD, (wl.key, seed, "X", group, T, d_in), device)


def base_weight(wl: Workload, module: int, seed: Optional[int] = None, device="cpu"):
    seed = wl.default_seed if seed is None else seed
    m = wl.modules[module]
    return normal_bf16((m.d_out, m.d_in), W_STD, (wl.key, seed, "W", module), device)


def adapter_weights(wl: Workload, adapter: int, module: int, rank: int,
                    seed: Optional[int] = None, device="cpu"):
    """(A [d_in x r], B [r x d_out]) for one adapter on one module."""
    seed = wl.default_seed if seed is None else seed
    m = wl.modules[module]
    A = normal_bf16((m.d_in, rank), AB_STD, (wl.key, seed, "A", adapter, module, rank), device)
    B = normal_bf16((rank, m.d_out), AB_STD, (wl.key, seed, "B", adapter, module, rank), device)
    return A, B


def small_workload(T: int, d_in: int, d_out: int, n_adapters: int, max_rank: int,
                   rank_choices: Sequence[int], n_modules: int = 1, key: int = 100) -> Workload:
    """An ad-hoc workload for tests: n_modules independent d_in->d_out linears."""
    mods = tuple(Module(f"m{i}", d_in, d_out, f"x{i}") for i in range(n_modules))
    return Workload(key, f"small-{T}-{d_in}-{d_out}", "test workload", mods, T,
                    n_adapters, max_rank, tuple(rank_choices), 2.0, key)


def uniform_ids(T: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """ids uniform over [lo, hi) for ad-hoc tests."""
    return _rng("uniform_ids", T, lo, hi, seed).integers(lo, hi, size=T).astype(np.int32)


def distinct_adapters(ids: np.ndarray) -> List[int]:
    return sorted(int(i) for i in set(ids.tolist()) if i >= 0)
