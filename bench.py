"""Benchmark of the heterogeneous-batch LoRA linear on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 5]

A step is one pass of the whole hot path over one batch: the grouping plan
of the batch's adapter ids (built in-kernel at decode), then the LoRA linear
of every module of the workload (shrink, base GEMM, expand, single bf16
rounding).  Linears that read the same X run as one lora_apply_group call.
The default workload is the largest single-GPU one: a full decode step of a
32-layer Llama-2-7B-shaped stack (224 linears, 64 tokens, 200 resident
rank-16 adapters), replayed as one captured hipGraph.

Timing: hip events on the stream the library launches on, one pair per step
over K steps between two device synchronisations; the median step is
reported (the mean beside it).  Inputs (X, W, ids, the adapter pool) are
resident in HBM; workloads whose state fits the 256 MB Infinity Cache rotate
R independent copies (cold numbers) and are also timed on one copy (warm,
labelled as such).

Printed: ONE JSON line with tokens/s, the LoRA overhead against the
library's own base-only path, the roofline of the dominant launch pair
(decode_main + decode_combine, or shrink + GEMM at large T) and the CPU
oracle's throughput on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as wk  # noqa: E402

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
# Measured HBM traffic per step comes from rocprofv3 FETCH_SIZE / WRITE_SIZE
# runs (scaled by a plain copy of known size), valid only for the kernel
# source it was measured on.
KERNEL_SOURCE = os.path.join(ROOT, "heterogeneous_rank_gemm_amd", "csrc", "decode.hip")
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA
METRIC = "LoRA-linear tokens/sec at 1 GPU; % overhead vs base-only GEMM; % roofline"


# ---------------------------------------------------------------------------
# algorithmic work (bytes and flops that the definition must touch)
# ---------------------------------------------------------------------------
def base_bytes(T: int, d_in: int, d_out: int, int4: bool = False) -> int:
    """W once, X once, out once (bf16); an INT4 weight is half a byte per
    weight plus one 4-byte group word per 128 weights."""
    w = d_in * d_out // 2 + d_out * (d_in // 128) * 4 if int4 else 2 * d_in * d_out
    return w + 2 * (T * d_in + T * d_out)


def lora_bytes(ids: np.ndarray, ranks: np.ndarray, d_in: int, d_out: int) -> int:
    """A and B of every distinct adapter in the batch, at its true rank."""
    return sum(2 * int(ranks[i]) * (d_in + d_out) for i in wk.distinct_adapters(ids))


def flops(ids: np.ndarray, ranks: np.ndarray, d_in: int, d_out: int) -> int:
    T = ids.shape[0]
    lora = sum(2 * int(ranks[i]) * (d_in + d_out) for i in ids.tolist() if i >= 0)
    return 2 * T * d_in * d_out + lora


def extra_flop_fraction(rank: int, d_in: int, d_out: int) -> float:
    """LoRA flops per token over base flops per token: r (d_in + d_out) / (d_in d_out)."""
    return rank * (d_in + d_out) / (d_in * d_out)


def step_work(wl: wk.Workload, ids: np.ndarray, ranks: np.ndarray, int4: bool = False):
    """(base bytes, lora bytes, flops, t_roof seconds) of one step."""
    bb = lb = fl = 0
    t_roof = 0.0
    for m in wl.modules:
        b1 = base_bytes(ids.shape[0], m.d_in, m.d_out, int4)
        l1 = lora_bytes(ids, ranks, m.d_in, m.d_out)
        f1 = flops(ids, ranks, m.d_in, m.d_out)
        bb += b1
        lb += l1
        fl += f1
        t_roof += max((b1 + l1) / (HBM_PEAK_GBS * 1e9), f1 / (MFMA_BF16_PEAK_TFS * 1e12))
    return bb, lb, fl, t_roof


# ---------------------------------------------------------------------------
# GPU set-up
# ---------------------------------------------------------------------------
def q4_weight(wl: wk.Workload, module: int, seed: int, torch):
    """A synthetic INT4 base weight of the module's shape in the device layout:
    random 4-bit codes (every 32-bit word is eight valid codes), zero points in
    4..11 and bf16 scales ~ |N(0.0045, 0.001)| (so the dequantized weight has a
    standard deviation near 0.02, like the bf16 weights)."""
    m = wl.modules[module]
    g = torch.Generator(device="cuda")
    g.manual_seed(wk.derive_seed(wl.key, seed, "q4", module) & 0x7FFFFFFF)
    Wq = torch.randint(-2 ** 31, 2 ** 31 - 1, (m.d_out, m.d_in // 8), generator=g, device="cuda",
                       dtype=torch.int64).to(torch.int32)
    s = (torch.randn((m.d_out, m.d_in // 128), generator=g, device="cuda") * 0.001 + 0.0045).abs()
    sbits = s.to(torch.bfloat16).view(torch.int16).to(torch.int32) & 0xFFFF
    z = torch.randint(4, 12, (m.d_out, m.d_in // 128), generator=g, device="cuda", dtype=torch.int32)
    return Wq, (sbits | (z << 16)).contiguous()


class Replica:
    """One independent copy of the workload's resident state."""

    def __init__(self, wl: wk.Workload, seed: int, torch, hrg, int4: bool = False, packed: bool = True):
        self.ids_np = wk.adapter_ids(wl, seed)
        self.ranks = wk.adapter_ranks(wl, seed)
        self.T = wl.T
        mods = wl.modules
        self.pool = hrg.LoraPool(wl.n_adapters, wl.n_adapters, wl.max_rank,
                                 [m.d_in for m in mods], [m.d_out for m in mods], wl.T)
        for i in range(wl.n_adapters):
            r = int(self.ranks[i])
            A, B = [], []
            for j in range(len(mods)):
                a, b = wk.adapter_weights(wl, i, j, r, seed, "cuda")
                A.append(a)
                B.append(b)
            self.pool.load_adapter(i, r, wk.adapter_alpha(wl, r), A, B)
            del A, B
        self.ids = torch.as_tensor(self.ids_np, device="cuda")
        self.X = {}
        for m in mods:
            if m.input_group not in self.X:
                self.X[m.input_group] = wk.activation(wl, m.input_group, m.d_in, seed, "cuda")
        self.int4 = int4
        if int4:
            self.W = None
            self.Wq = [q4_weight(wl, j, seed, torch) for j in range(len(mods))]
            big = max(m.d_in * m.d_out for m in mods)
            self.scratch = torch.empty(big, dtype=torch.bfloat16, device="cuda") \
                if wl.T > DECODE_MAX_T else None
        else:
            self.W = [wk.base_weight(wl, j, seed, "cuda") for j in range(len(mods))]
        # decode batches stream the base weights in the decode kernels' fragment
        # tiles (packed once, like a model's weights at load time)
        self.Wp = [self.pool.pack_weight(w) for w in self.W] \
            if packed and not int4 and wl.T <= DECODE_MAX_T else None
        self.out = [torch.empty((wl.T, m.d_out), dtype=torch.bfloat16, device="cuda")
                    for m in mods]
        self.xin = [self.X[m.input_group] for m in mods]
        self.groups = input_groups(wl)
        self.plan = self.pool.plan_create()
        self.pool.plan(self.ids, self.T, self.plan)


def input_groups(wl: wk.Workload):
    """The workload's linears in call order, those that read one X together
    (at most 8 per group, in order of first appearance): for a Llama layer
    [q, k, v], [o], [gate, up], [down]."""
    groups, where = [], {}
    for j, m in enumerate(wl.modules):
        k = where.get(m.input_group)
        if k is None or len(groups[k]) == 8:
            where[m.input_group] = len(groups)
            groups.append([j])
        else:
            groups[k].append(j)
    return groups


# Up to 64 tokens (decode) one launch pair groups the batch itself, so a
# step is just the applies; larger batches build one plan per step and every
# linear of the step reuses it.
DECODE_MAX_T = 64


def _apply_group(rep: Replica, hrg, g, plan):
    if rep.Wp is not None:
        hrg.lora_apply_group_packed(rep.pool.handle, g, rep.xin[g[0]], rep.ids, rep.T, [rep.Wp[j] for j in g],
                                    [rep.out[j] for j in g])
    elif rep.int4:
        hrg.lora_apply_group_q4(rep.pool.handle, g, rep.xin[g[0]], rep.ids, rep.T, [rep.Wq[j][0] for j in g],
                                [rep.Wq[j][1] for j in g], rep.scratch, [rep.out[j] for j in g], plan)
    else:
        hrg.lora_apply_group(rep.pool.handle, g, rep.xin[g[0]], rep.ids, rep.T, [rep.W[j] for j in g],
                             [rep.out[j] for j in g], plan)


def _base_group(rep: Replica, hrg, g):
    if rep.Wp is not None:
        hrg.lora_base_apply_group_packed(rep.pool.handle, g, rep.xin[g[0]], rep.T, [rep.Wp[j] for j in g],
                                         [rep.out[j] for j in g])
    elif rep.int4:
        hrg.lora_base_apply_group_q4(rep.pool.handle, g, rep.xin[g[0]], rep.T, [rep.Wq[j][0] for j in g],
                                     [rep.Wq[j][1] for j in g], rep.scratch, [rep.out[j] for j in g])
    else:
        hrg.lora_base_apply_group(rep.pool.handle, g, rep.xin[g[0]], rep.T, [rep.W[j] for j in g],
                                  [rep.out[j] for j in g])


def lora_step(rep: Replica, hrg):
    plan = None
    if rep.T > DECODE_MAX_T:
        hrg.lora_plan(rep.pool.handle, rep.ids, rep.T, rep.plan)
        plan = rep.plan
    for g in rep.groups:
        _apply_group(rep, hrg, g, plan)


def apply_only(rep: Replica, hrg):
    """The step without its plan launch (identical to lora_step at decode)."""
    plan = rep.plan if rep.T > DECODE_MAX_T else None
    for g in rep.groups:
        _apply_group(rep, hrg, g, plan)


def base_step(rep: Replica, hrg):
    for g in rep.groups:
        _base_group(rep, hrg, g)


def per_linear_step(rep: Replica, hrg):
    """The step as one lora_apply per linear (no grouping of shared inputs)."""
    plan = None
    if rep.T > DECODE_MAX_T:
        hrg.lora_plan(rep.pool.handle, rep.ids, rep.T, rep.plan)
        plan = rep.plan
    for j in range(len(rep.out)):
        if rep.int4:
            hrg.lora_apply_q4(rep.pool.handle, j, rep.xin[j], rep.ids, rep.T, rep.Wq[j][0], rep.Wq[j][1],
                              rep.scratch, rep.out[j], plan)
        else:
            hrg.lora_apply(rep.pool.handle, j, rep.xin[j], rep.ids, rep.T, rep.W[j], rep.out[j], plan)


def measured_traffic(workload_name: str):
    """HBM bytes per step recorded for this workload by rocprofv3 FETCH_SIZE +
    WRITE_SIZE runs (profiles/*_pmc_traffic.md), if the decode kernel source
    is unchanged since the counters were taken; else None."""
    import glob
    import hashlib
    import re
    try:
        src_hash = hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()
    except OSError:
        return None
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*_pmc_traffic.md"))):
        text = open(path).read()
        m = re.search(r"traffic_bytes_per_step:\s*(\d+)\s+workload:\s*(\S+)\s+source_sha256:\s*([0-9a-f]+)",
                      text)
        if m and m.group(2) == workload_name and m.group(3) == src_hash:
            return int(m.group(1))
    return None


def time_steps(fn, reps, steps: int, warmup: int, torch, hrg):
    """Per-step seconds over `steps` steps (rotating replicas), each step
    between two events on the current stream; returns (median, mean)."""
    for i in range(warmup):
        fn(reps[i % len(reps)], hrg)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        fn(reps[i % len(reps)], hrg)
        ev[i + 1].record()
    torch.cuda.synchronize()
    t = np.array([ev[i].elapsed_time(ev[i + 1]) * 1e-3 for i in range(steps)])
    return float(np.median(t)), float(t.mean())


def time_launches(rep, hrg, torch, rounds: int = 5):
    """Mean seconds of each grouped apply of the step, called eagerly with an
    event pair around every call (the launch pair decode_main +
    decode_combine at decode); returns the list per group."""
    plan = rep.plan if rep.T > DECODE_MAX_T else None
    if plan is not None:
        hrg.lora_plan(rep.pool.handle, rep.ids, rep.T, rep.plan)
    for g in rep.groups:          # warm
        _apply_group(rep, hrg, g, plan)
    torch.cuda.synchronize()
    acc = np.zeros(len(rep.groups))
    for _ in range(rounds):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * len(rep.groups))]
        for k, g in enumerate(rep.groups):
            ev[2 * k].record()
            _apply_group(rep, hrg, g, plan)
            ev[2 * k + 1].record()
        torch.cuda.synchronize()
        acc += np.array([ev[2 * k].elapsed_time(ev[2 * k + 1]) * 1e-3 for k in range(len(rep.groups))])
    return list(acc / rounds)


def capture(fn, rep, torch, hrg):
    """The step `fn` on `rep` captured as one hipGraph (after an eager warm-up
    on the capture stream); the decode path records kernel launches only."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(rep, hrg)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn(rep, hrg)
    torch.cuda.synchronize()
    return g


def graphed(fn, reps, torch, hrg):
    """A step function that replays `fn` captured per replica."""
    graphs = {id(rp): capture(fn, rp, torch, hrg) for rp in reps}
    return lambda rp, _hrg: graphs[id(rp)].replay()


# ---------------------------------------------------------------------------
# host <-> device paging (a separate measurement, not the contract line)
# ---------------------------------------------------------------------------
def paging_batches(wl: wk.Workload, n: int, mix: str, seed: int):
    """`n` fresh batches of the workload's T ids over its adapters: "uniform"
    (each id uniform) or "hot5" (5 hot adapters take 80 % of the tokens, the
    rest uniform over the others)."""
    g = np.random.Generator(np.random.PCG64(seed))
    out = []
    for _ in range(n):
        if mix == "uniform":
            ids = g.integers(0, wl.n_adapters, size=wl.T)
        else:
            hot = g.random(wl.T) < 0.8
            ids = np.where(hot, g.integers(0, 5, size=wl.T),
                           g.integers(5, wl.n_adapters, size=wl.T))
        out.append(ids.astype(np.int32))
    return out


def paging_bench(args, torch, hrg) -> dict:
    """One linear of the decode workload served from a host cache holding
    every adapter and a device pool of `slots` slots: each step is one
    lora_prefetch of a fresh batch plus its lora_apply, timed against the same
    batches with every adapter resident."""
    wl = wk.WORKLOADS[args.workload]
    if wl.T > DECODE_MAX_T or len(wl.modules) != 1:
        raise SystemExit("--paging measures a one-linear decode workload (1 or 2)")
    m = wl.modules[0]
    ranks = wk.adapter_ranks(wl, wl.default_seed)
    res = {"workload": wl.name, "slots": args.paging_slots, "host_cached": wl.n_adapters,
           "mix": args.paging_mix, "steps": args.steps}
    paged = hrg.LoraPool(args.paging_slots, wl.n_adapters, wl.max_rank, [m.d_in], [m.d_out], wl.T)
    paged.host_cache_create(wl.n_adapters)
    resident = hrg.LoraPool(wl.n_adapters, wl.n_adapters, wl.max_rank, [m.d_in], [m.d_out], wl.T)
    for i in range(wl.n_adapters):
        r = int(ranks[i])
        a, b = wk.adapter_weights(wl, i, 0, r, wl.default_seed, "cuda")
        paged.host_register(i, r, wk.adapter_alpha(wl, r), [a], [b])
        resident.load_adapter(i, r, wk.adapter_alpha(wl, r), [a], [b])
    if args.paging_mix == "hot5":
        for i in range(5):
            paged.pin(i, True)
    X = wk.activation(wl, m.input_group, m.d_in, wl.default_seed, "cuda")
    W = wk.base_weight(wl, 0, wl.default_seed, "cuda")
    out = torch.empty((wl.T, m.d_out), dtype=torch.bfloat16, device="cuda")
    n = args.warmup + args.steps
    batches = paging_batches(wl, n, args.paging_mix, 7)
    ids_dev = [torch.as_tensor(b, device="cuda") for b in batches]
    ids_host = [b.tolist() for b in batches]

    def run(pool, lo, hi, prefetch):
        for k in range(lo, hi):
            if prefetch:
                pool.prefetch(ids_host[k])
            hrg.lora_apply(pool.handle, 0, X, ids_dev[k], wl.T, W, out, None)

    for pool, prefetch, key in ((paged, True, "paged"), (resident, False, "resident")):
        run(pool, 0, args.warmup, prefetch)
        torch.cuda.synchronize()
        _, loads0, _ = paged.paging_stats()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        run(pool, args.warmup, n, prefetch)
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        res[f"{key}_us_per_step"] = round(e0.elapsed_time(e1) * 1e3 / args.steps, 2)
        res[f"{key}_wall_us_per_step"] = round(wall * 1e6 / args.steps, 2)
        if prefetch:
            _, loads1, page_bytes = paged.paging_stats()
            res["loads_per_step"] = round((loads1 - loads0) / args.steps, 2)
            res["h2d_bytes_per_step"] = round((loads1 - loads0) * page_bytes / args.steps)
    for pool in (paged, resident):
        st = pool.status()
        if st != "OK":
            raise RuntimeError(f"device status {st}")
    extra = (res["paged_us_per_step"] - res["resident_us_per_step"]) * 1e-6
    res["h2d_GBps_over_extra_time"] = round(res["h2d_bytes_per_step"] / extra / 1e9, 2) \
        if extra > 0 else None
    res["distinct_per_batch"] = round(float(np.mean([len(set(b.tolist())) for b in batches])), 2)
    paged.close()
    resident.close()
    return res


# ---------------------------------------------------------------------------
# adapter chains and target sets (separate measurements, not the contract line)
# ---------------------------------------------------------------------------
def _event_time(fn, steps: int, warmup: int, torch) -> float:
    """Seconds per call of fn() over `steps` calls between two synchronisations."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / steps


def chains_bench(args, torch, hrg) -> dict:
    """The q_proj decode linear with 200 rank-16 adapters plus 100 chains of two
    of them (ids 200..299, rank 16 + 16): a batch over all 300 ids against a
    batch over the 200 plain ids and the base-only call."""
    wl = wk.WORKLOADS[2]
    m = wl.modules[0]
    n_ad, n_ch = wl.n_adapters, 100
    pool = hrg.LoraPool(n_ad + n_ch, n_ad + n_ch, 32, [m.d_in], [m.d_out], wl.T)
    for i in range(n_ad):
        a, b = wk.adapter_weights(wl, i, 0, 16, wl.default_seed, "cuda")
        pool.load_adapter(i, 16, 32.0, [a], [b])
    g = np.random.Generator(np.random.PCG64(wk.derive_seed(wl.key, "chains")))
    for c in range(n_ch):
        pool.load_chain(n_ad + c, [int(x) for x in g.choice(n_ad, size=2, replace=False)])
    X = wk.activation(wl, m.input_group, m.d_in, wl.default_seed, "cuda")
    W = wk.base_weight(wl, 0, wl.default_seed, "cuda")
    out = torch.empty((wl.T, m.d_out), dtype=torch.bfloat16, device="cuda")
    ids_mixed = torch.as_tensor(g.integers(0, n_ad + n_ch, wl.T).astype(np.int32), device="cuda")
    ids_plain = torch.as_tensor(g.integers(0, n_ad, wl.T).astype(np.int32), device="cuda")
    res = {"workload": wl.name + "+100-chains-of-2", "T": wl.T, "steps": args.steps}
    for key, ids in (("mixed_chain_batch", ids_mixed), ("plain_batch", ids_plain)):
        t = _event_time(lambda: hrg.lora_apply(pool.handle, 0, X, ids, wl.T, W, out, None),
                        args.steps, args.warmup, torch)
        res[f"{key}_us"] = round(t * 1e6, 2)
    res["chain_tokens"] = int((ids_mixed >= n_ad).sum())
    t = _event_time(lambda: hrg.lora_base_apply(pool.handle, 0, X, wl.T, W, out),
                    args.steps, args.warmup, torch)
    res["base_only_us"] = round(t * 1e6, 2)
    if pool.status() != "OK":
        raise RuntimeError("device status")
    pool.close()
    return res


def target_sets_bench(args, torch, hrg) -> dict:
    """One Llama-2-7B decode layer (the seven linears of the 32-layer step,
    T = 64, 200 rank-16 adapters, uniform ids): every adapter targeting all
    seven linears, against even-numbered adapters targeting only q and v
    (the others still all seven), in a direct-mapped and a slot-table pool."""
    wl = wk.WORKLOADS[5]
    mods = wl.modules[:7]
    res = {"workload": "llama2-7b-decode-layer-T64-200xr16", "T": wl.T, "steps": args.steps}
    X = {}
    for mm in mods:
        if mm.input_group not in X:
            X[mm.input_group] = wk.activation(wl, mm.input_group, mm.d_in, wl.default_seed, "cuda")
    W = [wk.base_weight(wl, j, wl.default_seed, "cuda") for j in range(7)]
    out = [torch.empty((wl.T, mm.d_out), dtype=torch.bfloat16, device="cuda") for mm in mods]
    ids = torch.as_tensor(wk.adapter_ids(wl, wl.default_seed), device="cuda")
    # a direct-mapped pool (ids = slots) and a slot-table pool (max_ids > slots)
    for key, qv_only, max_ids in (("all_seven", False, wl.n_adapters),
                                  ("even_ids_q_v_only", True, wl.n_adapters),
                                  ("all_seven_slot_table", False, 256),
                                  ("even_ids_q_v_only_slot_table", True, 256)):
        pool = hrg.LoraPool(wl.n_adapters, max_ids, 16, [mm.d_in for mm in mods],
                            [mm.d_out for mm in mods], wl.T)
        for i in range(wl.n_adapters):
            A, B = [], []
            for j in range(7):
                if qv_only and i % 2 == 0 and j not in (0, 2):
                    A.append(None)
                    B.append(None)
                    continue
                a, b = wk.adapter_weights(wl, i, j, 16, wl.default_seed, "cuda")
                A.append(a)
                B.append(b)
            pool.load_adapter(i, 16, 32.0, A, B)

        def step():
            for j in range(7):
                hrg.lora_apply(pool.handle, j, X[mods[j].input_group], ids, wl.T, W[j], out[j], None)
        res[f"{key}_layer_us"] = round(_event_time(step, args.steps, args.warmup, torch) * 1e6, 2)
        if pool.status() != "OK":
            raise RuntimeError("device status")
        if key == "all_seven":
            def base():
                for j in range(7):
                    hrg.lora_base_apply(pool.handle, j, X[mods[j].input_group], wl.T, W[j], out[j])
            res["base_only_layer_us"] = round(_event_time(base, args.steps, args.warmup, torch) * 1e6, 2)
        pool.close()
    return res


# ---------------------------------------------------------------------------
# CPU oracle baseline
# ---------------------------------------------------------------------------
def host_info() -> dict:
    """nproc, the threads this process may run on, and the CPU model name."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {"nproc": os.cpu_count(), "affinity": affinity, "cpu_model": model}


def _blas_threads() -> int:
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        return max(int(i.get("num_threads", 1)) for i in info) if info else 1
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def _oracle_rate(wl: wk.Workload, ids_np, ranks, X, W, n_sample: int, seconds: float, seed: int):
    """Linears per second of the oracle over the first n_sample linears of
    `wl` (X, W: host tensors per linear), run for about `seconds`.  The
    adapters are drawn on the GPU, as the library's were, and copied back."""
    import oracle
    mods = wl.modules[:n_sample]
    reg = oracle.Registry(wl.n_adapters, wl.n_adapters, wl.max_rank, [m.d_in for m in mods],
                          [m.d_out for m in mods], wl.T)
    for i in wk.distinct_adapters(ids_np):
        r = int(ranks[i])
        A, B = [], []
        for j in range(n_sample):
            a, b = wk.adapter_weights(wl, i, j, r, seed, "cuda")
            A.append(a.cpu())
            B.append(b.cpu())
        reg.load(i, r, wk.adapter_alpha(wl, r), A, B)
    n_lin = 0
    t0 = time.perf_counter()
    while True:
        j = n_lin % n_sample
        oracle.lora_linear(reg, j, X[j], ids_np, W[j])
        n_lin += 1
        el = time.perf_counter() - t0
        if (el >= seconds and n_lin % n_sample == 0) or el >= 4 * seconds:
            break
    return n_lin, el


def cpu_baseline(wl: wk.Workload, rep: Replica, seconds: float, torch):
    """The oracle (float64 numpy, the base product through numpy's BLAS) timed
    on the host over a bounded sample: the linears of the first layer (all of
    them for one-layer workloads), repeated for about `seconds`, scaled to
    whole steps; plus the toy workload on one core."""
    n_sample = min(7, len(wl.modules))
    # the oracle sees the same bf16 bits as the GPU (copies of the replica's)
    X = [x.cpu() for x in rep.xin[:n_sample]]
    W = [w.cpu() for w in rep.W[:n_sample]]
    threads = _blas_threads()
    n_lin, el = _oracle_rate(wl, rep.ids_np, rep.ranks, X, W, n_sample, seconds, wl.default_seed)
    t_step = el / (n_lin / n_sample) * (len(wl.modules) / n_sample)
    out = {"value": round(wl.T / t_step, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"{n_lin} linears ({n_lin / n_sample:.2f} passes over the first {n_sample} "
                     f"of the {len(wl.modules)} linears of workload '{wl.name}', {wl.T} tokens) "
                     f"in {el:.1f} s, float64 numpy on {threads} BLAS threads; scaled to a whole step"}
    out.update(host_info())
    # one core, the toy workload (1024 -> 1024, 64 tokens, 4 rank-8 adapters)
    try:
        import threadpoolctl
        w1 = wk.WORKLOADS[1]
        ids1, ranks1 = wk.adapter_ids(w1), wk.adapter_ranks(w1)
        X1 = [wk.activation(w1, w1.modules[0].input_group, w1.modules[0].d_in, device="cuda").cpu()]
        W1 = [wk.base_weight(w1, 0, device="cuda").cpu()]
        with threadpoolctl.threadpool_limits(1):
            n1, el1 = _oracle_rate(w1, ids1, ranks1, X1, W1, 1, 2.0, w1.default_seed)
        out["one_core_toy"] = {"value": round(w1.T * n1 / el1, 1), "unit": "tokens/s",
                               "workload": w1.name, "linears": n1, "seconds": round(el1, 2)}
    except Exception as e:  # pragma: no cover
        out["one_core_toy"] = f"unavailable: {e}"
    return out


# ---------------------------------------------------------------------------
# chip peaks (measured denominators printed beside the published ones)
# ---------------------------------------------------------------------------
def peaks(torch, steps: int = 20) -> dict:
    """A streaming read of a 4 GiB device buffer and a register-resident bf16
    MFMA loop, both timed with events over `steps` launches."""
    import ctypes as C
    import heterogeneous_rank_gemm_amd as hrg
    lib = C.CDLL(hrg._lora.LIB_PATH)
    lib.hrg_probe_read.argtypes = [C.c_void_p, C.c_size_t, C.c_void_p, C.c_int, C.c_void_p]
    lib.hrg_probe_mfma.argtypes = [C.c_int, C.c_void_p, C.c_int, C.c_void_p]
    s = torch.cuda.current_stream().cuda_stream
    n = 4 << 30
    buf = torch.ones(n // 4, dtype=torch.int32, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    res = {"cus": cus}
    best = 0.0
    for blocks in (cus * 4, cus * 8, cus * 16):
        sink = torch.zeros(blocks * 4, dtype=torch.int32, device="cuda")
        for _ in range(3):
            assert lib.hrg_probe_read(buf.data_ptr(), n, sink.data_ptr(), blocks, s) == 0
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            lib.hrg_probe_read(buf.data_ptr(), n, sink.data_ptr(), blocks, s)
        e1.record()
        torch.cuda.synchronize()
        gbs = n * steps / (e0.elapsed_time(e1) * 1e-3) / 1e9
        res[f"read_GBps_{blocks}_blocks"] = round(gbs, 1)
        best = max(best, gbs)
    res["hbm_read_GBps"] = round(best, 1)
    res["hbm_spec_GBps"] = HBM_PEAK_GBS
    del buf
    iters, blocks = 4096, cus * 8
    sink = torch.zeros(blocks * 256, dtype=torch.float32, device="cuda")
    lib.hrg_probe_mfma(iters, sink.data_ptr(), blocks, s)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        lib.hrg_probe_mfma(iters, sink.data_ptr(), blocks, s)
    e1.record()
    torch.cuda.synchronize()
    flop = blocks * 4 * iters * 4 * 32768.0 * steps
    res["mfma_bf16_TFLOPs"] = round(flop / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)
    res["mfma_bf16_spec_TFLOPs"] = MFMA_BF16_PEAK_TFS
    return res


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=5, choices=sorted(wk.WORKLOADS))
    ap.add_argument("--rotate", type=int, default=8, help="independent copies of the state")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", choices=["auto", "on", "off"], default="auto",
                    help="replay each step as one captured hipGraph (auto: for multi-linear "
                         "decode steps)")
    ap.add_argument("--phase", choices=["all", "lora", "base", "linear"], default="all",
                    help="time only the LoRA step, the base-only step or the per-linear step "
                         "(for profiling)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (x steps), to scale "
                         "the rocprofv3 FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--peaks", action="store_true",
                    help="measure the chip's streaming-read GB/s and bf16 MFMA TFLOP/s instead")
    ap.add_argument("--layout", choices=["packed", "row"], default="packed",
                    help="decode batches: base weights in fragment tiles (lora_pack_weight) or "
                         "row-major")
    ap.add_argument("--int4", action="store_true",
                    help="INT4 (group 128) base weights instead of bf16 (lora_apply_group_q4)")
    ap.add_argument("--chains", action="store_true",
                    help="measure adapter chains instead (prints its own JSON line)")
    ap.add_argument("--target-sets", action="store_true",
                    help="measure per-adapter target sets instead (prints its own JSON line)")
    ap.add_argument("--paging", action="store_true",
                    help="measure host-cache paging instead (prints its own JSON line)")
    ap.add_argument("--paging-slots", type=int, default=64, help="device slots of the paged pool")
    ap.add_argument("--paging-mix", choices=["uniform", "hot5"], default="uniform")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the library has no multi-GPU path); "
              f"got --gpus {args.gpus}", file=sys.stderr)
        return 2

    import torch
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n,
                          "launches": args.steps}), flush=True)
        return 0
    import heterogeneous_rank_gemm_amd as hrg

    if args.peaks:
        print(json.dumps({"peaks": peaks(torch)}), flush=True)
        return 0
    if args.paging:
        print(json.dumps({"paging": paging_bench(args, torch, hrg)}), flush=True)
        return 0
    if args.chains:
        print(json.dumps({"chains": chains_bench(args, torch, hrg)}), flush=True)
        return 0
    if args.target_sets:
        print(json.dumps({"target_sets": target_sets_bench(args, torch, hrg)}), flush=True)
        return 0

    wl = wk.WORKLOADS[args.workload]
    R = 1 if wl.key == 5 else max(1, args.rotate)
    print(f"[bench] workload {wl.key} '{wl.name}', {R} replica(s)", file=sys.stderr, flush=True)
    reps = [Replica(wl, wl.default_seed + 1000 * r if r else wl.default_seed, torch, hrg, args.int4,
                    args.layout == "packed") for r in range(R)]
    torch.cuda.synchronize()
    print("[bench] state resident; timing", file=sys.stderr, flush=True)

    use_graph = args.graph == "on" or (args.graph == "auto" and wl.T <= DECODE_MAX_T
                                       and len(wl.modules) > 1)
    f_lora, f_apply, f_base, f_lin = lora_step, apply_only, base_step, per_linear_step
    if use_graph:
        print("[bench] capturing the steps as hipGraphs", file=sys.stderr, flush=True)
        f_lora = graphed(lora_step, reps, torch, hrg)
        f_apply = f_lora if wl.T <= DECODE_MAX_T else graphed(apply_only, reps, torch, hrg)
        f_base = graphed(base_step, reps, torch, hrg)
        if args.phase in ("all", "linear") and len(wl.modules) > 1:
            f_lin = graphed(per_linear_step, reps, torch, hrg)
    if args.phase != "all":
        fn = {"lora": f_lora, "base": f_base, "linear": f_lin}[args.phase]
        t_med, t_mean = time_steps(fn, reps, args.steps, args.warmup, torch, hrg)
        print(json.dumps({"phase": args.phase, "ms_per_step": t_med * 1e3, "mean_ms": t_mean * 1e3}),
              flush=True)
        return 0
    t_step, t_step_mean = time_steps(f_lora, reps, args.steps, args.warmup, torch, hrg)
    t_apply, _ = time_steps(f_apply, reps, args.steps, args.warmup, torch, hrg)
    t_base, t_base_mean = time_steps(f_base, reps, args.steps, args.warmup, torch, hrg)
    t_lin = None
    if len(wl.modules) > 1 and len(reps[0].groups) < len(wl.modules):
        t_lin, _ = time_steps(f_lin, reps, args.steps, args.warmup, torch, hrg)
    warm = None
    if R > 1:
        # one copy, so the Infinity Cache holds what it can (labelled warm)
        w_step, _ = time_steps(f_lora, reps[:1], args.steps, args.warmup, torch, hrg)
        w_base, _ = time_steps(f_base, reps[:1], args.steps, args.warmup, torch, hrg)
        warm = {"ms_per_step": round(w_step * 1e3, 5), "base_only_ms_per_step": round(w_base * 1e3, 5)}
    t_groups = time_launches(reps[0], hrg, torch)
    for rp in reps:
        st = rp.pool.status()
        if st != "OK":
            raise RuntimeError(f"device status {st}")

    works = [step_work(wl, rp.ids_np, rp.ranks, args.int4) for rp in reps]
    bb = float(np.mean([w[0] for w in works]))
    lb = float(np.mean([w[1] for w in works]))
    fl = float(np.mean([w[2] for w in works]))
    t_roof = float(np.mean([w[3] for w in works]))
    hbm_bound = (bb + lb) / (HBM_PEAK_GBS * 1e9) >= fl / (MFMA_BF16_PEAK_TFS * 1e12)
    # the dominant kernels, measured live: their algorithmic work over the
    # time of their launches in one step.  A step holds nothing but those
    # launches (the decode launch pairs; or the plan, shrink, small-segment
    # and GEMM launches), so the step's own events time them: replayed as a
    # graph they run back to back (rocprofv3's kernel times sum to the step
    # within 1 %), eagerly with the dispatch gaps between them.  Each grouped
    # apply timed alone between its own events (eager) is reported beside it.
    b0, l0, f0, _ = works[0]
    n_calls = len(reps[0].groups)
    t_eager = float(np.sum(t_groups))
    t_calls = t_step
    decode = wl.T <= DECODE_MAX_T
    kernel = ("decode_main + decode_combine: one launch pair per grouped apply, "
              f"{n_calls} calls per step" if decode else
              "shrink_kernel + expand_small_kernel + prefill_kernel per linear, plan_kernel per step")
    if hbm_bound:
        achieved = (b0 + l0) / t_calls / 1e9
        traffic = measured_traffic(wl.name) if decode and not args.int4 else None
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": kernel, "algorithmic_bytes_per_step": round(b0 + l0),
                "launch_seconds_per_step": t_calls, "eager_launch_seconds_per_step": t_eager,
                "calls_per_step": n_calls}
    else:
        achieved = f0 / t_calls / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFS, 4),
                "traffic": None, "kernel": kernel, "algorithmic_flops_per_step": round(f0),
                "launch_seconds_per_step": t_calls, "eager_launch_seconds_per_step": t_eager,
                "calls_per_step": n_calls}

    # the chip's measured peaks beside the published ones (the same probes as
    # --peaks), and the dominant unit's fraction of the measured one
    print("[bench] peak probes", file=sys.stderr, flush=True)
    pk = peaks(torch)
    if hbm_bound:
        roof["measured_peak"] = pk["hbm_read_GBps"]
    else:
        roof["measured_peak"] = pk["mfma_bf16_TFLOPs"]
    roof["frac_of_measured_peak"] = round(achieved / roof["measured_peak"], 4)

    cpu = None
    if not args.no_cpu_baseline and not args.int4:
        print("[bench] cpu oracle baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, reps[0], args.cpu_seconds, torch)

    line = {
        "metric": METRIC,
        "value": round(wl.T / t_step, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 (int4 base weight)" if args.int4 else "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.T,
                   "modules": [[m.d_in, m.d_out] for m in wl.modules[:7]],
                   "n_linears": len(wl.modules), "adapters": wl.n_adapters,
                   "ranks": list(wl.rank_choices), "max_rank": wl.max_rank,
                   "replicas_rotated": R, "hipgraph": use_graph,
                   "calls_per_step": n_calls,
                   "base_weight": "int4-g128" if args.int4 else
                   ("bf16, fragment tiles" if reps[0].Wp is not None else "bf16, row-major")},
        "timing": f"median of {args.steps} steps (event pair per step) after {args.warmup} warm-up steps",
        "mean_ms_per_step": round(t_step_mean * 1e3, 5),
        "lora_overhead_pct": round(100.0 * (t_step - t_base) / t_base, 2),
        "base_only_ms_per_step": round(t_base * 1e3, 5),
        "apply_ms_per_step": round(t_apply * 1e3, 5),
        "per_linear_row_major_ms_per_step": round(t_lin * 1e3, 5) if t_lin else None,
        "warm": warm,
        "step_roofline_frac": round(t_roof / t_step, 4),
        "algorithmic": {"base_bytes": bb, "lora_bytes": lb, "flops": fl,
                        "t_roof_us": round(t_roof * 1e6, 3),
                        "lora_overhead_floor_pct": round(100.0 * lb / bb, 2) if hbm_bound else None},
        "roofline": roof,
        "measured_peaks": pk,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    for rp in reps:
        rp.pool.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
