"""CPU oracle for the heterogeneous-batch LoRA-augmented linear layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call this module.
The product path (the HIP library and its binding) never touches it, and
this module imports nothing from the product: the two share no code.

It is a plain, slow, obviously correct numpy implementation in float64.
bf16 inputs are widened exactly (bf16 -> f64 is exact), products of two bf16
values are exact in f64, and only the sums round, so the result is the exact
value of the definition to within ~1e-15 relative.  It is *not* rounded to
bf16: the GPU's bf16 output is compared against it.

Pages cited:
  [LoRA-Land]  "LoRA-Land: turning the LLM into an operating system with
               hot-pluggable multi-task fine-tuned serving" (blog.itodd.wang)
  [vLLM-ch7]   "Multi-LoRA hot-plug: one model serving many tenants"
               (gufacode.com, vLLM chapter 7)
  [icman]      field report on Multi-LoRA in managed inference
               (icman.com.cn news 62580)

What it computes (the readings taken where the pages are garbled):
  * [LoRA-Land] section "2. multi-LoRA batch scheduling" gives the update as
    Y = X W_base^T plus the product X A B, with X A evaluated first into a
    rank-r intermediate.  [vLLM-ch7] "LoRA at a glance" gives the shapes as
    A (d x r) and B (r x d) and says r is usually 8..64.  Reading: W is
    d_out x d_in, A is d_in x r, B is r x d_out, and
        Y[t, :] = X[t, :] W^T + s_i * (X[t, :] A_i) B_i,   i = ids[t].
  * The scale s_i = alpha_i / r_i: [vLLM-ch7] "training a vLLM-compatible
    LoRA" configures lora_alpha=32 at r=16, and [icman] section 3.2 says
    alpha is usually twice the rank and controls the scaling ratio.  The
    true rank is used, never a padded one.
  * id -1 means "no adapter, pure base" ([vLLM-ch7] "switching LoRA per
    request": a request naming no LoRA runs the plain base).
  * Dynamic batching applies to each sample its own low-rank branch and adds
    it back onto the main path ([icman] section 2.1), so the batch result is
    the per-token result; the oracle computes it token by token.
  * Strict mode ([icman] section 4.1): a request whose adapter cannot be
    found is rejected rather than silently served by the base; the whole
    call fails and produces no output.
  * A rank above the configured maximum is refused ([vLLM-ch7] "starting a
    multi-LoRA service", --max-lora-rank; [icman] section 3.3).
  * Target sets: an adapter adds its branch only on the linears it targets
    ([icman] section 2.1: the low-rank branch is added on the target linear
    layers; [vLLM-ch7] performance notes: adapters of one batch with
    different target_modules send some sequences down a skip path).  A
    module the adapter does not target is pure base for its tokens.
  * Grouping the batch by LoRA id ([LoRA-Land] section 2, "Grouped
    Multi-LoRA Execution") is read as a stable sort of token indices by
    (id ascending, original index ascending), -1 first, with the maximal
    runs of equal id as segments.
"""
from __future__ import annotations

from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

# Status names.  The oracle has its own vocabulary; tests map the library's
# numeric codes onto these names.
OK = "OK"
INVALID_ARG = "INVALID_ARG"
POOL_FULL = "POOL_FULL"
RANK = "RANK"
EXISTS = "EXISTS"
NOT_LOADED = "NOT_LOADED"
ID_RANGE = "ID_RANGE"


class OracleError(Exception):
    def __init__(self, status: str, msg: str = ""):
        super().__init__(f"{status}: {msg}")
        self.status = status


# --------------------------------------------------------------------------
# bf16 decoding (bf16 is the top half of an IEEE binary32)
# --------------------------------------------------------------------------
def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact float64 values of bf16 bit patterns (uint16/int16 array or a
    torch bf16 tensor)."""
    try:
        import torch
        if isinstance(bits, torch.Tensor):
            bits = bits.detach().cpu().contiguous().view(torch.int16).numpy()
    except ImportError:  # pragma: no cover
        pass
    b = np.asarray(bits).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# the adapter registry ([vLLM-ch7] "vLLM multi-LoRA": unified memory pool;
# [icman] section 2.1: the adapter routing table)
# --------------------------------------------------------------------------
class Adapter:
    __slots__ = ("rank", "alpha", "scale", "A", "B")

    def __init__(self, rank: int, alpha: float, A: List[np.ndarray], B: List[np.ndarray]):
        self.rank = rank
        self.alpha = alpha
        self.scale = float(alpha) / float(rank)
        self.A = A  # per module, float64 [d_in x r]
        self.B = B  # per module, float64 [r x d_out]


class Registry:
    """Models what the pool must accept and reject.  Capacity is a count of
    resident adapters; ids are valid in [0, max_ids)."""

    def __init__(self, max_adapters: int, max_ids: int, max_rank: int,
                 d_in: Sequence[int], d_out: Sequence[int], max_tokens: int):
        if max_adapters < 1 or max_ids < 1 or not (1 <= max_rank <= 64):
            raise OracleError(INVALID_ARG, "pool sizes")
        if len(d_in) != len(d_out) or len(d_in) < 1:
            raise OracleError(INVALID_ARG, "module shapes")
        self.max_adapters = max_adapters
        self.max_ids = max_ids
        self.max_rank = max_rank
        self.d_in = list(d_in)
        self.d_out = list(d_out)
        self.max_tokens = max_tokens
        self.adapters: Dict[int, Adapter] = {}

    @property
    def n_modules(self) -> int:
        return len(self.d_in)

    def load(self, adapter_id: int, rank: int, alpha: float,
             A: Sequence, B: Sequence) -> None:
        """A[m] is d_in[m] x rank, B[m] is rank x d_out[m] (bf16 bits or floats)."""
        if not (0 <= adapter_id < self.max_ids):
            raise OracleError(ID_RANGE, f"id {adapter_id}")
        if not (1 <= rank <= self.max_rank):
            raise OracleError(RANK, f"rank {rank} outside [1, {self.max_rank}]")
        if adapter_id in self.adapters:
            raise OracleError(EXISTS, f"id {adapter_id} already loaded")
        if len(self.adapters) >= self.max_adapters:
            raise OracleError(POOL_FULL, "no free slot")
        if len(A) != self.n_modules or len(B) != self.n_modules:
            raise OracleError(INVALID_ARG, "one A and one B per module")
        As, Bs = [], []
        if all(A[m] is None and B[m] is None for m in range(self.n_modules)):
            raise OracleError(INVALID_ARG, "an adapter targets at least one module")
        for m in range(self.n_modules):
            if A[m] is None and B[m] is None:
                # the adapter does not target this module: tokens routed to it
                # take the skip path there ([vLLM-ch7] performance notes)
                As.append(None)
                Bs.append(None)
                continue
            if A[m] is None or B[m] is None:
                raise OracleError(INVALID_ARG, f"module {m}: A and B both given or both absent")
            a = _as_f64(A[m])
            b = _as_f64(B[m])
            if a.shape != (self.d_in[m], rank) or b.shape != (rank, self.d_out[m]):
                raise OracleError(INVALID_ARG, f"module {m} shapes {a.shape} {b.shape}")
            As.append(a)
            Bs.append(b)
        self.adapters[adapter_id] = Adapter(rank, alpha, As, Bs)

    def unload(self, adapter_id: int) -> None:
        if adapter_id not in self.adapters:
            raise OracleError(NOT_LOADED, f"id {adapter_id}")
        del self.adapters[adapter_id]

    def load_chain(self, chain_id: int, members: Sequence[int]) -> None:
        """A chain of loaded adapters under a new id ([LoRA-Land] "technical
        approach", item 3: LoRAs composed like a pipeline and applied in turn;
        section "3. hot-plug API and composition": set_adaptive_chain).  At a
        linear layer every member adds its own update, so the chain's term is
        the sum of the members' terms.  The members are snapshotted: unloading
        one later leaves the chain intact.  Limits: ids in range and loaded
        (NOT_LOADED), no repeats and no chains as members (INVALID_ARG), and
        the chain, an adapter of rank sum_c r_c, within the pool's max rank
        (RANK; [vLLM-ch7] "starting a multi-LoRA service", --max-lora-rank;
        [icman] section 3.3)."""
        if not (0 <= chain_id < self.max_ids):
            raise OracleError(ID_RANGE, f"id {chain_id}")
        members = [int(i) for i in members]
        if not members or len(set(members)) != len(members):
            raise OracleError(INVALID_ARG, "members: at least one, no repeats")
        for i in members:
            if not (0 <= i < self.max_ids):
                raise OracleError(ID_RANGE, f"member {i}")
        for i in members:
            if i not in self.adapters:
                raise OracleError(NOT_LOADED, f"member {i}")
            if isinstance(self.adapters[i], Chain):
                raise OracleError(INVALID_ARG, f"member {i} is a chain")
        ranks = [self.adapters[i].rank for i in members]
        if sum(ranks) > self.max_rank:
            raise OracleError(RANK, f"chain ranks {ranks} exceed max rank {self.max_rank}")
        if chain_id in self.adapters:
            raise OracleError(EXISTS, f"id {chain_id}")
        if len(self.adapters) >= self.max_adapters:
            raise OracleError(POOL_FULL, "no free slot")
        self.adapters[chain_id] = Chain([self.adapters[i] for i in members])

    def validate_ids(self, ids: np.ndarray) -> None:
        """Strict mode: every id is -1 or a loaded adapter; else the call fails.
        An out-of-range id is reported before an unloaded one."""
        ids = np.asarray(ids)
        for t in range(ids.shape[0]):
            i = int(ids[t])
            if i < -1 or i >= self.max_ids:
                raise OracleError(ID_RANGE, f"token {t} id {i}")
        for t in range(ids.shape[0]):
            i = int(ids[t])
            if i >= 0 and i not in self.adapters:
                raise OracleError(NOT_LOADED, f"token {t} id {i}")


class Chain:
    """Several adapters on one id: the sum of their low-rank terms."""
    __slots__ = ("members",)

    def __init__(self, members: List[Adapter]):
        self.members = list(members)


def _lora_term(ad, module: int, x: np.ndarray, cols=None) -> Optional[np.ndarray]:
    """s (x A) B of one adapter (x: one token row), the sum over a chain's
    members, or None when nothing targets the module."""
    if isinstance(ad, Chain):
        terms = [t for t in (_lora_term(m, module, x, cols) for m in ad.members) if t is not None]
        if not terms:
            return None
        acc = terms[0].copy()
        for t in terms[1:]:
            acc += t
        return acc
    if ad.A[module] is None:
        return None                                 # not a target of this adapter
    u = x @ ad.A[module]                            # shrink: d_in -> r
    B = ad.B[module] if cols is None else ad.B[module][:, cols]
    return ad.scale * (u @ B)                       # expand r -> d_out, scale


def _as_f64(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            if x.dtype == torch.bfloat16:
                return bf16_bits_to_f64(x)
            return x.detach().cpu().double().numpy()
    except ImportError:  # pragma: no cover
        pass
    x = np.asarray(x)
    if x.dtype in (np.uint16, np.int16):
        return bf16_bits_to_f64(x)
    return x.astype(np.float64)


# --------------------------------------------------------------------------
# grouping ([LoRA-Land] section 2: group the batch by LoRA id)
# --------------------------------------------------------------------------
def plan(ids: Sequence[int], max_ids: int):
    """Stable grouping of tokens by adapter id, written as a counting sort.

    Returns (perm, inv, seg_id, seg_off):
      perm[p]    original index of the token at sorted position p
      inv[t]     sorted position of token t   (inv[perm[p]] == p)
      seg_id[s]  adapter id of segment s (-1 first if present)
      seg_off    int32[S+1], segment s covers sorted positions
                 [seg_off[s], seg_off[s+1]); seg_off[S] == T
    """
    ids = [int(i) for i in ids]
    T = len(ids)
    for t, i in enumerate(ids):
        if i < -1 or i >= max_ids:
            raise OracleError(ID_RANGE, f"token {t} id {i}")
    # bucket b = id + 1, so -1 lands in bucket 0 and sorts first
    n_buckets = max_ids + 1
    count = [0] * n_buckets
    for i in ids:
        count[i + 1] += 1
    start = [0] * n_buckets
    running = 0
    for b in range(n_buckets):
        start[b] = running
        running += count[b]
    cursor = list(start)
    perm = [0] * T
    for t in range(T):          # ascending t: equal ids keep their order
        b = ids[t] + 1
        perm[cursor[b]] = t
        cursor[b] += 1
    inv = [0] * T
    for p in range(T):
        inv[perm[p]] = p
    seg_id: List[int] = []
    seg_off: List[int] = []
    for b in range(n_buckets):
        if count[b] > 0:
            seg_id.append(b - 1)
            seg_off.append(start[b])
    seg_off.append(T)
    return (np.asarray(perm, dtype=np.int32), np.asarray(inv, dtype=np.int32),
            np.asarray(seg_id, dtype=np.int32), np.asarray(seg_off, dtype=np.int32))


# --------------------------------------------------------------------------
# the linear ([LoRA-Land] section 2 formula; [icman] section 2.1 dynamic mode)
# --------------------------------------------------------------------------
def base_linear(X, W) -> np.ndarray:
    """Y0 = X W^T in float64 (X: T x d_in, W: d_out x d_in)."""
    return _as_f64(X) @ _as_f64(W).T


def lora_linear(reg: Registry, module: int, X, ids, W) -> np.ndarray:
    """Y[t,:] = X[t,:] W^T + s_i (X[t,:] A_i) B_i for every token t, i = ids[t].

    Raises OracleError (no output at all) if any id is out of range or not
    loaded.  Float64, unrounded."""
    ids = np.asarray(ids, dtype=np.int64)
    Xf = _as_f64(X)
    Wf = _as_f64(W)
    T = ids.shape[0]
    if Xf.shape != (T, reg.d_in[module]) or Wf.shape != (reg.d_out[module], reg.d_in[module]):
        raise OracleError(INVALID_ARG, "shapes")
    if T > reg.max_tokens:
        raise OracleError(INVALID_ARG, "T > max_tokens")
    reg.validate_ids(ids)
    Y = Xf @ Wf.T                                   # shared base path
    for t in range(T):                              # each token its own branch
        i = int(ids[t])
        if i < 0:
            continue                                # base only: no LoRA term
        term = _lora_term(reg.adapters[i], module, Xf[t, :])
        if term is not None:                        # None: not a target of this adapter
            Y[t, :] += term                         # added back onto the main path
    return Y


def lora_linear_sampled(reg: Registry, module: int, X_rows, ids_rows, W_cols,
                        cols: Optional[Sequence[int]] = None) -> np.ndarray:
    """The same definition on a sample: X_rows are the sampled tokens' rows,
    ids_rows their ids, W_cols the sampled output rows of W (len(cols) x d_in)
    and ``cols`` the output indices they stand for (all when None)."""
    ids_rows = np.asarray(ids_rows, dtype=np.int64)
    Xf = _as_f64(X_rows)
    Wf = _as_f64(W_cols)
    reg.validate_ids(ids_rows)
    cols = np.arange(reg.d_out[module]) if cols is None else np.asarray(cols)
    Y = Xf @ Wf.T
    for n in range(ids_rows.shape[0]):
        i = int(ids_rows[n])
        if i < 0:
            continue
        term = _lora_term(reg.adapters[i], module, Xf[n, :], cols)
        if term is not None:
            Y[n, :] += term
    return Y


def parity_metrics(out, Yref) -> Tuple[float, float, float]:
    """(max|out-Yref| / max|Yref|, sum|out-Yref| / sum|Yref|, mean element-wise
    relative error over |Yref| > 0).  ``out`` may be a bf16 tensor."""
    o = _as_f64(out)
    r = np.asarray(Yref, dtype=np.float64)
    d = np.abs(o - r)
    ar = np.abs(r)
    mx = float(d.max() / ar.max()) if ar.size and ar.max() > 0 else float(d.max(initial=0.0))
    rl1 = float(d.sum() / ar.sum()) if ar.sum() > 0 else float(d.sum())
    nz = ar > 0
    elem = float((d[nz] / ar[nz]).mean()) if nz.any() else 0.0
    return mx, rl1, elem


# Tolerances on bf16 outputs with fp32 accumulation.
MAX_REL_TOL = 1e-2   # max|out - Yref| <= 1e-2 * max|Yref|
RELL1_TOL = 2e-3     # sum|out - Yref| / sum|Yref| <= 2e-3


# --------------------------------------------------------------------------
# host <-> device paging of the pool ([vLLM-ch7] "how vLLM implements
# multi-LoRA", item 1: one device pool, adapters loaded on demand and swapped
# in and out; "starting a multi-LoRA service": --max-loras adapters resident
# on the GPU, --max-cpu-loras more kept in a CPU cache and swapped in on
# demand; [icman] section 2.2: an adapter that is not loaded is read into
# device memory, and when device memory runs short the least recently used
# inactive adapter is swapped out; a preload list keeps the hottest few
# resident)
# --------------------------------------------------------------------------
class PagedRegistry(Registry):
    """The pool with a host cache in front of it.

    Readings taken where the pages are silent:
      * Capacity: ``max_adapters`` device slots, shared by adapters loaded
        directly (never evicted) and host-cached adapters paged in.  The host
        cache holds ``max_cpu`` adapters; a full host cache refuses a new one
        (POOL_FULL) instead of forgetting an adapter.
      * A prefetch names the ids of the next batch.  Every host-cached id in
        it becomes addressable (paged in if it is not on the device); the
        host-cached ids of the previous prefetch that are not named again
        stop being addressable (strict mode then rejects them) but keep their
        device copy as a cache.
      * "Least recently used" counts prefetch calls: an id's last use is the
        number of the last prefetch that named it.  The victim is the cached,
        unpinned id not named by the current prefetch with the smallest
        (last use, id).  Misses take a free slot first.
      * Pinned ids (the preload list) are paged in when pinned, stay
        addressable and are never evicted.  Pinning does not count as a use;
        unpinning gives the id the recency of the latest prefetch (it was in
        use until then).  Pinning evicts only an id that is not addressable.
      * Unloading a host-cached id drops its device copy only.
      * If the misses of a prefetch outnumber the free slots plus the
        evictable ids, the call fails with POOL_FULL and changes nothing.

    ``self.adapters`` (the Registry's view) is always the addressable set, so
    ``lora_linear`` and ``validate_ids`` apply strict mode to it unchanged.
    """

    def __init__(self, max_adapters: int, max_ids: int, max_rank: int,
                 d_in: Sequence[int], d_out: Sequence[int], max_tokens: int, max_cpu: int):
        super().__init__(max_adapters, max_ids, max_rank, d_in, d_out, max_tokens)
        if not (1 <= max_cpu <= max_ids):
            raise OracleError(INVALID_ARG, "host cache size")
        self.max_cpu = max_cpu
        self.host: Dict[int, Adapter] = {}     # the host cache
        self.direct: Dict[int, Adapter] = {}   # loaded straight into the pool
        self.cached: set = set()               # host-cached ids with a device copy
        self.last_use: Dict[int, int] = {}
        self.pinned: set = set()
        self.calls = 0
        self.named: set = set()                # host-cached ids of the last prefetch
        self.loads_last_call: List[int] = []   # ids paged in by the last prefetch

    # the Registry's addressable view
    def _refresh(self) -> None:
        view = dict(self.direct)
        for i in self.cached:
            if i in self.named or i in self.pinned:
                view[i] = self.host[i]
        self.adapters = view

    def _slots_used(self) -> int:
        return len(self.direct) + len(self.cached)

    def load(self, adapter_id, rank, alpha, A, B) -> None:
        """Load straight into the pool (never evicted)."""
        if not (0 <= adapter_id < self.max_ids):
            raise OracleError(ID_RANGE, f"id {adapter_id}")
        if not (1 <= rank <= self.max_rank):
            raise OracleError(RANK, f"rank {rank}")
        if adapter_id in self.direct or adapter_id in self.host:
            raise OracleError(EXISTS, f"id {adapter_id}")
        if self._slots_used() >= self.max_adapters:
            raise OracleError(POOL_FULL, "no free slot")
        probe = Registry(1, self.max_ids, self.max_rank, self.d_in, self.d_out, self.max_tokens)
        probe.load(adapter_id, rank, alpha, A, B)
        self.direct[adapter_id] = probe.adapters[adapter_id]
        self._refresh()

    def unload(self, adapter_id: int) -> None:
        if not (0 <= adapter_id < self.max_ids):
            raise OracleError(ID_RANGE, f"id {adapter_id}")
        if adapter_id in self.direct:
            del self.direct[adapter_id]
        elif adapter_id in self.cached:
            self.cached.discard(adapter_id)
            self.pinned.discard(adapter_id)
            self.named.discard(adapter_id)
        else:
            raise OracleError(NOT_LOADED, f"id {adapter_id}")
        self._refresh()

    def host_register(self, adapter_id: int, rank: int, alpha: float, A: Sequence, B: Sequence) -> None:
        if not (0 <= adapter_id < self.max_ids):
            raise OracleError(ID_RANGE, f"id {adapter_id}")
        if not (1 <= rank <= self.max_rank):
            raise OracleError(RANK, f"rank {rank}")
        if adapter_id in self.host or adapter_id in self.direct:
            raise OracleError(EXISTS, f"id {adapter_id}")
        if len(self.host) >= self.max_cpu:
            raise OracleError(POOL_FULL, "host cache full")
        probe = Registry(1, self.max_ids, self.max_rank, self.d_in, self.d_out, self.max_tokens)
        probe.load(adapter_id, rank, alpha, A, B)
        self.host[adapter_id] = probe.adapters[adapter_id]

    def host_unregister(self, adapter_id: int) -> None:
        if not (0 <= adapter_id < self.max_ids):
            raise OracleError(ID_RANGE, f"id {adapter_id}")
        if adapter_id not in self.host:
            raise OracleError(NOT_LOADED, f"id {adapter_id}")
        del self.host[adapter_id]
        self.cached.discard(adapter_id)
        self.pinned.discard(adapter_id)
        self.named.discard(adapter_id)
        self.last_use.pop(adapter_id, None)
        self._refresh()

    def _victims(self, protect: set) -> List[int]:
        """Evictable cached ids, least recently used first."""
        c = [i for i in self.cached if i not in self.pinned and i not in protect]
        return sorted(c, key=lambda i: (self.last_use.get(i, 0), i))

    def pin(self, adapter_id: int, on: bool) -> None:
        if not (0 <= adapter_id < self.max_ids):
            raise OracleError(ID_RANGE, f"id {adapter_id}")
        if adapter_id not in self.host:
            raise OracleError(NOT_LOADED, f"id {adapter_id}")
        if not on:
            if adapter_id in self.pinned:
                # it was in use up to now: its recency is that of the latest call
                self.pinned.discard(adapter_id)
                self.last_use[adapter_id] = max(self.last_use.get(adapter_id, 0), self.calls)
            self._refresh()
            return
        if adapter_id not in self.cached:
            if self._slots_used() >= self.max_adapters:
                # never evict an id the current batch may address
                victims = self._victims(protect=set(self.adapters))
                if not victims:
                    raise OracleError(POOL_FULL, "no evictable slot")
                self.cached.discard(victims[0])
            self.cached.add(adapter_id)
        self.pinned.add(adapter_id)
        self._refresh()

    def prefetch(self, ids: Sequence[int]) -> List[int]:
        """Make the ids of the next batch addressable; returns the ids paged in."""
        ids = [int(i) for i in ids]
        for i in ids:
            if i < -1 or i >= self.max_ids:
                raise OracleError(ID_RANGE, f"id {i}")
        req: List[int] = []
        for i in ids:
            if i < 0 or i in self.direct:
                continue
            if i not in self.host:
                raise OracleError(NOT_LOADED, f"id {i}")
            if i not in req:
                req.append(i)
        misses = [i for i in req if i not in self.cached]
        free = self.max_adapters - self._slots_used()
        victims = self._victims(protect=set(req))
        if len(misses) > free + len(victims):
            raise OracleError(POOL_FULL, f"{len(misses)} misses, {free} free, {len(victims)} evictable")
        self.calls += 1
        for i in req:
            self.last_use[i] = self.calls
        for i in misses:
            if free > 0:
                free -= 1
            else:
                self.cached.discard(victims.pop(0))
            self.cached.add(i)
        self.named = set(req)
        self.loads_last_call = misses
        self._refresh()
        return misses

    def where(self, adapter_id: int) -> int:
        """0 unknown, 1 host cache only, 2 cached on the device but not
        addressable, 3 addressable."""
        if adapter_id in self.adapters:
            return 3
        if adapter_id in self.cached:
            return 2
        if adapter_id in self.host:
            return 1
        return 0


# --------------------------------------------------------------------------
# INT4 base weight ([vLLM-ch7] performance notes: an AWQ-INT4 base with bf16
# adapters).  Readings: group-wise asymmetric 4-bit weights along d_in, the
# AWQ group size of 128, q and the zero point z in 0..15, a bf16 scale s per
# (output row, group); the base GEMM works on the weight dequantized to the
# compute dtype, i.e. W[n, k] = bf16((q[n, k] - z[n, g]) * s[n, g]), g = k // 128
# (the product is exact in float64, then one round to nearest even).
# --------------------------------------------------------------------------
Q4_GROUP = 128


def round_to_bf16(x) -> np.ndarray:
    """Round float64 values that are exact in float32 to the nearest bf16
    (ties to even); returns float64."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    assert np.array_equal(f.astype(np.float64), np.asarray(x, dtype=np.float64)), "not exact in f32"
    b = f.view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    r = ((b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return (r.astype(np.uint32)).view(np.float32).astype(np.float64)


def dequant_q4(q, z, s) -> np.ndarray:
    """q: [N, K] integers 0..15; z: [N, K // 128] integers 0..15; s: [N, K // 128]
    bf16 scales (bits or tensor).  Returns the dequantized weight [N, K]
    (float64 holding bf16 values)."""
    q = np.asarray(q, dtype=np.int64)
    z = np.asarray(z, dtype=np.int64)
    sf = _as_f64(s)
    N, K = q.shape
    if K % Q4_GROUP or z.shape != (N, K // Q4_GROUP) or sf.shape != z.shape:
        raise OracleError(INVALID_ARG, "q4 shapes")
    if q.min(initial=0) < 0 or q.max(initial=0) > 15 or z.min(initial=0) < 0 or z.max(initial=0) > 15:
        raise OracleError(INVALID_ARG, "q4 values")
    g = np.arange(K) // Q4_GROUP
    exact = (q - z[:, g]).astype(np.float64) * sf[:, g]
    return round_to_bf16(exact)
