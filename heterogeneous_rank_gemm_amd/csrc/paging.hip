// Host <-> device paging of the adapter pool.
//
// The vLLM chapter "Multi-LoRA hot-plug: one model serving many tenants"
// keeps --max-loras adapters on the GPU and more in a CPU cache
// (--max-cpu-loras) that are swapped in on demand (sections "how vLLM
// implements multi-LoRA", item 1, and "starting a multi-LoRA service").  The
// icman report (section 2.2) reads a missing adapter into device memory,
// swaps out the least recently used inactive adapter when memory runs short,
// and keeps a preload list of the hottest few resident; its section 4.2 names
// cold loads as the latency cliff.
//
// Here the host cache is pinned memory holding every registered adapter
// already in the device page layout, so paging an adapter in is one
// host -> device copy of a slot.  A prefetch names the ids of the next batch:
//   * the host-cached ids it names become addressable (the routing table
//     points at their slot); those of the previous prefetch that it does not
//     name stop being addressable but keep their device copy as a cache;
//   * a named id without a device copy takes a free slot, else the slot of
//     the cached, unpinned, unnamed id with the smallest (last prefetch that
//     named it, id);
//   * the copies run on the pool's own copy stream, so they overlap whatever
//     is still running on the caller's stream: one launch reads the misses'
//     slots from the pinned host cache through its device mapping (measured
//     on MI355X: ~47 GB/s for 40 slots of 256 KB, against ~19 GB/s as 40
//     separate DMA copies).  Copies into free slots alone wait for nothing;
//     copies into evicted adapters' slots wait only for the work enqueued
//     before the first prefetch that stopped naming the most recently named
//     victim (every kernel that could read those pages), recorded as an
//     event at the start of that prefetch.  The caller's stream then waits
//     for the copies and updates the routing table in stream order.
// Strict mode is kept: a kernel that meets an id that is not addressable
// rejects the batch.
#include <algorithm>
#include <cstring>
#include <vector>

#include "internal.h"
#include "lora.h"
#include "pool_state.h"

namespace {

using hrg::DeviceGuard;

bool registered(const lora_pool_s* P, int32_t id) { return P->hcache && P->h_hslot[id] >= 0; }

uint16_t* host_slot(const lora_pool_s* P, int32_t id) {
  return P->hcache + (size_t)P->h_hslot[id] * P->slot_elems;
}

uint16_t* dev_slot(const lora_pool_s* P, int32_t slot) {
  return P->pages + (size_t)slot * P->slot_elems;
}

int4 entry(const lora_pool_s* P, int32_t id, int32_t slot) {
  if (slot < 0) return make_int4(id, -1, 0, 0);
  float sc = P->h_hscale[id];
  int bits;
  std::memcpy(&bits, &sc, 4);
  return make_int4(id, slot, P->h_hrank[id], bits);
}

// Points the host mirror of the routing table at `slot` (-1: not addressable).
void mirror(lora_pool_s* P, int32_t id, int32_t slot) {
  P->h_id2slot[id] = slot;
  if (slot >= 0) {
    P->h_slot_rank[slot] = P->h_hrank[id];
    P->h_slot_scale[slot] = P->h_hscale[id];
  }
}

bool is_named(const lora_pool_s* P, int32_t id) {
  return std::find(P->named.begin(), P->named.end(), id) != P->named.end();
}

// The evictable cached ids, least recently used first: unpinned and not in
// `keep` (an id -> bool table).
std::vector<int32_t> victims(const lora_pool_s* P, const std::vector<uint8_t>& keep) {
  std::vector<int32_t> v;
  for (int32_t id : P->cached_ids)
    if (!P->pinned[id] && !keep[id]) v.push_back(id);
  std::sort(v.begin(), v.end(), [P](int32_t a, int32_t b) {
    return P->last_use[a] != P->last_use[b] ? P->last_use[a] < P->last_use[b] : a < b;
  });
  return v;
}

// A slot for a new device copy of `id`: its own slot in a direct-mapped pool,
// else the lowest free one; -1 if none is free.
int32_t take_free_slot(lora_pool_s* P, int32_t id) {
  const bool direct = P->max_ids <= P->max_adapters;
  if (direct) {
    if (!P->free_slots.count(id)) return -1;
    P->free_slots.erase(id);
    return id;
  }
  if (P->free_slots.empty()) return -1;
  const int32_t s = *P->free_slots.begin();
  P->free_slots.erase(s);
  return s;
}

lora_status_t hip_fail() {
  (void)hipGetLastError();
  return LORA_ERR_HIP;
}

}  // namespace

namespace hrg {

lora_status_t paged_drop_device_copy(lora_pool_s* P, int32_t id, hipStream_t stream) {
  const int32_t slot = P->cached[id];
  if (slot < 0) return LORA_ERR_NOT_LOADED;
  DeviceGuard g(P->device);
  if (hipStreamSynchronize(P->copy_stream) != hipSuccess || hipStreamSynchronize(stream) != hipSuccess ||
      hrg::launch_set_slot(P->id2slot, P->slot_rank, P->slot_scale, P->id_info, P->id_bscale, id, -1, 0, 0.f, 0,
                           make_float4(0.f, 0.f, 0.f, 0.f), stream) !=
          hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return hip_fail();
  mirror(P, id, -1);
  P->cached[id] = -1;
  P->cached_ids.erase(id);
  P->pinned[id] = 0;
  P->named.erase(std::remove(P->named.begin(), P->named.end(), id), P->named.end());
  P->free_slots.insert(slot);
  return LORA_OK;
}

}  // namespace hrg

extern "C" {

lora_status_t lora_host_cache_create(lora_pool_t P, int32_t max_cpu_adapters) {
  if (!P || P->hcache || max_cpu_adapters < 1 || max_cpu_adapters > P->max_ids) return LORA_ERR_INVALID_ARG;
  DeviceGuard g(P->device);
  const size_t bytes = (size_t)max_cpu_adapters * P->slot_elems * sizeof(uint16_t);
  void* h = nullptr;
  if (hipHostMalloc(&h, bytes, hipHostMallocDefault) != hipSuccess) {
    (void)hipGetLastError();
    return LORA_ERR_OOM;
  }
  bool ok = hipStreamCreateWithFlags(&P->copy_stream, hipStreamNonBlocking) == hipSuccess &&
            hipEventCreateWithFlags(&P->copy_ev, hipEventDisableTiming) == hipSuccess;
  for (int i = 0; ok && i < hrg::kCallEvents; ++i)
    ok = hipEventCreateWithFlags(&P->call_ev[i], hipEventDisableTiming) == hipSuccess;
  if (!ok) {
    (void)hipGetLastError();
    (void)hipHostFree(h);
    if (P->copy_stream) (void)hipStreamDestroy(P->copy_stream);
    P->copy_stream = nullptr;
    if (P->copy_ev) (void)hipEventDestroy(P->copy_ev);
    P->copy_ev = nullptr;
    for (hipEvent_t& e : P->call_ev) {
      if (e) (void)hipEventDestroy(e);
      e = nullptr;
    }
    return LORA_ERR_HIP;
  }
  void* hd = nullptr;
  if (hipHostGetDevicePointer(&hd, h, 0) != hipSuccess || !hd) {
    (void)hipGetLastError();
    (void)hipHostFree(h);
    return LORA_ERR_HIP;
  }
  P->hcache = static_cast<uint16_t*>(h);
  P->hcache_dev = hd;
  P->max_cpu = max_cpu_adapters;
  P->h_hslot.assign(P->max_ids, -1);
  P->h_hrank.assign(P->max_ids, 0);
  P->h_hscale.assign(P->max_ids, 0.f);
  P->cached.assign(P->max_ids, -1);
  P->last_use.assign(P->max_ids, 0);
  P->pinned.assign(P->max_ids, 0);
  for (int32_t i = 0; i < max_cpu_adapters; ++i) P->free_hslots.insert(i);
  return LORA_OK;
}

lora_status_t lora_host_register(lora_pool_t P, int32_t id, int32_t rank, float alpha,
                                 const lora_bf16_t* const* A, const lora_bf16_t* const* B) {
  if (!P || !P->hcache || !A || !B) return LORA_ERR_INVALID_ARG;
  int32_t mask = 0;
  if (!hrg::target_mask(P->n_modules, reinterpret_cast<const void* const*>(A),
                        reinterpret_cast<const void* const*>(B), &mask))
    return LORA_ERR_INVALID_ARG;
  if (id < 0 || id >= P->max_ids) return LORA_ERR_ID_RANGE;
  if (rank < 1 || rank > P->max_rank) return LORA_ERR_RANK;
  if (P->h_hslot[id] >= 0 || P->h_id2slot[id] >= 0) return LORA_ERR_EXISTS;
  if (P->free_hslots.empty()) return LORA_ERR_POOL_FULL;
  DeviceGuard g(P->device);
  const int32_t hs = *P->free_hslots.begin();
  uint16_t* dst = P->hcache + (size_t)hs * P->slot_elems;
  // A free host slot has no copy in flight (unregister waits for them).
  std::memset(dst, 0, P->slot_elems * sizeof(uint16_t));
  std::vector<uint16_t> tmp;
  for (int32_t m = 0; m < P->n_modules; ++m) {
    const int32_t din = P->d_in[m], dout = P->d_out[m];
    if (!A[m]) continue;  // not a target of this adapter: its pages stay zero
    // A (d_in x rank) -> A^T page in fragment tiles; A may be host or device memory
    tmp.resize((size_t)din * rank);
    if (hipMemcpy(tmp.data(), A[m], tmp.size() * 2, hipMemcpyDefault) != hipSuccess) return hip_fail();
    uint16_t* pa = dst + P->a_off[m];
    for (int32_t k = 0; k < din; ++k)
      for (int32_t q = 0; q < rank; ++q) pa[hrg::frag_index(q, k, P->rpad, din)] = tmp[(size_t)k * rank + q];
    // B (rank x d_out) -> B^T in 16-rank chunks [rpad/16][d_out][16]
    tmp.resize((size_t)rank * dout);
    if (hipMemcpy(tmp.data(), B[m], tmp.size() * 2, hipMemcpyDefault) != hipSuccess) return hip_fail();
    uint16_t* pb = dst + P->b_off[m];
    for (int32_t q = 0; q < rank; ++q)
      for (int32_t n = 0; n < dout; ++n)
        pb[(size_t)(q / 16) * dout * 16 + (size_t)n * 16 + q % 16] = tmp[(size_t)q * dout + n];
  }
  P->free_hslots.erase(hs);
  P->h_hslot[id] = hs;
  P->h_hrank[id] = rank;
  P->h_hscale[id] = alpha / (float)rank;
  P->h_mask[id] = mask;
  P->last_use[id] = 0;
  P->pinned[id] = 0;
  return LORA_OK;
}

lora_status_t lora_host_unregister(lora_pool_t P, int32_t id, hipStream_t stream) {
  if (!P || !P->hcache) return LORA_ERR_INVALID_ARG;
  if (id < 0 || id >= P->max_ids) return LORA_ERR_ID_RANGE;
  if (!registered(P, id)) return LORA_ERR_NOT_LOADED;
  DeviceGuard g(P->device);
  if (P->cached[id] >= 0) {
    const lora_status_t st = hrg::paged_drop_device_copy(P, id, stream);
    if (st != LORA_OK) return st;
  } else if (hipStreamSynchronize(P->copy_stream) != hipSuccess) {
    return hip_fail();
  }
  P->free_hslots.insert(P->h_hslot[id]);
  P->h_hslot[id] = -1;
  P->h_hrank[id] = 0;
  P->h_hscale[id] = 0.f;
  P->last_use[id] = 0;
  P->pinned[id] = 0;
  P->named.erase(std::remove(P->named.begin(), P->named.end(), id), P->named.end());
  return LORA_OK;
}

lora_status_t lora_pin_adapter(lora_pool_t P, int32_t id, int32_t pin, hipStream_t stream) {
  if (!P || !P->hcache) return LORA_ERR_INVALID_ARG;
  if (id < 0 || id >= P->max_ids) return LORA_ERR_ID_RANGE;
  if (!registered(P, id)) return LORA_ERR_NOT_LOADED;
  DeviceGuard g(P->device);
  if (!pin) {
    if (!P->pinned[id]) return LORA_OK;
    P->pinned[id] = 0;
    // in use until now: the recency of the latest prefetch
    P->last_use[id] = std::max<int64_t>(P->last_use[id], P->calls);
    if (!is_named(P, id) && P->h_id2slot[id] >= 0) {
      const int4 e = entry(P, id, -1);
      const int32_t mk = 0;
      if (hrg::launch_set_slots(P->id2slot, P->slot_rank, P->slot_scale, P->id_info, P->id_bscale, &e, &mk, 1,
                                stream) !=
          hipSuccess)
        return hip_fail();
      mirror(P, id, -1);
    }
    return LORA_OK;
  }
  if (P->pinned[id]) return LORA_OK;
  int32_t slot = P->cached[id];
  if (slot < 0) {
    slot = take_free_slot(P, id);
    int32_t victim = -1;
    if (slot < 0) {
      // never evict an id that work on the stream may address
      std::vector<uint8_t> keep(P->max_ids, 0);
      for (int32_t i : P->cached_ids)
        if (P->h_id2slot[i] >= 0) keep[i] = 1;
      const std::vector<int32_t> v = victims(P, keep);
      if (v.empty()) return LORA_ERR_POOL_FULL;
      victim = v.front();
      slot = P->cached[victim];
    }
    // a setup call: wait for everything in flight before overwriting a slot
    if (hipStreamSynchronize(P->copy_stream) != hipSuccess || hipStreamSynchronize(stream) != hipSuccess ||
        hipMemcpyAsync(dev_slot(P, slot), host_slot(P, id), P->slot_elems * sizeof(uint16_t),
                       hipMemcpyHostToDevice, stream) != hipSuccess) {
      if (victim < 0) P->free_slots.insert(slot);
      return hip_fail();
    }
    if (victim >= 0) {
      P->cached[victim] = -1;
      P->cached_ids.erase(victim);
    }
    P->cached[id] = slot;
    P->cached_ids.insert(id);
    ++P->pages_loaded;
  }
  if (P->h_id2slot[id] != slot) {
    const int4 e = entry(P, id, slot);
    const int32_t mk = P->h_mask[id];
    if (hrg::launch_set_slots(P->id2slot, P->slot_rank, P->slot_scale, P->id_info, P->id_bscale, &e, &mk, 1,
                              stream) !=
        hipSuccess)
      return hip_fail();
    mirror(P, id, slot);
  }
  if (hipStreamSynchronize(stream) != hipSuccess) return hip_fail();
  P->pinned[id] = 1;
  return LORA_OK;
}

lora_status_t lora_prefetch(lora_pool_t P, const int32_t* ids, int32_t n, hipStream_t stream) {
  if (!P || !P->hcache || n < 0 || (n > 0 && !ids)) return LORA_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i)
    if (ids[i] < -1 || ids[i] >= P->max_ids) return LORA_ERR_ID_RANGE;
  // the host-cached ids of the batch, in order of first appearance
  std::vector<uint8_t> inreq(P->max_ids, 0);
  std::vector<int32_t> req;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t id = ids[i];
    if (id < 0) continue;
    if (!registered(P, id)) {
      if (P->h_id2slot[id] >= 0) continue;  // loaded directly: always addressable
      return LORA_ERR_NOT_LOADED;
    }
    if (!inreq[id]) {
      inreq[id] = 1;
      req.push_back(id);
    }
  }
  std::vector<int32_t> misses;
  for (int32_t id : req)
    if (P->cached[id] < 0) misses.push_back(id);
  const std::vector<int32_t> vic = victims(P, inreq);
  if (misses.size() > P->free_slots.size() + vic.size()) return LORA_ERR_POOL_FULL;
  if (P->max_ids <= P->max_adapters)  // direct-mapped: each id owns its slot
    for (int32_t id : misses)
      if (!P->free_slots.count(id)) return LORA_ERR_POOL_FULL;

  DeviceGuard g(P->device);
  const int64_t c = ++P->calls;
  hipEvent_t ev_c = P->call_ev[c % hrg::kCallEvents];
  if (hipEventRecord(ev_c, stream) != hipSuccess) return hip_fail();
  for (int32_t id : req) P->last_use[id] = c;

  // slots for the misses; the copies into evicted slots wait for the latest
  // release point among their victims (call events complete in call order)
  size_t vi = 0;
  int64_t release = 0;
  std::vector<int2> moves;
  for (int32_t id : misses) {
    int32_t slot = take_free_slot(P, id);
    if (slot < 0) {
      const int32_t v = vic[vi++];
      slot = P->cached[v];
      P->cached[v] = -1;
      P->cached_ids.erase(v);
      // every kernel that may read v's pages was enqueued before the first
      // prefetch after the last one that named v
      release = std::max<int64_t>(release, std::max<int64_t>(P->last_use[v] + 1, 1));
    }
    moves.push_back(make_int2(P->h_hslot[id], slot));
    P->cached[id] = slot;
    P->cached_ids.insert(id);
    ++P->pages_loaded;
  }
  if (!moves.empty()) {
    if (release > 0) {
      hipEvent_t rel = (c - release < hrg::kCallEvents) ? P->call_ev[release % hrg::kCallEvents] : ev_c;
      if (hipStreamWaitEvent(P->copy_stream, rel, 0) != hipSuccess) return hip_fail();
    }
    if (hrg::launch_page_in(P->hcache_dev, P->pages, moves.data(), (int)moves.size(),
                            P->slot_elems * sizeof(uint16_t) / 16, P->copy_stream) != hipSuccess ||
        hipEventRecord(P->copy_ev, P->copy_stream) != hipSuccess ||
        hipStreamWaitEvent(stream, P->copy_ev, 0) != hipSuccess)
      return hip_fail();
  }

  // routing-table changes, in stream order after the copies
  std::vector<int4> ups;
  std::vector<int32_t> masks;
  for (int32_t id : P->named)
    if (!inreq[id] && !P->pinned[id] && P->h_id2slot[id] >= 0) {
      ups.push_back(entry(P, id, -1));
      masks.push_back(0);
      mirror(P, id, -1);
    }
  for (int32_t id : req)
    if (P->h_id2slot[id] != P->cached[id]) {
      ups.push_back(entry(P, id, P->cached[id]));
      masks.push_back(P->h_mask[id]);
      mirror(P, id, P->cached[id]);
    }
  P->named = req;
  if (!ups.empty() && hrg::launch_set_slots(P->id2slot, P->slot_rank, P->slot_scale, P->id_info, P->id_bscale,
                                            ups.data(), masks.data(), (int)ups.size(), stream) != hipSuccess)
    return hip_fail();
  return LORA_OK;
}

lora_status_t lora_paging_query(lora_pool_t P, int32_t id, int32_t* where, int32_t* pinned) {
  if (!P) return LORA_ERR_INVALID_ARG;
  if (id < 0 || id >= P->max_ids) return LORA_ERR_ID_RANGE;
  int32_t w = 0, p = 0;
  if (P->h_id2slot[id] >= 0) {
    w = 3;
  } else if (P->hcache && P->cached[id] >= 0) {
    w = 2;
  } else if (registered(P, id)) {
    w = 1;
  }
  if (P->hcache) p = P->pinned[id];
  if (where) *where = w;
  if (pinned) *pinned = p;
  return LORA_OK;
}

lora_status_t lora_paging_stats(lora_pool_t P, int64_t* prefetches, int64_t* pages_loaded,
                                int64_t* bytes_per_page) {
  if (!P) return LORA_ERR_INVALID_ARG;
  if (prefetches) *prefetches = P->calls;
  if (pages_loaded) *pages_loaded = P->pages_loaded;
  if (bytes_per_page) *bytes_per_page = (int64_t)(P->slot_elems * sizeof(uint16_t));
  return LORA_OK;
}

}  // extern "C"
