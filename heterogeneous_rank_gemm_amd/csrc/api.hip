// Host side of the C ABI (include/lora.h): the unified adapter pool, its
// routing tables, the load / unload path, plans, and the apply entry points.
//
// The pool follows the vLLM chapter "Multi-LoRA hot-plug: one model serving
// many tenants" (section "how vLLM implements multi-LoRA": all adapters in
// one device memory pool) and the routing table of the icman report
// (section 2.1: adapter name -> location, loaded-in-VRAM flag), reduced to
// an integer id -> slot table mirrored on host and device.
#include <algorithm>
#include <mutex>
#include <new>
#include <set>
#include <vector>

#include "internal.h"
#include "lora.h"
#include "pool_state.h"

static_assert(hrg::kStatusNotLoaded == LORA_ERR_NOT_LOADED, "status code mismatch");
static_assert(hrg::kStatusIdRange == LORA_ERR_ID_RANGE, "status code mismatch");

namespace {

using hrg::ceil_div;
using hrg::round_up;

using hrg::DeviceGuard;

template <typename T>
hipError_t dmalloc(T** p, size_t n) {
  return hipMalloc(reinterpret_cast<void**>(p), std::max<size_t>(n, 1) * sizeof(T));
}

int max_tiles_for(const lora_pool_s* P) {
  return std::min(P->max_tokens, P->max_adapters) + ceil_div(P->max_tokens, hrg::kShrinkRows) + 1;
}

lora_status_t plan_alloc(lora_pool_s* P, lora_plan_s** out) {
  const size_t Tc = (size_t)P->max_tokens;
  const int mt = max_tiles_for(P);
  // perm, inv, row_seg, erow (Tc each); seg_id, seg_slot, seg_rank, seg_scale,
  // seg_e0 (Tc+1); seg_off (Tc+2); tile_info (4 mt) and small_info
  // (4 kMaxSmallRows), first: 16-byte aligned; counts (4)
  // seg_bscale (4 (Tc+1)) and small_bscale (4 kMaxSmallRows), 16-byte aligned, after the int4 tables
  const size_t n32 = 4 * Tc + 5 * (Tc + 1) + (Tc + 2) + 4 * (size_t)mt + 4 * (size_t)hrg::kMaxSmallRows +
                     4 * (Tc + 1) + 4 * (size_t)hrg::kMaxSmallRows + 4;
  lora_plan_s* pl = new (std::nothrow) lora_plan_s();
  if (!pl) return LORA_ERR_OOM;
  int32_t* blk = nullptr;
  if (dmalloc(&blk, n32) != hipSuccess) {
    delete pl;
    (void)hipGetLastError();
    return LORA_ERR_OOM;
  }
  pl->block = blk;
  int32_t* c = blk;
  auto take = [&](size_t n) { int32_t* r = c; c += n; return r; };
  pl->tab.tile_info = reinterpret_cast<int4*>(take(4 * (size_t)mt));
  pl->tab.small_info = reinterpret_cast<int4*>(take(4 * (size_t)hrg::kMaxSmallRows));
  pl->tab.seg_bscale = reinterpret_cast<float4*>(take(4 * (Tc + 1)));
  pl->tab.small_bscale = reinterpret_cast<float4*>(take(4 * (size_t)hrg::kMaxSmallRows));
  pl->tab.perm = take(Tc);
  pl->tab.inv = take(Tc);
  pl->tab.row_seg = take(Tc);
  pl->tab.seg_id = take(Tc + 1);
  pl->tab.seg_slot = take(Tc + 1);
  pl->tab.seg_rank = take(Tc + 1);
  pl->tab.seg_scale = reinterpret_cast<float*>(take(Tc + 1));
  pl->tab.seg_off = take(Tc + 2);
  pl->tab.erow = take(Tc);
  pl->tab.seg_e0 = take(Tc + 1);
  pl->tab.counts = take(4);
  pl->tab.max_tiles = mt;
  *out = pl;
  return LORA_OK;
}

void plan_free(lora_plan_s* pl) {
  if (!pl) return;
  if (pl->block) (void)hipFree(pl->block);
  delete pl;
}

lora_status_t run_plan(lora_pool_s* P, const int32_t* ids, int32_t T, lora_plan_s* pl, hipStream_t s) {
  hrg::PlanArgs a{};
  a.ids = ids;
  a.T = T;
  a.max_ids = P->max_ids;
  a.id_info = P->id_info;
  a.id_bscale = P->id_bscale;
  a.status = P->status;
  a.tab = pl->tab;
  if (hrg::launch_plan(a, s) != hipSuccess) return LORA_ERR_HIP;
  pl->T = T;
  pl->ids = ids;
  return LORA_OK;
}

bool module_ok(const lora_pool_s* P, int32_t m) { return P && m >= 0 && m < P->n_modules; }

// The decode path (T <= kDecodeMaxT) for a group of n linears that read the
// same X (one launch pair; a single linear is a group of one).
lora_status_t decode_group(lora_pool_s* P, int32_t n, const int32_t* modules, const lora_bf16_t* X,
                           const int32_t* ids, int32_t T, const lora_bf16_t* const* W,
                           const uint32_t* const* Wq, const uint32_t* const* Wsz, lora_bf16_t* const* out,
                           bool lora, bool wpacked, float* part, float* upart, hipStream_t stream) {
  const int K = P->d_in[modules[0]];
  hrg::DecodeArgs a{};
  a.X = X;
  a.ids = ids;
  a.T = T;
  a.K = K;
  a.KS = ceil_div(K, hrg::kDecodeChunk);
  a.n_mod = n;
  a.wq = Wq ? 1 : 0;
  a.wpacked = wpacked ? 1 : 0;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t m = modules[i], N = P->d_out[m];
    a.W[i] = W ? W[i] : nullptr;
    a.Wq[i] = Wq ? Wq[i] : nullptr;
    a.Wsz[i] = Wsz ? Wsz[i] : nullptr;
    a.out[i] = out[i];
    a.N[i] = N;
    a.module[i] = m;
    a.a_off[i] = P->a_off[m];
    a.b_off[i] = P->b_off[m];
    a.u0[i + 1] = a.u0[i] + ceil_div(N, 16);
    a.n0[i + 1] = a.n0[i] + round_up(N, 16);
    a.ct0[i + 1] = a.ct0[i] + ceil_div(N, hrg::kDecodeTileRows);
  }
  for (int32_t i = n + 1; i <= hrg::kMaxGroup; ++i) {
    a.u0[i] = a.u0[n];
    a.n0[i] = a.n0[n];
    a.ct0[i] = a.ct0[n];
  }
  a.npad = a.n0[n];
  a.max_ids = P->max_ids;
  a.id_info = P->id_info;
  a.id_bscale = P->id_bscale;
  a.pages = P->pages;
  a.slot_stride = P->slot_elems;
  a.part = part;
  a.upart = upart;
  a.direct = P->max_ids <= P->max_adapters ? 1 : 0;
  a.max_slots = P->max_adapters;
  a.rmax = P->max_rank;
  a.u_ld = P->rpad;
  a.status = P->status;
  a.lora = lora ? 1 : 0;
  // A items: (adapter, 16-rank block); a batch holds at most min(T, slots,
  // ids) distinct adapters.  Sized from the pool's capacity, never from how
  // many adapters are resident now: a captured graph replays this launch
  // after later loads and prefetches, and items the grid does not hold would
  // be skipped.  The kernel walks only the batch's own items.
  const int items_cap = std::min(T, std::min(P->max_adapters, P->max_ids)) * (P->rpad / 16);
  return hrg::launch_decode(a, items_cap, stream) == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

// Floats of the decode partial planes a group of up to kMaxGroup linears
// with one d_in needs: KS chunks x 64 tokens x the columns (each linear's
// rounded up to 16) of its largest members.
size_t decode_part_floats(const std::vector<int32_t>& d_in, const std::vector<int32_t>& d_out) {
  size_t best = 0;
  for (size_t i = 0; i < d_in.size(); ++i) {
    std::vector<int32_t> cols;
    for (size_t j = 0; j < d_in.size(); ++j)
      if (d_in[j] == d_in[i]) cols.push_back(round_up(d_out[j], 16));
    std::sort(cols.rbegin(), cols.rend());
    size_t sum = 0;
    for (size_t j = 0; j < cols.size() && j < (size_t)hrg::kMaxGroup; ++j) sum += cols[j];
    best = std::max(best, (size_t)ceil_div(d_in[i], hrg::kDecodeChunk) * hrg::kDecodeMaxT * sum);
  }
  return best;
}

}  // namespace

extern "C" {

const char* lora_status_string(lora_status_t s) {
  switch (s) {
    case LORA_OK: return "LORA_OK";
    case LORA_ERR_INVALID_ARG: return "LORA_ERR_INVALID_ARG";
    case LORA_ERR_OOM: return "LORA_ERR_OOM";
    case LORA_ERR_POOL_FULL: return "LORA_ERR_POOL_FULL";
    case LORA_ERR_RANK: return "LORA_ERR_RANK";
    case LORA_ERR_EXISTS: return "LORA_ERR_EXISTS";
    case LORA_ERR_NOT_LOADED: return "LORA_ERR_NOT_LOADED";
    case LORA_ERR_ID_RANGE: return "LORA_ERR_ID_RANGE";
    case LORA_ERR_HIP: return "LORA_ERR_HIP";
  }
  return "LORA_ERR_UNKNOWN";
}

lora_status_t lora_pool_create(lora_pool_t* pool, int32_t max_adapters, int32_t max_ids,
                               int32_t max_rank, int32_t n_modules, const int32_t* d_in,
                               const int32_t* d_out, int32_t max_tokens, hipStream_t stream) {
  if (!pool || !d_in || !d_out) return LORA_ERR_INVALID_ARG;
  if (max_adapters < 1 || max_ids < 1 || max_ids > hrg::kMaxIds) return LORA_ERR_INVALID_ARG;
  if (max_rank < 1 || max_rank > hrg::kMaxRank) return LORA_ERR_INVALID_ARG;
  if (n_modules < 1 || max_tokens < 1 || max_tokens > 65536) return LORA_ERR_INVALID_ARG;
  for (int32_t m = 0; m < n_modules; ++m) {
    if (d_in[m] < 8 || d_in[m] > 65536 || d_in[m] % 8) return LORA_ERR_INVALID_ARG;
    if (d_out[m] < 8 || d_out[m] > 65536 || d_out[m] % 8) return LORA_ERR_INVALID_ARG;
    // the decode kernels address a base weight with 32-bit byte offsets
    if ((int64_t)d_in[m] * d_out[m] * 2 > (int64_t)INT32_MAX) return LORA_ERR_INVALID_ARG;
  }
  lora_pool_s* P = new (std::nothrow) lora_pool_s();
  if (!P) return LORA_ERR_OOM;
  if (hipGetDevice(&P->device) != hipSuccess) {
    delete P;
    (void)hipGetLastError();
    return LORA_ERR_HIP;
  }
  P->max_adapters = max_adapters;
  P->max_ids = max_ids;
  P->max_rank = max_rank;
  P->rpad = round_up(max_rank, 16);
  P->n_modules = n_modules;
  P->max_tokens = max_tokens;
  P->d_in.assign(d_in, d_in + n_modules);
  P->d_out.assign(d_out, d_out + n_modules);
  size_t off = 0, max_dim = 0;
  for (int32_t m = 0; m < n_modules; ++m) {
    P->a_off.push_back(off);
    off += hrg::frag_elems(P->rpad, d_in[m]);  // A^T in fragment tiles
    P->b_off.push_back(off);
    off += (size_t)P->rpad * d_out[m];  // B^T in 16-rank chunks
    max_dim = std::max<size_t>(max_dim, std::max(d_in[m], d_out[m]));
  }
  // keep every slot 256-byte aligned
  P->slot_elems = (off + 127) / 128 * 128;
  P->split_stride = (size_t)max_tokens * P->rpad;

  bool ok = dmalloc(&P->pages, P->slot_elems * (size_t)max_adapters) == hipSuccess &&
            dmalloc(&P->id2slot, max_ids) == hipSuccess &&
            dmalloc(&P->slot_rank, max_adapters) == hipSuccess &&
            dmalloc(&P->slot_scale, max_adapters) == hipSuccess &&
            dmalloc(&P->id_info, max_ids) == hipSuccess &&
            dmalloc(&P->id_bscale, max_ids) == hipSuccess &&
            dmalloc(&P->status, 4) == hipSuccess &&
            dmalloc(&P->staging, max_dim * max_rank) == hipSuccess &&
            dmalloc(&P->upart, (size_t)hrg::kMaxSplits * P->split_stride) == hipSuccess &&
            dmalloc(&P->v_hi, (size_t)max_tokens * P->rpad) == hipSuccess &&
            dmalloc(&P->v_lo, (size_t)max_tokens * P->rpad) == hipSuccess;
  size_t max_din = 0, max_dout = 0;
  for (int32_t m = 0; m < n_modules; ++m) {
    max_din = std::max<size_t>(max_din, d_in[m]);
    max_dout = std::max<size_t>(max_dout, d_out[m]);
  }
  const size_t ks_max = (max_din + hrg::kDecodeChunk - 1) / hrg::kDecodeChunk;
  if (ok)
    ok = dmalloc(&P->E, (size_t)hrg::kMaxSmallRows * max_dout) == hipSuccess &&
         dmalloc(&P->dec_upart, ks_max * hrg::kMaxGroup * hrg::kDecodeMaxT * P->rpad) == hipSuccess &&
         dmalloc(&P->dec_part, decode_part_floats(P->d_in, P->d_out)) == hipSuccess;
  if (ok) ok = plan_alloc(P, &P->internal) == LORA_OK;
  if (!ok) {
    (void)hipGetLastError();
    lora_pool_destroy(P);
    return LORA_ERR_OOM;
  }
  P->h_id2slot.assign(max_ids, -1);
  P->h_mask.assign(max_ids, 0);
  P->h_chain.assign(max_ids, 0);
  P->h_slot_rank.assign(max_adapters, 0);
  P->h_slot_scale.assign(max_adapters, 0.f);
  for (int32_t i = 0; i < max_adapters; ++i) P->free_slots.insert(i);
  if (hrg::launch_clear_i32(P->id2slot, max_ids, -1, stream) != hipSuccess ||
      hrg::launch_clear_i32(reinterpret_cast<int32_t*>(P->id_info), 4 * max_ids, -1, stream) != hipSuccess ||
      hrg::launch_clear_i32(reinterpret_cast<int32_t*>(P->id_bscale), 4 * max_ids, 0, stream) != hipSuccess ||
      hrg::launch_clear_i32(P->slot_rank, max_adapters, 0, stream) != hipSuccess ||
      hrg::launch_clear_i32(reinterpret_cast<int32_t*>(P->slot_scale), max_adapters, 0, stream) != hipSuccess ||
      hrg::launch_clear_i32(P->status, 4, 0, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess) {
    (void)hipGetLastError();
    lora_pool_destroy(P);
    return LORA_ERR_HIP;
  }
  *pool = P;
  return LORA_OK;
}

lora_status_t lora_pool_destroy(lora_pool_t P) {
  if (!P) return LORA_ERR_INVALID_ARG;
  DeviceGuard g(P->device);
  (void)hipDeviceSynchronize();
  for (lora_plan_s* pl : P->plans) plan_free(pl);
  plan_free(P->internal);
  (void)hipFree(P->pages);
  (void)hipFree(P->id2slot);
  (void)hipFree(P->slot_rank);
  (void)hipFree(P->slot_scale);
  (void)hipFree(P->id_info);
  (void)hipFree(P->id_bscale);
  (void)hipFree(P->status);
  (void)hipFree(P->staging);
  (void)hipFree(P->upart);
  (void)hipFree(P->v_hi);
  (void)hipFree(P->v_lo);
  (void)hipFree(P->dec_upart);
  (void)hipFree(P->dec_part);
  (void)hipFree(P->E);
  if (P->hcache) (void)hipHostFree(P->hcache);
  if (P->copy_stream) (void)hipStreamDestroy(P->copy_stream);
  for (hipEvent_t e : P->call_ev)
    if (e) (void)hipEventDestroy(e);
  if (P->copy_ev) (void)hipEventDestroy(P->copy_ev);
  delete P;
  return LORA_OK;
}

lora_status_t lora_load_adapter(lora_pool_t P, int32_t id, int32_t rank, float alpha,
                                const lora_bf16_t* const* A, const lora_bf16_t* const* B,
                                hipStream_t stream) {
  if (!P || !A || !B) return LORA_ERR_INVALID_ARG;
  int32_t mask = 0;
  if (!hrg::target_mask(P->n_modules, reinterpret_cast<const void* const*>(A),
                        reinterpret_cast<const void* const*>(B), &mask))
    return LORA_ERR_INVALID_ARG;
  if (id < 0 || id >= P->max_ids) return LORA_ERR_ID_RANGE;
  if (rank < 1 || rank > P->max_rank) return LORA_ERR_RANK;
  if (P->h_id2slot[id] >= 0) return LORA_ERR_EXISTS;
  if (P->hcache && P->h_hslot[id] >= 0) return LORA_ERR_EXISTS;  // paged through the host cache
  if (P->free_slots.empty()) return LORA_ERR_POOL_FULL;
  DeviceGuard g(P->device);
  // a direct-mapped pool (max_ids <= max_adapters) keeps adapter id in slot id
  const int32_t slot = P->max_ids <= P->max_adapters ? id : *P->free_slots.begin();
  uint16_t* base = P->pages + (size_t)slot * P->slot_elems;
  for (int32_t m = 0; m < P->n_modules; ++m) {
    const size_t na = (size_t)P->d_in[m] * rank, nb = (size_t)rank * P->d_out[m];
    hrg::PackArgs pa{};
    if (!A[m]) {
      // not a target of this adapter: zero pages (rank 0 reads no source)
      pa = {P->staging, base + P->a_off[m], 0, P->rpad, P->d_in[m], 0};
      if (hrg::launch_pack(pa, stream) != hipSuccess) return LORA_ERR_HIP;
      pa = {P->staging, base + P->b_off[m], 0, P->rpad, P->d_out[m], 1};
      if (hrg::launch_pack(pa, stream) != hipSuccess) return LORA_ERR_HIP;
      continue;
    }
    if (hipMemcpyAsync(P->staging, A[m], na * 2, hipMemcpyDefault, stream) != hipSuccess)
      return (void)hipGetLastError(), LORA_ERR_HIP;
    pa = {P->staging, base + P->a_off[m], rank, P->rpad, P->d_in[m], 0};
    if (hrg::launch_pack(pa, stream) != hipSuccess) return LORA_ERR_HIP;
    if (hipMemcpyAsync(P->staging, B[m], nb * 2, hipMemcpyDefault, stream) != hipSuccess)
      return (void)hipGetLastError(), LORA_ERR_HIP;
    pa = {P->staging, base + P->b_off[m], rank, P->rpad, P->d_out[m], 1};
    if (hrg::launch_pack(pa, stream) != hipSuccess) return LORA_ERR_HIP;
  }
  const float scale = alpha / (float)rank;
  if (hrg::launch_set_slot(P->id2slot, P->slot_rank, P->slot_scale, P->id_info, P->id_bscale, id, slot, rank,
                           scale, mask, make_float4(scale, scale, scale, scale), stream) !=
          hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess) {
    (void)hipGetLastError();
    return LORA_ERR_HIP;
  }
  P->free_slots.erase(slot);
  P->h_id2slot[id] = slot;
  P->h_mask[id] = mask;
  P->h_slot_rank[slot] = rank;
  P->h_slot_scale[slot] = scale;
  return LORA_OK;
}

lora_status_t lora_unload_adapter(lora_pool_t P, int32_t id, hipStream_t stream) {
  if (!P) return LORA_ERR_INVALID_ARG;
  if (id < 0 || id >= P->max_ids) return LORA_ERR_ID_RANGE;
  // a host-cached adapter gives up its device copy only (paging.hip)
  if (P->hcache && P->h_hslot[id] >= 0) return hrg::paged_drop_device_copy(P, id, stream);
  const int32_t slot = P->h_id2slot[id];
  if (slot < 0) return LORA_ERR_NOT_LOADED;
  DeviceGuard g(P->device);
  if (hipStreamSynchronize(stream) != hipSuccess ||
      hrg::launch_set_slot(P->id2slot, P->slot_rank, P->slot_scale, P->id_info, P->id_bscale, id, -1, 0, 0.f, 0,
                           make_float4(0.f, 0.f, 0.f, 0.f), stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess) {
    (void)hipGetLastError();
    return LORA_ERR_HIP;
  }
  P->h_id2slot[id] = -1;
  P->h_chain[id] = 0;
  P->h_slot_rank[slot] = 0;
  P->h_slot_scale[slot] = 0.f;
  P->free_slots.insert(slot);
  return LORA_OK;
}

lora_status_t lora_load_chain(lora_pool_t P, int32_t chain_id, int32_t n, const int32_t* members,
                              hipStream_t stream) {
  if (!P) return LORA_ERR_INVALID_ARG;
  if (chain_id < 0 || chain_id >= P->max_ids) return LORA_ERR_ID_RANGE;
  if (n < 1 || !members) return LORA_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i)
    for (int32_t j = 0; j < i; ++j)
      if (members[i] == members[j]) return LORA_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i)
    if (members[i] < 0 || members[i] >= P->max_ids) return LORA_ERR_ID_RANGE;
  for (int32_t i = 0; i < n; ++i) {
    if (P->h_id2slot[members[i]] < 0) return LORA_ERR_NOT_LOADED;
    if (P->h_chain[members[i]]) return LORA_ERR_INVALID_ARG;
  }
  // every member takes at least one 16-rank block, and max_rank <= 64
  if (n > hrg::kMaxRank / 16) return LORA_ERR_RANK;
  // member c takes the 16-rank blocks [blk[c], blk[c] + nb[c]) of the chain's pages
  int32_t blk[4], nb[4], total = 0, rank = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t r = P->h_slot_rank[P->h_id2slot[members[i]]];
    blk[i] = total;
    nb[i] = (r + 15) / 16;
    rank = 16 * total + r;
    total += nb[i];
  }
  if (rank > P->max_rank) return LORA_ERR_RANK;
  if (P->h_id2slot[chain_id] >= 0 || (P->hcache && P->h_hslot[chain_id] >= 0)) return LORA_ERR_EXISTS;
  const bool direct = P->max_ids <= P->max_adapters;
  if (direct ? !P->free_slots.count(chain_id) : P->free_slots.empty()) return LORA_ERR_POOL_FULL;
  DeviceGuard g(P->device);
  const int32_t slot = direct ? chain_id : *P->free_slots.begin();
  uint16_t* base = P->pages + (size_t)slot * P->slot_elems;
  float bs[4] = {0.f, 0.f, 0.f, 0.f};
  int32_t mask = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t ms = P->h_id2slot[members[i]];
    for (int32_t b = blk[i]; b < blk[i] + nb[i]; ++b) bs[b] = P->h_slot_scale[ms];
    mask |= P->h_mask[members[i]];
  }
  for (int32_t m = 0; m < P->n_modules; ++m) {
    // zero pages, then each member's rank blocks at its offset (rows past a
    // member's rank are zero in its own pages)
    hrg::PackArgs pa = {P->staging, base + P->a_off[m], 0, P->rpad, P->d_in[m], 0};
    if (hrg::launch_pack(pa, stream) != hipSuccess) return LORA_ERR_HIP;
    pa = {P->staging, base + P->b_off[m], 0, P->rpad, P->d_out[m], 1};
    if (hrg::launch_pack(pa, stream) != hipSuccess) return LORA_ERR_HIP;
    for (int32_t i = 0; i < n; ++i) {
      const uint16_t* mb = P->pages + (size_t)P->h_id2slot[members[i]] * P->slot_elems;
      // member block b (16 ranks) -> chain block blk[i] + b: in fragment
      // tiles a block's steps of one 1024-deep column block are contiguous
      const int32_t din = P->d_in[m], k32 = (din + 31) / 32;
      bool ok = true;
      for (int32_t b = 0; b < nb[i] && ok; ++b)
        for (int32_t s0 = 0; s0 < k32 && ok; s0 += hrg::kFragChunk / 32) {
          const size_t steps = (size_t)std::min(hrg::kFragChunk / 32, k32 - s0);
          ok = hipMemcpyAsync(base + P->a_off[m] + hrg::frag_tile(blk[i] + b, s0, P->rpad, din) * 512,
                              mb + P->a_off[m] + hrg::frag_tile(b, s0, P->rpad, din) * 512, steps * 1024,
                              hipMemcpyDeviceToDevice, stream) == hipSuccess;
        }
      if (!ok ||
          hipMemcpyAsync(base + P->b_off[m] + (size_t)blk[i] * P->d_out[m] * 16, mb + P->b_off[m],
                         (size_t)nb[i] * P->d_out[m] * 16 * 2, hipMemcpyDeviceToDevice, stream) != hipSuccess)
        return (void)hipGetLastError(), LORA_ERR_HIP;
    }
  }
  if (hrg::launch_set_slot(P->id2slot, P->slot_rank, P->slot_scale, P->id_info, P->id_bscale, chain_id, slot,
                           rank | hrg::kChainRankFlag, bs[0], mask, make_float4(bs[0], bs[1], bs[2], bs[3]),
                           stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess) {
    (void)hipGetLastError();
    return LORA_ERR_HIP;
  }
  P->free_slots.erase(slot);
  P->h_id2slot[chain_id] = slot;
  P->h_slot_rank[slot] = rank;
  P->h_slot_scale[slot] = bs[0];
  P->h_mask[chain_id] = mask;
  P->h_chain[chain_id] = 1;
  return LORA_OK;
}

lora_status_t lora_pool_query(lora_pool_t P, int32_t id, int32_t* slot, int32_t* rank, float* scale) {
  if (!P) return LORA_ERR_INVALID_ARG;
  if (id < 0 || id >= P->max_ids) return LORA_ERR_ID_RANGE;
  const int32_t sl = P->h_id2slot[id];
  if (sl < 0) return LORA_ERR_NOT_LOADED;
  if (slot) *slot = sl;
  if (rank) *rank = P->h_slot_rank[sl];
  if (scale) *scale = P->h_slot_scale[sl];
  return LORA_OK;
}

lora_status_t lora_plan_create(lora_pool_t P, lora_plan_t* plan) {
  if (!P || !plan) return LORA_ERR_INVALID_ARG;
  DeviceGuard g(P->device);
  lora_plan_s* pl = nullptr;
  lora_status_t st = plan_alloc(P, &pl);
  if (st != LORA_OK) return st;
  P->plans.insert(pl);
  *plan = pl;
  return LORA_OK;
}

lora_status_t lora_plan_destroy(lora_pool_t P, lora_plan_t plan) {
  if (!P || !plan || !P->plans.count(plan)) return LORA_ERR_INVALID_ARG;
  DeviceGuard g(P->device);
  (void)hipDeviceSynchronize();
  P->plans.erase(plan);
  plan_free(plan);
  return LORA_OK;
}

lora_status_t lora_plan(lora_pool_t P, const int32_t* ids, int32_t T, lora_plan_t plan,
                        hipStream_t stream) {
  if (!P || !plan || (plan != P->internal && !P->plans.count(plan))) return LORA_ERR_INVALID_ARG;
  if (T < 0 || T > P->max_tokens || (T > 0 && !ids)) return LORA_ERR_INVALID_ARG;
  DeviceGuard g(P->device);
  return run_plan(P, ids, T, plan, stream);
}

// The batched path (T > kDecodeMaxT): K splits of the shrink for linears of
// depth K.  Splits of at least 1024 (at most kMaxSplits planes), streamed as
// 256-deep sub-chunks with the next one's loads in flight.  An item is a
// short chain of dependent loads, so up to 1024 blocks (two rounds of
// resident blocks) take them one each rather than fewer blocks walking two
// or more (MI355X, 4096-deep linear, 1024 tokens over about 105 adapters of
// ranks 8-64: 17.6 us with 512 blocks, 15.2 with 1024; with the sub-chunk
// ring, splits of 512, 1024, 2048: step 83.5, 83.0, 85.4 us; Llama-3-8B
// layer 1.964, 1.954, 1.952 ms).
static int shrink_kchunk(int K) { return std::max(1024, round_up(ceil_div(K, hrg::kMaxSplits), 256)); }

// The shrink of nl linears that read the same X (one launch: each item
// loads its X rows once for all of them), on a plan `pl` built for the
// batch.  Linear i's U planes land at P->upart + (i * ksplit + split) *
// split_stride.
static lora_status_t batched_shrink(lora_pool_s* P, int nl, const int32_t* modules, const lora_bf16_t* X,
                                    int32_t T, lora_plan_s* pl, hipStream_t stream) {
  const int K = P->d_in[modules[0]];
  const int kchunk = shrink_kchunk(K);
  const int ksplit = ceil_div(K, kchunk);
  const int max_items = max_tiles_for(P) * ksplit;
  const int grid = std::min(max_items, 1024);
  hrg::ShrinkArgs sa{};
  sa.X = X;
  sa.T = T;
  sa.K = K;
  sa.perm = pl->tab.perm;
  sa.tile_info = pl->tab.tile_info;
  sa.counts = pl->tab.counts;
  sa.pages = P->pages;
  sa.slot_stride = P->slot_elems;
  for (int i = 0; i < nl; ++i) sa.a_off[i] = P->a_off[modules[i]];
  sa.upart = P->upart;
  sa.split_stride = P->split_stride;
  sa.u_ld = P->rpad;
  sa.kchunk = kchunk;
  sa.nsplit = ksplit;
  sa.status = P->status;
  return hrg::launch_shrink(sa, nl, grid, ksplit, T, stream) == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

// The rest of one linear's batched apply: the small-segment expand and the
// GEMM with the fused expand, reading the linear's U planes at `upart`
// (lora), or the plain GEMM (base only).
static lora_status_t batched_finish(lora_pool_s* P, int32_t module, const lora_bf16_t* X, int32_t T,
                                    const lora_bf16_t* W, lora_bf16_t* out, lora_plan_s* pl, float* upart,
                                    bool lora, hipStream_t stream) {
  const int K = P->d_in[module], N = P->d_out[module];
  hrg::GemmArgs ga{};
  ga.X = X;
  ga.W = W;
  ga.out = out;
  ga.T = T;
  ga.N = N;
  ga.K = K;
  ga.status = P->status;
  if (!lora) {
    ga.perm = nullptr;
    return hrg::launch_prefill(ga, false, -1, stream) == hipSuccess ? LORA_OK : LORA_ERR_HIP;
  }
  ga.perm = pl->tab.perm;
  ga.v_hi = P->v_hi;
  ga.v_lo = P->v_lo;
  ga.u_ld = P->rpad;
  ga.row_seg = pl->tab.row_seg;
  ga.seg_id = pl->tab.seg_id;
  ga.seg_off = pl->tab.seg_off;
  ga.seg_slot = pl->tab.seg_slot;
  ga.seg_rank = pl->tab.seg_rank;
  ga.pages = P->pages;
  ga.slot_stride = P->slot_elems;
  ga.b_off = P->b_off[module];
  ga.upart = upart;
  ga.split_stride = P->split_stride;
  ga.nsplit = ceil_div(K, shrink_kchunk(K));
  ga.seg_scale = pl->tab.seg_scale;
  ga.seg_bscale = pl->tab.seg_bscale;
  ga.small_bscale = pl->tab.small_bscale;
  ga.seg_e0 = pl->tab.seg_e0;
  ga.erow = pl->tab.erow;
  ga.small_info = pl->tab.small_info;
  ga.counts = pl->tab.counts;
  ga.E = P->E;
  if (hrg::launch_expand_small(ga, stream) != hipSuccess) return LORA_ERR_HIP;
  return hrg::launch_prefill(ga, true, -1, stream) == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

// Host checks shared by every apply entry point (no side effects on error):
// n distinct linears of one d_in, sizes, pointers, the plan, INT4 rules.
static lora_status_t check_apply(lora_pool_t P, int32_t n, const int32_t* modules, const lora_bf16_t* X,
                                 const int32_t* ids, int32_t T, const lora_bf16_t* const* W,
                                 const uint32_t* const* Wq, const uint32_t* const* Wsz,
                                 lora_bf16_t* scratch, lora_bf16_t* const* out, lora_plan_t plan,
                                 bool lora) {
  if (!P || n < 1 || n > hrg::kMaxGroup || !modules || !out) return LORA_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i) {
    if (!module_ok(P, modules[i])) return LORA_ERR_INVALID_ARG;
    if (P->d_in[modules[i]] != P->d_in[modules[0]]) return LORA_ERR_INVALID_ARG;
    for (int32_t j = 0; j < i; ++j)
      if (modules[j] == modules[i]) return LORA_ERR_INVALID_ARG;
  }
  if (T < 0 || T > P->max_tokens) return LORA_ERR_INVALID_ARG;
  const int K = P->d_in[modules[0]];
  const bool q4 = Wq != nullptr || Wsz != nullptr;
  if (q4 && (!Wq || !Wsz || K % hrg::kQ4Group != 0 || (T > hrg::kDecodeMaxT && !scratch)))
    return LORA_ERR_INVALID_ARG;
  if (T == 0) return LORA_OK;
  if (!X || (!W && !q4) || (lora && !ids)) return LORA_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i) {
    if (!out[i]) return LORA_ERR_INVALID_ARG;
    if (q4 ? (!Wq[i] || !Wsz[i]) : !W[i]) return LORA_ERR_INVALID_ARG;
  }
  if (plan) {
    if (!P->plans.count(plan) || plan->T != T || plan->ids != ids) return LORA_ERR_INVALID_ARG;
  }
  // the batched path addresses X with 32-bit byte offsets
  if (T > hrg::kDecodeMaxT && (size_t)T * K * 2 > (size_t)INT32_MAX) return LORA_ERR_INVALID_ARG;
  return LORA_OK;
}

// The INT4 base weight (Wq, Wsz; W == nullptr) is dequantized in the decode
// kernel's registers, or into the caller's `scratch` (d_out x d_in bf16)
// before each linear's GEMM on the batched path.
static lora_status_t apply_impl(lora_pool_t P, int32_t n, const int32_t* modules, const lora_bf16_t* X,
                                const int32_t* ids, int32_t T, const lora_bf16_t* const* W,
                                const uint32_t* const* Wq, const uint32_t* const* Wsz,
                                lora_bf16_t* scratch, lora_bf16_t* const* out, lora_plan_t plan, bool lora,
                                hipStream_t stream, bool wpacked = false) {
  const lora_status_t st = check_apply(P, n, modules, X, ids, T, W, Wq, Wsz, scratch, out, plan, lora);
  if (st != LORA_OK || T == 0) return st;
  // fragment-tiled weights are the decode kernels' layout only
  if (wpacked && T > hrg::kDecodeMaxT) return LORA_ERR_INVALID_ARG;
  DeviceGuard g(P->device);
  if (T <= hrg::kDecodeMaxT)
    return decode_group(P, n, modules, X, ids, T, W, Wq, Wsz, out, lora, wpacked, P->dec_part, P->dec_upart,
                        stream);
  lora_plan_s* pl = plan;
  if (lora && !pl) {
    // one plan serves every linear of the call
    pl = P->internal;
    const lora_status_t s2 = run_plan(P, ids, T, pl, stream);
    if (s2 != LORA_OK) return s2;
  }
  // the linears in runs of up to L: one shrink launch per run (their U
  // planes side by side in the workspace), then each linear's expand and GEMM
  const int ksplit = ceil_div(P->d_in[modules[0]], shrink_kchunk(P->d_in[modules[0]]));
  const int L = lora ? std::max(1, std::min(hrg::shrink_linears(P->rpad), hrg::kMaxSplits / ksplit)) : n;
  for (int32_t i0 = 0; i0 < n; i0 += L) {
    const int nl = std::min<int>(L, n - i0);
    if (lora) {
      const lora_status_t s1 = batched_shrink(P, nl, modules + i0, X, T, pl, stream);
      if (s1 != LORA_OK) return s1;
    }
    for (int32_t i = i0; i < i0 + nl; ++i) {
      const int32_t m = modules[i];
      const lora_bf16_t* Wi = W ? W[i] : nullptr;
      if (Wq) {
        if (hrg::launch_q4_dequant(Wq[i], Wsz[i], P->d_out[m], P->d_in[m], scratch, stream) != hipSuccess)
          return LORA_ERR_HIP;
        Wi = scratch;
      }
      float* up = P->upart + (size_t)(i - i0) * ksplit * P->split_stride;
      const lora_status_t s3 = batched_finish(P, m, X, T, Wi, out[i], pl, up, lora, stream);
      if (s3 != LORA_OK) return s3;
    }
  }
  return LORA_OK;
}

lora_status_t lora_apply(lora_pool_t P, int32_t module, const lora_bf16_t* X, const int32_t* ids,
                         int32_t T, const lora_bf16_t* W, lora_bf16_t* out, lora_plan_t plan,
                         hipStream_t stream) {
  return apply_impl(P, 1, &module, X, ids, T, &W, nullptr, nullptr, nullptr, &out, plan, true, stream);
}

lora_status_t lora_base_apply(lora_pool_t P, int32_t module, const lora_bf16_t* X, int32_t T,
                              const lora_bf16_t* W, lora_bf16_t* out, hipStream_t stream) {
  return apply_impl(P, 1, &module, X, nullptr, T, &W, nullptr, nullptr, nullptr, &out, nullptr, false, stream);
}

lora_status_t lora_apply_noalloc(lora_pool_t P, int32_t module, const lora_bf16_t* X, const int32_t* ids,
                                 int32_t T, const lora_bf16_t* W, lora_bf16_t* out, hipStream_t stream) {
  const lora_status_t st = check_apply(P, 1, &module, X, ids, T, &W, nullptr, nullptr, nullptr, &out, nullptr, true);
  if (st != LORA_OK || T == 0) return st;
  if (T > hrg::kDecodeMaxT) return LORA_ERR_INVALID_ARG;
  // the partial planes: KS chunks x 64 tokens x the columns (rounded up to
  // 16), then KS x 64 x the padded rank for the shrink
  const int K = P->d_in[module], N = P->d_out[module];
  const size_t ks = (size_t)ceil_div(K, hrg::kDecodeChunk);
  const size_t part = ks * hrg::kDecodeMaxT * round_up(N, 16);
  const size_t part_pad = (part + 63) / 64 * 64;  // the shrink planes start 256-byte aligned
  const size_t upart = ks * hrg::kDecodeMaxT * P->rpad;
  if (part_pad + upart > hrg::kScratchFloats) return LORA_ERR_INVALID_ARG;
  DeviceGuard g(P->device);
  float* scr = nullptr;
  if (hrg::decode_scratch(&scr) != hipSuccess) return (void)hipGetLastError(), LORA_ERR_HIP;
  return decode_group(P, 1, &module, X, ids, T, &W, nullptr, nullptr, &out, true, false, scr, scr + part_pad,
                      stream);
}

lora_status_t lora_apply_group(lora_pool_t P, int32_t n, const int32_t* modules, const lora_bf16_t* X,
                               const int32_t* ids, int32_t T, const lora_bf16_t* const* W,
                               lora_bf16_t* const* out, lora_plan_t plan, hipStream_t stream) {
  if (!W) return LORA_ERR_INVALID_ARG;
  return apply_impl(P, n, modules, X, ids, T, W, nullptr, nullptr, nullptr, out, plan, true, stream);
}

lora_status_t lora_base_apply_group(lora_pool_t P, int32_t n, const int32_t* modules, const lora_bf16_t* X,
                                    int32_t T, const lora_bf16_t* const* W, lora_bf16_t* const* out,
                                    hipStream_t stream) {
  if (!W) return LORA_ERR_INVALID_ARG;
  return apply_impl(P, n, modules, X, nullptr, T, W, nullptr, nullptr, nullptr, out, nullptr, false, stream);
}

lora_status_t lora_pack_weight(const lora_bf16_t* W, int32_t N, int32_t K, lora_bf16_t* Wp, hipStream_t stream) {
  if (!W || !Wp || N < 8 || K < 8 || N > 65536 || K > 65536 || N % 8 || K % 8) return LORA_ERR_INVALID_ARG;
  if ((int64_t)hrg::frag_elems(N, K) * 2 > (int64_t)INT32_MAX) return LORA_ERR_INVALID_ARG;
  hrg::PackArgs pa = {W, Wp, N, N, K, 2};
  return hrg::launch_pack(pa, stream) == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

lora_status_t lora_packed_weight_elems(int32_t N, int32_t K, int64_t* elems) {
  if (!elems || N < 1 || K < 1) return LORA_ERR_INVALID_ARG;
  *elems = (int64_t)hrg::frag_elems(N, K);
  return LORA_OK;
}

lora_status_t lora_apply_group_packed(lora_pool_t P, int32_t n, const int32_t* modules, const lora_bf16_t* X,
                                      const int32_t* ids, int32_t T, const lora_bf16_t* const* Wp,
                                      lora_bf16_t* const* out, hipStream_t stream) {
  if (!Wp) return LORA_ERR_INVALID_ARG;
  return apply_impl(P, n, modules, X, ids, T, Wp, nullptr, nullptr, nullptr, out, nullptr, true, stream, true);
}

lora_status_t lora_base_apply_group_packed(lora_pool_t P, int32_t n, const int32_t* modules,
                                           const lora_bf16_t* X, int32_t T, const lora_bf16_t* const* Wp,
                                           lora_bf16_t* const* out, hipStream_t stream) {
  if (!Wp) return LORA_ERR_INVALID_ARG;
  return apply_impl(P, n, modules, X, nullptr, T, Wp, nullptr, nullptr, nullptr, out, nullptr, false, stream,
                    true);
}

lora_status_t lora_apply_q4(lora_pool_t P, int32_t module, const lora_bf16_t* X, const int32_t* ids,
                            int32_t T, const uint32_t* Wq, const uint32_t* Wsz, lora_bf16_t* W_scratch,
                            lora_bf16_t* out, lora_plan_t plan, hipStream_t stream) {
  if (!Wq || !Wsz) return LORA_ERR_INVALID_ARG;
  return apply_impl(P, 1, &module, X, ids, T, nullptr, &Wq, &Wsz, W_scratch, &out, plan, true, stream);
}

lora_status_t lora_base_apply_q4(lora_pool_t P, int32_t module, const lora_bf16_t* X, int32_t T,
                                 const uint32_t* Wq, const uint32_t* Wsz, lora_bf16_t* W_scratch,
                                 lora_bf16_t* out, hipStream_t stream) {
  if (!Wq || !Wsz) return LORA_ERR_INVALID_ARG;
  return apply_impl(P, 1, &module, X, nullptr, T, nullptr, &Wq, &Wsz, W_scratch, &out, nullptr, false, stream);
}

lora_status_t lora_apply_group_q4(lora_pool_t P, int32_t n, const int32_t* modules, const lora_bf16_t* X,
                                  const int32_t* ids, int32_t T, const uint32_t* const* Wq,
                                  const uint32_t* const* Wsz, lora_bf16_t* W_scratch, lora_bf16_t* const* out,
                                  lora_plan_t plan, hipStream_t stream) {
  if (!Wq || !Wsz) return LORA_ERR_INVALID_ARG;
  return apply_impl(P, n, modules, X, ids, T, nullptr, Wq, Wsz, W_scratch, out, plan, true, stream);
}

lora_status_t lora_base_apply_group_q4(lora_pool_t P, int32_t n, const int32_t* modules, const lora_bf16_t* X,
                                       int32_t T, const uint32_t* const* Wq, const uint32_t* const* Wsz,
                                       lora_bf16_t* W_scratch, lora_bf16_t* const* out, hipStream_t stream) {
  if (!Wq || !Wsz) return LORA_ERR_INVALID_ARG;
  return apply_impl(P, n, modules, X, nullptr, T, nullptr, Wq, Wsz, W_scratch, out, nullptr, false, stream);
}

lora_status_t lora_q4_pack(const uint8_t* q, const uint8_t* z, const lora_bf16_t* s, int32_t N, int32_t K,
                           uint32_t* Wq, uint32_t* Wsz) {
  if (!q || !z || !s || !Wq || !Wsz || N < 1 || K < hrg::kQ4Group || K % hrg::kQ4Group != 0)
    return LORA_ERR_INVALID_ARG;
  const int KW = K / 8, KG = K / hrg::kQ4Group;
  for (size_t i = 0; i < (size_t)N * K; ++i)
    if (q[i] > 15) return LORA_ERR_INVALID_ARG;
  for (size_t i = 0; i < (size_t)N * KG; ++i)
    if (z[i] > 15) return LORA_ERR_INVALID_ARG;
  for (int32_t n = 0; n < N; ++n) {
    for (int g = 0; g < KG; ++g) {
      Wsz[(size_t)n * KG + g] = (uint32_t)s[(size_t)n * KG + g] | ((uint32_t)z[(size_t)n * KG + g] << 16);
      for (int p = 0; p < 16; ++p) {
        const int j = p / 4, st = p % 4;
        uint32_t w = 0;
        for (int e = 0; e < 8; ++e)
          w |= (uint32_t)q[(size_t)n * K + hrg::kQ4Group * g + 32 * st + 8 * j + e] << (4 * e);
        Wq[(size_t)n * KW + 16 * g + p] = w;
      }
    }
  }
  return LORA_OK;
}

lora_status_t lora_status(lora_pool_t P, hipStream_t stream) {
  if (!P) return LORA_ERR_INVALID_ARG;
  DeviceGuard g(P->device);
  int32_t st = 0;
  if (hipStreamSynchronize(stream) != hipSuccess ||
      hipMemcpy(&st, P->status, sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess ||
      hrg::launch_clear_i32(P->status, 1, 0, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess) {
    (void)hipGetLastError();
    return LORA_ERR_HIP;
  }
  return (lora_status_t)st;
}

lora_status_t lora_debug_read_plan(lora_pool_t P, lora_plan_t plan, int32_t* perm, int32_t* inv,
                                   int32_t* seg_id, int32_t* seg_off, int32_t* T_out,
                                   int32_t* S_out, hipStream_t stream) {
  if (!P) return LORA_ERR_INVALID_ARG;
  lora_plan_s* pl = plan ? plan : P->internal;
  if (plan && !P->plans.count(plan)) return LORA_ERR_INVALID_ARG;
  if (pl->T < 0) return LORA_ERR_INVALID_ARG;  // never built
  DeviceGuard g(P->device);
  int32_t counts[4] = {0, 0, 0, 0};
  if (hipStreamSynchronize(stream) != hipSuccess ||
      hipMemcpy(counts, pl->tab.counts, sizeof(counts), hipMemcpyDeviceToHost) != hipSuccess)
    return (void)hipGetLastError(), LORA_ERR_HIP;
  const int32_t T = pl->T, S = counts[0];
  if (T_out) *T_out = T;
  if (S_out) *S_out = S;
  if (S < 0 || S > T + 1) return LORA_ERR_HIP;
  bool ok = true;
  if (perm && T) ok &= hipMemcpy(perm, pl->tab.perm, T * 4, hipMemcpyDeviceToHost) == hipSuccess;
  if (inv && T) ok &= hipMemcpy(inv, pl->tab.inv, T * 4, hipMemcpyDeviceToHost) == hipSuccess;
  if (seg_id && S) ok &= hipMemcpy(seg_id, pl->tab.seg_id, S * 4, hipMemcpyDeviceToHost) == hipSuccess;
  if (seg_off) ok &= hipMemcpy(seg_off, pl->tab.seg_off, (S + 1) * 4, hipMemcpyDeviceToHost) == hipSuccess;
  if (!ok) return (void)hipGetLastError(), LORA_ERR_HIP;
  return LORA_OK;
}

}  // extern "C"
