// Host-side state of a pool and a plan, shared by the C-ABI sources.
#pragma once
#include <hip/hip_runtime.h>

#include <set>
#include <vector>

#include "internal.h"
#include "lora.h"

namespace hrg {
// Prefetch calls whose start events are kept (the release point of an
// evicted adapter's slot); older release points fall back to the current call.
constexpr int kCallEvents = 64;
}  // namespace hrg

struct lora_plan_s {
  hrg::PlanTables tab;
  int32_t T = -1;
  const int32_t* ids = nullptr;
  void* block = nullptr;  // one allocation backing every table
};

struct lora_pool_s {
  int device = 0;
  int32_t max_adapters = 0, max_ids = 0, max_rank = 0, rpad = 0, n_modules = 0, max_tokens = 0;
  std::vector<int32_t> d_in, d_out;
  std::vector<size_t> a_off, b_off;  // element offsets of each module's pages inside a slot
  size_t slot_elems = 0;
  uint16_t* pages = nullptr;         // [max_adapters][slot_elems]
  int32_t* id2slot = nullptr;        // [max_ids]
  int32_t* slot_rank = nullptr;      // [max_adapters]
  float* slot_scale = nullptr;       // [max_adapters]
  int4* id_info = nullptr;           // [max_ids] {slot, rank, scale bits, module mask}
  float4* id_bscale = nullptr;       // [max_ids] scale of each 16-rank block (chains: per member)
  int32_t* status = nullptr;         // sticky device status
  uint16_t* staging = nullptr;       // one module's A or B as received
  float* upart = nullptr;            // [kMaxSplits][max_tokens][rpad] shrink partial planes (those of a
                                     // run of linears side by side, linear-major)
  size_t split_stride = 0;
  uint16_t* v_hi = nullptr;          // [max_tokens][rpad] s * U, bf16 high part (sorted rows)
  uint16_t* v_lo = nullptr;          // [max_tokens][rpad] bf16 low part
  // decode-path workspace
  float* E = nullptr;                // [kMaxSmallRows][max d_out] small-segment expand rows
  float* dec_part = nullptr;         // [ceil(max d_in / 1024)][64][max d_out rounded up to 64] base partials
  float* dec_upart = nullptr;        // [ceil(max d_in / 1024)][64][rpad] shrink partials
  std::vector<int32_t> h_id2slot, h_slot_rank;
  std::vector<int32_t> h_mask;       // [max_ids] modules a loaded or registered id targets (bit m)
  std::vector<uint8_t> h_chain;      // [max_ids] the id is a chain (lora_load_chain)
  std::vector<float> h_slot_scale;
  std::set<int32_t> free_slots;      // lowest free slot first
  lora_plan_s* internal = nullptr;
  std::set<lora_plan_s*> plans;
  // host cache and LRU paging (paging.hip); empty until lora_host_cache_create
  uint16_t* hcache = nullptr;        // pinned host [max_cpu][slot_elems], the device page layout
  void* hcache_dev = nullptr;        // its device mapping (read by the page-in kernel)
  int32_t max_cpu = 0;
  std::vector<int32_t> h_hslot;      // [max_ids] host-cache slot of a registered id (-1: none)
  std::vector<int32_t> h_hrank;      // [max_ids] rank of a registered id
  std::vector<float> h_hscale;       // [max_ids] alpha / rank of a registered id
  std::set<int32_t> free_hslots;
  std::vector<int32_t> cached;       // [max_ids] device slot holding a registered id's pages (-1)
  std::set<int32_t> cached_ids;
  std::vector<int64_t> last_use;     // [max_ids] number of the last prefetch that named the id
  std::vector<uint8_t> pinned;       // [max_ids]
  std::vector<int32_t> named;        // registered ids named by the last prefetch
  int64_t calls = 0;                 // prefetch calls so far
  int64_t pages_loaded = 0;          // host -> device slot copies so far (prefetch and pin)
  hipStream_t copy_stream = nullptr; // host -> device page copies
  hipEvent_t call_ev[hrg::kCallEvents] = {};  // recorded on the caller's stream as each prefetch starts
  hipEvent_t copy_ev = nullptr;      // the last prefetch's copies done
};

namespace hrg {

// The module mask of an adapter given its A and B pointer arrays: bit m set
// when module m has pages (modules >= 32 always count as targeted).  Returns
// false if a module has only one of A, B, if no module is targeted, or if a
// pool of more than 32 modules gets an adapter without some module.
inline bool target_mask(int32_t n_modules, const void* const* A, const void* const* B, int32_t* mask) {
  uint32_t m = 0xffffffffu;
  int present = 0;
  for (int32_t i = 0; i < n_modules; ++i) {
    if (!A[i] != !B[i]) return false;
    if (A[i]) {
      ++present;
    } else {
      if (i >= 32) return false;
      m &= ~(1u << i);
    }
  }
  if (present == 0) return false;
  *mask = (int32_t)m;
  return true;
}

// Drops the device copy of host-cached adapter `id` (NOT_LOADED if it has
// none); its host copy stays.  Synchronises `stream`.
lora_status_t paged_drop_device_copy(lora_pool_s* P, int32_t id, hipStream_t stream);

// Makes `dev` current for the scope of a call and restores the caller's device.
struct DeviceGuard {
  int prev = -1;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev) (void)hipSetDevice(dev);
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

}  // namespace hrg
