// Grouping a batch by adapter id: a stable counting sort of the tokens by
// (id, original index) with -1 first, the segment table of the maximal runs
// of equal id, and the list of shrink work tiles.  "Group the batch by LoRA
// id" is the "Grouped Multi-LoRA Execution" of the LoRA-Land post (section
// "2. multi-LoRA batch scheduling"); ids are validated here in strict mode
// (icman report section 4.1: reject, never silently serve the base).
#include <atomic>
#include <map>
#include <mutex>

#include "common.h"
#include "internal.h"

namespace hrg {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;
constexpr int kStageTok = 8192;  // tokens whose buckets are staged in LDS at a time

// Waves that place tokens in parallel: each takes a contiguous share of a
// staged block and owns a row of nb cursors in LDS (PW * nb ints, <= 64 KB).
__host__ __device__ inline int plan_place_waves(int nb) {
  return nb <= 1024 ? 16 : nb <= 2048 ? 8 : nb <= 4096 ? 4 : 1;
}

// Exclusive prefix sums, in thread order over the workgroup, of three
// per-thread values; tot[] gets the totals.
__device__ __forceinline__ void block_excl_scan3(int v[3], int* tot, int (*red)[kPlanWaves]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int inc[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    inc[i] = wave_incl_scan(v[i]);
    if (lane == 63) red[i][wave] = inc[i];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int x = lane < kPlanWaves ? red[i][lane] : 0;
      const int xi = wave_incl_scan(x);
      if (lane < kPlanWaves) red[i][lane] = xi - x;
      if (lane == 63) tot[i] = xi;  // lanes past the last wave add zeros
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 3; ++i) v[i] = red[i][wave] + inc[i] - v[i];
}

// One workgroup.  LDS: start[nb] (bucket counts, then exclusive offsets, then
// running bases), segidx[nb] (segment index of each non-empty bucket) and,
// with PW > 1, PW rows of nb placement cursors; nb = max_ids + 1, bucket b
// holds id b - 1.  Dependent global rounds: the ids, one id_info lookup per
// token (validation) and one per segment (its table entry); the rest works
// from LDS and registers.
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
  extern __shared__ int smem[];
  const int nb = a.max_ids + 1;
  const int PW = plan_place_waves(nb);
  const int nbits = 32 - __builtin_clz((unsigned)nb);  // bits of a bucket number (nb >= 1)
  int* start = smem;
  int* segidx = smem + nb;
  int* cur = smem + 2 * nb;  // [PW][nb] when PW > 1
  __shared__ int s_err, s_nsmall;
  __shared__ int s_red[3][kPlanWaves];
  __shared__ int s_tot[3];
  __shared__ uint16_t s_bucket[kStageTok];  // id + 1 of the tokens of one placement block
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.T;
  // a sticky error pending leaves the tables alone; the status is checked
  // once the ids are in (until then only LDS is written)
  const int st = *a.status;

  if (tid == 0) {
    s_err = 0;
    s_nsmall = 0;
  }
  for (int b = tid; b < nb; b += kPlanThreads) start[b] = 0;
  __syncthreads();

  // 1. validate every id and count tokens per bucket (a wave takes 64
  // consecutive tokens at a time, every lane through every round)
  for (int base = tid - lane; base < T; base += kPlanThreads) {
    const int t = base + lane;
    const int id = t < T ? a.ids[t] : -1;
    const bool ok = t < T && id >= -1 && id < a.max_ids;
    if (t < T && !ok) atomicMax(&s_err, kStatusIdRange);
    if (ok) {
      if (id >= 0 && a.id_info[id].x < 0) atomicMax(&s_err, kStatusNotLoaded);
      if (t < kStageTok) s_bucket[t] = (uint16_t)(id + 1);  // the first placement block, staged now
    }
    count_runs(start, id + 1, ok);
  }
  if (st != 0) return;
  __syncthreads();
  if (s_err != 0) {
    if (tid == 0) atomicMax(a.status, s_err);
    return;
  }
  // E rows: none until the small segments below claim theirs (the barrier
  // after the scans orders these stores before those)
  for (int p = tid; p < T; p += kPlanThreads) a.tab.erow[p] = -1;

  // 2. exclusive scans: counts -> bucket start offsets, non-empty -> segment index
  const int per = (nb + kPlanThreads - 1) / kPlanThreads;
  const int b0 = min(nb, tid * per), b1 = min(nb, b0 + per);
  {
    int v[3] = {0, 0, 0};
    for (int b = b0; b < b1; ++b) {
      v[0] += start[b];
      v[1] += start[b] > 0;
    }
    block_excl_scan3(v, s_tot, s_red);
    int crun = v[0], nrun = v[1];
    for (int b = b0; b < b1; ++b) {
      const int c = start[b];
      start[b] = crun;
      segidx[b] = nrun;
      crun += c;
      nrun += (c > 0);
    }
  }
  __syncthreads();
  const int S = s_tot[1];

  // 3. segment table (ascending id, -1 first), then the shrink tiles (each
  // adapter segment cut into runs of kShrinkRows sorted rows) and the small
  // segments (adapter segments of at most kSmallRows tokens; E rows in
  // segment order while they fit in kMaxSmallRows), placed by prefix sums
  // over the threads' buckets.  The counts need only the bucket sizes; the
  // id_info lookups and every table write come in the second pass.
  int v3[3] = {0, 0, 0};  // tiles, small rows, small segments
  for (int b = b0; b < b1; ++b) {
    const int nxt = (b + 1 < nb) ? start[b + 1] : T;
    const int len = nxt - start[b];
    if (len > 0 && b > 0) {
      v3[0] += (len + kShrinkRows - 1) / kShrinkRows;
      if (len <= kSmallRows) {
        v3[1] += len;
        v3[2] += 1;
      }
    }
  }
  block_excl_scan3(v3, s_tot, s_red);
  for (int b = b0; b < b1; ++b) {
    const int nxt = (b + 1 < nb) ? start[b + 1] : T;
    const int off = start[b], len = nxt - off;
    if (len <= 0) continue;
    const int s = segidx[b];
    const int id = b - 1;
    const int4 inf = id >= 0 ? a.id_info[id] : make_int4(-1, 0, 0, 0);
    const float sc0 = id >= 0 ? __builtin_bit_cast(float, inf.z) : 0.f;
    // a chain's blocks have their own scales (one more load, chains only)
    const float4 bsc = id >= 0 && (inf.y & kChainRankFlag) ? a.id_bscale[id] : make_float4(sc0, sc0, sc0, sc0);
    const int rank = id >= 0 ? (inf.y & (kChainRankFlag - 1)) : 0;
    a.tab.seg_bscale[s] = bsc;
    a.tab.seg_id[s] = id;
    a.tab.seg_off[s] = off;
    a.tab.seg_slot[s] = inf.x;
    a.tab.seg_rank[s] = rank;
    a.tab.seg_scale[s] = id >= 0 ? __builtin_bit_cast(float, inf.z) : 0.f;
    int e0 = -1;
    if (id >= 0) {
      const int nt = (len + kShrinkRows - 1) / kShrinkRows;
      for (int j = 0; j < nt; ++j) {
        if (v3[0] + j < a.tab.max_tiles)
          a.tab.tile_info[v3[0] + j] =
              make_int4(off + j * kShrinkRows, min(kShrinkRows, len - j * kShrinkRows), inf.x, rank);
      }
      v3[0] += nt;
      if (len <= kSmallRows) {
        if (v3[1] + len <= kMaxSmallRows) {
          e0 = v3[1];
          a.tab.small_info[v3[2]] = make_int4(off, len | (e0 << 8) | (rank << 20), inf.x, inf.z);
          a.tab.small_bscale[v3[2]] = bsc;
          atomicMax(&s_nsmall, v3[2] + 1);
          for (int i = 0; i < len; ++i) a.tab.erow[off + i] = e0 + i;
        }
        v3[1] += len;
        v3[2] += 1;
      }
    }
    a.tab.seg_e0[s] = e0;
  }
  __syncthreads();  // s_nsmall, s_tot
  if (tid == 0) {
    a.tab.seg_off[S] = T;
    a.tab.counts[0] = S;
    a.tab.counts[1] = min(s_tot[0], a.tab.max_tiles);
    a.tab.counts[2] = T;
    a.tab.counts[3] = s_nsmall;
  }

  // 4. stable placement, in blocks of kStageTok tokens whose buckets are
  // staged in LDS.  PW waves each take a contiguous share of a block:
  // per-wave bucket counts (LDS atomics), then for each bucket its running
  // base plus the counts of the waves before, then each wave places its
  // share 64 tokens at a time (one cursor update per distinct bucket among
  // the 64; a token's rank among its bucket's lanes keeps token order).
  for (int blk0 = 0; blk0 < T; blk0 += kStageTok) {
    const int blk1 = min(T, blk0 + kStageTok);
    const int share = (blk1 - blk0 + PW - 1) / PW;
    __syncthreads();  // the previous block is placed
    if (blk0 > 0)
      for (int t = blk0 + tid; t < blk1; t += kPlanThreads) s_bucket[t - blk0] = (uint16_t)(a.ids[t] + 1);
    if (PW > 1)
      for (int i = tid; i < PW * nb; i += kPlanThreads) cur[i] = 0;
    __syncthreads();
    const int t0 = PW > 1 ? blk0 + wave * share : blk0;
    const int t1 = PW > 1 ? min(blk1, t0 + share) : blk1;
    int* mycur = PW > 1 ? cur + wave * nb : start;
    if (PW > 1) {
      if (wave < PW) {
        // counts only: the order of the LDS increments does not matter
        for (int t = t0 + lane; t - lane < t1; t += 64) {
          const bool in = t < t1;
          count_runs(mycur, in ? (int)s_bucket[t - blk0] : 0, in);
        }
      }
      __syncthreads();
      for (int b = tid; b < nb; b += kPlanThreads) {
        int run = start[b];
        for (int w = 0; w < PW; ++w) {
          const int c = cur[w * nb + b];
          cur[w * nb + b] = run;
          run += c;
        }
        start[b] = run;
      }
      __syncthreads();
    }
    if (wave < PW) {
      for (int base = t0; base < t1; base += 64) {
        const int t = base + lane;
        const bool valid = t < t1;
        const int b = valid ? (int)s_bucket[t - blk0] : -1;
        // m = the lanes holding this lane's bucket: one ballot per bit of
        // the bucket number, each lane keeping the lanes that agree with it
        // on that bit
        uint64_t m = __ballot(valid);
        for (int k = 0; k < nbits; ++k) {
          const bool bit = (b >> k) & 1;
          const uint64_t on = __ballot(valid && bit);
          m &= bit ? on : ~on;
        }
        const int leader = valid ? __builtin_ctzll(m) : 0;  // the bucket's first lane
        const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
        const int cnt = __popcll(m);
        int first = 0;
        if (valid && lane == leader) {
          first = mycur[b];
          mycur[b] = first + cnt;
        }
        const int pos = __shfl(first, leader, 64) + rank;
        if (valid) {
          a.tab.perm[pos] = t;
          a.tab.inv[t] = pos;
          a.tab.row_seg[pos] = segidx[b];
        }
      }
    }
  }
}

hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
  const int nb = a.max_ids + 1;
  const int pw = plan_place_waves(nb);
  const size_t lds = (size_t)(2 + (pw > 1 ? pw : 0)) * nb * sizeof(int);
  // the dynamic LDS limit, raised once per device (setting it twice from
  // racing threads is harmless)
  static std::atomic<uint64_t> attr_devices{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? 1ull << dev : 0;
  if (bit == 0 || (attr_devices.load(std::memory_order_acquire) & bit) == 0) {
    // the most any nb needs: 2 (kMaxIds + 1) ints with pw = 1; with pw > 1,
    // (2 + pw) nb <= 6 * 4096 ints is less
    e = hipFuncSetAttribute((const void*)plan_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            2 * (kMaxIds + 1) * (int)sizeof(int));
    if (e != hipSuccess) return e;
    attr_devices.fetch_or(bit, std::memory_order_release);
  }
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), lds, s, a);
  return hipGetLastError();
}

int resident_blocks(const void* fn, int threads, size_t lds) {
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, int> cache;  // (kernel, device) -> blocks
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find({fn, dev});
  if (it != cache.end()) return it->second;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, lds) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    return 1;
  }
  const int n = std::max(1, per_cu * cus);
  cache[{fn, dev}] = n;
  return n;
}

// ---------------------------------------------------------------------------
// Small kernels of the load / unload path.

// Writes one adapter page.  Ranks q >= rank are zero ("mixed ranks are
// aligned to the maximum rank", vLLM chapter "Multi-LoRA hot-plug",
// performance notes).  A arrives d_in x r and is stored rank-major (A^T,
// rows x d_in); B arrives r x d_out and is stored as B^T in 16-rank chunks
// (rows/16 x d_out x 16), so a 16-byte read gives 8 ranks of one column.
__global__ void pack_kernel(PackArgs a) {
  // every destination element once: (row, column) of the padded page, then
  // its place in the layout (zeros past the source's rows and columns)
  const int cp = a.mode == 1 ? a.cols : round_up(a.cols, 32);
  const size_t n = a.mode == 1 ? (size_t)a.rows * a.cols : frag_elems(a.rows, a.cols);
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    int q, c;
    size_t d;
    if (a.mode != 1) {  // fragment tiles
      q = (int)(i / cp);
      c = (int)(i % cp);
      d = frag_index(q, c, a.rows, a.cols);
    } else {  // B^T chunks [rows/16][cols][16]
      const size_t chunk = i / ((size_t)a.cols * 16), rem = i % ((size_t)a.cols * 16);
      c = (int)(rem / 16);
      q = (int)(chunk * 16 + rem % 16);
      d = i;
    }
    uint16_t v = 0;
    if (q < a.rank && c < a.cols) v = a.mode == 0 ? a.src[(size_t)c * a.rank + q] : a.src[(size_t)q * a.cols + c];
    a.dst[d] = v;
  }
}

hipError_t launch_pack(const PackArgs& a, hipStream_t s) {
  const size_t n = a.mode == 1 ? (size_t)a.rows * a.cols : frag_elems(a.rows, a.cols);
  const int grid = (int)std::min<size_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(pack_kernel, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

// Routing-table update of one id: the id -> slot map, the per-slot rank and
// scale, and the packed per-id entry {slot, rank, scale} the decode kernels
// read with one load.
__global__ void set_slot_kernel(int32_t* id2slot, int32_t* slot_rank, float* slot_scale, int4* id_info,
                                float4* id_bscale, int32_t id, int32_t slot, int32_t rank, float scale,
                                int32_t mask, float4 bscale) {
  if (threadIdx.x == 0) {
    if (slot >= 0) {
      slot_rank[slot] = rank & (kChainRankFlag - 1);
      slot_scale[slot] = scale;
    }
    id2slot[id] = slot;
    id_info[id] = make_int4(slot, slot >= 0 ? rank : 0, __builtin_bit_cast(int, scale), slot >= 0 ? mask : 0);
    id_bscale[id] = slot >= 0 ? bscale : make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

hipError_t launch_set_slot(int32_t* id2slot, int32_t* slot_rank, float* slot_scale, int4* id_info,
                           float4* id_bscale, int32_t id, int32_t slot, int32_t rank, float scale,
                           int32_t mask, float4 bscale, hipStream_t s) {
  hipLaunchKernelGGL(set_slot_kernel, dim3(1), dim3(64), 0, s, id2slot, slot_rank, slot_scale, id_info,
                     id_bscale, id, slot, rank, scale, mask, bscale);
  return hipGetLastError();
}

// The same update for up to kSlotUpdatesPerLaunch distinct ids at once
// (passed by value, so the host needs no staging buffer).
struct SlotUpdates {
  int4 u[kSlotUpdatesPerLaunch];  // {id, slot (-1: not addressable), rank, scale bits}
  int32_t mask[kSlotUpdatesPerLaunch];  // modules the adapter targets (bit m: module m)
  int32_t n;
};

__global__ void set_slots_kernel(int32_t* id2slot, int32_t* slot_rank, float* slot_scale, int4* id_info,
                                 float4* id_bscale, SlotUpdates ups) {
  const int i = threadIdx.x;
  if (i < ups.n) {
    const int4 e = ups.u[i];
    if (e.y >= 0) {
      slot_rank[e.y] = e.z;
      slot_scale[e.y] = __builtin_bit_cast(float, e.w);
    }
    id2slot[e.x] = e.y;
    id_info[e.x] = make_int4(e.y, e.y >= 0 ? e.z : 0, e.w, e.y >= 0 ? ups.mask[i] : 0);
    // host-cached adapters have one scale for every rank block
    const float sc = e.y >= 0 ? __builtin_bit_cast(float, e.w) : 0.f;
    id_bscale[e.x] = make_float4(sc, sc, sc, sc);
  }
}

hipError_t launch_set_slots(int32_t* id2slot, int32_t* slot_rank, float* slot_scale, int4* id_info,
                            float4* id_bscale, const int4* updates, const int32_t* masks, int n,
                            hipStream_t s) {
  for (int i0 = 0; i0 < n; i0 += kSlotUpdatesPerLaunch) {
    SlotUpdates ups{};
    ups.n = std::min(kSlotUpdatesPerLaunch, n - i0);
    for (int j = 0; j < ups.n; ++j) {
      ups.u[j] = updates[i0 + j];
      ups.mask[j] = masks[i0 + j];
    }
    hipLaunchKernelGGL(set_slots_kernel, dim3(1), dim3(kSlotUpdatesPerLaunch), 0, s, id2slot, slot_rank,
                       slot_scale, id_info, id_bscale, ups);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Copies whole adapter slots from the pinned host cache (read over the bus
// through its device mapping) into the device pool, all of a prefetch's
// misses in one launch: many separate small DMA copies cost ~14 us each.
struct PageMoves {
  int2 m[kPageMovesPerLaunch];  // {host-cache slot, device slot}
  int32_t n;
};

__global__ void page_in_kernel(const uint4* __restrict__ hc, uint4* __restrict__ pages, PageMoves mv,
                               size_t slot_vec) {
  const size_t total = (size_t)mv.n * slot_vec;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (size_t)gridDim.x * blockDim.x) {
    const size_t k = i / slot_vec, v = i - k * slot_vec;
    const int2 e = mv.m[k];
    pages[(size_t)e.y * slot_vec + v] = hc[(size_t)e.x * slot_vec + v];
  }
}

hipError_t launch_page_in(const void* host_cache_dev, void* pages, const int2* moves, int n,
                          size_t slot_vec, hipStream_t s) {
  for (int i0 = 0; i0 < n; i0 += kPageMovesPerLaunch) {
    PageMoves mv{};
    mv.n = std::min(kPageMovesPerLaunch, n - i0);
    for (int j = 0; j < mv.n; ++j) mv.m[j] = moves[i0 + j];
    const size_t total = (size_t)mv.n * slot_vec;
    const int grid = (int)std::min<size_t>((total + 255) / 256, 1024);
    hipLaunchKernelGGL(page_in_kernel, dim3(grid), dim3(256), 0, s, static_cast<const uint4*>(host_cache_dev),
                       static_cast<uint4*>(pages), mv, slot_vec);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

__global__ void fill_i32_kernel(int32_t* p, int32_t n, int32_t v) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = v;
}

hipError_t launch_clear_i32(int32_t* p, int32_t n, int32_t value, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int grid = std::min((n + 255) / 256, 1024);
  hipLaunchKernelGGL(fill_i32_kernel, dim3(grid), dim3(256), 0, s, p, n, value);
  return hipGetLastError();
}

}  // namespace hrg
