// Grouping a batch by adapter id: a stable counting sort of the tokens by
// (id, original index) with -1 first, the segment table of the maximal runs
// of equal id, and the list of shrink work tiles.  "Group the batch by LoRA
// id" is the "Grouped Multi-LoRA Execution" of the LoRA-Land post (section
// "2. multi-LoRA batch scheduling"); ids are validated here in strict mode
// (icman report section 4.1: reject, never silently serve the base).
#include "common.h"
#include "internal.h"

namespace hrg {

constexpr int kPlanThreads = 1024;
constexpr int kStageTok = 8192;  // tokens whose buckets are staged in LDS at a time

// One workgroup.  LDS: start[nb] (bucket counts, then exclusive offsets, then
// placement cursors) and segidx[nb] (segment index of each non-empty bucket),
// nb = max_ids + 1; bucket b holds id b - 1.
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
  extern __shared__ int smem[];
  const int nb = a.max_ids + 1;
  int* start = smem;
  int* segidx = smem + nb;
  __shared__ int s_err;
  __shared__ int s_wsum[2][kPlanThreads / 64];
  __shared__ int s_tot[2];
  __shared__ uint16_t s_bucket[kStageTok];  // id + 1 of the tokens of one placement block
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.T;
  if (*a.status != 0) return;  // a sticky error is pending: leave the tables alone

  if (tid == 0) s_err = 0;
  for (int b = tid; b < nb; b += kPlanThreads) start[b] = 0;
  __syncthreads();

  // 1. validate every id and count tokens per bucket
  for (int t = tid; t < T; t += kPlanThreads) {
    const int id = a.ids[t];
    if (id < -1 || id >= a.max_ids) {
      atomicMax(&s_err, kStatusIdRange);
    } else {
      if (id >= 0 && a.id2slot[id] < 0) atomicMax(&s_err, kStatusNotLoaded);
      atomicAdd(&start[id + 1], 1);
    }
  }
  __syncthreads();
  if (s_err != 0) {
    if (tid == 0) atomicMax(a.status, s_err);
    return;
  }

  // 2. exclusive scans: counts -> bucket start offsets, non-empty -> segment index
  const int per = (nb + kPlanThreads - 1) / kPlanThreads;
  const int b0 = min(nb, tid * per), b1 = min(nb, b0 + per);
  int csum = 0, nsum = 0;
  for (int b = b0; b < b1; ++b) {
    const int c = start[b];
    csum += c;
    nsum += (c > 0);
  }
  const int ci = wave_incl_scan(csum), ni = wave_incl_scan(nsum);
  if (lane == 63) {
    s_wsum[0][wave] = ci;
    s_wsum[1][wave] = ni;
  }
  __syncthreads();
  if (wave == 0) {
    const int nw = kPlanThreads / 64;
    const int v0 = lane < nw ? s_wsum[0][lane] : 0, v1 = lane < nw ? s_wsum[1][lane] : 0;
    const int i0 = wave_incl_scan(v0), i1 = wave_incl_scan(v1);
    if (lane < nw) {
      s_wsum[0][lane] = i0 - v0;
      s_wsum[1][lane] = i1 - v1;
    }
    if (lane == nw - 1) {
      s_tot[0] = i0;
      s_tot[1] = i1;
    }
  }
  __syncthreads();
  int crun = s_wsum[0][wave] + ci - csum, nrun = s_wsum[1][wave] + ni - nsum;
  for (int b = b0; b < b1; ++b) {
    const int c = start[b];
    start[b] = crun;
    segidx[b] = nrun;
    crun += c;
    nrun += (c > 0);
  }
  __syncthreads();
  const int S = s_tot[1];

  // 3. segment table (ascending id, -1 first)
  for (int b = tid; b < nb; b += kPlanThreads) {
    const int nxt = (b + 1 < nb) ? start[b + 1] : T;
    if (nxt > start[b]) {
      const int s = segidx[b];
      const int id = b - 1;
      const int slot = id >= 0 ? a.id2slot[id] : -1;
      a.tab.seg_id[s] = id;
      a.tab.seg_off[s] = start[b];
      a.tab.seg_slot[s] = slot;
      a.tab.seg_rank[s] = slot >= 0 ? a.slot_rank[slot] : 0;
      a.tab.seg_scale[s] = slot >= 0 ? a.slot_scale[slot] : 0.f;
    }
  }
  if (tid == 0) {
    a.tab.seg_off[S] = T;
    a.tab.counts[0] = S;
    a.tab.counts[2] = T;
  }
  __syncthreads();

  if (wave == 1) {
    // 4b. shrink work tiles: every adapter segment split into runs of
    // kShrinkRows sorted rows (the base segment has no tiles).
    int run = 0;
    for (int base = 0; base < S; base += 64) {
      const int s = base + lane;
      int nt = 0, off0 = 0;
      if (s < S && a.tab.seg_id[s] >= 0) {
        off0 = a.tab.seg_off[s];
        nt = (a.tab.seg_off[s + 1] - off0 + kShrinkRows - 1) / kShrinkRows;
      }
      const int inc = wave_incl_scan(nt);
      const int o = run + inc - nt;
      for (int j = 0; j < nt; ++j) {
        if (o + j < a.tab.max_tiles) {
          a.tab.tile_seg[o + j] = s;
          a.tab.tile_row0[o + j] = off0 + j * kShrinkRows;
        }
      }
      run += __shfl(inc, 63, 64);
    }
    if (lane == 0) a.tab.counts[1] = min(run, a.tab.max_tiles);
  }

  if (wave == 2) {
    // 4c. small segments (adapter segments of at most kSmallRows tokens): E
    // rows in segment order while they fit in kMaxSmallRows
    int rows_run = 0, n_small = 0;
    for (int base = 0; base < S; base += 64) {
      const int s = base + lane;
      int rows = 0;
      if (s < S && a.tab.seg_id[s] >= 0) {
        const int len = a.tab.seg_off[s + 1] - a.tab.seg_off[s];
        if (len <= kSmallRows) rows = len;
      }
      const int inc = wave_incl_scan(rows);
      const int e0 = rows_run + inc - rows;
      const bool take = rows > 0 && e0 + rows <= kMaxSmallRows;
      const uint64_t tk = __ballot(take);
      if (s < S) a.tab.seg_e0[s] = take ? e0 : -1;
      if (take) a.tab.small_seg[n_small + __popcll(tk & ((1ull << lane) - 1ull))] = s;
      n_small += __popcll(tk);
      rows_run += __shfl(inc, 63, 64);
    }
    if (lane == 0) a.tab.counts[3] = n_small;
  }

  // 4a. stable placement in blocks of kStageTok tokens whose buckets are
  // staged in LDS by all waves; wave 0 then places the block, 64 at a time.
  for (int blk0 = 0; blk0 < T; blk0 += kStageTok) {
    const int blk1 = min(T, blk0 + kStageTok);
    __syncthreads();  // the previous block is placed
    for (int t = blk0 + tid; t < blk1; t += kPlanThreads) s_bucket[t - blk0] = (uint16_t)(a.ids[t] + 1);
    __syncthreads();
    if (wave == 0) {
      for (int base = blk0; base < blk1; base += 64) {
        const int t = base + lane;
        const bool valid = t < blk1;
        const int b = valid ? (int)s_bucket[t - blk0] : -1;
        uint64_t todo = __ballot(valid);
        int leader = 0, rank = 0, cnt = 0;
        while (todo) {
          const int ld = __builtin_ctzll(todo);  // wave-uniform
          const int vb = __builtin_amdgcn_readlane(b, ld);
          const uint64_t m = __ballot(b == vb) & todo;
          if ((m >> lane) & 1ull) {
            leader = ld;
            rank = __popcll(m & ((1ull << lane) - 1ull));
            cnt = __popcll(m);
          }
          todo &= ~m;
        }
        int first = 0;
        if (valid && lane == leader) first = atomicAdd(&start[b], cnt);
        const int pos = __shfl(first, leader, 64) + rank;
        if (valid) {
          a.tab.perm[pos] = t;
          a.tab.inv[t] = pos;
          a.tab.row_seg[pos] = segidx[b];
        }
      }
    }
  }

  // 5. E row of every sorted position (-1 outside the small segments)
  __syncthreads();
  for (int p = tid; p < T; p += kPlanThreads) {
    const int sg = a.tab.row_seg[p];
    const int e0 = a.tab.seg_e0[sg];
    a.tab.erow[p] = e0 >= 0 ? e0 + p - a.tab.seg_off[sg] : -1;
  }
}

hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
  const size_t lds = 2 * (size_t)(a.max_ids + 1) * sizeof(int);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)plan_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       2 * (kMaxIds + 1) * (int)sizeof(int));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), lds, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Small kernels of the load / unload path.

// Writes one adapter page.  Ranks q >= rank are zero ("mixed ranks are
// aligned to the maximum rank", vLLM chapter "Multi-LoRA hot-plug",
// performance notes).  A arrives d_in x r and is stored rank-major (A^T,
// rows x d_in); B arrives r x d_out and is stored as B^T in 16-rank chunks
// (rows/16 x d_out x 16), so a 16-byte read gives 8 ranks of one column.
__global__ void pack_kernel(PackArgs a) {
  const size_t n = (size_t)a.rows * a.cols;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    int q, c;
    if (a.mode == 0) {  // A^T [rows][cols]
      q = (int)(i / a.cols);
      c = (int)(i % a.cols);
    } else {  // B^T chunks [rows/16][cols][16]
      const size_t chunk = i / ((size_t)a.cols * 16), rem = i % ((size_t)a.cols * 16);
      c = (int)(rem / 16);
      q = (int)(chunk * 16 + rem % 16);
    }
    uint16_t v = 0;
    if (q < a.rank) v = a.mode == 0 ? a.src[(size_t)c * a.rank + q] : a.src[(size_t)q * a.cols + c];
    a.dst[i] = v;
  }
}

hipError_t launch_pack(const PackArgs& a, hipStream_t s) {
  const size_t n = (size_t)a.rows * a.cols;
  const int grid = (int)std::min<size_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(pack_kernel, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

// Routing-table update of one id: the id -> slot map, the per-slot rank and
// scale, and the packed per-id entry {slot, rank, scale} the decode kernels
// read with one load.
__global__ void set_slot_kernel(int32_t* id2slot, int32_t* slot_rank, float* slot_scale, int4* id_info,
                                int32_t id, int32_t slot, int32_t rank, float scale) {
  if (threadIdx.x == 0) {
    if (slot >= 0) {
      slot_rank[slot] = rank;
      slot_scale[slot] = scale;
    }
    id2slot[id] = slot;
    id_info[id] = make_int4(slot, slot >= 0 ? rank : 0, __builtin_bit_cast(int, scale), 0);
  }
}

hipError_t launch_set_slot(int32_t* id2slot, int32_t* slot_rank, float* slot_scale, int4* id_info,
                           int32_t id, int32_t slot, int32_t rank, float scale, hipStream_t s) {
  hipLaunchKernelGGL(set_slot_kernel, dim3(1), dim3(64), 0, s, id2slot, slot_rank, slot_scale, id_info,
                     id, slot, rank, scale);
  return hipGetLastError();
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
