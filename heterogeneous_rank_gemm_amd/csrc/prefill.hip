// Batched path (T > 64): one tiled bf16 MFMA GEMM per linear,
//
//   out[t, :] = bf16( s_i (U_t B_i)  +  X[t, :] W^T ),   i = ids[t],
//
// i.e. the LoRA-Land formula (section "2. multi-LoRA batch scheduling"): the
// shared base product plus every token's own low-rank term, rounded once.  The
// low-rank term enters as the accumulator's starting value ("expand first"),
// then the base product is accumulated on top in K order.  A row's arithmetic
// depends only on its own data (never on its neighbours in the tile), so id -1
// rows equal the base-only call bit for bit and rows may be permuted freely.
//
// Tile: BM tokens x BN output columns, K in steps of 64, 4 waves in a 2 x 2
// grid, each wave (BN/2) x (BM/2) as 32x32x16 MFMA blocks.  The MFMA
// A-operand is the W tile and the B-operand the X tile, so a lane ends up
// with 4 consecutive output columns of one token (8-byte stores).
//
// Operands move HBM -> LDS with buffer_load ... lds (no register staging)
// into 2-4 stages (as many 64-deep K-steps as fit: smaller tiles have shorter
// steps and need more DMA in flight) that live in separate LDS arrays: the
// compiler then knows the reads of one stage never wait for the DMA into the
// others.  One barrier per K-step publishes the next stage; the fragment
// reads of a stage are spread over the MFMAs of the step before, and the DMA
// of the step NS-1 ahead over the first 16-deep MFMA group.  LDS rows are 128 bytes,
// swizzled as chunk ^ (row & 7) ^ ((row >> 3) & 1), which keeps ds_read_b128
// free of bank conflicts.
//
// Out-of-range rows and the K tail read through the buffer resource's range
// check (zeros), so the loop has no branches.  K-steps past K (when their
// count is odd) add exact zeros.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace hrg {
namespace prefill_detail {

typedef __attribute__((address_space(3))) void lds_void_t;
constexpr int kBK = 64;
constexpr uint32_t kOob = 0x80000000u;  // buffer offset beyond every operand (< 2 GiB)

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ bf16x8 masked(bool keep, uint4 v) {
  const uint32_t m = keep ? 0xffffffffu : 0u;
  return __builtin_bit_cast(bf16x8, make_uint4(v.x & m, v.y & m, v.z & m, v.w & m));
}

// XCD-aware tile order: workgroup b runs on XCD (b mod 8); each XCD gets a
// contiguous range of logical tiles, walked in groups of GM token-tiles so
// that neighbours share X and W rows in that XCD's L2.  (256-row tiles: 4;
// the Llama-3-8B layer's base GEMMs 1685 -> 1658 us against groups of 8, 1745
// with 1, 1683 with 2, 1673 with 3, 1656 with 6; 128x128 tiles of the S-LoRA
// pool: 8 and 4 alike.)
template <int GM>
__device__ __forceinline__ void tile_coords(int b, int nblocks, int tiles_m, int tiles_n, int& tm,
                                            int& tn) {
  constexpr int kXcd = 8, kGroupM = GM;
  const int xcd = b % kXcd, idx = b / kXcd;
  const int q = nblocks / kXcd, r = nblocks % kXcd;
  const int logical = xcd * q + min(xcd, r) + idx;
  const int per_group = kGroupM * tiles_n;
  const int g = logical / per_group;
  const int first_m = g * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int in = logical % per_group;
  tm = first_m + in % gsize;
  tn = in / gsize;
}

// Scheduling hint: kM MFMAs with kV buffer loads and kD LDS reads spread
// evenly between them.
template <int kM, int kV, int kD, int Q = 0>
__device__ __forceinline__ void interleave_vd() {
  if constexpr (Q < kM) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    constexpr int nv = kV * (Q + 1) / kM - kV * Q / kM;
    if constexpr (nv > 0) __builtin_amdgcn_sched_group_barrier(0x020, nv, 0);
    constexpr int nd = kD * (Q + 1) / kM - kD * Q / kM;
    if constexpr (nd > 0) __builtin_amdgcn_sched_group_barrier(0x100, nd, 0);
    interleave_vd<kM, kV, kD, Q + 1>();
  }
}

// Scheduling hint: kM MFMAs with kX instructions of class kMask spread
// evenly between them (0x020 = global/buffer load, 0x100 = LDS read).
template <int kM, int kX, int kMask, int Q = 0>
__device__ __forceinline__ void interleave() {
  if constexpr (Q < kM) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    constexpr int n = kX * (Q + 1) / kM - kX * Q / kM;
    if constexpr (n > 0) __builtin_amdgcn_sched_group_barrier(kMask, n, 0);
    interleave<kM, kX, kMask, Q + 1>();
  }
}

// Issues one K-step (64 deep) of the W and X tiles into an LDS stage.  A lane
// whose 16-byte chunk lies past K reads out of range (zeros).  (A helper
// rather than a lambda: with hipcc, a lambda that captures a buffer resource
// inside a template kernel makes the host pass drop the kernel's launch stub.)
template <int NWB, int NXB>
__device__ __forceinline__ void dma_issue(__amdgpu_buffer_rsrc_t rw, __amdgpu_buffer_rsrc_t rx, uint16_t* ws,
                                          uint16_t* xs, const uint32_t* woff, const uint32_t* xoff, int wid,
                                          int c0, int K, int k0) {
  const uint32_t kb0 = (uint32_t)(k0 + c0 * 8 >= K) << 31;
  const uint32_t kb1 = (uint32_t)(k0 + (c0 ^ 1) * 8 >= K) << 31;
  const uint32_t k2 = 2u * (uint32_t)k0;
#pragma unroll
  for (int i = 0; i < NWB; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void_t*)(ws + (wid * NWB + i) * 512), 16,
                                             (woff[i] + k2) | ((i & 1) ? kb1 : kb0), 0, 0, 0);
#pragma unroll
  for (int i = 0; i < NXB; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void_t*)(xs + (wid * NXB + i) * 512), 16,
                                             (xoff[i] + k2) | ((i & 1) ? kb1 : kb0), 0, 0, 0);
}

// Waits until at most N of this wave's buffer loads are outstanding (the
// older ones -- the next stage's DMA -- have landed in LDS) and every LDS
// access has completed, then joins the workgroup barrier.  Unlike
// __syncthreads() it does not wait for the DMA of the stages further ahead.
// The count holds because every vector-memory instruction of the main loop
// is one of the DMA builtins (16 bytes per lane each: nothing to merge); the
// scheduling fences keep the compiler from moving any other memory
// instruction across the wait.
template <int N>
__device__ __forceinline__ void barrier_after_dma() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"i"(N) : "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Calls f(integral_constant<int, S>) for S = 0 .. NS-1, in order.
template <int NS, int S = 0, class F>
__device__ __forceinline__ void for_each_stage(F&& f) {
  if constexpr (S < NS) {
    f(std::integral_constant<int, S>{});
    for_each_stage<NS, S + 1>(f);
  }
}

}  // namespace prefill_detail
using namespace prefill_detail;

// QC: rank chunks of 16 held per segment in the expand (0 for base-only).
template <int BM, int BN, bool LORA, int QC>
__global__ __launch_bounds__(256) void prefill_kernel(GemmArgs a) {
  constexpr int FM = BM / 64, FN = BN / 64;    // 32x32 blocks per wave (tokens, columns)
  constexpr int NXB = BM / 32, NWB = BN / 32;  // 1-KB DMA blocks per wave and stage
  // LDS stages: as many 64-deep K steps as fit in 128-144 KB (2 for 256x256,
  // 3 for 256x128 and 128x256, 4 for 128x128), each in its own arrays
  constexpr int NS = (BM + BN) >= 512 ? 2 : (BM + BN) >= 384 ? 3 : 4;
  __shared__ __attribute__((aligned(16))) uint16_t w0[BN * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t x0[BM * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t w1[BN * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t x1[BM * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t w2[NS > 2 ? BN * kBK : 8];
  __shared__ __attribute__((aligned(16))) uint16_t x2[NS > 2 ? BM * kBK : 8];
  __shared__ __attribute__((aligned(16))) uint16_t w3[NS > 3 ? BN * kBK : 8];
  __shared__ __attribute__((aligned(16))) uint16_t x3[NS > 3 ? BM * kBK : 8];

  // the plan's status is requested with the token order below (one round
  // of loads) and checked before anything is issued on either
  int st = 0;
  if constexpr (LORA) st = *a.status;
  const int T = a.T, N = a.N, K = a.K;
  // this launch's rows: [row0, row1) of the sorted batch (row1 - row0 is a
  // multiple of BM unless row1 = T)
  const int tiles_m = (a.row1 - a.row0 + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  tile_coords<BM >= 256 ? 4 : 8>(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int m0 = a.row0 + tm * BM, n0 = tn * BN;
  const int l = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wid & 1, wm = wid >> 1;

  // ---- DMA addressing: wave wid, instruction i covers rows 8b..8b+7 of block b
  // (b = wid * NB + i); lane l fetches row 8b + l/8, 16-byte chunk
  // (l & 7) ^ swz(row) so that the lane-ordered LDS write lands swizzled.
  const uint16_t* wtile = a.W + (size_t)n0 * K;
  const int wrows = min(BN, N - n0);
  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc((void*)wtile, (short)0, wrows * K * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.X, (short)0, T * K * 2, 0x00020000);
  const int c0 = (l & 7) ^ (l >> 3);  // chunk of even blocks; odd blocks fetch c0 ^ 1
  uint32_t woff[NWB], xoff[NXB];
#pragma unroll
  for (int i = 0; i < NWB; ++i) {
    const int row = 8 * (wid * NWB + i) + (l >> 3);
    woff[i] = row < wrows ? (uint32_t)(row * K + (c0 ^ (i & 1)) * 8) * 2u : kOob;
  }
  // the token order: every load issued (rows past T read row T - 1, then
  // point past the operand), so one wait covers them all; the base-only
  // kernel takes rows in order
#pragma unroll
  for (int i = 0; i < NXB; ++i) {
    const int p = m0 + 8 * (wid * NXB + i) + (l >> 3);
    int tok;
    if constexpr (LORA) tok = a.perm[min(p, T - 1)];
    else tok = p;
    // a row past T: the offset's top bit puts it past the operand (a mask
    // rather than a select, so the load is not moved under a branch)
    xoff[i] = (uint32_t)(tok * K + (c0 ^ (i & 1)) * 8) * 2u | (p < T ? 0u : kOob);
  }
  // the output rows of this lane's 32-row blocks, requested in the same
  // round and held from there (an empty asm below keeps the loads from
  // sinking to the stores, one wait each)
  int otok[FM];
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    const int p = m0 + wm * (BM / 2) + 32 * j + (l & 31);
    if constexpr (LORA) otok[j] = a.perm[min(p, T - 1)];
    else otok[j] = p;
  }
  // also in that round: each 32-row block's E rows and its first and last
  // rows' segments (the expand below starts from them; any load issued
  // after the K-step DMA would wait for all of it)
  int erj[FM], rs0[FM], rs1[FM];
  if constexpr (LORA) {
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int rb = m0 + wm * (BM / 2) + 32 * j;
      erj[j] = a.erow[min(rb + (l & 31), T - 1)];
      rs0[j] = a.row_seg[min(rb, T - 1)];
      rs1[j] = a.row_seg[min(rb + 31, T - 1)];
    }
#pragma unroll
    for (int j = 0; j < FM; ++j) asm volatile("" : "+v"(otok[j]), "+v"(erj[j]), "+v"(rs0[j]), "+v"(rs1[j]));
#pragma unroll
    for (int i = 0; i < NXB; ++i) asm volatile("" : "+v"(xoff[i]));  // formed here, not beside the DMA
  }
  if constexpr (LORA) {
    if (st != 0) return;  // strict mode: a failed plan leaves out untouched
  }
  auto issue = [&](uint16_t* ws, uint16_t* xs, int k0) __attribute__((always_inline)) {
    dma_issue<NWB, NXB>(rw, rx, ws, xs, woff, xoff, wid, c0, K, k0);
  };

  f32x16 acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // DMA of the first NS-1 K-steps; with LoRA it goes out after the E rows'
  // and the first walkers' table loads (which then never wait for it) and
  // before the expand's page loads, so their latencies overlap
  auto prologue = [&]() __attribute__((always_inline)) {
    for_each_stage<NS>([&](auto sc) __attribute__((always_inline)) {
      constexpr int S = decltype(sc)::value;
      if constexpr (S < NS - 1) {
        if constexpr (S == 0) issue(w0, x0, 0);
        else if constexpr (S == 1) issue(w1, x1, kBK);
        else issue(w2, x2, 2 * kBK);
      }
    });
  };
  if constexpr (LORA) {
    // ---- rows of small segments start from their fp32 E rows (the same
    // MFMA chain as below, run by the small-segment launch).  A block with
    // any such row loads for all its lanes, through the buffer range check:
    // a lane of another row, or a column past N, reads zeros (what its
    // accumulator holds), so no load waits behind a branch.
    const __amdgpu_buffer_rsrc_t re =
        __builtin_amdgcn_make_buffer_rsrc((void*)a.E, (short)0, kMaxSmallRows * N * 4, 0x00020000);
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int p = m0 + wm * (BM / 2) + 32 * j + (l & 31);
      const int er = p < T ? erj[j] : -1;
      if (__ballot(er >= 0) == 0) continue;  // wave-uniform
#pragma unroll
      for (int i = 0; i < FN; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = n0 + wn * (BN / 2) + 32 * i + 8 * q + 4 * (l >> 5);
          const uint32_t off = er >= 0 && col < N ? (uint32_t)(er * N + col) * 4u : kOob;
          const float4 v = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(re, off, 0, 0));
          acc[i][j][4 * q + 0] = v.x;
          acc[i][j][4 * q + 1] = v.y;
          acc[i][j][4 * q + 2] = v.z;
          acc[i][j][4 * q + 3] = v.w;
        }
      }
    }

  }
  if constexpr (!LORA) prologue();

  if constexpr (LORA) {
    // ---- expand first: acc = s_i * (U_t B_i) for every token of a (not
    // small) adapter segment.  V = s U arrives from the shrink as bf16 hi +
    // lo parts (V ~= hi + lo to about 2^-16); the B page is stored transposed
    // in 16-rank chunks, [rpad/16][N][16], so both operands are 16-byte reads.
    // Each 32-row block j of the wave walks its own work items (segment,
    // pair of rank chunks).  Its segments' table entries arrive in one round
    // of loads (lane i: the block's i-th segment), so an item's slot, rows
    // and rank are register reads; the FM walkers advance in lockstep through
    // a ring of D items whose B fragments are requested D-1 items ahead.
    // Every ring load is issued (an item past a walker's last, and a chunk
    // past an adapter's rank, go out of range: nothing read, never applied),
    // so the loads' completion is counted exactly.
    constexpr int QB = QC < 2 ? QC : 2;  // rank chunks per work item
    constexpr int kBudget = FN >= 4 ? 96 : 198;  // 256-column tiles keep 256 accumulators live
    // ring of D items in flight per walker: deeper where the tile leaves
    // registers free (one block per compute unit), but never at the cost of
    // running the walkers one after another (each group is its own chain of
    // dependent loads)
    constexpr int kPerWalker4 = 4 * QB * FN * 4 + QC * 8 + 6;
    constexpr int D = (FN * QB <= 4 && FM <= 2 && kPerWalker4 * FM <= kBudget) ? 4 : 2;
    constexpr int kPerWalker = D * QB * FN * 4 + QC * 8 + 6;
    // walkers per group: the expand's registers (V, D B buffers) stay
    // within a budget
    constexpr int JG = kPerWalker * FM <= kBudget ? FM : (kPerWalker * 2 <= kBudget ? 2 : 1);
    const int qc_pool = a.u_ld >> 4;
    const uint16_t* dummy_page = a.pages + a.b_off;  // slot 0: any valid address
#pragma unroll
    for (int g = 0; g < FM / JG; ++g) {
      bf16x8 vh[JG][QC], vl[JG][QC];
      int pj[JG], nit[JG];
      // lane i (mod 32): the block's i-th segment -- first row, end, slot,
      // number of items, first item
      int s_off[JG], s_end[JG], s_slot[JG], s_nqc[JG], s_it0[JG], s_nit[JG];
      int s_rk[JG], s_id[JG], s_e0[JG];
      bool s_mine[JG];
#pragma unroll
      for (int j = 0; j < JG; ++j) {
        const int rb = m0 + wm * (BM / 2) + 32 * (g * JG + j);  // first sorted row of block g*JG+j
        const bool act = rb < T;
        pj[j] = rb + (l & 31);
        const int pc = min(pj[j], T - 1);
#pragma unroll
        for (int qc = 0; qc < QC; ++qc) {
          const size_t e = (size_t)pc * a.u_ld + 16 * qc + 8 * (l >> 5);
          if (act && qc < qc_pool) {
            vh[j][qc] = __builtin_bit_cast(bf16x8, ld16(a.v_hi + e));
            vl[j][qc] = __builtin_bit_cast(bf16x8, ld16(a.v_lo + e));
          } else {
            vh[j][qc] = zero_bf16x8();
            vl[j][qc] = zero_bf16x8();
          }
        }
        const int sg = act ? rs0[g * JG + j] : 0;
        const int sl = act ? rs1[g * JG + j] : -1;
        const int sx = sg + (l & 31);
        const bool mine = sx <= sl && l < 32;
        const int sc = min(sx, max(sl, 0));
        s_off[j] = a.seg_off[sc];
        s_end[j] = a.seg_off[sc + 1];
        s_slot[j] = a.seg_slot[sc];
        s_rk[j] = a.seg_rank[sc];
        s_id[j] = a.seg_id[sc];
        s_e0[j] = a.seg_e0[sc];
        s_mine[j] = mine;
      }
      // the K-step DMA goes out behind the first walkers' loads: vmcnt
      // counts in issue order, so waiting for these does not wait for it
      if (g == 0) prologue();
#pragma unroll
      for (int j = 0; j < JG; ++j) {
        s_nqc[j] = (s_rk[j] + 15) >> 4;
        const bool big = s_mine[j] && s_id[j] >= 0 && s_e0[j] < 0;
        s_nit[j] = big ? (s_nqc[j] + QB - 1) / QB : 0;
        const int inc = wave_incl_scan(s_nit[j]);
        s_it0[j] = inc - s_nit[j];
        nit[j] = __builtin_amdgcn_readlane(inc, 63);
      }
      // item k of walker j: (segment lane, first chunk), or -1 past its last
      auto item_lane = [&](int j, int k) __attribute__((always_inline)) -> int {
        const uint64_t m = __ballot(k >= s_it0[j] && k < s_it0[j] + s_nit[j]);
        return m ? (int)__builtin_ctzll(m) : -1;
      };
      bf16x8 bq[D][JG][QB][FN];
      auto load_b = [&](bf16x8 (&bb)[QB][FN], int j, int k) __attribute__((always_inline)) {
        const int il = item_lane(j, k);
        const uint16_t* bt = dummy_page;
        int c = 0, nq = 0;
        if (il >= 0) {
          bt = a.pages + (size_t)__builtin_amdgcn_readlane(s_slot[j], il) * a.slot_stride + a.b_off;
          c = (k - __builtin_amdgcn_readlane(s_it0[j], il)) * QB;
          nq = __builtin_amdgcn_readlane(s_nqc[j], il);
        }
        // the page through a buffer resource: a chunk past the adapter's
        // rank, or any chunk of an item past the walker's last, is requested
        // out of range (zeros, nothing read; never applied)
        const __amdgpu_buffer_rsrc_t rbt =
            __builtin_amdgcn_make_buffer_rsrc((void*)bt, (short)0, a.u_ld * N * 2, 0x00020000);
#pragma unroll
        for (int qc = 0; qc < QB; ++qc) {
          const bool real = c + qc < nq;
          const uint32_t cq = real ? (uint32_t)(c + qc) : 0u;
#pragma unroll
          for (int i = 0; i < FN; ++i) {
            const int n = min(n0 + wn * (BN / 2) + 32 * i + (l & 31), N - 1);
            const uint32_t off = ((cq * (uint32_t)N + (uint32_t)n) * 16u + 8u * (uint32_t)(l >> 5)) * 2u;
            bb[qc][i] = __builtin_bit_cast(
                bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rbt, off | (real ? 0u : kOob), 0, 0));
          }
        }
      };
      // acc[.][j] += B^T (V masked to the rows of the item's segment), chunks c .. c+QB-1
      auto apply_b = [&](const bf16x8 (&bb)[QB][FN], const bf16x8 (&h_)[QC], const bf16x8 (&l_)[QC],
                         f32x16 (&accj)[FN], int p, int j, int k) __attribute__((always_inline)) {
        const int il = item_lane(j, k);
        if (il < 0) return;
        const int off = __builtin_amdgcn_readlane(s_off[j], il);
        const int end = __builtin_amdgcn_readlane(s_end[j], il);
        const int nqc = __builtin_amdgcn_readlane(s_nqc[j], il);
        const int c = (k - __builtin_amdgcn_readlane(s_it0[j], il)) * QB;
        const bool in = p >= off && p < end;
        const uint32_t m = in ? 0xffffffffu : 0u;
        const uint32_t first = c == 0 ? 0xffffffffu : 0u;  // chunk c + qc is qc or qc + QB
#pragma unroll
        for (int qc = 0; qc < QB; ++qc) {
          if (c + qc < nqc) {
            uint4 h = __builtin_bit_cast(uint4, h_[qc]), o = __builtin_bit_cast(uint4, l_[qc]);
            if constexpr (QC > QB) {
              const uint4 h2 = __builtin_bit_cast(uint4, h_[qc + QB]);
              const uint4 o2 = __builtin_bit_cast(uint4, l_[qc + QB]);
              h = make_uint4((h.x & first) | (h2.x & ~first), (h.y & first) | (h2.y & ~first),
                             (h.z & first) | (h2.z & ~first), (h.w & first) | (h2.w & ~first));
              o = make_uint4((o.x & first) | (o2.x & ~first), (o.y & first) | (o2.y & ~first),
                             (o.z & first) | (o2.z & ~first), (o.w & first) | (o2.w & ~first));
            }
            const bf16x8 mh = __builtin_bit_cast(bf16x8, make_uint4(h.x & m, h.y & m, h.z & m, h.w & m));
            const bf16x8 ml = __builtin_bit_cast(bf16x8, make_uint4(o.x & m, o.y & m, o.z & m, o.w & m));
#pragma unroll
            for (int i = 0; i < FN; ++i) {
              accj[i] = mfma32(bb[qc][i], mh, accj[i]);
              accj[i] = mfma32(bb[qc][i], ml, accj[i]);
            }
          }
        }
      };
      int nmax = 0;
#pragma unroll
      for (int j = 0; j < JG; ++j) nmax = max(nmax, nit[j]);
      if (nmax > 0) {
        f32x16 accT[JG][FN];  // acc transposed so a block's columns pass as one array
#pragma unroll
        for (int j = 0; j < JG; ++j)
#pragma unroll
          for (int i = 0; i < FN; ++i) accT[j][i] = acc[i][g * JG + j];
        // items 0 .. D-2; each phase then requests the item D-1 ahead
        for_each_stage<D - 1>([&](auto dc) __attribute__((always_inline)) {
          constexpr int B = decltype(dc)::value;
#pragma unroll
          for (int j = 0; j < JG; ++j) load_b(bq[B][j], j, B);
        });
        // phase P of round k0: item k0 + P is in bq[P]; item k0 + P + D - 1
        // goes to bq[(P + D - 1) % D]
        bool more = true;
        auto phase = [&](auto pc, int k0) __attribute__((always_inline)) {
          constexpr int P = decltype(pc)::value;
          const int k = k0 + P;
#pragma unroll
          for (int j = 0; j < JG; ++j) load_b(bq[(P + D - 1) % D][j], j, k + D - 1);
#pragma unroll
          for (int j = 0; j < JG; ++j) apply_b(bq[P][j], vh[j], vl[j], accT[j], pj[j], j, k);
          more = k + 1 < nmax;
        };
        for (int k0 = 0; more; k0 += D) {
          phase(std::integral_constant<int, 0>{}, k0);
          if (!more) break;
          phase(std::integral_constant<int, 1>{}, k0);
          if constexpr (D > 2) {
            if (!more) break;
            phase(std::integral_constant<int, 2>{}, k0);
            if (!more) break;
            phase(std::integral_constant<int, 3>{}, k0);
          }
        }
#pragma unroll
        for (int j = 0; j < JG; ++j)
#pragma unroll
          for (int i = 0; i < FN; ++i) acc[i][g * JG + j] = accT[j][i];
      }
    }
  }

  // ---- base product, K-steps of 64 through two LDS stages
  bf16x8 fa[2][FN], fb[2][FM];
  auto rd = [&](const uint16_t* ws, const uint16_t* xs, int kk, int f) __attribute__((always_inline)) {
    const int cc = 2 * kk + (l >> 5);
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const int row = wn * (BN / 2) + 32 * i + (l & 31);
      fa[f][i] = lds_bf16x8(ws + row * kBK + ((cc ^ swz(row)) * 8));
    }
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int row = wm * (BM / 2) + 32 * j + (l & 31);
      fb[f][j] = lds_bf16x8(xs + row * kBK + ((cc ^ swz(row)) * 8));
    }
  };
  auto mm = [&](int f) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j) acc[i][j] = mfma32(fa[f][i], fb[f][j], acc[i][j]);
  };
  // One barrier per K-step.  Between two barriers: the DMA of the step NS-1
  // ahead (into the stage read by the step before), this step's fragment
  // reads, the previous step's last 16-deep MFMA group and this step's first
  // three.  The barrier waits only for the next step's DMA.  The DMA is
  // spread over the MFMA groups: issued in one burst it fills the texture
  // address queue and stalls the issuing wave (SQ_VMEM_TA_CMD_FIFO_FULL).
  // With two stages the DMA must land within the step, so it goes out over
  // the first half; with three or four it may trail, and goes out over the
  // whole step (MI355X: Llama-3-8B layer base-only 1.89 -> 1.80 ms with
  // 256x256 tiles over half a step, 1.88 over the whole; 4096-wide linear
  // with 1024 tokens, 128x128 tiles, 43.4 -> 40.6 us over the whole step).
  constexpr int kM = FN * FM, kD = FN + FM, kV = NWB + NXB;
  // stage S's arrays, named directly (through a pointer table the compiler
  // loses which LDS object a read touches and waits for every DMA in flight)
  auto wst = [&](auto sc) -> uint16_t* {
    constexpr int S = decltype(sc)::value;
    if constexpr (S == 0) return w0;
    else if constexpr (S == 1) return w1;
    else if constexpr (S == 2) return w2;
    else return w3;
  };
  auto xst = [&](auto sc) -> uint16_t* {
    constexpr int S = decltype(sc)::value;
    if constexpr (S == 0) return x0;
    else if constexpr (S == 1) return x1;
    else if constexpr (S == 2) return x2;
    else return x3;
  };
  auto step = [&](uint16_t* ws, uint16_t* xs, uint16_t* wnx, uint16_t* xnx, int knext)
                  __attribute__((always_inline)) {
    issue(wnx, xnx, knext);
    rd(ws, xs, 0, 0);
    mm(1);
    rd(ws, xs, 1, 1);
    mm(0);
    rd(ws, xs, 2, 0);
    mm(1);
    rd(ws, xs, 3, 1);
    mm(0);
    __builtin_amdgcn_sched_group_barrier(0x100, kD, 0);
    if constexpr (NS == 2) {
      interleave<kM, kV / 2, 0x020>();
      interleave_vd<kM, kV - kV / 2, kD>();
      interleave<kM, kD, 0x100>();
      interleave<kM, kD, 0x100>();
    } else {
      interleave<kM, kV / 4, 0x020>();
      interleave_vd<kM, kV / 4, kD>();
      interleave_vd<kM, kV / 4, kD>();
      interleave_vd<kM, kV - 3 * (kV / 4), kD>();
    }
    barrier_after_dma<(NS - 2) * kV>();
  };
#pragma unroll
  for (int i = 0; i < FN; ++i) fa[1][i] = zero_bf16x8();
#pragma unroll
  for (int j = 0; j < FM; ++j) fb[1][j] = zero_bf16x8();
  const int nk = (K + kBK - 1) / kBK;
  // K-steps 0 .. NS-2 went out before the expand
  barrier_after_dma<(NS - 2) * kV>();
  for (int kt = 0; kt < nk; kt += NS) {
    for_each_stage<NS>([&](auto sc) __attribute__((always_inline)) {
      constexpr int S = decltype(sc)::value;
      const auto pc = std::integral_constant<int, (S + NS - 1) % NS>{};  // the stage read last step
      step(wst(sc), xst(sc), wst(pc), xst(pc), (kt + S + NS - 1) * kBK);
    });
  }
  mm(1);

  // ---- single rounding, 4 consecutive columns per lane and 32-row block
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    const int p = m0 + wm * (BM / 2) + 32 * j + (l & 31);
    if (p >= T) continue;
    uint16_t* orow = a.out + (size_t)otok[j] * N;
#pragma unroll
    for (int i = 0; i < FN; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * (BN / 2) + 32 * i + 8 * g + 4 * (l >> 5);
        if (n >= N) continue;  // N % 8 == 0: the 4 columns are all in or all out
        const uint32_t lo = (uint32_t)f32_to_bf16_bits(acc[i][j][4 * g + 0]) |
                            ((uint32_t)f32_to_bf16_bits(acc[i][j][4 * g + 1]) << 16);
        const uint32_t hi = (uint32_t)f32_to_bf16_bits(acc[i][j][4 * g + 2]) |
                            ((uint32_t)f32_to_bf16_bits(acc[i][j][4 * g + 3]) << 16);
        *reinterpret_cast<uint2*>(orow + n) = make_uint2(lo, hi);
      }
    }
  }
}

// Small segments (at most kSmallRows tokens): E[e0 + p - off][n] = s (U_p B)[n]
// in fp32 for every token p of the segment.  In the GEMM such a segment would
// cost a walker item (a full 32-row MFMA block) per segment per column tile,
// all on the few tiles that hold the batch's long tail of rare adapters; here
// the items spread over the whole chip.  One wave per (segment, 128 columns).
// The arithmetic is the GEMM expand's exactly: the same 32-row blocks and
// lanes (rows of other segments masked to zero), the same MFMA, chunk order
// and hi-then-lo order, starting from zero -- so the GEMM, starting those
// rows' accumulators from E, gives the bits it would give walking them.
// sum of the nsplit fp32 planes p[sp * stride] in split order, loads issued
// eight at a time
__device__ __forceinline__ float4 sum_planes4(const float* p, size_t stride, int nsplit) {
  float4 u = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < nsplit; s0 += 8) {
    float4 pv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) pv[j] = *reinterpret_cast<const float4*>(p + (size_t)min(s0 + j, nsplit - 1) * stride);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (s0 + j >= nsplit) continue;
      if (s0 + j == 0) {
        u = pv[j];
      } else {
        u.x += pv[j].x;
        u.y += pv[j].y;
        u.z += pv[j].z;
        u.w += pv[j].w;
      }
    }
  }
  return u;
}

// V = s U split into bf16 hi + lo (V ~= hi + lo to about 2^-16)
__device__ __forceinline__ void split_hi_lo(float v, uint16_t& h, uint16_t& lo) {
  const __bf16 hb = (__bf16)v;
  h = __builtin_bit_cast(uint16_t, hb);
  lo = __builtin_bit_cast(uint16_t, (__bf16)(v - (float)hb));
}

// One launch after the shrink, two kinds of blocks:
//  * the first fin_blocks: V = s * (the shrink's planes summed in split
//    order) as bf16 hi + lo, for every row of an adapter segment that the
//    GEMM expands itself (not in E);
//  * the rest: the small segments' s U B rows into E.  A block takes one
//    small segment and four 128-column groups (one per wave); it forms the
//    segment's V rows the same way, in LDS, while its B loads are in flight.
// V's bits are the same whichever block forms them.
template <int QC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void expand_small_kernel(GemmArgs a, int fin_blocks) {
  __shared__ __attribute__((aligned(16))) uint16_t vs[2][kSmallRows][kMaxRank];  // hi, lo
  const int N = a.N, T = a.T, w = a.u_ld;
  const int tid = threadIdx.x, l = tid & 63, wid = tid >> 6;
  if ((int)blockIdx.x < fin_blocks) {
    if (*a.status != 0) return;
    for (int idx = blockIdx.x * 256 + tid; idx < T * (w / 4); idx += fin_blocks * 256) {
      const int p = idx / (w / 4), q = 4 * (idx % (w / 4));
      // the planes, the row's segment and E row in one round, the segment's
      // entry in the next
      const float4 u = sum_planes4(a.upart + (size_t)p * w + q, a.split_stride, a.nsplit);
      const int sg = a.row_seg[p];
      const int er = a.erow[p];
      if (er >= 0 || a.seg_slot[sg] < 0 || q >= ((a.seg_rank[sg] + 15) & ~15)) continue;
      const float sc = pick4(a.seg_bscale[sg], q >> 4);  // the scale of q's 16-rank block
      uint16_t h[4], lo[4];
      split_hi_lo(sc * u.x, h[0], lo[0]);
      split_hi_lo(sc * u.y, h[1], lo[1]);
      split_hi_lo(sc * u.z, h[2], lo[2]);
      split_hi_lo(sc * u.w, h[3], lo[3]);
      *reinterpret_cast<uint2*>(a.v_hi + (size_t)p * w + q) =
          make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
      *reinterpret_cast<uint2*>(a.v_lo + (size_t)p * w + q) =
          make_uint2(lo[0] | ((uint32_t)lo[1] << 16), lo[2] | ((uint32_t)lo[3] << 16));
    }
    return;
  }
  const int ng = (N + 127) / 128, ngb = (ng + 3) / 4;
  const int eb = (int)gridDim.x - fin_blocks;
  // the status, the count and the first item's segment entry in one round
  // (the grid holds at most kMaxSmallRows * ngb items, so the entry is in
  // bounds; one past the count is never used)
  int item = (int)blockIdx.x - fin_blocks;
  const int st = *a.status;
  const int nitems = a.counts[3] * ngb;
  int4 si = a.small_info[min(item / ngb, kMaxSmallRows - 1)];
  float4 sb = a.small_bscale[min(item / ngb, kMaxSmallRows - 1)];
  if (st != 0) return;  // strict mode: a failed plan leaves out untouched
  for (; item < nitems; item += eb) {
    if (item != (int)blockIdx.x - fin_blocks) {
      si = a.small_info[item / ngb];
      sb = a.small_bscale[item / ngb];
    }
    const int g = min(4 * (item % ngb) + wid, ng - 1);  // a wave past the last group repeats it, no store
    const bool gok = 4 * (item % ngb) + wid < ng;
    const int off = si.x, len = si.y & 255, e0 = (si.y >> 8) & 0xfff, rank = si.y >> 20;
    const int end = off + len;
    const int nqc = (rank + 15) >> 4;
    const uint16_t* bt = a.pages + (size_t)si.z * a.slot_stride + a.b_off;
    // this wave's B rows one 16-rank chunk at a time (the first goes out
    // before V is formed): 16 registers for B instead of 16 QC, so that every
    // item of the launch fits on the chip at once
    bf16x8 bb[4];
    auto load_b = [&](int qc) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = min(g * 128 + 32 * i + (l & 31), N - 1);
        bb[i] = __builtin_bit_cast(bf16x8, ld16(bt + ((size_t)qc * N + n) * 16 + 8 * (l >> 5)));
      }
    };
    load_b(0);
    // the segment's V rows: thread = (row, 4 ranks)
    const int wq = nqc * 4;
    if (tid < len * wq) {
      const int r = tid / wq, q = 4 * (tid % wq);
      const float4 u = sum_planes4(a.upart + (size_t)(off + r) * w + q, a.split_stride, a.nsplit);
      const float sc = pick4(sb, q >> 4);  // the scale of q's 16-rank block
      split_hi_lo(sc * u.x, vs[0][r][q], vs[1][r][q]);
      split_hi_lo(sc * u.y, vs[0][r][q + 1], vs[1][r][q + 1]);
      split_hi_lo(sc * u.z, vs[0][r][q + 2], vs[1][r][q + 2]);
      split_hi_lo(sc * u.w, vs[0][r][q + 3], vs[1][r][q + 3]);
    }
    __syncthreads();
    for (int rb = off & ~31; rb < end; rb += 32) {
      const int p = rb + (l & 31);
      const bool in = p >= off && p < end;
      const uint32_t m = in ? 0xffffffffu : 0u;
      const int pr = in ? p - off : 0;
      f32x16 acc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
      // rank chunks in order, hi then lo (the GEMM walker's order)
      for (int qc = 0; qc < nqc; ++qc) {
        if (qc > 0 || rb != (off & ~31)) load_b(qc);  // chunk 0 of the first row block is loaded
        const uint4 hh = *reinterpret_cast<const uint4*>(&vs[0][pr][16 * qc + 8 * (l >> 5)]);
        const uint4 oo = *reinterpret_cast<const uint4*>(&vs[1][pr][16 * qc + 8 * (l >> 5)]);
        const bf16x8 mh = __builtin_bit_cast(bf16x8, make_uint4(hh.x & m, hh.y & m, hh.z & m, hh.w & m));
        const bf16x8 ml = __builtin_bit_cast(bf16x8, make_uint4(oo.x & m, oo.y & m, oo.z & m, oo.w & m));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[i] = mfma32(bb[i], mh, acc[i]);
          acc[i] = mfma32(bb[i], ml, acc[i]);
        }
      }
      if (in && gok) {
        float* er = a.E + (size_t)(e0 + p - off) * N;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = g * 128 + 32 * i + 8 * q + 4 * (l >> 5);
            if (col < N)
              *reinterpret_cast<float4*>(er + col) =
                  make_float4(acc[i][4 * q], acc[i][4 * q + 1], acc[i][4 * q + 2], acc[i][4 * q + 3]);
          }
      }
    }
    __syncthreads();  // the next item rewrites vs
  }
}

template <int QC>
static void launch_expand_small_cfg(const GemmArgs& a, hipStream_t s) {
  // V blocks: enough for about one 4-rank group per thread, at most 512;
  // small-segment blocks: at most kMaxSmallRows segments x ceil(N / 512)
  // items, at most 1024 blocks, each walking its share
  const int fin = std::min((a.T * (a.u_ld / 4) + 255) / 256, 512);
  const int items = kMaxSmallRows * (((a.N + 127) / 128 + 3) / 4);
  const int eb = std::min(items, 1024);
  hipLaunchKernelGGL(expand_small_kernel<QC>, dim3(fin + eb), dim3(256), 0, s, a, fin);
}

hipError_t launch_expand_small(const GemmArgs& a, hipStream_t s) {
  const int qc = a.u_ld / 16;
  if (qc <= 1)
    launch_expand_small_cfg<1>(a, s);
  else if (qc == 2)
    launch_expand_small_cfg<2>(a, s);
  else
    launch_expand_small_cfg<4>(a, s);
  return hipGetLastError();
}

template <int BM, int BN>
static hipError_t launch_cfg(const GemmArgs& a, bool lora, hipStream_t s) {
  const int tiles = ((a.row1 - a.row0 + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  if (!lora) {
    hipLaunchKernelGGL((prefill_kernel<BM, BN, false, 0>), dim3(tiles), dim3(256), 0, s, a);
  } else {
    const int qc = a.u_ld / 16;  // 16-rank chunks in the pool's pages
    if (qc <= 1)
      hipLaunchKernelGGL((prefill_kernel<BM, BN, true, 1>), dim3(tiles), dim3(256), 0, s, a);
    else if (qc == 2)
      hipLaunchKernelGGL((prefill_kernel<BM, BN, true, 2>), dim3(tiles), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((prefill_kernel<BM, BN, true, 4>), dim3(tiles), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

// Relative time of a round of tiles (per unit of K) for each shape, measured
// on MI355X; the launcher picks the shapes with the least estimated time,
// counting whole rounds.  The shapes up to 128x128 fill the LDS with their
// stages: one tile per compute unit, a round of 256.  A 64x64 tile (64 KB of
// LDS) runs two per compute unit: a round of 512 costs 0.26, one with at
// most one tile per unit 0.16 (measured on the Llama-3-8B layer: 256 tiles
// over the last 256 rows of a 4096-column linear in 20 us, 1088 tiles over
// all 4352 rows of a 1024-column one in 71 us).
struct Shape {
  int bm, bn;
  double cost;       // a full round
  double cost_half;  // a last round with at most one tile per compute unit
  int per_round;
};
constexpr int kNumShapes = 5;
static const Shape kShapes[kNumShapes] = {{256, 256, 1.00, 1.00, 256},
                                          {256, 128, 0.56, 0.56, 256},
                                          {128, 256, 0.56, 0.56, 256},
                                          {128, 128, 0.32, 0.32, 256},
                                          {64, 64, 0.26, 0.16, 512}};
static double shape_time(int i, int rows, int N) {
  const Shape& sh = kShapes[i];
  const long tiles = (long)((rows + sh.bm - 1) / sh.bm) * ((N + sh.bn - 1) / sh.bn);
  const long full = tiles / sh.per_round, rem = tiles % sh.per_round;
  return (double)full * sh.cost + (rem == 0 ? 0.0 : rem <= 256 ? sh.cost_half : sh.cost);
}

int prefill_choose(int T, int N) {
  int best = 0;
  double best_t = 1e30;
  for (int i = 0; i < kNumShapes; ++i) {
    const double t = shape_time(i, T, N);
    if (t < best_t * 0.999) {
      best_t = t;
      best = i;
    }
  }
  return best;
}

static hipError_t launch_shape(const GemmArgs& a, bool lora, int shape, hipStream_t s) {
  switch (shape) {
    case 0: return launch_cfg<256, 256>(a, lora, s);
    case 1: return launch_cfg<256, 128>(a, lora, s);
    case 2: return launch_cfg<128, 256>(a, lora, s);
    case 3: return launch_cfg<128, 128>(a, lora, s);
    default: return launch_cfg<64, 64>(a, lora, s);
  }
}

hipError_t launch_prefill(const GemmArgs& args, bool lora, int shape, hipStream_t s) {
  if (args.T <= 0) return hipSuccess;
  GemmArgs a = args;
  a.row0 = 0;
  a.row1 = a.T;
  if (shape >= 0) return launch_shape(a, lora, shape, s);
  // one shape for every row, or 256x256 tiles over the first rows (a whole
  // number of 256-row tiles) and small tiles (128x128 or 64x64) over the
  // rest: a second, short round of small tiles instead of a mostly empty
  // round of big ones
  const int one = prefill_choose(a.T, a.N);
  const double t_one = shape_time(one, a.T, a.N);
  // (among equal estimates the most rows in big tiles: the small tiles then
  // share the memory with fewer others)
  int tm = 0, tail = 3;
  double t_two = 1e30;
  for (int r = 256; r < a.T; r += 256) {
    for (int sh : {3, 4}) {
      const double t = shape_time(0, r, a.N) + shape_time(sh, a.T - r, a.N) + 0.03;
      if (t <= t_two * 1.001) {
        t_two = std::min(t, t_two);
        tm = r;
        tail = sh;
      }
    }
  }
  if (tm > 0) {
    if (t_two < t_one * 0.999) {
      a.row1 = tm;
      hipError_t e = launch_shape(a, lora, 0, s);
      if (e != hipSuccess) return e;
      a.row0 = tm;
      a.row1 = a.T;
      return launch_shape(a, lora, tail, s);
    }
  }
  return launch_shape(a, lora, one, s);
}

}  // namespace hrg
