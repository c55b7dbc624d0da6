// Grouped "shrink": U[p, q] = sum_k X[perm[p], k] * A_s[k, q] for every
// sorted row p of adapter segment s and q < rank(s).  Evaluating X A first
// gives the low-rank intermediate of the LoRA-Land post (section "2.
// multi-LoRA batch scheduling"), which keeps the extra work small.
//
// Work unit: (shrink tile, K-split).  A tile is up to 64 sorted rows of ONE
// segment, so the adapter's A^T page (fragment tiles: one contiguous 1 KB
// per 16 ranks x 32-deep MFMA step) is streamed once per tile and K-split,
// 256 deep at a time through two register sets; the 16x16x32 bf16 MFMA does
// the contraction.  Linears that read the same X (q/k/v, gate/up) are shrunk
// by one launch: an item multiplies the X rows it loads once by the pages of
// all of them (NL linears of NQ rank blocks, NL * NQ <= 4).
// Each of the 4 waves covers an interleaved quarter of the K range; the four
// partial results are summed in a fixed order through LDS (deterministic),
// and each K-split writes its own fp32 partial plane of U.  The small-segment
// launch that follows sums the planes in split order (deterministic), scales
// by s = alpha/r and forms V = s U as bf16 hi + lo parts (V ~= hi + lo to
// about 2^-16) for the expand.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace hrg {

constexpr int kShrinkThreads = 256;
constexpr int kRedLd = 65;  // padded row of the cross-wave reduction buffer

__device__ __forceinline__ bf16x8 keep_bf(bool keep, uint4 v) {
  const uint32_t m = keep ? 0xffffffffu : 0u;
  return __builtin_bit_cast(bf16x8, make_uint4(v.x & m, v.y & m, v.z & m, v.w & m));
}

// Calls f(integral_constant<int, S>) for S = 0 .. N-1, in order.
template <int N, int S = 0, class F>
__device__ __forceinline__ void for_each_set(F&& f) {
  if constexpr (S < N) {
    f(std::integral_constant<int, S>{});
    for_each_set<N, S + 1>(f);
  }
}

// Register sets of the sub-chunk ring: two (the next sub-chunk in flight
// during the current one's MFMAs).  Three or four sets, where the registers
// allow them, measured no faster.
constexpr int kShrinkSets = 2;

constexpr uint32_t kShrinkOob = 0x80000000u;  // buffer offset past every operand (< 2 GiB)

// The tokens of a tile's rows this lane gathers: row 16 mb + (lane & 15).
__device__ __forceinline__ void tile_tokens(const ShrinkArgs& a, int4 ti, int (&tok)[4]) {
  const int l = threadIdx.x & 63;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int p = 16 * mb + (l & 15);
    tok[mb] = a.perm[ti.x + (p < ti.y ? p : 0)];
  }
}

// NQ: 16-rank blocks held per item (the pool's rank rounded up to 16, in
// blocks; an adapter of lower rank masks the rest).
// `tok` holds this item's gathered tokens (requested during the previous
// item), so the A and X loads go out together.  The next item's tile entry
// (index `next`) is requested into *tn with them and its tokens into tokn
// once it lands, so neither lookup costs a round of its own.
template <int NQ, int NL, int NS>
__device__ __forceinline__ void shrink_item(const ShrinkArgs& a, float (*red)[64 * kRedLd], int4 ti, int split,
                                            int next, const int (&tok)[4], int4* tn, int (&tokn)[4]) {
  constexpr int NB = NQ * NL;  // rank blocks of the item: linear j / NQ, block j % NQ
  const int row0 = ti.x, rows = ti.y, slot = ti.z, rank = ti.w;
  const int nq = (rank + 15) / 16;  // 16-wide rank blocks actually computed
  const int nm = (rows + 15) / 16;  // 16-row blocks with at least one row
  const int K = a.K;
  const int k0 = split * a.kchunk;
  const int k1 = min(K, k0 + a.kchunk);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const uint16_t* Ap = a.pages + (size_t)slot * a.slot_stride;

  // the A tiles follow from the tile entry alone: rank block nb's tile of
  // step s is 1 KB at frag_tile(nb, s), this lane's 16 bytes at 16 l
  const int k32 = (K + 31) / 32;
  const int rp = a.u_ld;  // rows of the page in fragment tiles (the pool's rank rounded up to 16)
  // the A pages and X through buffer resources: a sub-chunk past the item's
  // range is requested with an offset past the operand (zeros, no memory
  // traffic), so every load is still issued and the waits stay exact
  __amdgpu_buffer_rsrc_t ra[NL];
  const int a_bytes = (int)(frag_elems(a.u_ld, K) * 2);
#pragma unroll
  for (int m = 0; m < NL; ++m)
    ra[m] = __builtin_amdgcn_make_buffer_rsrc((void*)(Ap + a.a_off[m]), (short)0, a_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)a.X, (short)0, a.T * K * 2, 0x00020000);
  bool qv[NQ];
#pragma unroll
  for (int nb = 0; nb < NQ; ++nb) qv[nb] = 16 * nb + (l & 15) < rank;
  const int koff = 8 * (l >> 4);
  // 256-deep sub-chunks: wave w takes the 32-deep steps 32 w + 128 s
  // (s = 0, 1) of each, through a ring of NS register sets: the next
  // sub-chunks' A and X loads are in flight while the current one's MFMAs
  // run.  Every load is issued whatever the item's rank and rows (a rank
  // block past the adapter's rank re-reads block 0 and a row past the tile
  // re-reads row 0: L2 hits, never applied; a sub-chunk past the item's
  // range goes out of range: zeros, no memory traffic), so the compiler
  // counts each wait exactly instead of waiting for every set before the
  // first MFMA.  (Out-of-range requests in place of re-reading the last
  // sub-chunk: Llama-3-8B layer step 1844 -> 1837 us.)
  constexpr int kSub = 256;
  const int nsub = (k1 - k0 + kSub - 1) / kSub;
  const int klast = k0 + (nsub - 1) * kSub;
  uint32_t xrow[4];
  bool rv[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int p = 16 * mb + (l & 15);
    rv[mb] = p < rows;
    xrow[mb] = (uint32_t)tok[mb] * (uint32_t)K * 2u;
  }
  uint4 av[NS][2][NB], xv[NS][2][4];
  auto load = [&](auto bc, int kb) __attribute__((always_inline)) {
    constexpr int b = decltype(bc)::value;
    const uint32_t past = kb > klast ? kShrinkOob : 0u;  // wave-uniform
    kb = min(kb, klast);
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int step = min((kb + 128 * st + 32 * w) / 32, k32 - 1);
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int nb = j % NQ;
        const uint32_t off = (uint32_t)((frag_tile(nb < nq ? nb : 0, step, rp, K) * 512 + (size_t)l * 8) * 2);
        const uint32_t skip = nb < nq ? past : kShrinkOob;  // a block past the adapter's rank: nothing read
        av[b][st][j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ra[j / NQ], off | skip, 0, 0));
      }
    }
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int kc = min(kb + 128 * st + 32 * w + koff, K - 8);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        xv[b][st][mb] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, (xrow[mb] + (uint32_t)kc * 2u) | past, 0, 0));
    }
  };

  f32x4 acc[4][NB];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[mb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto mm = [&](auto bc, int kb) __attribute__((always_inline)) {
    constexpr int b = decltype(bc)::value;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const bool kv = kb + 128 * st + 32 * w + koff < k1;  // a lane's 8 elements are all in or out
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        if (mb >= nm) continue;
        const bf16x8 xa = keep_bf(rv[mb] && kv, xv[b][st][mb]);
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int nb = j % NQ;
          if (nb >= nq) continue;
          acc[mb][j] = mfma16(xa, keep_bf(qv[nb] && kv, av[b][st][j]), acc[mb][j]);
        }
      }
    }
  };
  for_each_set<NS - 1>([&](auto bc) __attribute__((always_inline)) {
    load(bc, k0 + decltype(bc)::value * kSub);
  });
  // the next item's tile entry, then its tokens (they land during the MFMAs)
  *tn = a.tile_info[next];
  tile_tokens(a, *tn, tokn);
  bool more = true;
  for (int i = 0; more; i += NS) {
    for_each_set<NS>([&](auto pc) __attribute__((always_inline)) {
      constexpr int P = decltype(pc)::value;
      if (!more) return;
      load(std::integral_constant<int, (P + NS - 1) % NS>{}, k0 + (i + P + NS - 1) * kSub);
      mm(pc, k0 + (i + P) * kSub);
      more = i + P + 1 < nsub;
    });
  }

  // cross-wave reduction in fixed wave order (column 16 j + q of the
  // buffer: rank 16 (j % NQ) + q of linear j / NQ)
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    if (mb >= nm) continue;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (j % NQ >= nq) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * mb + 4 * (l >> 4) + i;
        const int q = 16 * j + (l & 15);
        red[w][r * kRedLd + q] = acc[mb][j][i];
      }
    }
  }
  __syncthreads();
  const int width = nq * 16;
#pragma unroll
  for (int m = 0; m < NL; ++m) {
    float* up = a.upart + (size_t)(m * a.nsplit + split) * a.split_stride + (size_t)row0 * a.u_ld;
    for (int idx = threadIdx.x; idx < rows * width; idx += kShrinkThreads) {
      const int r = idx / width, q = idx % width;
      const int c = 16 * NQ * m + q;
      const float v = ((red[0][r * kRedLd + c] + red[1][r * kRedLd + c]) + red[2][r * kRedLd + c]) +
                      red[3][r * kRedLd + c];
      up[(size_t)r * a.u_ld + q] = v;
    }
  }

}

// A fixed grid walks the (tile, split) items of the plan's tile list; the
// split count is fixed by K on the host, the tile count only on the device.
template <int NQ, int NL>
__global__ __launch_bounds__(kShrinkThreads) void shrink_kernel(ShrinkArgs a) {
  __shared__ float red[4][64 * kRedLd];
  // the first item's tile entry is requested with the status and the count
  // (the grid never exceeds max_tiles * nsplit items, so the read is in
  // bounds; an entry past the count is never used), each next one while the
  // current item runs
  const int st = *a.status;
  const int nitems = a.counts[1] * a.nsplit;
  int4 ti = a.tile_info[blockIdx.x / a.nsplit];
  if (st != 0 || (int)blockIdx.x >= nitems) return;
  int tok[4];
  tile_tokens(a, ti, tok);
  for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
    int4 tn;
    int tokn[4];
    __syncthreads();  // the previous item is done with red
    const int next = min(item + (int)gridDim.x, nitems - 1) / a.nsplit;
    shrink_item<NQ, NL, kShrinkSets>(a, red, ti, item % a.nsplit, next, tok, &tn, tokn);
    ti = tn;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) tok[mb] = tokn[mb];
  }
}

hipError_t launch_shrink(const ShrinkArgs& a, int nl, int grid, int ksplit, int T, hipStream_t s) {
  if (grid <= 0 || ksplit <= 0 || T <= 0) return hipSuccess;
  const int nq = a.u_ld / 16;
  if (nl < 1 || nl > shrink_linears(a.u_ld)) return hipErrorInvalidValue;
  if (nq <= 1) {
    switch (nl) {
      case 1: hipLaunchKernelGGL((shrink_kernel<1, 1>), dim3(grid), dim3(kShrinkThreads), 0, s, a); break;
      case 2: hipLaunchKernelGGL((shrink_kernel<1, 2>), dim3(grid), dim3(kShrinkThreads), 0, s, a); break;
      case 3: hipLaunchKernelGGL((shrink_kernel<1, 3>), dim3(grid), dim3(kShrinkThreads), 0, s, a); break;
      default: hipLaunchKernelGGL((shrink_kernel<1, 4>), dim3(grid), dim3(kShrinkThreads), 0, s, a); break;
    }
  } else if (nq == 2) {
    if (nl == 1)
      hipLaunchKernelGGL((shrink_kernel<2, 1>), dim3(grid), dim3(kShrinkThreads), 0, s, a);
    else
      hipLaunchKernelGGL((shrink_kernel<2, 2>), dim3(grid), dim3(kShrinkThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((shrink_kernel<4, 1>), dim3(grid), dim3(kShrinkThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace hrg
