// Base GEMM  Y0 = X W^T  on bf16 MFMA, with the LoRA "expand" fused into the
// epilogue:  out[t, :] = bf16( Y0[t, :] + s_i (U[t, :] B_i) ),  i = ids[t].
//
// The shared base path is the first term of the LoRA-Land formula (section
// "2. multi-LoRA batch scheduling"); the per-token side path is added back
// onto it before the single rounding (icman report, section 2.1: in dynamic
// batching every sample's low-rank branch is added back to the main path).
//
// Layout: X [T][K], W [N][K] (both K-contiguous, an "NT" GEMM), out [T][N].
// The LoRA instantiation walks the rows in the plan's sorted order (rows are
// gathered through perm on load and scattered back on store), so the rows of
// one adapter are contiguous inside an M-tile.  The base instantiation uses
// the identity order.  A row's fp32 base sum does not depend on where it sits
// inside a tile, so id -1 rows match the base-only kernel bit for bit.
//
// Expand: per adapter segment that meets the tile, V = s * sum_splits(U) is
// split into bf16 hi + lo parts (V ~= hi + lo to ~2^-16 relative) and
// multiplied with the adapter's B tile on the MFMA, accumulating into the
// same fp32 registers as the base sum.
#include "common.h"
#include "internal.h"

namespace hrg {

// XCD-aware tile order: the hardware hands workgroup b to XCD (b mod 8).
// Give each XCD a contiguous range of logical tiles, and walk the logical
// tiles in groups of GROUP_M tile-rows so neighbours share X rows / W rows
// in that XCD's L2.
__device__ __forceinline__ void tile_coords(int b, int nblocks, int tiles_m, int tiles_n,
                                            int& tm, int& tn) {
  constexpr int kXcd = 8;
  const int xcd = b % kXcd, idx = b / kXcd;
  const int q = nblocks / kXcd, r = nblocks % kXcd;
  const int logical = xcd * q + min(xcd, r) + idx;
  constexpr int kGroupM = 8;
  const int per_group = kGroupM * tiles_n;
  const int g = logical / per_group;
  const int first_m = g * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int in = logical % per_group;
  tm = first_m + in % gsize;
  tn = in / gsize;
}

template <int BM, int BN, int BK, int WM, int WN, bool LORA>
__global__ __launch_bounds__(WM* WN * 64) void gemm_kernel(GemmArgs a) {
  constexpr int NT = WM * WN * 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int KC = BK / 8;  // 16-byte chunks per tile row
  static_assert(KC == 8, "swizzle assumes 8 chunks per row");
  constexpr int LA = BM * KC / NT, LB = BN * KC / NT;
  static_assert(LA * NT == BM * KC && LB * NT == BN * KC, "tile / thread mismatch");
  constexpr int kStage = (BM + BN) * BK;  // elements per LDS stage
  constexpr int kRPad = kMaxRank + 8;     // padded V / B^T row in the epilogue
  constexpr int kEpi = 2 * BM * kRPad + BN * kRPad;
  constexpr int kLds = (2 * kStage > kEpi) ? 2 * kStage : kEpi;
  __shared__ __attribute__((aligned(16))) uint16_t lds[kLds];

  if constexpr (LORA) {
    if (*a.status != 0) return;
  }
  const int T = a.T, N = a.N, K = a.K;
  const int tiles_m = (T + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x, l = tid & 63, wid = tid >> 6;
  const int wm = wid / WN, wn = wid % WN;

  // global -> register staging slots (fixed row / chunk per slot)
  const uint16_t* arow[LA];
  bool aval[LA];
  int akc[LA], alds[LA];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int c = tid + i * NT;
    const int row = c / KC, kc = c % KC;
    const int p = m0 + row;
    aval[i] = p < T;
    const int tok = aval[i] ? (a.perm ? a.perm[p] : p) : 0;
    arow[i] = a.X + (size_t)tok * K + kc * 8;
    akc[i] = kc * 8;
    alds[i] = row * BK + ((kc ^ (row & 7)) * 8);
  }
  const uint16_t* brow[LB];
  bool bval[LB];
  int bkc[LB], blds[LB];
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int c = tid + i * NT;
    const int row = c / KC, kc = c % KC;
    const int n = n0 + row;
    bval[i] = n < N;
    brow[i] = a.W + (size_t)(bval[i] ? n : 0) * K + kc * 8;
    bkc[i] = kc * 8;
    blds[i] = BM * BK + row * BK + ((kc ^ (row & 7)) * 8);
  }

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  uint4 ra[LA], rb[LB];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < LA; ++i)
      ra[i] = (aval[i] && k0 + akc[i] < K) ? *reinterpret_cast<const uint4*>(arow[i] + k0)
                                           : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int i = 0; i < LB; ++i)
      rb[i] = (bval[i] && k0 + bkc[i] < K) ? *reinterpret_cast<const uint4*>(brow[i] + k0)
                                           : make_uint4(0u, 0u, 0u, 0u);
  };
  auto lstore = [&](int stage) {
    uint16_t* base = lds + stage * kStage;
#pragma unroll
    for (int i = 0; i < LA; ++i) *reinterpret_cast<uint4*>(base + alds[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < LB; ++i) *reinterpret_cast<uint4*>(base + blds[i]) = rb[i];
  };

  const int nk = (K + BK - 1) / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
    const uint16_t* As = lds + cur * kStage;
    const uint16_t* Bs = As + BM * BK;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int c = 2 * kk + (l >> 5);
      bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int row = wm * WTM + 32 * i + (l & 31);
        af[i] = lds_bf16x8(As + row * BK + ((c ^ (row & 7)) * 8));
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int row = wn * WTN + 32 * j + (l & 31);
        bfr[j] = lds_bf16x8(Bs + row * BK + ((c ^ (row & 7)) * 8));
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < nk) {
      lstore(cur ^ 1);
    }
    __syncthreads();
  }

  if constexpr (LORA) {
    // ---------------- fused expand ----------------
    const int pend = min(m0 + BM, T);
    uint16_t* Vhi = lds;
    uint16_t* Vlo = lds + BM * kRPad;
    uint16_t* Bt = lds + 2 * BM * kRPad;
    const int u_w = a.u_ld;  // staged rank width (pool r_max rounded to 16)
    // stage V = s * sum_split U for every row of the tile (zero outside adapters)
    for (int idx = tid; idx < BM * u_w; idx += NT) {
      const int row = idx / u_w, q = idx % u_w;
      const int p = m0 + row;
      float v = 0.f;
      if (p < T) {
        const int sg = a.row_seg[p];
        const int rk = a.seg_rank[sg];
        if (a.seg_id[sg] >= 0 && q < ((rk + 15) & ~15)) {
          const float* up = a.upart + (size_t)p * a.u_ld + q;
          float u = 0.f;
          for (int sp = 0; sp < a.nsplit; ++sp) u += up[(size_t)sp * a.split_stride];
          v = a.seg_scale[sg] * u;
        }
      }
      const __bf16 h = (__bf16)v;
      const __bf16 lo = (__bf16)(v - (float)h);
      Vhi[row * kRPad + q] = __builtin_bit_cast(uint16_t, h);
      Vlo[row * kRPad + q] = __builtin_bit_cast(uint16_t, lo);
    }
    const int s_first = a.row_seg[m0];
    const int s_last = a.row_seg[pend - 1];
    for (int sg = s_first; sg <= s_last; ++sg) {
      if (a.seg_id[sg] < 0) continue;
      const int rk = a.seg_rank[sg];
      const int rp = (rk + 15) & ~15;
      const int ra = max(a.seg_off[sg], m0) - m0;
      const int rb = min(a.seg_off[sg + 1], pend) - m0;
      const uint16_t* Bp = a.pages + (size_t)a.seg_slot[sg] * a.slot_stride + a.b_off;
      __syncthreads();  // previous segment's MFMAs are done with Bt (and V is staged)
      // B^T tile: Bt[n][q] = B[q][n0 + n] for q < rank, else 0
      for (int idx = tid; idx < rp * (BN / 8); idx += NT) {
        const int q = idx / (BN / 8), nc = (idx % (BN / 8)) * 8;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (q < rk && n0 + nc < N) v = *reinterpret_cast<const uint4*>(Bp + (size_t)q * N + n0 + nc);
        const uint16_t* e = reinterpret_cast<const uint16_t*>(&v);
#pragma unroll
        for (int t = 0; t < 8; ++t) Bt[(nc + t) * kRPad + q] = e[t];
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int rblk = wm * WTM + 32 * i;
        if (rblk + 32 <= ra || rblk >= rb) continue;  // wave-uniform
        const int row = rblk + (l & 31);
        const bool in = row >= ra && row < rb;
        for (int kq = 0; kq < rp / 16; ++kq) {
          const int q = 16 * kq + 8 * (l >> 5);
          const bf16x8 vh = in ? lds_bf16x8(Vhi + row * kRPad + q) : zero_bf16x8();
          const bf16x8 vl = in ? lds_bf16x8(Vlo + row * kRPad + q) : zero_bf16x8();
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const int n = wn * WTN + 32 * j + (l & 31);
            const bf16x8 bb = lds_bf16x8(Bt + n * kRPad + q);
            acc[i][j] = mfma32(vh, bb, acc[i][j]);
            acc[i][j] = mfma32(vl, bb, acc[i][j]);
          }
        }
      }
    }
  }

  // ---------------- store (single rounding) ----------------
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wm * WTM + 32 * i + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
      const int p = m0 + row;
      if (p >= T) continue;
      const int tok = a.perm ? a.perm[p] : p;
      uint16_t* orow = a.out + (size_t)tok * N;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int n = n0 + wn * WTN + 32 * j + (l & 31);
        if (n < N) orow[n] = f32_to_bf16_bits(acc[i][j][r]);
      }
    }
  }
}

// Tile choice depends only on (T, N, K), so lora_apply and lora_base_apply
// run the same K traversal for the same shape.
template <int BM, int BN, int BK, int WM, int WN>
static hipError_t launch_cfg(const GemmArgs& a, bool lora, hipStream_t s) {
  const int tiles = ((a.T + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  if (lora)
    hipLaunchKernelGGL((gemm_kernel<BM, BN, BK, WM, WN, true>), dim3(tiles), dim3(WM * WN * 64), 0, s, a);
  else
    hipLaunchKernelGGL((gemm_kernel<BM, BN, BK, WM, WN, false>), dim3(tiles), dim3(WM * WN * 64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& a, bool lora, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  if (a.T <= 64) return launch_cfg<64, 64, 64, 2, 2>(a, lora, s);
  return launch_cfg<128, 128, 64, 2, 2>(a, lora, s);
}

}  // namespace hrg
