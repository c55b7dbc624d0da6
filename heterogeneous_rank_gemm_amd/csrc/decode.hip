// Decode-shaped LoRA linear (T <= 64 tokens): two launches, no inter-block
// waiting.
//
// At decode the linear is bound by bytes: W once, plus the A and B pages of
// every distinct adapter in the batch.  X is small (T x K), but every column
// tile needs all of it, so it is staged once per K chunk in LDS and never
// re-read from L2 per 16 columns.
//
// Launch 1 (decode_main): a grid of (row tile, 512-wide K chunk) blocks of
// 8 waves.  Every block stages X[:, chunk] (64 x 512 bf16) in LDS; each wave
// owns a block of 16 rows, loads its whole 16 x 512 slice up front, and runs
// the bf16 MFMA 16x16x32 against the X chunk.  Two kinds of row tiles:
//   * W tiles: 8 x 16 rows of the base weight; the fp32 partial sums go to
//     part[chunk][t][n].
//   * A tiles: 8 items (adapter, 16 ranks), i.e. 16 rows of an adapter's A^T
//     page.  The block groups the batch by adapter id (LoRA-Land post,
//     section "2. multi-LoRA batch scheduling": Grouped Multi-LoRA
//     Execution), so each adapter's page is streamed once per chunk; the
//     partial shrink U_c[t, q] = X[t, chunk] . A[chunk, q] is kept for the
//     adapter's own tokens in upart[chunk][t][q].
// Launch 2 (decode_combine), one thread per (token, 4 columns):
//     V[t, q]   = (alpha/r) * sum_chunks upart[c][t][q]
//     out[t, n] = bf16( sum_chunks part[c][t][n]  +  sum_q V[t, q] B_i[q, n] )
//   chunks added in order, the expand in fp32, a single rounding (icman
//   report, section 2.1: the low-rank branch is added back to the main path).
//   Rows with id -1 get no LoRA term at all.
//
// The base-only entry runs the same launches without A tiles and without the
// expand, so id -1 rows match it bit for bit.  Every block that depends on the
// ids validates all of them the same way (strict mode, icman report section
// 4.1): on an invalid batch nothing is written to `out`.
#include "common.h"
#include "internal.h"

namespace hrg {

constexpr int kMainThreads = 512;
constexpr int kMainWaves = kMainThreads / 64;
constexpr int kSteps = kDecodeChunk / 32;  // MFMA K steps per chunk
constexpr int kXs = kDecodeChunk + 8;      // LDS row of the X chunk (16-byte pad)
static_assert(kMainWaves * 16 == kDecodeTileRows, "tile rows");

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
// v if keep, else zero -- with a mask, so the compiler never selects between
// addresses (which would push register arrays to scratch memory)
__device__ __forceinline__ uint4 keep_if(bool keep, uint4 v) {
  const uint32_t m = keep ? 0xffffffffu : 0u;
  return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
}
__device__ __forceinline__ float lo_f(uint32_t v) { return __builtin_bit_cast(float, v << 16); }
__device__ __forceinline__ float hi_f(uint32_t v) { return __builtin_bit_cast(float, v & 0xffff0000u); }

// Token t's adapter lookup (lane t of a wave, t < 64): id, pool slot, true
// rank and scale, or bad = the status code of an invalid id.  All lanes load
// in parallel, so a wave pays one round of dependent loads, not one per token.
struct TokInfo {
  int id = -1, slot = -1, rank = 0, bad = 0;
  float scale = 0.f;
};

__device__ __forceinline__ TokInfo token_info(const DecodeArgs& a, int t) {
  TokInfo ti;
  if (t < a.T) {
    const int id = a.ids[t];
    if (id < -1 || id >= a.max_ids) {
      ti.bad = kStatusIdRange;
    } else if (id >= 0) {
      const int4 e = a.id_info[id];  // {slot, rank, scale bits}: one load after ids
      if (e.x < 0) {
        ti.bad = kStatusNotLoaded;
      } else {
        ti.id = id;
        ti.slot = e.x;
        ti.rank = e.y;
        ti.scale = __builtin_bit_cast(float, e.z);
      }
    }
  }
  return ti;
}

__global__ __launch_bounds__(kMainThreads) __attribute__((amdgpu_waves_per_eu(4))) void decode_main(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[64 * kXs];
  __shared__ int s_bad;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g4 = lane >> 4, r16 = lane & 15;
  const int T = a.T, N = a.N, K = a.K;
  if (a.lora && *a.status != 0) return;

  // Block order: the A blocks first (a_blocks, a multiple of 8, so they start
  // early and spread over all XCDs round-robin), then the W blocks.  For the W
  // blocks the hardware hands block b to XCD (b mod 8); each XCD takes a
  // contiguous run of (tile, chunk) pairs so neighbouring tiles share its L2.
  int tile, c;
  bool a_tile;
  if ((int)blockIdx.x < a.a_blocks) {
    a_tile = true;
    tile = a.NT + (int)blockIdx.x / a.KS;
    c = (int)blockIdx.x % a.KS;
    if (tile >= a.NT + a.n_atiles) return;  // padding block
  } else {
    a_tile = false;
    const int g = (int)blockIdx.x - a.a_blocks;
    const int G = a.NT * a.KS;
    const int xcd = g % 8, qd = G / 8, rm = G % 8;
    const int logical = xcd * qd + min(xcd, rm) + g / 8;
    tile = logical / a.KS;
    c = logical % a.KS;
  }
  const int k0 = c * kDecodeChunk, klen = min(K, k0 + kDecodeChunk) - k0;

  // ---- this wave's 16 rows ----
  const uint16_t* row = nullptr;  // row r16 of the block of 16, at k0
  bool row_ok = false;
  int n0 = 0;                     // W tile: first column
  int qb = 0;                     // A tile: rank block of the adapter
  uint64_t members = 0;           // A tile: tokens of the adapter
  if (!a_tile) {
    n0 = tile * kDecodeTileRows + 16 * w;
    row_ok = n0 + r16 < N;
    row = a.W + (size_t)(row_ok ? n0 + r16 : 0) * K + k0;
  } else {
    // one round of lookups: lane t holds token t's id, slot and rank
    TokInfo ti = token_info(a, lane);
    if (w == 0 && lane == 0) s_bad = 0;
    __syncthreads();
    if (w == 0 && ti.bad) atomicMax(&s_bad, ti.bad);
    __syncthreads();
    if (s_bad) return;  // the combine launch rejects the batch
    // item = the (8 (tile - NT) + w)-th (adapter, 16-rank block) of the batch,
    // adapters in order of first occurrence
    const int item = 8 * (tile - a.NT) + w;
    uint64_t todo = __ballot(ti.id >= 0);
    int seen = 0;
    while (todo) {
      const int leader = __builtin_ctzll(todo);  // wave-uniform: readlane, not an LDS shuffle
      const int v = __builtin_amdgcn_readlane(ti.id, leader);
      const int r = __builtin_amdgcn_readlane(ti.rank, leader);
      const uint64_t m = __ballot(ti.id == v) & todo;
      todo &= ~m;
      const int nq = (r + 15) / 16;
      if (item < seen + nq) {
        const int slot = __builtin_amdgcn_readlane(ti.slot, leader);
        qb = item - seen;
        members = m;
        const int q = 16 * qb + r16;
        row_ok = q < r;
        row = a.pages + (size_t)slot * a.slot_stride + a.a_off + (size_t)(row_ok ? q : 0) * K + k0;
        break;
      }
      seen += nq;
    }
  }
  const bool active = row != nullptr;  // an A-tile wave past the last item has nothing to do
  if (!active) row = a.X + k0;         // dummy in-bounds source, results discarded

  // ---- loads: X chunk first (needed first), then the whole 16 x 512 slice ----
  // X goes through registers (8 x 16 bytes per thread) so that writing it to
  // LDS waits only for the X loads; the slice's MFMAs then start as soon as
  // their own step has landed (the vector-memory counter retires in order).
  constexpr int kXLoads = 64 * (kDecodeChunk / 8) / kMainThreads;  // 8 per thread
  uint4 xv[kXLoads];
#pragma unroll
  for (int i = 0; i < kXLoads; ++i) {
    const int idx = tid + i * kMainThreads;
    const int r = idx / (kDecodeChunk / 8), kc = (idx % (kDecodeChunk / 8)) * 8;
    xv[i] = ld16(a.X + (size_t)min(r, T - 1) * K + k0 + min(kc, klen - 8));
  }
  __builtin_amdgcn_sched_barrier(0);
  uint4 rw[kSteps];
#pragma unroll
  for (int s = 0; s < kSteps; ++s) rw[s] = ld16(row + min(32 * s + 8 * g4, klen - 8));
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < kXLoads; ++i) {
    const int idx = tid + i * kMainThreads;
    const int r = idx / (kDecodeChunk / 8), kc = (idx % (kDecodeChunk / 8)) * 8;
    *reinterpret_cast<uint4*>(xs + r * kXs + kc) = keep_if(r < T && kc < klen, xv[i]);
  }
  __syncthreads();
  if (!active) return;

  const int nm = (T + 15) / 16;
  f32x4 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    const int k = 32 * s + 8 * g4;
    const bf16x8 wb = __builtin_bit_cast(bf16x8, keep_if(k < klen && row_ok, rw[s]));
    // all four 16-token row blocks: rows >= T hold stale LDS and are never stored
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = mfma16(lds_bf16x8(xs + (16 * i + r16) * kXs + k), wb, acc[i]);
  }

  // ---- partial tile out: acc[i][e] is token 16 i + 4 g4 + e, row r16 of the block ----
  if (!a_tile) {
    if (row_ok) {
      float* pp = a.part + (size_t)c * 64 * N + n0 + r16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i >= nm) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * i + 4 * g4 + e;
          if (t < T) pp[(size_t)t * N] = acc[i][e];
        }
      }
    }
  } else if (row_ok) {
    float* up = a.upart + (size_t)c * 64 * a.u_ld + 16 * qb + r16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i >= nm) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * i + 4 * g4 + e;
        if ((members >> t) & 1ull) up[(size_t)t * a.u_ld] = acc[i][e];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// combine: block = 16 tokens x 64 columns, thread = (token, 4 columns)
constexpr int kCombThreads = 256;

__global__ __launch_bounds__(kCombThreads) void decode_combine(DecodeArgs a) {
  __shared__ float vsh[16][kMaxRank + 1];
  __shared__ int t_slot[16], t_rank[16];
  __shared__ float t_scale[16];
  __shared__ int flag;
  const int tid = threadIdx.x;
  const int T = a.T, N = a.N, KS = a.KS;
  const int t0 = blockIdx.y * 16;
  if (a.lora) {
    if (*a.status != 0) return;
    if (tid == 0) flag = 0;
    __syncthreads();
    if (tid < 64) {
      const TokInfo ti = token_info(a, tid);  // every token: strict-mode check
      if (ti.bad) atomicMax(&flag, ti.bad);
      if (tid >= t0 && tid < t0 + 16) {
        t_slot[tid - t0] = ti.slot;
        t_rank[tid - t0] = ti.rank;
        t_scale[tid - t0] = ti.scale;
      }
    }
    __syncthreads();
    if (flag) {
      if (tid == 0 && blockIdx.x == 0 && blockIdx.y == 0) atomicMax(a.status, flag);
      return;  // strict mode: out untouched
    }
  }
  const int tr = tid >> 4, quad = tid & 15;
  const int t = t0 + tr;
  const int n = blockIdx.x * 64 + quad * 4;
  const bool mine = t < T && n < N;
  // independent loads first: the chunk partials and the first 16 rows of B
  const float* pp = a.part + (size_t)min(t, T - 1) * N + min(n, N - 4);
  float4 pv[8];
  const int slot = a.lora ? t_slot[tr] : -1;
  const int rank = a.lora ? t_rank[tr] : 0;
  // B^T page in 16-rank chunks [rpad/16][N][16]: the 4 columns' first chunk is
  // 64 contiguous values (ranks past the adapter's rank are zero)
  const uint16_t* Bp = a.pages + (size_t)max(slot, 0) * a.slot_stride + a.b_off + (size_t)min(n, N - 4) * 16;
  uint4 bv[8];
  if (slot >= 0) {
#pragma unroll
    for (int k = 0; k < 8; ++k) bv[k] = *reinterpret_cast<const uint4*>(Bp + 8 * k);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) pv[j] = *reinterpret_cast<const float4*>(pp + (size_t)min(j, KS - 1) * 64 * N);
  if (a.lora) {
    // V[t][q] = (alpha / r) * sum of the shrink partials in chunk order
    for (int idx = tid; idx < 16 * kMaxRank; idx += kCombThreads) {
      const int r = idx / kMaxRank, q = idx % kMaxRank;
      float v = 0.f;
      if (t0 + r < T && q < t_rank[r]) {
        const float* up = a.upart + (size_t)(t0 + r) * a.u_ld + q;
        float u = up[0];
        for (int c0 = 1; c0 < KS; c0 += 8) {
          float uv[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) uv[j] = up[(size_t)min(c0 + j, KS - 1) * 64 * a.u_ld];
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (c0 + j < KS) u += uv[j];
        }
        v = t_scale[r] * u;
      }
      vsh[r][q] = v;
    }
    __syncthreads();
  }
  if (!mine) return;
  // base: chunk partials in chunk order
  float4 s = pv[0];
  for (int c0 = 0; c0 < KS; c0 += 8) {
    if (c0 > 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        pv[j] = *reinterpret_cast<const float4*>(pp + (size_t)min(c0 + j, KS - 1) * 64 * N);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (c0 + j > 0 && c0 + j < KS) {
        s.x += pv[j].x;
        s.y += pv[j].y;
        s.z += pv[j].z;
        s.w += pv[j].w;
      }
    }
  }
  if (slot >= 0) {
    float e[4] = {0.f, 0.f, 0.f, 0.f};
    for (int c = 0; 16 * c < rank; ++c) {
      if (c > 0) {
#pragma unroll
        for (int k = 0; k < 8; ++k) bv[k] = *reinterpret_cast<const uint4*>(Bp + (size_t)c * N * 16 + 8 * k);
      }
      const float* v = &vsh[tr][16 * c];
#pragma unroll
      for (int col = 0; col < 4; ++col) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint4 u = bv[2 * col + h];
          const float* vh = v + 8 * h;
          e[col] += vh[0] * lo_f(u.x);
          e[col] += vh[1] * hi_f(u.x);
          e[col] += vh[2] * lo_f(u.y);
          e[col] += vh[3] * hi_f(u.y);
          e[col] += vh[4] * lo_f(u.z);
          e[col] += vh[5] * hi_f(u.z);
          e[col] += vh[6] * lo_f(u.w);
          e[col] += vh[7] * hi_f(u.w);
        }
      }
    }
    s.x += e[0];
    s.y += e[1];
    s.z += e[2];
    s.w += e[3];
  }
  const uint32_t o0 = (uint32_t)f32_to_bf16_bits(s.x) | ((uint32_t)f32_to_bf16_bits(s.y) << 16);
  const uint32_t o1 = (uint32_t)f32_to_bf16_bits(s.z) | ((uint32_t)f32_to_bf16_bits(s.w) << 16);
  *reinterpret_cast<uint2*>(a.out + (size_t)t * N + n) = make_uint2(o0, o1);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(decode_main, dim3(a.a_blocks + a.NT * a.KS), dim3(kMainThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine, dim3((a.N + 63) / 64, (a.T + 15) / 16), dim3(kCombThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace hrg
