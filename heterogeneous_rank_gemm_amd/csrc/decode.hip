// Decode-shaped LoRA linear (T <= 64 tokens): two launches, no inter-block
// waiting.
//
// At decode the linear is bound by bytes: W once, plus the A and B pages of
// every distinct adapter in the batch.  X is small (T x K), but every column
// tile needs all of it, so it is staged once per K chunk in LDS and never
// re-read from L2 per 16 columns.
//
// Launch 1 (decode_main): a grid of (column tile, 1024-deep K chunk) blocks.
// Each block's first four waves copy X[:, chunk] (64 x 1024 bf16, 132 KB with
// row padding) into LDS by direct DMA and own 16 rows of W each; every wave
// loads its whole 16 x 1024 slice into registers up front (32 KB in flight per
// wave) and runs bf16 MFMA 16x16x32 against the X chunk as the slice lands.
// Two kinds of waves:
//   * W waves (the first four of a block): 16 rows of the base weight; the
//     fp32 partial sums go to part[chunk][t][n].
//   * A waves (the rest): one item (adapter, 16 ranks) each, i.e. 16 rows of
//     an adapter's A^T page.  The wave groups the batch by adapter id
//     (LoRA-Land post, section "2. multi-LoRA batch scheduling": Grouped
//     Multi-LoRA Execution), so each adapter's page is streamed once per
//     chunk; the partial shrink U_c[t, q] = X[t, chunk] . A[chunk, q] is kept
//     for the adapter's own tokens in upart[chunk][t][q].
// Riding in the W tiles' blocks, the A items add no second round of blocks.
// Items past what those waves hold go to extra blocks of A waves only.  The
// A waves' id loads go out before the weight stream fills the memory
// queues; a load issued behind that stream waits for most of it, so every
// further dependent round costs several microseconds.  A direct-mapped pool
// (adapter id in slot id) therefore needs no slot-table round at all.
// Launch 2 (decode_combine), one thread per (token, 4 columns):
//     V[t, q]   = (alpha/r) * sum_chunks upart[c][t][q]
//     out[t, n] = bf16( sum_chunks part[c][t][n]  +  sum_q V[t, q] B_i[q, n] )
//   chunks added in order, the expand in fp32, a single rounding (icman
//   report, section 2.1: the low-rank branch is added back to the main path).
//   Rows with id -1 get no LoRA term at all.
//
// The base-only entry runs the same launches without A waves and without the
// expand, so id -1 rows match it bit for bit.  Every combine block validates
// all the ids the same way (strict mode, icman report section 4.1): on an
// invalid batch nothing is written to `out`.
#include "common.h"
#include "internal.h"

namespace hrg {

constexpr int kSteps = kDecodeChunk / 32;  // MFMA K steps per chunk (32)
constexpr int kXs = kDecodeChunk + 8;      // LDS row of the X chunk (16-byte pad)
constexpr uint32_t kOobOff = 0x80000000u;  // buffer offset past every operand
static_assert(4 * 16 == kDecodeTileRows, "tile rows");

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
// v if keep, else zero -- with a mask, so the compiler never selects between
// addresses (which would push register arrays to scratch memory)
__device__ __forceinline__ uint4 keep_if(bool keep, uint4 v) {
  const uint32_t m = keep ? 0xffffffffu : 0u;
  return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
}
__device__ __forceinline__ float lo_f(uint32_t v) { return __builtin_bit_cast(float, v << 16); }
__device__ __forceinline__ float hi_f(uint32_t v) { return __builtin_bit_cast(float, v & 0xffff0000u); }

// Whether an adapter with module mask `mask` targets linear `m` (modules >= 32
// are always targeted).
__device__ __forceinline__ bool targets(int mask, int m) { return m >= 32 || ((mask >> m) & 1); }

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
      const int4 e = a.id_info[id];  // {slot, rank, scale bits, module mask}: one load after ids
      if (e.x < 0) {
        ti.bad = kStatusNotLoaded;
      } else {
        ti.id = id;
        ti.slot = e.x;
        // an adapter that does not target this linear has no rank here
        ti.rank = targets(e.w, a.module) ? (e.y & (kChainRankFlag - 1)) : 0;
        ti.scale = __builtin_bit_cast(float, e.z);
      }
    }
  }
  return ti;
}

// Waits until at most N of this wave's vector-memory operations are
// outstanding and every LDS access has completed, then joins the workgroup
// barrier.  (__syncthreads() would wait for all of them.)
template <int N>
__device__ __forceinline__ void barrier_after(void) {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"i"(N) : "memory");
}

// NA: A waves riding in each W block (0 on the base-only path).
//
// W blocks (the first np = nbc * KS): block b keeps K chunk c = b mod KS and
// walks the column tiles bi, bi + nbc, ... (bi = b div KS), so its X chunk is
// staged once however many tiles it takes.  Each W wave streams its 16 rows
// of those tiles as a sequence of 512-deep halves through two register
// buffers: the next half's loads are in flight while the current half's
// MFMAs run (with 16 KB per wave and half in flight, the chip keeps about
// 32 MB of reads outstanding, ample for the memory's latency).  The loads
// and partial stores follow a fixed pattern (rows past N and tokens past T
// land in the padding of `part`), so the loads' completion is counted
// exactly.
// WQ: the base weight is INT4 (a.Wq, a.Wsz); each W wave loads a quarter of
// the bytes and dequantizes its fragments in registers before the MFMAs.
template <int NA, bool WQ>
__global__ __launch_bounds__(64 * (4 + NA)) void decode_main(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[64 * kXs];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g4 = lane >> 4, r16 = lane & 15;
  const int T = a.T, N = a.N, K = a.K, KS = a.KS;
  const int nbc = a.np / KS;  // W blocks per K chunk

  int c, bi;
  const bool w_block = (int)blockIdx.x < a.np;
  if (w_block) {
    c = (int)blockIdx.x % KS;
    bi = (int)blockIdx.x / KS;
  } else {  // blocks of A waves only
    const int g = (int)blockIdx.x - a.np;
    c = g % KS;
    bi = g / KS;
  }
  const int k0 = c * kDecodeChunk, klen = min(K, k0 + kDecodeChunk) - k0;
  const bool a_wave = !w_block || w >= 4;

  // ---- an A wave's 16 rows ----
  const uint16_t* row = nullptr;  // row r16 of the block of 16, at k0
  bool row_ok = false;
  int qb = 0;                     // rank block of the adapter
  uint64_t members = 0;           // tokens of the adapter
  if (a_wave) {
    // In a W block the A waves copy no X: they join the block barrier before
    // their lookups, so the W waves never wait there for them (the X copy
    // takes longer than the barrier wait it replaces; the A slices stay off
    // the critical path).
    // item = the item-th (adapter, 16-rank block) of the batch, adapters in
    // order of first occurrence.  Lane t holds token t's id.  A direct-mapped
    // pool keeps adapter id in slot id, so the page address follows from the
    // ids alone (every rank block up to the pool's padded rank is an item;
    // rows past an adapter's rank are zero); otherwise one more round of
    // loads fetches each token's slot and rank.  Both load rounds go out
    // before the weight stream fills the memory queues.
    const int item = w_block ? bi + nbc * (w - 4) : nbc * NA + (4 + NA) * bi + w;
    int id = -1, slot = -1, rank = 0, bad = 0;
    if (a.direct) {
      if (lane < T) id = a.ids[lane];
      // the id load stays in flight across the barrier
      if (w_block) __builtin_amdgcn_s_barrier();
      if (id >= a.max_slots || id < -1) bad = 1;  // the combine launch rejects the batch
      slot = id;
      rank = a.u_ld;
    } else {
      if (w_block) __builtin_amdgcn_s_barrier();
      const TokInfo ti = token_info(a, lane);
      id = ti.id;
      slot = ti.slot;
      rank = ti.rank;
      bad = ti.bad;
    }
    if (__ballot(bad != 0) == 0) {
      // m = the lanes holding this lane's adapter: one ballot per bit of the
      // id, each lane keeping the lanes that agree with it on that bit
      const bool v = id >= 0;
      const int nbits = 32 - __builtin_clz((unsigned)max(max(a.max_ids, a.max_slots), 1));
      uint64_t m = __ballot(v);
      for (int k = 0; k < nbits; ++k) {
        const bool bit = (id >> k) & 1;
        const uint64_t on = __ballot(v && bit);
        m &= bit ? on : ~on;
      }
      // an adapter's first lane owns ceil(rank / 16) consecutive items, the
      // adapters in order of first occurrence (= lane order of first lanes)
      const bool first = v && lane == (int)__builtin_ctzll(m);
      const int nq = first ? (rank + 15) / 16 : 0;
      const int incl = wave_incl_scan(nq);
      const uint64_t hit = __ballot(first && item >= incl - nq && item < incl);
      if (hit) {
        const int leader = (int)__builtin_ctzll(hit);  // wave-uniform: readlane, not an LDS shuffle
        const int r = __builtin_amdgcn_readlane(rank, leader);
        const int sl = __builtin_amdgcn_readlane(slot, leader);
        qb = item - __builtin_amdgcn_readlane(incl - nq, leader);
        members = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(m >> 32), leader) << 32) |
                  (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)m, leader);
        const int q = 16 * qb + r16;
        row_ok = q < min(r, a.rmax);
        row = a.pages + (size_t)sl * a.slot_stride + a.a_off + (size_t)(row_ok ? q : 0) * K + k0;
      }
    }
    // drain the lookups here, so that no wait for them is left to the merge
    // with the W path (where it would also wait for the X DMA below)
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  }

  // ---- X chunk -> LDS by DMA: waves 0..3 copy tokens 16w .. 16w+15, two
  // 1-KB pieces per token row.  Rows >= T and columns >= K read zeros.
  if (w < 4) {
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc((void*)a.X, (short)0, T * K * 2, 0x00020000);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int r = 16 * w + (i >> 1), h = i & 1;
      const int k = k0 + 512 * h + 8 * lane;
      // rows >= T lie past the buffer's range (zeros); columns >= K are
      // sent past it
      const uint32_t off = k < K ? (uint32_t)(r * K + k) * 2u : kOobOff;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void_t*)(xs + r * kXs + 512 * h), 16, off, 0, 0, 0);
    }
  }

  f32x4 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // acc[i] += X[16 i .. 16 i + 15, k .. k + 31] . W slice, for each step s
  // of a register block of kHalf / 32 steps starting at kh
  constexpr int kHalf = kDecodeChunk / 2, kHS = kHalf / 32;

  if constexpr (WQ) {
    if (!a_wave) {
      const int ntile = (a.NT - bi + nbc - 1) / nbc;  // >= 1: the host keeps nbc <= NT
      const int nhalf = 2 * ntile;
      constexpr int kHG = kHalf / kQ4Group;  // groups per half (4)
      const int KW = K / 8, KG = K / kQ4Group;
      uint4 rq[2][kHG];     // per group: the lane's 4 words, one per 32-deep step
      uint32_t rz[2][kHG];  // per group: {bf16 scale, zero point}
      // reads past the end of Wq / Wsz return zeros; groups past the chunk
      // are masked below
      const __amdgpu_buffer_rsrc_t rqs =
          __builtin_amdgcn_make_buffer_rsrc((void*)a.Wq, (short)0, N * KW * 4, 0x00020000);
      const __amdgpu_buffer_rsrc_t rzs =
          __builtin_amdgcn_make_buffer_rsrc((void*)a.Wsz, (short)0, N * KG * 4, 0x00020000);
      auto load = [&](uint4 (&bq)[kHG], uint32_t (&bz)[kHG], int s) __attribute__((always_inline)) {
        const int sc = min(s, nhalf - 1);
        const int n = (bi + (sc >> 1) * nbc) * kDecodeTileRows + 16 * w + r16;
        const int nn = n < N ? n : 0;
        const int g0 = (k0 + kHalf * (sc & 1)) / kQ4Group;
        const int offq = (nn * KW + 16 * g0 + 4 * g4) * 4;
        const int offz = (nn * KG + g0) * 4;
#pragma unroll
        for (int gi = 0; gi < kHG; ++gi)
          bq[gi] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rqs, offq + 64 * gi, 0, 0));
        // the half's four group words as one load (kHG + 1 loads per half in all)
        const uint4 zz = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rzs, offz, 0, 0));
        bz[0] = zz.x;
        bz[1] = zz.y;
        bz[2] = zz.z;
        bz[3] = zz.w;
      };
      static_assert(kHG == 4, "one 16-byte load of group words per half");
      load(rq[0], rz[0], 0);
      // the X DMA (issued before these kHG + 1 loads) has landed in every wave
      barrier_after<kHG + 1>();
      auto phase = [&](auto hc, auto nc, int s) __attribute__((always_inline)) {
        constexpr int H = decltype(hc)::value;
        constexpr bool NEXT = decltype(nc)::value;
        if constexpr (NEXT) load(rq[1 - H], rz[1 - H], s + 1);
#pragma unroll
        for (int gi = 0; gi < kHG; ++gi) {
          // a group past the chunk (klen is a multiple of the group) gets
          // scale 0 and offset 0: its weights dequantize to exact zeros
          const bool in = kHalf * H + kQ4Group * gi < klen;
          float2 g = q4_group(rz[H][gi]);
          g.x = in ? g.x : 0.f;
          g.y = in ? g.y : 0.f;
          const uint32_t words[4] = {rq[H][gi].x, rq[H][gi].y, rq[H][gi].z, rq[H][gi].w};
#pragma unroll
          for (int st = 0; st < 4; ++st) {
            const int k = kHalf * H + kQ4Group * gi + 32 * st + 8 * g4;
            const bf16x8 wb = dequant_q4x8(words[st], g.x, g.y);
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
              acc[tb] = mfma16(wb, lds_bf16x8(xs + (16 * tb + r16) * kXs + k), acc[tb]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (H == 1) {
          const int n = (bi + (s >> 1) * nbc) * kDecodeTileRows + 16 * w + 4 * g4;
          float* pp = a.part + (size_t)c * 64 * a.npad + (size_t)r16 * a.npad + n;
#pragma unroll
          for (int tb = 0; tb < 4; ++tb) {
            *reinterpret_cast<float4*>(pp + (size_t)(16 * tb) * a.npad) =
                make_float4(acc[tb][0], acc[tb][1], acc[tb][2], acc[tb][3]);
            acc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
        }
      };
      for (int s = 0; s < nhalf - 2; s += 2) {
        phase(std::integral_constant<int, 0>{}, std::true_type{}, s);
        phase(std::integral_constant<int, 1>{}, std::true_type{}, s + 1);
      }
      phase(std::integral_constant<int, 0>{}, std::true_type{}, nhalf - 2);
      phase(std::integral_constant<int, 1>{}, std::false_type{}, nhalf - 1);
      return;
    }
  }
  if (!WQ && !a_wave) {
    const int ntile = (a.NT - bi + nbc - 1) / nbc;  // >= 1: the host keeps nbc <= NT
    const int nhalf = 2 * ntile;
    uint4 rw[2][kHS];
    // one buffer resource over W: a half is one offset plus immediates, and
    // reads past the end of W return zeros (reads past the chunk within W are
    // masked below)
    const __amdgpu_buffer_rsrc_t rws =
        __builtin_amdgcn_make_buffer_rsrc((void*)a.W, (short)0, N * K * 2, 0x00020000);
    auto load = [&](uint4 (&buf)[kHS], int s) __attribute__((always_inline)) {
      const int sc = min(s, nhalf - 1);
      // row r16 of this wave's 16 rows of tile sc / 2 (rows past N read row
      // 0; their results land in the padding of `part`)
      const int n = (bi + (sc >> 1) * nbc) * kDecodeTileRows + 16 * w + r16;
      const int off = ((n < N ? n : 0) * K + k0 + kHalf * (sc & 1) + 8 * g4) * 2;
#pragma unroll
      for (int i = 0; i < kHS; ++i)
        buf[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rws, off + 64 * i, 0, 0));
    };
    load(rw[0], 0);
    // the X DMA (issued before these loads) has landed in every wave
    barrier_after<kHS>();
    // phase H of a tile: half H in rw[H]; the next half (if NEXT) goes to
    // rw[1 - H]
    auto phase = [&](auto hc, auto nc, int s) __attribute__((always_inline)) {
      constexpr int H = decltype(hc)::value;
      constexpr bool NEXT = decltype(nc)::value;
      if constexpr (NEXT) load(rw[1 - H], s + 1);
#pragma unroll
      for (int i = 0; i < kHS; ++i) {
        const int k = kHalf * H + 32 * i + 8 * g4;
        const bf16x8 wb = __builtin_bit_cast(bf16x8, keep_if(k < klen, rw[H][i]));
        // W as the A operand: a lane's results are 4 consecutive columns of
        // one token, stored as one 16-byte write
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
          acc[tb] = mfma16(wb, lds_bf16x8(xs + (16 * tb + r16) * kXs + k), acc[tb]);
        // at most four steps' X fragments in registers at a time
        if (i % 4 == 3) __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (H == 1) {
        // the tile's partial sums: acc[tb][e] is token 16 tb + r16, column
        // n + e of this wave's 16
        const int n = (bi + (s >> 1) * nbc) * kDecodeTileRows + 16 * w + 4 * g4;
        float* pp = a.part + (size_t)c * 64 * a.npad + (size_t)r16 * a.npad + n;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          *reinterpret_cast<float4*>(pp + (size_t)(16 * tb) * a.npad) =
              make_float4(acc[tb][0], acc[tb][1], acc[tb][2], acc[tb][3]);
          acc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
    };
    // every tile but the last requests the next tile's first half during its
    // second half; the last one requests nothing (a wave does not end with
    // loads in flight)
    for (int s = 0; s < nhalf - 2; s += 2) {
      phase(std::integral_constant<int, 0>{}, std::true_type{}, s);
      phase(std::integral_constant<int, 1>{}, std::true_type{}, s + 1);
    }
    phase(std::integral_constant<int, 0>{}, std::true_type{}, nhalf - 2);
    phase(std::integral_constant<int, 1>{}, std::false_type{}, nhalf - 1);
    return;
  }

  // ---- an A wave: its whole 16 x 1024 slice, issued at once ----
  const bool active = row != nullptr;  // an A wave past the last item has nothing to do
  if (!active) row = a.X + k0;         // dummy in-bounds source, results discarded
  uint4 rwa[kSteps];
#pragma unroll
  for (int s = 0; s < kSteps; ++s) rwa[s] = ld16(row + min(32 * s + 8 * g4, klen - 8));
  // blocks of A waves only: waves 0..3 copied X, everyone waits for it here
  if (!w_block) barrier_after<kSteps>();
  if (!active) return;
  // An adapter with at most 16 tokens in the batch (the usual case at decode)
  // needs one 16-token MFMA block, not four: lane r16 reads the X row of the
  // adapter's r16-th token, a quarter of the MFMAs and LDS reads.
  const int cnt = __popcll(members);
  if (cnt <= 16) {
    uint64_t m = members;  // X row of this lane: the r16-th member (row 0 past the last)
    for (int i = 0; i < r16; ++i) m &= m - 1;
    const int xr = m ? (int)__builtin_ctzll(m) : 0;
    f32x4 acc1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const int k = 32 * s + 8 * g4;
      const bf16x8 wb = __builtin_bit_cast(bf16x8, keep_if(k < klen && row_ok, rwa[s]));
      acc1 = mfma16(lds_bf16x8(xs + xr * kXs + k), wb, acc1);
    }
    if (row_ok) {
      // acc1[e] belongs to member 4 g4 + e
      uint64_t mm = members;
      for (int i = 0; i < 4 * g4; ++i) mm &= mm - 1;
      float* up = a.upart + (size_t)c * 64 * a.u_ld + 16 * qb + r16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (mm) up[(size_t)__builtin_ctzll(mm) * a.u_ld] = acc1[e];
        mm &= mm - 1;
      }
    }
    return;
  }
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    const int k = 32 * s + 8 * g4;
    const bf16x8 wb = __builtin_bit_cast(bf16x8, keep_if(k < klen && row_ok, rwa[s]));
    // all four 16-token row blocks: rows >= T hold zeros and are never stored
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = mfma16(lds_bf16x8(xs + (16 * i + r16) * kXs + k), wb, acc[i]);
  }
  if (row_ok) {
    const int nm = (T + 15) / 16;
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
// combine: block = 16 tokens x 64 columns, thread = (token, 4 columns).
// Round 1 of loads depends on nothing: the ids, the chunk partials and the
// shrink partials of the block's V, and in a direct-mapped pool the thread's
// B rows (its token's id comes by a scalar load).  Round 2: every token's
// {slot, rank, scale} (each block checks the whole batch, strict mode).
// Otherwise the B rows need the slot and come in a third round.
constexpr int kCombThreads = 256;
constexpr int kVPer = 16 * kMaxRank / kCombThreads;  // V elements per thread

// sum over the KS chunk planes p[c * stride], c = 0, 1, ... in order; loads
// issued four at a time
__device__ __forceinline__ float sum_chunks(const float* p, size_t stride, int KS) {
  float s = 0.f;
  for (int c0 = 0; c0 < KS; c0 += 4) {
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = p[(size_t)min(c0 + j, KS - 1) * stride];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (c0 + j < KS) s += v[j];
  }
  return s;
}

__global__ __launch_bounds__(kCombThreads) void decode_combine(DecodeArgs a) {
  __shared__ float vsh[16][kMaxRank + 1];
  __shared__ int4 s_info[16];  // the block's tokens: {slot (-1: none), rank, scale bits, 0}
  __shared__ float4 s_bsc[16];  // the block's tokens: scale of each 16-rank block
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  const int T = a.T, N = a.N, KS = a.KS;
  const int t0 = blockIdx.y * 16;
  const int tr = tid >> 4, quad = tid & 15;
  const int t = t0 + tr;
  const int n = blockIdx.x * 64 + quad * 4;
  const bool mine = t < T && n < N;

  // ---- round 1 ----
  // (the ids for the whole-batch check are stored to LDS only after every
  // other load of this round is out, so that no load waits for them)
  int st = 0, idv = -1;
  if (a.lora) {
    st = *a.status;
    if (tid < 64 && tid < T) idv = a.ids[tid];
  }
  const float* pp = a.part + (size_t)min(t, T - 1) * a.npad + min(n, N - 4);
  float4 pv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) pv[j] = *reinterpret_cast<const float4*>(pp + (size_t)min(j, KS - 1) * 64 * a.npad);
  float u[kVPer];
  uint4 bv[8];
  int slot = -1, rank = 0;
  const uint16_t* Bp = nullptr;
  if (a.lora) {
    // this wave's four tokens' ids by wave-uniform (scalar) loads, so that a
    // direct-mapped pool's B rows go out in this round, beside the partials,
    // instead of after a round trip of vector loads
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tw = t0 + 4 * wv;  // tr = 4 wv + (tr & 3)
    const int i0 = tw < T ? a.ids[tw] : -1;
    const int i1 = tw + 1 < T ? a.ids[tw + 1] : -1;
    const int i2 = tw + 2 < T ? a.ids[tw + 2] : -1;
    const int i3 = tw + 3 < T ? a.ids[tw + 3] : -1;
    const int q4 = tr & 3;
    const int my_id = q4 == 0 ? i0 : q4 == 1 ? i1 : q4 == 2 ? i2 : i3;
    // B^T page in 16-rank chunks [rpad/16][N][16]: the 4 columns' chunk is 64
    // contiguous values (ranks past the adapter's rank are zero)
    if (a.direct && mine && my_id >= 0 && my_id < a.max_slots) {
      Bp = a.pages + (size_t)my_id * a.slot_stride + a.b_off + (size_t)n * 16;
#pragma unroll
      for (int k = 0; k < 8; ++k) bv[k] = *reinterpret_cast<const uint4*>(Bp + 8 * k);
    }
    // V[t][q] = (alpha / r) * sum of the shrink partials in chunk order; the
    // loads of all kVPer entries go out together, four chunks at a time
    const float* up[kVPer];
    bool uq[kVPer];
#pragma unroll
    for (int e = 0; e < kVPer; ++e) {
      const int idx = tid + kCombThreads * e;
      const int r = idx / kMaxRank, q = idx % kMaxRank;
      uq[e] = q < a.u_ld;
      up[e] = a.upart + (size_t)min(t0 + r, T - 1) * a.u_ld + (uq[e] ? q : 0);
      u[e] = 0.f;
    }
    const size_t ustr = (size_t)64 * a.u_ld;
    // the first four chunks' V partial loads go out now, the rest after the
    // routing lookups
    float v[kVPer][4];
#pragma unroll
    for (int e = 0; e < kVPer; ++e)
#pragma unroll
      for (int j = 0; j < 4; ++j) v[e][j] = up[e][(size_t)min(j, KS - 1) * ustr];

    // ---- round 2: the whole batch's routing entries (strict mode), lane t
    // from its own id register (wave 0 only), while round 1 is in flight ----
    if (tid < 64) {
      if (tid == 0) s_bad = 0;  // before the wave's atomics, in program order
      const int id = idv;
      int bad = 0;
      int4 e = make_int4(-1, 0, 0, 0);
      if (id < -1 || id >= a.max_ids) {
        bad = kStatusIdRange;
      } else if (id >= 0) {
        e = a.id_info[id];  // {slot, rank, scale bits}
        if (tid >= t0 && tid < t0 + 16) {
          // a chain's blocks have their own scales (one more load, chains only)
          const float sc = __builtin_bit_cast(float, e.z);
          s_bsc[tid - t0] = (e.y & kChainRankFlag) ? a.id_bscale[id] : make_float4(sc, sc, sc, sc);
        }
        e.y &= kChainRankFlag - 1;
        if (e.x < 0) bad = kStatusNotLoaded;
      }
      if (bad) atomicMax(&s_bad, bad);
      // a token whose adapter does not target this linear takes the base only
      if (!bad && e.x >= 0 && !targets(e.w, a.module)) e = make_int4(-1, 0, 0, 0);
      if (tid >= t0 && tid < t0 + 16) s_info[tid - t0] = bad ? make_int4(-1, 0, 0, 0) : e;
    }
    for (int c0 = 0; c0 < KS; c0 += 4) {
      if (c0 > 0) {
#pragma unroll
        for (int e = 0; e < kVPer; ++e)
#pragma unroll
          for (int j = 0; j < 4; ++j) v[e][j] = up[e][(size_t)min(c0 + j, KS - 1) * ustr];
      }
#pragma unroll
      for (int e = 0; e < kVPer; ++e)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (c0 + j < KS && uq[e]) u[e] += v[e][j];
    }
    __syncthreads();  // s_bad, s_info
    if (s_bad) {
      if (tid == 0 && blockIdx.x == 0 && blockIdx.y == 0) atomicMax(a.status, s_bad);
      return;  // strict mode: out untouched
    }
    if (st != 0) return;  // a pending error (st is the same in every thread)
#pragma unroll
    for (int e = 0; e < kVPer; ++e) {
      const int idx = tid + kCombThreads * e;
      const int r = idx / kMaxRank, q = idx % kMaxRank;
      const int4 inf = s_info[r];
      const bool on = t0 + r < T && inf.x >= 0 && q < inf.y;
      vsh[r][q] = on ? pick4(s_bsc[r], q >> 4) * u[e] : 0.f;
    }
    __syncthreads();  // vsh
    slot = s_info[tr].x;
    rank = s_info[tr].y;
  }
  if (!mine) return;
  if (slot >= 0 && !a.direct) {
    // ---- round 3 (pool not direct-mapped) ----
    Bp = a.pages + (size_t)slot * a.slot_stride + a.b_off + (size_t)n * 16;
#pragma unroll
    for (int k = 0; k < 8; ++k) bv[k] = *reinterpret_cast<const uint4*>(Bp + 8 * k);
  }

  // base: chunk partials in chunk order
  float4 s = pv[0];
  for (int c0 = 0; c0 < KS; c0 += 4) {
    if (c0 > 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        pv[j] = *reinterpret_cast<const float4*>(pp + (size_t)min(c0 + j, KS - 1) * 64 * a.npad);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
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
          const uint4 w = bv[2 * col + h];
          const float* vh = v + 8 * h;
          e[col] += vh[0] * lo_f(w.x);
          e[col] += vh[1] * hi_f(w.x);
          e[col] += vh[2] * lo_f(w.y);
          e[col] += vh[3] * hi_f(w.y);
          e[col] += vh[4] * lo_f(w.z);
          e[col] += vh[5] * hi_f(w.z);
          e[col] += vh[6] * lo_f(w.w);
          e[col] += vh[7] * hi_f(w.w);
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

hipError_t launch_decode(const DecodeArgs& args, int items, hipStream_t s) {
  DecodeArgs a = args;
  // W blocks: every (tile, chunk) pair if the chip holds them at once, else
  // as many whole sets of KS chunk blocks as it holds (one block per compute
  // unit: the X chunk fills most of the LDS), each walking several tiles
  const int resident = resident_blocks(reinterpret_cast<const void*>(&decode_main<0, false>), 256, 0);
  a.np = std::min(a.NT * a.KS, std::max(1, resident / a.KS) * a.KS);
  const int nbc = a.np / a.KS;
  a.na = 0;
  a.a_tiles = 0;
  if (a.lora) {
    // items ride in the W blocks (na waves each, 1, 2 or 4); the rest get
    // extra blocks of A waves only
    const int per_block = (items + nbc - 1) / nbc;
    a.na = per_block <= 1 ? 1 : per_block <= 2 ? 2 : 4;
    a.a_tiles = (std::max(0, items - nbc * a.na) + 3 + a.na) / (4 + a.na);
  }
  const dim3 grid(a.np + a.a_tiles * a.KS);
  if (a.Wq) {
    switch (a.na) {
      case 0: hipLaunchKernelGGL((decode_main<0, true>), grid, dim3(256), 0, s, a); break;
      case 1: hipLaunchKernelGGL((decode_main<1, true>), grid, dim3(320), 0, s, a); break;
      case 2: hipLaunchKernelGGL((decode_main<2, true>), grid, dim3(384), 0, s, a); break;
      case 4: hipLaunchKernelGGL((decode_main<4, true>), grid, dim3(512), 0, s, a); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (a.na) {
      case 0: hipLaunchKernelGGL((decode_main<0, false>), grid, dim3(256), 0, s, a); break;
      case 1: hipLaunchKernelGGL((decode_main<1, false>), grid, dim3(320), 0, s, a); break;
      case 2: hipLaunchKernelGGL((decode_main<2, false>), grid, dim3(384), 0, s, a); break;
      case 4: hipLaunchKernelGGL((decode_main<4, false>), grid, dim3(512), 0, s, a); break;
      default: return hipErrorInvalidValue;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine, dim3((a.N + 63) / 64, (a.T + 15) / 16), dim3(kCombThreads), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// INT4 -> bf16 weight for the batched path: one thread per packed word (eight
// weights, one 16-byte store).
__global__ void q4_dequant_kernel(const uint32_t* __restrict__ Wq, const uint32_t* __restrict__ Wsz, int N,
                                  int K, uint16_t* __restrict__ W) {
  const int KW = K / 8, KG = K / kQ4Group;
  const size_t total = (size_t)N * KW;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (size_t)gridDim.x * blockDim.x) {
    const int n = (int)(i / KW), p = (int)(i % KW);
    const int g = p / 16, j = (p % 16) / 4, st = p % 4;
    const float2 gz = q4_group(Wsz[(size_t)n * KG + g]);
    const bf16x8 v = dequant_q4x8(Wq[i], gz.x, gz.y);
    *reinterpret_cast<uint4*>(W + (size_t)n * K + kQ4Group * g + 32 * st + 8 * j) = __builtin_bit_cast(uint4, v);
  }
}

hipError_t launch_q4_dequant(const uint32_t* Wq, const uint32_t* Wsz, int N, int K, uint16_t* W,
                             hipStream_t s) {
  const size_t total = (size_t)N * (K / 8);
  const int grid = (int)std::min<size_t>((total + 255) / 256, 8192);
  hipLaunchKernelGGL(q4_dequant_kernel, dim3(grid), dim3(256), 0, s, Wq, Wsz, N, K, W);
  return hipGetLastError();
}

}  // namespace hrg
