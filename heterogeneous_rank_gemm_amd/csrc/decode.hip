// Decode-shaped LoRA linear (T <= 64 tokens): two launches, no inter-block
// waiting, for a group of up to kMaxGroup linears that read the same X (the
// q/k/v and gate/up projections of a transformer layer read one hidden
// state; a single linear is a group of one).
//
// At decode the linear is bound by bytes: W once, plus the A and B pages of
// every distinct adapter in the batch.  X is small (T x K), but every column
// of W needs all of it, so it is staged once per K chunk in LDS and never
// re-read from L2 per 16 columns.  A group shares that staging: one launch
// streams every linear's W rows against the one X chunk, where separate
// launches would each stage X again and each pay a ramp and a tail.
//
// Launch 1 (decode_main): blocks of WPB waves, each block keeping one
// 1024-deep K chunk of X (64 x 1024 bf16, 133 KB with row padding) in LDS,
// copied by direct DMA.  The chunk's work is a list of 16-row units:
//   * W units: 16 rows of one linear's base weight; the fp32 partial sums go
//     to part[chunk][t][column];
//   * A units: one (adapter, 16-rank block) item on one linear, i.e. 16 rows
//     of the adapter's A^T page.  The batch is grouped by adapter id
//     (LoRA-Land post, section "2. multi-LoRA batch scheduling": Grouped
//     Multi-LoRA Execution), so each adapter's page is streamed once per
//     chunk; the partial shrink U_c[t, q] = X[t, chunk] . A[chunk, q] is kept
//     for the adapter's own tokens in upart[chunk][linear][t][q].
// The W units come first and the A units last; wave i of a chunk takes units
// i, i + NWc, i + 2 NWc, ... (NWc waves per chunk), so every wave streams
// about the same number of bytes and no adapter work is left to a second
// round of blocks.  A bf16 unit streams through a ring of four 256-deep
// quarters (three in flight while one is multiplied); an INT4 unit through
// two 512-deep halves.
// Where the grid still fills the chip, a block takes two consecutive chunks:
// it walks its units over the first, restages X, walks them again over the
// second and adds each unit's two sums in registers, so one fp32 plane is
// written per chunk pair instead of per chunk.  The sums are added in one
// order either way: each chunk from zero in K order, the chunks of a pair,
// then the pairs in order; the combine launch adds pairs of single-chunk
// planes itself.  So the choice never changes a bit of the output.
// Launch 2 (decode_combine), one thread per (token, 4 columns):
//     V[t, q]   = (alpha/r) * sum_planes upart[c][linear][t][q]
//     out[t, n] = bf16( sum_planes part[c][t][n]  +  sum_q V[t, q] B_i[q, n] )
//   planes added in the order above, the expand in fp32, a single rounding (icman
//   report, section 2.1: the low-rank branch is added back to the main path).
//   Rows with id -1 get no LoRA term at all.
//
// The base-only entry runs the same launches without A units and without the
// expand, so id -1 rows match it bit for bit.  Every combine block validates
// all the ids the same way (strict mode, icman report section 4.1): on an
// invalid batch nothing is written to `out`.
#include <mutex>
#include <utility>

#include "common.h"
#include "internal.h"

namespace hrg {

constexpr int kHalf = kDecodeChunk / 2;    // K of one register block (a "half")
constexpr int kHS = kHalf / 32;            // MFMA K steps per half (16)
constexpr int kQS = 8;                     // MFMA K steps per quarter of a chunk
// LDS row of the X chunk: 32 bytes of pad, so rows start two 16-byte bank
// quads apart.  The LDS serves a 128-bit read in four cycles of 16 lanes,
// {0-7, 24-31}, {8-15, 16-23}, {32-39, 56-63}, {40-47, 48-55}; an MFMA step
// reads piece g4 of row r16 in lane 16 g4 + r16, so lane quads sit at
// 2 r16 + g4 (mod 16): distinct within every cycle (with one quad of pad,
// r16 + g4, one pair per cycle collided: 4 extra cycles per read).
constexpr int kXs = kDecodeChunk + 16;
constexpr int kXPieces = 2 * 64;           // 1-KB DMA pieces of an X chunk
constexpr uint32_t kOobOff = 0x80000000u;  // buffer offset past every operand
constexpr int kBufFlags = 0x00020000;      // buffer resource word 3 (raw, dword data)

typedef __attribute__((address_space(3))) void lds_void_t;

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

// The kernel's argument block in the kernarg segment (constant memory).  The
// per-linear tables are read through it with a wave-uniform index: one scalar
// load each, where indexing the by-value argument with a variable would copy
// the whole table to scratch memory.
typedef const __attribute__((address_space(4))) DecodeArgs* KArgs;
__device__ __forceinline__ KArgs kargs() {
  return (KArgs)__builtin_amdgcn_kernarg_segment_ptr();
}

// A buffer resource over [p, p + bytes) whose words the compiler knows to be
// wave-uniform (p and bytes must be): without the readfirstlanes it may keep
// an address computed by vector instructions in VGPRs and then wrap every
// load in a loop over the distinct values.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* p, int bytes) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0,
                                           __builtin_amdgcn_readfirstlane(bytes), kBufFlags);
}

// The linear of the group whose range [p[m], p[m+1]) holds x (p[0] = 0; the
// host fills p[i] = p[n] for i > n).
__device__ __forceinline__ int group_of(const int32_t (&p)[kMaxGroup + 1], int x) {
  // (constant indices: no scratch copy)
  int m = 0;
#pragma unroll
  for (int i = 1; i < kMaxGroup; ++i) m += x >= p[i] ? 1 : 0;
  return m;
}

// One 16-row unit of a wave's walk: where its rows come from (needed until
// its second half is requested) and where its results go (needed until its
// store).  Every field is wave-uniform but the offsets.
struct UnitSrc {
  __amdgpu_buffer_rsrc_t rs;  // rows of the unit's source: a W, Wq or A page
  __amdgpu_buffer_rsrc_t rz;  // INT4 W units: the linear's group words (Wsz)
  uint32_t off;               // this lane's byte offset at the chunk start (kOobOff: no row)
  uint32_t offz;              // INT4 W units: the lane's group-word offset
  int istep;                  // bytes from one 32-deep step to the next: 64 in a
                              // row-major W, 1024 in fragment tiles (wave-uniform;
                              // the loads take it as their scalar offset)
};
struct UnitDst {
  int kind;                   // 0: W rows, 1: A rows
  int m;                      // linear of the group
  int col;                    // W: first column in `part`; A: first rank (16 x rank block)
  uint64_t members;           // A: the adapter's tokens
};

// f(0), f(1), ..., f(n - 1) with compile-time indices, inlined: a loop body
// too large for the unroller's limit still indexes register arrays only with
// constants (a variable index would move them to scratch memory).
template <typename F, int... J>
__device__ __forceinline__ void static_for(F&& f, std::integer_sequence<int, J...>) {
  (f(std::integral_constant<int, J>{}), ...);
}

// a for pass 0, b for pass 1 (chosen at compile time)
template <int P>
__device__ __forceinline__ f32x4 (&pick(f32x4 (&a)[4], f32x4 (&b)[4]))[4] {
  if constexpr (P == 0)
    return a;
  else
    return b;
}

// Waits until at most N of this wave's vector-memory operations are
// outstanding and every LDS access has completed, then joins the workgroup
// barrier (__syncthreads() would wait for all of them).  Exact only where
// the N youngest operations are known: here they are N explicit 16-byte
// buffer loads (nothing the compiler can merge or split) that the scheduling
// fences keep after the X copy and before the wait.
template <int N>
__device__ __forceinline__ void barrier_after(void) {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"i"(N) : "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// The walk: WPB waves per block, all alike.
// WQ: the base weights are INT4 (a.Wq, a.Wsz); a W unit loads a quarter of
// the bytes and dequantizes its fragments in registers before the MFMAs.
// CPB: K chunks per block.  With two, a block keeps X of one chunk at a time
// in LDS, walks its units over the first chunk, restages X and walks them
// over the second, its waves holding every unit's sums in registers (at most
// kMaxUnits per wave; the host sizes the grid for that): one partial plane
// per pair of chunks, half the fp32 partials written and read back (they are
// a fifth of the step's traffic otherwise).
//
// Either way the sums are added in one order: each chunk's products from
// zero in K order (an MFMA chain), the two chunks of a pair added, then the
// pairs in order.  With one chunk per block the combine launch adds the
// pairs' planes; with two the block does, so both give the same bits and
// the host may pick either per launch.
constexpr int kMaxUnits = 8;

template <int WPB, bool WQ, int CPB>
__global__ __launch_bounds__(64 * WPB) void decode_main(DecodeArgs a) {
  static_assert(CPB == 1 || (CPB == 2 && WPB == 4 && !WQ), "two chunks per block: bf16, one wave per SIMD");
  __shared__ __attribute__((aligned(16))) uint16_t xs[64 * kXs];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g4 = lane >> 4, r16 = lane & 15;
  const int T = a.T, K = a.K, KS = a.KS, n_mod = a.n_mod;
  const int KP = a.KP;  // partial planes: the chunk groups (KS / CPB rounded up)
  const int plane = (int)blockIdx.x % KP, bi = (int)blockIdx.x / KP;
  const int npass = min(CPB, KS - plane * CPB);  // chunks of this block
  int c = plane * CPB;  // the chunk in LDS
  int k0 = c * kDecodeChunk, klen = min(K, k0 + kDecodeChunk) - k0;
  const int wi = bi * WPB + w;  // this wave among the chunk's NWc waves
  const int NWc = a.NWc;
  const int NUW = a.u0[kMaxGroup];  // W units of the group (16 rows each)
  const KArgs ka = kargs();
  // the wave's units are wi, wi + NWc, ...: first its W units, then its A units
  const int nw = wi < NUW ? (NUW - wi + NWc - 1) / NWc : 0;

  // ---- round 0: the token ids (lane t), before anything else ----
  int id = -1;
  if (a.lora && lane < T) id = a.ids[lane];

  // ---- X chunk -> LDS by DMA: the block's waves share the 128 pieces (two
  // 1-KB pieces per token row).  Rows >= T and columns >= K read zeros. ----
  auto stage_x = [&]() __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rx = uniform_rsrc(a.X, T * K * 2);
    // (the first piece opaque when the copy runs twice: its addresses are
    // formed in the loop, not kept from the first copy to the second)
    int i0 = w;
    if constexpr (CPB == 2) asm volatile("" : "+s"(i0));
    for (int i = i0; i < kXPieces; i += WPB) {
      const int r = i >> 1, h = i & 1;
      const int k = k0 + 512 * h + 8 * lane;
      // rows >= T lie past the buffer's range (zeros); columns >= K are sent past it
      const uint32_t off = k < K ? (uint32_t)(r * K + k) * 2u : kOobOff;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void_t*)(xs + r * kXs + 512 * h), 16, off, 0, 0, 0);
    }
  };
  stage_x();

  // a W unit's rows: row r16 of the 16, at chunk start kk
  auto w_unit = [&](int u, int kk, UnitSrc& sr, UnitDst& ds) __attribute__((always_inline)) {
    const int m = group_of(a.u0, u);
    const int N = ka->N[m];
    const int row0 = (u - ka->u0[m]) * 16;
    const int row = row0 + r16;
    ds.kind = 0;
    ds.m = m;
    ds.col = ka->n0[m] + row0;
    ds.members = 0;
    if constexpr (WQ) {
      const int KW = K / 8, KG = K / kQ4Group;
      sr.rs = uniform_rsrc(ka->Wq[m], N * KW * 4);
      sr.rz = uniform_rsrc(ka->Wsz[m], N * KG * 4);
      sr.off = row < N ? (uint32_t)(row * KW + 16 * (kk / kQ4Group) + 4 * g4) * 4u : kOobOff;
      sr.offz = row < N ? (uint32_t)(row * KG + kk / kQ4Group) * 4u : kOobOff;
      sr.istep = 0;
    } else if (a.wpacked) {
      // fragment tiles: the unit's 16 rows are row group u - u0[m]; its
      // tiles of the chunk are one contiguous 32 KB (1 KB per 32-deep
      // step, this lane's 16 bytes at 16 lane)
      sr.rs = uniform_rsrc(ka->W[m], (int)frag_elems(N, K) * 2);
      sr.rz = sr.rs;
      sr.off = (uint32_t)((frag_tile(u - ka->u0[m], kk / 32, N, K) * 64 + lane) * 16);
      sr.offz = 0;
      sr.istep = 1024;
    } else {
      sr.rs = uniform_rsrc(ka->W[m], N * K * 2);
      sr.rz = sr.rs;
      sr.off = row < N ? (uint32_t)(row * K + kk + 8 * g4) * 2u : kOobOff;
      sr.offz = 0;
      sr.istep = 64;
    }
  };
  // Register buffers of the INT4 walk, two halves each: its bf16 A units
  // take 16 loads of 16 bytes per lane per half, its INT4 W units 4 of codes
  // and 1 of group words.  (The bf16 walk uses the quarter ring below.)
  constexpr int kQL = 5;
  uint4 buf[2][WQ ? kHS : 1];   // bf16 halves (the A units of the INT4 walk)
  uint4 qbuf[2][WQ ? kQL : 1];  // INT4 W halves (WQ only)
  auto load_b = [&](uint4 (&b)[kHS], const UnitSrc& sr, auto hc) __attribute__((always_inline)) {
    constexpr int H = decltype(hc)::value;
#pragma unroll
    for (int i = 0; i < kHS; ++i)
      b[i] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(
                     sr.rs, sr.off, __builtin_amdgcn_readfirstlane((kHS * H + i) * sr.istep), 0));
  };
  // the bf16 walk's ring: four quarters of 8 steps (256 deep, 8 KB per wave)
  uint4 rq[4][kQS];
  auto load_r = [&](uint4 (&b)[kQS], const UnitSrc& sr, auto qc) __attribute__((always_inline)) {
    constexpr int Q = decltype(qc)::value;
#pragma unroll
    for (int i = 0; i < kQS; ++i)
      b[i] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(
                     sr.rs, sr.off, __builtin_amdgcn_readfirstlane((kQS * Q + i) * sr.istep), 0));
  };
  auto load_q = [&](uint4 (&b)[WQ ? kQL : 1], const UnitSrc& sr, auto hc) __attribute__((always_inline)) {
    if constexpr (WQ) {
      constexpr int H = decltype(hc)::value;
      // four groups of 128: the lane's four words of each (one per 32-deep
      // step) as one 16-byte load, then the half's four group words
#pragma unroll
      for (int gi = 0; gi < 4; ++gi)
        b[gi] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(sr.rs, sr.off + 256 * H + 64 * gi, 0, 0));
      b[4] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(sr.rz, sr.offz + 16 * H, 0, 0));
    }
  };
  const auto H0 = std::integral_constant<int, 0>{};
  const auto H1 = std::integral_constant<int, 1>{};

  // ---- the start of the wave's first W unit (three quarters, or an INT4
  // half) goes out after the X copy; the barrier waits for the copy (and the
  // ids before it), not for it ----
  UnitSrc csrc;
  UnitDst cdst;
  const auto Q0 = std::integral_constant<int, 0>{};
  const auto Q1 = std::integral_constant<int, 1>{};
  const auto Q2 = std::integral_constant<int, 2>{};
  const auto Q3 = std::integral_constant<int, 3>{};
  if (nw > 0) {
    w_unit(wi, k0, csrc, cdst);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (WQ) {
      load_q(qbuf[0], csrc, H0);
      barrier_after<kQL>();
    } else {
      // three quarters in flight before the walk starts
      load_r(rq[0], csrc, Q0);
      load_r(rq[1], csrc, Q1);
      load_r(rq[2], csrc, Q2);
      barrier_after<3 * kQS>();
    }
  } else {
    barrier_after<0>();
  }

  // ---- routing entries: a slot-table pool needs one more round after the
  // ids; it goes out now and is first needed by the grouping, after the W units ----
  int slot = id, rank = a.u_ld, mask = -1, bad = 0;
  if (a.lora) {
    if (a.direct) {
      // a direct-mapped pool keeps adapter id in slot id: the pages follow
      // from the ids alone (every rank block up to the padded rank is an
      // item; rows past an adapter's rank are zero)
      if (id >= a.max_slots || id < -1) bad = 1;  // the combine launch rejects the batch
    } else {
      slot = -1;
      rank = 0;
      if (id < -1 || id >= a.max_ids) {
        bad = 1;
      } else if (id >= 0) {
        const int4 e = a.id_info[id];  // {slot, rank, scale bits, module mask}
        if (e.x < 0) bad = 1;
        slot = e.x;
        rank = e.y & (kChainRankFlag - 1);
        mask = e.w;
      }
    }
  }

  // ---- grouping (done when the first A unit is due): the batch's adapters
  // in order of first occurrence, each owning ceil(rank / 16) consecutive
  // items; the A units are item-major over the linears, so the active ones
  // follow the W units without a gap ----
  bool first = false;
  int nq = 0, incl = 0, nu = nw;
  uint64_t grp = 0;  // the lanes holding this lane's adapter
  auto group = [&]() __attribute__((always_inline)) {
    int n_items = 0;
    if (a.lora && __ballot(bad != 0) == 0) {
      // one ballot per bit of the id, each lane keeping the lanes that agree
      // with it on that bit
      const bool v = id >= 0;
      const int nbits = 32 - __builtin_clz((unsigned)max(max(a.max_ids, a.max_slots), 1));
      grp = __ballot(v);
      for (int k = 0; k < nbits; ++k) {
        const bool bit = (id >> k) & 1;
        const uint64_t on = __ballot(v && bit);
        grp &= bit ? on : ~on;
      }
      first = v && lane == (int)__builtin_ctzll(grp);
      nq = first ? (rank + 15) / 16 : 0;
      incl = wave_incl_scan(nq);
      n_items = __builtin_amdgcn_readlane(incl, 63);
    }
    const int NU = NUW + n_mod * n_items;
    nu = wi < NU ? (NU - wi + NWc - 1) / NWc : 0;
  };
  // an A unit's rows: rank block qb of the item's adapter on linear m, at
  // chunk start kk
  auto a_unit = [&](int v, int kk, UnitSrc& sr, UnitDst& ds) __attribute__((always_inline)) {
    const int m = v % n_mod, item = v / n_mod;
    const uint64_t hit = __ballot(first && item >= incl - nq && item < incl);
    const int leader = (int)__builtin_ctzll(hit);  // wave-uniform: readlane, not an LDS shuffle
    const int sl = __builtin_amdgcn_readlane(slot, leader);
    const int r = __builtin_amdgcn_readlane(rank, leader);
    const int mk = __builtin_amdgcn_readlane(mask, leader);
    const int qb = item - __builtin_amdgcn_readlane(incl - nq, leader);
    ds.kind = 1;
    ds.m = m;
    ds.col = 16 * qb;
    ds.members = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(grp >> 32), leader) << 32) |
                 (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)grp, leader);
    // the page holds A^T in fragment tiles: rank block qb's tiles of the
    // chunk are one contiguous 32 KB (ranks past the adapter's are zero);
    // an adapter that does not target this linear streams nothing here
    const bool ok = 16 * qb < min(r, a.rmax) && targets(mk, ka->module[m]);
    const uint16_t* page = a.pages + (size_t)sl * a.slot_stride + ka->a_off[m];
    sr.rs = uniform_rsrc(page, (int)frag_elems(a.u_ld, K) * 2);
    sr.rz = sr.rs;
    sr.off = ok ? (uint32_t)((frag_tile(qb, kk / 32, a.u_ld, K) * 64 + lane) * 16) : kOobOff;
    sr.offz = 0;
    sr.istep = 1024;
  };
  // a unit past the wave's last: no row, no bytes (the loads that a loop
  // issues unconditionally for it return zeros without touching memory)
  auto none = [&](UnitSrc& sr, UnitDst& ds) __attribute__((always_inline)) {
    sr.rs = uniform_rsrc(a.X, 0);
    sr.rz = sr.rs;
    sr.off = kOobOff;
    sr.offz = kOobOff;
    sr.istep = 0;
    ds.kind = -1;
    ds.m = 0;
    ds.col = 0;
    ds.members = 0;
  };
  // the unit after the last W unit: the first A unit, or none
  auto after_w = [&](int j, UnitSrc& sr, UnitDst& ds) __attribute__((always_inline)) {
    group();
    if (j < nu)
      a_unit(wi + j * NWc - NUW, k0, sr, ds);
    else
      none(sr, ds);
  };

  f32x4 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // acc[tb] += (16 rows x 32) . X[16 tb .. 16 tb + 15, k .. k + 31]^T over the
  // half's 16 steps; the unit's rows are the MFMA's A operand, so a lane ends
  // with 4 consecutive rows (columns of the output, or ranks) of one token.
  // The X fragments of step i + 1 are read from LDS while step i's MFMAs run.
  auto compute_b = [&](const uint4 (&b)[kHS], auto hc, f32x4 (&acc)[4]) __attribute__((always_inline)) {
    constexpr int H = decltype(hc)::value;
    __builtin_amdgcn_sched_barrier(0);
    // the chunk's depth, opaque here: the 16 lane masks of the K tail are
    // formed where they are used instead of being hoisted out of the walk
    // (32 live 64-bit masks would spill the scalar registers)
    int kl = klen;
    asm volatile("" : "+s"(kl));
    // the lane's X offset, opaque too: the fragments are read again for
    // every unit, never kept across units in registers
    int xo = r16 * kXs + 8 * g4;
    asm volatile("" : "+v"(xo));
    bf16x8 xf[2][4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) xf[0][tb] = lds_bf16x8(xs + xo + 16 * tb * kXs + kHalf * H);
#pragma unroll
    for (int i = 0; i < kHS; ++i) {
      if (i + 1 < kHS) {
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
          xf[(i + 1) & 1][tb] = lds_bf16x8(xs + xo + 16 * tb * kXs + kHalf * H + 32 * i + 32);
      }
      const bf16x8 wb = __builtin_bit_cast(bf16x8, keep_if(kHalf * H + 32 * i + 8 * g4 < kl, b[i]));
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) acc[tb] = mfma16(wb, xf[i & 1][tb], acc[tb]);
    }
    // order: step 0's reads, then each step's MFMAs with the next step's reads between them
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i + 1 < kHS; ++i) {
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto compute_r = [&](const uint4 (&b)[kQS], auto qc, f32x4 (&acc)[4]) __attribute__((always_inline)) {
    constexpr int Q = decltype(qc)::value;
    __builtin_amdgcn_sched_barrier(0);
    int kl = klen;  // opaque: the tail masks are formed where used (see compute_b)
    asm volatile("" : "+s"(kl));
    int xo = r16 * kXs + 8 * g4;  // opaque likewise (see compute_b)
    asm volatile("" : "+v"(xo));
    bf16x8 xf[2][4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) xf[0][tb] = lds_bf16x8(xs + xo + 16 * tb * kXs + 32 * kQS * Q);
#pragma unroll
    for (int i = 0; i < kQS; ++i) {
      if (i + 1 < kQS) {
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
          xf[(i + 1) & 1][tb] = lds_bf16x8(xs + xo + 16 * tb * kXs + 32 * kQS * Q + 32 * i + 32);
      }
      const bf16x8 wb = __builtin_bit_cast(bf16x8, keep_if(32 * kQS * Q + 32 * i + 8 * g4 < kl, b[i]));
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) acc[tb] = mfma16(wb, xf[i & 1][tb], acc[tb]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i + 1 < kQS; ++i) {
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto compute_q = [&](const uint4 (&b)[WQ ? kQL : 1], auto hc, f32x4 (&acc)[4]) __attribute__((always_inline)) {
    if constexpr (WQ) {
      constexpr int H = decltype(hc)::value;
      const uint4 zz = b[4];
      const uint32_t gw[4] = {zz.x, zz.y, zz.z, zz.w};
      int xo = r16 * kXs + 8 * g4;  // opaque (see compute_b)
      asm volatile("" : "+v"(xo));
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        // a group past the chunk (klen is a multiple of the group) gets
        // scale 0 and offset 0: its weights dequantize to exact zeros
        const bool in = kHalf * H + kQ4Group * gi < klen;
        float2 g = q4_group(gw[gi]);
        g.x = in ? g.x : 0.f;
        g.y = in ? g.y : 0.f;
        const uint32_t words[4] = {b[gi].x, b[gi].y, b[gi].z, b[gi].w};
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const int k = kHalf * H + kQ4Group * gi + 32 * st + 8 * g4;
          const bf16x8 wb = dequant_q4x8(words[st], g.x, g.y);
#pragma unroll
          for (int tb = 0; tb < 4; ++tb)
            acc[tb] = mfma16(wb, lds_bf16x8(xs + xo + 16 * tb * kXs + k - 8 * g4), acc[tb]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  // acc[tb][e]: token 16 tb + r16, row 4 g4 + e of the unit
  auto store_to = [&](const UnitDst& d, f32x4 (&acc)[4]) __attribute__((always_inline)) {
    if (d.kind == 0) {
      // rows past the linear's N land in its padding columns of `part`
      float* pp = a.part + (size_t)plane * 64 * a.npad + (size_t)r16 * a.npad + d.col + 4 * g4;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
        *reinterpret_cast<float4*>(pp + (size_t)(16 * tb) * a.npad) =
            make_float4(acc[tb][0], acc[tb][1], acc[tb][2], acc[tb][3]);
    } else if (d.kind == 1) {
      float* up = a.upart + ((size_t)(plane * n_mod + d.m) * 64 + r16) * a.u_ld + d.col + 4 * g4;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
        if ((d.members >> (16 * tb + r16)) & 1ull)
          *reinterpret_cast<float4*>(up + (size_t)(16 * tb) * a.u_ld) =
              make_float4(acc[tb][0], acc[tb][1], acc[tb][2], acc[tb][3]);
    }
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) acc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  auto store = [&](const UnitDst& d) __attribute__((always_inline)) { store_to(d, acc); };

  // bf16: unit j's first three quarters are in flight when its step starts;
  // each quarter's MFMAs run while the next unit's corresponding quarter is
  // requested.  INT4: unit j's first half is in flight, its second half is
  // requested before the first half's MFMAs, the next unit's first half
  // before the second half's.  Every load is issued unconditionally (past the
  // wave's last unit, rows of no bytes), so the compiler counts each wait
  // exactly.  W units first (INT4 or bf16), then the A units (bf16 pages).
  if constexpr (CPB == 2) {
    // Two chunks.  The wave's units are the same in both passes (the batch
    // is grouped once); unit j's first-chunk sums stay in accs[j] until its
    // second-chunk sums are added to them.  The passes are two copies of
    // straight code (no loop for the sums to flow around).
    f32x4 accs[kMaxUnits][4];
#pragma unroll
    for (int j = 0; j < kMaxUnits; ++j)
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) accs[j][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the second chunk's products of a unit, from zero; then added to the
    // first chunk's
    f32x4 acc2[4];
    auto fresh = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) acc2[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
    };
    auto add_pair = [&](f32x4 (&sum)[4]) __attribute__((always_inline)) {
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int e = 0; e < 4; ++e) sum[tb][e] += acc2[tb][e];
    };
    auto pass = [&](auto pc, bool more) __attribute__((always_inline)) {
      constexpr int P = decltype(pc)::value;
      // the wave's first unit, stride and counts, opaque here: the units'
      // descriptors are formed where they are used, not kept from one pass
      // to the next
      int wj = wi, nwc = NWc, nwp = nw, nup = nu;
      asm volatile("" : "+s"(wj), "+s"(nwc), "+s"(nwp), "+s"(nup));
      if constexpr (P == 0) {
        if (nwp == 0) {
          group();
          nup = nu;
          if (nup > 0) {
            a_unit(wj - NUW, k0, csrc, cdst);
            load_r(rq[0], csrc, Q0);
            load_r(rq[1], csrc, Q1);
            load_r(rq[2], csrc, Q2);
          }
        }
      } else {
        // every wave is done with the chunk in LDS before the next replaces
        // it; the pass's first unit is already in flight
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        ++c;
        k0 += kDecodeChunk;
        klen = min(K, k0 + kDecodeChunk) - k0;
        stage_x();
        barrier_after<0>();
      }
      {
        // the ring as below; after the pass's last unit comes the next
        // pass's first, at the next chunk
        static_for([&](auto jc) __attribute__((always_inline)) {
          constexpr int j = decltype(jc)::value;
          if (j < nup) {
            UnitSrc nsrc;
            UnitDst ndst;
            auto& acc = pick<P>(accs[j], acc2);
            if constexpr (P == 1) fresh();
            load_r(rq[3], csrc, Q3);
            compute_r(rq[0], Q0, acc);
            if (j + 1 < nwp) {
              w_unit(wj + (j + 1) * nwc, k0, nsrc, ndst);
            } else {
              if constexpr (P == 0) {
                if (j + 1 == nwp) {
                  group();  // nu may grow
                  nup = nu;
                }
              }
              if (j + 1 < nup)
                a_unit(wj + (j + 1) * nwc - NUW, k0, nsrc, ndst);
              else if (more && nwp > 0)
                w_unit(wj, k0 + kDecodeChunk, nsrc, ndst);
              else if (more)
                a_unit(wj - NUW, k0 + kDecodeChunk, nsrc, ndst);
              else
                none(nsrc, ndst);
            }
            load_r(rq[0], nsrc, Q0);
            compute_r(rq[1], Q1, acc);
            load_r(rq[1], nsrc, Q1);
            compute_r(rq[2], Q2, acc);
            load_r(rq[2], nsrc, Q2);
            compute_r(rq[3], Q3, acc);
            if constexpr (P == 1) add_pair(accs[j]);
            csrc = nsrc;
          }
        }, std::make_integer_sequence<int, kMaxUnits>{});
      }
    };
    pass(std::integral_constant<int, 0>{}, npass > 1);
    if (npass > 1) pass(std::integral_constant<int, 1>{}, false);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // one plane per pair of chunks
    int wj = wi, nwc = NWc;  // opaque (see the passes)
    asm volatile("" : "+s"(wj), "+s"(nwc));
#pragma unroll
    for (int j = 0; j < kMaxUnits; ++j) {
      if (j < nu) {
        UnitSrc sr;
        UnitDst ds;
        if (j < nw)
          w_unit(wj + j * nwc, k0, sr, ds);
        else
          a_unit(wj + j * nwc - NUW, k0, sr, ds);
        store_to(ds, accs[j]);
      }
    }
    return;
  } else if constexpr (WQ) {
    int j = 0;
    // W units (INT4, two halves through two register buffers), then the A
    // units (bf16 pages, likewise)
    for (; j < nw; ++j) {
      UnitDst ndst;
      load_q(qbuf[1], csrc, H1);
      compute_q(qbuf[0], H0, acc);
      if (j + 1 < nw) {
        w_unit(wi + (j + 1) * NWc, k0, csrc, ndst);
        load_q(qbuf[0], csrc, H0);
        compute_q(qbuf[1], H1, acc);
      } else {
        compute_q(qbuf[1], H1, acc);
        after_w(j + 1, csrc, ndst);
        load_b(buf[0], csrc, H0);
      }
      store(cdst);
      cdst = ndst;
    }
    if (nw == 0) {
      group();
      if (nu == 0) return;  // nothing in flight: the barrier waited for every load
      a_unit(wi - NUW, k0, csrc, cdst);
      load_b(buf[0], csrc, H0);
    }
    for (; j < nu; ++j) {
      load_b(buf[1], csrc, H1);
      compute_b(buf[0], H0, acc);
      UnitDst ndst;
      if (j + 1 < nu)
        a_unit(wi + (j + 1) * NWc - NUW, k0, csrc, ndst);
      else
        none(csrc, ndst);
      load_b(buf[0], csrc, H0);
      compute_b(buf[1], H1, acc);
      store(cdst);
      cdst = ndst;
    }
  } else {
    // bf16: a ring of four quarters; while one quarter's MFMAs run the next
    // three are in flight (24 KB per wave), W units first, then A units
    if (nw == 0) {
      group();
      if (nu == 0) return;  // nothing in flight: the barrier waited for every load
      a_unit(wi - NUW, k0, csrc, cdst);
      load_r(rq[0], csrc, Q0);
      load_r(rq[1], csrc, Q1);
      load_r(rq[2], csrc, Q2);
    }
    for (int j = 0; j < nu; ++j) {
      UnitSrc nsrc;
      UnitDst ndst;
      load_r(rq[3], csrc, Q3);
      compute_r(rq[0], Q0, acc);
      if (j + 1 < nw)
        w_unit(wi + (j + 1) * NWc, k0, nsrc, ndst);
      else if (j + 1 == nw)
        after_w(j + 1, nsrc, ndst);  // groups the batch; nu may grow
      else if (j + 1 < nu)
        a_unit(wi + (j + 1) * NWc - NUW, k0, nsrc, ndst);
      else
        none(nsrc, ndst);
      load_r(rq[0], nsrc, Q0);
      compute_r(rq[1], Q1, acc);
      load_r(rq[1], nsrc, Q1);
      compute_r(rq[2], Q2, acc);
      load_r(rq[2], nsrc, Q2);
      compute_r(rq[3], Q3, acc);
      store(cdst);
      csrc = nsrc;
      cdst = ndst;
    }
  }
  // the last (empty) request has returned before the wave ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ---------------------------------------------------------------------------
// combine: block = 16 tokens x 64 columns of one linear, thread = (token, 4
// columns).  Round 1 of loads depends on nothing: the ids, the chunk partials
// and the shrink partials of the block's V, and in a direct-mapped pool the
// thread's B rows (its token's id comes by a scalar load).  Round 2: every
// token's {slot, rank, scale} (each block checks the whole batch, strict
// mode).  Otherwise the B rows need the slot and come in a third round.
// RP: the pool's rank rounded up to 16, 32 or 64 (the block's V is 16 x RP).
// A rank-16 pool's combine asks for six waves per SIMD (74 registers, no
// spills), so that a large group's blocks (gate/up: 1376) are all resident at
// once instead of a quarter of them starting a generation late.
constexpr int kCombThreads = 256;

template <int RP>
__global__ __launch_bounds__(kCombThreads, RP == 16 ? 6 : 1) void decode_combine(DecodeArgs a) {
  constexpr int kVPer = 16 * RP / kCombThreads;  // V elements per thread
  __shared__ float vsh[16][kMaxRank + 1];
  __shared__ int4 s_info[16];  // the block's tokens: {slot (-1: none), rank, scale bits, 0}
  __shared__ float4 s_bsc[16];  // the block's tokens: scale of each 16-rank block
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  const int T = a.T, KS = a.KP;  // (here: the partial planes, summed in K order)
  // one chunk per plane: the planes of a chunk pair are added first, as a
  // two-chunk block adds them
  const bool pair = a.CPB == 1;
  const KArgs ka = kargs();
  const int mg = group_of(a.ct0, (int)blockIdx.x);  // the block's linear
  const int N = ka->N[mg];
  const int t0 = blockIdx.y * 16;
  const int tr = tid >> 4, quad = tid & 15;
  const int t = t0 + tr;
  const int n = ((int)blockIdx.x - ka->ct0[mg]) * 64 + quad * 4;
  const bool mine = t < T && n < N;
  const size_t pstr = (size_t)64 * a.npad;  // one plane of `part`

  // ---- round 1 ----
  // (the ids for the whole-batch check are stored to LDS only after every
  // other load of this round is out, so that no load waits for them)
  int st = 0, idv = -1;
  if (a.lora) {
    st = *a.status;
    if (tid < 64 && tid < T) idv = a.ids[tid];
  }
  const float* pp = a.part + (size_t)min(t, T - 1) * a.npad + ka->n0[mg] + min(n, N - 4);
  float4 pv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) pv[j] = *reinterpret_cast<const float4*>(pp + (size_t)min(j, KS - 1) * pstr);
  float u[kVPer];
  uint4 bv[8];
  int slot = -1, rank = 0;
  const uint16_t* Bp = nullptr;
  const size_t b_off = ka->b_off[mg];
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
      Bp = a.pages + (size_t)my_id * a.slot_stride + b_off + (size_t)n * 16;
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
      const int r = idx / RP, q = idx % RP;
      uq[e] = q < a.u_ld;
      up[e] = a.upart + ((size_t)mg * 64 + min(t0 + r, T - 1)) * a.u_ld + (uq[e] ? q : 0);
      u[e] = 0.f;
    }
    const size_t ustr = (size_t)a.n_mod * 64 * a.u_ld;  // one plane of upart
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
      if (!bad && e.x >= 0 && !targets(e.w, ka->module[mg])) e = make_int4(-1, 0, 0, 0);
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
      for (int e = 0; e < kVPer; ++e) {
        if (pair) {
#pragma unroll
          for (int h = 0; h < 2; ++h)
            if (c0 + 2 * h < KS && uq[e]) u[e] += c0 + 2 * h + 1 < KS ? v[e][2 * h] + v[e][2 * h + 1] : v[e][2 * h];
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (c0 + j < KS && uq[e]) u[e] += v[e][j];
        }
      }
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
      const int r = idx / RP, q = idx % RP;
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
    Bp = a.pages + (size_t)slot * a.slot_stride + b_off + (size_t)n * 16;
#pragma unroll
    for (int k = 0; k < 8; ++k) bv[k] = *reinterpret_cast<const uint4*>(Bp + 8 * k);
  }

  // base: the partial planes in K order (chunk pairs first)
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  auto add4 = [](float4 x, float4 y) { return make_float4(x.x + y.x, x.y + y.y, x.z + y.z, x.w + y.w); };
  for (int c0 = 0; c0 < KS; c0 += 4) {
    if (c0 > 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        pv[j] = *reinterpret_cast<const float4*>(pp + (size_t)min(c0 + j, KS - 1) * pstr);
    }
    if (pair) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = c0 + 2 * h;
        if (c < KS) {
          const float4 q = c + 1 < KS ? add4(pv[2 * h], pv[2 * h + 1]) : pv[2 * h];
          s = c == 0 ? q : add4(s, q);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (c0 + j < KS) s = c0 + j == 0 ? pv[j] : add4(s, pv[j]);
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
  *reinterpret_cast<uint2*>(ka->out[mg] + (size_t)t * N + n) = make_uint2(o0, o1);
}

template <bool WQ, int CPB>
hipError_t launch_main(const DecodeArgs& a, int wpb, int grid, hipStream_t s) {
  if constexpr (WQ) {
    // the INT4 walk: one or two waves per SIMD (its registers fit in half
    // of a SIMD's file)
    if (wpb == 8)
      hipLaunchKernelGGL((decode_main<8, true, 1>), dim3(grid), dim3(512), 0, s, a);
    else if (wpb == 4)
      hipLaunchKernelGGL((decode_main<4, true, 1>), dim3(grid), dim3(256), 0, s, a);
    else
      return hipErrorInvalidValue;
  } else if constexpr (CPB == 2) {
    // (the units' sums of two chunks: one wave per SIMD)
    if (wpb != 4) return hipErrorInvalidValue;
    hipLaunchKernelGGL((decode_main<4, false, 2>), dim3(grid), dim3(256), 0, s, a);
  } else {
    switch (wpb) {
      case 4: hipLaunchKernelGGL((decode_main<4, WQ, 1>), dim3(grid), dim3(256), 0, s, a); break;
      case 5: hipLaunchKernelGGL((decode_main<5, WQ, 1>), dim3(grid), dim3(320), 0, s, a); break;
      case 6: hipLaunchKernelGGL((decode_main<6, WQ, 1>), dim3(grid), dim3(384), 0, s, a); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

static int resident_of(bool wq, int cpb, int wpb) {
  const int threads = 64 * wpb;
  const void* fn = nullptr;
  if (cpb == 2) {
    fn = reinterpret_cast<const void*>(&decode_main<4, false, 2>);
  } else if (wq) {
    fn = wpb == 8 ? reinterpret_cast<const void*>(&decode_main<8, true, 1>)
                  : reinterpret_cast<const void*>(&decode_main<4, true, 1>);
  } else {
    fn = wpb == 4 ? reinterpret_cast<const void*>(&decode_main<4, false, 1>)
                  : wpb == 5 ? reinterpret_cast<const void*>(&decode_main<5, false, 1>)
                             : reinterpret_cast<const void*>(&decode_main<6, false, 1>);
  }
  return resident_blocks(fn, threads, 0);
}

// The launch shape for `cpb` chunks per block: waves per block and blocks
// per plane.  Waves per block: the shape whose waves are busiest on average
// relative to the busiest one (the launch lasts as long as its busiest wave,
// and the compute units' share of the bandwidth does not depend on how many
// waves split it); one block per compute unit (the X chunk fills most of
// the LDS); a tie keeps fewer waves.  With two chunks per block a wave holds
// at most kMaxUnits units' sums, which may take more blocks than the compute
// units hold at once.
struct Shape {
  int wpb, nbc, resident;
};
static Shape decode_shape(const DecodeArgs& a, int cpb, int units) {
  const int KP = ceil_div(a.KS, cpb);
  Shape best{4, 1, 1};
  double best_eff = -1.0;
  // (at most six waves: with 24 KB in flight per wave, more outstanding
  // reads per compute unit lower the stream rate -- measured 6.0 TB/s at
  // 128 KB per compute unit, 5.4 at 256 KB)
  for (int wpb : {4, 5, 6, 8}) {
    // the two-chunk walk holds every unit's sums: one wave per SIMD; the
    // INT4 walk runs one or two per SIMD (eight waves per block), the bf16
    // one-chunk walk four to six waves per block
    if (cpb == 2 && wpb != 4) continue;
    if (a.wq ? (wpb != 4 && wpb != 8) : wpb == 8) continue;
    const int resident = resident_of(a.wq != 0, cpb, wpb);
    int nbc = std::max(1, std::min(resident / KP, ceil_div(units, wpb)));
    if (cpb == 2) nbc = std::max(nbc, ceil_div(units, wpb * kMaxUnits));
    const int mx = ceil_div(units, nbc * wpb);
    const double eff = (double)units / ((double)nbc * wpb * mx);
    // (the INT4 walk is bound by each SIMD's issue, not by the bytes: two
    // waves per SIMD hide each other's waits, worth some idle waves)
    const bool pair_waves = a.wq && wpb == 8 && eff >= best_eff - 0.25;
    if (eff > best_eff + 1e-9 || pair_waves) {
      best_eff = eff;
      best = Shape{wpb, nbc, resident};
    }
  }
  return best;
}

hipError_t launch_decode(const DecodeArgs& args, int items_cap, hipStream_t s) {
  DecodeArgs a = args;
  // units per K chunk the grid must hold: every W unit plus every A item the
  // batch could have on every linear
  const int units = a.u0[kMaxGroup] + (a.lora ? a.n_mod * items_cap : 0);
  // Chunks per block: two (half the partial planes) where the two-chunk
  // grid still fills nine tenths of the compute units' block slots, else one
  // (a small linear needs every compute unit streaming).  Both add in the
  // same order, so the choice never changes a bit of the output.
  int cpb = 1;
  Shape sh = decode_shape(a, 1, units);
  if (a.KS >= 2 && !a.wq) {
    const Shape s2 = decode_shape(a, 2, units);
    if (10 * s2.nbc * ceil_div(a.KS, 2) >= 9 * s2.resident) {
      cpb = 2;
      sh = s2;
    }
  }
  a.CPB = cpb;
  a.KP = ceil_div(a.KS, cpb);
  a.NWc = sh.nbc * sh.wpb;
  const int grid = sh.nbc * a.KP;
  hipError_t e;
  if (cpb == 2)
    e = launch_main<false, 2>(a, sh.wpb, grid, s);
  else if (a.wq)
    e = launch_main<true, 1>(a, sh.wpb, grid, s);
  else
    e = launch_main<false, 1>(a, sh.wpb, grid, s);
  if (e != hipSuccess) return e;
  const dim3 cgrid(a.ct0[kMaxGroup], (a.T + 15) / 16);
  if (a.u_ld <= 16)
    hipLaunchKernelGGL(decode_combine<16>, cgrid, dim3(kCombThreads), 0, s, a);
  else if (a.u_ld <= 32)
    hipLaunchKernelGGL(decode_combine<32>, cgrid, dim3(kCombThreads), 0, s, a);
  else
    hipLaunchKernelGGL(decode_combine<64>, cgrid, dim3(kCombThreads), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fixed scratch of the allocation-free decode entry point: the K-chunk
// partial planes live here instead of in the pool's workspace.  Every GPU the
// library runs on holds its own copy until the process ends; host code
// reaches a device's copy only through the address hipGetSymbolAddress
// returns for it (the array's name is a host-side stand-in).
static __device__ __align__(256) float scratch[kScratchFloats];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t decode_scratch(float** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = static_cast<float*>(g_scratch_ptr[dev]);
  return hipSuccess;
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
