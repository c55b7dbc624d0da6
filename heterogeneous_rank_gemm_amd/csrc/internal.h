// Internal interface between the host API (api.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hrg {

constexpr int kMaxIds = 16384;       // plan histogram lives in LDS
constexpr int kMaxRank = 64;
// id_info.y = rank | kChainRankFlag for a chain: only then do the kernels
// read id_bscale (the scale of each 16-rank block); a plain adapter's blocks
// all use id_info.z.
constexpr int kChainRankFlag = 1 << 16;
constexpr int kShrinkRows = 64;      // rows per shrink work tile
constexpr int kMaxSplits = 32;       // K-splits of the shrink
// Segments of at most kSmallRows tokens are expanded by a separate launch into
// fp32 rows of E (at most kMaxSmallRows such tokens per plan); the GEMM starts
// those rows' accumulators from E instead of walking every small segment.
constexpr int kSmallRows = 8;
constexpr int kMaxSmallRows = 512;
// Device status codes (values of lora_status_t; a larger code wins).
constexpr int kStatusNotLoaded = 6;
constexpr int kStatusIdRange = 7;

inline __host__ __device__ int round_up(int x, int m) { return (x + m - 1) / m * m; }
inline __host__ __device__ int ceil_div(int x, int m) { return (x + m - 1) / m; }

// Fragment tiles (the "packed" layout) of a rows x cols bf16 matrix M: tiles
// of 16 rows by 32 columns, 1 KB each.  Inside a tile the 16 bytes of lane
// l = 16 j + r hold M[16 g + r][32 s + 8 j .. 32 s + 8 j + 7], exactly the
// operand a lane supplies to one 16x16x32 bf16 MFMA step, so a wave loads a
// tile with one contiguous 1-KB instruction.  Tiles are ordered by 1024-deep
// column block, then row group, then step: a decode unit (16 rows of one
// 1024-deep K chunk) is one contiguous 32 KB.  Measured on MI355X by pure
// reads in the decode walk's order: the row-major layout (every 16-byte
// operand load touching 16 rows) 4.6 TB/s, tiles ordered row group first
// 4.7 TB/s (the waves of a chunk meet on a few memory channels), this order
// 6.0-6.2 TB/s with 64-128 KB in flight per compute unit.  Rows and columns
// are zero-padded to multiples of 16 and 32.
constexpr int kFragChunk = 1024;  // columns of a tile block (the decode K chunk)
inline __host__ __device__ size_t frag_elems(int rows, int cols) {
  return (size_t)round_up(rows, 16) * round_up(cols, 32);
}
// 1-KB tile index of (row group g, step s) in a rows x cols matrix
inline __host__ __device__ size_t frag_tile(int g, int s, int rows, int cols) {
  const int k32 = (cols + 31) / 32, ng = (rows + 15) / 16;
  const int c = s / (kFragChunk / 32), left = k32 - c * (kFragChunk / 32);
  const int sc = left < kFragChunk / 32 ? left : kFragChunk / 32;  // steps of this column block
  return (size_t)c * ng * (kFragChunk / 32) + (size_t)g * sc + (s - c * (kFragChunk / 32));
}
inline __host__ __device__ size_t frag_index(int r, int c, int rows, int cols) {
  return (frag_tile(r >> 4, c >> 5, rows, cols) * 64 + 16 * ((c & 31) >> 3) + (r & 15)) * 8 + (c & 7);
}

// Device tables of one plan.  Sizes: T_cap = pool max_tokens.
struct PlanTables {
  int32_t* perm;       // [T_cap]   sorted position -> token
  int32_t* inv;        // [T_cap]   token -> sorted position
  int32_t* row_seg;    // [T_cap]   sorted position -> segment
  int32_t* seg_id;     // [T_cap+1] segment -> adapter id (-1 first if present)
  int32_t* seg_off;    // [T_cap+2] segment start offsets, seg_off[S] = T
  int32_t* seg_slot;   // [T_cap+1] pool slot (-1 for the base segment)
  int32_t* seg_rank;   // [T_cap+1] true rank (0 for the base segment)
  float* seg_scale;    // [T_cap+1] alpha / rank
  int4* tile_info;     // [max_tiles] shrink work tile: {first sorted row, rows, pool slot, rank}
  int32_t* seg_e0;     // [T_cap+1] first E row of a small segment, -1 otherwise
  int32_t* erow;       // [T_cap]   sorted position -> E row, -1 if not in a small segment
  int4* small_info;    // [kMaxSmallRows] the small segments in order: {first sorted row,
                       //   rows | first E row << 8 | rank << 20, pool slot, alpha / rank bits}
  float4* seg_bscale;  // [T_cap+1] per-16-rank-block scales of each segment's adapter
  float4* small_bscale;  // [kMaxSmallRows] the same for each small segment
  int32_t* counts;     // [0] = S, [1] = number of shrink tiles, [2] = T, [3] = small segments
  int32_t max_tiles;
};

struct PlanArgs {
  const int32_t* ids;
  int32_t T;
  int32_t max_ids;
  const int4* id_info;     // [max_ids] {slot (-1: not resident), rank, scale bits, module mask}
  const float4* id_bscale; // [max_ids] scale of each 16-rank block (a chain's members differ)
  int32_t* status;
  PlanTables tab;
};

// Linears whose shrink one launch computes together (they read the same X):
// rank blocks of all of them per item, at most 4.
constexpr int kMaxShrinkLinears = 4;

struct ShrinkArgs {
  const uint16_t* X;      // [T][K], T * K * 2 < 2^31
  int32_t T, K;
  const int32_t* perm;
  const int4* tile_info;
  const int32_t* counts;
  const uint16_t* pages;  // A^T page of (slot, module): pages + slot*slot_stride + a_off[m]
  size_t slot_stride;
  size_t a_off[kMaxShrinkLinears];  // the item's linears (nl of them, one d_in)
  float* upart;           // [linear][split][T_cap][u_ld] fp32 partial planes (plane m * nsplit + split)
  size_t split_stride;
  int32_t u_ld;
  int32_t kchunk;         // K per split
  int32_t nsplit;         // splits (planes) per tile
  const int32_t* status;
};

struct GemmArgs {
  const uint16_t* X;      // [T][K], T * K * 2 < 2^31
  const uint16_t* W;      // [N][K]
  uint16_t* out;          // [T][N]
  int32_t T, N, K;
  int32_t row0, row1;     // sorted rows [row0, row1) of this launch (set by launch_prefill)
  const int32_t* perm;    // sorted row -> token; nullptr = identity (base-only)
  // expand (unused by the base-only instantiation)
  uint16_t* v_hi;         // [T_cap][u_ld] s * U, bf16 high part, sorted rows
  uint16_t* v_lo;         // [T_cap][u_ld] bf16 low part
  int32_t u_ld;
  // the shrink's partial planes, summed into V by the small-segment launch
  const float* upart;     // [nsplit][T_cap][u_ld]
  size_t split_stride;
  int32_t nsplit;
  const float* seg_scale;
  const float4* seg_bscale;   // per-16-rank-block scales of each segment (V = s U per block)
  const float4* small_bscale; // the same per small segment
  const int32_t* row_seg;
  const int32_t* seg_id;
  const int32_t* seg_off;
  const int32_t* seg_slot;
  const int32_t* seg_rank;
  const uint16_t* pages;  // B^T page of (slot, module): pages + slot*slot_stride + b_off,
  size_t slot_stride;     //   16-rank chunks [rpad/16][N][16]
  size_t b_off;
  const int32_t* status;
  // small segments: their rows' s (U B) terms in fp32, E [kMaxSmallRows][N]
  const int32_t* seg_e0;
  const int32_t* erow;
  const int4* small_info;
  const int32_t* counts;
  float* E;
};

// Decode path (T <= kDecodeMaxT): launch 1 computes the K-chunk partials of
// the base GEMM (W rows) and of the shrink (A rows) of a group of linears that
// read the same X, launch 2 combines them with the expand.  Workspace: part
// [KS][64][npad] and upart [KS][n_mod][64][u_ld] (fp32).
constexpr int kDecodeMaxT = 64;
constexpr int kDecodeTileRows = 64;   // combine columns per block
constexpr int kDecodeChunk = 1024;    // K per block
constexpr int kMaxGroup = 8;          // linears of one grouped decode launch

struct DecodeArgs {
  const uint16_t* X;      // [T][K], shared by every linear of the group
  const int32_t* ids;     // [T]
  int32_t T, K, KS;       // KS = ceil(K / kDecodeChunk)
  int32_t CPB, KP;        // K chunks per block (1 or 2) and partial planes, ceil(KS / CPB)
                          // (set by launch_decode)
  int32_t n_mod;          // linears in the group, 1..kMaxGroup
  // per linear of the group (entries >= n_mod unused)
  const uint16_t* W[kMaxGroup];    // [N][K] bf16 base weight, or
  const uint32_t* Wq[kMaxGroup];   // [N][K/8] packed INT4 weight (layout below)
  const uint32_t* Wsz[kMaxGroup];  // [N][K/128] {bf16 scale, zero point << 16}
  uint16_t* out[kMaxGroup];        // [T][N]
  int32_t N[kMaxGroup];
  int32_t module[kMaxGroup];       // pool module index (target mask bit)
  size_t a_off[kMaxGroup], b_off[kMaxGroup];  // the module's pages inside a slot
  int32_t u0[kMaxGroup + 1];   // first 16-row W unit of each linear; u0[n_mod] = W units
  int32_t n0[kMaxGroup + 1];   // first column of each linear in `part` (multiples of 16)
  int32_t ct0[kMaxGroup + 1];  // first 64-column combine tile of each linear
  int32_t max_ids;
  const int4* id_info;    // [max_ids] {slot (-1: not resident), rank, scale bits, module mask}
  const float4* id_bscale; // [max_ids] scale of each 16-rank block
  const uint16_t* pages;
  size_t slot_stride;
  float* part;            // [KP][64][npad] (room for KS planes)
  float* upart;           // [KP][n_mod][64][u_ld] (room for KS planes)
  int32_t npad;           // n0[n_mod]
  int32_t direct;         // pool keeps adapter id in slot id (max_ids <= max_adapters)
  int32_t max_slots;      // resident slots of the pool
  int32_t rmax;           // rows of an A page (the pool's max rank)
  int32_t u_ld;           // the pool's rank rounded up to 16
  int32_t* status;
  int32_t NWc;            // waves per K chunk (set by launch_decode)
  int32_t lora;
  int32_t wq;             // INT4 base weights (Wq, Wsz) instead of W
  int32_t wpacked;        // every W[i] is in fragment tiles (frag_elems(N, K) elements)
};

// INT4 base weight layout (group size kQ4Group along K; K % kQ4Group == 0).
// Word p of group g of row n (Wq[n][16 g + p], p = 4 j + s) holds the eight
// weights k = 128 g + 32 s + 8 j + e, e = 0..7, nibble e at bits 4e..4e+3: a
// lane that supplies k in [8 j, 8 j + 8) of the MFMA's 32-deep steps reads
// the four steps of a group as one 16-byte load.  Wsz[n][g] = bf16 scale bits
// | zero point << 16.  The weight is bf16((q - z) * scale).
constexpr int kQ4Group = 128;
// Dequantizes an INT4 weight into a bf16 [N][K] buffer (one launch).
hipError_t launch_q4_dequant(const uint32_t* Wq, const uint32_t* Wsz, int N, int K, uint16_t* W,
                             hipStream_t s);

// Page layouts inside a slot (rows past the adapter's rank are zero):
//   A page: A^T (rpad x d_in) in fragment tiles, frag_elems(rpad, d_in)
//           elements (pack mode 0, src d_in x rank)
//   B page: B^T in 16-rank chunks [rpad/16][d_out][16], element (q, n) at
//           (q / 16) * d_out * 16 + n * 16 + q % 16  (pack mode 1, src rank x d_out)
// Pack mode 2 writes a caller's row-major base weight (src N x K, `rank` = N
// rows) in fragment tiles for the decode kernels.
struct PackArgs {
  const uint16_t* src;    // staged A (d_in x rank), B (rank x d_out) or W (N x K), row-major
  uint16_t* dst;
  int32_t rank, rows;     // valid source rows (the true rank; N); page rows (rpad for A and B, N)
  int32_t cols;           // d_in for A, d_out for B, K for W
  int32_t mode;           // 0: A page, 1: B page, 2: W in fragment tiles
};

// Blocks of `fn` (block size `threads`, dynamic LDS `lds`) the current device
// holds at once: the occupancy per compute unit times the compute units.
// Cached per kernel; at least 1.
int resident_blocks(const void* fn, int threads, size_t lds);

// Launchers (return hipSuccess or the launch error).
hipError_t launch_plan(const PlanArgs& a, hipStream_t s);
// Shrink partial planes, then the split reduction into V (two launches).
// nl linears (1 .. 4 / (rank blocks of the pool), see shrink_linears)
hipError_t launch_shrink(const ShrinkArgs& a, int nl, int grid, int ksplit, int T, hipStream_t s);
inline int shrink_linears(int u_ld) { return kMaxShrinkLinears / (u_ld <= 16 ? 1 : u_ld <= 32 ? 2 : 4); }
// shape < 0 picks the tile shapes from (T, N): one shape for every row, or
// 256x256 tiles over the first rows (whole 256-row tiles) and 128x128 or
// 64x64 tiles over the rest, as two launches; 0..4 force 256x256, 256x128,
// 128x256, 128x128, 64x64 (tokens x columns) for every row.  Every shape
// gives the same bits.
hipError_t launch_prefill(const GemmArgs& a, bool lora, int shape, hipStream_t s);
// The E rows of the small segments (one launch, before the GEMM).
hipError_t launch_expand_small(const GemmArgs& a, hipStream_t s);
int prefill_choose(int T, int N);
// The allocation-free decode entry point keeps its partial planes in a fixed
// device array of kScratchFloats floats (16 MiB per GPU).  decode_scratch
// returns the current device's copy (looked up once per device).
constexpr size_t kScratchFloats = (size_t)4 << 20;
constexpr int kMaxDevices = 64;
hipError_t decode_scratch(float** ptr);
// Picks the waves per block and the blocks per K chunk for the group's W
// units plus `items_cap` A items per linear (the most a batch can hold), then
// launches both kernels.
hipError_t launch_decode(const DecodeArgs& a, int items_cap, hipStream_t s);
hipError_t launch_pack(const PackArgs& a, hipStream_t s);
// Routing-table update of one id; `mask` = the modules the adapter targets
// (bit m: module m; modules >= 32 are always targeted), kept in id_info.w.
// `bscale`: the scale of each 16-rank block (all equal to `scale` but for
// chains), kept in id_bscale.
hipError_t launch_set_slot(int32_t* id2slot, int32_t* slot_rank, float* slot_scale, int4* id_info,
                           float4* id_bscale, int32_t id, int32_t slot, int32_t rank, float scale,
                           int32_t mask, float4 bscale, hipStream_t s);
hipError_t launch_clear_i32(int32_t* p, int32_t n, int32_t value, hipStream_t s);
// Routing-table updates of several distinct ids, each {id, slot (-1: not
// addressable), rank, scale bits}; launched in chunks of kSlotUpdatesPerLaunch.
constexpr int kSlotUpdatesPerLaunch = 64;
// Page-in of host-cached adapters: one launch copies up to kPageMovesPerLaunch
// whole slots, {host-cache slot, device slot} each, reading the pinned host
// cache through its device mapping.  slot_vec = 16-byte vectors per slot.
constexpr int kPageMovesPerLaunch = 64;
hipError_t launch_page_in(const void* host_cache_dev, void* pages, const int2* moves, int n,
                          size_t slot_vec, hipStream_t s);
hipError_t launch_set_slots(int32_t* id2slot, int32_t* slot_rank, float* slot_scale, int4* id_info,
                            float4* id_bscale, const int4* updates, const int32_t* masks, int n,
                            hipStream_t s);

}  // namespace hrg
