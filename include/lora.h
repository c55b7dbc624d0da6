/*
 * lora.h -- C ABI of the heterogeneous-batch LoRA-augmented linear for
 * AMD Instinct MI355X (gfx950).
 *
 * One call computes, for every token row t of a batch,
 *
 *     out[t, :] = bf16( X[t, :] W^T  +  (alpha_i / r_i) (X[t, :] A_i) B_i ),
 *     i = ids[t]; id -1 means "base only" (no LoRA term at all),
 *
 * with fp32 accumulation and exactly one round-to-nearest-even to bf16 per
 * output.  All adapters live in one device pool owned by the library.
 *
 * Pages this interface follows (cited by title and section):
 *   [LoRA-Land]  "LoRA-Land: turning the LLM into an operating system with
 *                hot-pluggable multi-task fine-tuned serving" (blog.itodd.wang)
 *   [vLLM-ch7]   "Multi-LoRA hot-plug: one model serving many tenants"
 *                (gufacode.com, vLLM chapter 7)
 *   [icman]      field report on Multi-LoRA in managed inference
 *                (icman.com.cn news 62580)
 *
 * Conventions for every entry point
 *   - All matrices are row-major and hold bf16 bit patterns (lora_bf16_t).
 *   - W is d_out x d_in, X is T x d_in, out is T x d_out   (out = X W^T ...).
 *     A is d_in x r and B is r x d_out ([vLLM-ch7] "LoRA at a glance" gives
 *     A (d x r), B (r x d); [LoRA-Land] section "2. multi-LoRA batch
 *     scheduling" evaluates X A first, then B).
 *   - X, W, ids and out are caller-owned DEVICE buffers; the library never
 *     frees or keeps them beyond the call's stream work.
 *   - Every call returns a lora_status_t.  Errors that the host can detect
 *     (null pointers, shapes, module index, sizes, rank, capacity) return
 *     synchronously and have no side effects.
 *   - Work is enqueued on the caller's stream; calls on one pool must be
 *     ordered on one stream (they share the pool's workspace).  Calls that
 *     overlap on different streams race.
 *   - A pool's host-side state is not locked: calls on one pool (and its
 *     plans) come from one host thread at a time; different pools may be
 *     driven from different threads.
 *   - d_in and d_out must be multiples of 8 (16-byte rows of bf16).
 */
#ifndef HRG_LORA_H
#define HRG_LORA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t lora_bf16_t;              /* bf16 bit pattern */
typedef struct lora_pool_s* lora_pool_t;     /* opaque adapter pool */
typedef struct lora_plan_s* lora_plan_t;     /* opaque grouping plan */

typedef enum {
  LORA_OK = 0,
  LORA_ERR_INVALID_ARG = 1, /* null pointer, bad shape, bad module, T > max_tokens, ... */
  LORA_ERR_OOM = 2,         /* device allocation failed (create, plan_create only) */
  LORA_ERR_POOL_FULL = 3,   /* every resident slot is in use */
  LORA_ERR_RANK = 4,        /* rank outside [1, max_rank] */
  LORA_ERR_EXISTS = 5,      /* id already loaded (no silent overwrite) */
  LORA_ERR_NOT_LOADED = 6,  /* id not resident (strict mode: never falls back to base) */
  LORA_ERR_ID_RANGE = 7,    /* id outside [-1, max_ids) */
  LORA_ERR_HIP = 8          /* a HIP runtime call failed */
} lora_status_t;

/* Human-readable name of a status code (static string). */
const char* lora_status_string(lora_status_t s);

/*
 * lora_pool_create -- the unified adapter pool ([vLLM-ch7] "how vLLM
 * implements multi-LoRA": all adapters in one device memory pool;
 * [LoRA-Land] "3. hot-plug API": the kernel object sized by max_adapters).
 *
 *   pool          out: the new pool handle
 *   max_adapters  resident slots (like --max-loras / --max-active-adapters)
 *   max_ids       adapter ids are valid in [0, max_ids); 1..16384
 *   max_rank      page rank; every adapter's pages are zero-padded to it
 *                 ([vLLM-ch7] "performance notes": mixed ranks are aligned
 *                 to the largest); 1..64 (--max-lora-rank 64)
 *   n_modules     number of LoRA-augmented linears served by the pool
 *   d_in, d_out   host arrays [n_modules]; multiples of 8, 8..65536, and
 *                 d_in * d_out * 2 <= 2^31 - 1 (a base weight under 2 GiB:
 *                 the decode kernels address it with 32-bit byte offsets)
 *   max_tokens    largest T accepted by lora_apply / lora_plan; 1..65536
 *   stream        stream used to initialise the device tables
 *
 * Memory: max_adapters * sum_m max_rank*(d_in[m]+d_out[m]) * 2 bytes of
 * pages plus O(max_ids + max_tokens*max_rank) of tables and workspace, all
 * allocated here.  Returns INVALID_ARG, OOM or HIP; *pool is untouched on error.
 */
lora_status_t lora_pool_create(lora_pool_t* pool, int32_t max_adapters, int32_t max_ids,
                               int32_t max_rank, int32_t n_modules, const int32_t* d_in,
                               const int32_t* d_out, int32_t max_tokens, hipStream_t stream);

/* Frees the pool and every plan still attached to it.  Synchronises the device. */
lora_status_t lora_pool_destroy(lora_pool_t pool);

/*
 * lora_load_adapter -- hot-load one adapter ([LoRA-Land] "3. hot-plug API":
 * load moves A and B to the GPU and builds an index; [vLLM-ch7] "dynamic
 * online/offline": loading without restarting the service).
 *
 *   id     adapter id in [0, max_ids)                      else ID_RANGE
 *   rank   true rank r, 1 <= r <= max_rank                 else RANK
 *   alpha  scaling numerator; the scale is alpha / r (fp32)
 *          ([vLLM-ch7] PEFT config lora_alpha=32 at r=16; [icman] 3.2)
 *   A      host array [n_modules] of pointers, A[m] is d_in[m] x r
 *   B      host array [n_modules] of pointers, B[m] is r x d_out[m]
 *          A[m], B[m] may point to host or device memory; they are copied
 *          before the call returns and may be freed afterwards.
 *          Target sets ([vLLM-ch7] performance notes: adapters with different
 *          target_modules in one batch send some sequences down a skip path;
 *          [icman] 2.1: the branch is added on the target linears only):
 *          A[m] == B[m] == NULL means the adapter does not target module m,
 *          and its tokens get exactly lora_base_apply's rows there.  One of
 *          the two NULL, no module targeted, or an untargeted module in a
 *          pool of more than 32 modules is INVALID_ARG.
 *
 * EXISTS also if the id is in the pool's host cache (lora_host_register).
 * Slot choice: a pool with max_ids <= max_adapters is direct-mapped and
 * keeps adapter id in slot id (the decode kernels then address its pages
 * from the ids alone, without a round of slot-table loads); otherwise the
 * adapter takes the lowest free slot.  An id already resident returns EXISTS
 * ([icman] 4.3 warns against silent overwrites); a full pool returns
 * POOL_FULL (eviction is the caller's policy).  Synchronises `stream`.
 */
lora_status_t lora_load_adapter(lora_pool_t pool, int32_t id, int32_t rank, float alpha,
                                const lora_bf16_t* const* A, const lora_bf16_t* const* B,
                                hipStream_t stream);

/*
 * lora_unload_adapter -- release an adapter's slot ([LoRA-Land] "3. hot-plug
 * API": unload frees the adapter's caches; [vLLM-ch7] unload endpoint).
 * Waits for `stream` first, so work already enqueued there never reads a
 * recycled page.  NOT_LOADED if the id is not resident, ID_RANGE if out of range.
 * For an adapter in the host cache (lora_host_register) it drops the device
 * copy only (NOT_LOADED if there is none); the host copy stays.
 */
lora_status_t lora_unload_adapter(lora_pool_t pool, int32_t id, hipStream_t stream);

/*
 * lora_load_chain -- a chain of resident adapters under a new id ([LoRA-Land]
 * "technical approach", item 3: several LoRAs composed like a pipeline and
 * applied in turn; section "3. hot-plug API and composition":
 * set_adaptive_chain).  At a linear layer each member adds its own update,
 * so a token routed to the chain gets
 *     out = bf16( X W^T + sum_c (alpha_c / r_c) (X A_c) B_c ),
 * with one rounding.  The chain is a new adapter whose pages hold the
 * members' pages side by side in whole 16-rank blocks (member c's blocks
 * carry its scale); the members are copied (snapshotted), so unloading one
 * later leaves the chain as it was.  Unload the chain with
 * lora_unload_adapter.
 *   members  host array [n], n >= 1, distinct resident ids that are not
 *            chains (host-cached adapters must be addressable at the call)
 * ID_RANGE (chain_id or a member out of range), INVALID_ARG (n, repeats, a
 * chain as member), NOT_LOADED (a member not addressable), RANK (the blocks
 * of all members but the last plus the last's rank exceed max_rank), EXISTS,
 * POOL_FULL.  The RANK rule is this library's page layout, stricter than the
 * pages' (a chain is one adapter of rank sum_c r_c <= max rank): every member
 * but the last takes whole 16-rank blocks, so ranks 5 + 5 + 5 need 37 page
 * rows, not 15.  The chain's target set is the union of its members'.
 * lora_pool_query reports the chain's rank as that total and its scale as the
 * first member's.  Synchronises `stream`.
 */
lora_status_t lora_load_chain(lora_pool_t pool, int32_t chain_id, int32_t n, const int32_t* members,
                              hipStream_t stream);

/* Host-side lookup: slot, true rank and scale of a resident id (any out
 * pointer may be NULL).  NOT_LOADED / ID_RANGE as above. */
lora_status_t lora_pool_query(lora_pool_t pool, int32_t id, int32_t* slot, int32_t* rank,
                              float* scale);

/*
 * Plans: the grouping of a batch by adapter id ([LoRA-Land] section "2.
 * multi-LoRA batch scheduling": group the batch by LoRA id, "Grouped
 * Multi-LoRA Execution").  The plan is a stable sort of token indices by
 * (id ascending, index ascending), -1 first, plus the segment table of the
 * maximal runs of equal id.  One plan can serve every linear of a step.
 *
 * lora_plan_create allocates device tables sized for the pool's max_tokens.
 */
lora_status_t lora_plan_create(lora_pool_t pool, lora_plan_t* plan);
lora_status_t lora_plan_destroy(lora_pool_t pool, lora_plan_t plan);

/*
 * lora_plan -- build `plan` from device ids[T] on `stream` (no host sync).
 * Ids are validated on the device (strict mode, [icman] 4.1): an id outside
 * [-1, max_ids) or not resident sets the pool's sticky error status; every
 * later lora_apply on the pool then leaves its output untouched until
 * lora_status() reports and clears the error.  T = 0 is valid (S = 0).
 * INVALID_ARG if T < 0, T > max_tokens, or ids is NULL with T > 0.
 */
lora_status_t lora_plan(lora_pool_t pool, const int32_t* ids, int32_t T, lora_plan_t plan,
                        hipStream_t stream);

/*
 * lora_apply -- the heterogeneous-batch LoRA linear for module `module`
 * ([LoRA-Land] section 2 formula; [vLLM-ch7] "heterogeneous batching": one
 * forward computes every request's own side path; [icman] 2.1 dynamic
 * batching mode).
 *
 *   X     device, T x d_in[module]
 *   ids   device int32[T], each -1 or a resident id
 *   W     device, d_out[module] x d_in[module] (the frozen base weight)
 *   out   device, T x d_out[module]; written in the original token order
 *   plan  NULL: the call plans `ids` itself.  Otherwise a plan built by
 *         lora_plan from the same `ids` pointer and T (INVALID_ARG if not).
 *
 * Asynchronous; id errors are reported through the sticky status (see
 * lora_plan / lora_status), and then `out` is not written.  T = 0 is a no-op.
 * Rows with id -1 are bit-identical to lora_base_apply's rows.
 */
lora_status_t lora_apply(lora_pool_t pool, int32_t module, const lora_bf16_t* X,
                         const int32_t* ids, int32_t T, const lora_bf16_t* W, lora_bf16_t* out,
                         lora_plan_t plan, hipStream_t stream);

/*
 * lora_base_apply -- out = bf16(X W^T) with the same GEMM kernels and tile
 * choice as lora_apply but no LoRA term ([vLLM-ch7] "switching LoRA per
 * request": a request naming no LoRA runs the plain base).  It is the
 * denominator of the LoRA-overhead figure.  Same argument rules as lora_apply.
 */
lora_status_t lora_base_apply(lora_pool_t pool, int32_t module, const lora_bf16_t* X, int32_t T,
                              const lora_bf16_t* W, lora_bf16_t* out, hipStream_t stream);

/*
 * lora_apply_group / lora_base_apply_group -- lora_apply / lora_base_apply
 * for n linears that read the same X, in one call ([LoRA-Land] section "2.
 * multi-LoRA batch scheduling": one forward serves the whole grouped batch;
 * the q/k/v and gate/up projections of a layer read one hidden state).
 *
 *   n        1..8 linears
 *   modules  host int32[n]: distinct pool modules with one d_in
 *   W        host array [n] of device pointers, W[i] is d_out[modules[i]] x d_in
 *   out      host array [n] of device pointers, out[i] is T x d_out[modules[i]]
 *   X, ids, T, plan, stream as lora_apply
 *
 * Each out[i] is exactly what lora_apply (lora_base_apply) on module
 * modules[i] writes, bit for bit.  At T <= 64 the group runs as one launch
 * pair that stages X once for all n linears; at larger T one plan serves the
 * n linears in turn.  Errors as lora_apply, plus INVALID_ARG for n outside
 * 1..8, a repeated module or modules of different d_in.
 */
lora_status_t lora_apply_group(lora_pool_t pool, int32_t n, const int32_t* modules, const lora_bf16_t* X,
                               const int32_t* ids, int32_t T, const lora_bf16_t* const* W,
                               lora_bf16_t* const* out, lora_plan_t plan, hipStream_t stream);
lora_status_t lora_base_apply_group(lora_pool_t pool, int32_t n, const int32_t* modules, const lora_bf16_t* X,
                                    int32_t T, const lora_bf16_t* const* W, lora_bf16_t* const* out,
                                    hipStream_t stream);

/*
 * Decode-layout base weights.  The decode kernels (T <= 64) stream the base
 * weight once per call and are bound by its bytes; with the row-major layout
 * every 16-byte MFMA operand load of a wave touches 16 rows, which the memory
 * path serves at about three quarters of the rate of contiguous reads.  A
 * weight packed once into fragment tiles (16 rows x 32 columns, 1 KB each,
 * inside a tile lane l = 16 j + r holds row 16 g + r,
 * columns 32 s + 8 j .. + 7; rows and columns zero-padded to multiples of 16
 * and 32; tiles ordered by 1024-column block, then row group, then column)
 * is read as contiguous 1-KB pieces, a 16-row unit of one 1024-deep chunk
 * as 32 contiguous kilobytes.  The adapters' A pages in the
 * pool already use this layout.
 *
 * lora_packed_weight_elems -- elements (bf16) of the packed form of an N x K
 *   weight: round_up(N, 16) * round_up(K, 32).  INVALID_ARG on N or K < 1 or
 *   a NULL elems.
 * lora_pack_weight -- writes the packed form of the row-major device weight
 *   W (N x K, bf16) into the device buffer Wp (lora_packed_weight_elems
 *   elements, caller-owned), on `stream`.  N and K multiples of 8 in
 *   8..65536 with a packed size under 2 GiB, else INVALID_ARG.  W and Wp must
 *   not overlap.
 * lora_apply_group_packed / lora_base_apply_group_packed -- lora_apply_group
 *   / lora_base_apply_group with every Wp[i] packed from the linear's
 *   row-major weight; outputs bit-identical to the row-major calls (the same
 *   products in the same order).  Decode batches only: T <= 64, else
 *   INVALID_ARG (the batched path takes the row-major weight).  The grouping
 *   is built in the launch, so there is no plan argument.
 */
lora_status_t lora_packed_weight_elems(int32_t N, int32_t K, int64_t* elems);
lora_status_t lora_pack_weight(const lora_bf16_t* W, int32_t N, int32_t K, lora_bf16_t* Wp, hipStream_t stream);
lora_status_t lora_apply_group_packed(lora_pool_t pool, int32_t n, const int32_t* modules, const lora_bf16_t* X,
                                      const int32_t* ids, int32_t T, const lora_bf16_t* const* Wp,
                                      lora_bf16_t* const* out, hipStream_t stream);
lora_status_t lora_base_apply_group_packed(lora_pool_t pool, int32_t n, const int32_t* modules,
                                           const lora_bf16_t* X, int32_t T, const lora_bf16_t* const* Wp,
                                           lora_bf16_t* const* out, hipStream_t stream);

/*
 * lora_apply_noalloc -- lora_apply for callers that cannot allocate device
 * memory during the call: code under hipGraph capture that must not meet an
 * allocation, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, results (bit for bit) and errors as lora_apply on a decode batch
 * (no plan argument: the launch groups the batch itself), but the kernels'
 * scratch (the K-chunk partial planes) is a fixed array of 16 MiB per GPU
 * inside the library instead of the pool's workspace, and the call makes no
 * allocation of any kind.
 *   limits  T <= 64, and ceil(d_in / 1024) * 64 * (round_up(d_out, 16) +
 *           rank rounded up to 16) floats <= 4 Mi (e.g. d_in 4096 with d_out
 *           up to 16320, d_in 11008 with d_out up to 5888); else INVALID_ARG
 *           with no work enqueued.
 * The array is shared by every call on a GPU and keeps the last call's
 * contents (nothing in it needs to start at zero): calls that overlap on one
 * GPU, from any pool or stream, race.  Serialise them (one stream, or events).
 */
lora_status_t lora_apply_noalloc(lora_pool_t pool, int32_t module, const lora_bf16_t* X, const int32_t* ids,
                                 int32_t T, const lora_bf16_t* W, lora_bf16_t* out, hipStream_t stream);

/*
 * INT4 base weight ([vLLM-ch7] performance notes: an AWQ-INT4 base with bf16
 * adapters).  The frozen base weight is stored group-wise in 4 bits along
 * d_in: groups of 128, q and the zero point z in 0..15, a bf16 scale s per
 * (output row, group), and the GEMM uses W[n, k] = bf16((q - z) * s).  The
 * adapters stay bf16.  d_in must be a multiple of 128.
 *
 * lora_q4_pack -- host-side packing into the device layout.
 *   q    host uint8 [N][K], values 0..15 (row n = output feature)
 *   z    host uint8 [N][K/128], values 0..15
 *   s    host bf16 bits [N][K/128]
 *   Wq   host out uint32 [N][K/8]: word 16 g + 4 j + st of row n holds the
 *        weights k = 128 g + 32 st + 8 j + e, e = 0..7, in bits 4e..4e+3
 *   Wsz  host out uint32 [N][K/128]: s bits | z << 16
 * INVALID_ARG on a null pointer, K not a multiple of 128, or a value > 15.
 */
lora_status_t lora_q4_pack(const uint8_t* q, const uint8_t* z, const lora_bf16_t* s, int32_t N,
                           int32_t K, uint32_t* Wq, uint32_t* Wsz);

/*
 * lora_apply_q4 / lora_base_apply_q4 -- lora_apply / lora_base_apply with the
 * packed INT4 base weight (Wq, Wsz: caller-owned device buffers in the layout
 * above, d_out x d_in of module `module`).  At T <= 64 the decode kernel
 * dequantizes the weight in registers (a quarter of the bf16 weight's bytes);
 * at larger T the call first dequantizes it into W_scratch (caller-owned
 * device buffer of d_out x d_in bf16, required then, else may be NULL) and
 * runs the bf16 GEMM on it.  Other arguments, errors and guarantees as
 * lora_apply / lora_base_apply (id -1 rows equal lora_base_apply_q4's bit for
 * bit).  INVALID_ARG if d_in % 128 != 0.
 */
lora_status_t lora_apply_q4(lora_pool_t pool, int32_t module, const lora_bf16_t* X, const int32_t* ids,
                            int32_t T, const uint32_t* Wq, const uint32_t* Wsz, lora_bf16_t* W_scratch,
                            lora_bf16_t* out, lora_plan_t plan, hipStream_t stream);
lora_status_t lora_base_apply_q4(lora_pool_t pool, int32_t module, const lora_bf16_t* X, int32_t T,
                                 const uint32_t* Wq, const uint32_t* Wsz, lora_bf16_t* W_scratch,
                                 lora_bf16_t* out, hipStream_t stream);

/*
 * lora_apply_group_q4 / lora_base_apply_group_q4 -- lora_apply_group /
 * lora_base_apply_group with INT4 base weights ([vLLM-ch7] performance
 * notes; [LoRA-Land] section "2. multi-LoRA batch scheduling" for the
 * grouping): Wq and Wsz are host arrays [n] of device pointers, Wq[i] and
 * Wsz[i] the packed weight of linear modules[i] (layout above).  At T <= 64
 * the n linears run as one launch pair that stages X once; at larger T
 * each linear is dequantized into W_scratch in turn (caller-owned, at least
 * the largest d_out x d_in of the group in bf16; required then, else may be
 * NULL) before its GEMM.  Each out[i] equals lora_apply_q4
 * (lora_base_apply_q4) on that linear alone, bit for bit.  Errors as
 * lora_apply_group, plus INVALID_ARG if d_in % 128 != 0.
 */
lora_status_t lora_apply_group_q4(lora_pool_t pool, int32_t n, const int32_t* modules, const lora_bf16_t* X,
                                  const int32_t* ids, int32_t T, const uint32_t* const* Wq,
                                  const uint32_t* const* Wsz, lora_bf16_t* W_scratch, lora_bf16_t* const* out,
                                  lora_plan_t plan, hipStream_t stream);
lora_status_t lora_base_apply_group_q4(lora_pool_t pool, int32_t n, const int32_t* modules,
                                       const lora_bf16_t* X, int32_t T, const uint32_t* const* Wq,
                                       const uint32_t* const* Wsz, lora_bf16_t* W_scratch,
                                       lora_bf16_t* const* out, hipStream_t stream);

/*
 * lora_status -- synchronise `stream`, return the pool's sticky device
 * status (OK, NOT_LOADED or ID_RANGE; ID_RANGE wins if both occurred) and
 * clear it.
 */
lora_status_t lora_status(lora_pool_t pool, hipStream_t stream);

/*
 * lora_debug_read_plan -- copy a plan's tables to host memory (testing aid;
 * synchronises `stream`).  plan NULL reads the pool's internal plan (the one
 * the last lora_apply without a plan built).  Host buffers: perm[T], inv[T],
 * seg_id[S], seg_off[S+1] with T <= max_tokens and S <= T + 1; *T_out and
 * *S_out receive the sizes.  Any table pointer may be NULL to skip it.
 */
lora_status_t lora_debug_read_plan(lora_pool_t pool, lora_plan_t plan, int32_t* perm,
                                   int32_t* inv, int32_t* seg_id, int32_t* seg_off,
                                   int32_t* T_out, int32_t* S_out, hipStream_t stream);

/*
 * Host <-> device paging of the pool.  [vLLM-ch7] "how vLLM implements
 * multi-LoRA" (item 1: adapters loaded on demand and swapped in and out of
 * one device pool) and "starting a multi-LoRA service" (--max-loras on the
 * GPU, --max-cpu-loras in a CPU cache swapped in on demand); [icman] 2.2 (a
 * missing adapter is read into device memory, the least recently used
 * inactive adapter is swapped out when memory runs short, a preload list
 * keeps the hottest few resident) and 4.2 (cold loads are the latency cliff).
 *
 * lora_host_cache_create -- give the pool a host cache of up to
 * max_cpu_adapters adapters (1..max_ids) in pinned host memory, kept in the
 * device page layout, plus a copy stream of the pool's own.  Once per pool;
 * INVALID_ARG on a second call, OOM if the pinned allocation fails.
 * Memory: max_cpu_adapters x (the pool's per-slot page bytes) of host memory.
 */
lora_status_t lora_host_cache_create(lora_pool_t pool, int32_t max_cpu_adapters);

/*
 * lora_host_register -- copy an adapter into the host cache (not to the
 * device).  Arguments as lora_load_adapter (NULL pairs: untargeted modules);
 * A[m], B[m] may be host or device memory and may be freed when the call
 * returns.  ID_RANGE, RANK, EXISTS (id
 * already host-cached or loaded directly), POOL_FULL (host cache full; the
 * caller unregisters, the library never forgets an adapter on its own),
 * INVALID_ARG without a host cache.  Blocking; no stream work.
 */
lora_status_t lora_host_register(lora_pool_t pool, int32_t id, int32_t rank, float alpha,
                                 const lora_bf16_t* const* A, const lora_bf16_t* const* B);

/*
 * lora_host_unregister -- forget a host-cached adapter, dropping its device
 * copy too.  Synchronises `stream` and the copy stream.  NOT_LOADED if the id
 * is not host-cached.
 */
lora_status_t lora_host_unregister(lora_pool_t pool, int32_t id, hipStream_t stream);

/*
 * lora_prefetch -- make the adapters of the next batch addressable.
 *
 *   ids  HOST array [n] of the batch's ids (repeats and -1 allowed)
 *
 * Every host-cached id named becomes addressable; host-cached ids named by
 * the previous prefetch and not by this one stop being addressable (strict
 * mode then rejects them in lora_apply) but keep their device copy as a
 * cache.  Adapters loaded directly with lora_load_adapter are always
 * addressable and never evicted.  A named id without a device copy takes a
 * free slot, else the slot of the cached, unpinned, unnamed adapter with the
 * smallest (number of the last prefetch that named it, id): least recently
 * used.  The page copies run asynchronously on the pool's copy stream and
 * overlap the work already on `stream`: a copy into an evicted adapter's slot
 * waits only for the work enqueued before the first prefetch that stopped
 * naming it; `stream` then waits for the copies and updates the routing table
 * in order.  So a batch's applies must be enqueued after the prefetch that
 * names its adapters and before the next prefetch call.
 * Errors, with no side effects: ID_RANGE (an id outside [-1, max_ids); wins),
 * NOT_LOADED (an id neither host-cached nor loaded), POOL_FULL (more misses
 * than free plus evictable slots), INVALID_ARG (no host cache, ids NULL with
 * n > 0, n < 0).  The host returns before the copies finish; the host cache
 * is not modified while they run (unregister waits for them).  The call
 * changes host-side state, so it must not be captured into a hipGraph
 * (capture the applies; call lora_prefetch before each replay instead).
 */
lora_status_t lora_prefetch(lora_pool_t pool, const int32_t* ids, int32_t n, hipStream_t stream);

/*
 * lora_pin_adapter -- the preload list.  pin != 0 pages a host-cached adapter
 * in now (free slot, else the least recently used adapter that is not
 * addressable; POOL_FULL if there is none), makes it addressable and exempts
 * it from eviction; synchronises `stream`.  pin == 0 returns it to the LRU
 * with the recency of the latest prefetch; it stays addressable only if the
 * last prefetch named it.  NOT_LOADED if not host-cached.
 */
lora_status_t lora_pin_adapter(lora_pool_t pool, int32_t id, int32_t pin, hipStream_t stream);

/*
 * lora_paging_query -- where an id is (host state, no device work):
 *   *where  0 unknown, 1 host cache only, 2 device copy but not addressable,
 *           3 addressable (host-cached and named or pinned, or loaded directly)
 *   *pinned 1 if on the preload list
 * Either pointer may be NULL.  ID_RANGE if the id is out of range.
 */
lora_status_t lora_paging_query(lora_pool_t pool, int32_t id, int32_t* where, int32_t* pinned);

/*
 * lora_paging_stats -- counters of the paging path (host state, no device
 * work): prefetch calls so far, adapter slots copied host -> device so far
 * (by prefetch and pin), and the bytes of one such copy (every module's pages
 * of one slot, padded to max_rank).  Any pointer may be NULL.
 */
lora_status_t lora_paging_stats(lora_pool_t pool, int64_t* prefetches, int64_t* pages_loaded,
                                int64_t* bytes_per_page);

#ifdef __cplusplus
}
#endif
#endif /* HRG_LORA_H */
