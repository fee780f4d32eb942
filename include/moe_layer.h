/*
 * moe_layer.h - C ABI of the MI355X (gfx950) MoE-layer library.
 *
 * One sparse Mixture-of-Experts layer: a router picks the top-k of E routed
 * experts per token, each expert is a SwiGLU MLP whose weights are affine
 * int4/int8 group-quantized and stored as one fixed-stride blob in a device
 * slot pool, and a sigmoid-gated shared expert is added to the weighted sum.
 *
 * Sources (the pages describe the Swiftlet expert-streaming runtime):
 *   - Swiftlet README translation, section "How it works": every layer routes
 *     each token to 10 of 512 (80B) or 8 of 256 (35B) experts; the router and
 *     shared expert are resident; routed experts are fixed-stride blobs, one
 *     fetch per expert; hot experts live in a bounded slot pool.
 *   - same page, section "Relation to TurboFieldfare": MLX affine int4/int8
 *     group quantization computed on the GPU, byte-addressed kernels with
 *     64-bit offsets for multi-GB shards, explicit hazard management.
 *   - same page, section "Correctness": placement (cache or disk) never changes
 *     the answer.
 *
 * The pages leave the formulas open; this library computes (readings):
 *   w[r,c] = s[r, c/64] * q[r,c] + b[r, c/64]     q unsigned, groups of 64 along
 *                                                 the input axis, int4 low nibble
 *                                                 first in little-endian words
 *   l = R x;  S = first k experts by (-l, id)     ties go to the lower id
 *   p_i = exp(l_{S_i} - m) / sum_{j in S} exp(l_j - m),  m = max_{j in S} l_j
 *   E(x) = Wd (silu(Wg x) * (Wu x))
 *   y = sum_{i<k} p_i E_{S_i}(x) + sigmoid(g . x) E_shared(x)
 *
 * Blob format (own format; the pages give none).  Offsets inside one blob of
 * intermediate size I (Q = I*H*bits/8 bytes, S = I*H/64 * sizeof(scale)):
 *   [0,Q) gate codes [I,H]   [Q,2Q) up codes [I,H]   [2Q,3Q) down codes [H,I]
 *   then gate/up/down scales (S bytes each), then gate/up/down biases (S each).
 * Matrices are row-major [out, in].  The stride is the blob size rounded up to
 * 4096 bytes.  Expert e starts at pool_base + slot_table[e] (a 64-bit byte
 * offset).  The shared-expert buffer holds one blob with the shared
 * intermediate size and, at byte offset shared_stride, the gate vector [H] in
 * the activation dtype.
 *
 * Conventions for every entry point:
 *   - All data pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or retains them.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *     work on it and return; nothing is synchronous unless stated.
 *   - Return 0 (MOE_OK) or a negative MOE_E* code; moe_last_error() gives the
 *     text (thread-local).  Arguments are checked on the host before any
 *     device call; a rejected call enqueues nothing.
 *   - Work is deterministic: the same inputs give bitwise identical outputs on
 *     every call, and the output does not depend on where in the pool a blob
 *     sits (no floating-point atomics).
 */
#ifndef MOE_LAYER_H
#define MOE_LAYER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define MOE_OK 0
#define MOE_EINVAL (-1)   /* bad descriptor, size, pointer or alignment        */
#define MOE_ENODEV (-2)   /* no usable gfx950 device                            */
#define MOE_EHIP (-3)     /* a HIP call or kernel launch failed                 */
#define MOE_ENOMEM (-4)   /* workspace smaller than moe_workspace_bytes()       */
#define MOE_ERANGE (-5)   /* a kernel saw a slot offset outside the pool, or an
                             expert id outside [0, E); that pair was skipped    */
#define MOE_ENOSPC (-6)   /* residency manager: more experts than slots         */
#define MOE_ETIMEOUT (-7) /* the fused decode kernel's bounded wait expired: some
                             of its blocks never became resident (the GPU was
                             shared with other work); the output is invalid    */
#define MOE_EIO (-8)      /* expert store: a file could not be opened, read or
                             written, or it is not a store of the stated shape */
#define MOE_EOVERFLOW (-9) /* the MFMA prefill path rounded a value outside the
                             float16 range (an input, an h value or a partial
                             down row; see its precision notes): the output
                             holds inf or NaN                                   */

/* Storage dtypes. */
#define MOE_F32 0
#define MOE_BF16 1

/*
 * Layer descriptor (plain value, caller-owned).
 *   hidden        H; a power of two, 64 .. 2048
 *   n_experts     E; 1 .. 1024
 *   top_k         k; 1 .. min(E, 64)
 *   inter         I, routed-expert intermediate size; power of two, 64 .. 2048
 *   shared_inter  shared-expert intermediate size; power of two, 64 .. 2048
 *   bits          4 or 8
 *   group_size    must be 64
 *   act_dtype     dtype of x, the router matrix and the shared gate vector
 *   sb_dtype      dtype of the quantization scales and biases
 *   out_dtype     dtype of out
 *   blob_stride   bytes between consecutive slots; >= moe_blob_bytes(d, 0)
 *                 and a multiple of 256
 *   shared_stride byte offset of the gate vector in the shared buffer;
 *                 >= moe_blob_bytes(d, 1) and a multiple of 256
 *   pool_bytes    size of the pool in bytes; every slot offset used must
 *                 satisfy 0 <= off, off % 256 == 0, off + blob bytes <= pool_bytes
 */
typedef struct moe_desc {
  int32_t hidden;
  int32_t n_experts;
  int32_t top_k;
  int32_t inter;
  int32_t shared_inter;
  int32_t bits;
  int32_t group_size;
  int32_t act_dtype;
  int32_t sb_dtype;
  int32_t out_dtype;
  int64_t blob_stride;
  int64_t shared_stride;
  int64_t pool_bytes;
} moe_desc;

/* Unpadded size in bytes of one routed (shared == 0) or shared (shared != 0)
 * blob for this descriptor; -1 if the descriptor is invalid.  Pure function. */
int64_t moe_blob_bytes(const moe_desc* d, int32_t shared);

/* Workspace bytes needed for calls with up to T_max tokens; 0 if the
 * descriptor is invalid.  Pure function. */
size_t moe_workspace_bytes(const moe_desc* d, int32_t T_max);

/*
 * Prepare a workspace for first use: clears all of it with a kernel on
 * `stream` (no memset, so this may run inside a captured graph).  Call once
 * after allocating it; every later call leaves it ready for the next call.
 * The fused path tags its exchange words with a 32-bit per-workspace call
 * counter: re-initialise a workspace at least every 2^31 calls if calls with
 * different T share it.
 */
int moe_workspace_init(void* workspace, size_t ws_bytes, void* stream);

/*
 * Forward pass of one MoE layer.
 *   d           layer descriptor
 *   T           number of tokens, >= 0 (T == 0 enqueues nothing)
 *   x           [T, H] activations, act_dtype, 16-byte aligned
 *   router_w    [E, H] router matrix, act_dtype, row-major, 16-byte aligned
 *   slot_table  [E] int64 byte offsets of each expert's blob in the pool
 *   pool_base   base of the slot pool, 256-byte aligned
 *   shared_w    shared-expert blob + gate vector (see above), 256-byte aligned
 *   out         [T, H] output, out_dtype
 *   workspace   device scratch of ws_bytes >= moe_workspace_bytes(d, T),
 *               256-byte aligned, prepared once by moe_workspace_init; must
 *               not be used by two calls that may run concurrently
 *   topk_ids    optional [T, k] int32 output: chosen experts, descending logit
 *   topk_w      optional [T, k] float32 output: renormalised weights
 * Errors: MOE_EINVAL, MOE_ENOMEM, MOE_EHIP as above.  Out-of-range slot
 * offsets are detected on the device (see moe_status_check).
 */
int moe_layer_forward(const moe_desc* d, int32_t T, const void* x, const void* router_w,
                      const int64_t* slot_table, const void* pool_base, const void* shared_w,
                      void* out, void* workspace, size_t ws_bytes, int32_t* topk_ids,
                      float* topk_w, void* stream);

/*
 * Which kernels run.  moe_layer_forward picks by T and the descriptor:
 *   - T = 1 on the 80B/35B layer shape (hidden 2048, intermediate sizes 512,
 *     int4 codes, bf16 activations and scales, E a multiple of 256 up to
 *     512, top_k <= 10): ONE launch, the stack kernel of moe_stack_forward
 *     with one layer (router, top-k, gate/up, down and the ordered combine;
 *     blocks exchange the logits and h as tagged words).
 *   - other T <= 8 with bf16 activations and scales (or float32 activations,
 *     scales and output): the fused decode path.  T = 1 with int4 codes is
 *     one launch; otherwise two (the first computes the router logits, the
 *     shared expert's gate/up rows and the gate, exchanges the logits between
 *     blocks as tagged words, takes top-k and dispatch redundantly in every
 *     block and computes the routed gate/up rows; the second the down rows
 *     and the combine).
 *   - T >= 16 with bf16 activations and H, I, SI multiples of 256: the MFMA
 *     prefill path.
 *   - otherwise: the staged path (six launches).
 * The single-launch kernels need every block of their grid resident, i.e.
 * the GPU's compute units not taken by other work; a bounded wait that
 * expires raises MOE_ETIMEOUT in moe_status_check.
 * moe_layer_forward_staged always runs the staged path.  For T <= 8 the
 * staged and the decode paths give bitwise identical results.
 */
int moe_layer_forward_staged(const moe_desc* d, int32_t T, const void* x, const void* router_w,
                             const int64_t* slot_table, const void* pool_base, const void* shared_w,
                             void* out, void* workspace, size_t ws_bytes, int32_t* topk_ids,
                             float* topk_w, void* stream);

/*
 * The same layer on scalar kernels: one GPU thread per output value (a
 * router logit, a token's routing and gate, one element of h, one element of
 * a down row, one output element), with no cross-lane operations.  The pages
 * check their fast GPU kernels against scalar ones that give identical output
 * (Swiftlet README translation, "Correctness"; linlog.top article,
 * "Correctness guarantees").  These kernels state the order in which the fast
 * kernels associate every sum and follow it, so for any T their results
 * equal moe_layer_forward_staged bit for bit (and, for T <= 8, the fast decode
 * paths of moe_layer_forward).  Slow by design: a check, not a production
 * path.  Same arguments, workspace and errors as moe_layer_forward.
 */
int moe_layer_forward_scalar(const moe_desc* d, int32_t T, const void* x, const void* router_w,
                             const int64_t* slot_table, const void* pool_base, const void* shared_w, void* out,
                             void* workspace, size_t ws_bytes, int32_t* topk_ids, float* topk_w, void* stream);

/*
 * First half of moe_layer_forward: router logits, top-k and renormalised
 * weights into topk_ids [T, k] / topk_w [T, k] (both required).
 */
int moe_router_topk(const moe_desc* d, int32_t T, const void* x, const void* router_w,
                    int32_t* topk_ids, float* topk_w, void* workspace, size_t ws_bytes,
                    void* stream);

/*
 * Second half: experts and combine from given routing (topk_ids / topk_w, as
 * written by moe_router_topk).  moe_router_topk followed by this call gives
 * the same bits as moe_layer_forward.  An id outside [0, E) contributes
 * nothing and raises MOE_ERANGE in moe_status_check.
 */
int moe_experts_forward(const moe_desc* d, int32_t T, const void* x, const int32_t* topk_ids,
                        const float* topk_w, const int64_t* slot_table, const void* pool_base,
                        const void* shared_w, void* out, void* workspace, size_t ws_bytes,
                        void* stream);

/*
 * Timing hook for profilers and benchmarks: the next moe_layer_forward,
 * moe_layer_forward_staged, moe_router_topk or moe_experts_forward call made
 * on this host thread launches its j-th kernel (j = 0, 1, ...) with events[2j]
 * and events[2j+1] attached (hipExtLaunchKernel), so the runtime stamps them
 * with that dispatch's own start and end: hipEventElapsedTime of the pair is
 * the kernel's execution time.  Kernels beyond capacity / 2 launch untimed.
 * The number of events used (2 per timed kernel) is stored in *n_recorded
 * (host memory, written before that call returns).  The setting applies to
 * that one call only and is cleared by it (also when it fails); events == NULL
 * clears it now.  `events` holds hipEvent_t handles created by the caller with
 * timing enabled; they stay owned by the caller.  Returns MOE_EINVAL if
 * capacity < 1 or n_recorded is NULL while events is not.
 */
int moe_set_launch_events(void* const* events, int32_t capacity, int32_t* n_recorded);

/*
 * Synchronises `stream`, then reports and clears the device-side error flags
 * of `workspace`: MOE_ETIMEOUT if a fused-kernel wait expired, else MOE_ERANGE
 * if any kernel since the last check skipped a pair for a bad slot offset or
 * expert id, else MOE_EOVERFLOW if the prefill path met a value outside the
 * float16 range, else MOE_OK.  Blocking.
 */
int moe_status_check(void* workspace, void* stream);

/* The step after the layer in a stack of layers: x_next = x + y for the
 * layer input x [T, H] (act_dtype: MOE_BF16 or MOE_F32) and the layer output
 * y [T, H] (fp32), the sum taken in fp32 and, for bf16, rounded to nearest
 * even into bf16.  The pages run token after token through the whole layer
 * stack on the device, and report the decode loop as bound by dispatch rather
 * than by expert reads (Swiftlet README translation, "Status"; linlog.top
 * article, section "Capability limits"); chaining each layer's output into
 * the next layer's input is the plain reading of that loop.  x_next may be x
 * (in place).  Device pointers, caller-owned; asynchronous on `stream`.
 * MOE_EINVAL on bad sizes, dtype or NULL pointers. */
int moe_residual_add(int32_t T, int32_t H, int32_t act_dtype, const void* x, const float* y, void* x_next,
                     void* stream);

/* moe_layer_forward, then the stack step into x_next [T, H] (the activation
 * dtype): the same bits as moe_layer_forward followed by moe_residual_add on
 * its output, for the same passages.  The fused decode path writes x_next in
 * its ordered combine, without a launch of its own; the other paths launch
 * the step after the layer.  Needs out_dtype MOE_F32; x_next 16-byte aligned
 * and not x.  MOE_EINVAL otherwise. */
int moe_layer_forward_chain(const moe_desc* desc, int32_t T, const void* x, const void* router_w,
                            const int64_t* slot_table, const void* pool_base, const void* shared_w, void* out,
                            void* x_next, void* workspace, size_t ws_bytes, int32_t* topk_ids, float* topk_w,
                            void* stream);

/*
 * A stack of n_layers MoE layers with the same descriptor, run in order: the
 * pages run every token through the whole layer stack on the GPU and report
 * the decode loop as bound by dispatch rather than by expert reads (Swiftlet
 * README translation, "How it works" and "Status"; linlog.top article,
 * "Capability limits").  Layer l (0 <= l < n_layers) reads
 *   input      x + l * x_stride, or, when x_chain is not NULL and l > 0,
 *              x_chain + (l - 1) * chain_stride
 *   router     router_w + l * router_stride
 *   slot table (const uint8_t*) slot_table + l * slot_stride  (int64 [E])
 *   shared     shared_w + l * shared_stride
 * all in one pool (pool_base, desc->pool_bytes), and writes
 *   out        out + l * out_stride
 *   x_chain    x_chain + l * chain_stride = its input + its output (the stack
 *              step of moe_residual_add), when x_chain is not NULL
 *   topk_ids / topk_w  (optional) [n_layers][T][k].
 * Strides are in bytes; each must hold one layer's data and keep the
 * alignment that moe_layer_forward asks of its pointer (checked when
 * n_layers > 1).  x_chain needs out_dtype MOE_F32 and may not overlap x or
 * out.  The result equals n_layers calls of moe_layer_forward (or, with
 * x_chain, moe_layer_forward_chain) bit for bit.  On the 80B/35B layer
 * shape (hidden 2048, intermediate sizes 512, int4 codes, bf16 activations
 * and scales, E a multiple of 256 up to 512, top_k <= 10) the whole stack is
 * ONE launch for T = 1 (chained or not) and for 2 <= T <= 8 without x_chain;
 * that launch keeps every block of the grid resident (the GPU's compute
 * units must not be taken by other work; a bounded wait that expires raises
 * MOE_ETIMEOUT in moe_status_check).  Otherwise the layers run as separate
 * calls.  The timing hook (moe_set_launch_events) counts the whole stack as
 * one call.  MOE_EINVAL, MOE_ENOMEM, MOE_EHIP as for moe_layer_forward.
 */
int moe_stack_forward(const moe_desc* d, int32_t n_layers, int32_t T, const void* x, int64_t x_stride,
                      const void* router_w, int64_t router_stride, const int64_t* slot_table, int64_t slot_stride,
                      const void* pool_base, const void* shared_w, int64_t shared_stride, void* out,
                      int64_t out_stride, void* x_chain, int64_t chain_stride, int32_t* topk_ids, float* topk_w,
                      void* workspace, size_t ws_bytes, void* stream);

/*
 * moe_layer_forward without a caller workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The workspace is a fixed array of
 * 16 MiB inside the library, one per GPU (each GPU the library runs on
 * holds it until the process ends); it is cleared by a fill kernel on
 * `stream` at the first call on each device, and every call leaves it ready
 * for the next.  Calls that would need more than 16 MiB of workspace
 * (moe_workspace_bytes(d, T) > 16 MiB, e.g. the 80B layer shape beyond
 * T = 96) return MOE_ENOMEM.  The call makes no device allocation
 * (no hipMalloc / hipFree), and returns after enqueueing like
 * moe_layer_forward, with the same results bit for bit.
 *   status  optional (NULL or 4-byte aligned device pointer): after the
 *           layer, receives this GPU's device error flags (bit 0: a pair
 *           skipped for a bad slot offset or id, MOE_ERANGE; bit 1: a
 *           bounded wait expired, MOE_ETIMEOUT; bit 2: a value outside the
 *           float16 range in the prefill path, MOE_EOVERFLOW), which are
 *           then cleared.
 *           With NULL they accumulate unreported.
 * All calls on one GPU share its array: calls that may overlap on one GPU
 * (several streams, several host threads) race and must not be made.
 */
int moe_layer_forward_noalloc(const moe_desc* d, int32_t T, const void* x, const void* router_w,
                              const int64_t* slot_table, const void* pool_base, const void* shared_w, void* out,
                              int32_t* topk_ids, float* topk_w, uint32_t* status, void* stream);

/* Text of the last error on this thread ("" if none). */
const char* moe_last_error(void);

/* ------------------------------------------------------------------------
 * Partial residency (expert streaming from pinned host memory).
 *
 * The pages keep only part of the experts in fast memory and stream the rest
 * from a larger store on demand, with a bounded cache pool that favours
 * frequently and recently used experts, and order GPU work with explicit
 * hazard management (linlog.top article, core design 3, the expert cache
 * pool; Swiftlet README translation, "How it works" and "Relation to
 * TurboFieldfare"; kerneldigest.dev article, inference flow, the cache step).  Here: a pool of n_slots fixed-stride HBM
 * slots (pool_base, caller-owned, n_slots * stride bytes, 256-aligned) caching
 * blobs of a pinned host store (host_pinned, caller-owned, laid out
 * [n_layers][n_experts][stride], allocated with hipHostMalloc).
 *
 * Use per layer call:
 *   1. moe_router_topk(...) then copy topk_ids to the host (after a sync);
 *   2. moe_cache_acquire(cache, layer, ids_host, T*k, slot_table_host,
 *      copy_stream, ready): fills slot_table_host[e] (byte offsets into
 *      pool_base) for every expert the ids name, enqueues the host->HBM
 *      copies of the misses on copy_stream and records `ready` after them;
 *   3. on the compute stream: hipStreamWaitEvent(ready), copy the slot table
 *      to the device, moe_experts_forward(...), record compute_done;
 *   4. moe_cache_release(cache, layer, compute_done).
 * The output equals that of a fully resident pool bit for bit (placement
 * never changes results).
 *
 * Policy: a miss takes an empty slot (lowest first), else evicts the resident
 * blob with the fewest uses, ties to the oldest last use, then the lower
 * (layer, id).  Uses count once per acquire that needs the blob, over the
 * cache's whole life (an evicted blob keeps its count; moe_cache_set_policy
 * can make counts restart at eviction instead).  Blobs the current call
 * needs are never evicted by it,
 * nor are blobs of acquires not yet released.
 * Ordering (no host waits): a victim slot is overwritten only after the
 * compute_done event of the last released call that read it (if that event
 * was recorded again since, the wait covers the later work too, which is
 * still correct); copies of one cache run in issue order even when
 * copy_stream changes between calls, so `ready` also covers hits on blobs
 * whose copies are still in flight.
 *
 * Planning mode: pool_base = host_pinned = NULL runs the policy alone (no
 * device calls; copy_stream and the events are ignored and may be NULL).
 * Not thread-safe: one host thread per cache.
 */
typedef struct moe_cache moe_cache;

/* NULL on bad arguments (n_slots < 1, stride not a positive multiple of 256,
 * pool_base unaligned, exactly one of pool_base / host_pinned NULL). */
moe_cache* moe_cache_create(int32_t n_slots, int64_t stride, void* pool_base, const void* host_pinned,
                            int32_t n_layers, int32_t n_experts);

/* ids_host: n expert ids (duplicates allowed).  Returns MOE_OK, MOE_EINVAL
 * (bad argument or id outside [0, n_experts)), MOE_ENOSPC (more distinct
 * experts than slots, or too few slots free of unreleased acquires) or
 * MOE_EHIP (a copy could not be issued).  After MOE_EHIP (or MOE_EIO from a
 * store read) no expert this call missed is left resident, the hits it held
 * are released, and copies issued before the failure still order later
 * ones; the cache stays usable if the device does. */
int moe_cache_acquire(moe_cache* cache, int32_t layer, const int32_t* ids_host, int32_t n,
                      int64_t* slot_table_host, void* copy_stream, void* ready);

/* Ends the oldest unreleased acquire of `layer`: its slots become evictable,
 * each after compute_done (a hipEvent_t the caller keeps alive). */
int moe_cache_release(moe_cache* cache, int32_t layer, void* compute_done);

void moe_cache_stats(const moe_cache* cache, int64_t* hits, int64_t* misses, int64_t* evictions);

/* Policy flags (moe_cache_set_policy).  MOE_CACHE_KEEP_COUNTS (set when a
 * cache is created): a blob's use count survives its eviction, so a
 * frequently used expert that a burst of others pushed out comes back with
 * its count and is not the next victim.  With the flag clear, counts restart
 * at eviction, and a cycle of blobs longer than the pool degenerates to
 * least-recently-used order.  Either way the policy changes only which blobs
 * stay resident, never the outputs. */
#define MOE_CACHE_KEEP_COUNTS 1

/* Sets the policy flags of a cache (0 or MOE_CACHE_KEEP_COUNTS) for its later
 * acquires.  MOE_EINVAL on a NULL cache or unknown flags. */
int moe_cache_set_policy(moe_cache* cache, int32_t flags);

/* Failure injection, for tests of the error path: the copy that is the
 * nth_copy-th (0 = the next) to be issued from now on fails as a failed
 * hipMemcpyAsync would (MOE_EHIP from moe_cache_acquire); -1 disarms.  In
 * planning mode the copies that would be issued are counted.  After a failed
 * acquire no expert that call missed is left resident, the hits it held are
 * released, and the cache stays usable. */
int moe_cache_inject_fault(moe_cache* cache, int32_t nth_copy);

/* Slot index holding (layer, id), or -1. */
int moe_cache_slot_of(const moe_cache* cache, int32_t layer, int32_t id);

void moe_cache_destroy(moe_cache* cache);

/* ------------------------------------------------------------------------
 * Expert store: the slow tier as one container file on disk.
 *
 * The pages repack the routed experts into fixed-stride blobs in one
 * container, so that fetching an expert is one positioned read at an offset
 * computed from its (layer, id), without mapping the file into memory
 * (linlog.top article, core design 2, fixed-stride reads; Swiftlet README
 * translation, "How it works"; kerneldigest.dev article, inference flow, the
 * cache-miss step).  File layout (little-endian):
 *   bytes [0, 4096): header = 8-byte magic "MOEBLOB1", int32 n_layers,
 *     int32 n_experts, int64 stride, int64 blob_bytes, zeros to 4096;
 *   blob (layer, id) at 4096 + (layer * n_experts + id) * stride, stride
 *     bytes, laid out as a pool blob (moe_blob_bytes() <= stride).
 * stride is a positive multiple of 4096, so every blob is page-aligned in the
 * file (positioned reads with O_DIRECT need that).  Errors of the moe_store_*
 * calls are reported by moe_cache_last_error().
 */
typedef struct moe_store moe_store;

#define MOE_STORE_DIRECT 1   /* moe_store_open: read with O_DIRECT, past the
                                page cache (not every file system allows it) */

/* Creates (or truncates) the file, writes the header and sizes the file;
 * the blobs read as zeros until written.  NULL on error. */
moe_store* moe_store_create(const char* path, int32_t n_layers, int32_t n_experts, int64_t stride,
                            int64_t blob_bytes);

/* Opens a store read-only; flags = 0 or MOE_STORE_DIRECT.  NULL on error
 * (bad magic or shape, file shorter than its header says: MOE_EIO). */
moe_store* moe_store_open(const char* path, int32_t flags);

int moe_store_info(const moe_store* store, int32_t* n_layers, int32_t* n_experts, int64_t* stride,
                   int64_t* blob_bytes);

/* One positioned read of blob (layer, id): stride bytes into dst_host.
 * A MOE_STORE_DIRECT store reads into its own page-aligned buffer and copies
 * out (direct transfers into HIP pinned memory fail).  Blocking.  MOE_EINVAL
 * or MOE_EIO.  One thread per store. */
int moe_store_read(moe_store* store, int32_t layer, int32_t id, void* dst_host);

/* Writes stride bytes from src_host as blob (layer, id) of a store made by
 * moe_store_create.  Blocking. */
int moe_store_write(moe_store* store, int32_t layer, int32_t id, const void* src_host);

/* Closes the file.  A cache made on the store must be destroyed first. */
void moe_store_close(moe_store* store);

/* A cache whose misses come from a store instead of a pinned host copy of
 * every blob: the geometry (stride, n_layers, n_experts) is the store's.
 * Each miss in moe_cache_acquire is one moe_store_read into the next of
 * n_staging (1..64) pinned staging buffers (staging_pinned, caller-owned,
 * n_staging * stride bytes from hipHostMalloc), then the same
 * hipMemcpyAsync into the slot on the
 * copy stream.  A staging buffer is read into again only after the copy out
 * of it has finished: acquire then waits on the host (hipEventSynchronize),
 * which may include compute that the copy stream was told to wait for.
 * Keep the staging memory until the copy stream has finished the last
 * acquire's copies.  A failed read (MOE_EIO from acquire) is rolled back like
 * a failed copy.  NULL on bad arguments. */
moe_cache* moe_cache_create_from_store(int32_t n_slots, void* pool_base, moe_store* store, void* staging_pinned,
                                       int32_t n_staging);

/* Text of the last moe_cache_* or moe_store_* error on this thread. */
const char* moe_cache_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_LAYER_H */
