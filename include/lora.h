/*
 * lora.h -- C ABI of the MI355X (gfx950) multi-adapter LoRA library.
 *
 * One batch, many adapters.  For every row i of a batch whose base output
 * y_i = W x_i is already computed, the library adds the row's adapter delta
 *
 *      y_i += (alpha_s / r_s) * B_s (A_s x_i),     s = ids[i],
 *
 * and leaves rows with no adapter (id -1) untouched.  The delta is computed in
 * two steps, add_shrink (v = A x, rank r) then add_expand (y += scale * B v),
 * with the rows grouped by adapter so that one kernel serves the whole
 * heterogeneous batch.  Sources: page "Multi-LoRA Serving: one base, many
 * adapters", section 2 (per-row equation; flowchart: group rows by adapter id,
 * shared base GEMM, add_shrink, add_expand, per-row merge) and section 3.1
 * (LoRA math: B is d x r, A is r x k, Delta W = B A never formed); page "LoRA
 * serving: multi-adapter dynamic loading", section 2 (all adapters' A and B
 * stacked into one tensor, one integer id per request as the indirection, one
 * batched kernel for the whole batch).
 *
 * Conventions shared by every call:
 *   - Every call returns a lora_status; nothing aborts the process and no C++
 *     exception crosses this boundary.  Host-checkable errors are returned
 *     before anything is enqueued on the stream.
 *   - "stream" is a hipStream_t passed as void* (NULL = the default stream).
 *     GPU work is asynchronous and stream-ordered: load -> apply -> evict on
 *     one stream is safe without host synchronisation.
 *   - Tensor pointers are device pointers unless an argument says otherwise.
 *     Rows of x and y are dense along their width; row i starts at element
 *     i * ldx (x) or i * ldy (y).
 *   - Element types: LORA_F32 = IEEE float, LORA_BF16 = bfloat16 (the upper
 *     half of an IEEE float).  x, y and the adapter weights of one stack share
 *     the stack's dtype.  Arithmetic is fp32; each output element is rounded
 *     once (round-to-nearest-even) from fp32(y_in) + scale * fp32(B v).
 *   - Alignment: k, every slice width, ldx and ldy must be multiples of 8, and
 *     x, y and weight sources 16-byte aligned.
 *   - A stack or segments object must not be used from two host threads at
 *     once, and calls that share one on different streams must be ordered by
 *     the caller (they share device scratch).
 */
#ifndef RANK_ADAPTER_GEMM_LORA_AMD_LORA_H
#define RANK_ADAPTER_GEMM_LORA_AMD_LORA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct lora_stack lora_stack;       /* owns the adapter pool in HBM   */
typedef struct lora_segments lora_segments; /* owns one batch's grouping      */

typedef enum lora_dtype { LORA_F32 = 0, LORA_BF16 = 1 } lora_dtype;

typedef enum lora_status {
    LORA_OK = 0,
    LORA_E_ARG = 1,       /* null pointer, bad size, misalignment, mismatch  */
    LORA_E_RANK = 2,      /* rank < 1 or rank > r_max                        */
    LORA_E_SLOT = 3,      /* slot index outside [0, n_slots)                 */
    LORA_E_OCCUPIED = 4,  /* load into a slot that holds an adapter          */
    LORA_E_EMPTY = 5,     /* evict of a slot that holds none                 */
    LORA_E_NOMEM = 6,     /* device allocation failed                        */
    LORA_E_HIP = 7,       /* a HIP runtime call failed                       */
    LORA_E_BAD_IDS = 8,   /* (reported by lora_get_device_status)            */
    LORA_E_UNSUPPORTED = 9, /* shape or option outside this build's limits   */
    LORA_E_CAPACITY = 10, /* more adapters than the slots or host tier hold  */
    LORA_E_NOT_FOUND = 11 /* adapter id not registered                       */
} lora_status;

/* Path of the row tiles of one segment (see lora_segments_set_dense_min). */
typedef enum lora_path { LORA_PATH_BGMV = 0, LORA_PATH_SGMV = 1 } lora_path;

/* Limits of this build. */
#define LORA_MAX_SLOTS 1024
#define LORA_MAX_RANK 128
#define LORA_MAX_SLICES 8

/* ------------------------------------------------------------------ stacks */

/*
 * Create a stack: the adapter pool of one layer projection group.
 *
 * The pool holds n_slots adapters of rank up to r_max; logically
 * A_all[n_slots][n_slices][r_max][k] and B_all[n_slots][D][r_max] with
 * D = sum(slice_d) (the slot count plays the part of the per-batch adapter cap
 * and r_max that of the maximum LoRA rank that sizes the slots: page
 * "Multi-LoRA Serving: one base, many adapters", section 3.2).  n_slices > 1
 * fuses several projections that read the same x (q/k/v, gate/up): slice q
 * writes columns [off_q, off_q + slice_d[q]) of y, each slice with its own A_q
 * and B_q, all sharing the row's adapter id and scale.  max_rows bounds
 * n_rows of every lora_apply on this stack (it sizes the stack's fp32 scratch
 * for v).  The physical layout of the pool is private; bf16 stacks whose
 * slices are whole 64-column blocks also keep a second, operand-ordered copy
 * of A (about n_slots * n_slices * round_up(r_max, 16) * k * 2 bytes more),
 * rebuilt in stream order by every load.
 *
 *   out       receives the new stack (set to NULL on failure)
 *   dtype     element type of weights, x and y
 *   n_slots   1 .. LORA_MAX_SLOTS;  r_max 1 .. LORA_MAX_RANK
 *   k         input width (multiple of 8)
 *   n_slices  1 .. LORA_MAX_SLICES; slice_d: HOST array [n_slices] of widths
 *             (each a multiple of 8)
 *   max_rows  >= 1
 *
 * The pool and slot table start empty (every slot rank 0).  Allocates device
 * memory on the current HIP device; all later calls must run with that device
 * current.  Errors: LORA_E_ARG, LORA_E_UNSUPPORTED, LORA_E_NOMEM, LORA_E_HIP.
 */
lora_status lora_stack_create(lora_stack **out, lora_dtype dtype, int n_slots, int r_max,
                              int64_t k, int n_slices, const int64_t *slice_d,
                              int64_t max_rows);

/* Free a stack (NULL is accepted).  Synchronises the device first so no
 * enqueued kernel still reads the pool. */
lora_status lora_stack_destroy(lora_stack *st);

/*
 * Load one adapter into an empty slot (page "LoRA hot-loading and adapter
 * routing", adapter-lifecycle section: validate the rank against the cap, copy
 * A and B to GPU memory, register; page "Multi-LoRA Serving", section 6: an
 * adapter above the rank cap is refused at load).
 *
 *   A      [n_slices][rank][k]  dense, true rank
 *   B      [D][rank]            dense, true rank, slices stacked along D
 *   alpha  the adapter's scaling numerator: scale = alpha / rank (true rank)
 *   src_is_host  nonzero: A and B are host pointers; the call returns after
 *                they have been consumed (it synchronises the stream).
 *                zero: device pointers; the copy is stream-ordered and the
 *                caller keeps them alive until the stream passes it.
 *
 * Errors: LORA_E_SLOT, LORA_E_RANK, LORA_E_OCCUPIED (evict first), LORA_E_ARG,
 * LORA_E_HIP.
 */
lora_status lora_load_slot(lora_stack *st, int slot, int rank, float alpha, const void *A,
                           const void *B, int src_is_host, void *stream);

/* Mark a slot empty, in stream order (page "LoRA hot-loading and adapter
 * routing", adapter-lifecycle section: unloading).  Rows that still name the
 * slot in a later lora_build_segments count as bad ids.  Errors: LORA_E_SLOT,
 * LORA_E_EMPTY. */
lora_status lora_evict_slot(lora_stack *st, int slot, void *stream);

/*
 * Host view of one slot: rank (0 = empty), alpha, and the number of adapter
 * parameters it holds, rank * (n_slices * k + D) -- the r(d + k) count of page
 * "Multi-LoRA Serving", section 3.1, summed over slices.  Any output pointer
 * may be NULL.  Errors: LORA_E_ARG, LORA_E_SLOT.
 */
lora_status lora_slot_info(const lora_stack *st, int slot, int *rank, float *alpha,
                           int64_t *live_params);

/*
 * Fold the adapter of one slot into a dense weight, or take it out again
 * (page "LoRA serving: multi-adapter dynamic loading", section 1: merging an
 * adapter into the base weight, W' = W + (alpha/r) B A, serves that one
 * adapter at the base model's cost, and subtracting the same product unmerges;
 * page "Multi-LoRA Serving", section 3.1: B is d x r, A is r x k).  For every
 * row o of slice q (rows [off_q, off_q + slice_d[q])) and column i < k:
 *
 *      W[o][i] = round(fp32(W[o][i]) + sign * scale * sum_j B[o][j] A_q[j][i]),
 *
 * scale = alpha / rank (the same fp32 value the apply path uses), the sum in
 * fp32, one rounding to the stack's dtype per element.
 *
 *   W      DEVICE [D][ldw] in the stack's dtype (row o = output feature, the
 *          layout of a linear layer's weight), updated in place; columns
 *          >= k are not touched.  16-byte aligned.
 *   ldw    >= k, multiple of 8
 *   sign   +1 merge, -1 unmerge
 *
 * Merge followed by unmerge returns W up to the two roundings.  Reads the pool
 * in stream order (after a load on the same stream).  Errors: LORA_E_SLOT,
 * LORA_E_EMPTY (the slot holds no adapter), LORA_E_ARG, LORA_E_UNSUPPORTED
 * (more than 65535 * 64 rows), LORA_E_HIP.
 */
lora_status lora_merge_slot(const lora_stack *st, int slot, void *W, int64_t ldw, int sign,
                            void *stream);

/* ---------------------------------------------------------------- segments */

/*
 * Create a segments object able to group up to max_rows rows over up to
 * n_slots slots (device arrays: perm, seg_off, active, counts, tile plan).
 * Errors: LORA_E_ARG, LORA_E_UNSUPPORTED, LORA_E_NOMEM.
 */
lora_status lora_segments_create(lora_segments **out, int64_t max_rows, int n_slots);

/* Free a segments object (NULL is accepted); synchronises the device first. */
lora_status lora_segments_destroy(lora_segments *seg);

/*
 * Tile policy of later lora_build_segments calls: a slot whose group has at
 * least m_min rows is served by the SGMV path (dense MFMA tiles of 16 or 64
 * rows), a smaller group by the BGMV path (16-row tiles, wavefront-reduction
 * dot products).  m_min = 1 sends every group to SGMV; m_min > max_rows sends
 * every group to BGMV.  Default 1 (measured: the MFMA tiles are faster even
 * for one-row groups).  Stacks without MFMA tiles (fp32; slices not multiples
 * of 64) run the BGMV code on every tile.  Errors: LORA_E_ARG (m_min < 1).
 */
lora_status lora_segments_set_dense_min(lora_segments *seg, int m_min);

/*
 * Launch shape of the expand of later lora_add_expand / lora_apply /
 * lora_build_apply calls on this segments object: 256-column chunks of one
 * row tile per workgroup.  0 (the default) chooses from the shapes alone: for
 * stacks of rank <= 16 with 16-row dense tiles whose groups average at most
 * 16 rows (n_rows <= 16 n_slots) and at least 2048 (tile, chunk) pairs in the
 * launch bound, 4 when the output has at most 32 chunks, else 2 (many small
 * groups: each workgroup then keeps the next chunk's y and B in flight while
 * it computes the current one); otherwise 1.  1..16 forces that many where the
 * several-chunk expand applies (bf16 stacks with dense tiles, 16-row tiles,
 * r_max <= 64, v of every slice and one B block within the LDS budget) and is
 * ignored elsewhere.  A tuning knob: results are bit-identical for every
 * value.  Errors: LORA_E_ARG (chunks < 0 or > 16).
 */
lora_status lora_segments_set_expand_chunks(lora_segments *seg, int chunks);

/*
 * Bound on the polls a one-launch call (lora_build_apply / lora_apply run as
 * one kernel) makes while an expand workgroup waits for the shrink workgroups
 * of its tile.  The wait always ends by construction (an expand workgroup
 * waits only on earlier-dispatched shrink workgroups that wait on nothing), so
 * the bound is a guard; the default (2^18 polls) is well under a second.  A
 * workgroup that gives up leaves its rows of y untouched and counts a timeout;
 * later one-launch calls on the object then leave y untouched until
 * lora_get_device_status reports LORA_E_HIP, which also resets the object's
 * hand-over state.  polls = 0 checks once (a host-side way to exercise the
 * guard without any kernel misbehaving).  Errors: LORA_E_ARG (polls < 0).
 */
lora_status lora_segments_set_wait_limit(lora_segments *seg, int polls);

/*
 * Group the rows of one batch by adapter slot, on the device (page "LoRA
 * hot-loading and adapter routing", batched multi-adapter execution section:
 * one group of row indices per adapter id; page "Multi-LoRA Serving",
 * section 2 flowchart: group rows by adapter id).
 *
 *   ids     DEVICE int32 [n_rows]; -1 = no adapter.  A row is valid when
 *           0 <= ids[i] < n_slots and the slot holds an adapter at this
 *           point of the stream; any other id except -1 is a bad id: counted,
 *           and the row is left untouched like a none row.
 *   n_rows  0 .. max_rows of seg
 *
 * Result (device, bit-exact and unique): perm = row indices grouped by slot in
 * ascending slot order, ascending row index inside a group, then the rows
 * without a valid adapter in ascending index order; seg_off[s] = first
 * position of slot s in perm, seg_off[n_slots] = number of valid rows; active
 * = slots with at least one row, ascending; counts = {valid rows, active
 * slots, bad ids}.  The launch does not depend on the ids' values.  The
 * segments remain bound to this stack's slot count and n_rows.
 * Errors: LORA_E_ARG, LORA_E_HIP.
 */
lora_status lora_build_segments(const lora_stack *st, const int32_t *ids, int64_t n_rows,
                                lora_segments *seg, void *stream);

/* ------------------------------------------------------------------- apply */

/*
 * add_shrink: v = A_s x_i for every valid row, every slice, in fp32, into the
 * stack's scratch (page "Multi-LoRA Serving", section 2 flowchart and section
 * 3.4: add_shrink, rank-r, grouped per adapter).  x: [n_rows][ldx].
 * Errors: LORA_E_ARG, LORA_E_HIP.
 */
lora_status lora_add_shrink(const lora_stack *st, const void *x, int64_t ldx,
                            const lora_segments *seg, void *stream);

/*
 * add_expand with the per-row merge: y_i[off_q + o] = round(y_i + scale_s *
 * (B_s v_i)[off_q + o]) for every valid row, using the v of the preceding
 * lora_add_shrink on this stack (same page, same sections: add_expand, delta
 * = B v * alpha / r, then the per-row merge y_i = base_i + delta_i).  Rows
 * without a valid adapter and columns >= D are never written.
 * y: [n_rows][ldy], updated in place.  Errors: LORA_E_ARG, LORA_E_HIP.
 */
lora_status lora_add_expand(const lora_stack *st, void *y, int64_t ldy,
                            const lora_segments *seg, void *stream);

/*
 * lora_add_shrink followed by lora_add_expand: y_i += (alpha/r) B (A x_i) for
 * every valid row of the batch grouped by seg, with the same bits.  The launch
 * grid depends only on (n_rows, k, slice widths), never on the adapter mix, so
 * the call can be captured in a HIP graph and replayed for any mix.  Where the
 * shrink and expand workgroups of a batch of 16-row tiles fit the chip at once
 * (as for the one-launch lora_build_apply), both run in one kernel, v handed
 * over through the segments object's per-tile flags; calls on one segments
 * object must then not overlap.  Errors: LORA_E_ARG, LORA_E_HIP.
 */
lora_status lora_apply(const lora_stack *st, void *y, int64_t ldy, const void *x, int64_t ldx,
                       const lora_segments *seg, void *stream);

/*
 * lora_build_segments followed by lora_add_shrink, as one call: the grouping
 * of the rows by adapter id that comes before add_shrink (page "Multi-LoRA
 * Serving", section 2 flowchart; page "LoRA hot-loading and adapter
 * routing", batched multi-adapter execution) and the shrink itself.  The
 * segments left in seg and the v left in the stack's scratch are the same as
 * those of the two calls.  For small batches (n_rows <= 1024 and a shrink
 * grid of at most 512 workgroups, two per compute unit) the grouping runs
 * inside the shrink kernel (each of its workgroups groups the ids in LDS): one
 * launch instead of two on the decode critical path.  Other batches take the
 * two launches.  ids is read at the call's stream position.  All argument checks
 * happen before anything is enqueued.  Errors: LORA_E_ARG, LORA_E_HIP.
 */
lora_status lora_build_shrink(const lora_stack *st, const void *x, int64_t ldx,
                              const int32_t *ids, int64_t n_rows, lora_segments *seg,
                              void *stream);

/*
 * lora_build_shrink followed by lora_add_expand: one call for a whole batch
 * (grouping, add_shrink, add_expand with the per-row merge), with the results
 * and segments of lora_build_segments + lora_apply (y bit-identical: the same
 * tile arithmetic on the same tile plan).  Decode-sized batches run as ONE
 * kernel (lora_build_apply_plan tells which):
 *   - bf16 stacks of one slice with r_max <= 16, <= 63 slots and <= 256 rows
 *     (the decode batches): every workgroup groups the ids itself, and the
 *     shrink workgroups hand v to the expand workgroups as tagged 32-bit
 *     words in the segments object (value and launch tag in one device-scope
 *     atomic access, per-tile epochs: nothing is cleared between launches);
 *   - other batches the fused grouping serves on 16-row tiles, whose grid of
 *     (k-splits + 256-column chunks) x tile bound is at most the workgroups
 *     the chip holds at once plus a quarter: v stored device-coherent and
 *     handed over through per-tile flags that the tile's last expand
 *     workgroup clears.
 * In both, captured graphs replay correctly for any adapter mix.  A wait that
 * never ends is impossible by construction (an expand workgroup waits only on
 * earlier-dispatched shrink workgroups that wait on nothing); as a guard the
 * waits are bounded (lora_segments_set_wait_limit), a workgroup whose wait
 * gives up leaves its rows of y untouched, and from then on every one-launch
 * call on the segments object leaves y untouched until lora_get_device_status
 * reports the timeout (LORA_E_HIP) and resets the hand-over state.  Other
 * batches take 2, 3 or 5 launches.  Calls on one segments object must not
 * overlap (the hand-over state is per object).  n_rows == 0 only writes the
 * (empty) segments.  Errors: LORA_E_ARG, LORA_E_HIP.
 */
lora_status lora_build_apply(const lora_stack *st, void *y, int64_t ldy, const void *x,
                             int64_t ldx, const int32_t *ids, int64_t n_rows, lora_segments *seg,
                             void *stream);

/*
 * lora_build_apply for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the one-launch decode of lora_build_apply with no segments object.  Its
 * hand-over state -- per-tile epochs and counters and the tagged v partials,
 * 1,223,680 bytes -- lives in a static device array that the library holds on
 * each GPU it runs on until the process ends; nothing is allocated per call
 * (the array's address is looked up once per device, on the first call with
 * that device current).  y and the grouping's arithmetic are those of
 * lora_build_apply on the same batch (bit-identical y); no segments are
 * written.
 *
 *   y, ldy, x, ldx, ids, n_rows   as lora_build_apply (device pointers)
 *   timeouts   DEVICE int32 or NULL: waits that gave up are added to it (a
 *              guard that by construction never fires; rows of a tile whose
 *              wait gave up are left untouched)
 *
 * Served shapes: bf16 stacks of one slice with r_max <= 16 and an output width
 * of whole 64-column blocks, k a multiple of 128, at most 63 slots, 1 .. 256
 * rows (the decode batches), and a grid that fits the chip at once.  Anything
 * else returns LORA_E_UNSUPPORTED before anything is enqueued (n_rows == 0
 * returns LORA_OK and does nothing).  Every call on one GPU shares the array:
 * calls that overlap on one GPU (other streams, other threads) race and must
 * be ordered by the caller.  Errors: LORA_E_ARG, LORA_E_UNSUPPORTED, LORA_E_HIP.
 */
lora_status lora_build_apply_noalloc(const lora_stack *st, void *y, int64_t ldy, const void *x,
                                     int64_t ldx, const int32_t *ids, int64_t n_rows,
                                     int32_t *timeouts, void *stream);

/*
 * Kernel launches a lora_build_apply of n_rows rows on (st, seg) makes, with
 * seg's current tile policy: 1 (one kernel: the decode path), 2 (grouping
 * inside the shrink, then the expand), 3 (grouping, shrink, expand) or 5 (the
 * chunked grouping's three kernels, shrink, expand); 1 for n_rows == 0.  The
 * count depends only on shapes, never on the adapter mix (page "LoRA serving:
 * multi-adapter dynamic loading", section 6: mix-dependent launch shapes are
 * what breaks graph capture), so it is also the node count of a captured
 * call.  Host only: nothing is enqueued; seg is not modified.  Errors:
 * LORA_E_ARG (null pointer, n_rows < 0 or beyond either object's max_rows,
 * mismatched objects).
 */
lora_status lora_build_apply_plan(const lora_stack *st, int64_t n_rows, const lora_segments *seg,
                                  int32_t *n_launches);

/* --------------------------------------------------------------- residency */

/*
 * Adapter residency around one stack: a host tier of registered adapters in
 * pinned memory (max_cpu_adapters of them), GPU residency of up to n_slots
 * (the stack's slots) with least-recently-used eviction, and the mapping of a
 * batch's per-row adapter ids to slot ids.  Page "LoRA hot-loading and adapter
 * routing", adapter-lifecycle section (load on first use after a rank check;
 * past the limit the least recently used adapter is unloaded and reloaded on
 * its next use); page "Multi-LoRA Serving: one base, many adapters", section
 * 3.2 (adapters resident on the GPU with an optional CPU-side cache: max_loras
 * and max_cpu_loras) and section 6 (a batch with more distinct adapters than
 * max_loras cannot run in one step); page "LoRA serving: multi-adapter dynamic
 * loading", section 4 (loading copies A and B to the GPU; unloading is
 * immediate).
 *
 * Not thread-safe; one manager per stack.  All GPU work goes on the stream
 * passed to each call; the caller runs the batch's lora_build_segments /
 * lora_apply on that stream too (or orders the streams), so loads and
 * evictions land between batches.  Direct lora_load_slot / lora_evict_slot
 * calls on the stack are followed at the next map_batch: a slot the caller
 * loaded is left to the caller, one the caller emptied becomes usable, and an
 * adapter whose slot the caller evicted is loaded again when next used.
 * After LORA_E_HIP the manager's view of the slots is undefined: destroy it.
 */
typedef struct lora_residency lora_residency;

/* Counters of lora_residency_stats, by index. */
enum {
    LORA_RES_HITS = 0,          /* adapter uses served by a resident slot        */
    LORA_RES_LOADS = 1,         /* host -> GPU loads (misses)                    */
    LORA_RES_EVICTIONS = 2,     /* slots freed for another adapter or unregister */
    LORA_RES_HOST_DROPS = 3,    /* host-tier entries dropped to admit a new one  */
    LORA_RES_BYTES_LOADED = 4,  /* adapter bytes copied host -> GPU (true rank)  */
    LORA_RES_HOST_ENTRIES = 5,  /* registered adapters now in the host tier      */
    LORA_RES_RESIDENT = 6,      /* adapters now resident on the GPU              */
    LORA_RES_NSTATS = 7
};

/*
 * Create a manager.  With a stack (st != NULL) the manager owns the stack's
 * slots that are empty now (slots the caller already loaded are never used)
 * and the shape arguments are ignored.  With st == NULL it only plans: same
 * decisions and slot ids, no data moved, no GPU call (n_slots, r_max, k,
 * n_slices, slice_d, dtype give the shape, as in lora_stack_create).
 * max_cpu_adapters >= 1 bounds the host tier.  The stack must outlive the
 * manager.  Errors: LORA_E_ARG, LORA_E_NOMEM.
 */
lora_status lora_residency_create(lora_residency **out, lora_stack *st, int n_slots, int r_max,
                                  int64_t k, int n_slices, const int64_t *slice_d,
                                  lora_dtype dtype, int max_cpu_adapters);

/* Free the manager and its pinned host tier (waits for copies still reading
 * it).  The slots it loaded stay loaded in the stack.  NULL is accepted. */
lora_status lora_residency_destroy(lora_residency *m);

/*
 * Register an adapter under a caller-chosen id >= 0: A [n_slices][rank][k]
 * and B [D][rank] (HOST pointers, dense, true rank, the stack's dtype) are
 * copied into the pinned host tier; the call returns once they are copied.
 * The rank is checked here (page "Multi-LoRA Serving", section 6: an adapter
 * above the rank cap is refused at load).  When the host tier is full the
 * least recently used adapter that is not resident on the GPU is dropped
 * (LORA_E_CAPACITY when every entry is resident); the registration itself
 * counts as a use.  A host tier of at least n_slots plus the distinct adapters
 * of one batch never drops an adapter the next batch needs while the caller
 * registers it.  Errors: LORA_E_ARG,
 * LORA_E_RANK, LORA_E_OCCUPIED (id already registered), LORA_E_CAPACITY,
 * LORA_E_NOMEM, LORA_E_HIP.
 */
lora_status lora_residency_register(lora_residency *m, int64_t adapter_id, int rank, float alpha,
                                    const void *A, const void *B);

/* Drop an adapter: its slot (if resident) is evicted in stream order and its
 * host copy freed once no copy reads it.  Errors: LORA_E_ARG,
 * LORA_E_NOT_FOUND, LORA_E_HIP. */
lora_status lora_residency_unregister(lora_residency *m, int64_t adapter_id, void *stream);

/*
 * Map one batch: row_adapter (HOST int64 [n_rows], -1 = no adapter) ->
 * ids_out (HOST int32 [n_rows], the slot of each row's adapter, -1 for none),
 * the ids lora_build_segments takes.  Every adapter the batch uses is made
 * resident first: already resident is a hit; otherwise it goes to an empty
 * slot (lowest index) or replaces the least recently used resident adapter
 * this batch does not use (ties: lowest slot), copied from the host tier in
 * stream order.  "Used" advances once per batch (and per registration).
 * Checked before anything
 * changes: LORA_E_NOT_FOUND (an id not registered), LORA_E_CAPACITY (more
 * distinct adapters than usable slots: split the batch), LORA_E_ARG.  Also
 * LORA_E_HIP.
 */
lora_status lora_residency_map_batch(lora_residency *m, const int64_t *row_adapter, int64_t n_rows,
                                     int32_t *ids_out, void *stream);

/* Slot holding an adapter (-1 when registered but not resident).  Errors:
 * LORA_E_ARG, LORA_E_NOT_FOUND. */
lora_status lora_residency_slot_of(const lora_residency *m, int64_t adapter_id, int *slot);

/* Counters (HOST int64 [LORA_RES_NSTATS], indices above).  Errors: LORA_E_ARG. */
lora_status lora_residency_stats(const lora_residency *m, int64_t *stats);

/* --------------------------------------------------------------- inspection */

/*
 * Copy the grouping to HOST arrays and synchronise the stream.  perm
 * [n_rows], seg_off [n_slots + 1], active [n_slots] (entries past counts[1]
 * are -1), counts [3] = {valid rows, active slots, bad ids}.  Any output
 * pointer may be NULL.  Errors: LORA_E_ARG, LORA_E_HIP.
 */
lora_status lora_segments_download(const lora_segments *seg, int32_t *perm, int32_t *seg_off,
                                   int32_t *active, int32_t *counts, void *stream);

/* Number of bad ids seen by the last lora_build_segments (synchronises the
 * stream).  Returns LORA_E_BAD_IDS when it is nonzero, LORA_OK otherwise;
 * LORA_E_HIP if a one-launch call on this object gave up waiting for its
 * shrink since the last such report (rows of the affected tiles were left
 * untouched, and calls after it left y untouched); the report resets the
 * object's hand-over state, so the next call computes normally. */
lora_status lora_get_device_status(const lora_segments *seg, int64_t *n_bad, void *stream);

/* Number of row tiles the last lora_build_segments gave each path (host
 * copy; synchronises the stream).  Either pointer may be NULL. */
lora_status lora_segments_tile_counts(const lora_segments *seg, int32_t *n_bgmv,
                                      int32_t *n_sgmv, void *stream);

/* Static description of a status code. */
const char *lora_status_string(lora_status s);

#ifdef __cplusplus
}
#endif

#endif /* RANK_ADAPTER_GEMM_LORA_AMD_LORA_H */
