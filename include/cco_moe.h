/*
 * cco_moe.h -- zero-copy MoE dispatch -> expert -> combine over a symmetric
 * heap, one MI355X (gfx950).
 *
 * Sources, cited by page title and section:
 *   [blog]  "MORI CCO: Next-Generation Collective Communication Object for
 *           GPUs" (AMD technical article).
 *   [guide] "MORI CCO Guide", sections "Concepts", "Memory and Windows",
 *           "C++ API".
 *
 * The symmetric heap is one flat device buffer sliced into equal slots; a
 * window is carved at the same offset in every slot, so the address of a
 * window in slot s is  base + s * stride + offset  ([blog] "What is MORI
 * CCO?").  Slots stand in for ranks: on one GPU every slot is a region of
 * that GPU's own HBM, and "sending to a peer" is a store at a slot address.
 *
 * Conventions (after [guide] "C++ API": status-returning calls with
 * out-parameters, paired create/destroy, and resources owned by the object
 * that created them and freed with it):
 *   - every call returns a cco_status (0 = success) unless stated;
 *   - argument errors are reported before anything is launched;
 *   - plan / dispatch / expert / combine are asynchronous on `stream` and
 *     allocate nothing; they must be issued in that order on one stream for
 *     the same T and the same idx.  The object's routing state, status word
 *     and GEMM tile queues serve every pass, so two passes of one object
 *     must not overlap on the device (use separate objects for concurrent
 *     streams);
 *   - errors found on the device (a bad expert id, a slot overflow) go to a
 *     per-object status word that cco_moe_status reads; the next plan
 *     recomputes it.  Rows that do not fit are dropped, never written out of
 *     bounds;
 *   - one cco_moe may not be used from two host threads at once; separate
 *     objects are independent.
 *
 * Data types: bf16 is passed as uint16_t bit patterns; weights are fp32;
 * expert ids and sizes int32.  All tensors are dense row-major.
 *
 * Expert-to-slot map: experts are split into S contiguous blocks of E/S,
 * expert e lives in slot e / (E/S).
 * Row order inside a slot: by ascending expert id, and inside one expert by
 * the flat pair index t*K + j (a stable counting sort).  One row per
 * (token, k) pair, duplicates included.
 */
#ifndef CCO_MOE_H
#define CCO_MOE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CCO_OK = 0,
  CCO_INFO_COPIED = 1,         /* combine copied a foreign expert output in */
  CCO_ERR_INVALID_ARG = -1,    /* bad argument, found on the host */
  CCO_ERR_OUT_OF_MEMORY = -2,  /* device allocation failed (create calls only) */
  CCO_ERR_HIP = -3,            /* a HIP runtime call failed */
  CCO_ERR_CAPACITY = -4,       /* device: a slot received more than cap rows */
  CCO_ERR_BAD_EXPERT = -5,     /* device: an expert id outside [0, E) */
  CCO_ERR_HEAP_FULL = -6,      /* the heap's slots have no room for this object */
  CCO_ERR_TOO_LARGE = -7,      /* the batch exceeds the fixed scratch of cco_moe_plan_noalloc */
  CCO_ERR_TIMEOUT = -8,        /* device: a wait of cco_moe_fused gave up; outputs undefined */
  CCO_ERR_DISABLED = -9        /* the entry point is switched off in the library */
} cco_status;

/* Opaque handles. */
typedef struct cco_sym_heap cco_sym_heap;
typedef struct cco_moe cco_moe;

/* Shape of one MoE layer.
 *   max_tokens   largest T any call will pass (sizes the receive windows)
 *   hidden       H, bf16 elements per token row; multiple of 8 (16-byte
 *                rows); with inter > 0 also a multiple of 256
 *   topk         K >= 1, at most 32, experts per token
 *   num_experts  E >= 1, at most 1024, a multiple of the heap's slot count
 *   inter        I, SwiGLU intermediate size, a multiple of 128, with one
 *                expert's gate+up weights (4 * I * H bytes) under 2 GiB;
 *                0 selects identity experts (the expert output is the
 *                dispatched row itself and combine reads the receive window)
 * T * K and the per-slot capacity must fit in int32.  Shapes outside these
 * limits are rejected (-1 / 0 bytes) before anything is allocated.
 */
typedef struct {
  int32_t max_tokens;
  int32_t hidden;
  int32_t topk;
  int32_t num_experts;
  int32_t inter;
} cco_moe_shape;

/* Device pointers of the routing state that plan writes (owned by the
 * cco_moe; valid until the heap is destroyed). */
typedef struct {
  int32_t *pos;        /* [max_tokens][K]: row inside slot(idx[t][j]); -1 for a
                        * pair whose row would fall at or past the slot's
                        * capacity (dropped) or whose id is invalid */
  int32_t *counts;     /* [E]: rows routed to each expert */
  int32_t *expert_off; /* [E]: first row of each expert inside its slot */
  int32_t *slot_total; /* [S]: rows received by each slot (the receive count) */
  int32_t *status;     /* [1]: device status word (0 or a negative cco_status) */
} cco_moe_routing;

/* Byte offsets of the windows inside every slot (identical in all slots).
 * A window that the shape does not need has size 0. */
typedef struct {
  uint64_t disp_x, disp_x_bytes;       /* dispatched rows  [cap][H] bf16 */
  uint64_t disp_meta, disp_meta_bytes; /* per-row {src = t*K+j, w, expert} [cap] x 12 B */
  uint64_t hbuf, hbuf_bytes;           /* SwiGLU intermediate [cap][I] bf16 */
  uint64_t out_tok, out_tok_bytes;     /* expert output [cap][H] bf16 */
  int64_t cap;                         /* rows per slot */
} cco_moe_layout;

/* ---------------------------------------------------------- the heap --- */

/* Create a symmetric heap: ONE device allocation of nslots slots of
 * `stride` bytes, stride = per_slot_bytes rounded up to 2 MiB, on HIP device
 * `device`.  [guide] "Memory and Windows": symmetric memory sits at the same
 * offset on every rank; here every rank is a slot of one buffer.
 * Errors: CCO_ERR_INVALID_ARG (out == NULL, nslots < 1, per_slot_bytes == 0,
 * bad device), CCO_ERR_OUT_OF_MEMORY, CCO_ERR_HIP. */
int cco_sym_heap_create(int device, int32_t nslots, uint64_t per_slot_bytes,
                        cco_sym_heap **out);

/* Free the heap's buffer and every cco_moe created on it ([guide] "Memory
 * and Windows": resources are released with their owner).  NULL is a no-op.
 * Synchronises the device first. */
int cco_sym_heap_destroy(cco_sym_heap *heap);

/* base + slot * stride + offset ([blog] "What is MORI CCO?", the peer
 * address formula).  Returns NULL if slot or offset is out of range. */
void *cco_sym_heap_slot_ptr(const cco_sym_heap *heap, int32_t slot, uint64_t offset);

/* Heap geometry; any out-pointer may be NULL. */
int cco_sym_heap_info(const cco_sym_heap *heap, void **base, uint64_t *stride,
                      int32_t *nslots, uint64_t *used);

/* ----------------------------------------------------------- the MoE --- */

/* Bytes of slot space one cco_moe of this shape needs on a heap with nslots
 * slots (0 if the shape is invalid).  Pure host function. */
uint64_t cco_moe_required_slot_bytes(const cco_moe_shape *shape, int32_t nslots);

/* Window layout of such an object, relative to its first byte in a slot
 * (pure host function; CCO_ERR_INVALID_ARG for an invalid shape). */
int cco_moe_layout_of(const cco_moe_shape *shape, int32_t nslots, cco_moe_layout *out);

/* Carve the windows of one MoE layer out of every slot of `heap`, at the
 * heap's next free offset (the same in every slot), and allocate its
 * routing state: the plan's per-pair arrays and scratch, and, with experts
 * (inter > 0), a workspace for the expert GEMMs' split tiles of 256 KiB per
 * compute unit (64 MiB on MI355X).  The heap owns the result.  [blog] "Zero-copy MoE
 * dispatch -> expert -> combine": the op object is built on the
 * communicator and every intermediate it hands out is a view of symmetric
 * memory.
 * Errors: CCO_ERR_INVALID_ARG (shape checks above, E % nslots != 0),
 * CCO_ERR_HEAP_FULL, CCO_ERR_OUT_OF_MEMORY, CCO_ERR_HIP. */
int cco_moe_create(cco_sym_heap *heap, const cco_moe_shape *shape, cco_moe **out);

/* Window offsets of this object inside each slot (absolute, from the slot's
 * first byte). */
int cco_moe_get_layout(const cco_moe *m, cco_moe_layout *out);

/* Routing-state device pointers. */
int cco_moe_get_routing(const cco_moe *m, cco_moe_routing *out);

/* Plan ([blog] "Zero-copy MoE dispatch": dispatch returns the receive count
 * and a routing object that combine reuses).
 *   topk_idx  device int32 [T][K], expert ids, row-major, caller-owned,
 *             4-byte aligned
 *   T         0 <= T <= max_tokens (T == 0 is a no-op that zeroes the counts)
 * Computes per-expert counts, slot-local expert offsets, per-slot totals and
 * pos[t][j] = expert_off[e] + number of earlier pairs (flat order t*K+j)
 * with the same expert e, or -1 when that row is at or past the slot's
 * capacity (the pair is dropped: dispatch, expert and combine skip it).
 * Device errors: CCO_ERR_BAD_EXPERT, CCO_ERR_CAPACITY (reported by
 * cco_moe_status). */
int cco_moe_plan(cco_moe *m, const int32_t *topk_idx, int32_t T, void *stream);

/* Dispatch ([blog] "Zero-copy MoE dispatch", step 1: each token row is
 * written straight into the receive window of the slot that owns each of
 * its experts; no staging copy).
 *   x        device bf16 [T][H], 16-byte aligned
 *   weights  device fp32 [T][K] routing weights, 4-byte aligned (carried
 *            into the per-row metadata; applied by combine)
 * For every pair: DISP_X[slot(e)][pos] = x[t] bit for bit and
 * DISP_META[slot(e)][pos] = {t*K + j, w[t][j], e}.  Needs the same T and
 * idx as the preceding plan.  Errors: CCO_ERR_INVALID_ARG (T differs from
 * the plan's, NULL or misaligned pointers), before any launch. */
int cco_moe_dispatch(cco_moe *m, const uint16_t *x, const float *weights,
                     int32_t T, void *stream);

/* Dispatch of tokens the caller has already quantized to 8 bits, with
 * their scales ([blog] "Zero-copy MoE dispatch", step 1: the op's dispatch
 * takes the tokens, their weights, their scales and the expert ids, and
 * hands back received tokens, weights and scales).  The bytes move
 * unchanged; no format is assumed for the 8-bit values or the scales.
 *   x8       device, T rows of H bytes (H % 16 == 0), 16-byte aligned
 *   scales   device fp32 [T][ns], 4-byte aligned; may be NULL when ns == 0
 *   ns       scales per token, 0 <= 4 * ns <= H
 *   weights  device fp32 [T][K], as for cco_moe_dispatch
 * A receive row keeps its 2H bytes: DISP_X row bytes [0, H) = x8[t] and
 * [H, H + 4 ns) = scales[t] as stored; the rest of the row is not written.
 * DISP_META as for cco_moe_dispatch.  Needs the same T and idx as the
 * preceding plan.  Moves half the token bytes of the bf16 dispatch.
 * Until the next cco_moe_dispatch, cco_moe_expert reads these rows as OCP
 * e4m3 values with fp32 block scales (see there), and a combine of identity
 * experts through the receive window refuses them (CCO_ERR_INVALID_ARG); a
 * caller's own expert reads cco_moe_dispatch_view and writes
 * cco_moe_combine_in_view.
 * Errors: CCO_ERR_INVALID_ARG for the checks above, before any launch. */
int cco_moe_dispatch_fp8(cco_moe *m, const uint8_t *x8, const float *scales, int32_t ns,
                         const float *weights, int32_t T, void *stream);

/* Expert ([blog] "Zero-copy MoE dispatch", step 2: the expert reads the
 * receive window in place and writes the combine staging window, row i to
 * row i).  SwiGLU per expert e on its rows X of DISP_X:
 *   h = bf16( silu(X Wg^T) * (X Wu^T) )  -> HBUF  (fp32 accumulation)
 *   y = bf16( h Wd^T )                   -> OUT_TOK
 *   w13  device bf16 [E][2I][H]: rows 0..I-1 gate, rows I..2I-1 up;
 *        16-byte aligned
 *   w2   device bf16 [E][H][I], 16-byte aligned
 * (both K-contiguous, like nn.Linear.weight).  Row counts are read on the
 * device; nothing is copied to the host.  Results are deterministic for a
 * given routing on a given device: in GEMMs of few tile rounds (and at
 * least 16 K-steps of 64) the last tiles sum their K-steps in ranges,
 * added in range order.  With
 * inter == 0 this is a no-op (identity experts; w13 and w2 may be NULL).
 * After cco_moe_dispatch_fp8 the rows X are the 8-bit receive rows, read in
 * place ([blog] "Zero-copy MoE dispatch", step 1: the received tokens come
 * with their scales; that the expert applies them as below is this
 * library's reading, the page leaves it open): byte k of a row is an OCP
 * e4m3fn code (1 sign, 4 exponent bits of bias 7, 3 mantissa bits; no
 * infinities, S.1111.111 is NaN), and value k of the row is
 *   X[k] = bf16( binary32(e4m3(code k) * scale[k / (H / ns)]) )
 * with the ns fp32 scales after the H codes (scale 1 when ns == 0): each
 * product rounded to nearest even in binary32, then to bf16.  The GEMMs
 * then run as for bf16 rows, so the results equal the bf16 path's on
 * those X bit for bit.  H / ns must be 64 times a power of two (the scale
 * blocks are whole runs of the GEMM's 64-value K-steps), else
 * CCO_ERR_INVALID_ARG before any launch. */
int cco_moe_expert(cco_moe *m, const uint16_t *w13, const uint16_t *w2, void *stream);

/* Receive window of `slot` ([blog] "Zero-copy MoE dispatch -> expert ->
 * combine", step 1: the received tokens the op's dispatch returns are not a
 * new tensor but a view of the "disp_out" region of symmetric memory, which
 * the dispatching peers wrote directly): DISP_X base, [cap][H] bf16 (after
 * cco_moe_dispatch_fp8: the same 2H-byte rows holding the 8-bit codes and
 * their scales, see there); rows [expert_off[e], expert_off[e] + counts[e])
 * belong to expert e, and the first slot_total[slot] rows are the ones
 * received.  Borrowed: valid until the heap is destroyed, overwritten by
 * the next dispatch.  NULL if slot is out of range or m is NULL. */
void *cco_moe_dispatch_view(cco_moe *m, int32_t slot);

/* Combine staging window of `slot` ([blog] "Zero-copy MoE dispatch":
 * combine_in_view): OUT_TOK base, or DISP_X for identity experts. */
void *cco_moe_combine_in_view(cco_moe *m, int32_t slot);

/* Combine ([blog] "Zero-copy MoE dispatch", step 3: each token reads its
 * rows back from the slots that own its experts and sums them with its
 * routing weights).
 *   expert_out  host array of S device pointers, the expert output of each
 *               slot ([slot_total][H] bf16, row i for receive row i), or
 *               NULL to use the staging views.  A slot whose pointer is not
 *               its staging view is first copied into the view (one device
 *               copy of its rows) and the call returns CCO_INFO_COPIED
 *               ([blog] "Zero-copy MoE dispatch", note on the data_ptr
 *               match).
 *   weights     device fp32 [T][K], 4-byte aligned
 *   out         device bf16 [T][H], caller-owned, 16-byte aligned; a
 *               foreign expert output must be 16-byte aligned too
 *   out[t] = bf16( sum_j w[t][j] * y[slot(e)][pos[t][j]] ), fp32 fused
 *   multiply-add in j = 0..K-1 order, rounded once to nearest even; dropped
 *   pairs (pos -1) contribute nothing.
 * Errors: CCO_ERR_INVALID_ARG (T differs from the plan's, NULL or
 * misaligned pointers), before any launch. */
int cco_moe_combine(cco_moe *m, const void *const *expert_out, const float *weights,
                    uint16_t *out, int32_t T, void *stream);

/* SWITCHED OFF: returns CCO_ERR_DISABLED before any launch unless the
 * library is compiled with CCO_BUILD_FUSED (its kernel faulted the GPU on
 * its first run and the cause is not yet shown).  The contract below is the one it is built to.
 *
 * The whole path -- plan, dispatch, expert (SwiGLU gate/up and down),
 * combine -- in ONE persistent kernel launch ([blog] "Mega-MoE: mega-kernel
 * co-design with FlyDSL": dispatch, expert GEMM and combine fused into one
 * kernel with no synchronisation between kernels; "In-kernel
 * compute-communication fusion": the stages overlap at tile granularity).
 * Arguments as for cco_moe_plan, cco_moe_dispatch, cco_moe_expert and
 * cco_moe_combine with expert_out = NULL, in that order, and it leaves the
 * object in the same state: routing state, receive, intermediate and
 * staging windows, and `out`.  Plan, dispatch and combine (of the same expert
 * rows) are bit-identical to the separate calls; the expert tiles are the
 * same, except that this path never sums a tile in K-ranges (the separate
 * GEMMs do for the last tiles of a GEMM with few rounds), so those tiles may
 * differ by rounding.
 * Inside the launch a down tile starts once the gate/up tiles of its rows
 * are done, and a block of tokens is combined once the down tiles of its
 * rows are; expert tiles start once their expert's rows have arrived.  The
 * waits are bounded: if the grid cannot make progress (for example when
 * other work holds some of the compute units), the status word becomes
 * CCO_ERR_TIMEOUT after about two seconds and the kernel exits.
 * Errors: CCO_ERR_INVALID_ARG (as the separate calls, and for top-k above
 * 8), CCO_ERR_HIP; device errors as cco_moe_plan, plus CCO_ERR_TIMEOUT (all
 * read by cco_moe_status). */
int cco_moe_fused(cco_moe *m, const int32_t *topk_idx, const uint16_t *x, const float *weights,
                  const uint16_t *w13, const uint16_t *w2, uint16_t *out, int32_t T,
                  void *stream);

/* Copy one slot's expert output from a buffer of the caller's into that
 * slot's combine staging window on the GPU's copy engines (SDMA), not on
 * compute units ([blog] "Multiple communication transports": SDMA serves
 * background bulk copies that keep the CUs free; "GEMM + all-to-all
 * fusion": GEMM output tiles move by SDMA as they become ready, while the
 * remaining tiles compute).  A caller whose expert writes buffers of its own
 * (the pages' data_ptr mismatch, [blog] "Zero-copy MoE dispatch", note)
 * issues this per slot, on a stream of its own, as each slot's output is
 * done, and then calls cco_moe_combine with expert_out = NULL.
 *   slot    0 <= slot < S
 *   src     device bf16 [rows][H], 16-byte aligned, not overlapping the
 *           window (src equal to the staging view copies nothing)
 *   rows    rows to copy, 0 <= rows <= cap: the slot's receive count, which
 *           the caller holds (cco_moe_status; the pages' total_recv).  Rows
 *           of the window past `rows` keep what they held, so a count below
 *           the receive count leaves combine reading stale rows.
 * Asynchronous on `stream`.  Errors: CCO_ERR_INVALID_ARG (before any copy),
 * CCO_ERR_HIP. */
int cco_moe_stage_in_sdma(cco_moe *m, int32_t slot, const void *src, int32_t rows,
                          void *stream);

/* Receive counts and device status, read on the host ([blog] "Zero-copy
 * MoE dispatch -> expert -> combine", step 1: after dispatch the host
 * synchronises and reads the device-side receive count, total_recv, to
 * slice the received tokens).  The path itself never needs this call: the
 * expert and combine kernels read the counts on the device.
 *   stream         the stream the path runs on; synchronised first
 *   slot_total     host int32 [S] or NULL: rows received by each slot
 *   expert_counts  host int32 [E] or NULL: rows routed to each expert
 * Returns the device status word of the last plan (CCO_OK,
 * CCO_ERR_BAD_EXPERT or CCO_ERR_CAPACITY), CCO_ERR_INVALID_ARG for a NULL
 * m, or CCO_ERR_HIP. */
int cco_moe_status(cco_moe *m, void *stream, int32_t *slot_total, int32_t *expert_counts);

/* The plan of cco_moe_plan, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, hosts that forbid
 * allocation): no cco_moe object, every output in caller memory, and the
 * kernels' scratch (per-chunk histograms, a chunk ticket, each pair's
 * expert id) in a fixed array of about 3 MiB that the library holds on each
 * GPU it runs on until the process ends.  Calls nothing that allocates.
 *   topk_idx    device int32 [T][K] expert ids (may be NULL when T == 0)
 *   T, K, E, S  tokens, top-k (1..32), experts (1..1024), slots (E % S == 0)
 *   cap         rows per slot (0 <= cap <= INT32_MAX); a pair whose row
 *               would fall at or past cap gets pos -1 and the status word
 *               CCO_ERR_CAPACITY
 *   pos         device int32 [T][K] (may be NULL when T == 0)
 *   counts, expert_off  device int32 [E];  slot_total  device int32 [S]
 *   status      device int32 [1]: CCO_OK, CCO_ERR_BAD_EXPERT or
 *               CCO_ERR_CAPACITY once the stream reaches it
 * Outputs are those cco_moe_plan writes for the same idx, S and cap.  All
 * pointers 4-byte aligned; runs on the current device, asynchronously on
 * `stream`.  Errors, before any launch: CCO_ERR_TOO_LARGE for T * K above
 * 2^19 pairs; CCO_ERR_INVALID_ARG for the other limits and for NULL or
 * misaligned pointers.  Every call on one GPU shares that GPU's scratch:
 * calls that overlap on one GPU (two streams or two host threads) race, so
 * serialise them. */
int cco_moe_plan_noalloc(const int32_t *topk_idx, int32_t T, int32_t K, int32_t E, int32_t S,
                         int64_t cap, int32_t *pos, int32_t *counts, int32_t *expert_off,
                         int32_t *slot_total, int32_t *status, void *stream);

/* Per-kernel timing with HIP events on the launch stream.  While enabled,
 * each kernel launch of this object is bracketed by a pair of events; the
 * summary returns, per kernel kind, the number of timed launches and their
 * total milliseconds.  Kinds: 0 plan-count (the whole plan for a batch of
 * at most 2048 (token, k) pairs, which runs in one launch), 1 plan-rank,
 * 2 dispatch, 3 expert gate/up, 4 expert down, 5 combine, 6 combine
 * copy-in, 7 8-bit dispatch, 8 staging copy on the copy engines, 9 the
 * single-launch path of cco_moe_fused.
 * Reading the summary synchronises the recorded events and resets it. */
#define CCO_NUM_KERNEL_KINDS 10
int cco_moe_set_timing(cco_moe *m, int enable);
int cco_moe_timing_summary(cco_moe *m, int32_t *launches, double *total_ms);

/* Human-readable name of a status code (static string). */
const char *cco_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* CCO_MOE_H */
