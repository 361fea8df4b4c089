/*
 * moe_ep.h -- C ABI of libmoe_ep.so: MoE token dispatch and combine on one
 * AMD Instinct MI355X (gfx950).
 *
 * The operations follow the problem statement of the expert-parallel buffer
 * API documented on the NeMo AutoModel page
 * "nemo_automodel.components.moe.uccl_ep.buffer" (sections Buffer.get_dispatch_layout,
 * Buffer.dispatch, Buffer.combine, Buffer.low_latency_dispatch,
 * Buffer.low_latency_combine, Buffer.get_low_latency_rdma_size_hint) and the
 * routing expansion of the "dots-infra/ultraep architecture" page (Overview;
 * GPU operations: Load computation, Placement planning, Routing expansion).
 * Everything runs on one GPU: the R logical ranks of the expert-parallel group
 * are partitions of one HBM buffer.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Pointers named as device memory are caller-owned device pointers (for
 *    example a torch tensor's data_ptr()). The library allocates nothing,
 *    frees nothing and keeps no state between calls beyond a per-device
 *    architecture check, so calls from several host threads are safe.
 *  - Every call enqueues its kernels on the caller's stream and returns
 *    without waiting for them (no host synchronisation, no host-visible
 *    counts). A NULL stream is the default stream.
 *  - Return value: MOE_OK (0), or a negative MOE_ERR_* code from a host-side
 *    check. When a check fails, nothing has been enqueued.
 *  - Data errors that only the device can see (an expert id outside [-1, E),
 *    a low-latency expert receiving more than M rows, a slot outside the
 *    receive buffer) make the kernels skip the offending pair and OR a
 *    MOE_STATUS_* bit into *status, when the caller passes a status word.
 *    The caller zeroes it; it can be read after synchronising the stream.
 *  - T = 0 (an empty batch) is valid: counts and offsets are written as zeros,
 *    dispatch and combine do nothing.
 *  - No output needs to be zero-initialised beforehand.
 *  - Row-major layouts everywhere. bf16 values travel as raw 16-bit patterns
 *    (uint16_t). Pointers to bf16 rows, f32 rows and the receive buffer must be
 *    16-byte aligned, and H must be a multiple of 8 (one 16-byte vector is
 *    8 bf16 values). Routing pointers (topk_idx, phys_idx: int64) must be
 *    8-byte aligned (the kernels read them as 8-byte words); MOE_ERR_ALIGN
 *    otherwise.
 *  - Limits: 1 <= E <= 1024, 1 <= R, E % R == 0, 1 <= K <= 64,
 *    0 <= T, T*K + E*(A-1) < 2^31, 8 <= H <= 2^20, 1 <= A <= 2^16.
 */
#ifndef MOE_EP_H
#define MOE_EP_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 5

/* Host-side return codes. */
#define MOE_OK 0
#define MOE_ERR_NULL (-1)      /* a required pointer is NULL */
#define MOE_ERR_SHAPE (-2)     /* a size is out of range or inconsistent */
#define MOE_ERR_CAPACITY (-3)  /* receive buffer smaller than the worst case */
#define MOE_ERR_LL (-4)        /* low latency: T > M, or src_rank not in [0, R) */
#define MOE_ERR_ALIGN (-5)     /* a row pointer is not 16-byte aligned, or an id pointer
                                  not 8-byte aligned */
#define MOE_ERR_WORKSPACE (-6) /* workspace missing or smaller than required */
#define MOE_ERR_LAUNCH (-7)    /* the HIP runtime refused a kernel launch */
#define MOE_ERR_ARCH (-8)      /* the current device is not gfx950 */
#define MOE_ERR_DEVICE (-9)    /* the HIP runtime could not be queried */
#define MOE_ERR_FLAGS (-10)    /* an unsupported FP8 flag combination */
#define MOE_ERR_SCRATCH (-11)  /* the layout workspace would exceed MOE_STATIC_SCRATCH_BYTES */

/* Size of the library's static per-GPU layout workspace
 * (moe_layout_dispatch_static). */
#define MOE_STATIC_SCRATCH_BYTES (4u << 20)

/* FP8 cast options (Buffer.low_latency_dispatch: round_scale, use_ue8m0). */
#define MOE_FP8_ROUND_SCALE 1 /* scales rounded up to powers of two */
#define MOE_FP8_UE8M0 2       /* scales stored as packed exponent bytes; needs
                                 MOE_FP8_ROUND_SCALE and H % 512 == 0 */
#define MOE_FP8_SCALE_ROWS 4  /* low-latency scales row-major (see below) */

/* Device-side status bits (OR-ed into *status). */
#define MOE_STATUS_BAD_EXPERT 1   /* an id outside [-1, E): the pair is skipped */
#define MOE_STATUS_LL_OVERFLOW 2  /* low latency: an expert got more than M pairs */
#define MOE_STATUS_BAD_SLOT 4     /* a slot outside [-1, recv_rows): the pair is skipped */
#define MOE_STATUS_BAD_REPLICA 8  /* reroute: replica table entry out of range */

/* Problem shape. T tokens, hidden size H, E experts spread evenly over R
 * logical ranks (L = E/R local experts each, expert e lives on rank e / L),
 * K selections per token, and expert alignment A (Buffer.dispatch,
 * expert_alignment: every expert's row count is rounded up to a multiple of A). */
typedef struct {
  int32_t T, H, E, R, K, A;
} moe_shape;

/* Device arrays written by the layout calls; together they are the
 * communication handle that Buffer.dispatch hands on to Buffer.combine.
 * Pointers marked "may be NULL" are skipped when NULL. */
typedef struct {
  int32_t *count;            /* [E] pairs per expert (num_tokens_per_expert). Low latency:
                                rows received per expert from this source, min(pairs, M). */
  int32_t *offset;           /* [E+1] first row of each expert; offset[E] = rows used.
                                Low latency: stripe base (e*R + src_rank)*M, and E*R*M.
                                May be NULL in low-latency mode. */
  int32_t *rank_token_count; /* [R] distinct tokens sent to each rank (num_tokens_per_rank).
                                May be NULL. */
  uint8_t *is_token_in_rank; /* [T*R] 1 if token t sends to rank r, else 0. May be NULL. */
  int32_t *slot;             /* [T*K] receive row of pair (t,k); -1 if not sent. */
  int32_t *row_src;          /* Contiguous: [moe_recv_rows_worst] pair index t*K+k held by
                                each row in [0, offset[E]), -1 on alignment padding.
                                Low latency: [E*M], pair held by stripe row j of expert e at
                                e*M + j, -1 where empty. May be NULL. */
  int32_t *status;           /* [1] sticky MOE_STATUS_* bits. May be NULL. */
  int32_t *recv_stats;       /* [E] cumulative receive counts (Buffer.low_latency_dispatch,
                                cumulative_local_expert_recv_stats; rank r's local expert l
                                is entry r*L + l): every layout call adds count[e] to entry e.
                                The caller initialises it. May be NULL. */
} moe_layout_t;

/* ABI version (MOE_ABI_VERSION) of the loaded library. */
int moe_abi_version(void);

/* Static text for a MOE_OK / MOE_ERR_* code. */
const char *moe_strerror(int code);

/* Worst-case rows of the contiguous receive buffer: T*K + E*(A-1); -1 for an
 * invalid shape. Sizing the buffer this way needs no host read of the counts
 * (Buffer.dispatch, num_worst_tokens: no CPU sync, graph-capturable). */
int64_t moe_recv_rows_worst(const moe_shape *shape);

/* Rows of the union of the R low-latency receive buffers: each rank holds
 * [L, R*M, H] (Buffer.low_latency_dispatch, return value; sizing as in
 * Buffer.get_low_latency_rdma_size_hint), so all of them together are
 * E*R*M rows. -1 for invalid arguments. */
int64_t moe_ll_recv_rows(int32_t E, int32_t R, int32_t M);

/* Device workspace bytes that moe_layout / moe_ll_layout (and the layout +
 * dispatch calls) need for this shape: 0 for at most 1024 pairs, or at most
 * 4096 pairs with A = 1. (Low-latency calls ignore A but are asked for the
 * workspace of the shape as given.) */
size_t moe_layout_workspace_bytes(const moe_shape *shape);

/* Contiguous dispatch layout (Buffer.get_dispatch_layout and the layout half of
 * Buffer.dispatch).
 *   topk_idx [T*K] int64 device: expert of each pair, -1 = no selection.
 *   out: count, offset, slot required; the rest may be NULL.
 *   Result: count[e] = pairs with id e; offset[0] = 0,
 *   offset[e+1] = offset[e] + ceil(count[e]/A)*A; the j-th pair of expert e in
 *   pair order t*K+k gets slot offset[e] + j (stable, so the layout is unique);
 *   alignment padding rows are not written by dispatch.
 *   ws: device workspace of ws_bytes >= moe_layout_workspace_bytes(shape), may
 *   be NULL when that is 0. */
int moe_layout(const moe_shape *shape, const int64_t *topk_idx, const moe_layout_t *out,
               void *ws, size_t ws_bytes, hipStream_t stream);

/* Low-latency padded layout (Buffer.low_latency_dispatch): this GPU is source
 * rank src_rank with T <= M tokens. The j-th pair of expert e (pair order)
 * gets slot (e*R + src_rank)*M + j, a row of the [E, R*M, H] union of the R
 * receive buffers (rank e/L's buffer, local expert e%L, stripe src_rank).
 * out->count receives the per-expert receive counts min(pairs, M); pairs with
 * j >= M get slot -1 and set MOE_STATUS_LL_OVERFLOW. shape->A is ignored. */
int moe_ll_layout(const moe_shape *shape, int32_t M, int32_t src_rank, const int64_t *topk_idx,
                  const moe_layout_t *out, void *ws, size_t ws_bytes, hipStream_t stream);

/* Layout and dispatch in one call (Buffer.dispatch given topk_idx and no handle):
 * the same results as moe_layout followed by moe_dispatch -- every array of out
 * and every row of recv_x bit for bit -- and the same argument rules as those
 * two calls (shape->H is used). Batches of at most 4096 pairs with A = 1 run
 * as a single kernel in which each workgroup re-derives the layout from the
 * routing while its token rows load; other batches launch the layout kernels,
 * then the scatter. A slot at or past recv_rows sets MOE_STATUS_BAD_SLOT and is not
 * written. */
int moe_layout_dispatch(const moe_shape *shape, const int64_t *topk_idx, const moe_layout_t *out,
                        const uint16_t *x, uint16_t *recv_x, int64_t recv_rows, void *ws,
                        size_t ws_bytes, hipStream_t stream);

/* moe_layout_dispatch for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments without the workspace, the same results,
 * bit for bit. Batches that need a layout workspace (moe_layout_workspace_bytes
 * > 0) use a static array of MOE_STATIC_SCRATCH_BYTES that the library holds on
 * each GPU until the process ends; a shape that needs more returns
 * MOE_ERR_SCRATCH before anything is enqueued. Nothing is allocated or freed,
 * and nothing in the array needs clearing between calls. All calls on one GPU
 * share that array: calls that may overlap on one GPU (other streams, other
 * host threads without ordering) race on it and must be serialised, for
 * example on one stream. MOE_ERR_DEVICE if the array's address cannot be
 * looked up. */
int moe_layout_dispatch_static(const moe_shape *shape, const int64_t *topk_idx,
                               const moe_layout_t *out, const uint16_t *x, uint16_t *recv_x,
                               int64_t recv_rows, hipStream_t stream);

/* Low-latency layout and dispatch in one call: the same results as moe_ll_layout
 * followed by moe_dispatch (recv_rows is normally moe_ll_recv_rows(E, R, M)). */
int moe_ll_layout_dispatch(const moe_shape *shape, int32_t M, int32_t src_rank,
                           const int64_t *topk_idx, const moe_layout_t *out, const uint16_t *x,
                           uint16_t *recv_x, int64_t recv_rows, void *ws, size_t ws_bytes,
                           hipStream_t stream);

/* Per-expert load of the batch (ultraep GPU operations, Load computation):
 * load[e] = pairs with id e, e in [0, E). Ids outside [-1, E) set
 * MOE_STATUS_BAD_EXPERT. status may be NULL. */
int moe_expert_load(int32_t T, int32_t K, int32_t E, const int64_t *topk_idx, int32_t *load,
                    int32_t *status, hipStream_t stream);

/* Dispatch scatter (Buffer.dispatch / Buffer.low_latency_dispatch with bf16 x):
 * recv_x[slot[t*K+k]] = x[t] bit for bit, for every pair with slot != -1.
 *   x [T*H] bf16, slot [T*K] (from moe_layout or moe_ll_layout),
 *   recv_x [recv_rows*H] bf16. Rows no pair maps to are left untouched.
 *   status may be NULL. */
int moe_dispatch(const moe_shape *shape, const uint16_t *x, const int32_t *slot,
                 uint16_t *recv_x, int64_t recv_rows, int32_t *status, hipStream_t stream);

/* Combine (Buffer.low_latency_combine: reduce with weights; Buffer.combine with
 * topk_weights = NULL is the plain sum):
 *   out[t] = bf16_rne( sum over k = 0..K-1 with slot != -1 of w[t*K+k] * y[slot[t*K+k]] )
 * summed in float in ascending k, every product and sum rounded to float
 * (no fused multiply-add), starting from +0; a token with no valid pair gets +0.
 *   y [recv_rows*H] bf16 (expert outputs, same row layout as recv_x),
 *   topk_weights [T*K] f32 or NULL for all ones, out [T*H] bf16,
 *   out_f32 [T*H] f32 (the unrounded sums) or NULL. status may be NULL. */
int moe_combine(const moe_shape *shape, const uint16_t *y, int64_t recv_rows,
                const int32_t *slot, const float *topk_weights, uint16_t *out, float *out_f32,
                int32_t *status, hipStream_t stream);

/* Combine with an active-rank mask (the NIXL EP change notes, "Combine active
 * rank mask optimization": the combine loops check each destination rank's
 * mask entry). As moe_combine, except that a pair whose expert e lives on a
 * masked rank -- rank_mask[e / L] != 0, L = E/R -- contributes nothing (and a
 * bad slot on such a pair is not reported): the masked rank's expert output is
 * treated as absent.
 *   topk_idx [T*K] int64: the routing the slots were made from;
 *   rank_mask [R] int32: nonzero = masked. Both device memory, read with
 *   plain loads (the mask is data written before the launch). */
int moe_combine_masked(const moe_shape *shape, const uint16_t *y, int64_t recv_rows,
                       const int32_t *slot, const int64_t *topk_idx, const float *topk_weights,
                       const int32_t *rank_mask, uint16_t *out, float *out_f32, int32_t *status,
                       hipStream_t stream);

/* ---------------------------------------------------------------------
 * Normal-mode dispatch: one receive row per (token, rank reached)
 * (Buffer.dispatch with is_token_in_rank / num_tokens_per_rank, returning
 * recv_topk_idx, recv_topk_weights and the per-expert receive counts;
 * Buffer.combine, which adds the rows back without weights). The R ranks'
 * receive buffers are one buffer: rank r owns rows
 * [rank_offset[r], rank_offset[r+1]), its tokens in ascending order.
 * Needs R <= 64.
 * ------------------------------------------------------------------- */
typedef struct {
  int32_t *rank_slot;         /* [T*R] row of (t, r), -1 if token t reaches no expert on r */
  int32_t *rank_offset;       /* [R+1] first row of each rank; rank_offset[R] = rows used */
  int32_t *recv_src;          /* [recv_cap] token held by each row. May be NULL. */
  int64_t *recv_topk_idx;     /* [recv_cap*K] per row: the rank-local id e - r*L of each
                                 selected expert that lives on the row's rank, -1 otherwise.
                                 May be NULL. */
  float *recv_topk_weights;   /* [recv_cap*K] the weight where the id is local, else 0.
                                 May be NULL (needs topk_weights when set). */
  int32_t *recv_expert_count; /* [E] pairs per expert rounded up to shape->A (the receive
                                 count of each local expert). May be NULL. */
  int32_t *status;            /* [1] sticky MOE_STATUS_* bits. May be NULL. */
} moe_rank_layout_t;

/* Worst-case rows of the normal-mode receive buffer: T * min(K, R). */
int64_t moe_rank_recv_rows_worst(const moe_shape *shape);

/* Normal-mode layout. topk_idx [T*K] int64; topk_weights [T*K] f32 or NULL.
 * recv_cap = rows the recv_* arrays hold (normally moe_rank_recv_rows_worst);
 * a row at or past it sets MOE_STATUS_BAD_SLOT and gets rank_slot -1. */
int moe_rank_layout(const moe_shape *shape, const int64_t *topk_idx, const float *topk_weights,
                    const moe_rank_layout_t *out, int64_t recv_cap, hipStream_t stream);

/* Normal-mode dispatch: recv_x[rank_slot[t*R + r]] = x[t] for every row,
 * bit for bit; rows no token maps to are left untouched. */
int moe_rank_dispatch(const moe_shape *shape, const uint16_t *x, const int32_t *rank_slot,
                      uint16_t *recv_x, int64_t recv_rows, int32_t *status, hipStream_t stream);

/* Normal-mode layout and dispatch in one call (Buffer.dispatch in normal
 * mode): the results of moe_rank_layout followed by moe_rank_dispatch, bit for
 * bit, including the status bits (out->status). Batches of at most 1024
 * tokens with K <= 8 take one launch that derives each token's rows while its
 * row is loaded; larger ones take the two launches. x [T*H] bf16 and recv_x
 * [recv_rows*H] are 16-byte aligned. */
int moe_rank_layout_dispatch(const moe_shape *shape, const int64_t *topk_idx,
                             const float *topk_weights, const moe_rank_layout_t *out,
                             int64_t recv_cap, const uint16_t *x, uint16_t *recv_x,
                             int64_t recv_rows, hipStream_t stream);

/* Normal-mode combine (Buffer.combine, addition without weights):
 *   out[t] = bf16_rne( sum over r = 0..R-1 with rank_slot[t*R + r] != -1 of y[row] )
 * in float, ascending r, from +0 (out_f32 [T*H] receives the float sums, or
 * NULL). With out_topk_weights [T*K] (and recv_topk_weights [recv_rows*K]),
 * also out_topk_weights[t*K + k] = sum over the same rows of
 * recv_topk_weights[row*K + k], ascending r: the original weights come back. */
int moe_rank_combine(const moe_shape *shape, const uint16_t *y, int64_t recv_rows,
                     const int32_t *rank_slot, const float *recv_topk_weights, uint16_t *out,
                     float *out_f32, float *out_topk_weights, int32_t *status,
                     hipStream_t stream);

/* Replica plan (ultraep GPU operations, Placement planning): the C most loaded
 * experts (load descending, ties to the lower id) get a second physical
 * replica. Rank r holds L' = L + C/R physical experts: r*L' + l (l < L) is the
 * primary of logical expert r*L + l, and the i-th hottest expert's replica is
 * (i mod R)*L' + L + i/R.
 *   load [E] int32 (e.g. from moe_expert_load); outputs replica_count [E]
 *   (1 or 2), replica_phys [E*2] (primary, replica or -1), phys_to_logical [E+C].
 *   Needs E <= 1024, 0 <= C <= E, C % R == 0. */
int moe_plan_replicas(int32_t E, int32_t R, int32_t C, const int32_t *load,
                      int32_t *replica_count, int32_t *replica_phys, int32_t *phys_to_logical,
                      hipStream_t stream);

/* Routing expansion (ultraep GPU operations, Routing expansion): logical
 * routing -> physical routing. The pair (t,k) on expert e uses replica
 * t mod replica_count[e]: phys_idx[t*K+k] = replica_phys[2e + t mod count];
 * -1 stays -1. Entries that fall outside [0, E_phys) set MOE_STATUS_BAD_REPLICA
 * and give -1. phys_idx [T*K] int64 can feed moe_layout with E = E_phys.
 * Needs 1 <= E <= 1024. */
int moe_reroute(int32_t T, int32_t K, int32_t E, const int64_t *topk_idx,
                const int32_t *replica_count, const int32_t *replica_phys, int32_t E_phys,
                int64_t *phys_idx, int32_t *status, hipStream_t stream);

/* ---------------------------------------------------------------------
 * FP8 dispatch (Buffer.low_latency_dispatch with use_fp8, round_scale and
 * use_ue8m0, and its returns; Buffer.dispatch with x given as a tuple of
 * float8_e4m3fn rows and float scales).
 *
 * The cast, per token row and per group of 128 channels:
 *   amax  = the group's largest |x|, taken as at least 1e-4;
 *   scale = amax / 448 (float, correctly rounded; 448 is the largest finite
 *           E4M3 value); with MOE_FP8_ROUND_SCALE rounded up to the next
 *           power of two;
 *   code  = E4M3 (OCP "fn" encoding: no infinity) nearest to x / scale
 *           (float division, ties to even, saturating at 448; the sign is
 *           kept, so -0 gives 0x80);
 * so x ~= value(code) * scale. With MOE_FP8_UE8M0 a power-of-two scale is
 * stored as its biased exponent byte (scale = 2^(byte - 127)), groups
 * 4w..4w+3 in bytes 0..3 (low to high) of int32 word w. x must be finite:
 * a NaN or infinity gives unspecified codes and scale for its group.
 * H must be a multiple of 128 (of 512 with MOE_FP8_UE8M0); flags is 0,
 * MOE_FP8_ROUND_SCALE or MOE_FP8_ROUND_SCALE | MOE_FP8_UE8M0, optionally
 * OR MOE_FP8_SCALE_ROWS; anything else returns MOE_ERR_FLAGS. Code and bf16 row pointers must be 16-byte aligned,
 * scale pointers 4-byte aligned.
 * ------------------------------------------------------------------- */

/* The cast alone, row-major: q [T*H] E4M3 codes; scale [T*H/128] float, or
 * with MOE_FP8_UE8M0 [T*H/512] int32 words (MOE_FP8_SCALE_ROWS has no effect
 * here). Produces the (codes, scales) tuple that moe_dispatch_fp8 takes. */
int moe_quantize_fp8(int32_t T, int32_t H, const uint16_t *x, uint8_t *q, void *scale,
                     int32_t flags, hipStream_t stream);

/* Low-latency layout and FP8 dispatch in one call (Buffer.low_latency_dispatch,
 * use_fp8 = True): the layout arrays exactly as moe_ll_layout, and for every
 * pair with a slot, the token's codes in row slot of recv_q [recv_rows*H] and
 * its scales in the column-major scale tensor of the page's return value:
 * recv_scale is [E][H/128][R*M] float -- the scale of group g for row i of
 * expert e's R*M rows (slot = e*R*M + i) is at (e*(H/128) + g)*R*M + i -- or,
 * with MOE_FP8_UE8M0, [E][H/512][R*M] int32 words placed the same way.
 * recv_rows <= E*R*M (normally moe_ll_recv_rows(E, R, M)). With
 * MOE_FP8_SCALE_ROWS (an option of this library, not of the page) the scales
 * are row-major instead: [recv_rows][H/128] floats or [recv_rows][H/512]
 * words, the scales of row slot at slot*(H/128) + g. The column-major format
 * spreads each pair's scales over H/128 cache lines shared with the expert's
 * other tokens; the row-major one keeps them in contiguous bytes of the row,
 * which is cheaper to write. Entries no pair maps to are left untouched. */
int moe_ll_layout_dispatch_fp8(const moe_shape *shape, int32_t M, int32_t src_rank,
                               const int64_t *topk_idx, const moe_layout_t *out,
                               const uint16_t *x, uint8_t *recv_q, void *recv_scale,
                               int64_t recv_rows, int32_t flags, void *ws, size_t ws_bytes,
                               hipStream_t stream);

/* The FP8 low-latency scatter given the slots of moe_ll_layout (same output
 * layout as moe_ll_layout_dispatch_fp8; M is the per-rank capacity the slots
 * were made with). A slot outside [-1, recv_rows) sets MOE_STATUS_BAD_SLOT
 * and is skipped. status may be NULL. */
int moe_ll_dispatch_fp8(const moe_shape *shape, int32_t M, const uint16_t *x,
                        const int32_t *slot, uint8_t *recv_q, void *recv_scale,
                        int64_t recv_rows, int32_t flags, int32_t *status, hipStream_t stream);

/* Dispatch of an already cast tuple (Buffer.dispatch, x = (E4M3 [T, H],
 * float [T, H/128])): for every pair with slot != -1, row slot of
 * recv_q [recv_rows*H] receives the token's codes and row slot of
 * recv_scale [recv_rows*H/128] its scales, bit for bit (row-major, like the
 * input). Rows no pair maps to are left untouched. status may be NULL. */
int moe_dispatch_fp8(const moe_shape *shape, const uint8_t *x_q, const float *x_scale,
                     const int32_t *slot, uint8_t *recv_q, float *recv_scale,
                     int64_t recv_rows, int32_t *status, hipStream_t stream);

/* Replica weight sync (ultraep Overview: replicas get synchronized weights
 * before expert execution; GPU operations: Replica weight sync). w [E_phys*S]
 * bf16 is the physical expert buffer, expert p's S parameters at p*S; each
 * logical expert's master weights sit in its primary slot. For every expert e
 * with replica_count[e] == 2, the replica slot replica_phys[2e+1] receives a
 * bit copy of the primary slot replica_phys[2e]. S % 8 == 0; w 16-byte
 * aligned. Table entries outside [0, E_phys) set MOE_STATUS_BAD_REPLICA and
 * that expert is skipped. (Restoring the weights after backward needs no data
 * movement: the replica slots are scratch.) */
int moe_replica_weight_sync(int32_t E, int32_t E_phys, int64_t S, const int32_t *replica_count,
                            const int32_t *replica_phys, uint16_t *w, int32_t *status,
                            hipStream_t stream);

/* Replica gradient reduction (ultraep Overview: replica gradients are reduced
 * during backward; GPU operations: Replica gradient reduction). g [E_phys*S]
 * f32: for every expert e with a second replica,
 * g[prim*S + i] = g[prim*S + i] + g[rep*S + i] (one float add), leaving the
 * master gradient in the primary slot. Same argument rules as
 * moe_replica_weight_sync. */
int moe_replica_grad_reduce(int32_t E, int32_t E_phys, int64_t S, const int32_t *replica_count,
                            const int32_t *replica_phys, float *g, int32_t *status,
                            hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_EP_H */
