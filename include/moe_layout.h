/*
 * moe_layout.h -- C ABI of the MI355X (gfx950) MoE token layout / dispatch /
 * combine library (libmoe_layout.so).
 *
 * What it computes is the data-parallel hot path of expert-parallel token
 * exchange, on one GPU: the P expert-parallel ranks are P virtual partitions
 * of one receive buffer in HBM.
 *
 *   "Add an opt-in DeepEP transport for the AutoEP expert all-to-all"
 *   (DeepSpeed PR), sections "Why" and "Scope and safety": the exchange
 *   receives tokens before their top-k expansion, together with their expert
 *   ids and weights; it replicates each token to the ranks that host its
 *   experts, presents the arrivals grouped by expert, and its combine forms
 *   the weighted top-k sum in token order again.  Backward needs no entry
 *   points of its own: each backward pass is the opposite row movement, run
 *   on the handle the forward dispatch produced.  The review-fix commit on
 *   that page makes dispatch hand back the received weights and makes both
 *   backward passes return the router-weight gradient.
 *
 *   "[MoE] Apply router scores before W2 projection" (torchtitan issue),
 *   sections "Motivation" and "Implementation": when the router scores are
 *   absorbed into W2's input, dispatch also returns each receive row's score
 *   in the rows' expert-major order, the scaling is done in float32 and
 *   rounded back to the row type, and the combine is a plain sum.
 *
 * Conventions (every entry point):
 *   - All tensor pointers are DEVICE pointers; the caller owns every buffer,
 *     the workspace and the stream.  Row-major, contiguous.
 *   - Calls are stream-ordered on `stream` and never block the host, except
 *     moe_handle_check, which synchronises the stream.
 *   - Arguments are validated on the host before anything is launched; a
 *     rejected call launches nothing and returns a negative MOE_ERR_* code.
 *   - T = tokens, K = top-k, E = experts, P = partitions (virtual EP ranks),
 *     H = row width in elements, R = receive rows: T*K, or T*K + E*(m-1)
 *     for a handle whose expert segments are padded to a multiple of m
 *     (moe_handle_create_padded; moe_recv_capacity returns R).
 *   - Expert e belongs to partition e / (E/P); E must be a multiple of P.
 *   - Element types: MOE_F32 (float) or MOE_BF16 (bfloat16 bits).  Every
 *     row is a whole number of 16-byte chunks: H*sizeof(elem) % 16 == 0.
 *   - Floating-point contract: products and sums in IEEE float32, each
 *     rounded on its own (no fused multiply-add); sums over k run in k order
 *     from +0.0; bfloat16 results are rounded to nearest, ties to even.
 *     Router-weight gradients use a fixed segment-major order (see
 *     moe_combine_bwd), so results are bitwise reproducible.
 */
#ifndef MOE_LAYOUT_H
#define MOE_LAYOUT_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define MOE_OK                 0
#define MOE_ERR_INVALID_ARG   -1  /* null pointer, negative size, missing companion argument */
#define MOE_ERR_SHAPE         -2  /* K < 1, K > E, E % P != 0, H*elem % 16 != 0, H < 1 */
#define MOE_ERR_UNSUPPORTED   -3  /* unknown dtype/itype, P > 64, E > 1024, K > 32, T*K >= 2^31 */
#define MOE_ERR_ALIGNMENT     -4  /* row pointers not 16-byte aligned, others not elem-aligned */
#define MOE_ERR_WORKSPACE     -5  /* workspace smaller than moe_workspace_size() */
#define MOE_ERR_HANDLE        -6  /* bad handle, or a data call before moe_layout */
#define MOE_ERR_HIP           -7  /* a HIP runtime call failed */
#define MOE_ERR_SCRATCH       -8  /* moe_layout_noalloc: the histogram exceeds its static scratch */

/* ---- element and index types ------------------------------------------- */
enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 };
enum moe_itype { MOE_I32 = 0, MOE_I64 = 1 };

/* ---- limits -------------------------------------------------------------- */
#define MOE_MAX_K 32
#define MOE_MAX_E 1024
#define MOE_MAX_P 64

/* ---- device status bits (read with moe_handle_check) --------------------- */
#define MOE_STATUS_BAD_EXPERT   1  /* a topk_idx entry outside [0, E) */
#define MOE_STATUS_BAD_POSITION 2  /* a data kernel met a receive row outside [0, R) */

/* ---- handle fields (moe_handle_field) ------------------------------------ */
enum moe_field {
  MOE_FIELD_NUM_TOKENS_PER_EXPERT = 0, /* int32 [E]   (t,k) pairs per expert               */
  MOE_FIELD_NUM_TOKENS_PER_RANK   = 1, /* int32 [P]   distinct tokens per partition         */
  MOE_FIELD_IS_TOKEN_IN_RANK      = 2, /* uint8 [T,P] 1 if any of t's experts is on r       */
  MOE_FIELD_EXPERT_OFFSET         = 3, /* int32 [E+1] exclusive prefix of expert segment
                                          rows (counts, padded to the handle's multiple) */
  MOE_FIELD_RANK_OFFSET           = 4, /* int32 [P+1] first receive row of each partition   */
  MOE_FIELD_SEND_OFFSET           = 5, /* int32 [P+1] exclusive prefix of num_tokens_per_rank */
  MOE_FIELD_TOKEN_SLOT            = 6, /* int32 [T,P] t's slot in r's send list, or -1      */
  MOE_FIELD_RECV_POS              = 7, /* int32 [T,K] receive row of pair (t,k)            */
  MOE_FIELD_RECV_TOKEN            = 8, /* int32 [R]   token of each receive row, -1 if none */
  MOE_FIELD_RECV_K                = 9, /* int32 [R]   k of each receive row, -1 if none     */
  MOE_FIELD_STATUS                = 10,/* int32 [1]   device status bits                   */
  MOE_FIELD_SEND_TOKEN            = 11 /* int32 [T*min(K,P)] token of each send row
                                          (rows >= send_offset[P] unspecified)          */
};

/* Optional launch knobs; zero means "library default" except for
 * nontemporal, whose default applies when the struct is NULL.  A row is cut
 * into 16-byte chunks and the chunks into segments of 64 (one wavefront
 * access); the row kernels run one wavefront per (token, segment group).   */
typedef struct moe_tuning {
  int chunks_per_lane;  /* consecutive segments per wavefront, i.e. chunks of one row each
                           lane keeps in flight: 0 (= 1), 1, 2 or 4                        */
  int nontemporal;      /* 0: default loads/stores; 1: receive-row loads and stores
                           marked non-temporal; 2 (default): token-row stores too    */
  int waves_per_block;  /* wavefronts per workgroup of the row kernels: 0 (= 4; the
                           LDS-staged gather takes 1 when a row is whole segments and
                           their number is not a multiple of 8), 1, 2, 4, 8              */
  int layout_pairs;     /* (t,k) pairs per layout tile: 0 (= 512), 512, 1024, 2048, 4096      */
  int gather_mode;      /* receive rows of the gathers (moe_combine, unscaled moe_dispatch_bwd):
                           0 (default) by row width: staged in LDS by direct loads for rows
                           of 4 KiB and wider, in registers otherwise; 1 always LDS-staged;
                           2 always in registers                                         */
} moe_tuning;

typedef struct moe_handle_s* moe_handle_t;

/* Bytes of device workspace a layout of this shape needs (pure host).
 * Returns MOE_ERR_* on an invalid shape (same rules as moe_layout).  The
 * _padded form is for handles created with that pad_multiple.  A workspace
 * sized for the largest T serves every smaller T: calls with a varying
 * number of tokens need no new allocation. */
int moe_workspace_size(int64_t T, int K, int E, int P, size_t* bytes);
int moe_workspace_size_padded(int64_t T, int K, int E, int P, int pad_multiple, size_t* bytes);

/* Create / destroy a handle.  `tuning` may be NULL.  Host memory only: the
 * handle records views into the caller's workspace, never owns device memory. */
int moe_handle_create(moe_handle_t* out, const moe_tuning* tuning);
int moe_handle_destroy(moe_handle_t h);

/* A handle whose layouts pad every expert's segment of receive rows to a
 * multiple of pad_multiple (1..1024; 1 = moe_handle_create), fixed for the
 * handle's life (the DiffusionGemma dispatcher page lists pad_multiple as
 * set once at construction).  Segment e holds its n_e pairs, in the usual
 * order, then pad_multiple*ceil(n_e/pad_multiple) - n_e padding rows, so
 * every expert_offset is a multiple of pad_multiple (grouped-GEMM tiles).
 * Calls that write receive rows (moe_dispatch, moe_expand, the grad_y rows
 * of moe_combine_bwd) write zero rows there, and zero scores when they write
 * scores (the zero-sentinel scores of the padded permute, "[MoE] Apply
 * router scores before W2 projection", "Implementation"); rows past
 * expert_offset[E] are not written.  Calls that read receive rows never
 * read padding.  Receive buffers hold R = T*K + E*(pad_multiple-1) rows. */
int moe_handle_create_padded(moe_handle_t* out, const moe_tuning* tuning, int pad_multiple);

/* Layout of one routing decision (method steps: counts, offsets, stable
 * positions).  Fills every handle field inside `workspace`.
 *
 *   topk_idx   [T,K] int32 (itype MOE_I32) or int64 (MOE_I64), device.
 *   workspace  device, >= moe_workspace_size(T,K,E,P) bytes (the _padded
 *              size for a padded handle), 256-byte aligned; it holds the
 *              handle's arrays and must outlive every later call on this
 *              handle.  MOE_ERR_WORKSPACE if it is smaller.
 *
 * Definitions (a stable counting sort of the (t,k) pairs by expert id):
 *   recv_pos[t,k] = expert_offset[e] + #{(t',k') < (t,k) lexicographically
 *                    with topk_idx[t',k'] == e},  e = topk_idx[t,k];
 *   expert_offset[e] = sum over e' < e of n_e' (rounded up to the handle's
 *                    pad multiple, see moe_handle_create_padded);
 *   so rows are grouped by expert in ascending id (hence by partition), and
 *   inside an expert by token, then k.  The order depends on the routing
 *   only, so an activation-checkpoint replay of the same routing reproduces
 *   every position ("perf(dllm): use the DeepEP dispatcher in the
 *   DiffusionGemma recipes", section "Why hybridep + activation
 *   checkpointing fails", shows what a replay-nondeterministic dispatch does).
 *   token_slot[t,r] numbers the tokens with is_token_in_rank[t,r] in
 *   increasing t (a token is sent once per partition, not once per expert:
 *   the deduplication of the DeepSpeed transport PR's "Why" section).
 *
 * T = 0 is valid and yields an empty layout; every data call on it returns
 * MOE_OK after its non-pointer checks, reads and writes nothing, and accepts
 * NULL for any array (an empty tensor's data pointer).  Entries of topk_idx outside
 * [0,E) are an input error detected on the device: MOE_STATUS_BAD_EXPERT is
 * set and those pairs are placed after the last expert's rows (so every
 * position stays inside [0,R)); the other fields are then unspecified.
 * Duplicate ids within a token are accepted and ordered by k.
 * The handle must not be used on two streams at once.                      */
int moe_layout(moe_handle_t h, const void* topk_idx, int itype, int64_t T, int K,
               int E, int P, void* workspace, size_t workspace_bytes,
               hipStream_t stream);

/* moe_layout for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, results and handle as moe_layout; the difference is where the
 * layout's scratch lives.  moe_layout keeps its per-tile histogram in the
 * caller's workspace; this call keeps it in a static array inside the
 * library, one per GPU, held until the process ends, so the workspace only
 * has to hold the handle's arrays (moe_workspace_size() bytes always
 * suffice; the histogram section at their end is not touched).  The call
 * itself allocates nothing: no hipMalloc, hipFree or allocating library
 * routine.  Limit: the histogram, (E+1+P) * (tiles+1) * 4 bytes, must fit
 * in 2 MiB (tiles: T*K/512, at most 128 until a tile reaches its cap of
 * 2048 tokens at K = 8, then T/2048); a larger shape is refused on the host
 * with MOE_ERR_SCRATCH, before any launch.  Every call
 * on one GPU shares that GPU's array: layouts that overlap in time on one
 * GPU (two streams, or two host threads) race on it and must be ordered by
 * the caller; each call writes every histogram entry it reads, so nothing
 * has to be cleared between calls.                                        */
int moe_layout_noalloc(moe_handle_t h, const void* topk_idx, int itype, int64_t T, int K,
                       int E, int P, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* Forward dispatch: recv[recv_pos[t,k], :] = x[t, :].
 * Defined by "Add an opt-in DeepEP transport for the AutoEP expert
 * all-to-all", sections "What this adds" and "Scope and safety" (tokens
 * before top-k expansion in, arrivals grouped by expert out), with the
 * received weights of its review fix (recv_scores) and the float32 row
 * scaling of "[MoE] Apply router scores before W2 projection",
 * "Implementation" (scale_rows).
 *
 *   x             [T,H] dtype, 16-byte aligned.
 *   topk_weights  [T,K] float32 or NULL; required when scale_rows or
 *                 recv_scores is given.
 *   scale_rows    0: copy rows bit for bit.  1: scores absorbed before W2,
 *                 recv = round(float32(x[t]) * w[t,k]).
 *   recv          [R,H] dtype, 16-byte aligned (output).
 *   recv_scores   [R] float32 or NULL (output): recv_scores[recv_pos[t,k]] = w[t,k].
 * Each x row is read once and stored to its receive rows partition by
 * partition.                                                              */
int moe_dispatch(moe_handle_t h, const void* x, int dtype, int64_t H,
                 const float* topk_weights, int scale_rows, void* recv,
                 float* recv_scores, hipStream_t stream);

/* Forward combine: out[t] = round(sum_k w[t,k] * y[recv_pos[t,k]]), or the
 * plain sum when topk_weights is NULL (scores absorbed).  float32, k order.
 * Defined by "Add an opt-in DeepEP transport for the AutoEP expert
 * all-to-all", section "Scope and safety" (the combine reduces the weighted
 * sum back to token order), and "[MoE] Apply router scores before W2
 * projection", "Implementation" (a plain sum once the scores are absorbed).
 *   y [R,H], out [T,H] dtype, 16-byte aligned.
 * Errors: MOE_ERR_HANDLE before moe_layout; MOE_ERR_SHAPE / _ALIGNMENT /
 * _INVALID_ARG for a bad row width, pointer or missing array (checked on the
 * host, nothing launched); receive rows out of [0,R) set
 * MOE_STATUS_BAD_POSITION on the device and are skipped.                  */
int moe_combine(moe_handle_t h, const void* y, int dtype, int64_t H,
                const float* topk_weights, void* out, hipStream_t stream);

/* Backward of moe_combine (a dispatch of the output gradient), per
 * "Add an opt-in DeepEP transport for the AutoEP expert all-to-all",
 * section "Scope and safety" (the gradient of a combine is a dispatch on the
 * forward's handle) and the same page's review fix (the weight gradient is
 * returned, never dropped):
 *   grad_y[recv_pos[t,k]] = round(w[t,k] * grad_out[t])  (copy if no weights)
 *   grad_w[t,k] = <grad_out[t], y[recv_pos[t,k]]>        (if grad_w != NULL)
 * grad_w needs topk_weights and y.  The dot product is float32 in a fixed
 * order: the row is cut into 16-byte chunks and the chunks into segments of
 * 64; each chunk's partial adds its element products in order from +0.0
 * (product rounded, then sum rounded); each segment folds its 64 partials
 * L[l] += L[l xor s] for s = 32,16,8,4,2,1 (absent chunks are +0.0) and
 * takes partial 0; the result adds the segment values in order from +0.0.
 * Needs ceil(H*elem/1024) * K * 4 <= 65536 (else MOE_ERR_UNSUPPORTED).
 *   grad_out [T,H], y [R,H], grad_y [R,H] dtype; grad_w [T,K] float32.     */
/* grad_y may be NULL when grad_w is given: then only the router-weight
 * gradient is computed (the rows of a staged backward come from moe_send and
 * moe_expand). */
int moe_combine_bwd(moe_handle_t h, const void* grad_out, int dtype, int64_t H,
                    const float* topk_weights, const void* y, void* grad_y,
                    float* grad_w, hipStream_t stream);

/* Backward of moe_dispatch (a combine of the receive-row gradient), per
 * "Add an opt-in DeepEP transport for the AutoEP expert all-to-all",
 * section "Scope and safety" (the gradient of a dispatch is a combine on the
 * forward's handle); with scores absorbed, "[MoE] Apply router scores before
 * W2 projection", "Implementation" and "Tests and verifications" (the score
 * gradient flows through W2's input scaling):
 *   grad_x[t] = round(sum_k [w[t,k] *] grad_recv[recv_pos[t,k]])
 *   grad_s[t,k] = <grad_recv[recv_pos[t,k]], x[t]>        (if grad_s != NULL)
 * Pass topk_weights iff the forward dispatch scaled its rows (the scaling is
 * differentiated straight through its rounding).  grad_s needs topk_weights
 * and x; same dot order and size limit as moe_combine_bwd.
 *   grad_recv [R,H], x [T,H], grad_x [T,H] dtype; grad_s [T,K] float32.   */
/* grad_x may be NULL when grad_s is given: then only the score gradient is
 * computed (the rows of a staged backward come from moe_reduce_partitions and
 * moe_combine_partitions). */
int moe_dispatch_bwd(moe_handle_t h, const void* grad_recv, int dtype, int64_t H,
                     const float* topk_weights, const void* x, void* grad_x,
                     float* grad_s, hipStream_t stream);

/* ---- staged exchange ------------------------------------------------------
 * The payload a cross-GPU transport moves, staged in one GPU's HBM: a send
 * buffer with one row per (token, destination partition) pair, at row
 * send_offset[r] + token_slot[t,r] ("Add an opt-in DeepEP transport for the
 * AutoEP expert all-to-all", section "Why": a token is sent once per
 * destination rank, not once per selected expert; arrivals are grouped by
 * expert; the combine reduces back to token order).  send_offset[P] rows are
 * used; buffers take a capacity of at least moe_send_capacity() rows, known
 * on the host without a device sync.  Staged dispatch = moe_send +
 * moe_expand (bitwise equal to moe_dispatch); staged combine =
 * moe_reduce_partitions + moe_combine_partitions (its own summation order,
 * below).  A staged backward uses the same calls: the combine's backward is
 * moe_send + moe_expand of the output gradient (scaled), the dispatch's is
 * moe_reduce_partitions + moe_combine_partitions of the receive-row gradient;
 * the router-weight gradients come from moe_combine_bwd / moe_dispatch_bwd
 * with NULL row outputs.
 *
 * Row pointers 16-byte aligned, dtype as in the other calls; send_rows is
 * the caller's buffer capacity in rows (MOE_ERR_SHAPE if below
 * moe_send_capacity()).                                                    */

/* Rows a send buffer must hold: T * min(K, P), an upper bound of send_offset[P]. */
int moe_send_capacity(moe_handle_t h, int64_t* rows);

/* Rows a receive buffer (recv, y, grad_y, grad_recv, recv_scores) holds for
 * the current layout: T*K, plus E*(pad_multiple-1) on a padded handle.
 * Known on the host; no device sync. */
int moe_recv_capacity(moe_handle_t h, int64_t* rows);

/* Source side: send[send_offset[r] + token_slot[t,r]] = x[t] for every
 * partition r of token t (each x row is read once).  x [T,H].            */
int moe_send(moe_handle_t h, const void* x, int dtype, int64_t H, void* send, int64_t send_rows,
             hipStream_t stream);

/* Receiver side: recv[recv_pos[t,k]] = send[send_offset[r] + token_slot[t,r]]
 * for every pair whose expert is on partition r (each send row is read
 * once); scale_rows, recv_scores and padding rows as in moe_dispatch.
 * recv [R,H].                                                             */
int moe_expand(moe_handle_t h, const void* send, int dtype, int64_t H, int64_t send_rows,
               const float* topk_weights, int scale_rows, void* recv, float* recv_scores,
               hipStream_t stream);

/* Receiver side of the two-level combine: for every (token, partition) send
 * row, partial = round(sum [w[t,k] *] y[recv_pos[t,k]]) over the token's k
 * with an expert on that partition, in k order, float32 from +0.0 (product
 * and sum rounded on their own); rounded to the row type, the type a
 * transport sends.  y [R,H]; partial [send_rows,H]; weights may be NULL
 * (plain sum).                                                             */
int moe_reduce_partitions(moe_handle_t h, const void* y, int dtype, int64_t H,
                          const float* topk_weights, void* partial, int64_t send_rows,
                          hipStream_t stream);

/* Source side: out[t] = round(sum of float32(partial[send row of (t,r)]))
 * over t's partitions r in ascending order, float32 from +0.0.  out [T,H]. */
int moe_combine_partitions(moe_handle_t h, const void* partial, int dtype, int64_t H,
                           int64_t send_rows, void* out, hipStream_t stream);

/* Device pointer and byte size of one handle field (no synchronisation). */
int moe_handle_field(moe_handle_t h, int field, void** dev_ptr, size_t* bytes);

/* Shape recorded by the last moe_layout on this handle. */
int moe_handle_dims(moe_handle_t h, int64_t* T, int* K, int* E, int* P);

/* Synchronises `stream`, then reads the device status word (MOE_STATUS_* bits). */
int moe_handle_check(moe_handle_t h, hipStream_t stream, int* device_status);

/* ---- CU budget -------------------------------------------------------------
 * A stream whose kernels may run only on compute units [cu_first, cu_first +
 * cu_count) of the current device (a hardware CU mask; default priority).
 * The exchange calls issued on it use at most that many CUs, and a GEMM on a
 * stream with the other CUs runs beside them: the analogue of the SM budget
 * of the pages' transport kernels ("Add an opt-in DeepEP transport for the
 * AutoEP expert all-to-all", section "Choosing the SM budget": too few SMs
 * slow the exchange itself and too many slow the GEMMs beside it, so the
 * budget is a whole-step trade-off; the page's follow-up work lists
 * overlapping the exchange with compute).  CU
 * indices are the HIP runtime's, numbered round-robin over the XCDs, so a
 * range of consecutive indices spreads evenly over them; the runtime refuses
 * a mask that leaves an XCD without a CU, so cu_count is at least the XCD
 * count (8 on MI355X).  MOE_ERR_INVALID_ARG for a NULL out, cu_first < 0 or
 * cu_count < 1; MOE_ERR_SHAPE if the range passes the device's CU count or
 * holds fewer CUs than XCDs; MOE_ERR_HIP if the runtime refuses.  Destroy
 * with moe_stream_destroy.                                                 */
int moe_stream_create_cu_budget(int cu_first, int cu_count, hipStream_t* out);
int moe_stream_destroy(hipStream_t stream);

/* Message for a status code (static string). */
const char* moe_strerror(int status);

/* Library version string. */
const char* moe_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_LAYOUT_H */
