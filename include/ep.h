/*
 * ep.h -- C ABI of libep: MoE expert-parallel dispatch and combine on one
 * AMD Instinct MI355X (gfx950), with the EP ranks of a multi-node job laid
 * out as buffer partitions in the GPU's own HBM.
 *
 * The API follows the two-level resource model and the call sequence of
 * NCCL-EP ("NCCL EP paper notes", lpnh.cn: core functions, tensor
 * abstraction and tensor layouts): a group created once per model holds the
 * algorithm mode and all communication buffers; a handle created per forward
 * pass from topk_idx holds the routing state shared by the matching dispatch
 * and combine.  The data path is DeepEP's ("NVSHMEM and DeepEP: GPU-initiated
 * communication"): node-limited routing, FP8 payload with one fp32 scale per
 * 128 elements, fixed slots in the low-latency (LL) mode and node-
 * deduplicated same-position rows followed by an intra-node forward in the
 * high-throughput (HT) mode, and a BF16 weighted combine.
 *
 * Conventions
 *  - Every pointer inside an ep_tensor_t is a device pointer unless a
 *    function says otherwise; the caller owns it and keeps it alive until the
 *    work enqueued on the stream has finished.
 *  - Every operation is enqueued on the caller's HIP stream (passed as
 *    ep_stream_t, i.e. a hipStream_t; NULL is the default stream) and returns
 *    without waiting, except the functions documented as blocking.
 *  - A group, and every handle made from it, is used from one stream at a
 *    time; the library takes no locks.
 *  - Arguments are validated on the host before any HIP call; a rejected call
 *    enqueues nothing.  Routing entries are checked on the device and
 *    reported through the group's device error word (ep_get_device_error).
 *  - Nothing throws, aborts or exits across this boundary.
 */
#ifndef EP_H
#define EP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ----------------------------------------------------------------------- */
/* Status codes                                                              */
/* ----------------------------------------------------------------------- */
typedef enum {
    EP_OK = 0,
    EP_ERR_INVALID_ARGUMENT = 1, /* bad config, descriptor, handle or size   */
    EP_ERR_CAPACITY = 2,         /* more tokens than max_tokens_per_rank, or
                                    no free handle slot                      */
    EP_ERR_OUT_OF_MEMORY = 3,    /* device allocation (or alloc_fn) failed    */
    EP_ERR_HIP = 4,              /* a HIP runtime call failed; see
                                    ep_last_hip_error()                      */
    EP_ERR_UNSUPPORTED = 5       /* valid but outside the library's limits    */
} ep_status_t;

/* Algorithm mode, chosen once at group creation (NCCL-EP: the group's
 * config selects HT or LL). */
typedef enum { EP_MODE_LL = 0, EP_MODE_HT = 1 } ep_mode_t;

/* HT stage-2 layout ("NVSHMEM and DeepEP", high-throughput mode: the
 * traffic study compares one copy per expert with one per destination GPU).
 *   PER_EXPERT: one row per valid (token, k), grouped by expert.
 *   PER_RANK:   one row per (token, distinct destination rank), grouped by
 *               rank, with the token's entries local to that rank (DeepEP's
 *               received top-k form); the experts' weighted partial sums come
 *               back per rank and the combine sums them. */
typedef enum { EP_HT_STAGE2_PER_EXPERT = 0, EP_HT_STAGE2_PER_RANK = 1 } ep_ht_stage2_t;

/* Element types (NCCL-EP tensor abstraction: FP32/BF16/FP16/FP8). */
typedef enum {
    EP_DTYPE_F32 = 0,
    EP_DTYPE_BF16 = 1,
    EP_DTYPE_F16 = 2,
    EP_DTYPE_FP8_E4M3 = 3, /* OCP E4M3 (max 448, no infinities)          */
    EP_DTYPE_I32 = 4,
    EP_DTYPE_U8 = 5        /* raw bytes (packed rows and messages)       */
} ep_dtype_t;

/* Semantic tag of a tensor (NCCL-EP's tensor tags; the page lists the
 * device-side receive counter twice, the second read here as the host-side
 * one). */
typedef enum {
    EP_TAG_NONE = 0,
    EP_TAG_TOKENS = 1,
    EP_TAG_TOPK_IDX = 2,
    EP_TAG_TOPK_WEIGHTS = 3,
    EP_TAG_SCALES = 4,
    EP_TAG_RECV_EXPERT_COUNTER_DEVICE = 5,
    EP_TAG_RECV_EXPERT_COUNTER_HOST = 6,
    EP_TAG_TOKENS_PER_EXPERT = 7
} ep_tensor_tag_t;

/* Bits of the device error word. */
#define EP_DEVERR_BAD_INDEX 1  /* a topk_idx entry outside [0, num_experts)  */
#define EP_DEVERR_DUP_INDEX 2  /* a topk_idx entry repeating an earlier one  */
#define EP_DEVERR_ROW_RANGE 4  /* combine: a row beyond expert_out's rows    */

/* An n-dimensional tensor descriptor (NCCL-EP's ncclNDTensor_t): element
 * type, up to 3 dimensions, strides in ELEMENTS, and a semantic tag.  The
 * innermost dimension must be contiguous (stride 1) and data 16-byte
 * aligned wherever a function says so. */
typedef struct {
    void *data;
    int32_t dtype;       /* ep_dtype_t      */
    int32_t ndim;        /* 1..3            */
    int64_t sizes[3];
    int64_t strides[3];
    int32_t tag;         /* ep_tensor_tag_t */
} ep_tensor_t;

/* A hipStream_t. */
typedef void *ep_stream_t;

/* Group configuration (NCCL-EP group config: mode, number of experts,
 * maximum tokens per rank, buffer sizing, custom allocator hooks).
 *
 * Topology: num_nodes x ranks_per_node EP ranks; rank r sits on node
 * r / ranks_per_node; expert e lives on rank e / (num_experts / R).  The
 * first num_src_ranks ranks are the sources whose tokens this GPU routes,
 * dispatches and combines (token i of a [num_src_ranks * T] batch belongs to
 * source rank i / T). */
typedef struct {
    int32_t mode;                /* ep_mode_t                                  */
    int32_t num_nodes;           /* N                                          */
    int32_t ranks_per_node;      /* G                                          */
    int32_t num_experts;         /* E, divisible by N*G                        */
    int32_t top_k;               /* K, 1..32                                   */
    int32_t max_nodes_per_token; /* M; 0 (or >= N) = no node limit             */
    int32_t hidden;              /* H, multiple of 128 for FP8, of 16 for BF16 */
    int32_t max_tokens_per_rank; /* T_max: LL slots per (expert, source)       */
    int32_t num_src_ranks;       /* S, 1..R                                    */
    int32_t payload;             /* EP_DTYPE_FP8_E4M3 or EP_DTYPE_BF16         */
    int32_t max_handles;         /* live handles at once; 0 means 2            */
    int32_t num_cus;             /* cap on CUs used by dispatch/combine; 0=all */
    int32_t ll_buffers;          /* LL receive buffers used in turn: 1 or 2;
                                    0 means 2 (double buffering, NCCL-EP LL) */
    int32_t ht_stage2;           /* ep_ht_stage2_t (HT only)                   */
    int32_t ht_buffers;          /* HT stage-row sets (stage-1 and stage-2 rows
                                    with metadata) used in turn: 1 or 2; 0
                                    means 1.  With 2 a dispatch may run while
                                    the previous handle's rows are read.     */
    /* Optional allocator hooks: both or neither.  alloc_fn returns device
     * memory of at least `bytes` bytes aligned to 256, or NULL. */
    void *(*alloc_fn)(size_t bytes, void *ctx);
    void (*free_fn)(void *ptr, void *ctx);
    void *alloc_ctx;
} ep_config_t;

typedef struct ep_group *ep_group_t;
typedef struct ep_handle *ep_handle_t;

/* ----------------------------------------------------------------------- */
/* Resources                                                                 */
/* ----------------------------------------------------------------------- */

/* Create a group (NCCL-EP ncclEpCreateGroup).  Validates the configuration
 * and allocates, once, every buffer the hot path writes, so that no call
 * below allocates device memory:
 *   LL: ll_buffers fixed-slot receive spaces, expert-major, E x S x T_max
 *       messages of (row + 16) bytes; rank r's partition is experts
 *       [r*E/R, (r+1)*E/R), i.e. a contiguous [E/R][S][T_max] block.
 *   HT: ht_buffers sets of stage-1 rows (one per token and destination
 *       node) and stage-2 rows (one per token and expert), each with
 *       structure-of-arrays metadata, sized for the worst case S*T_max tokens.
 *   Per handle slot: routing maps and counters for S*T_max tokens.
 * `stream` orders the initialisation.  On failure nothing stays allocated.
 * Errors: EP_ERR_INVALID_ARGUMENT (NULL pointers, inconsistent topology,
 * hidden not a multiple of 128 with FP8, only one allocator hook,
 * ll_buffers or ht_buffers outside 0..2),
 * EP_ERR_UNSUPPORTED (E > 1024, K > 32, N > 64, hidden > 16384,
 * num_src_ranks > R, or more LL slots, HT rows or map entries than 32-bit
 * indices address), EP_ERR_OUT_OF_MEMORY, EP_ERR_HIP. */
ep_status_t ep_create_group(const ep_config_t *config, ep_stream_t stream,
                            ep_group_t *out);

/* Free a group and everything it owns (NCCL-EP ncclEpGroupDestroy).  Blocks
 * until the device is idle.  Handles made from it become invalid. */
ep_status_t ep_destroy_group(ep_group_t group);

/* Bytes of device memory the group holds. */
ep_status_t ep_group_memory(ep_group_t group, int64_t *bytes);

/* Host-side counters of the group's calls that returned EP_OK (a staged
 * dispatch or combine counts when enqueued; its receive stage counts under
 * complete_calls).  Nothing here reads the device.  With the environment
 * variable EP_LOG=2 each counted call also prints one line to stderr. */
typedef struct {
    int64_t route_calls;
    int64_t handles_created;
    int64_t dispatch_calls;
    int64_t combine_calls;
    int64_t complete_calls;
    int64_t combine_backward_calls;
    int64_t dispatch_backward_calls;
    int64_t quantize_calls;
    int64_t tokens_routed;      /* rows of scores routed                  */
    int64_t tokens_dispatched;  /* tokens of the handles dispatched       */
    int64_t tokens_combined;    /* tokens of the handles combined         */
} ep_stats_t;
ep_status_t ep_group_stats(ep_group_t group, ep_stats_t *stats);

/* ----------------------------------------------------------------------- */
/* Routing (A1)                                                              */
/* ----------------------------------------------------------------------- */

/* Node-limited top-k routing ("NVSHMEM and DeepEP", high-throughput section:
 * score every node by the sum of its best ceil(K/M) expert scores -- the best
 * 2 at K=8, M=4 --, keep the M best nodes, pick the K best experts in them).
 *   scores   : F32 [n, E], row stride >= E, tag TOKENS or NONE.
 *   topk_idx : I32 [n, K] out, contiguous, tag TOPK_IDX or NONE.
 * Ties go to the lower node index and then to the lower expert index; the
 * K experts of a token are written in descending score order.  Node sums
 * are float32, largest term first.  n may be 0.  NaN scores are outside the
 * contract. */
ep_status_t ep_route(ep_group_t group, const ep_tensor_t *scores,
                     ep_tensor_t *topk_idx, ep_stream_t stream);

/* ----------------------------------------------------------------------- */
/* Handles (A2: counts, prefix sums, slot and row maps)                      */
/* ----------------------------------------------------------------------- */

/* Build the routing state of one forward pass (NCCL-EP ncclEpCreateHandle)
 * from topk_idx: I32 [n, K] contiguous with n = S*T, T <= T_max.  Token i
 * belongs to source rank s = i / T and is token t = i % T of it.
 *   LL: counts[e][s] and slot(i,k) = number of earlier entries (t ascending,
 *       then k) of the same source with the same expert.
 *   HT: stage-1 rows: one per (token, distinct destination node n), sent to
 *       the same-position rank d = n*G + s%G; rows grouped by d, ordered by
 *       (s, t) inside d.  Stage-2 rows: one per (token, k), grouped by expert
 *       (hence by rank and local expert), ordered by (s, t) inside an expert.
 * Entries outside [0,E) or repeating an earlier entry of the same token get
 * no slot/row (-1) and set a device error bit.  The handle's storage comes
 * from the group; nothing is allocated.
 * Errors: EP_ERR_CAPACITY (T > T_max or all handle slots in use),
 * EP_ERR_INVALID_ARGUMENT. */
ep_status_t ep_create_handle(ep_group_t group, const ep_tensor_t *topk_idx,
                             ep_stream_t stream, ep_handle_t *out);

/* Routing and handle creation in one pass: ep_route of `scores` into
 * topk_idx, then ep_create_handle from it, with the same results as the two
 * calls ("NVSHMEM and DeepEP", high-throughput section: the routing decision
 * fixes every count and position of the dispatch; "NCCL EP paper notes",
 * core functions: the handle is built from topk_idx).  The routing and the
 * counting share one kernel whenever the routing's fast path applies
 * (E a multiple of 128 up to 512, a node spanning a power-of-two number of
 * 32-lane groups, node sums of at most 2 scores, 16-byte aligned score
 * rows); otherwise the two run back to back.
 *   scores   : F32 [n, E], row stride >= E; n = S*T, T <= T_max.
 *   topk_idx : I32 [n, K] out, contiguous; the caller owns it (the handle
 *              keeps its own copy).
 * Errors: as ep_route and ep_create_handle together. */
ep_status_t ep_route_handle(ep_group_t group, const ep_tensor_t *scores, ep_tensor_t *topk_idx,
                            ep_stream_t stream, ep_handle_t *out);

/* Return the handle's storage to the group (NCCL-EP ncclEpHandleDestroy).
 * Stream-ordered reuse: work already enqueued with the handle may still run.
 * The value must not be used afterwards: until a new handle takes the same
 * slot, every call rejects it with EP_ERR_INVALID_ARGUMENT (as it rejects a
 * pointer that is no handle at all); after that it names the new handle. */
ep_status_t ep_destroy_handle(ep_handle_t handle);

/* Rows received by `rank` (NCCL-EP ncclEpHandleGetNumRecvTokens).  BLOCKING:
 * waits for the handle's stream work and copies the counts to the host --
 * the HT mode's CPU synchronisation.  rank = -1 gives the total.
 *   LL: messages in the rank's slots (over its experts and all sources).
 *   HT: stage-2 rows of the rank.  */
ep_status_t ep_handle_get_num_recv(ep_handle_t handle, int32_t rank, int64_t *n);

/* Views of the handle's device arrays (read-only for the caller). */
typedef enum {
    EP_MAP_LL_SLOT = 0,   /* I32 [n, K]: global slot (e*S+s)*T_max + slot, or -1 */
    EP_MAP_LL_COUNT = 1,  /* I32 [E, S]                                          */
    EP_MAP_HT_NODE_ROW = 2, /* I32 [n, N]: global stage-1 row, or -1            */
    EP_MAP_HT_ROW = 3,    /* I32 [n, K]: global stage-2 row, or -1.  PER_RANK: the
                             row of the entry's rank at the token's first entry
                             on that rank, -1 at its other entries            */
    EP_MAP_HT_RANK_COUNT = 4,  /* I32 [R]: stage-1 rows per destination rank    */
    EP_MAP_HT_RANK_OFFSET = 5, /* I32 [R]: exclusive prefix sum of the above    */
    EP_MAP_HT_EXPERT_COUNT = 6,  /* I32 [E]: stage-2 rows per expert
                                    (PER_RANK: [R] rows per rank)             */
    EP_MAP_HT_EXPERT_OFFSET = 7  /* exclusive prefix sum of the above          */
} ep_map_t;
/* The counts are written when the handle is made.  The slot / row maps and
 * the HT offsets are written by the handle's dispatch; asked for before a
 * dispatch has run, they are computed by a maps-only pass that this call
 * enqueues on the handle's stream (no rows are written). */
ep_status_t ep_handle_get_map(ep_handle_t handle, int32_t which, ep_tensor_t *view);

/* The handle's maps and counts without a group and without allocating:
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  It
 * computes what ep_create_handle followed by ep_handle_get_map gives for
 * `topk_idx` under `config`, bit for bit, and writes it to the caller's
 * buffers.
 *   config   : the topology, K, M, T_max, S, mode and HT stage-2 kind, as
 *              for ep_create_group (hidden, payload, handles, buffers, CU
 *              cap and allocator hooks are not used).
 *   topk_idx : I32 [n, K] contiguous, n = S*T with T <= T_max.
 *   maps     : eight pointers indexed by ep_map_t.  LL: maps[EP_MAP_LL_SLOT]
 *              (I32 [n, K]) and maps[EP_MAP_LL_COUNT] (I32 [E, S]).  HT:
 *              maps[EP_MAP_HT_NODE_ROW] (I32 [n, N]), maps[EP_MAP_HT_ROW]
 *              (I32 [n, K]) and the counts / offsets [R], [R], [E2], [E2]
 *              (E2 = E, or R with the per-rank stage 2), 1-D or [., 1].
 *              Every map of the mode is required and contiguous; the other
 *              mode's entries must be NULL.  Device memory, caller-owned.
 *   device_error : optional I32 [1] device buffer: set to 0, then to the
 *              EP_DEVERR_* bits of invalid or repeated entries.
 * Its working storage (a copy of topk_idx, in-tile ranks, tile counts, a
 * counter) is a fixed device array of EP_NOALLOC_SCRATCH_BYTES inside the
 * library, one per GPU, kept until the process ends.  Every call on a GPU
 * shares that GPU's array: calls that overlap on one GPU (other streams or
 * threads) race and give wrong maps.  Stream-ordered and capturable (no
 * memset or allocation is enqueued).
 * Errors: EP_ERR_INVALID_ARGUMENT (descriptors, shapes), EP_ERR_CAPACITY
 * (T > T_max, or more working storage than EP_NOALLOC_SCRATCH_BYTES: about
 * 8*n*K + 4*n*N + 4*ceil(T/16)*S*(E2 + N) bytes in HT, 8*n*K +
 * 4*ceil(T/16)*S*E in LL, i.e. up to about 51,000 tokens at K = N = 8,
 * E = 256), EP_ERR_UNSUPPORTED (limits as for ep_create_group), EP_ERR_HIP. */
#define EP_NOALLOC_SCRATCH_BYTES (8 * 1024 * 1024)
ep_status_t ep_layout_noalloc(const ep_config_t *config, const ep_tensor_t *topk_idx,
                              ep_tensor_t *const maps[8], ep_tensor_t *device_error,
                              ep_stream_t stream);

/* ----------------------------------------------------------------------- */
/* Dispatch (A3 quantise + A4 LL pack | A5 HT stage 1 + A6 HT stage 2)       */
/* ----------------------------------------------------------------------- */

/* Send every token to its experts (NCCL-EP ncclEpDispatch) -- here: write
 * it into the group's receive partitions.
 *
 * Two stages, as in NCCL-EP (send and receive phases joined by per-(expert,
 * source) counters).  The send stage quantises and packs every message into
 * its receive slot; since the partitions are local HBM, the messages land in
 * their final place.  The receive stage reads the per-(expert, source)
 * counters into the caller's recv_counts.  With send_only == 0 both stages
 * run in this call.  With send_only != 0 (LL only, NCCL-EP's staged mode)
 * only the send stage is enqueued; ep_complete(handle) enqueues the receive
 * stage, and recv_counts must stay valid until then.  In LL the group keeps
 * ll_buffers receive buffers and each dispatch takes the next one in turn
 * (ep_handle_get_buffer returns the handle's); with two, a dispatch may be
 * in flight while the previous handle is combined.  In HT the group keeps
 * ht_buffers sets of stage-1 / stage-2 rows (1 unless configured) and each
 * HT dispatch takes the next set in turn, overwriting the rows of the handle
 * that used it before: a handle's rows and partitions hold its data until
 * the dispatch that next takes its set (its maps and counts, and so its
 * combine, stay valid).
 *   tokens : BF16 [n, H] (n as in the handle), rows 16-byte aligned; or
 *            FP8_E4M3 [n, H] together with
 *   scales : F32 [n, H/128] (tag SCALES) -- already quantised tokens are
 *            packed as they are.  NULL when tokens are BF16.
 *   topk_weights : optional F32 [n, K]; HT forwards it in the stage-1
 *            metadata.  Ignored in LL.
 *   recv_counts  : optional I32 out, tag TOKENS_PER_EXPERT: LL [E, S]
 *            counts per (expert, source) or [E] tokens per expert; HT [E]
 *            stage-2 rows per expert (PER_RANK: [R] rows per rank).  With
 *            tag RECV_EXPERT_COUNTER_HOST (NCCL-EP's host-side receive
 *            counter) data is pinned host memory (hipHostMalloc, or a
 *            registered-at-allocation pinned buffer) that the receive stage
 *            writes directly: once the stream reaches that point the counts
 *            are on the host with no copy.  Pageable host memory is
 *            rejected with EP_ERR_INVALID_ARGUMENT.
 *   send_only : 0, or (LL) enqueue the send stage only; HT returns
 *            EP_ERR_UNSUPPORTED (the staged mode is an LL feature).
 * With an FP8 payload each 128-element block is quantised as
 *   scale = amax/448 (fp32 division), q = E4M3(x/scale) (fp32 division,
 *   nearest-even, saturating), amax == 0 -> scale 0 and codes 0;
 *   token values must be finite: in a block holding +-inf the scale is +inf
 *   and the finite elements get the codes of x/inf (+-0), but the code of
 *   an infinite or NaN element is unspecified;
 * row = [q: H bytes][scales: H/128 fp32] (7392 B at H = 7168).  A BF16
 * payload row is the H bf16 values (14336 B).
 *   LL message = row + 16-byte header int32 {src_token, src_rank, k, 0}
 *     (7408 / 14352 B), stored at message index (e*S + s)*T_max + slot
 *     (message i starts at byte i * pitch, pitch = size rounded up to 128).
 *   HT stage 1: row at node_row(i,n), metadata per row: src_token, src_rank,
 *     topk_idx[K], topk_weights[K].  HT stage 2: row at row(i,k), metadata
 *     per row: src_rank, src_token, k.
 * Stale contents beyond the counts are left in place (never cleared). */
ep_status_t ep_dispatch(ep_handle_t handle, const ep_tensor_t *tokens,
                        const ep_tensor_t *scales, const ep_tensor_t *topk_weights,
                        ep_tensor_t *recv_counts, int32_t send_only,
                        ep_stream_t stream);

/* FP8 E4M3 quantisation alone ("NVSHMEM and DeepEP", FP8 dispatch with one
 * fp32 scale per 128 elements; "NCCL EP paper notes": quantisation is part of
 * the send stage's preparation).  ep_dispatch quantises BF16 tokens itself;
 * this call is for callers that want the FP8 tokens on their own, to keep
 * them or to dispatch them more than once, passing them to ep_dispatch as
 * pre-quantised tokens (tokens FP8, scales F32).  The codes and scales are
 * the ones ep_dispatch writes when it quantises BF16 tokens itself:
 * scale = amax/448 per 128-element block, codes the nearest-even,
 * saturating E4M3 of x/scale; an all-zero block gets scale 0 and codes 0.
 * Non-finite token values are handled as in ep_dispatch (the codes of
 * infinite and NaN elements are unspecified).
 *   tokens: BF16 [n, H], rows 16-byte aligned, innermost contiguous.
 *   q:      FP8_E4M3 [n, H] out, rows 16-byte aligned.
 *   scales: F32 [n, H/128] out.
 * Errors: EP_ERR_INVALID_ARGUMENT (a group whose payload is not FP8, or a
 * descriptor that does not match). */
ep_status_t ep_quantize(ep_group_t group, const ep_tensor_t *tokens, ep_tensor_t *q,
                        ep_tensor_t *scales, ep_stream_t stream);

/* Group-owned receive buffers, as U8/I32/F32 views (device memory).  Rows
 * and messages start on 128-byte boundaries: the U8 views' row stride
 * (strides[0]) is the row / message size rounded up to 128 bytes.  When H is
 * a multiple of 512 the dispatch writes the padding after each row (message)
 * it fills with zeros, so that every cache line of a row is written whole;
 * otherwise the padding is never written.  Rows and slots the handle does
 * not use are never written. */
typedef enum {
    EP_BUF_LL_RECV = 0,        /* U8 [E*S*T_max, row+16]                     */
    EP_BUF_HT_STAGE1 = 1,      /* U8 [rows1_max, row]                         */
    EP_BUF_HT_STAGE1_TOKEN = 2,  /* I32 [rows1_max]                           */
    EP_BUF_HT_STAGE1_SRC = 3,    /* I32 [rows1_max]                           */
    EP_BUF_HT_STAGE1_TOPK = 4,   /* I32 [rows1_max, K]                        */
    EP_BUF_HT_STAGE1_WEIGHTS = 5, /* F32 [rows1_max, K]                       */
    EP_BUF_HT_STAGE2 = 6,      /* U8 [S*T_max*K, row]                         */
    EP_BUF_HT_STAGE2_SRC = 7,    /* I32 [S*T_max*K]                           */
    EP_BUF_HT_STAGE2_TOKEN = 8,  /* I32 [S*T_max*K]                           */
    EP_BUF_HT_STAGE2_K = 9,      /* I32 [S*T_max*K]: k of the row's (first) entry */
    EP_BUF_HT_STAGE2_TOPK = 10,  /* PER_RANK: I32 [S*T_max*K, K] the token's entries
                                    on the row's rank as local expert ids, else -1 */
    EP_BUF_HT_STAGE2_WEIGHTS = 11 /* PER_RANK: F32 [S*T_max*K, K] their weights, else 0 */
} ep_buffer_t;
ep_status_t ep_get_buffer(ep_group_t group, int32_t which, ep_tensor_t *view);

/* As ep_get_buffer, but the receive buffer (LL) or stage-row set (HT) is
 * the one the handle's last dispatch wrote (ep_get_buffer returns the
 * group's first; an HT handle not yet dispatched gets the first set).  EP_ERR_INVALID_ARGUMENT for an LL handle not yet dispatched,
 * and for a handle whose rows a later dispatch on the group has overwritten:
 * the next dispatch (of any handle) that takes the same receive buffer or
 * stage-row set -- the group's ll_buffers / ht_buffers of them are taken in
 * turn.  The handle's maps, counts and combine stay valid. */
ep_status_t ep_handle_get_buffer(ep_handle_t handle, int32_t which, ep_tensor_t *view);

/* One destination rank's partition of a receive buffer: the view of
 * ep_handle_get_buffer narrowed to the rows or slots rank `rank` receives
 * ("NVSHMEM and DeepEP", low-latency and high-throughput sections: each rank
 * owns the receive region of its local experts; the 64 ranks are partitions
 * of this GPU's memory).
 *   LL (EP_BUF_LL_RECV): the rank's [E/R][S][T_max] block of message slots,
 *       [E/R*S*T_max, row+16], of the buffer the handle's dispatch wrote;
 *       which slots hold messages is given by EP_MAP_LL_COUNT.
 *   HT, stage 1 (EP_BUF_HT_STAGE1*): the rank's stage-1 rows, offset and
 *       count from EP_MAP_HT_RANK_OFFSET / _COUNT.
 *   HT, stage 2 (EP_BUF_HT_STAGE2*): the rows of the rank's E/R experts (with
 *       the per-rank stage 2: the rank's rows), expert after expert.
 * The view is taken from the handle (HT bounds are this routing's counts),
 * so the HT forms synchronise the handle's stream and read two counters, as
 * ep_handle_get_num_recv does; the LL form does not block.  The rows hold
 * data once the handle's dispatch has run.  EP_ERR_INVALID_ARGUMENT for a
 * rank outside [0, R), a buffer id of the other mode, an LL handle not yet
 * dispatched, or a handle whose rows a later dispatch has overwritten (as
 * for ep_handle_get_buffer). */
ep_status_t ep_get_partition(ep_handle_t handle, int32_t rank, int32_t which, ep_tensor_t *view);

/* ----------------------------------------------------------------------- */
/* Combine (A7)                                                              */
/* ----------------------------------------------------------------------- */

/* Gather each token's K expert outputs and reduce them in the original token
 * order (NCCL-EP ncclEpCombine; "NVSHMEM and DeepEP": combine stays BF16):
 *   out[i][h] = bf16_rne( fma chain over k = 0..K-1 from +0 of
 *                         w[i][k] * Y[row(i,k)][h] )   in fp32,
 * where row(i,k) is the LL message index or the HT stage-2 row of the
 * handle; invalid entries contribute nothing.
 *   expert_out   : BF16 [rows, H] (or [E, S*T_max, H] in LL), innermost
 *                  contiguous, rows 16-byte aligned.  A row index >= rows
 *                  sets EP_DEVERR_ROW_RANGE and is skipped.
 *   topk_weights : F32 [n, K] contiguous, or NULL for unit weights.  With
 *                  the PER_RANK stage 2 the rows are the ranks' weighted
 *                  partial sums: weights must be NULL, and the combine sums
 *                  the token's rank rows in the order of the entries that
 *                  name them.
 *   out          : BF16 [n, H], innermost contiguous, rows 16-byte aligned.
 *   send_only    : 0, or (LL) NCCL-EP's staged mode: the combine's receive
 *                  stage (the gather-reduce into out) is enqueued by
 *                  ep_complete(handle); expert_out, topk_weights and out must
 *                  stay valid and unchanged until then.  HT returns
 *                  EP_ERR_UNSUPPORTED.
 * EP_ERR_INVALID_ARGUMENT if the handle's dispatch still awaits ep_complete. */
ep_status_t ep_combine(ep_handle_t handle, const ep_tensor_t *expert_out,
                       const ep_tensor_t *topk_weights, ep_tensor_t *out,
                       int32_t send_only, ep_stream_t stream);

/* Finish the handle's staged (send_only) dispatch or combine (NCCL-EP
 * ncclEpComplete): enqueue its receive stage on `stream`.  Stream-ordered:
 * the outputs are ready when the stream reaches this point.  A handle has at
 * most one staged operation; EP_ERR_INVALID_ARGUMENT if it has none. */
ep_status_t ep_complete(ep_handle_t handle, ep_stream_t stream);

/* ----------------------------------------------------------------------- */
/* Backward pass: reuse of the forward handle                                */
/* ----------------------------------------------------------------------- */

/* In training the backward pass reuses each layer's handle: the loss
 * gradient goes to the experts and the experts' gradients come back to the
 * tokens (NCCL-EP paper notes, usage: HT training example).  These are the
 * adjoints of ep_combine and ep_dispatch over the handle's row map (the FP8
 * quantisation of the forward dispatch is taken as the identity).  Neither
 * uses the receive buffers; both need the handle's maps (written by its
 * dispatch, or computed on first use) and no staged operation pending
 * (else EP_ERR_INVALID_ARGUMENT).  Rows that no entry points at are not
 * written. */

/* Backward of ep_combine.  For every valid entry (i, k) with row
 * r = row(i,k):
 *   grad_expert_out[r][h] = bf16_rne(w[i][k] * grad_out[i][h])  (one fp32
 *                           multiply) -- a BF16 dispatch of the gradient;
 *   grad_weights[i][k]    = sum over h of grad_out[i][h] * expert_out[r][h]
 *                           in fp32 (deterministic order; within the fp32
 *                           dot-product error bound of the exact sum).
 * Invalid entries write no row and get grad_weights 0.
 *   grad_out        : BF16 [n, H], rows 16-byte aligned.
 *   expert_out      : BF16 expert-output rows as for ep_combine, or NULL
 *                     (then grad_weights must be NULL).
 *   topk_weights    : F32 [n, K] contiguous.
 *   grad_expert_out : BF16 rows at the dispatch geometry ([rows, H], or LL
 *                     [E, S*T_max, H]).
 *   grad_weights    : optional F32 [n, K] contiguous.
 * EP_ERR_UNSUPPORTED with the PER_RANK stage 2 (the experts apply the
 * weights there, so the combine has none to differentiate). */
ep_status_t ep_combine_backward(ep_handle_t handle, const ep_tensor_t *grad_out,
                                const ep_tensor_t *expert_out,
                                const ep_tensor_t *topk_weights,
                                ep_tensor_t *grad_expert_out,
                                ep_tensor_t *grad_weights, ep_stream_t stream);

/* Backward of ep_dispatch:
 *   grad_tokens[i][h] = bf16_rne( fp32 sum over valid k, in k order, from +0,
 *                                 of grad_expert_in[row(i,k)][h] )
 * -- the combine with unit weights.
 *   grad_expert_in : BF16 rows at the dispatch geometry.
 *   grad_tokens    : BF16 [n, H], rows 16-byte aligned. */
ep_status_t ep_dispatch_backward(ep_handle_t handle, const ep_tensor_t *grad_expert_in,
                                 ep_tensor_t *grad_tokens, ep_stream_t stream);

/* ----------------------------------------------------------------------- */
/* Identity expert (test aid and debugging)                                  */
/* ----------------------------------------------------------------------- */

/* Turn packed rows back into BF16 rows: y = bf16_rne(decode(q) * scale) for
 * an FP8 payload (one fp32 multiply), a plain copy for a BF16 payload.
 *   rows : U8 [n, >= row bytes] with the group's payload layout.
 *   y    : BF16 [n, H].  */
ep_status_t ep_dequantize_rows(ep_group_t group, const ep_tensor_t *rows,
                               ep_tensor_t *y, ep_stream_t stream);

/* ----------------------------------------------------------------------- */
/* Errors                                                                    */
/* ----------------------------------------------------------------------- */

const char *ep_status_string(ep_status_t status);

/* BLOCKING: wait for the device, return the group's device error bits
 * (EP_DEVERR_*) accumulated since the last call, and clear them. */
ep_status_t ep_get_device_error(ep_group_t group, int32_t *code);

/* The last hipError_t seen by this thread inside the library (0 = none). */
int ep_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* EP_H */
