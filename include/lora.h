/*
 * lora.h -- C ABI of the routed LoRA delta library for MI355X (gfx950).
 *
 * The library adds, for every token row t of a mixed batch whose sequence
 * carries adapter slot s != 0,
 *
 *     y[t, off_j : off_j + h_j] += scale[s][j] * B[s][j] @ (A[s][j] @ x[t])
 *
 * to a projection's fp32 partial sum y, for each output slice j of the lane
 * (TensorFold PR #47, third commit message: the delta is added to the fp32
 * partial sum before the cross-rank reduction; xLLM PR #2014, "New
 * subsystems": fused QKV with GQA k/v slices, fused gate/up, and the
 * row-parallel o_proj / down_proj lanes).  Slot 0 is the base model: its rows
 * are neither read nor written (tokenspeed PR #976, third commit message: id 0
 * is the base model; TensorFold PR #47, third commit message: a slot-0 row is
 * not read or written, and a layer no adapter edits launches nothing).
 *
 * Conventions for every call
 *   - Return value: LORA_OK (0) or a negative lora_status.  No exception or
 *     abort crosses this boundary.  lora_last_error() gives a thread-local
 *     message for the last failing call on the calling thread.
 *   - Arguments are validated on the host before anything is enqueued, so a
 *     call that fails has launched nothing and written no device memory.
 *   - Device buffers (x, y, pool memory, routing memory, workspace) belong to
 *     the caller; the library never allocates or frees device memory.  The
 *     library owns only its opaque host handles and, inside a routing handle,
 *     two small pinned host staging buffers and a stream with two events.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Device work is enqueued on it asynchronously; nothing synchronises
 *     except where a call says so.  A compute call on a batch with both
 *     decode and matrix-core segments runs its decode kernels on a second
 *     stream owned by the routing handle, which waits for `stream`'s earlier
 *     work and which `stream` waits for before its later work (events; two
 *     parallel branches under graph capture), so for the caller the call is
 *     still ordered on `stream` alone.
 *   - A handle must not be used by two threads at once.  Buffers written by
 *     a call must not be read or written on another stream until that
 *     stream's work is ordered after the call.
 *   - Device pointers to x, y and the workspace must be 16-byte aligned;
 *     widths h_in and h_out[j] must be multiples of 8, ldx a multiple of 8
 *     and ldy a multiple of 4 (elements).
 */
#ifndef ADAPTER_DELTAS_LORA_H
#define ADAPTER_DELTAS_LORA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum lora_status {
    LORA_OK = 0,
    LORA_ERR_ARG = -1,              /* null pointer, bad enum or flag          */
    LORA_ERR_SHAPE = -2,            /* width, stride or alignment not allowed  */
    LORA_ERR_DTYPE = -3,            /* unsupported element type                */
    LORA_ERR_RANK = -4,             /* rank < 1 or > max_rank                  */
    LORA_ERR_CAPACITY = -5,         /* buffer or handle too small for request  */
    LORA_ERR_UNKNOWN_ADAPTER = -6,  /* admitted id not resident in the pool    */
    LORA_ERR_SLOT = -7,             /* slot 0 or outside 1..max_slots          */
    LORA_ERR_MISMATCH = -8,         /* routing built for another pool shape    */
    LORA_ERR_HIP = -9               /* a HIP runtime call failed               */
} lora_status;

typedef enum lora_dtype {
    LORA_DTYPE_BF16 = 1,
    LORA_DTYPE_FP16 = 2,
    LORA_DTYPE_FP32 = 3
} lora_dtype;

#define LORA_MAX_SLICES 4
#define LORA_MAX_RANK 256

/*
 * One lane: a projection the delta is added to.  For a row-parallel share
 * (o_proj, down_proj, attention wo_b, shared-expert w2 under tensor
 * parallelism) h_in is the number of input columns this GPU holds; A is cut
 * by those columns and B is held whole (TensorFold PR #47, first commit
 * message; xLLM PR #2014, LoRARowParallelLinear fused mode).
 */
typedef struct lora_lane_desc {
    int32_t h_in;                     /* input width on this GPU, >0, %8 == 0 */
    int32_t n_slices;                 /* 1..LORA_MAX_SLICES                   */
    int32_t h_out[LORA_MAX_SLICES];   /* per-slice output width, %8 == 0      */
    int32_t max_slots;                /* adapter slots 1..max_slots           */
    int32_t max_rank;                 /* 1..LORA_MAX_RANK                     */
    int32_t x_dtype;                  /* LORA_DTYPE_BF16 or LORA_DTYPE_FP16   */
} lora_lane_desc;

typedef struct lora_pool lora_pool;        /* opaque host handle */
typedef struct lora_routing lora_routing;  /* opaque host handle */

typedef struct lora_routing_info {
    int32_t n_tokens;            /* rows covered by the candidate batch       */
    int32_t n_active;            /* admitted rows with an adapter (slot != 0) */
    int32_t n_segments;          /* decode + prefill + gather segments        */
    int32_t n_decode_segments;   /* <= LORA_DECODE_SEG_ROWS rows, one slot    */
    int32_t n_prefill_segments;  /* <= LORA_PREFILL_SEG_ROWS rows, one slot   */
    int32_t n_distinct;          /* distinct adapters admitted (not base)     */
    int32_t n_admitted_seqs;
    int32_t n_seqs;
    int32_t n_gather_segments;   /* <= LORA_PREFILL_SEG_ROWS rows, one slot   */
} lora_routing_info;

#define LORA_DECODE_SEG_ROWS 8
#define LORA_PREFILL_SEG_ROWS 64
/* Decode rows of an adapter whose largest slice rank is at least this go to
 * gather segments and the matrix-core path; the others to decode segments
 * and the GEMV path.  The choice depends only on the row's own adapter. */
#define LORA_GATHER_MIN_RANK 128

/* Thread-local text of the last error on this thread ("" if none). */
const char *lora_last_error(void);

/* Library version string. */
const char *lora_version(void);

/* ------------------------------------------------------------------ pool --
 * Device-resident adapter factors of one lane (xLLM PR #2014, "New
 * subsystems": LoRARuntime keeps a per-projection device pool; tokenspeed PR
 * #976, third commit message: a registry id travels on the request and maps
 * to a recyclable GPU buffer slot).
 *
 * Pool memory is one caller-allocated device buffer of lora_pool_bytes()
 * bytes (256-byte aligned).  It holds, per slot and slice, A as
 * [rank_pad][h_in] bf16 and B transposed as [rank_pad][h_j] bf16, zero-padded
 * from the adapter's rank to rank_pad = max_rank rounded up to 16, plus the
 * per-slot rank and fp32 scale.  Slot 0 has no storage.
 */
int32_t lora_pool_bytes(const lora_lane_desc *desc, int64_t *bytes_out);

/* Binds a pool handle to caller memory and clears the slot metadata (enqueued
 * on `stream`).  Errors: ARG (null), SHAPE (widths), DTYPE (x_dtype), RANK
 * (max_rank), CAPACITY (dev_bytes < lora_pool_bytes). */
int32_t lora_pool_create(const lora_lane_desc *desc, void *dev_mem, int64_t dev_bytes,
                         void *stream, lora_pool **pool_out);

int32_t lora_pool_destroy(lora_pool *pool);

/*
 * Loads one adapter's factors for every slice of the lane into a slot.
 *
 *   adapter_id   registry id, > 0 (0 is the base model and cannot be loaded)
 *   slot         1..max_slots, or -1 for the slot already holding this id,
 *                else the lowest free slot.  A slot held by another id is
 *                taken over (that id is evicted).
 *   A[j]         PEFT lora_A of slice j, bf16 [rank[j]][lda[j]] row-major;
 *                columns [a_col0, a_col0 + h_in) are this GPU's share
 *   B[j]         PEFT lora_B of slice j, bf16 [h_out[j]][ldb[j]] row-major;
 *                columns [0, rank[j]) are read
 *   rank[j]      1..max_rank (per-module rank: TensorFold PR #47, first
 *                commit message)
 *   scale[j]     finite fp32 multiplier of slice j (PEFT lora_alpha / r,
 *                times any strength the caller applies)
 *   src_on_device 0: A/B are host pointers (packed on the host, copied, and
 *                the call waits for the copy); 1: device pointers (packed by a
 *                kernel on `stream`, no wait)
 *   slot_out     optional; receives the slot used
 *
 * Errors: ARG, SLOT, RANK (rank out of range), SHAPE (lda < a_col0 + h_in,
 * ldb < rank), CAPACITY (no free slot), HIP.
 */
int32_t lora_pool_load(lora_pool *pool, int32_t adapter_id, int32_t slot,
                       const void *const *A, const int64_t *lda, int64_t a_col0,
                       const void *const *B, const int64_t *ldb,
                       const int32_t *rank, const float *scale,
                       int32_t src_on_device, void *stream, int32_t *slot_out);

/*
 * lora_pool_load for a lane whose input arrives transformed, x' = M x (the
 * packed shared expert's down projection reads the rotated, scaled fp16
 * hidden state its expert kernels leave; TensorFold PR #47, first and third
 * commit messages: the shared expert's A is folded once at load).  Slice j is
 * stored with A'[k][c] = bf16(sum_i A[j][k][a_col0 + i] * fold[i][c]), an fp32
 * fma chain over i ascending rounded to nearest even, so that A' x' = A x
 * up to that rounding when fold = M^-1.  B, ranks and scales as in
 * lora_pool_load.
 *
 *   A, B    device pointers (as lora_pool_load with src_on_device = 1)
 *   fold    device fp32 [h_in][ld_fold], row-major; fold[i][c] multiplies
 *           column a_col0 + i of A into column c of A'
 *   ld_fold >= h_in
 *
 * Work is enqueued on `stream`; the source buffers and fold must stay valid
 * until it has run.  Errors: as lora_pool_load; ARG (null fold), SHAPE
 * (ld_fold < h_in or fold not 4-byte aligned).
 */
int32_t lora_pool_load_folded(lora_pool *pool, int32_t adapter_id, int32_t slot,
                              const void *const *A, const int64_t *lda, int64_t a_col0,
                              const void *const *B, const int64_t *ldb, const int32_t *rank,
                              const float *scale, const float *fold, int64_t ld_fold,
                              void *stream, int32_t *slot_out);

/* Forgets an adapter id; its slot becomes free and the slot's ranks on the
 * device are zeroed with a blocking copy (so lora_build_routing_device sees it
 * as holding no adapter); work still reading the slot must have finished.
 * Errors: ARG, UNKNOWN_ADAPTER (not resident), HIP. */
int32_t lora_pool_unload(lora_pool *pool, int32_t adapter_id);

/* Slot of a resident id (UNKNOWN_ADAPTER if absent). */
int32_t lora_pool_slot_of(const lora_pool *pool, int32_t adapter_id, int32_t *slot_out);

/* -------------------------------------------------------------- routing --
 * Per-batch routing, built once per batch.  It records, per segment, the
 * slot and the rank of each slice in the pool it was built against, and can
 * be used with any pool (another layer, another lane) that holds the same
 * ids in the same slots with the same ranks on that pool's slices; a compute
 * call checks this and returns LORA_ERR_MISMATCH otherwise.  To serve lanes
 * with different slice counts, build against the pool with the most slices.
 *
 * Routing memory is one caller-allocated device buffer of
 * lora_routing_bytes(max_tokens) bytes.  The handle also owns two pinned host
 * staging buffers, so building the next batch's routing can overlap the
 * device work of the previous one, and one stream (default priority) with
 * two events for the decode kernels of mixed batches, on the device current
 * at lora_routing_create; lora_routing_destroy waits for that stream.
 */
int32_t lora_routing_bytes(int32_t max_tokens, int64_t *bytes_out);

int32_t lora_routing_create(int32_t max_tokens, int32_t max_seqs, void *dev_mem,
                            int64_t dev_bytes, lora_routing **routing_out);

int32_t lora_routing_destroy(lora_routing *routing);

/*
 * Admission, slot assignment and segments for one candidate batch.
 *
 *   seq_adapter_id  host int32 [n_seq]: registry id per sequence, 0 = base
 *                   (xLLM PR #2014, "Wire-up": one id per sequence, aligned
 *                   with the query lengths)
 *   seq_len         host int32 [n_seq]: rows of the sequence in this batch
 *                   (>= 0); sequence i covers rows [sum(seq_len[:i]), ...)
 *   max_loras       distinct-adapter cap, 0 = no cap.  Sequences are walked
 *                   in order; base sequences are never charged, an adapter
 *                   already admitted costs nothing, a sequence that would
 *                   bring a new adapter past the cap is deferred and the walk
 *                   goes on (tokenspeed PR #976, first commit message).  Rows
 *                   of deferred sequences are left untouched.
 *   prefill_min_len sequences at least this long form prefill segments of
 *                   <= LORA_PREFILL_SEG_ROWS contiguous rows with one slot
 *                   (TensorFold PR #47: prompt chunks run one slot for all
 *                   their rows) and take the matrix-core path; shorter ones
 *                   are decode rows, grouped by slot (in order of first
 *                   appearance, token order within a slot) into segments of
 *                   <= LORA_DECODE_SEG_ROWS rows for the GEMV path, or, for
 *                   an adapter with a slice rank >= LORA_GATHER_MIN_RANK, into
 *                   gather segments of <= LORA_PREFILL_SEG_ROWS rows for the
 *                   matrix-core path.  The choice depends only on the
 *                   sequence's own length and adapter.
 *   admitted_out    optional host uint8 [n_seq]: 1 admitted, 0 deferred
 *   n_distinct_out  optional: distinct adapters admitted
 *
 * The per-token slot array, the active-row list and the segment table are
 * written to pinned staging and copied to the routing's device memory on
 * `stream`.  Errors: ARG, SHAPE (negative length), CAPACITY (more than
 * max_tokens rows or max_seqs sequences), UNKNOWN_ADAPTER (an admitted id not
 * resident in `pool`: never treated as base; TensorFold PR #47, second commit
 * message), HIP.  On error the routing keeps its previous contents.
 */
int32_t lora_build_routing(const lora_pool *pool, int32_t n_seq,
                           const int32_t *seq_adapter_id, const int32_t *seq_len,
                           int32_t max_loras, int32_t prefill_min_len,
                           lora_routing *routing, uint8_t *admitted_out,
                           int32_t *n_distinct_out, void *stream);

int32_t lora_routing_get_info(const lora_routing *routing, lora_routing_info *info_out);

/*
 * The host half of lora_build_routing with no device involved: the same
 * admission, slot assignment and segments, resolved against an explicit table
 * of resident ids and written to host memory.  lora_build_routing runs exactly
 * this planning and then copies the words to the device.
 *
 *   resident_id/resident_slot  [n_resident] id -> slot (1..max_slots)
 *   resident_rank optional [n_resident][4]: rank of each slice (0 if NULL)
 *   words_out     host int32 [words_capacity]; receives the packed tables:
 *                 16-word segments {slot, first active row, rows, kind
 *                 (0 decode, 1 prefill, 2 gather), rank of slices 0..3, token
 *                 rows (decode: one per row, the last repeated; prefill: the
 *                 first, rows being consecutive; gather: unused, the token
 *                 rows being those of its active rows)} at word
 *                 offsets_out[0], decode segments first, then prefill, then
 *                 gather; the token row of each active row at offsets_out[1]
 *                 (then the rows outside the delta, ascending); one slot per
 *                 token row at offsets_out[2]; and, from the next multiple
 *                 of 4 words on, 4 words per active row {slot, rank0 |
 *                 rank1 << 16, rank2 | rank3 << 16, 0}, then (possibly
 *                 none) one word per live decode shrink task {segment |
 *                 slice << 24 | 8-rank block << 26} at offsets_out[3]; at
 *                 offsets_out[4] an 8-word header {offset from the header,
 *                 count} per lane slice count 1..4 of the matrix-core shrink
 *                 task tables that follow (count 0: no table; the kernels
 *                 then number tasks by block index), one word per task
 *                 {segment counted from the first prefill or gather segment
 *                 | first rank tile << 24 | (tiles - 1) << 30}, a segment's
 *                 16-rank tiles numbered across its slices (slice 0's, then
 *                 slice 1's, ...); word b is run by block b, which the
 *                 device places on XCD b % 8: a segment's tasks sit in one
 *                 such residue class, heaviest first, and places left
 *                 empty hold -1
 *   offsets_out   host int32 [5]
 *   info_out      counts, as lora_routing_get_info
 *   admitted_out  optional host uint8 [n_seq]
 *
 * Errors as lora_build_routing, plus SLOT (bad resident entry) and CAPACITY
 * (words_capacity too small; lora_routing_bytes(max_tokens) / 4 words always
 * suffice).
 */
int32_t lora_plan_routing(int32_t n_seq, const int32_t *seq_adapter_id, const int32_t *seq_len,
                          int32_t max_loras, int32_t prefill_min_len, int32_t n_resident,
                          const int32_t *resident_id, const int32_t *resident_slot,
                          const int32_t *resident_rank, int32_t max_slots, int32_t max_tokens,
                          int32_t *words_out,
                          int64_t words_capacity, int32_t *offsets_out,
                          lora_routing_info *info_out, uint8_t *admitted_out);

/* Device pointer to the routing's per-token slot array (int32 [n_tokens], 0
 * for rows outside the batch), valid once the work a build call enqueued (the
 * copy of a host plan, or the routing kernel) has run on its stream. */
int32_t lora_routing_token_slots(const lora_routing *routing, const int32_t **dev_ptr_out);

#define LORA_DEVICE_ROUTING_MAX_TOKENS 8192

/*
 * Routing of a decode batch built on the device, with no host planning and
 * no host-device copy, so that one captured graph of this call and the
 * compute calls serves any mix of adapters: the slot of each row is read from
 * device memory when the graph runs (TensorFold PR #47, third commit message).
 * A batch padded to a captured size gives each padded row its original's slot
 * and x row; the padded row's y row then gets exactly its original's result
 * (or the caller writes slot 0 there and the row is skipped).
 *
 *   tok_slot  device int32 [n_tokens]: the pool slot of each token row, 0 =
 *             base; every row is a decode row.  Admission and id -> slot
 *             resolution are the caller's (as lora_plan_routing does them).
 *   n_tokens  0..min(max_tokens, LORA_DEVICE_ROUTING_MAX_TOKENS)
 *
 * One kernel on `stream` writes the same kinds of segment lora_build_routing
 * writes for decode rows (decode segments, and gather segments for adapters
 * with a slice rank >= LORA_GATHER_MIN_RANK), so every row's delta is
 * bit-identical to the one a host-built routing gives.  A row whose slot is
 * out of range or holds no adapter is never treated as base silently: it is
 * left untouched and counted as invalid in the device counts.  The host only
 * knows upper bounds afterwards: lora_routing_get_info reports n_active =
 * n_tokens and segment counts that are bounds (the workspace is sized for
 * them); the kernels read the exact counts from the device.  The routing can
 * be used with any pool that holds adapters in every slot the building pool
 * held them in, with the same ranks (MISMATCH otherwise, as with
 * lora_build_routing).  Errors: ARG, CAPACITY (n_tokens too large), HIP.
 */
int32_t lora_build_routing_device(const lora_pool *pool, const int32_t *tok_slot,
                                  int32_t n_tokens, lora_routing *routing, void *stream);

/*
 * Expert LoRA of a mixture-of-experts layer (xLLM PR #2014, "Not in this PR":
 * the fused MoE expert LoRA delta, a grouped GEMM over experts and adapters).
 * An adapter that edits the experts holds one LoRA pair per expert.  A pool
 * of an expert projection holds the pair of (adapter slot a, expert e) in
 * slot LORA_MOE_SLOT(a, e, n_experts); its max_slots is a multiple of
 * n_experts (n_experts times the adapter slots).
 */
#define LORA_MOE_SLOT(adapter_slot, expert, n_experts) \
    (((adapter_slot) - 1) * (n_experts) + (expert) + 1)

/*
 * Routing of the dispatched rows of a MoE layer's expert projection, built on
 * the device like lora_build_routing_device (same limits, same segments, same
 * bit-exactness), for decode batches.
 *
 *   tok_slot    device int32 [n_tokens]: adapter slot of each token (0 = base)
 *   row_token   device int32 [n_rows]: token of each dispatched row
 *   row_expert  device int32 [n_rows]: expert of each dispatched row
 *   n_rows      0..min(max_tokens, LORA_DEVICE_ROUTING_MAX_TOKENS)
 *   n_experts   >= 1, divides the pool's max_slots
 *
 * Row p takes the pair in slot LORA_MOE_SLOT(tok_slot[row_token[p]],
 * row_expert[p], n_experts).  x and y of the compute calls are indexed by
 * dispatched row (the caller's gathered expert inputs and the expert outputs
 * before the weighted combine).  A row of a base token is skipped; a row
 * whose adapter holds no pair for its expert is skipped and counted as
 * unedited (the adapter leaves that expert alone); a row naming a token,
 * expert or adapter slot out of range is skipped and counted as invalid.
 * Errors: ARG, SHAPE (n_experts), CAPACITY, HIP.
 */
int32_t lora_build_routing_moe(const lora_pool *pool, const int32_t *tok_slot,
                               int32_t n_tokens, const int32_t *row_token,
                               const int32_t *row_expert, int32_t n_rows, int32_t n_experts,
                               lora_routing *routing, void *stream);

/*
 * Routing of a batch given the pool slot of every row, planned on the host
 * (like lora_build_routing, copied on `stream`): for MoE batches of any size,
 * prefill chunks included, whose dispatched rows the caller has resolved to
 * (adapter, expert) slots with LORA_MOE_SLOT.
 *
 *   row_slot     host int32 [n_rows]: slot of each row, 0 = skip the row;
 *                every other value must be a slot that holds an adapter
 *   row_prefill  host uint8 [n_rows] or NULL (all rows decode): 1 for a row
 *                of a prefill token
 *
 * A decode row of a slot whose largest slice rank is below
 * LORA_GATHER_MIN_RANK takes the GEMV path (decode segments); a prefill row,
 * or a row of a higher-rank slot, takes the matrix-core path in gather
 * segments of up to LORA_PREFILL_SEG_ROWS rows of one slot (the grouped GEMM
 * over (adapter, expert) pairs).  A row's bits depend only on its own x row,
 * its slot's factors and its kind.  Errors: ARG, SHAPE, CAPACITY (n_rows >
 * max_tokens), SLOT (a row names a slot that holds no adapter), HIP.
 */
int32_t lora_build_routing_rows(const lora_pool *pool, int32_t n_rows, const int32_t *row_slot,
                                const uint8_t *row_prefill, lora_routing *routing,
                                void *stream);

/*
 * The host half of lora_build_routing_rows with no device involved: the same
 * segments from per-row slots, against an explicit rank table, written to
 * host memory in lora_plan_routing's packed layout (gather segments of up to
 * 16 rows when the gathered rows average at most 16 per slot, else up to
 * LORA_PREFILL_SEG_ROWS).
 *
 *   slot_rank  host int32 [max_slots + 1][4]: rank of each slice of each slot;
 *              a slot holds an adapter iff its slice-0 rank is >= 1
 *   the rest   as lora_build_routing_rows and lora_plan_routing
 *
 * Errors: ARG, SHAPE, SLOT (a row names a slot with no adapter), CAPACITY.
 */
int32_t lora_plan_rows(int32_t n_rows, const int32_t *row_slot, const uint8_t *row_prefill,
                       int32_t max_slots, const int32_t *slot_rank, int32_t *words_out,
                       int64_t words_capacity, int32_t *offsets_out,
                       lora_routing_info *info_out);

/* Device pointer to int32 [8] counts of a device-built routing, written by its
 * kernel: [0] active rows, [1] decode segments, [2] prefill segments (0),
 * [3] gather segments, [4] rows whose slot held no adapter (invalid), [5] MoE
 * rows whose adapter does not edit their expert.  ARG if the routing was
 * built on the host. */
int32_t lora_routing_device_counts(const lora_routing *routing, const int32_t **dev_ptr_out);

/* --------------------------------------------------------------- compute --
 * x:  [n_tokens][ldx] bf16 or fp16 (the lane's x_dtype), this GPU's input
 *     columns; only rows of active tokens are read.
 * y:  [n_tokens][ldy] fp32 partial sum; slice j occupies columns
 *     [sum(h_out[:j]), sum(h_out[:j+1])).  Only active rows, columns
 *     [0, sum(h_out)) are read and written.
 * v:  [n_active][n_slices][rank_pad] fp32, rows in the routing's active-row
 *     order: v[p][j][k] = fp32(scale[s][j] * (A[s][j] x)[k]) for k < rank;
 *     entries at k >= rank are unspecified.
 *
 * Within a row every sum runs in an order fixed by the lane's widths and the
 * adapter's rank alone, so a row's bits depend only on its own x row, its
 * adapter's factors and its own path (GEMV for decode rows; matrix cores for
 * prefill rows and for the decode rows of an adapter with a slice rank >=
 * LORA_GATHER_MIN_RANK), never on the other rows of the batch, the slot it
 * sits in, max_rank or the launch shape (TensorFold PR #47, third commit
 * message).
 */

/* v for all active rows (shrink: A @ x, times scale).  Errors: ARG, SHAPE,
 * MISMATCH (a slot of the routing is empty in this pool or holds other
 * ranks), HIP. */
int32_t lora_shrink(const lora_pool *pool, const lora_routing *routing,
                    const void *x, int64_t ldx, float *v, void *stream);

/* y += B @ v for all active rows (expand).  Errors as lora_shrink. */
int32_t lora_expand(const lora_pool *pool, const lora_routing *routing,
                    const float *v, float *y, int64_t ldy, void *stream);

/* Bytes of workspace lora_delta_apply needs for this pool and routing. */
int32_t lora_workspace_bytes(const lora_pool *pool, const lora_routing *routing,
                             int64_t *bytes_out);

/*
 * y += scale * B @ (A @ x) for all active rows: lora_shrink followed by
 * lora_expand on the same stream, so the result is bit-identical to calling
 * them in turn.  The workspace (caller device memory, >= lora_workspace_bytes)
 * holds v between the two.  With no active row nothing is launched and
 * LORA_OK is returned.  Errors as lora_shrink, plus CAPACITY (workspace).
 */
int32_t lora_delta_apply(const lora_pool *pool, const lora_routing *routing,
                         const void *x, int64_t ldx, float *y, int64_t ldy,
                         void *workspace, int64_t workspace_bytes, void *stream);

/*
 * The base projection with the delta in its fp32 partial sum, in one pass over
 * the output (TensorFold PR #47, third commit message and PR body "What this
 * changes": the delta is added in fp32 to the partial sum the base projection
 * produces, before the cross-rank reduction):
 *
 *     y[t] = x[t] W^T                    for every row t < n_rows
 *          + scale[s][j] B[s][j] (A[s][j] x[t])  on slice j's columns,
 *                                        for a row whose slot s != 0
 *
 * The delta is added to the product's fp32 accumulator before the one store
 * of y; y is written, not read.  Rows of the base model and rows the
 * routing defers get x W^T alone.
 *
 *   routing  a routing built on the host (lora_build_routing or
 *            lora_build_routing_rows) for exactly n_rows rows, or NULL for the
 *            base product alone (the same kernel with no delta)
 *   W        device bf16 [sum(h_out)][ldw]: the projection's weight in the
 *            linear layer's [out_features, in_features] orientation (the
 *            slices' rows stacked as in y; a row-parallel share holds this
 *            GPU's h_in input columns), 16-byte aligned, ldw >= h_in, % 8 == 0
 *   x, y     as lora_delta_apply; the lane's x must be bf16
 *   workspace  device memory of lora_linear_workspace_bytes bytes (v of the
 *            active rows as bf16 pairs v_hi + v_lo per rank, about 16
 *            significant bits), ignored when routing is NULL
 *
 * Sums: each output is a chain of 32-element matrix-core steps over h_in in
 * ascending order from zero, continued over the delta's terms in the same
 * accumulator: per 32-rank chunk of the row's slice, B times v_hi, then B
 * times v_lo, with zeros for the terms of other rows' adapters.  A row's bits
 * depend on its own x row, W and adapter only (not on the other rows of the
 * batch), and base rows equal the product of a call with routing NULL.  A
 * row tile (64 or 128 consecutive active rows) holds at most 1024 delta steps
 * (one per slot, slice and 16 ranks); a batch that would need more in one
 * tile -- many distinct high-rank adapters side by side -- is computed as the
 * base product followed by lora_delta_apply, whose sums it then has.
 * Errors: ARG (null pool, W or buffers; a
 * routing built on the device), SHAPE (n_rows != the routing's rows, widths,
 * strides, alignment), DTYPE (fp16 lane), MISMATCH, CAPACITY (workspace), HIP.
 */
int32_t lora_linear_workspace_bytes(const lora_pool *pool, const lora_routing *routing,
                                    int64_t *bytes_out);
int32_t lora_linear_delta(const lora_pool *pool, const lora_routing *routing, int32_t n_rows,
                          const void *W, int64_t ldw, const void *x, int64_t ldx, float *y,
                          int64_t ldy, void *workspace, int64_t workspace_bytes, void *stream);

/*
 * lora_delta_apply for callers that cannot allocate device memory: code under
 * HIP graph capture, serving loops that must not call hipMalloc, harnesses
 * that forbid allocation.  The caller passes inputs and outputs only; v lives
 * in a static device array of the library, LORA_NOALLOC_SCRATCH_BYTES bytes on
 * each GPU it runs on, held until the process ends.  The kernels and the bits
 * are those of lora_delta_apply.  The first call on a GPU looks up the
 * array's device address there (not a stream operation; make that first call
 * outside graph capture); no call allocates or frees device or pinned memory.
 *
 * Every call on one GPU shares that GPU's array, so calls that overlap on the
 * same GPU (other streams, other threads, other graphs replayed at once) race
 * on v and give wrong results: order them.  The array keeps the last call's
 * contents; nothing in it needs to start at zero.
 *
 * Errors as lora_delta_apply, plus CAPACITY when lora_workspace_bytes for
 * this pool and routing exceeds LORA_NOALLOC_SCRATCH_BYTES (nothing is
 * launched; use lora_delta_apply with a workspace), and HIP if the device or
 * the array's address cannot be found.
 */
#define LORA_NOALLOC_SCRATCH_BYTES 8388608
int32_t lora_delta_apply_noalloc(const lora_pool *pool, const lora_routing *routing,
                                 const void *x, int64_t ldx, float *y, int64_t ldy,
                                 void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ADAPTER_DELTAS_LORA_H */
