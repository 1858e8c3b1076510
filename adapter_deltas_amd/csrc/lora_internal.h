// Internal types shared by the host-side ABI code and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>
#include <unordered_map>
#include <vector>

#include "lora.h"

namespace lora {

constexpr int kDecodeSegRows = LORA_DECODE_SEG_ROWS;    // rows per decode segment
constexpr int kPrefillSegRows = LORA_PREFILL_SEG_ROWS;  // rows per prefill segment
constexpr int kSmallGatherRows = 16;                    // gather segments of small groups
constexpr int kRankAlign = 16;                          // rank padding of the pool
constexpr int kKBlock = 8;                              // ranks per decode shrink task
constexpr int kSubChunk = 512;                          // h_in elements per wave pass
constexpr int kParts = 8;                               // interleaved h_in parts (one wave each)
constexpr int kExpandTile = 512;                        // columns per decode expand task
constexpr int kFusedMaxRank = 16;                       // ranks of the one-launch decode delta
#ifndef LORA_FUSED_MAX_EXTRA_BYTES
#define LORA_FUSED_MAX_EXTRA_BYTES (4 << 20)
#endif
constexpr int64_t kFusedMaxExtraBytes = LORA_FUSED_MAX_EXTRA_BYTES;  // and the A its tiles re-read
constexpr int kMfmaExpandCols = 128;                    // columns per prefill expand task
#ifndef LORA_EXPAND_BLOCKS
#define LORA_EXPAND_BLOCKS 8192
#endif
constexpr int kExpandTargetBlocks = LORA_EXPAND_BLOCKS; // prefill expand grid to aim for
constexpr int kExpandMaxGroup = 32;                     // prefill segments per expand task
constexpr int kShrinkMinBlocks = 128;                   // prefill shrink grid below which tasks shrink
constexpr int kShrinkMaxTiles = 4;                      // rank tiles of one host-built shrink task
constexpr int kPlanComputeUnits = 256;                  // device size a host-only plan assumes
constexpr int kXcds = 8;                                // XCDs: block b of a grid runs on XCD b % 8
constexpr int32_t kMfmaTaskNone = -1;                   // an empty place of a shrink task table
constexpr int kMetaStride = 4;                          // slices per slot in metadata

enum SegKind : int32_t { kSegDecode = 0, kSegPrefill = 1, kSegGather = 2 };
constexpr int kGatherMinRank = LORA_GATHER_MIN_RANK;

// A segment descriptor is kSegWords int32 words:
//   [0] slot  [1] first active row (row of v)  [2] rows  [3] kind
//   [4..7]  rank of slices 0..3 in the pool the routing was built against
//   [8..15] decode: token row of each segment row (the last one repeated
//           past the segment's rows); prefill: [8] = first token row, the
//           segment's rows being consecutive; gather: unused, the token row
//           of segment row r being the row table's entry [1] + r.
constexpr int kSegWords = 16;
static_assert(kDecodeSegRows == 8, "descriptor holds 8 token rows");

// Geometry of a lane's pool, passed by value to kernels.
struct LaneGeom {
    int32_t h_in;
    int32_t n_slices;
    int32_t rank_pad;
    int32_t x_fp16;
    int32_t h_out[LORA_MAX_SLICES];
    int32_t col_off[LORA_MAX_SLICES];   // column of slice j in y
    int32_t H_out;
    int32_t v_stride;                   // floats per v row = n_slices * rank_pad
    int64_t a_slot_stride;              // bf16 elements of A per slot
    int64_t bt_slot_stride;             // bf16 elements of B^T per slot
    int64_t bt_slice_off[LORA_MAX_SLICES];
};

// Delta steps (one per slot, slice and 16 ranks) a row tile of the base
// projection holds in LDS; a batch with more in one tile takes the base
// product and lora_delta_apply instead.
constexpr int kLinearMaxSteps = 1024;

// v in the split form the base projection's delta K-steps read: per row, per
// slice, per group of 16 ranks, 16 bf16 values v_hi = bf16(v) and then 16 bf16
// values v_lo = bf16(v - v_hi) (nearest even; v = v_hi + v_lo to about 16
// significant bits).  A row is n_slices * vsplit_groups(rank_pad) * 32 bf16.
__host__ __device__ inline int vsplit_groups(int rank_pad) { return (rank_pad + 15) / 16; }

// Column tiles of tile_cols columns: slice j has ceil(h_out[j] / tile_cols) of
// them (slices past n_slices have width 0, so none), and the tiles of a
// segment are numbered slice after slice.  Tiles of the lane per segment:
__host__ __device__ inline int lane_tiles(const LaneGeom &g, int tile_cols)
{
    return (g.h_out[0] + tile_cols - 1) / tile_cols + (g.h_out[1] + tile_cols - 1) / tile_cols +
           (g.h_out[2] + tile_cols - 1) / tile_cols + (g.h_out[3] + tile_cols - 1) / tile_cols;
}

// Device views of a pool.  Slot s >= 1 is stored at index s - 1; the
// metadata tables have a row for slot 0 that stays zero.
struct PoolDev {
    const uint16_t *A;     // [max_slots][n_slices][rank_pad][h_in]
    const uint16_t *Bt;    // [max_slots][sum_j rank_pad * h_j]   B^T, rank-major
    const uint16_t *Bn;    // [max_slots][sum_j h_j * rank_pad]   B, output-major
    const int32_t *rank;   // [max_slots + 1][kMetaStride]
    const float *scale;    // [max_slots + 1][kMetaStride]
};

// Device views of a routing.
struct RoutingDev {
    const int32_t *seg;       // kSegWords words per segment
    const int32_t *tok_slot;  // slot per token row
    const int32_t *rows;      // token row of each active row (host-built: then the
                              // other rows of the batch)
    const int32_t *counts;    // device-built routing: exact counts (else null)
    int32_t spread;           // > 0: segments dealt to the XCDs this many at a time
                              // (the count is a bound; spread_task), else xcd_task
};
// Blocks of a launch over n segments of `per` tasks each.  When n is a bound
// (device-built routing, spread > 0) its segments are dealt to the XCDs
// `spread` at a time (spread_task) on a grid padded to whole rounds.
inline int64_t seg_grid(const RoutingDev &r, int64_t n, int64_t per)
{
    const int64_t deal = (int64_t)r.spread * per;
    const int64_t round = (int64_t)kXcds * r.spread;
    return r.spread > 0 ? kXcds * deal * ((n + round - 1) / round) : n * per;
}

// Entries of a device-built routing's counts.
enum DeviceCount : int { kCntActive = 0, kCntDecode = 1, kCntPrefill = 2, kCntGather = 3,
                         kCntInvalid = 4, kCntUnedited = 5, kCntWords = 8 };

// Dispatch table of a MoE layer's expert rows, for device routing: row p is
// token row_token[p] sent to expert row_expert[p]; its pool slot is that of
// (the token's adapter slot a, the expert e): (a - 1) * n_experts + e + 1.
struct MoeDispatch {
    const int32_t *row_token;
    const int32_t *row_expert;
    int n_tokens;
    int n_experts;
    int n_adapter_slots;   // max_slots / n_experts
};

// Arguments of the base projection with the delta in its epilogue.
struct LinearArgs {
    const uint16_t *W;        // [N][ldw] bf16: the projection's weight (out x in)
    int64_t ldw;
    const uint16_t *x;        // [*][ldx] bf16
    int64_t ldx;
    float *y;                 // [*][ldy] fp32, written
    int64_t ldy;
    int M, N, K;              // rows of the batch, sum(h_out), h_in
    const int32_t *rows;      // GEMM row m -> token row (null: m itself)
    int n_delta;              // GEMM rows m < n_delta carry a delta; v row m
    const int32_t *row_meta;  // per GEMM row m < n_delta: [slot, rank0 | rank1 << 16,
                              // rank2 | rank3 << 16, 0]
    const float *v;           // v of rows m < n_delta in the split bf16 form
};

// ---- launchers (kernels_*.hip) ----
hipError_t launch_linear(const LaneGeom &g, const PoolDev &p, const LinearArgs &a,
                         hipStream_t s);
// Rows per tile (64 or 128) launch_linear takes for an M x N product.
int linear_tile_rows(int64_t M, int64_t N);
// With `tasks` (n_tasks words, gemv_task_word) only those tasks are launched.
hipError_t launch_shrink_gemv(const LaneGeom &g, const PoolDev &p, const RoutingDev &r,
                              int n_seg, int kb_per_slice, const void *x, int64_t ldx,
                              float *v, int vsplit, hipStream_t s,
                              const int32_t *tasks = nullptr, int n_tasks = 0);
// A GEMV shrink task (decode segment si, slice j, rank block kb) in a word.
inline int32_t gemv_task_word(int32_t si, int j, int kb)
{
    return si | (j << 24) | (kb << 26);
}
// A matrix-core shrink task of a host-built table: segment si (counted from
// the first prefill or gather segment, < 2^24) and cnt (1..kShrinkMaxTiles)
// consecutive rank tiles from number c0 (< 64) of the segment's tiles
// numbered across its slices.
inline int32_t mfma_task_word(int32_t si, int c0, int cnt)
{
    return (int32_t)((uint32_t)si | ((uint32_t)c0 << 24) | ((uint32_t)(cnt - 1) << 30));
}
hipError_t launch_delta_gemv(const LaneGeom &g, const PoolDev &p, const RoutingDev &r,
                             int n_seg, const void *x, int64_t ldx, float *y, int64_t ldy,
                             hipStream_t s);
hipError_t launch_expand_gemv(const LaneGeom &g, const PoolDev &p, const RoutingDev &r,
                              int n_seg, int rows_per_wave, int lane_cols, const float *v,
                              float *y, int64_t ldy, hipStream_t s);
hipError_t launch_shrink_mfma(const LaneGeom &g, const PoolDev &p, const RoutingDev &r,
                              bool gather, int seg_begin, int n_seg, int nt_per_slice,
                              const void *x, int64_t ldx, float *v, int vsplit, hipStream_t s,
                              const uint32_t *tab = nullptr, int n_tab = 0, int tab_tiles = 0,
                              int tab_rows = 0);
hipError_t launch_expand_mfma(const LaneGeom &g, const PoolDev &p, const RoutingDev &r,
                              bool gather, int seg_begin, int n_seg, int group, int max_rank,
                              int max_seg_rows, const float *v, float *y, int64_t ldy,
                              hipStream_t s);
hipError_t launch_route_decode(const int32_t *tok_slot, int n_tok, const MoeDispatch *moe,
                               const int32_t *rank_tab, int max_slots, int max_dec,
                               int max_gather, int32_t *seg, int32_t *rows, int32_t *tok,
                               int32_t *counts, hipStream_t s);
hipError_t launch_fold_a(uint16_t *dst, const uint16_t *src, int64_t lda, int64_t a_col0,
                         int rank, int h_in, const float *F, int64_t ldf, hipStream_t s);
hipError_t launch_pack_a(uint16_t *dst, const uint16_t *src, int64_t lda, int64_t a_col0,
                         int rank, int rank_pad, int h_in, hipStream_t s);
hipError_t launch_pack_bt(uint16_t *dst, const uint16_t *src, int64_t ldb, int rank,
                          int rank_pad, int h_out, hipStream_t s);
hipError_t launch_pack_bn(uint16_t *dst, const uint16_t *src, int64_t ldb, int rank,
                          int rank_pad, int h_out, hipStream_t s);
hipError_t launch_set_meta(int32_t *rank_tab, float *scale_tab, int slot, int n_slices,
                           const int32_t *ranks, const float *scales, hipStream_t s);
hipError_t launch_clear_meta(int32_t *rank_tab, float *scale_tab, int n_rows,
                             hipStream_t s);

// ---- host side shared between the ABI's source files ----
// Record a thread-local error message and return `code`.
int32_t fail(int32_t code, const char *fmt, ...);
int32_t hip_fail(hipError_t e, const char *what);

}  // namespace lora

struct lora_pool;
struct lora_routing;
namespace lora {
// lora_delta_apply after the handle check: validates x, y and the workspace
// (v, workspace_bytes bytes at `workspace`) and enqueues the kernels.
int32_t delta_apply_ws(const lora_pool *p, const lora_routing *r, const void *x, int64_t ldx,
                       float *y, int64_t ldy, void *workspace, int64_t workspace_bytes,
                       hipStream_t st);
}  // namespace lora

// ---- opaque handles ----
struct lora_pool {
    lora_lane_desc desc;
    lora::LaneGeom geom;
    uint16_t *A;
    uint16_t *Bt;
    uint16_t *Bn;
    int32_t *rank_tab;
    float *scale_tab;
    std::vector<int32_t> h_rank;     // [(max_slots + 1) * kMetaStride]
    std::vector<float> h_scale;
    std::unordered_map<int32_t, int32_t> id_to_slot;
    std::vector<int32_t> slot_to_id;  // [max_slots + 1], 0 = free
};

namespace lora {
// Host tables of one batch's routing.  Packed layout (int32 words):
// [segments: kSegWords each][active rows][pad to 4][token slots][pad to 4].
struct Plan {
    std::vector<int32_t> seg, rows, tok;
    // per active row (the first n_active entries of rows): its slot and the
    // slot's ranks, 4 words [slot, rank0 | rank1 << 16, rank2 | rank3 << 16, 0]
    std::vector<int32_t> meta;
    // most delta steps of one 64- and one 128-row tile of the active rows
    // (every slice of the slot counted)
    int32_t tile_steps[2] = {0, 0};
    // the live GEMV shrink tasks, one word each (gemv_task_word), decode
    // segments in order, slices, then rank blocks of kKBlock
    std::vector<int32_t> tasks;
    // the matrix-core shrink tasks of the prefill and gather segments, one
    // table per lane slice count s = 1 .. kMetaStride (mtask_n[s] words from
    // mtask_off[s] of mtasks; none: 0), see mfma_task_word.  Packed after an
    // 8-word header {offset from the header, count} per s.
    std::vector<int32_t> mtasks;
    int32_t mtask_off[kMetaStride + 1] = {}, mtask_n[kMetaStride + 1] = {};
    // per table: most tiles of a task and most rows of a segment (the
    // kernel's tile and row template sizes cover them)
    int32_t mtask_tiles[kMetaStride + 1] = {}, mtask_rows[kMetaStride + 1] = {};
    static constexpr int kMtaskHeader = 2 * kMetaStride;
    std::vector<int32_t> slot_ranks;   // per distinct slot: kMetaStride ranks
    std::vector<uint8_t> adm;
    std::vector<int32_t> distinct_slots;
    int32_t max_gather_rows = 0;        // rows of the largest gather segment
    lora_routing_info info{};
    int64_t off_row() const { return (int64_t)seg.size(); }  // multiple of 4
    int64_t off_tok() const { return (off_row() + (int64_t)rows.size() + 3) / 4 * 4; }
    int64_t off_meta() const { return (off_tok() + (int64_t)tok.size() + 3) / 4 * 4; }
    int64_t off_tasks() const { return off_meta() + (int64_t)meta.size(); }
    int64_t off_mtask_header() const { return off_tasks() + (int64_t)tasks.size(); }
    int64_t off_mtasks() const { return off_mtask_header() + kMtaskHeader; }
    int64_t words() const { return off_mtasks() + (int64_t)mtasks.size(); }
    void pack(int32_t *w) const
    {
        int64_t o = 0;
        for (int32_t a : seg) w[o++] = a;
        for (int32_t a : rows) w[o++] = a;
        while (o < off_tok()) w[o++] = 0;
        for (int32_t a : tok) w[o++] = a;
        while (o < off_meta()) w[o++] = 0;
        for (int32_t a : meta) w[o++] = a;
        for (int32_t a : tasks) w[o++] = a;
        for (int sc = 1; sc <= kMetaStride; ++sc) {
            w[o++] = mtask_n[sc] ? kMtaskHeader + mtask_off[sc] : 0;
            w[o++] = mtask_n[sc];
        }
        for (int32_t a : mtasks) w[o++] = a;
    }
};
}  // namespace lora

struct lora_routing {
    int32_t max_tokens;
    int32_t max_seqs;
    int32_t *dev;                     // caller memory
    int64_t dev_words;
    int32_t *stage[2];                // pinned host staging
    hipEvent_t stage_done[2];
    int32_t stage_next;
    // device views of the current batch (offsets into dev)
    int32_t off_seg, off_row, off_tok;
    int32_t off_meta;                 // per active row slot and ranks (host-built only)
    int32_t tile_steps[2];            // Plan::tile_steps of the current batch
    int32_t off_tasks, n_tasks;       // the live GEMV shrink tasks (host-built only)
    int32_t off_mtasks[lora::kMetaStride + 1];   // matrix-core shrink task table per lane
    int32_t n_mtasks[lora::kMetaStride + 1];     // slice count (host-built only; 0: none)
    int32_t mtask_tiles[lora::kMetaStride + 1];  // most tiles of a task of each table
    int32_t mtask_rows[lora::kMetaStride + 1];   // most rows of a segment of each table
    int32_t n_cu;                     // compute units of the device the routing is on
    lora_routing_info info;
    int32_t pool_max_slots;           // slots of the pool the ids were resolved in
    bool device_built;                // counts on the device, info holds bounds
    int32_t off_counts;
    int32_t max_gather_rows;          // rows of the largest gather segment (bound)
    int32_t decode_rows;              // rows of the decode segments (0: not known on the host)
    int32_t expand_lane_cols;         // columns per lane of the decode expand: 8 or 4 (0: 8)
    int32_t seg_spread;               // RoutingDev::spread (device-built only)
    hipStream_t side;                 // decode kernels of a mixed batch (default priority)
    hipEvent_t fork_ev, join_ev;      // fork from / join into the caller's stream
    std::vector<int32_t> distinct_slots;
    std::vector<int32_t> slot_ranks;  // kMetaStride per distinct slot
    lora::Plan plan;                  // host tables, reused between builds
};
