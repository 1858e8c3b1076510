// Host side of the C ABI declared in include/lora.h: validation, the adapter
// pool, admission and routing, and kernel launches.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <limits>
#include <new>

#include "lora_internal.h"

// Segments per deal of a device-built routing's launches (spread_task).
// MoE segments each hold one (adapter, expert) slot's few rows and share no
// factors: dealt one at a time, moe_decode's delta went from 38.3 to 33.2 us
// per lane-layer (the same with 2 or 4 a deal).  A dense batch's consecutive
// segments of one adapter share its A and B: dealing 1, 2 or 3 at a time made
// its graph step 2-25% slower than xcd_task's ranges (0).
constexpr int32_t kSpreadMoe = 1, kSpreadDense = 0;

using namespace lora;

namespace {
thread_local std::string g_err;
}  // namespace

namespace lora {

int32_t fail(int32_t code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int32_t hip_fail(hipError_t e, const char *what)
{
    return fail(LORA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace lora

namespace {

int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int32_t check_desc(const lora_lane_desc *d)
{
    if (!d) return fail(LORA_ERR_ARG, "lane descriptor is null");
    if (d->n_slices < 1 || d->n_slices > LORA_MAX_SLICES)
        return fail(LORA_ERR_SHAPE, "n_slices=%d outside 1..%d", d->n_slices, LORA_MAX_SLICES);
    if (d->h_in <= 0 || d->h_in % 8 || d->h_in > (1 << 22))
        return fail(LORA_ERR_SHAPE, "h_in=%d must be a positive multiple of 8 (<= 2^22)", d->h_in);
    int64_t H = 0;
    for (int j = 0; j < d->n_slices; ++j) {
        if (d->h_out[j] <= 0 || d->h_out[j] % 8 || d->h_out[j] > (1 << 22))
            return fail(LORA_ERR_SHAPE, "h_out[%d]=%d must be a positive multiple of 8", j,
                        d->h_out[j]);
        H += d->h_out[j];
    }
    if (H > (1 << 24)) return fail(LORA_ERR_SHAPE, "sum of h_out %lld too large", (long long)H);
    if (d->max_slots < 1 || d->max_slots > 65535)
        return fail(LORA_ERR_SHAPE, "max_slots=%d outside 1..65535", d->max_slots);
    if (d->max_rank < 1 || d->max_rank > LORA_MAX_RANK)
        return fail(LORA_ERR_RANK, "max_rank=%d outside 1..%d", d->max_rank, LORA_MAX_RANK);
    if (d->x_dtype != LORA_DTYPE_BF16 && d->x_dtype != LORA_DTYPE_FP16)
        return fail(LORA_ERR_DTYPE, "x_dtype=%d: only bf16 (1) and fp16 (2) inputs", d->x_dtype);
    return LORA_OK;
}

void make_geom(const lora_lane_desc &d, LaneGeom &g)
{
    std::memset(&g, 0, sizeof g);
    g.h_in = d.h_in;
    g.n_slices = d.n_slices;
    g.rank_pad = (int32_t)round_up(d.max_rank, kRankAlign);
    g.x_fp16 = d.x_dtype == LORA_DTYPE_FP16;
    int32_t col = 0;
    for (int j = 0; j < d.n_slices; ++j) {
        g.h_out[j] = d.h_out[j];
        g.col_off[j] = col;
        g.bt_slice_off[j] = (int64_t)g.rank_pad * col;
        col += d.h_out[j];
    }
    g.H_out = col;
    g.v_stride = d.n_slices * g.rank_pad;
    g.a_slot_stride = (int64_t)d.n_slices * g.rank_pad * d.h_in;
    g.bt_slot_stride = (int64_t)g.rank_pad * col;
}

struct PoolLayout {
    int64_t a_off, bt_off, bn_off, rank_off, scale_off, total;
};

PoolLayout pool_layout(const lora_lane_desc &d, const LaneGeom &g)
{
    PoolLayout L;
    int64_t o = 0;
    L.a_off = o;
    o = round_up(o + (int64_t)d.max_slots * g.a_slot_stride * 2, 256);
    L.bt_off = o;
    o = round_up(o + (int64_t)d.max_slots * g.bt_slot_stride * 2, 256);
    L.bn_off = o;
    o = round_up(o + (int64_t)d.max_slots * g.bt_slot_stride * 2, 256);
    L.rank_off = o;
    o = round_up(o + (int64_t)(d.max_slots + 1) * kMetaStride * 4, 256);
    L.scale_off = o;
    o = round_up(o + (int64_t)(d.max_slots + 1) * kMetaStride * 4, 256);
    L.total = o;
    return L;
}

uint16_t *slot_a(const lora_pool *p, int slot, int j)
{
    return p->A + (int64_t)(slot - 1) * p->geom.a_slot_stride +
           (int64_t)j * p->geom.rank_pad * p->geom.h_in;
}

uint16_t *slot_bt(const lora_pool *p, int slot, int j)
{
    return p->Bt + (int64_t)(slot - 1) * p->geom.bt_slot_stride + p->geom.bt_slice_off[j];
}

uint16_t *slot_bn(const lora_pool *p, int slot, int j)
{
    return p->Bn + (int64_t)(slot - 1) * p->geom.bt_slot_stride + p->geom.bt_slice_off[j];
}

PoolDev pool_dev(const lora_pool *p)
{
    return PoolDev{p->A, p->Bt, p->Bn, p->rank_tab, p->scale_tab};
}

RoutingDev routing_dev(const lora_routing *r)
{
    return RoutingDev{r->dev + r->off_seg, r->dev + r->off_tok, r->dev + r->off_row,
                      r->device_built ? r->dev + r->off_counts : nullptr,
                      r->device_built ? r->seg_spread : 0};
}

// Largest rank over the routing's distinct slots and the lane's slices.
int batch_max_rank(const lora_pool *p, const lora_routing *r)
{
    int m = 0;
    if (r->device_built) {   // the slots are only known on the device
        for (int32_t rk : p->h_rank) m = std::max(m, rk);
        return m;
    }
    for (int32_t s : r->distinct_slots)
        for (int j = 0; j < p->desc.n_slices; ++j)
            m = std::max(m, p->h_rank[(size_t)s * kMetaStride + j]);
    return m;
}

// Largest slice rank of the slots whose decode rows take the GEMV path (a
// slot with a slice rank >= kGatherMinRank sends its decode rows to gather
// segments): the rank blocks a decode kernel's grid has to cover.
int gemv_max_rank(const lora_pool *p, const lora_routing *r)
{
    auto slot_max = [p](int32_t s) {
        int m = 0;
        for (int j = 0; j < kMetaStride; ++j) m = std::max(m, p->h_rank[(size_t)s * kMetaStride + j]);
        return m;
    };
    int m = 0;
    auto take = [&](int32_t s) {
        const int sm = slot_max(s);
        if (sm < kGatherMinRank) m = std::max(m, sm);
    };
    if (r->device_built) {
        for (int32_t s = 1; s <= p->desc.max_slots; ++s) take(s);
    } else {
        for (int32_t s : r->distinct_slots) take(s);
    }
    return m;
}

int32_t check_pair(const lora_pool *p, const lora_routing *r)
{
    if (!p || !r) return fail(LORA_ERR_ARG, "pool or routing is null");
    if (r->pool_max_slots > p->desc.max_slots)
        return fail(LORA_ERR_MISMATCH, "routing resolved slots up to %d, pool has %d",
                    r->pool_max_slots, p->desc.max_slots);
    for (size_t i = 0; i < r->distinct_slots.size(); ++i) {
        const int32_t s = r->distinct_slots[i];
        if (s < 1 || s > p->desc.max_slots || p->slot_to_id[s] == 0)
            return fail(LORA_ERR_MISMATCH, "routing uses slot %d, which this pool does not hold",
                        s);
        for (int j = 0; j < p->desc.n_slices; ++j)
            if (r->slot_ranks[i * kMetaStride + j] != p->h_rank[(size_t)s * kMetaStride + j])
                return fail(LORA_ERR_MISMATCH,
                            "slot %d slice %d has rank %d in this pool but %d in the pool the "
                            "routing was built against",
                            s, j, p->h_rank[(size_t)s * kMetaStride + j],
                            r->slot_ranks[i * kMetaStride + j]);
    }
    return LORA_OK;
}

int32_t check_x(const lora_pool *p, const void *x, int64_t ldx)
{
    if (!x) return fail(LORA_ERR_ARG, "x is null");
    if (!aligned16(x)) return fail(LORA_ERR_SHAPE, "x must be 16-byte aligned");
    if (ldx < p->desc.h_in || ldx % 8)
        return fail(LORA_ERR_SHAPE, "ldx=%lld must be >= h_in=%d and a multiple of 8",
                    (long long)ldx, p->desc.h_in);
    return LORA_OK;
}

int32_t check_y(const lora_pool *p, const float *y, int64_t ldy)
{
    if (!y) return fail(LORA_ERR_ARG, "y is null");
    if (!aligned16(y)) return fail(LORA_ERR_SHAPE, "y must be 16-byte aligned");
    if (ldy < p->geom.H_out || ldy % 4)
        return fail(LORA_ERR_SHAPE, "ldy=%lld must be >= sum(h_out)=%d and a multiple of 4",
                    (long long)ldy, p->geom.H_out);
    return LORA_OK;
}

int32_t check_v(const float *v)
{
    if (!v) return fail(LORA_ERR_ARG, "v is null");
    if (!aligned16(v)) return fail(LORA_ERR_SHAPE, "v must be 16-byte aligned");
    return LORA_OK;
}

// Streams of one call.  The decode kernels (GEMV) and the matrix-core
// kernels of a batch touch disjoint rows of v and y, so for a batch with
// both kinds the decode kernels run on the routing's second stream, forked
// from the caller's stream and joined back into it with events (under graph
// capture: two parallel branches); otherwise everything runs on the caller's
// stream.
struct CallStreams {
    hipStream_t main;   // the caller's stream: matrix-core kernels
    hipStream_t dec;    // decode kernels
};

int32_t fork_streams(const lora_routing *r, hipStream_t s, CallStreams &cs)
{
    const lora_routing_info &I = r->info;
    cs.main = cs.dec = s;
    const bool mixed = I.n_decode_segments > 0 && I.n_prefill_segments + I.n_gather_segments > 0;
    if (!mixed || !r->side) return LORA_OK;
    hipError_t e = hipEventRecord(r->fork_ev, s);
    if (e == hipSuccess) e = hipStreamWaitEvent(r->side, r->fork_ev, 0);
    if (e != hipSuccess) return hip_fail(e, "forking the decode stream");
    cs.dec = r->side;
    return LORA_OK;
}

int32_t join_streams(const lora_routing *r, const CallStreams &cs)
{
    if (cs.dec == cs.main) return LORA_OK;
    hipError_t e = hipEventRecord(r->join_ev, cs.dec);
    if (e == hipSuccess) e = hipStreamWaitEvent(cs.main, r->join_ev, 0);
    if (e != hipSuccess) return hip_fail(e, "joining the decode stream");
    return LORA_OK;
}

// bf16 values per active row of v in the base projection's split form.
int linear_v_len(const lora_pool *p)
{
    return p->geom.n_slices * vsplit_groups(p->geom.rank_pad) * 32;
}

// The kernels of each call.  With decode = false the decode segments are left
// to the caller (the one-launch decode delta of lora_delta_apply).
// vsplit > 0: v in the split form of the base projection (rows of vsplit bf16).
int32_t enqueue_shrink(const lora_pool *p, const lora_routing *r, const void *x, int64_t ldx,
                       float *v, const CallStreams &cs, bool decode = true, int vsplit = 0)
{
    hipStream_t s = cs.main;
    const lora_routing_info &I = r->info;
    const int kmax = batch_max_rank(p, r);
    RoutingDev rd = routing_dev(r);
    PoolDev pd = pool_dev(p);
    if (decode && I.n_decode_segments > 0) {
        // rank blocks of the GEMV slots only (higher-rank slots are gathered);
        // a host-built routing may list the live tasks only
        const int kb = (gemv_max_rank(p, r) + kKBlock - 1) / kKBlock;
        const bool tab = !r->device_built && r->n_tasks > 0;
        hipError_t e = launch_shrink_gemv(p->geom, pd, rd, I.n_decode_segments, kb, x, ldx, v,
                                          vsplit, cs.dec, tab ? r->dev + r->off_tasks : nullptr,
                                          tab ? r->n_tasks : 0);
        if (e != hipSuccess) return hip_fail(e, "shrink (decode) launch");
    }
    const int nt = (kmax + 15) / 16;
    // a host-built table of the matrix-core tasks for this lane's slice count
    const int sc = p->geom.n_slices;
    const bool mtab = !r->device_built && sc >= 1 && sc <= kMetaStride && r->n_mtasks[sc] > 0;
    const uint32_t *tab =
        mtab ? reinterpret_cast<const uint32_t *>(r->dev + r->off_mtasks[sc]) : nullptr;
    const int n_tab = mtab ? r->n_mtasks[sc] : 0;
    const int tab_tiles = mtab ? r->mtask_tiles[sc] : 0, tab_rows = mtab ? r->mtask_rows[sc] : 0;
    if (I.n_prefill_segments > 0 && I.n_gather_segments > 0) {
        // Prefill and gather segments follow each other in the table, and the
        // host plan's row table holds the token row of every one of their
        // rows: one launch of the gather form covers both (it takes each row
        // from the table; the sums are the same).
        hipError_t e = launch_shrink_mfma(p->geom, pd, rd, true, I.n_decode_segments,
                                          I.n_prefill_segments + I.n_gather_segments, nt, x,
                                          ldx, v, vsplit, s, tab, n_tab,
                                          tab_tiles, tab_rows);
        if (e != hipSuccess) return hip_fail(e, "shrink (prefill + gather) launch");
    } else if (I.n_prefill_segments > 0) {
        hipError_t e = launch_shrink_mfma(p->geom, pd, rd, false, I.n_decode_segments,
                                          I.n_prefill_segments, nt, x, ldx, v, vsplit, s, tab,
                                          n_tab, tab_tiles, tab_rows);
        if (e != hipSuccess) return hip_fail(e, "shrink (prefill) launch");
    } else if (I.n_gather_segments > 0) {
        hipError_t e = launch_shrink_mfma(p->geom, pd, rd, true, I.n_decode_segments,
                                          I.n_gather_segments, nt, x, ldx, v, vsplit, s, tab,
                                          n_tab, tab_tiles, tab_rows);
        if (e != hipSuccess) return hip_fail(e, "shrink (gather) launch");
    }
    return LORA_OK;
}

int32_t enqueue_expand(const lora_pool *p, const lora_routing *r, const float *v, float *y,
                       int64_t ldy, const CallStreams &cs, bool decode = true)
{
    hipStream_t s = cs.main;
    const lora_routing_info &I = r->info;
    RoutingDev rd = routing_dev(r);
    PoolDev pd = pool_dev(p);
    if (decode && I.n_decode_segments > 0) {
        // Waves of 4 rows (two per task) when the decode segments are close
        // to full (at least 7 of 8 rows on average): fewer waves load the
        // task's B tile.  With emptier segments the second half of such a
        // wave would mostly repeat a row, so waves take 2 rows (measured on
        // decode_mix, 7.2 rows a segment: 7.08 -> 6.56 us per call; on
        // moe_decode, 2.3 rows: 20.0 -> 21.0 us).  The choice changes which
        // wave computes a row, not its sums.
        const int rpw = r->decode_rows >= 7 * I.n_decode_segments ? 4 : 2;
        // Columns per lane: 4 (256-column tasks, twice the workgroups, half
        // the fmas per wave) for sparse segments, 8 otherwise (measured per
        // call with 8 / 4: moe_decode, 2.3 rows a segment, 20.4 / 19.0 us;
        // decode_mix 6.56 / 6.78; many_tenants 21.3 / 24.4).
        const int lc = r->expand_lane_cols == 4 ? 4 : 8;
        hipError_t e = launch_expand_gemv(p->geom, pd, rd, I.n_decode_segments, rpw, lc, v, y,
                                          ldy, cs.dec);
        if (e != hipSuccess) return hip_fail(e, "expand (decode) launch");
    }
    // Consecutive segments share a task (and its staged B tile) while the
    // grid still has about kExpandTargetBlocks workgroups.
    const int64_t per_group = lane_tiles(p->geom, kMfmaExpandCols);
    auto group_for = [&](int n) {
        const int64_t fit = (int64_t)n * per_group / kExpandTargetBlocks;
        return (int)std::max<int64_t>(1, std::min<int64_t>(kExpandMaxGroup, fit));
    };
    const int kmax = batch_max_rank(p, r);
    if (I.n_prefill_segments > 0 && I.n_gather_segments > 0) {
        // one launch of the gather form over both kinds (as in the shrink)
        const int n = I.n_prefill_segments + I.n_gather_segments;
        hipError_t e = launch_expand_mfma(p->geom, pd, rd, true, I.n_decode_segments, n,
                                          group_for(n), kmax, kPrefillSegRows, v, y, ldy, s);
        if (e != hipSuccess) return hip_fail(e, "expand (prefill + gather) launch");
        return LORA_OK;
    }
    if (I.n_prefill_segments > 0) {
        hipError_t e = launch_expand_mfma(p->geom, pd, rd, false, I.n_decode_segments,
                                          I.n_prefill_segments, group_for(I.n_prefill_segments),
                                          kmax, kPrefillSegRows, v, y, ldy, s);
        if (e != hipSuccess) return hip_fail(e, "expand (prefill) launch");
    }
    if (I.n_gather_segments > 0) {
        hipError_t e = launch_expand_mfma(p->geom, pd, rd, true,
                                          I.n_decode_segments + I.n_prefill_segments,
                                          I.n_gather_segments, group_for(I.n_gather_segments),
                                          kmax, std::max(1, r->max_gather_rows), v, y, ldy, s);
        if (e != hipSuccess) return hip_fail(e, "expand (gather) launch");
    }
    return LORA_OK;
}

// The row table lists the active rows (the rows of v, in v's order) and then
// every other row of the batch in row order, so that a kernel walking all
// rows of the batch (the base projection with the delta in its epilogue)
// takes them from one table, active rows first.  Kernels of the delta read
// only the first n_active entries.
// Slot and ranks of every active row (rows holds the active rows only when
// this is called), for the base projection's delta.
template <class Ranks>
void fill_row_meta(Plan &pl, Ranks ranks)
{
    pl.meta.resize(pl.rows.size() * 4);
    {
        int32_t *w = pl.meta.data();
        int32_t last = -1, r01 = 0, r23 = 0;   // rows of one slot come together
        for (int32_t t : pl.rows) {
            const int32_t s = pl.tok[(size_t)t];
            if (s != last) {
                last = s;
                r01 = (ranks(s, 0) & 0xffff) | (ranks(s, 1) << 16);
                r23 = (ranks(s, 2) & 0xffff) | (ranks(s, 3) << 16);
            }
            w[0] = s;
            w[1] = r01;
            w[2] = r23;
            w[3] = 0;
            w += 4;
        }
    }
    // delta steps of each 64- and 128-row tile: per distinct slot, one per 16
    // ranks of every slice (a bound on what the tile's columns need)
    auto steps = [&](int32_t s) {
        int32_t n = 0;
        for (int j = 0; j < kMetaStride; ++j) n += (ranks(s, j) + 15) / 16;
        return n;
    };
    // (the slot of active row m is meta[4 m], read in order)
    const int64_t n = (int64_t)pl.rows.size();
    const int32_t *slot_of = pl.meta.data();
    int32_t top = 0;
    for (int64_t m = 0; m < n; ++m) top = std::max(top, slot_of[4 * m]);
    std::vector<int64_t> seen((size_t)top + 1, -1);   // last tile that counted each slot
    for (int b = 0; b < 2; ++b) {
        const int64_t bm = b == 0 ? 64 : 128;
        int32_t most = 0;
        std::fill(seen.begin(), seen.end(), -1);
        for (int64_t m0 = 0; m0 < n; m0 += bm) {
            int32_t tot = 0;
            for (int64_t m = m0; m < std::min(n, m0 + bm); ++m) {
                const int32_t s = slot_of[4 * m];
                if (seen[(size_t)s] != m0) {
                    seen[(size_t)s] = m0;
                    tot += steps(s);
                }
            }
            most = std::max(most, tot);
        }
        pl.tile_steps[b] = most;
    }
}

// The live GEMV shrink tasks of the plan's decode segments: ceil(rank / 8)
// rank blocks per slice of each.  Kept only while they fit the routing's
// words (2 * kSegWords + 2 per token row; at most 16 per row are taken by the
// segment tables and 4 by the per-row table) and leave at least a quarter of
// a full grid's tasks out (reading the task is one more dependent load).
void fill_gemv_tasks(Plan &pl, int32_t max_tokens)
{
    pl.tasks.clear();
    const int64_t n_seg = (int64_t)pl.seg.size() / kSegWords;
    int32_t most_kb = 0, n_dec = 0;
    for (int64_t si = 0; si < n_seg; ++si) {
        const int32_t *d = &pl.seg[(size_t)(si * kSegWords)];
        if (d[3] != kSegDecode) continue;
        ++n_dec;
        for (int j = 0; j < kMetaStride; ++j) {
            const int32_t nk = (d[4 + j] + kKBlock - 1) / kKBlock;
            most_kb = std::max(most_kb, nk);
            for (int32_t kb = 0; kb < nk; ++kb)
                pl.tasks.push_back(gemv_task_word((int32_t)si, j, kb));
        }
    }
    const int64_t full = (int64_t)n_dec * kMetaStride * most_kb;
    const int64_t budget = (int64_t)max_tokens * (2 * kSegWords + 2) - pl.off_tasks() - 64;
    if ((int64_t)pl.tasks.size() * 4 > full * 3 || (int64_t)pl.tasks.size() > budget)
        pl.tasks.clear();
}

// The matrix-core shrink tasks of the plan's prefill and gather segments, one
// table per lane slice count s (1 .. the slices with a rank).  A task is
// bound by the bytes its compute unit reads, about (rows + 16 * tiles) * h_in
// * 2: a segment's tiles of all s slices are cut into as few tasks of at most
// kShrinkMaxTiles tiles as fit, and, while the tasks are fewer than the
// device's compute units, the heaviest segments are cut finer (the smallest
// largest task whose count still fits one task per unit).  A segment's
// tasks go to one XCD, and each XCD's tasks are stored heaviest first, so a
// grid larger than the device starts the long ones first.  A table of fewer
// than kShrinkMinBlocks tasks is not kept (the block-index tasks split rows
// for small batches), nor tables that do not fit the routing's words.
void fill_mfma_tasks(Plan &pl, int32_t max_tokens, int32_t n_cu)
{
    pl.mtasks.clear();
    for (int s = 0; s <= kMetaStride; ++s)
        pl.mtask_off[s] = pl.mtask_n[s] = pl.mtask_tiles[s] = pl.mtask_rows[s] = 0;
    const int64_t n_seg = (int64_t)pl.seg.size() / kSegWords;
    int64_t first = 0;
    while (first < n_seg && pl.seg[(size_t)(first * kSegWords) + 3] == kSegDecode) ++first;
    if (first == n_seg || n_seg - first >= (int64_t)1 << 24) return;
    int max_s = 0;
    for (int64_t si = first; si < n_seg; ++si) {
        const int32_t *d = &pl.seg[(size_t)(si * kSegWords)];
        if (d[3] == kSegDecode) return;       // not the expected order: no tables
        for (int j = 0; j < kMetaStride; ++j)
            if (d[4 + j] > 0) max_s = std::max(max_s, j + 1);
    }
    struct Item { int32_t si, c0, cnt, cost; };
    std::vector<int32_t> rows, tiles, m, seg_tasks, order, xcd_of;
    std::vector<int64_t> seg_cost, bucket;
    std::vector<Item> items, sorted;
    for (int sc = 1; sc <= max_s; ++sc) {
        rows.clear();
        tiles.clear();
        int64_t m0 = 0;
        for (int64_t si = first; si < n_seg; ++si) {
            const int32_t *d = &pl.seg[(size_t)(si * kSegWords)];
            int32_t t = 0;
            for (int j = 0; j < sc; ++j) t += (d[4 + j] + 15) / 16;
            rows.push_back(std::min(d[2], (int32_t)kPrefillSegRows));
            tiles.push_back(t);
            m0 += (t + kShrinkMaxTiles - 1) / kShrinkMaxTiles;
        }
        const size_t ns = rows.size();
        m.assign(ns, 0);
        auto chunks_at = [&](int32_t c, bool store) {   // tasks if no task costs more than c
            int64_t total = 0;
            for (size_t i = 0; i < ns; ++i) {
                if (tiles[i] == 0) continue;
                const int32_t kmax = std::min((c - rows[i]) / 16, kShrinkMaxTiles);
                if (kmax < 1) return INT64_MAX;
                const int32_t mi = (tiles[i] + kmax - 1) / kmax;
                if (store) m[i] = mi;
                total += mi;
            }
            return total;
        };
        int32_t hi = 0, lo = 0;
        for (size_t i = 0; i < ns; ++i) {
            if (tiles[i] == 0) continue;
            hi = std::max(hi, rows[i] + 16 * std::min(tiles[i], (int32_t)kShrinkMaxTiles));
            lo = std::max(lo, rows[i] + 16);
        }
        if (hi == 0) continue;
        int32_t c = hi;
        if (m0 < n_cu) {
            while (lo < hi) {                       // smallest cost whose tasks fit the units
                const int32_t mid = lo + (hi - lo) / 2;
                if (chunks_at(mid, false) <= n_cu) hi = mid;
                else lo = mid + 1;
            }
            c = hi;
        }
        chunks_at(c, true);
        items.clear();
        for (size_t i = 0; i < ns; ++i) {
            if (tiles[i] == 0) continue;
            const int32_t base = tiles[i] / m[i], extra = tiles[i] % m[i];
            int32_t c0 = 0;
            for (int32_t k = 0; k < m[i]; ++k) {
                const int32_t cnt = base + (k < extra ? 1 : 0);
                items.push_back({(int32_t)i, c0, cnt, rows[i] + 16 * cnt});
                c0 += cnt;
            }
        }
        if ((int64_t)items.size() < kShrinkMinBlocks) continue;
        // Block b runs on XCD b % kXcds.  The tasks of one segment share its
        // x rows, so a segment goes to one XCD (its L2 then reads them once):
        // segments by decreasing cost to the XCD with the least cost among
        // those with room for its tasks (an equal share of the units).
        seg_cost.assign(ns, 0);
        seg_tasks.assign(ns, 0);
        for (const Item &it : items) {
            seg_cost[(size_t)it.si] += it.cost;
            ++seg_tasks[(size_t)it.si];
        }
        // segments by decreasing cost, equal costs in segment order (a
        // counting sort: costs are small integers)
        int64_t top = 0;
        for (size_t i = 0; i < ns; ++i) top = std::max(top, seg_cost[i]);
        bucket.assign((size_t)top + 2, 0);
        for (size_t i = 0; i < ns; ++i)
            if (seg_tasks[i]) ++bucket[(size_t)(top - seg_cost[i]) + 1];
        for (size_t k = 1; k < bucket.size(); ++k) bucket[k] += bucket[k - 1];
        order.assign((size_t)bucket.back(), 0);
        for (size_t i = 0; i < ns; ++i)
            if (seg_tasks[i]) order[(size_t)bucket[(size_t)(top - seg_cost[i])]++] = (int32_t)i;
        const int64_t room = std::max<int64_t>((int64_t)(items.size() + kXcds - 1) / kXcds,
                                               n_cu / kXcds);
        int64_t xcost[kXcds] = {}, xcount[kXcds] = {};
        xcd_of.assign(ns, 0);
        for (int32_t i : order) {
            int best = -1;
            for (int x = 0; x < kXcds; ++x)
                if (xcount[x] + seg_tasks[i] <= room && (best < 0 || xcost[x] < xcost[best]))
                    best = x;
            if (best < 0)
                for (int x = 0; x < kXcds; ++x)
                    if (best < 0 || xcount[x] < xcount[best]) best = x;
            xcd_of[i] = best;
            xcost[best] += seg_cost[i];
            xcount[best] += seg_tasks[i];
        }
        // per XCD heaviest first (tasks by decreasing cost, equal costs in
        // segment order), interleaved so that block b is its XCD's
        // (b / kXcds)-th task; empty places hold kMfmaTaskNone
        {
            int32_t most = 0;
            for (const Item &it : items) most = std::max(most, it.cost);
            bucket.assign((size_t)most + 2, 0);
            for (const Item &it : items) ++bucket[(size_t)(most - it.cost) + 1];
            for (size_t k = 1; k < bucket.size(); ++k) bucket[k] += bucket[k - 1];
            sorted.resize(items.size());
            for (const Item &it : items) sorted[(size_t)bucket[(size_t)(most - it.cost)]++] = it;
            items.swap(sorted);
        }
        int64_t longest = 0;
        for (int x = 0; x < kXcds; ++x) longest = std::max(longest, xcount[x]);
        pl.mtask_off[sc] = (int32_t)pl.mtasks.size();
        pl.mtask_n[sc] = (int32_t)(longest * kXcds);
        pl.mtasks.resize(pl.mtasks.size() + (size_t)(longest * kXcds), kMfmaTaskNone);
        int64_t next[kXcds] = {};
        for (const Item &it : items) {
            const int x = xcd_of[(size_t)it.si];
            pl.mtasks[(size_t)(pl.mtask_off[sc] + next[x]++ * kXcds + x)] =
                mfma_task_word(it.si, it.c0, it.cnt);
            pl.mtask_tiles[sc] = std::max(pl.mtask_tiles[sc], it.cnt);
            pl.mtask_rows[sc] = std::max(pl.mtask_rows[sc], rows[(size_t)it.si]);
        }
    }
    const int64_t budget = (int64_t)max_tokens * (2 * kSegWords + 2) - pl.off_mtasks() - 64;
    if ((int64_t)pl.mtasks.size() > budget) {
        pl.mtasks.clear();
        for (int s = 0; s <= kMetaStride; ++s) pl.mtask_off[s] = pl.mtask_n[s] = 0;
    }
}

void append_inactive_rows(Plan &pl)
{
    const size_t n_active = pl.rows.size(), n = pl.tok.size();
    pl.rows.resize(n_active + n + 1);
    int32_t *w = pl.rows.data();
    size_t k = n_active;
    for (size_t t = 0; t < n; ++t) {   // branch-free: every row is written, kept if inactive
        w[k] = (int32_t)t;
        k += pl.tok[t] == 0;
    }
    pl.rows.resize(k);
}

template <class Ranks>
void push_seg(std::vector<int32_t> &seg, int32_t slot, int32_t v_row, int32_t n, int32_t kind,
              Ranks ranks)
{
    seg.push_back(slot);
    seg.push_back(v_row);
    seg.push_back(n);
    seg.push_back(kind);
    for (int j = 0; j < kMetaStride; ++j) seg.push_back(ranks(slot, j));
}

// Admission, per-token slots and segments of one candidate batch, on the host.
// `resolve(id)` gives the slot of a resident id, or 0; `ranks(slot, j)` the
// rank of slice j held in that slot.
template <class Resolve, class Ranks>
int32_t plan_routing(int32_t n_seq, const int32_t *seq_adapter_id, const int32_t *seq_len,
                     int32_t max_loras, int32_t prefill_min_len, int32_t max_tokens,
                     int32_t max_slots, Resolve resolve, Ranks ranks, Plan &pl, int32_t n_cu)
{
    if (n_seq < 0) return fail(LORA_ERR_SHAPE, "n_seq < 0");
    if (n_seq > 0 && (!seq_adapter_id || !seq_len))
        return fail(LORA_ERR_ARG, "null per-sequence array");
    if (max_loras < 0) return fail(LORA_ERR_ARG, "max_loras < 0");
    if (prefill_min_len < 1) return fail(LORA_ERR_ARG, "prefill_min_len < 1");
    int64_t T = 0;
    for (int i = 0; i < n_seq; ++i) {
        if (seq_len[i] < 0) return fail(LORA_ERR_SHAPE, "seq_len[%d] < 0", i);
        if (seq_adapter_id[i] < 0) return fail(LORA_ERR_ARG, "seq_adapter_id[%d] < 0", i);
        T += seq_len[i];
    }
    if (T > max_tokens)
        return fail(LORA_ERR_CAPACITY, "batch has %lld rows > max_tokens=%d", (long long)T,
                    max_tokens);

    // Admission (tokenspeed PR #976, max_loras batch cap): walk in order; base
    // is free, an adapter already admitted is free, a new adapter past the cap
    // is deferred and the walk goes on; max_loras == 0 means no cap.
    std::vector<uint8_t> &adm = pl.adm;
    adm.assign((size_t)n_seq, 0);
    std::vector<int32_t> seq_slot((size_t)n_seq, 0);
    std::vector<int32_t> distinct_ids;
    std::unordered_map<int32_t, int32_t> id_slot;
    for (int i = 0; i < n_seq; ++i) {
        const int32_t id = seq_adapter_id[i];
        if (id == 0) {
            adm[i] = 1;
            continue;
        }
        auto it = id_slot.find(id);
        if (it != id_slot.end()) {
            adm[i] = 1;
            seq_slot[i] = it->second;
        } else if (max_loras == 0 || (int32_t)distinct_ids.size() < max_loras) {
            const int32_t s = resolve(id);
            if (s < 1 || s > max_slots)
                return fail(LORA_ERR_UNKNOWN_ADAPTER,
                            "sequence %d names adapter %d, which is not resident", i, id);
            id_slot.emplace(id, s);
            distinct_ids.push_back(id);
            adm[i] = 1;
            seq_slot[i] = s;
        }
    }

    // Per-token slots; decode rows counted per slot in order of first appearance.
    pl.tok.assign((size_t)T, 0);
    std::vector<int32_t> count((size_t)max_slots + 1, 0);
    std::vector<int32_t> slot_order;
    int64_t row0 = 0, n_dec = 0, n_pre = 0;
    for (int i = 0; i < n_seq; ++i) {
        const int32_t L = seq_len[i], s = seq_slot[i];
        if (s != 0 && L > 0) {
            std::fill(pl.tok.begin() + row0, pl.tok.begin() + row0 + L, s);
            if (L >= prefill_min_len) {
                n_pre += L;
            } else {
                if (count[s] == 0) slot_order.push_back(s);
                count[s] += L;
                n_dec += L;
            }
        }
        row0 += L;
    }
    // Decode rows of an adapter with a slice rank >= kGatherMinRank take the
    // matrix-core path in gather segments; the others the GEMV path.
    auto gathered = [&](int32_t s) {
        int32_t m = 0;
        for (int j = 0; j < kMetaStride; ++j) m = std::max(m, ranks(s, j));
        return m >= kGatherMinRank;
    };
    // Active rows (the rows of v): GEMV decode rows by slot in order of first
    // appearance, then prefill rows, then gathered decode rows by slot.
    std::vector<int32_t> start((size_t)max_slots + 1, 0);
    int64_t n_dec_gemv = 0;
    {
        int64_t acc = 0;
        for (int32_t s : slot_order)
            if (!gathered(s)) {
                start[s] = (int32_t)acc;
                acc += count[s];
            }
        n_dec_gemv = acc;
        acc += n_pre;
        for (int32_t s : slot_order)
            if (gathered(s)) {
                start[s] = (int32_t)acc;
                acc += count[s];
            }
    }
    pl.rows.assign((size_t)(n_dec + n_pre), 0);
    pl.seg.clear();
    // decode rows: token order within a slot; GEMV slots in chunks of kDecodeSegRows
    {
        std::vector<int32_t> fill = start;
        row0 = 0;
        for (int i = 0; i < n_seq; ++i) {
            const int32_t L = seq_len[i], s = seq_slot[i];
            if (s != 0 && L > 0 && L < prefill_min_len)
                for (int32_t t = 0; t < L; ++t) pl.rows[(size_t)fill[s]++] = (int32_t)(row0 + t);
            row0 += L;
        }
        for (int32_t s : slot_order)
            if (!gathered(s))
                for (int32_t b = 0; b < count[s]; b += kDecodeSegRows) {
                    const int32_t n = std::min(kDecodeSegRows, count[s] - b);
                    push_seg(pl.seg, s, start[s] + b, n, kSegDecode, ranks);
                    for (int32_t c = 0; c < kDecodeSegRows; ++c)
                        pl.seg.push_back(pl.rows[(size_t)(start[s] + b + std::min(c, n - 1))]);
                }
    }
    const int32_t n_dec_seg = (int32_t)(pl.seg.size() / kSegWords);
    // prefill sequences: contiguous chunks of kPrefillSegRows rows, one slot each
    {
        int64_t pos = n_dec_gemv;
        row0 = 0;
        for (int i = 0; i < n_seq; ++i) {
            const int32_t L = seq_len[i], s = seq_slot[i];
            if (s != 0 && L >= prefill_min_len)
                for (int32_t b = 0; b < L; b += kPrefillSegRows) {
                    const int32_t n = std::min(kPrefillSegRows, L - b);
                    push_seg(pl.seg, s, (int32_t)pos, n, kSegPrefill, ranks);
                    pl.seg.push_back((int32_t)(row0 + b));
                    for (int32_t c = 1; c < kDecodeSegRows; ++c) pl.seg.push_back(0);
                    for (int32_t t = 0; t < n; ++t) pl.rows[(size_t)pos++] = (int32_t)(row0 + b + t);
                }
            row0 += L;
        }
    }
    const int32_t n_pre_seg = (int32_t)(pl.seg.size() / kSegWords) - n_dec_seg;
    // gathered decode rows: chunks of kPrefillSegRows rows of one slot
    pl.max_gather_rows = 0;
    for (int32_t s : slot_order)
        if (gathered(s))
            for (int32_t b = 0; b < count[s]; b += kPrefillSegRows) {
                const int32_t n = std::min(kPrefillSegRows, count[s] - b);
                push_seg(pl.seg, s, start[s] + b, n, kSegGather, ranks);
                for (int32_t c = 0; c < kDecodeSegRows; ++c) pl.seg.push_back(0);
                pl.max_gather_rows = std::max(pl.max_gather_rows, n);
            }
    const int32_t n_seg = (int32_t)(pl.seg.size() / kSegWords);
    pl.info.n_tokens = (int32_t)T;
    pl.info.n_active = (int32_t)(n_dec + n_pre);
    pl.info.n_segments = n_seg;
    pl.info.n_decode_segments = n_dec_seg;
    pl.info.n_prefill_segments = n_pre_seg;
    pl.info.n_gather_segments = n_seg - n_dec_seg - n_pre_seg;
    pl.info.n_distinct = (int32_t)distinct_ids.size();
    pl.info.n_seqs = n_seq;
    fill_row_meta(pl, ranks);
    append_inactive_rows(pl);
    fill_gemv_tasks(pl, max_tokens);
    fill_mfma_tasks(pl, max_tokens, n_cu);
    int32_t na = 0;
    for (int i = 0; i < n_seq; ++i) na += adm[i];
    pl.info.n_admitted_seqs = na;
    pl.distinct_slots.clear();
    pl.slot_ranks.clear();
    for (int32_t id : distinct_ids) {
        const int32_t s = id_slot[id];
        pl.distinct_slots.push_back(s);
        for (int j = 0; j < kMetaStride; ++j) pl.slot_ranks.push_back(ranks(s, j));
    }
    return LORA_OK;
}


// Segments of a batch given one slot per row (0 = skip), on the host: the
// dispatched rows of a MoE layer, whose (adapter, expert) slots the caller
// resolved.  A decode row of a slot whose largest slice rank is below
// kGatherMinRank takes the GEMV path (decode segments of up to
// kDecodeSegRows rows); a prefill row, or a row of a higher-rank slot, takes
// the matrix-core path (gather segments of up to kPrefillSegRows rows of one
// slot).  A row's path so depends only on its own kind and slot.  Rows of a
// slot are in row order; v holds the GEMV rows, then the gathered rows.
template <class Ranks>
void plan_rows(int32_t n_rows, const int32_t *row_slot, const uint8_t *row_prefill,
               int32_t max_slots, Ranks ranks, Plan &pl, int32_t n_cu)
{
    auto high_rank = [&](int32_t s) {
        int32_t m = 0;
        for (int j = 0; j < kMetaStride; ++j) m = std::max(m, ranks(s, j));
        return m >= kGatherMinRank;
    };
    // rows per (slot, path), counted, then placed in row order: GEMV rows
    // of the slots in first-appearance order, then gathered rows likewise
    std::vector<int32_t> n_gemv((size_t)max_slots + 1, 0), n_gath((size_t)max_slots + 1, 0);
    std::vector<uint8_t> is_gath((size_t)n_rows, 0);
    std::vector<uint8_t> high((size_t)max_slots + 1, 0);   // high_rank of each slot seen
    std::vector<int32_t> order;
    pl.tok.assign((size_t)n_rows, 0);
    // (slot 0's counts are kept too, and never read: no branch on base rows)
    for (int32_t i = 0; i < n_rows; ++i) {
        const int32_t s = row_slot[i];
        pl.tok[(size_t)i] = s;
        if (s != 0 && n_gemv[s] == 0 && n_gath[s] == 0) {
            order.push_back(s);
            high[(size_t)s] = high_rank(s);
        }
        const bool g = (row_prefill && row_prefill[i]) || high[(size_t)s];
        is_gath[(size_t)i] = g;
        ++(g ? n_gath : n_gemv)[s];
    }
    std::vector<int32_t> at_gemv((size_t)max_slots + 1, 0), at_gath((size_t)max_slots + 1, 0);
    int64_t n_gemv_rows = 0, g_rows = 0, g_slots = 0;
    for (int32_t s : order) {
        at_gemv[s] = (int32_t)n_gemv_rows;
        n_gemv_rows += n_gemv[s];
    }
    for (int32_t s : order) {
        at_gath[s] = (int32_t)(n_gemv_rows + g_rows);
        g_rows += n_gath[s];
        g_slots += n_gath[s] > 0;
    }
    pl.rows.assign((size_t)(n_gemv_rows + g_rows), 0);
    {
        std::vector<int32_t> fg = at_gemv, fa = at_gath;
        for (int32_t i = 0; i < n_rows; ++i) {
            const int32_t s = row_slot[i];
            if (s == 0) continue;
            pl.rows[(size_t)(is_gath[(size_t)i] ? fa[s]++ : fg[s]++)] = i;
        }
    }
    pl.seg.clear();
    for (int32_t s : order)
        for (int32_t b = 0; b < n_gemv[s]; b += kDecodeSegRows) {
            const int32_t n = std::min(kDecodeSegRows, n_gemv[s] - b);
            push_seg(pl.seg, s, at_gemv[s] + b, n, kSegDecode, ranks);
            for (int32_t c = 0; c < kDecodeSegRows; ++c)
                pl.seg.push_back(pl.rows[(size_t)(at_gemv[s] + b + std::min(c, n - 1))]);
        }
    const int32_t n_dec_seg = (int32_t)(pl.seg.size() / kSegWords);
    // Groups of a few rows each (the usual MoE case: many (adapter, expert)
    // pairs) are cut into segments of kSmallGatherRows, so that the expand
    // runs one wave per segment; larger groups keep kPrefillSegRows rows and
    // read their factors fewer times.  Gathered rows' bits do not depend on
    // how they are cut.
    const int32_t g_size = g_rows <= (int64_t)kSmallGatherRows * g_slots ? kSmallGatherRows
                                                                         : kPrefillSegRows;
    pl.max_gather_rows = 0;
    for (int32_t s : order)
        for (int32_t b = 0; b < n_gath[s]; b += g_size) {
            const int32_t n = std::min(g_size, n_gath[s] - b);
            push_seg(pl.seg, s, at_gath[s] + b, n, kSegGather, ranks);
            for (int32_t c = 0; c < kDecodeSegRows; ++c) pl.seg.push_back(0);
            pl.max_gather_rows = std::max(pl.max_gather_rows, n);
        }
    const int32_t n_seg = (int32_t)(pl.seg.size() / kSegWords);
    pl.info = lora_routing_info{};
    pl.info.n_tokens = n_rows;
    pl.info.n_active = (int32_t)pl.rows.size();
    pl.info.n_segments = n_seg;
    pl.info.n_decode_segments = n_dec_seg;
    pl.info.n_prefill_segments = 0;
    pl.info.n_gather_segments = n_seg - n_dec_seg;
    pl.info.n_distinct = (int32_t)order.size();
    pl.info.n_seqs = pl.info.n_admitted_seqs = n_rows;
    fill_row_meta(pl, ranks);
    append_inactive_rows(pl);
    fill_gemv_tasks(pl, n_rows);
    fill_mfma_tasks(pl, n_rows, n_cu);
    pl.adm.clear();
    pl.distinct_slots = order;
    pl.slot_ranks.clear();
    for (int32_t s : order)
        for (int j = 0; j < kMetaStride; ++j) pl.slot_ranks.push_back(ranks(s, j));
}

int32_t upload_plan(const lora_pool *p, lora_routing *r, void *stream);

}  // namespace

extern "C" {

const char *lora_last_error(void) { return g_err.c_str(); }

const char *lora_version(void) { return "adapter_deltas_amd 0.1 (gfx950)"; }

// ------------------------------------------------------------------ pool --

int32_t lora_pool_bytes(const lora_lane_desc *desc, int64_t *bytes_out)
{
    if (int32_t rc = check_desc(desc)) return rc;
    if (!bytes_out) return fail(LORA_ERR_ARG, "bytes_out is null");
    LaneGeom g;
    make_geom(*desc, g);
    *bytes_out = pool_layout(*desc, g).total;
    return LORA_OK;
}

int32_t lora_pool_create(const lora_lane_desc *desc, void *dev_mem, int64_t dev_bytes,
                         void *stream, lora_pool **pool_out)
{
    if (int32_t rc = check_desc(desc)) return rc;
    if (!dev_mem || !pool_out) return fail(LORA_ERR_ARG, "dev_mem or pool_out is null");
    if (reinterpret_cast<uintptr_t>(dev_mem) % 256)
        return fail(LORA_ERR_SHAPE, "pool memory must be 256-byte aligned");
    LaneGeom g;
    make_geom(*desc, g);
    PoolLayout L = pool_layout(*desc, g);
    if (dev_bytes < L.total)
        return fail(LORA_ERR_CAPACITY, "pool memory %lld bytes < %lld needed",
                    (long long)dev_bytes, (long long)L.total);
    lora_pool *p = new (std::nothrow) lora_pool();
    if (!p) return fail(LORA_ERR_CAPACITY, "out of host memory");
    p->desc = *desc;
    p->geom = g;
    char *base = static_cast<char *>(dev_mem);
    p->A = reinterpret_cast<uint16_t *>(base + L.a_off);
    p->Bt = reinterpret_cast<uint16_t *>(base + L.bt_off);
    p->Bn = reinterpret_cast<uint16_t *>(base + L.bn_off);
    p->rank_tab = reinterpret_cast<int32_t *>(base + L.rank_off);
    p->scale_tab = reinterpret_cast<float *>(base + L.scale_off);
    p->h_rank.assign((size_t)(desc->max_slots + 1) * kMetaStride, 0);
    p->h_scale.assign((size_t)(desc->max_slots + 1) * kMetaStride, 0.f);
    p->slot_to_id.assign((size_t)desc->max_slots + 1, 0);
    hipError_t e = launch_clear_meta(p->rank_tab, p->scale_tab, desc->max_slots + 1,
                                     static_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
        delete p;
        return hip_fail(e, "clearing pool metadata");
    }
    *pool_out = p;
    return LORA_OK;
}

int32_t lora_pool_destroy(lora_pool *pool)
{
    delete pool;
    return LORA_OK;
}

int32_t lora_pool_load(lora_pool *p, int32_t adapter_id, int32_t slot, const void *const *A,
                       const int64_t *lda, int64_t a_col0, const void *const *B,
                       const int64_t *ldb, const int32_t *rank, const float *scale,
                       int32_t src_on_device, void *stream, int32_t *slot_out)
{
    if (!p || !A || !lda || !B || !ldb || !rank || !scale)
        return fail(LORA_ERR_ARG, "null argument to lora_pool_load");
    if (adapter_id <= 0)
        return fail(LORA_ERR_ARG, "adapter id %d: ids are > 0 (0 is the base model)", adapter_id);
    if (src_on_device != 0 && src_on_device != 1)
        return fail(LORA_ERR_ARG, "src_on_device must be 0 or 1");
    const lora_lane_desc &d = p->desc;
    if (slot == 0 || slot < -1 || slot > d.max_slots)
        return fail(LORA_ERR_SLOT, "slot %d: slots are 1..%d (or -1 for any)", slot, d.max_slots);
    if (a_col0 < 0) return fail(LORA_ERR_SHAPE, "a_col0 < 0");
    for (int j = 0; j < d.n_slices; ++j) {
        if (!A[j] || !B[j]) return fail(LORA_ERR_ARG, "slice %d: null factor", j);
        if (rank[j] < 1 || rank[j] > d.max_rank)
            return fail(LORA_ERR_RANK, "slice %d: rank %d outside 1..%d", j, rank[j], d.max_rank);
        if (!std::isfinite(scale[j]))
            return fail(LORA_ERR_ARG, "slice %d: scale is not finite", j);
        if (lda[j] < a_col0 + d.h_in)
            return fail(LORA_ERR_SHAPE, "slice %d: lda %lld < a_col0 + h_in = %lld", j,
                        (long long)lda[j], (long long)(a_col0 + d.h_in));
        if (ldb[j] < rank[j])
            return fail(LORA_ERR_SHAPE, "slice %d: ldb %lld < rank %d", j, (long long)ldb[j],
                        rank[j]);
    }
    auto it = p->id_to_slot.find(adapter_id);
    int target = slot;
    if (target == -1) {
        if (it != p->id_to_slot.end()) {
            target = it->second;
        } else {
            for (int s = 1; s <= d.max_slots; ++s)
                if (p->slot_to_id[s] == 0) {
                    target = s;
                    break;
                }
            if (target == -1)
                return fail(LORA_ERR_CAPACITY, "all %d slots are taken", d.max_slots);
        }
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    const LaneGeom &g = p->geom;
    // An id moving to another slot leaves its old slot empty: that slot's
    // ranks go to zero on the device too (as lora_pool_unload does), so a
    // routing built on the device treats it as holding no adapter.
    const int32_t vacated =
        (it != p->id_to_slot.end() && it->second != target) ? it->second : 0;
    hipError_t e = hipSuccess;
    if (vacated) e = launch_set_meta(p->rank_tab, p->scale_tab, vacated, 0, nullptr, nullptr, st);
    if (e != hipSuccess) return hip_fail(e, "clearing the vacated slot's ranks");
    if (src_on_device) {
        for (int j = 0; j < d.n_slices && e == hipSuccess; ++j) {
            e = launch_pack_a(slot_a(p, target, j), static_cast<const uint16_t *>(A[j]), lda[j],
                              a_col0, rank[j], g.rank_pad, d.h_in, st);
            if (e == hipSuccess)
                e = launch_pack_bt(slot_bt(p, target, j), static_cast<const uint16_t *>(B[j]),
                                   ldb[j], rank[j], g.rank_pad, d.h_out[j], st);
            if (e == hipSuccess)
                e = launch_pack_bn(slot_bn(p, target, j), static_cast<const uint16_t *>(B[j]),
                                   ldb[j], rank[j], g.rank_pad, d.h_out[j], st);
        }
        if (e == hipSuccess) e = launch_set_meta(p->rank_tab, p->scale_tab, target, d.n_slices,
                                                  rank, scale, st);
        if (e != hipSuccess) return hip_fail(e, "packing adapter factors");
    } else {
        std::vector<uint16_t> pa((size_t)g.a_slot_stride, 0), pb((size_t)g.bt_slot_stride, 0);
        std::vector<uint16_t> pn((size_t)g.bt_slot_stride, 0);
        for (int j = 0; j < d.n_slices; ++j) {
            const uint16_t *a = static_cast<const uint16_t *>(A[j]);
            const uint16_t *b = static_cast<const uint16_t *>(B[j]);
            uint16_t *da = pa.data() + (size_t)j * g.rank_pad * d.h_in;
            for (int k = 0; k < rank[j]; ++k)
                std::memcpy(da + (size_t)k * d.h_in, a + k * lda[j] + a_col0,
                            (size_t)d.h_in * 2);
            uint16_t *db = pb.data() + g.bt_slice_off[j];
            const int hj = d.h_out[j];
            uint16_t *dn = pn.data() + g.bt_slice_off[j];
            for (int o = 0; o < hj; ++o)
                for (int k = 0; k < rank[j]; ++k) {
                    db[(size_t)k * hj + o] = b[o * ldb[j] + k];
                    dn[(size_t)o * g.rank_pad + k] = b[o * ldb[j] + k];
                }
        }
        e = hipMemcpyAsync(slot_a(p, target, 0), pa.data(), pa.size() * 2,
                           hipMemcpyHostToDevice, st);
        if (e == hipSuccess)
            e = hipMemcpyAsync(slot_bt(p, target, 0), pb.data(), pb.size() * 2,
                               hipMemcpyHostToDevice, st);
        if (e == hipSuccess)
            e = hipMemcpyAsync(slot_bn(p, target, 0), pn.data(), pn.size() * 2,
                               hipMemcpyHostToDevice, st);
        if (e == hipSuccess)
            e = launch_set_meta(p->rank_tab, p->scale_tab, target, d.n_slices, rank, scale, st);
        if (e == hipSuccess) e = hipStreamSynchronize(st);
        if (e != hipSuccess) return hip_fail(e, "copying adapter factors");
    }
    // bookkeeping: evict this id from an old slot, and the old occupant of target
    if (vacated) {
        p->slot_to_id[vacated] = 0;
        for (int j = 0; j < kMetaStride; ++j) {
            p->h_rank[(size_t)vacated * kMetaStride + j] = 0;
            p->h_scale[(size_t)vacated * kMetaStride + j] = 0.f;
        }
    }
    if (int32_t old = p->slot_to_id[target]; old != 0 && old != adapter_id)
        p->id_to_slot.erase(old);
    p->id_to_slot[adapter_id] = target;
    p->slot_to_id[target] = adapter_id;
    for (int j = 0; j < kMetaStride; ++j) {
        p->h_rank[(size_t)target * kMetaStride + j] = j < d.n_slices ? rank[j] : 0;
        p->h_scale[(size_t)target * kMetaStride + j] = j < d.n_slices ? scale[j] : 0.f;
    }
    if (slot_out) *slot_out = target;
    return LORA_OK;
}

int32_t lora_pool_load_folded(lora_pool *p, int32_t adapter_id, int32_t slot,
                              const void *const *A, const int64_t *lda, int64_t a_col0,
                              const void *const *B, const int64_t *ldb, const int32_t *rank,
                              const float *scale, const float *fold, int64_t ld_fold,
                              void *stream, int32_t *slot_out)
{
    if (!p || !A || !lda || !rank) return fail(LORA_ERR_ARG, "null argument");
    if (!fold) return fail(LORA_ERR_ARG, "fold is null");
    if (ld_fold < p->desc.h_in)
        return fail(LORA_ERR_SHAPE, "ld_fold=%lld < h_in=%d", (long long)ld_fold, p->desc.h_in);
    if (reinterpret_cast<uintptr_t>(fold) % 4) return fail(LORA_ERR_SHAPE, "fold is not 4-byte aligned");
    int32_t target = 0;
    if (int32_t rc = lora_pool_load(p, adapter_id, slot, A, lda, a_col0, B, ldb, rank, scale, 1,
                                    stream, &target))
        return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    for (int j = 0; j < p->desc.n_slices; ++j) {
        hipError_t e = launch_fold_a(slot_a(p, target, j), static_cast<const uint16_t *>(A[j]),
                                     lda[j], a_col0, rank[j], p->desc.h_in, fold, ld_fold, st);
        if (e != hipSuccess) return hip_fail(e, "folding A");
    }
    if (slot_out) *slot_out = target;
    return LORA_OK;
}

int32_t lora_pool_unload(lora_pool *p, int32_t adapter_id)
{
    if (!p) return fail(LORA_ERR_ARG, "pool is null");
    auto it = p->id_to_slot.find(adapter_id);
    if (it == p->id_to_slot.end())
        return fail(LORA_ERR_UNKNOWN_ADAPTER, "adapter %d is not resident", adapter_id);
    const int32_t slot = it->second;
    // The slot's ranks go to zero on the device too, so that a routing built
    // on the device sees it as holding no adapter.
    const int32_t zero[kMetaStride] = {};
    hipError_t e = hipMemcpy(p->rank_tab + (size_t)slot * kMetaStride, zero,
                             sizeof zero, hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(e, "clearing the slot's ranks");
    for (int j = 0; j < kMetaStride; ++j) {
        p->h_rank[(size_t)slot * kMetaStride + j] = 0;
        p->h_scale[(size_t)slot * kMetaStride + j] = 0.f;
    }
    p->slot_to_id[slot] = 0;
    p->id_to_slot.erase(it);
    return LORA_OK;
}

int32_t lora_pool_slot_of(const lora_pool *p, int32_t adapter_id, int32_t *slot_out)
{
    if (!p || !slot_out) return fail(LORA_ERR_ARG, "null argument");
    auto it = p->id_to_slot.find(adapter_id);
    if (it == p->id_to_slot.end())
        return fail(LORA_ERR_UNKNOWN_ADAPTER, "adapter %d is not resident", adapter_id);
    *slot_out = it->second;
    return LORA_OK;
}

// --------------------------------------------------------------- routing --

int32_t lora_routing_bytes(int32_t max_tokens, int64_t *bytes_out)
{
    if (max_tokens < 1 || max_tokens > (1 << 26))
        return fail(LORA_ERR_SHAPE, "max_tokens=%d outside 1..2^26", max_tokens);
    if (!bytes_out) return fail(LORA_ERR_ARG, "bytes_out is null");
    // segments (kSegWords each: at most one per active row on the host, a
    // decode and a gather bound of at most max_tokens each on the device)
    // + row list + token slots + device counts
    *bytes_out = round_up((int64_t)max_tokens * (2 * kSegWords + 2) * 4 + 256, 256);
    return LORA_OK;
}

int32_t lora_routing_create(int32_t max_tokens, int32_t max_seqs, void *dev_mem,
                            int64_t dev_bytes, lora_routing **routing_out)
{
    int64_t need = 0;
    if (int32_t rc = lora_routing_bytes(max_tokens, &need)) return rc;
    if (max_seqs < 1 || max_seqs > (1 << 26))
        return fail(LORA_ERR_SHAPE, "max_seqs=%d outside 1..2^26", max_seqs);
    if (!dev_mem || !routing_out) return fail(LORA_ERR_ARG, "dev_mem or routing_out is null");
    if (reinterpret_cast<uintptr_t>(dev_mem) % 16)
        return fail(LORA_ERR_SHAPE, "routing memory must be 16-byte aligned");
    if (dev_bytes < need)
        return fail(LORA_ERR_CAPACITY, "routing memory %lld bytes < %lld needed",
                    (long long)dev_bytes, (long long)need);
    lora_routing *r = new (std::nothrow) lora_routing();
    if (!r) return fail(LORA_ERR_CAPACITY, "out of host memory");
    r->max_tokens = max_tokens;
    r->max_seqs = max_seqs;
    r->dev = static_cast<int32_t *>(dev_mem);
    r->dev_words = need / 4;
    r->stage[0] = r->stage[1] = nullptr;
    r->stage_done[0] = r->stage_done[1] = nullptr;
    for (int i = 0; i < 2; ++i) {
        hipError_t e = hipHostMalloc(reinterpret_cast<void **>(&r->stage[i]), need,
                                     hipHostMallocDefault);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&r->stage_done[i], hipEventDisableTiming);
        if (e != hipSuccess) {
            lora_routing_destroy(r);
            return hip_fail(e, "allocating routing staging");
        }
    }
    r->stage_next = 0;
    {
        // the second stream of mixed batches, at the default priority
        hipError_t e = hipStreamCreateWithFlags(&r->side, hipStreamNonBlocking);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&r->fork_ev, hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&r->join_ev, hipEventDisableTiming);
        if (e != hipSuccess) {
            lora_routing_destroy(r);
            return hip_fail(e, "creating the routing's second stream");
        }
    }
    std::memset(&r->info, 0, sizeof r->info);
    r->off_seg = r->off_row = r->off_tok = r->off_meta = 0;
    r->tile_steps[0] = r->tile_steps[1] = 0;
    r->off_tasks = r->n_tasks = 0;
    for (int sc = 0; sc <= kMetaStride; ++sc)
        r->off_mtasks[sc] = r->n_mtasks[sc] = r->mtask_tiles[sc] = r->mtask_rows[sc] = 0;
    {
        // compute units of the current device (the shrink task tables are cut for them)
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            n > 0)
            r->n_cu = n;
        else
            r->n_cu = kPlanComputeUnits;
    }
    r->pool_max_slots = 0;
    r->device_built = false;
    r->off_counts = 0;
    r->max_gather_rows = 0;
    *routing_out = r;
    return LORA_OK;
}

int32_t lora_routing_destroy(lora_routing *r)
{
    if (!r) return LORA_OK;
    if (r->side) {
        (void)hipStreamSynchronize(r->side);
        (void)hipStreamDestroy(r->side);
    }
    if (r->fork_ev) (void)hipEventDestroy(r->fork_ev);
    if (r->join_ev) (void)hipEventDestroy(r->join_ev);
    for (int i = 0; i < 2; ++i) {
        if (r->stage_done[i]) {
            (void)hipEventSynchronize(r->stage_done[i]);
            (void)hipEventDestroy(r->stage_done[i]);
        }
        if (r->stage[i]) (void)hipHostFree(r->stage[i]);
    }
    delete r;
    return LORA_OK;
}

int32_t lora_build_routing(const lora_pool *p, int32_t n_seq, const int32_t *seq_adapter_id,
                           const int32_t *seq_len, int32_t max_loras, int32_t prefill_min_len,
                           lora_routing *r, uint8_t *admitted_out, int32_t *n_distinct_out,
                           void *stream)
{
    if (!p || !r) return fail(LORA_ERR_ARG, "pool or routing is null");
    if (n_seq > r->max_seqs)
        return fail(LORA_ERR_CAPACITY, "n_seq=%d > max_seqs=%d", n_seq, r->max_seqs);
    Plan &pl = r->plan;
    auto resolve = [p](int32_t id) -> int32_t {
        auto it = p->id_to_slot.find(id);
        return it == p->id_to_slot.end() ? 0 : it->second;
    };
    auto ranks = [p](int32_t slot, int j) -> int32_t {
        return p->h_rank[(size_t)slot * kMetaStride + j];
    };
    if (int32_t rc = plan_routing(n_seq, seq_adapter_id, seq_len, max_loras, prefill_min_len,
                                  r->max_tokens, p->desc.max_slots, resolve, ranks, pl, r->n_cu))
        return rc;
    if (int32_t rc = upload_plan(p, r, stream)) return rc;
    if (admitted_out)
        for (int i = 0; i < n_seq; ++i) admitted_out[i] = pl.adm[i];
    if (n_distinct_out) *n_distinct_out = pl.info.n_distinct;
    return LORA_OK;
}

int32_t lora_build_routing_rows(const lora_pool *p, int32_t n_rows, const int32_t *row_slot,
                                const uint8_t *row_prefill, lora_routing *r, void *stream)
{
    if (!p || !r) return fail(LORA_ERR_ARG, "pool or routing is null");
    if (n_rows < 0) return fail(LORA_ERR_SHAPE, "n_rows < 0");
    if (n_rows > 0 && !row_slot) return fail(LORA_ERR_ARG, "row_slot is null");
    if (n_rows > r->max_tokens)
        return fail(LORA_ERR_CAPACITY, "n_rows=%d > max_tokens=%d", n_rows, r->max_tokens);
    auto ranks = [p](int32_t slot, int j) -> int32_t {
        return p->h_rank[(size_t)slot * kMetaStride + j];
    };
    for (int32_t i = 0; i < n_rows; ++i) {
        const int32_t s = row_slot[i];
        if (s != 0 && (s < 1 || s > p->desc.max_slots || p->slot_to_id[s] == 0))
            return fail(LORA_ERR_SLOT, "row %d names slot %d, which holds no adapter", i, s);
    }
    plan_rows(n_rows, row_slot, row_prefill, p->desc.max_slots, ranks, r->plan, r->n_cu);
    return upload_plan(p, r, stream);
}

}  // extern "C"

namespace {

// Copies r->plan to the routing's device memory (through pinned staging, on
// `stream`) and makes it the routing's current batch.
int32_t upload_plan(const lora_pool *p, lora_routing *r, void *stream)
{
    const Plan &pl = r->plan;
    const int64_t words = pl.words();
    if (words > r->dev_words)
        return fail(LORA_ERR_CAPACITY, "routing needs %lld words > %lld", (long long)words,
                    (long long)r->dev_words);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int b = r->stage_next;
    hipError_t e = hipEventSynchronize(r->stage_done[b]);
    if (e != hipSuccess) return hip_fail(e, "waiting for routing staging");
    pl.pack(r->stage[b]);
    if (words > 0) {
        e = hipMemcpyAsync(r->dev, r->stage[b], (size_t)words * 4, hipMemcpyHostToDevice, st);
        if (e == hipSuccess) e = hipEventRecord(r->stage_done[b], st);
        if (e != hipSuccess) return hip_fail(e, "copying routing to the device");
        r->stage_next = b ^ 1;
    }
    r->off_seg = 0;
    r->off_row = (int32_t)pl.off_row();
    r->off_tok = (int32_t)pl.off_tok();
    r->off_meta = (int32_t)pl.off_meta();
    r->off_tasks = (int32_t)pl.off_tasks();
    r->n_tasks = (int32_t)pl.tasks.size();
    for (int sc = 0; sc <= kMetaStride; ++sc) {
        r->off_mtasks[sc] = (int32_t)(pl.off_mtasks() + pl.mtask_off[sc]);
        r->n_mtasks[sc] = pl.mtask_n[sc];
        r->mtask_tiles[sc] = pl.mtask_tiles[sc];
        r->mtask_rows[sc] = pl.mtask_rows[sc];
    }
    r->tile_steps[0] = pl.tile_steps[0];
    r->tile_steps[1] = pl.tile_steps[1];
    r->device_built = false;
    r->info = pl.info;
    r->pool_max_slots = p->desc.max_slots;
    r->distinct_slots = pl.distinct_slots;
    r->slot_ranks = pl.slot_ranks;
    r->max_gather_rows = pl.max_gather_rows;
    r->decode_rows = 0;
    for (int32_t i = 0; i < pl.info.n_decode_segments; ++i)
        r->decode_rows += pl.seg[(size_t)i * kSegWords + 2];
    // fewer than 4 rows a decode segment on average: sparse
    r->expand_lane_cols = r->decode_rows < 4 * pl.info.n_decode_segments ? 4 : 8;
    return LORA_OK;
}

}  // namespace

extern "C" {

int32_t lora_plan_routing(int32_t n_seq, const int32_t *seq_adapter_id, const int32_t *seq_len,
                          int32_t max_loras, int32_t prefill_min_len, int32_t n_resident,
                          const int32_t *resident_id, const int32_t *resident_slot,
                          const int32_t *resident_rank, int32_t max_slots, int32_t max_tokens,
                          int32_t *words_out,
                          int64_t words_capacity, int32_t *offsets_out,
                          lora_routing_info *info_out, uint8_t *admitted_out)
{
    if (n_resident < 0 || (n_resident > 0 && (!resident_id || !resident_slot)))
        return fail(LORA_ERR_ARG, "bad resident table");
    if (max_slots < 1 || max_slots > 65535)
        return fail(LORA_ERR_SHAPE, "max_slots=%d outside 1..65535", max_slots);
    if (max_tokens < 1) return fail(LORA_ERR_SHAPE, "max_tokens < 1");
    std::unordered_map<int32_t, int32_t> table;
    std::vector<int32_t> rank_of((size_t)(max_slots + 1) * kMetaStride, 0);
    for (int i = 0; i < n_resident; ++i) {
        if (resident_id[i] <= 0 || resident_slot[i] < 1 || resident_slot[i] > max_slots)
            return fail(LORA_ERR_SLOT, "resident entry %d: id %d slot %d", i, resident_id[i],
                        resident_slot[i]);
        table[resident_id[i]] = resident_slot[i];
        if (resident_rank)
            for (int j = 0; j < kMetaStride; ++j)
                rank_of[(size_t)resident_slot[i] * kMetaStride + j] =
                    resident_rank[i * kMetaStride + j];
    }
    auto resolve = [&table](int32_t id) -> int32_t {
        auto it = table.find(id);
        return it == table.end() ? 0 : it->second;
    };
    auto ranks = [&rank_of](int32_t slot, int j) -> int32_t {
        return rank_of[(size_t)slot * kMetaStride + j];
    };
    Plan pl;
    if (int32_t rc = plan_routing(n_seq, seq_adapter_id, seq_len, max_loras, prefill_min_len,
                                  max_tokens, max_slots, resolve, ranks, pl, kPlanComputeUnits))
        return rc;
    if (!words_out || !offsets_out || !info_out)
        return fail(LORA_ERR_ARG, "null output");
    if (pl.words() > words_capacity)
        return fail(LORA_ERR_CAPACITY, "plan needs %lld words > %lld", (long long)pl.words(),
                    (long long)words_capacity);
    pl.pack(words_out);
    offsets_out[0] = 0;
    offsets_out[1] = (int32_t)pl.off_row();
    offsets_out[2] = (int32_t)pl.off_tok();
    offsets_out[3] = (int32_t)pl.off_tasks();
    offsets_out[4] = (int32_t)pl.off_mtask_header();
    *info_out = pl.info;
    if (admitted_out)
        for (int i = 0; i < n_seq; ++i) admitted_out[i] = pl.adm[i];
    return LORA_OK;
}

int32_t lora_plan_rows(int32_t n_rows, const int32_t *row_slot, const uint8_t *row_prefill,
                       int32_t max_slots, const int32_t *slot_rank, int32_t *words_out,
                       int64_t words_capacity, int32_t *offsets_out,
                       lora_routing_info *info_out)
{
    if (max_slots < 1 || max_slots > 65535)
        return fail(LORA_ERR_SHAPE, "max_slots=%d outside 1..65535", max_slots);
    if (n_rows < 0) return fail(LORA_ERR_SHAPE, "n_rows < 0");
    if ((n_rows > 0 && !row_slot) || !slot_rank || !words_out || !offsets_out || !info_out)
        return fail(LORA_ERR_ARG, "null argument");
    auto ranks = [slot_rank](int32_t slot, int j) -> int32_t {
        return slot_rank[(size_t)slot * kMetaStride + j];
    };
    for (int32_t i = 0; i < n_rows; ++i) {
        const int32_t s = row_slot[i];
        if (s != 0 && (s < 1 || s > max_slots || ranks(s, 0) < 1))
            return fail(LORA_ERR_SLOT, "row %d names slot %d, which holds no adapter", i, s);
    }
    Plan pl;
    plan_rows(n_rows, row_slot, row_prefill, max_slots, ranks, pl, kPlanComputeUnits);
    if (pl.words() > words_capacity)
        return fail(LORA_ERR_CAPACITY, "plan needs %lld words > %lld", (long long)pl.words(),
                    (long long)words_capacity);
    pl.pack(words_out);
    offsets_out[0] = 0;
    offsets_out[1] = (int32_t)pl.off_row();
    offsets_out[2] = (int32_t)pl.off_tok();
    offsets_out[3] = (int32_t)pl.off_tasks();
    offsets_out[4] = (int32_t)pl.off_mtask_header();
    *info_out = pl.info;
    return LORA_OK;
}

}  // extern "C"

namespace {

// Routing of n_tokens decode rows built on the device (rows = tokens, or the
// dispatched rows of a MoE layer when moe is set).
int32_t build_routing_device(const lora_pool *p, const int32_t *tok_slot, int32_t n_tokens,
                             const MoeDispatch *moe, lora_routing *r, void *stream)
{
    // Bounds: a slot's decode rows make ceil(n / 8) decode or ceil(n / 64)
    // gather segments, so either kind has at most n_tokens / size + slots.
    // A kind no resident adapter takes gets no room (and no launch).
    bool any_dec = false, any_gather = false;
    for (int32_t s = 1; s <= p->desc.max_slots; ++s) {
        if (p->slot_to_id[s] == 0) continue;
        int rmax = 0;
        for (int j = 0; j < kMetaStride; ++j)
            rmax = std::max(rmax, p->h_rank[(size_t)s * kMetaStride + j]);
        (rmax >= kGatherMinRank ? any_gather : any_dec) = true;
    }
    const int64_t slots = std::min<int64_t>(n_tokens, p->desc.max_slots);
    const int32_t max_dec = !any_dec ? 0 : (int32_t)std::min<int64_t>(
        n_tokens, (n_tokens + kDecodeSegRows - 1) / kDecodeSegRows + slots);
    const int32_t max_gather = !any_gather ? 0 : (int32_t)std::min<int64_t>(
        n_tokens, (n_tokens + kPrefillSegRows - 1) / kPrefillSegRows + slots);
    const int64_t off_row = (int64_t)(max_dec + max_gather) * kSegWords;
    const int64_t off_tok = round_up(off_row + n_tokens, 4);
    const int64_t off_counts = round_up(off_tok + n_tokens, 4);
    if (off_counts + kCntWords > r->dev_words)
        return fail(LORA_ERR_CAPACITY, "routing memory too small for %d tokens", n_tokens);
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = launch_route_decode(tok_slot, n_tokens, moe, p->rank_tab, p->desc.max_slots,
                                       max_dec, max_gather, r->dev, r->dev + off_row,
                                       r->dev + off_tok, r->dev + off_counts, st);
    if (e != hipSuccess) return hip_fail(e, "routing kernel launch");
    r->off_seg = 0;
    r->off_row = (int32_t)off_row;
    r->off_tok = (int32_t)off_tok;
    r->off_counts = (int32_t)off_counts;
    r->device_built = true;
    r->n_tasks = 0;
    for (int sc = 0; sc <= kMetaStride; ++sc) r->n_mtasks[sc] = 0;
    r->max_gather_rows = kPrefillSegRows;   // segment sizes are known on the device only
    r->decode_rows = 0;
    // A MoE layer's dispatched rows spread over (adapter, expert) pairs, so
    // its decode segments are sparse; other device-built batches are taken
    // as dense (segment fill is known on the device only).
    r->expand_lane_cols = moe ? 4 : 8;
    r->seg_spread = moe ? kSpreadMoe : kSpreadDense;
    r->pool_max_slots = p->desc.max_slots;
    // Every resident slot may appear in the tables: a pool used with this
    // routing must hold all of them with the same ranks.
    r->distinct_slots.clear();
    r->slot_ranks.clear();
    for (int32_t s = 1; s <= p->desc.max_slots; ++s) {
        if (p->slot_to_id[s] == 0) continue;
        r->distinct_slots.push_back(s);
        for (int j = 0; j < kMetaStride; ++j)
            r->slot_ranks.push_back(p->h_rank[(size_t)s * kMetaStride + j]);
    }
    lora_routing_info &I = r->info;
    std::memset(&I, 0, sizeof I);
    I.n_tokens = n_tokens;
    I.n_active = n_tokens;                  // bounds: the exact counts are on the device
    I.n_decode_segments = max_dec;
    I.n_prefill_segments = 0;
    I.n_gather_segments = max_gather;
    I.n_segments = max_dec + max_gather;
    I.n_seqs = I.n_admitted_seqs = n_tokens;
    return LORA_OK;
}

int32_t check_device_rows(const lora_pool *p, lora_routing *r, int32_t n_rows)
{
    if (!p || !r) return fail(LORA_ERR_ARG, "pool or routing is null");
    if (n_rows < 0) return fail(LORA_ERR_SHAPE, "row count < 0");
    if (n_rows > r->max_tokens || n_rows > LORA_DEVICE_ROUTING_MAX_TOKENS)
        return fail(LORA_ERR_CAPACITY, "%d rows > max_tokens=%d or > %d", n_rows,
                    r->max_tokens, LORA_DEVICE_ROUTING_MAX_TOKENS);
    return LORA_OK;
}

}  // namespace

extern "C" {

int32_t lora_build_routing_device(const lora_pool *p, const int32_t *tok_slot,
                                  int32_t n_tokens, lora_routing *r, void *stream)
{
    if (int32_t rc = check_device_rows(p, r, n_tokens)) return rc;
    if (n_tokens > 0 && !tok_slot) return fail(LORA_ERR_ARG, "tok_slot is null");
    return build_routing_device(p, tok_slot, n_tokens, nullptr, r, stream);
}

int32_t lora_build_routing_moe(const lora_pool *p, const int32_t *tok_slot, int32_t n_tokens,
                               const int32_t *row_token, const int32_t *row_expert,
                               int32_t n_rows, int32_t n_experts, lora_routing *r,
                               void *stream)
{
    if (int32_t rc = check_device_rows(p, r, n_rows)) return rc;
    if (n_tokens < 0) return fail(LORA_ERR_SHAPE, "n_tokens < 0");
    if (n_experts < 1 || p->desc.max_slots % n_experts)
        return fail(LORA_ERR_SHAPE, "n_experts=%d must be >= 1 and divide max_slots=%d",
                    n_experts, p->desc.max_slots);
    if (n_rows > 0 && (!row_token || !row_expert || (n_tokens > 0 && !tok_slot)))
        return fail(LORA_ERR_ARG, "tok_slot, row_token or row_expert is null");
    const MoeDispatch moe{row_token, row_expert, n_tokens, n_experts,
                          p->desc.max_slots / n_experts};
    return build_routing_device(p, tok_slot, n_rows, &moe, r, stream);
}

int32_t lora_routing_device_counts(const lora_routing *r, const int32_t **dev_ptr_out)
{
    if (!r || !dev_ptr_out) return fail(LORA_ERR_ARG, "routing or dev_ptr_out is null");
    if (!r->device_built) return fail(LORA_ERR_ARG, "the routing was built on the host");
    *dev_ptr_out = r->dev + r->off_counts;
    return LORA_OK;
}

int32_t lora_routing_get_info(const lora_routing *r, lora_routing_info *info_out)
{
    if (!r || !info_out) return fail(LORA_ERR_ARG, "null argument");
    *info_out = r->info;
    return LORA_OK;
}

int32_t lora_routing_token_slots(const lora_routing *r, const int32_t **dev_ptr_out)
{
    if (!r || !dev_ptr_out) return fail(LORA_ERR_ARG, "null argument");
    *dev_ptr_out = r->dev + r->off_tok;
    return LORA_OK;
}

// --------------------------------------------------------------- compute --

int32_t lora_shrink(const lora_pool *p, const lora_routing *r, const void *x, int64_t ldx,
                    float *v, void *stream)
{
    if (int32_t rc = check_pair(p, r)) return rc;
    if (r->info.n_active == 0) return LORA_OK;
    if (int32_t rc = check_x(p, x, ldx)) return rc;
    if (int32_t rc = check_v(v)) return rc;
    CallStreams cs;
    if (int32_t rc = fork_streams(r, static_cast<hipStream_t>(stream), cs)) return rc;
    const int32_t rc = enqueue_shrink(p, r, x, ldx, v, cs);
    const int32_t rj = join_streams(r, cs);
    return rc ? rc : rj;
}

int32_t lora_expand(const lora_pool *p, const lora_routing *r, const float *v, float *y,
                    int64_t ldy, void *stream)
{
    if (int32_t rc = check_pair(p, r)) return rc;
    if (r->info.n_active == 0) return LORA_OK;
    if (int32_t rc = check_v(v)) return rc;
    if (int32_t rc = check_y(p, y, ldy)) return rc;
    CallStreams cs;
    if (int32_t rc = fork_streams(r, static_cast<hipStream_t>(stream), cs)) return rc;
    const int32_t rc = enqueue_expand(p, r, v, y, ldy, cs);
    const int32_t rj = join_streams(r, cs);
    return rc ? rc : rj;
}

int32_t lora_workspace_bytes(const lora_pool *p, const lora_routing *r, int64_t *bytes_out)
{
    if (int32_t rc = check_pair(p, r)) return rc;
    if (!bytes_out) return fail(LORA_ERR_ARG, "bytes_out is null");
    *bytes_out = round_up((int64_t)r->info.n_active * p->geom.v_stride * 4, 256);
    return LORA_OK;
}

int32_t lora_delta_apply(const lora_pool *p, const lora_routing *r, const void *x, int64_t ldx,
                         float *y, int64_t ldy, void *workspace, int64_t workspace_bytes,
                         void *stream)
{
    if (int32_t rc = check_pair(p, r)) return rc;
    if (r->info.n_active == 0) return LORA_OK;
    if (!workspace) return fail(LORA_ERR_ARG, "workspace is null");
    return delta_apply_ws(p, r, x, ldx, y, ldy, workspace, workspace_bytes,
                          static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace lora {

int32_t delta_apply_ws(const lora_pool *p, const lora_routing *r, const void *x, int64_t ldx,
                       float *y, int64_t ldy, void *workspace, int64_t workspace_bytes,
                       hipStream_t st)
{
    if (int32_t rc = check_pair(p, r)) return rc;
    if (r->info.n_active == 0) return LORA_OK;
    if (int32_t rc = check_x(p, x, ldx)) return rc;
    if (int32_t rc = check_y(p, y, ldy)) return rc;
    int64_t need = 0;
    lora_workspace_bytes(p, r, &need);
    if (!workspace) return fail(LORA_ERR_ARG, "workspace is null");
    if (!aligned16(workspace)) return fail(LORA_ERR_SHAPE, "workspace must be 16-byte aligned");
    if (workspace_bytes < need)
        return fail(LORA_ERR_CAPACITY, "workspace %lld bytes < %lld needed",
                    (long long)workspace_bytes, (long long)need);
    float *v = static_cast<float *>(workspace);
    // Decode segments of small ranks: shrink and expand in one launch, with
    // the same arithmetic as the two kernels (bit-identical results).  Each
    // column tile of a slice recomputes the segment's v, re-reading the
    // slice's A; the one launch is taken while those extra bytes stay below
    // about a microsecond of HBM time, the cost of the launch it saves.
    int64_t extra_tiles = 0;
    for (int j = 0; j < p->desc.n_slices; ++j)
        extra_tiles += (p->desc.h_out[j] + kExpandTile - 1) / kExpandTile - 1;
    const int kmax = gemv_max_rank(p, r);   // the one launch serves decode segments only
    const int64_t extra_bytes = extra_tiles * kmax * (int64_t)p->desc.h_in * 2 *
                                r->info.n_decode_segments;
    const bool fused = r->info.n_decode_segments > 0 && kmax <= kFusedMaxRank &&
                       extra_bytes <= kFusedMaxExtraBytes;
    CallStreams cs;
    if (int32_t rc = fork_streams(r, st, cs)) return rc;
    int32_t rc = LORA_OK;
    if (fused) {
        hipError_t e = launch_delta_gemv(p->geom, pool_dev(p), routing_dev(r),
                                         r->info.n_decode_segments, x, ldx, y, ldy, cs.dec);
        if (e != hipSuccess) rc = hip_fail(e, "delta (decode) launch");
    }
    if (rc == LORA_OK) rc = enqueue_shrink(p, r, x, ldx, v, cs, !fused);
    if (rc == LORA_OK) rc = enqueue_expand(p, r, v, y, ldy, cs, !fused);
    const int32_t rj = join_streams(r, cs);
    return rc ? rc : rj;
}

}  // namespace lora

extern "C" {

int32_t lora_linear_workspace_bytes(const lora_pool *p, const lora_routing *r,
                                    int64_t *bytes_out)
{
    if (!p || !bytes_out) return fail(LORA_ERR_ARG, "pool or bytes_out is null");
    if (!r) {
        *bytes_out = 0;
        return LORA_OK;
    }
    if (int32_t rc = check_pair(p, r)) return rc;
    *bytes_out = round_up((int64_t)r->info.n_active * linear_v_len(p) * 2, 256);
    return LORA_OK;
}

int32_t lora_linear_delta(const lora_pool *p, const lora_routing *r, int32_t n_rows,
                          const void *W, int64_t ldw, const void *x, int64_t ldx, float *y,
                          int64_t ldy, void *workspace, int64_t workspace_bytes, void *stream)
{
    if (!p) return fail(LORA_ERR_ARG, "pool is null");
    if (n_rows < 0) return fail(LORA_ERR_SHAPE, "n_rows < 0");
    if (p->desc.x_dtype != LORA_DTYPE_BF16)
        return fail(LORA_ERR_DTYPE, "the base projection takes bf16 x (the lane's x is fp16)");
    if (r) {
        if (int32_t rc = check_pair(p, r)) return rc;
        if (r->device_built)
            return fail(LORA_ERR_ARG, "the base projection needs a routing built on the host");
        if (r->info.n_tokens != n_rows)
            return fail(LORA_ERR_SHAPE, "routing covers %d rows, n_rows is %d",
                        r->info.n_tokens, n_rows);
    }
    if (n_rows == 0) return LORA_OK;
    if (!W) return fail(LORA_ERR_ARG, "W is null");
    if (!aligned16(W)) return fail(LORA_ERR_SHAPE, "W must be 16-byte aligned");
    if (ldw < p->desc.h_in || ldw % 8)
        return fail(LORA_ERR_SHAPE, "ldw=%lld must be >= h_in=%d and a multiple of 8",
                    (long long)ldw, p->desc.h_in);
    if (int32_t rc = check_x(p, x, ldx)) return rc;
    if (int32_t rc = check_y(p, y, ldy)) return rc;
    const int n_act = r ? r->info.n_active : 0;
    float *v = static_cast<float *>(workspace);
    if (n_act > 0) {
        int64_t need = 0;
        lora_linear_workspace_bytes(p, r, &need);
        if (!workspace) return fail(LORA_ERR_ARG, "workspace is null");
        if (!aligned16(workspace))
            return fail(LORA_ERR_SHAPE, "workspace must be 16-byte aligned");
        if (workspace_bytes < need)
            return fail(LORA_ERR_CAPACITY, "workspace %lld bytes < %lld needed",
                        (long long)workspace_bytes, (long long)need);
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    LinearArgs a{};
    a.W = static_cast<const uint16_t *>(W);
    a.ldw = ldw;
    a.x = static_cast<const uint16_t *>(x);
    a.ldx = ldx;
    a.y = y;
    a.ldy = ldy;
    a.M = n_rows;
    a.N = p->geom.H_out;
    a.K = p->desc.h_in;
    a.rows = r ? r->dev + r->off_row : nullptr;
    if (n_act > 0 &&
        r->tile_steps[linear_tile_rows(n_rows, p->geom.H_out) == 64 ? 0 : 1] > kLinearMaxSteps) {
        // more delta steps in one row tile than the kernel holds: the base
        // product, then the delta added by lora_delta_apply (the workspace
        // holds v in fp32 as well)
        hipError_t e = launch_linear(p->geom, pool_dev(p), a, st);
        if (e != hipSuccess) return hip_fail(e, "base projection launch");
        return delta_apply_ws(p, r, x, ldx, y, ldy, workspace, workspace_bytes, st);
    }
    if (n_act > 0) {
        // v of the active rows, in the routing's order and the split bf16
        // form the projection's delta K-tiles read, by the shrink kernels
        CallStreams cs;
        if (int32_t rc = fork_streams(r, st, cs)) return rc;
        const int32_t rc = enqueue_shrink(p, r, x, ldx, v, cs, true, linear_v_len(p));
        const int32_t rj = join_streams(r, cs);
        if (rc) return rc;
        if (rj) return rj;
    }
    a.n_delta = n_act;
    a.row_meta = r ? r->dev + r->off_meta : nullptr;
    a.v = v;
    hipError_t e = launch_linear(p->geom, pool_dev(p), a, st);
    if (e != hipSuccess) return hip_fail(e, "base projection launch");
    return LORA_OK;
}

}  // extern "C"
