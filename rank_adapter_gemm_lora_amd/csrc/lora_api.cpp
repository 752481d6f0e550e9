// lora_api.cpp -- host runtime behind include/lora.h: argument checks, the
// adapter pool and slot table, the segments object, and the kernel launches.
// Every entry point returns a status; no exception leaves this file.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>

#include "internal.h"

using namespace lora;

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

lora_status from_hip(hipError_t e)
{
    if (e == hipSuccess)
        return LORA_OK;
    (void)hipGetLastError();   // clear the sticky error of this thread
    return e == hipErrorOutOfMemory ? LORA_E_NOMEM : LORA_E_HIP;
}

#define LORA_TRY(expr)                              \
    do {                                            \
        const lora_status st_ = from_hip(expr);     \
        if (st_ != LORA_OK)                         \
            return st_;                             \
    } while (0)

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// k-splits of the shrink.  Small batches split k (at least 512 per split) so
// that the k-reduction spreads over many workgroups; the expand re-reads every
// split's partials once per column chunk, so the split count also shrinks as
// the batch grows (at most 4096 / rows).  Depends only on the shape, never on
// the ids.
// Rows per dense tile.  Dense groups of batches up to 4096 rows are cut into
// 16-row tiles (more workgroups for few rows), of larger batches into 64-row
// tiles (each B chunk and A row then serves 64 rows).  Stacks of rank 32 and
// up take 64-row tiles from 1024 rows on when the batch still gives 512 or
// more expand workgroups: a 16-row tile would reread more of B and A than it
// moves of y and x.
int sgmv_rows_for(const lora_stack *st, int64_t n_rows)
{
    if (n_rows > 4096)
        return kSgmvTileRows;
    if (n_rows > kFusedMaxRows && st->r_max >= 32 && n_rows * st->D >= ((int64_t)1 << 23))
        return kSgmvTileRows;
    return kBgmvTileRows;
}

// k-splits of the shrink: about 256 tile workgroups in all (tile_rows-row
// tiles), at least 512 k per split, at most kMaxKSplit, a power of two.
// Batches of 64-row tiles whose v is small (vrow = slices x r_max <= 48
// floats a row, so each extra split adds little to what every expand chunk
// rereads) take at least two: one split per tile leaves ~one long stream per
// workgroup.  Measured with two against one (k = 4096): q/k/v prefill, 35 K
// rows, rank 16: step 305.5 -> 298.0 us (four splits: the expand +8.6 us);
// 12 K rows, rank 16: 99.2 -> 94.6 us; 20 K rows, three slices of rank 8:
// 193.5 -> 191.5 us; but 16 K rows at rank 64 (vrow 64): 172.6 -> 180.9 us.
int choose_ks(int64_t k, int64_t n_rows, int tile_rows, int64_t vrow)
{
    int64_t ks = std::max<int64_t>(1, k / 512);
    const int64_t least = (tile_rows == kSgmvTileRows && vrow <= 48) ? 2 : 1;
    ks = std::min<int64_t>(ks, std::max<int64_t>(least, 256 * tile_rows / std::max<int64_t>(1, n_rows)));
    ks = std::min<int64_t>(ks, kMaxKSplit);
    // powers of two keep blocks of one split on one XCD
    int64_t p = 1;
    while (p * 2 <= ks)
        p *= 2;
    return (int)p;
}


bool current_device_is(int dev)
{
    int cur = -1;
    return hipGetDevice(&cur) == hipSuccess && cur == dev;
}

void free_stack(lora_stack *st)
{
    if (!st)
        return;
    (void)hipFree(st->A_pool);
    (void)hipFree(st->A_img);
    (void)hipFree(st->B_pool);
    (void)hipFree(st->d_rank);
    (void)hipFree(st->d_scale);
    (void)hipFree(st->vpart);
    delete st;
}

void free_segments(lora_segments *seg)
{
    if (!seg)
        return;
    (void)hipFree(seg->perm);
    (void)hipFree(seg->seg_off);
    (void)hipFree(seg->active);
    (void)hipFree(seg->counts);
    (void)hipFree(seg->tiles);
    (void)hipFree(seg->keys);
    (void)hipFree(seg->chunk);
    (void)hipFree(seg->chunk_bad);
    (void)hipFree(seg->binfo);
    (void)hipFree(seg->sync);
    (void)hipFree(seg->vtag);
    delete seg;
}

// Most slices one 256-column expand chunk touches.
int expand_nq_max(const lora_stack *st)
{
    int nq_max = 1;
    for (int64_t c0 = 0; c0 < st->D; c0 += kExpandCols) {
        const int64_t c1 = std::min<int64_t>(c0 + kExpandCols, st->D) - 1;
        int q0 = 0, q1 = 0;
        while (q0 + 1 < st->n_slices && c0 >= st->slice_off[q0 + 1])
            ++q0;
        while (q1 + 1 < st->n_slices && c1 >= st->slice_off[q1 + 1])
            ++q1;
        nq_max = std::max(nq_max, q1 - q0 + 1);
    }
    return nq_max;
}

// Dynamic LDS of the expand: row indices, the slot table (few slots), v of a
// tile for the slices of one chunk, and B (for MFMA tiles a [256][b_win] block
// of the chunk, b_win ranks at a time: the whole rank when it fits, else the
// widest multiple of 16 that does; one 8 KB pass for vector tiles).  b_win 0:
// no window fits.
struct ExpandLds {
    int v_off, b_off, bytes, b_win;
};

ExpandLds expand_lds(const lora_stack *st, bool mfma, int tile_rows)
{
    const int64_t table = st->n_slots <= kExpandTableSlots ? 8 * kExpandTableSlots : 0;
    const int64_t rows = mfma ? tile_rows : kBgmvTileRows;
    // v rows of nq slices x rp ranks plus 4 floats (the kernel's padded pitch)
    const int64_t v_bytes = round_up(rows * (expand_nq_max(st) * st->rp_max + 4) * 4, 16);
    ExpandLds l;
    l.v_off = (int)(kExpandLdsTable + table);
    l.b_off = (int)(l.v_off + v_bytes);
    l.b_win = 0;
    int64_t b_bytes = 8 * kExpandCols * 4;
    if (mfma) {
        const int64_t room = kExpandLdsMax - l.b_off;
        for (int64_t w = round_up(st->rp_max, 16); w >= 16; w -= 16) {
            const int64_t need = (int64_t)kExpandCols * std::min<int64_t>(w, st->rp_max) * 2;
            if (std::max(need, b_bytes) <= room) {
                l.b_win = (int)w;
                b_bytes = std::max(need, b_bytes);
                break;
            }
        }
    }
    l.bytes = (int)(l.b_off + b_bytes);
    return l;
}

// MFMA tiles need bf16, slices made of whole 64-column blocks, and the v of a
// 64-row tile plus at least a 16-rank window of B within the expand's LDS
// budget; otherwise the dense tiles of a batch are served by the vector code.
// The several-chunk expand's LDS: as expand_lds, with v of a 16-row tile for
// every slice and one B block of the widest rank.
ExpandLds expand_stream_lds(const lora_stack *st)
{
    const int64_t table = st->n_slots <= kExpandTableSlots ? 8 * kExpandTableSlots : 0;
    const int64_t v_bytes =
        round_up((int64_t)kBgmvTileRows * (st->n_slices * st->rp_max + 4) * 4, 16);
    ExpandLds l;
    l.v_off = (int)(kExpandLdsTable + table);
    l.b_off = (int)(l.v_off + v_bytes);
    l.b_win = (int)round_up(st->rp_max, 16);
    const int64_t b_bytes = std::max<int64_t>((int64_t)kExpandCols * st->rp_max * 2, 8 * kExpandCols * 4);
    l.bytes = (int)(l.b_off + b_bytes);
    return l;
}

// Chunks per expand workgroup, from the shapes alone.  Several pay off where
// the groups average less than one 16-row tile (so most tiles carry a few rows
// and each workgroup's fixed cost -- its record, v, the first round trip --
// is spread over more columns) at low rank.  Measured on 1024 rows x 100
// rank-16 adapters: into 28672 columns (112 chunks) expand 60.6 / 50.4 / 50.8
// us with 1 / 2 / 4 chunks; into 7168 columns (28 chunks) 17.7 / 16.2 / 15.0
// us.  Elsewhere one: the one-chunk kernel keeps more workgroups per CU
// (decode, 32 rows per slot: 5.7 / 6.7 / 9.4 us; rank-64 MLP gate/up: 28.1 /
// 30.4 / 34.8 us).
int choose_cpw(const lora_stack *st, int64_t n_rows, int forced)
{
    if (forced > 0)
        return forced;
    const int64_t chunks = (st->D + kExpandCols - 1) / kExpandCols;
    const int64_t pairs = chunks * max_tiles_for(n_rows, st->n_slots);
    if (st->rp_max > 16 || n_rows > (int64_t)kBgmvTileRows * st->n_slots || pairs < 2048)
        return 1;
    return chunks <= 32 ? 4 : 2;
}

bool stack_has_mfma_path(const lora_stack *st)
{
    if (st->dtype != LORA_BF16)
        return false;
    for (int q = 0; q < st->n_slices; ++q)
        if (st->slice_d[q] % 64 != 0)
            return false;
    return expand_lds(st, true, kSgmvTileRows).b_win > 0;
}

lora_status check_apply_common(const lora_stack *st, const lora_segments *seg)
{
    if (!st || !seg || !seg->built)
        return LORA_E_ARG;
    if (seg->n_slots != st->n_slots || seg->n_rows > st->max_rows)
        return LORA_E_ARG;
    if (!current_device_is(st->device) || seg->device != st->device)
        return LORA_E_ARG;
    return LORA_OK;
}

ApplyArgs make_args(const lora_stack *st, const lora_segments *seg)
{
    ApplyArgs a;
    std::memset(&a, 0, sizeof a);
    a.A = st->A_pool;
    a.A_img = st->A_img;
    a.B = st->B_pool;
    a.rank = st->d_rank;
    a.scale = st->d_scale;
    a.n_slots = st->n_slots;
    a.k = st->k;
    a.n_slices = st->n_slices;
    a.r_max = st->r_max;
    a.D = st->D;
    for (int q = 0; q <= st->n_slices; ++q)
        a.slice_off[q] = st->slice_off[q];
    a.a_slot_stride = (int64_t)st->n_slices * st->r_max * st->k;
    a.b_slot_stride = st->D * st->rp_max;
    a.vpart = st->vpart;
    a.max_rows = st->max_rows;
    // the tile height the batch was grouped with (the stack that built the
    // segments may differ from this one: one grouping per batch serves every
    // projection)
    a.sgmv_rows = seg->built ? seg->built_sgmv_rows : sgmv_rows_for(st, seg->n_rows);
    a.ks = choose_ks(st->k, seg->n_rows, a.sgmv_rows, (int64_t)st->n_slices * st->r_max);
    a.mfma_ok = stack_has_mfma_path(st) ? 1 : 0;
    // v staging sized for this batch's dense tile height (16 rows up to 4096
    // rows): a smaller footprint lets more expand workgroups share a CU
    const ExpandLds l = expand_lds(st, a.mfma_ok != 0, a.sgmv_rows);
    a.b_win = l.b_win > 0 ? l.b_win : 16;   // (unused by the vector code)
    a.lds_v_off = l.v_off;
    a.lds_b_off = l.b_off;
    a.lds_bytes = l.bytes;
    a.cpw = 1;
    if (a.mfma_ok && a.sgmv_rows == kBgmvTileRows && st->rp_max <= 64) {
        const int cpw = choose_cpw(st, seg->n_rows, seg->expand_chunks);
        const ExpandLds ls = expand_stream_lds(st);
        if (cpw > 1 && ls.bytes <= kExpandLdsMax) {
            a.cpw = cpw;
            a.lds_v_off = ls.v_off;
            a.lds_b_off = ls.b_off;
            a.lds_bytes = ls.bytes;
        }
    }
    a.counts = seg->counts;
    a.tiles = seg->tiles;
    a.sync = seg->sync;
    a.wait_limit = seg->wait_limit;
    if (st->n_cu == 0 &&
        hipDeviceGetAttribute(&st->n_cu, hipDeviceAttributeMultiprocessorCount, st->device) != hipSuccess)
        st->n_cu = 0;
    a.n_cu = st->n_cu;
    a.all_dense = a.mfma_ok && seg->built_dense_min <= 1 ? 1 : 0;
    return a;
}

}  // namespace

// Load one adapter into an empty slot, in stream order.  kind: where A and B
// are (host memory is pinned when the copy is to be asynchronous); sync: wait
// for the copies before returning (the caller's buffers are then free).
lora_status lora::load_slot(lora_stack *st, int slot, int rank, float alpha, const void *A,
                            const void *B, hipMemcpyKind kind, bool sync, hipStream_t s)
{
    if (!st)
        return LORA_E_ARG;
    if (slot < 0 || slot >= st->n_slots)
        return LORA_E_SLOT;
    if (rank < 1 || rank > st->r_max)
        return LORA_E_RANK;
    if (st->h_rank[slot] != 0)
        return LORA_E_OCCUPIED;
    if (!A || !B || !std::isfinite(alpha) || !current_device_is(st->device))
        return LORA_E_ARG;

    const size_t es = st->esize;
    char *a_dst = static_cast<char *>(st->A_pool) +
                  (size_t)slot * st->n_slices * st->r_max * st->k * es;
    char *b_dst = static_cast<char *>(st->B_pool) + (size_t)slot * st->D * st->rp_max * es;
    const int rp = (int)round_up(rank, 8);

    // the kernels read A rows up to r_max and B ranks up to rp: those past the
    // rank must be zero (nothing to clear when the copies cover them)
    if (rank < st->r_max)
        LORA_TRY(launch_zero(a_dst, (size_t)st->n_slices * st->r_max * st->k * es, s));
    if (rp != rank)
        LORA_TRY(launch_zero(b_dst, (size_t)st->D * rp * es, s));
    // A: [n_slices][rank][k] -> [n_slices][r_max][k]
    LORA_TRY(hipMemcpy2DAsync(a_dst, (size_t)st->r_max * st->k * es, A, (size_t)rank * st->k * es,
                              (size_t)rank * st->k * es, st->n_slices, kind, s));
    // B: [D][rank] -> [D][rp], rp = rank rounded up to 8 (rank-contiguous rows)
    if (rp == rank)
        LORA_TRY(hipMemcpyAsync(b_dst, B, (size_t)st->D * rank * es, kind, s));
    else
        LORA_TRY(hipMemcpy2DAsync(b_dst, (size_t)rp * es, B, (size_t)rank * es, (size_t)rank * es,
                                  st->D, kind, s));
    if (st->A_img) {
        // the slot's operand image, from the region just written
        ImageArgs im;
        std::memset(&im, 0, sizeof im);
        im.A_pool = st->A_pool;
        im.A_img = st->A_img;
        im.k = st->k;
        im.n_slices = st->n_slices;
        im.r_max = st->r_max;
        im.n_jobs = 1;
        im.slot[0] = slot;
        LORA_TRY(launch_build_image(im, s));
    }
    LORA_TRY(launch_set_slot(st->d_rank, st->d_scale, slot, rank, alpha / (float)rank, s));
    if (sync)
        LORA_TRY(hipStreamSynchronize(s));
    st->h_rank[slot] = rank;
    st->h_alpha[slot] = alpha;
    return LORA_OK;
}

void lora::note_loaded(lora_stack *st, int slot, int rank, float alpha)
{
    st->h_rank[slot] = rank;
    st->h_alpha[slot] = alpha;
}

bool lora::x_ok(const lora_stack *st, const void *x, int64_t ldx)
{
    return x && aligned16(x) && ldx >= st->k && ldx % 8 == 0;
}

bool lora::y_ok(const lora_stack *st, const void *y, int64_t ldy)
{
    return y && aligned16(y) && ldy >= st->D && ldy % 8 == 0;
}

int lora::max_tiles_for(int64_t n_rows, int n_slots)
{
    return (int)((n_rows + kBgmvTileRows - 1) / kBgmvTileRows + std::min<int64_t>(n_slots, n_rows));
}

// Tile bound of the shrink and expand grids of a built batch: with 64-row
// dense tiles and every group dense (dense_min 1), a group of c rows gives
// ceil(c / 64) tiles, so the batch at most ceil(n / 64) + (groups) tiles;
// otherwise groups may be cut into 16-row tiles.  Shapes and the segments
// object's policy only, never the mix.
int lora::grid_tiles(int64_t n_rows, int n_slots, int sgmv_rows, int dense_min)
{
    if (sgmv_rows == kSgmvTileRows && dense_min <= 1)
        return (int)((n_rows + kSgmvTileRows - 1) / kSgmvTileRows + std::min<int64_t>(n_slots, n_rows));
    return max_tiles_for(n_rows, n_slots);
}

lora_status lora::status_of(hipError_t e) { return from_hip(e); }

bool lora::device_is_current(int dev) { return current_device_is(dev); }

// k-splits of the one-launch decode: the most (a power of two, at most
// kDecodeMaxKs and at least 512 k per split) that leave every wavefront's
// k-quarter whole 32-k matrix-core steps; 0 when none does.
int lora::decode_ks(int64_t k)
{
    if (k % 128 != 0)
        return 0;
    int ks = 1;
    while (ks * 2 <= kDecodeMaxKs && k / (ks * 2) >= 512 && (k / 8) % (16 * ks * 2) == 0)
        ks *= 2;
    return ks;
}

// The one-launch decode serves bf16 stacks of one slice with rank <= 16 and
// whole 64-column output blocks, batches of 1 .. 256 rows over at most 63
// slots, while the grid fits the chip at once with a quarter to spare
// (workgroups of tiles the mix leaves empty exit after the grouping), and
// the hand-over state holds vt_tiles tiles.
bool lora::decode_fits(const lora_stack *st, int64_t n_rows, int cpw, int vt_tiles)
{
    if (st->dtype != LORA_BF16 || !st->A_img || st->n_slices != 1 || st->r_max > 16 || st->D % 64 != 0 ||
        n_rows < 1 || n_rows > kDecodeMaxRows || st->n_slots > kDecodeMaxSlots || decode_ks(st->k) == 0)
        return false;
    const int64_t tiles = max_tiles_for(n_rows, st->n_slots);
    if (tiles > vt_tiles)
        return false;
    if (st->n_cu == 0 &&
        hipDeviceGetAttribute(&st->n_cu, hipDeviceAttributeMultiprocessorCount, st->device) != hipSuccess)
        st->n_cu = 0;
    const int wpc = decode_wgs_per_cu(decode_ks(st->k), cpw);
    const int64_t capacity = (int64_t)wpc * st->n_cu;
    const int64_t ncg = (st->D + 256 * cpw - 1) / (256 * cpw);
    return capacity > 0 && (decode_ks(st->k) + ncg) * tiles <= capacity + capacity / 4;
}

// Launch arguments of the one-launch decode, without its hand-over state and
// segments outputs (the caller sets those).
DecodeArgs lora::decode_args_for(const lora_stack *st, const int32_t *ids, int64_t n_rows, const void *x,
                                 int64_t ldx, void *y, int64_t ldy, int cpw)
{
    DecodeArgs a;
    std::memset(&a, 0, sizeof a);
    a.ids = ids;
    a.n = (int)n_rows;
    a.n_slots = st->n_slots;
    a.slot_rank = st->d_rank;
    a.slot_scale = st->d_scale;
    a.A_img = st->A_img;
    a.B = st->B_pool;
    a.b_slot_stride = st->D * st->rp_max;
    a.r_max = st->r_max;
    a.k = st->k;
    a.D = st->D;
    a.x = x;
    a.ldx = ldx;
    a.y = y;
    a.ldy = ldy;
    a.ks = decode_ks(st->k);
    a.cpw = cpw;
    a.ncg = (int)((st->D + 256 * cpw - 1) / (256 * cpw));
    a.tiles_bound = max_tiles_for(n_rows, st->n_slots);
    a.wait_limit = kWaitSpinsDefault;
    return a;
}

extern "C" {

const char *lora_status_string(lora_status s)
{
    switch (s) {
    case LORA_OK: return "ok";
    case LORA_E_ARG: return "invalid argument";
    case LORA_E_RANK: return "rank outside [1, r_max]";
    case LORA_E_SLOT: return "slot outside [0, n_slots)";
    case LORA_E_OCCUPIED: return "slot already holds an adapter";
    case LORA_E_EMPTY: return "slot holds no adapter";
    case LORA_E_NOMEM: return "device allocation failed";
    case LORA_E_HIP: return "HIP runtime error";
    case LORA_E_BAD_IDS: return "batch contained ids naming no loaded slot";
    case LORA_E_UNSUPPORTED: return "shape outside the limits of this build";
    case LORA_E_CAPACITY: return "more adapters than the slots or the host tier hold";
    case LORA_E_NOT_FOUND: return "adapter id not registered";
    }
    return "unknown status";
}

lora_status lora_stack_create(lora_stack **out, lora_dtype dtype, int n_slots, int r_max, int64_t k,
                              int n_slices, const int64_t *slice_d, int64_t max_rows)
{
    if (!out)
        return LORA_E_ARG;
    *out = nullptr;
    if ((dtype != LORA_F32 && dtype != LORA_BF16) || !slice_d || n_slots < 1 || r_max < 1 ||
        k < 8 || k % 8 != 0 || n_slices < 1 || max_rows < 1)
        return LORA_E_ARG;
    if (n_slots > LORA_MAX_SLOTS || r_max > LORA_MAX_RANK || n_slices > LORA_MAX_SLICES ||
        n_slices * r_max > kMaxSliceRank || max_rows > (int64_t)INT32_MAX / 2)
        return LORA_E_UNSUPPORTED;
    int64_t D = 0;
    for (int q = 0; q < n_slices; ++q) {
        if (slice_d[q] < 8 || slice_d[q] % 8 != 0)
            return LORA_E_ARG;
        D += slice_d[q];
    }

    lora_stack *st = new (std::nothrow) lora_stack();
    if (!st)
        return LORA_E_NOMEM;
    st->A_pool = st->A_img = st->B_pool = nullptr;
    st->d_rank = nullptr;
    st->d_scale = nullptr;
    st->vpart = nullptr;
    st->n_cu = 0;
    st->one_launch_wpc = -1;
    st->apply_wpc = -1;
    if (hipGetDevice(&st->device) != hipSuccess) {
        delete st;
        return LORA_E_HIP;
    }
    st->dtype = dtype;
    st->esize = dtype == LORA_F32 ? 4 : 2;
    st->n_slots = n_slots;
    st->r_max = r_max;
    st->rp_max = (int)round_up(r_max, 8);
    st->k = k;
    st->n_slices = n_slices;
    st->slice_off[0] = 0;
    for (int q = 0; q < n_slices; ++q) {
        st->slice_d[q] = slice_d[q];
        st->slice_off[q + 1] = st->slice_off[q] + slice_d[q];
    }
    st->D = D;
    st->max_rows = max_rows;
    st->h_rank.assign(n_slots, 0);
    st->h_alpha.assign(n_slots, 0.f);

    const size_t a_bytes = (size_t)n_slots * n_slices * r_max * k * st->esize;
    // the operand image pads each slice's ranks to whole 16-row chunks
    const size_t img_bytes = stack_has_mfma_path(st)
                                 ? (size_t)n_slots * n_slices * round_up(r_max, kImgRows) * k * st->esize
                                 : 0;
    const size_t b_bytes = (size_t)n_slots * D * st->rp_max * st->esize;
    const size_t v_bytes = (size_t)max_rows * n_slices * r_max * sizeof(float);
    hipError_t e = hipSuccess;
    if (e == hipSuccess) e = hipMalloc(&st->A_pool, a_bytes);
    if (e == hipSuccess && img_bytes) e = hipMalloc(&st->A_img, img_bytes);
    if (e == hipSuccess) e = hipMalloc(&st->B_pool, b_bytes);
    if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void **>(&st->d_rank), sizeof(int32_t) * n_slots);
    if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void **>(&st->d_scale), sizeof(float) * n_slots);
    if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void **>(&st->vpart), kMaxKSplit * v_bytes);
    if (e == hipSuccess) e = hipMemset(st->A_pool, 0, a_bytes);
    if (e == hipSuccess && img_bytes) e = hipMemset(st->A_img, 0, img_bytes);
    if (e == hipSuccess) e = hipMemset(st->B_pool, 0, b_bytes);
    if (e == hipSuccess) e = hipMemset(st->d_rank, 0, sizeof(int32_t) * n_slots);
    if (e == hipSuccess) e = hipMemset(st->d_scale, 0, sizeof(float) * n_slots);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        free_stack(st);
        return from_hip(e);
    }
    *out = st;
    return LORA_OK;
}

lora_status lora_stack_destroy(lora_stack *st)
{
    if (!st)
        return LORA_OK;
    const hipError_t e = hipDeviceSynchronize();
    free_stack(st);
    return from_hip(e);
}

lora_status lora_load_slot(lora_stack *st, int slot, int rank, float alpha, const void *A,
                           const void *B, int src_is_host, void *stream)
{
    return lora::load_slot(st, slot, rank, alpha, A, B,
                           src_is_host ? hipMemcpyHostToDevice : hipMemcpyDeviceToDevice,
                           src_is_host != 0, reinterpret_cast<hipStream_t>(stream));
}

lora_status lora_evict_slot(lora_stack *st, int slot, void *stream)
{
    if (!st)
        return LORA_E_ARG;
    if (slot < 0 || slot >= st->n_slots)
        return LORA_E_SLOT;
    if (st->h_rank[slot] == 0)
        return LORA_E_EMPTY;
    if (!current_device_is(st->device))
        return LORA_E_ARG;
    LORA_TRY(launch_set_slot(st->d_rank, st->d_scale, slot, 0, 0.f,
                             reinterpret_cast<hipStream_t>(stream)));
    st->h_rank[slot] = 0;
    st->h_alpha[slot] = 0.f;
    return LORA_OK;
}

lora_status lora_slot_info(const lora_stack *st, int slot, int *rank, float *alpha,
                           int64_t *live_params)
{
    if (!st)
        return LORA_E_ARG;
    if (slot < 0 || slot >= st->n_slots)
        return LORA_E_SLOT;
    const int r = st->h_rank[slot];
    if (rank)
        *rank = r;
    if (alpha)
        *alpha = st->h_alpha[slot];
    if (live_params)
        *live_params = (int64_t)r * (st->n_slices * st->k + st->D);
    return LORA_OK;
}

lora_status lora_merge_slot(const lora_stack *st, int slot, void *W, int64_t ldw, int sign,
                            void *stream)
{
    if (!st)
        return LORA_E_ARG;
    if (slot < 0 || slot >= st->n_slots)
        return LORA_E_SLOT;
    const int rank = st->h_rank[slot];
    if (rank == 0)
        return LORA_E_EMPTY;
    if (!W || (reinterpret_cast<uintptr_t>(W) & 15) != 0 || ldw < st->k || ldw % 8 != 0 ||
        (sign != 1 && sign != -1) || !current_device_is(st->device))
        return LORA_E_ARG;
    MergeArgs a{};
    const size_t es = st->esize;
    a.A = static_cast<const char *>(st->A_pool) + (size_t)slot * st->n_slices * st->r_max * st->k * es;
    a.B = static_cast<const char *>(st->B_pool) + (size_t)slot * st->D * st->rp_max * es;
    a.W = W;
    a.ldw = ldw;
    a.k = st->k;
    a.rank = rank;
    a.rp = (int)round_up(rank, 8);
    a.r_max = st->r_max;
    // the same fp32 scale the apply path reads from the slot table
    const float scale = st->h_alpha[slot] / (float)rank;
    a.s = sign > 0 ? scale : -scale;
    a.n_slices = st->n_slices;
    int64_t tiles = 0;
    for (int q = 0; q <= st->n_slices; ++q) {
        a.slice_off[q] = st->slice_off[q];
        a.tile0[q] = (int)tiles;
        if (q < st->n_slices)
            tiles += merge_row_tiles(st->slice_d[q]);
    }
    if (tiles > 65535)
        return LORA_E_UNSUPPORTED;
    if (st->n_cu == 0 &&
        hipDeviceGetAttribute(&st->n_cu, hipDeviceAttributeMultiprocessorCount, st->device) != hipSuccess)
        st->n_cu = 0;
    if (st->n_cu < 1)
        return LORA_E_HIP;
    a.n_cu = st->n_cu;
    LORA_TRY(launch_merge(st->dtype == LORA_F32 ? DT_F32 : DT_BF16, a,
                          reinterpret_cast<hipStream_t>(stream)));
    return LORA_OK;
}

lora_status lora_segments_create(lora_segments **out, int64_t max_rows, int n_slots)
{
    if (!out)
        return LORA_E_ARG;
    *out = nullptr;
    if (max_rows < 1 || n_slots < 1)
        return LORA_E_ARG;
    if (n_slots > LORA_MAX_SLOTS || max_rows > (int64_t)INT32_MAX / 2)
        return LORA_E_UNSUPPORTED;
    lora_segments *seg = new (std::nothrow) lora_segments();
    if (!seg)
        return LORA_E_NOMEM;
    seg->perm = seg->seg_off = seg->active = seg->counts = nullptr;
    seg->tiles = nullptr;
    seg->keys = seg->chunk = seg->chunk_bad = nullptr;
    seg->binfo = nullptr;
    if (hipGetDevice(&seg->device) != hipSuccess) {
        delete seg;
        return LORA_E_HIP;
    }
    seg->max_rows = max_rows;
    seg->n_slots_cap = n_slots;
    seg->max_tiles = max_tiles_for(max_rows, n_slots);
    // every group on dense (matrix-core) tiles by default: measured faster
    // than the vector tiles even for one-row groups (many-adapter decode
    // 103 -> 83 us); the vector path still serves stacks without matrix-core
    // tiles and any group below a larger threshold set by the caller
    seg->dense_min = 1;
    seg->expand_chunks = 0;
    seg->sync = nullptr;
    seg->vtag = nullptr;
    seg->vtag_tiles = n_slots <= kDecodeMaxSlots
                          ? max_tiles_for(std::min<int64_t>(max_rows, kDecodeMaxRows), n_slots)
                          : 0;
    seg->wait_limit = kWaitSpinsDefault;
    seg->built = 0;
    seg->built_dense_min = 1;
    seg->built_sgmv_rows = kBgmvTileRows;
    seg->n_rows = 0;
    seg->n_slots = 0;
    hipError_t e = hipSuccess;
    if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void **>(&seg->perm), sizeof(int32_t) * max_rows);
    if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void **>(&seg->seg_off), sizeof(int32_t) * (n_slots + 1));
    if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void **>(&seg->active), sizeof(int32_t) * n_slots);
    if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void **>(&seg->counts), sizeof(int32_t) * kCntSlots);
    if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void **>(&seg->tiles), sizeof(ShrinkTile) * seg->max_tiles);
    const int64_t n_chunks = (max_rows + kChunkRows - 1) / kChunkRows;
    if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void **>(&seg->keys), sizeof(int32_t) * max_rows);
    if (e == hipSuccess)
        e = hipMalloc(reinterpret_cast<void **>(&seg->chunk), sizeof(int32_t) * n_chunks * (n_slots + 1));
    if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void **>(&seg->chunk_bad), sizeof(int32_t) * n_chunks);
    if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void **>(&seg->binfo), sizeof(int4) * (n_slots + 1));
    const size_t sync_ints = kSyncFlags + (size_t)seg->max_tiles * kSyncTileInts;
    if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void **>(&seg->sync), sizeof(int32_t) * sync_ints);
    if (e == hipSuccess) e = hipMemset(seg->sync, 0, sizeof(int32_t) * sync_ints);
    const size_t vtag_words = (size_t)kDecodeWordsPerTile * seg->vtag_tiles;
    if (e == hipSuccess && vtag_words > 0)
        e = hipMalloc(reinterpret_cast<void **>(&seg->vtag), sizeof(uint32_t) * vtag_words);
    if (e == hipSuccess && vtag_words > 0)
        e = hipMemset(seg->vtag, 0, sizeof(uint32_t) * vtag_words);
    if (e == hipSuccess) e = hipMemset(seg->counts, 0, sizeof(int32_t) * kCntSlots);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        free_segments(seg);
        return from_hip(e);
    }
    *out = seg;
    return LORA_OK;
}

lora_status lora_segments_destroy(lora_segments *seg)
{
    if (!seg)
        return LORA_OK;
    const hipError_t e = hipDeviceSynchronize();
    free_segments(seg);
    return from_hip(e);
}

lora_status lora_segments_set_dense_min(lora_segments *seg, int m_min)
{
    if (!seg || m_min < 1)
        return LORA_E_ARG;
    seg->dense_min = m_min;
    return LORA_OK;
}

lora_status lora_segments_set_expand_chunks(lora_segments *seg, int chunks)
{
    if (!seg || chunks < 0 || chunks > kMaxExpandChunks)
        return LORA_E_ARG;
    seg->expand_chunks = chunks;
    return LORA_OK;
}

lora_status lora_segments_set_wait_limit(lora_segments *seg, int polls)
{
    if (!seg || polls < 0)
        return LORA_E_ARG;
    seg->wait_limit = polls;
    return LORA_OK;
}

namespace {

lora_status check_build(const lora_stack *st, const int32_t *ids, int64_t n_rows,
                        const lora_segments *seg)
{
    if (!st || !seg || n_rows < 0 || n_rows > seg->max_rows || st->n_slots > seg->n_slots_cap)
        return LORA_E_ARG;
    if ((n_rows > 0 && !ids) || (reinterpret_cast<uintptr_t>(ids) & 3u) != 0)
        return LORA_E_ARG;
    if (!current_device_is(st->device) || seg->device != st->device)
        return LORA_E_ARG;
    return LORA_OK;
}

SegBuildArgs make_seg_args(const lora_stack *st, const int32_t *ids, int64_t n_rows,
                           lora_segments *seg)
{
    SegBuildArgs a;
    a.ids = ids;
    a.n = n_rows;
    a.n_slots = st->n_slots;
    a.slot_rank = st->d_rank;
    a.dense_min = seg->dense_min;
    a.sgmv_rows = sgmv_rows_for(st, n_rows);
    a.perm = seg->perm;
    a.seg_off = seg->seg_off;
    a.active = seg->active;
    a.counts = seg->counts;
    a.tiles = seg->tiles;
    a.keys = seg->keys;
    a.chunk = seg->chunk;
    a.chunk_bad = seg->chunk_bad;
    a.binfo = seg->binfo;
    return a;
}

void mark_built(lora_segments *seg, const lora_stack *st, int64_t n_rows)
{
    seg->built = 1;
    seg->built_dense_min = seg->dense_min;
    seg->built_sgmv_rows = sgmv_rows_for(st, n_rows);
    seg->n_rows = n_rows;
    seg->n_slots = st->n_slots;
}

// Grouping inside the shrink pays while the shrink grid fits on the chip in one
// go: every workgroup repeats the grouping, so a grid of several waves of
// workgroups would pay it several times over, more than the separate launch.
// Measured: 384 workgroups (512 rows, 16 slots, 8 k-splits) still gain ~2 us
// over the separate grouping launch; 656 (1024 rows, 100 slots, 4 k-splits)
// lose ~2.7 us.
constexpr int kFusedMaxBlocks = 512;   // two workgroups per compute unit

bool fused_build_pays(const lora_stack *st, int64_t n_rows)
{
    if (n_rows <= 0 || n_rows > kFusedMaxRows)
        return false;
    return (int64_t)choose_ks(st->k, n_rows, sgmv_rows_for(st, n_rows), (int64_t)st->n_slices * st->r_max) *
               max_tiles_for(n_rows, st->n_slots) <=
           kFusedMaxBlocks;
}

// Grouping, shrink and expand in one launch: batches the fused grouping
// serves, on 16-row tiles with one column chunk per expand workgroup, while the
// whole grid (shrink plus expand workgroups, each grouping the batch in LDS)
// fits on the chip at once, with a quarter to spare for the workgroups of tiles
// the mix leaves empty (they exit after the grouping).  Measured on q-proj
// 4096 -> 4096 at 256 rows: 1 to 4 adapters (grids of 408 and 480 at 512
// resident) 12.7 -> 12.0 us; 16 adapters (768) 13.4 -> 15.2 us, as expand
// workgroups queued behind waiting ones; rank 128 (one workgroup per CU by
// LDS) 27.4 -> 28.9 us.
bool one_launch_pays(const lora_stack *st, const ApplyArgs &a, int64_t n_rows)
{
    if (!fused_build_pays(st, n_rows) || a.sgmv_rows != kBgmvTileRows || a.cpw != 1)
        return false;
    if (st->one_launch_wpc < 0) {
        int n_cu = 0;
        if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, st->device) != hipSuccess)
            n_cu = 0;
        st->n_cu = n_cu;
        st->one_launch_wpc = build_apply_wgs_per_cu(st->dtype == LORA_BF16 ? DT_BF16 : DT_F32, a.lds_bytes);
    }
    const int64_t capacity = (int64_t)st->one_launch_wpc * st->n_cu;
    const int64_t tiles = max_tiles_for(n_rows, st->n_slots);
    const int64_t chunks = (st->D + kExpandCols - 1) / kExpandCols;
    return capacity > 0 && (a.ks + chunks) * tiles <= capacity + capacity / 4;
}

// The launch arguments of a batch of n_rows on this stack and segments object,
// the object itself untouched (its fields are plain values and pointers).
ApplyArgs args_for_rows(const lora_stack *st, const lora_segments *seg, int64_t n_rows)
{
    lora_segments tmp = *seg;
    mark_built(&tmp, st, n_rows);
    return make_args(st, &tmp);
}

// lora_apply in one launch: batches of 16-row tiles with one column chunk per
// expand workgroup whose grid fits the chip at once, a quarter to spare (the
// same rule as the one-launch lora_build_apply, for apply_kernel's residency).
bool apply_one_launch_pays(const lora_stack *st, const ApplyArgs &a, int64_t n_rows)
{
    if (n_rows <= 0 || a.sgmv_rows != kBgmvTileRows || a.cpw != 1)
        return false;
    if (st->apply_wpc < 0) {
        if (st->n_cu == 0 &&
            hipDeviceGetAttribute(&st->n_cu, hipDeviceAttributeMultiprocessorCount, st->device) != hipSuccess)
            st->n_cu = 0;
        st->apply_wpc = apply_wgs_per_cu(st->dtype == LORA_BF16 ? DT_BF16 : DT_F32, a.lds_bytes);
    }
    const int64_t capacity = (int64_t)st->apply_wpc * st->n_cu;
    const int64_t tiles = max_tiles_for(n_rows, st->n_slots);
    const int64_t chunks = (st->D + kExpandCols - 1) / kExpandCols;
    return capacity > 0 && (a.ks + chunks) * tiles <= capacity + capacity / 4;
}

// 256-column chunks per expand workgroup of the one-launch decode: 1 (the
// caller's 2 or 4 on request).  Measured on the decode workload: 8.3 / 8.4 /
// 8.7 us per step for 1 / 2 / 4 -- the merge into y runs on more SIMDs.
int decode_cpw(const lora_stack *, const lora_segments *seg)
{
    const int f = seg->expand_chunks;
    return f == 2 || f == 4 ? f : 1;
}

bool decode_pays(const lora_stack *st, const lora_segments *seg, int64_t n_rows)
{
    return seg->vtag && seg->dense_min == 1 &&
           decode_fits(st, n_rows, decode_cpw(st, seg), seg->vtag_tiles);
}

DecodeArgs decode_args(const lora_stack *st, lora_segments *seg, const int32_t *ids, int64_t n_rows,
                       const void *x, int64_t ldx, void *y, int64_t ldy)
{
    DecodeArgs a = decode_args_for(st, ids, n_rows, x, ldx, y, ldy, decode_cpw(st, seg));
    a.vtag = seg->vtag;
    a.vtag_tiles = seg->vtag_tiles;
    a.tile_state = seg->sync + kSyncFlags;
    a.timeouts = seg->sync + kSyncTimeouts;
    a.poison = seg->sync + kSyncTimeouts;
    a.wait_limit = seg->wait_limit;
    a.perm = seg->perm;
    a.seg_off = seg->seg_off;
    a.active = seg->active;
    a.counts = seg->counts;
    a.tiles = seg->tiles;
    return a;
}

// Kernel launches lora_build_apply makes for n_rows.
int build_apply_launches(const lora_stack *st, int64_t n_rows, const lora_segments *seg)
{
    if (n_rows <= 0)
        return 1;   // the empty grouping
    if (decode_pays(st, seg, n_rows))
        return 1;
    if (fused_build_pays(st, n_rows))
        return one_launch_pays(st, args_for_rows(st, seg, n_rows), n_rows) ? 1 : 2;
    return n_rows <= kFusedMaxRows ? 3 : 5;   // one-workgroup or chunked grouping
}

}  // namespace


lora_status lora_build_segments(const lora_stack *st, const int32_t *ids, int64_t n_rows,
                                lora_segments *seg, void *stream)
{
    const lora_status c = check_build(st, ids, n_rows, seg);
    if (c != LORA_OK)
        return c;
    LORA_TRY(launch_seg_build(make_seg_args(st, ids, n_rows, seg),
                              reinterpret_cast<hipStream_t>(stream)));
    mark_built(seg, st, n_rows);
    return LORA_OK;
}

lora_status lora_add_shrink(const lora_stack *st, const void *x, int64_t ldx,
                            const lora_segments *seg, void *stream)
{
    const lora_status c = check_apply_common(st, seg);
    if (c != LORA_OK)
        return c;
    if (seg->n_rows == 0)
        return LORA_OK;
    if (!x_ok(st, x, ldx))
        return LORA_E_ARG;
    ApplyArgs a = make_args(st, seg);
    a.x = x;
    a.ldx = ldx;
    LORA_TRY(launch_shrink(st->dtype == LORA_BF16 ? DT_BF16 : DT_F32, a,
                           grid_tiles(seg->n_rows, st->n_slots, a.sgmv_rows, seg->built_dense_min),
                           reinterpret_cast<hipStream_t>(stream)));
    return LORA_OK;
}

lora_status lora_add_expand(const lora_stack *st, void *y, int64_t ldy, const lora_segments *seg,
                            void *stream)
{
    const lora_status c = check_apply_common(st, seg);
    if (c != LORA_OK)
        return c;
    if (seg->n_rows == 0)
        return LORA_OK;
    if (!y_ok(st, y, ldy))
        return LORA_E_ARG;
    ApplyArgs a = make_args(st, seg);
    a.y = y;
    a.ldy = ldy;
    LORA_TRY(launch_expand(st->dtype == LORA_BF16 ? DT_BF16 : DT_F32, a,
                           grid_tiles(seg->n_rows, st->n_slots, a.sgmv_rows, seg->built_dense_min),
                           reinterpret_cast<hipStream_t>(stream)));
    return LORA_OK;
}

lora_status lora_apply(const lora_stack *st, void *y, int64_t ldy, const void *x, int64_t ldx,
                       const lora_segments *seg, void *stream)
{
    const lora_status c = check_apply_common(st, seg);
    if (c != LORA_OK)
        return c;
    if (seg->n_rows == 0)
        return LORA_OK;
    // validate both halves before enqueueing either
    if (!x_ok(st, x, ldx) || !y_ok(st, y, ldy))
        return LORA_E_ARG;
    ApplyArgs a = make_args(st, seg);
    if (apply_one_launch_pays(st, a, seg->n_rows)) {
        a.x = x;
        a.ldx = ldx;
        a.y = y;
        a.ldy = ldy;
        LORA_TRY(launch_apply(st->dtype == LORA_BF16 ? DT_BF16 : DT_F32, a,
                              max_tiles_for(seg->n_rows, st->n_slots),
                              reinterpret_cast<hipStream_t>(stream)));
        return LORA_OK;
    }
    const lora_status s1 = lora_add_shrink(st, x, ldx, seg, stream);
    if (s1 != LORA_OK)
        return s1;
    return lora_add_expand(st, y, ldy, seg, stream);
}

lora_status lora_build_shrink(const lora_stack *st, const void *x, int64_t ldx,
                              const int32_t *ids, int64_t n_rows, lora_segments *seg, void *stream)
{
    const lora_status c = check_build(st, ids, n_rows, seg);
    if (c != LORA_OK)
        return c;
    if (n_rows > st->max_rows || (n_rows > 0 && !x_ok(st, x, ldx)))
        return LORA_E_ARG;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const SegBuildArgs sb = make_seg_args(st, ids, n_rows, seg);
    if (!fused_build_pays(st, n_rows)) {
        LORA_TRY(launch_seg_build(sb, s));
        mark_built(seg, st, n_rows);
        return lora_add_shrink(st, x, ldx, seg, stream);
    }
    mark_built(seg, st, n_rows);
    ApplyArgs a = make_args(st, seg);
    a.x = x;
    a.ldx = ldx;
    LORA_TRY(launch_build_shrink(st->dtype == LORA_BF16 ? DT_BF16 : DT_F32, a, sb,
                                 max_tiles_for(n_rows, st->n_slots), s));
    return LORA_OK;
}

lora_status lora_build_apply(const lora_stack *st, void *y, int64_t ldy, const void *x,
                             int64_t ldx, const int32_t *ids, int64_t n_rows, lora_segments *seg,
                             void *stream)
{
    const lora_status c = check_build(st, ids, n_rows, seg);
    if (c != LORA_OK)
        return c;
    if (n_rows > st->max_rows)
        return LORA_E_ARG;
    if (n_rows > 0 && (!x_ok(st, x, ldx) || !y_ok(st, y, ldy)))
        return LORA_E_ARG;
    if (decode_pays(st, seg, n_rows)) {
        LORA_TRY(launch_decode(decode_args(st, seg, ids, n_rows, x, ldx, y, ldy),
                               reinterpret_cast<hipStream_t>(stream)));
        mark_built(seg, st, n_rows);
        return LORA_OK;
    }
    if (n_rows > 0 && fused_build_pays(st, n_rows)) {
        // one launch when the whole grid fits the chip (the decode step)
        ApplyArgs a = args_for_rows(st, seg, n_rows);
        if (one_launch_pays(st, a, n_rows)) {
            a.x = x;
            a.ldx = ldx;
            a.y = y;
            a.ldy = ldy;
            LORA_TRY(launch_build_apply(st->dtype == LORA_BF16 ? DT_BF16 : DT_F32, a,
                                        make_seg_args(st, ids, n_rows, seg),
                                        max_tiles_for(n_rows, st->n_slots),
                                        reinterpret_cast<hipStream_t>(stream)));
            mark_built(seg, st, n_rows);
            return LORA_OK;
        }
    }
    const lora_status s1 = lora_build_shrink(st, x, ldx, ids, n_rows, seg, stream);
    if (s1 != LORA_OK || n_rows == 0)
        return s1;
    return lora_add_expand(st, y, ldy, seg, stream);
}

lora_status lora_build_apply_plan(const lora_stack *st, int64_t n_rows, const lora_segments *seg,
                                  int32_t *n_launches)
{
    if (!st || !seg || !n_launches || n_rows < 0 || n_rows > st->max_rows || n_rows > seg->max_rows ||
        seg->n_slots_cap < st->n_slots || !current_device_is(st->device) || seg->device != st->device)
        return LORA_E_ARG;
    *n_launches = build_apply_launches(st, n_rows, seg);
    return LORA_OK;
}

lora_status lora_segments_download(const lora_segments *seg, int32_t *perm, int32_t *seg_off,
                                   int32_t *active, int32_t *counts, void *stream)
{
    if (!seg || !seg->built)
        return LORA_E_ARG;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (perm && seg->n_rows > 0)
        LORA_TRY(hipMemcpyAsync(perm, seg->perm, sizeof(int32_t) * seg->n_rows, hipMemcpyDeviceToHost, s));
    if (seg_off)
        LORA_TRY(hipMemcpyAsync(seg_off, seg->seg_off, sizeof(int32_t) * (seg->n_slots + 1),
                                hipMemcpyDeviceToHost, s));
    if (active)
        LORA_TRY(hipMemcpyAsync(active, seg->active, sizeof(int32_t) * seg->n_slots,
                                hipMemcpyDeviceToHost, s));
    if (counts)
        LORA_TRY(hipMemcpyAsync(counts, seg->counts, sizeof(int32_t) * 3, hipMemcpyDeviceToHost, s));
    LORA_TRY(hipStreamSynchronize(s));
    return LORA_OK;
}

lora_status lora_get_device_status(const lora_segments *seg, int64_t *n_bad, void *stream)
{
    if (!seg || !seg->built)
        return LORA_E_ARG;
    int32_t c[kCntSlots], sy[kSyncFlags];
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    LORA_TRY(hipMemcpyAsync(c, seg->counts, sizeof c, hipMemcpyDeviceToHost, s));
    LORA_TRY(hipMemcpyAsync(sy, seg->sync, sizeof sy, hipMemcpyDeviceToHost, s));
    LORA_TRY(hipStreamSynchronize(s));
    if (n_bad)
        *n_bad = c[kCntBad];
    if (sy[kSyncTimeouts] > 0) {
        // a one-launch apply gave up waiting for its v: reset the hand-over
        // state (flags, counters, epochs, tagged v) so that later calls start
        // clean; nothing runs on this stream meanwhile (it was synchronised)
        const size_t sync_ints = kSyncFlags + (size_t)seg->max_tiles * kSyncTileInts;
        LORA_TRY(hipMemsetAsync(seg->sync, 0, sizeof(int32_t) * sync_ints, s));
        if (seg->vtag)
            LORA_TRY(hipMemsetAsync(seg->vtag, 0,
                                    sizeof(uint32_t) * kDecodeWordsPerTile * seg->vtag_tiles, s));
        LORA_TRY(hipStreamSynchronize(s));
        return LORA_E_HIP;
    }
    return c[kCntBad] > 0 ? LORA_E_BAD_IDS : LORA_OK;
}

lora_status lora_segments_tile_counts(const lora_segments *seg, int32_t *n_bgmv, int32_t *n_sgmv,
                                      void *stream)
{
    if (!seg || !seg->built)
        return LORA_E_ARG;
    int32_t c[kCntSlots];
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    LORA_TRY(hipMemcpyAsync(c, seg->counts, sizeof c, hipMemcpyDeviceToHost, s));
    LORA_TRY(hipStreamSynchronize(s));
    if (n_bgmv)
        *n_bgmv = c[kCntBgmv];
    if (n_sgmv)
        *n_sgmv = c[kCntSgmv];
    return LORA_OK;
}

}  // extern "C"
