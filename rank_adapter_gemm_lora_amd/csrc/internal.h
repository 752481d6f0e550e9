// internal.h -- host-side structures of the library and the launchers of its
// kernels.  Not part of the public ABI (that is include/lora.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "lora.h"

namespace lora {

enum : int { DT_F32 = 0, DT_BF16 = 1 };   // element types of x, y and the pool

constexpr int kBgmvTileRows = 16;   // rows per BGMV shrink tile (small groups)
constexpr int kSgmvTileRows = 64;   // rows per SGMV shrink tile (dense groups, MFMA)
constexpr int kExpandCols = 256;    // output columns per expand workgroup
constexpr int kApplyThreads = 256;  // threads of every shrink / expand / decode workgroup
constexpr int kExpandLdsTable = 256;   // expand LDS: row indices first, then the slot table
constexpr int kExpandTableSlots = 256; // slot table in LDS up to this many slots
constexpr int kExpandLdsMax = 65536;   // dynamic LDS of one expand workgroup, at most
constexpr int kTileBgmv = 0;
constexpr int kTileSgmv = 1;
constexpr int kMaxKSplit = 16;      // most k-splits of one shrink
constexpr int kMaxExpandChunks = 16; // most 256-column chunks per expand workgroup
constexpr int kMaxSliceRank = 256;  // n_slices * r_max bound (LDS staging of v)
constexpr int kChunkRows = 256;     // rows per chunk of the large-batch grouping

// Device counts written by the segment builder.
enum : int {
    kCntValid = 0,    // rows with a valid adapter (= seg_off[n_slots])
    kCntActive = 1,   // slots with at least one row
    kCntBad = 2,      // ids that are neither -1 nor a loaded slot
    kCntSgmv = 3,     // SGMV shrink tiles (stored first in the tile list)
    kCntBgmv = 4,     // BGMV shrink tiles (stored after the SGMV tiles)
    kCntSlots = 8
};

// One tile: up to 64 rows of one slot (SGMV) or up to 16 (BGMV), with the
// rows' indices inline so one load brings the whole work description.  The
// shrink and the expand walk the same list.
struct alignas(16) ShrinkTile {
    int32_t slot, p0, cnt, path;   // p0: first position of the tile in the grouping
    int32_t rows[kSgmvTileRows];
};

struct SegBuildArgs {
    const int32_t *ids;
    int64_t n;
    int n_slots;
    const int32_t *slot_rank;
    int dense_min;     // groups with >= dense_min rows take the SGMV path
    int sgmv_rows;     // rows per SGMV tile (16 for small batches, 64 for large)
    int32_t *perm;
    int32_t *seg_off;
    int32_t *active;
    int32_t *counts;
    lora::ShrinkTile *tiles;
    // scratch of the chunked grouping (batches above 1024 rows)
    int32_t *keys;        // [max_rows] bucket of each row
    int32_t *chunk;       // [chunks][n_slots + 1] histograms, then their prefixes
    int32_t *chunk_bad;   // [chunks] bad ids per chunk
    int4 *binfo;          // [n_slots + 1] group offset, first tile, tile shift, path
};

// Everything a shrink or expand kernel reads about the stack and the batch.
struct ApplyArgs {
    // stack
    const void *A;             // pool [n_slots][n_slices][r_max][k]
    const void *A_img;         // operand image of the pool (MFMA stacks), see kImgRows
    const void *B;             // pool, slot s: [D][rp_s] at s * b_slot_stride
    const int32_t *rank;       // [n_slots]
    const float *scale;        // [n_slots] alpha / rank
    int n_slots;
    int64_t k;
    int n_slices;
    int r_max;
    int64_t D;
    int64_t slice_off[LORA_MAX_SLICES + 1];
    int64_t a_slot_stride;     // elements
    int64_t b_slot_stride;     // elements
    float *vpart;              // [ks][max_rows][n_slices * r_max] k-split partials of v
    int64_t max_rows;
    int ks;                    // k-splits of the shrink
    int mfma_ok;               // dense tiles may use MFMA (bf16, 64-aligned slices)
    int sgmv_rows;             // rows per dense tile of this batch (16 or 64)
    int b_win;                 // expand (MFMA): ranks of B staged in LDS at once (multiple of 16)
    int lds_v_off;             // expand: dynamic LDS byte offsets of v and B staging
    int lds_b_off;
    int lds_bytes;             // expand: dynamic LDS bytes
    int cpw;                   // expand: 256-column chunks per workgroup (1: one chunk)
    int32_t *sync;             // one-launch apply: timeouts, per-tile flags and counters
    int wait_limit;            // one-launch apply: polls before a wait gives up
    int n_cu;                  // compute units of the device (persistent grids)
    int all_dense;             // every tile of the batch is an MFMA (SGMV) tile
    int tile_bound;            // run expand: tile bound of the launch
    int lds_order_off;         // run expand: dynamic LDS byte offset of the unit costs
    // batch
    const int32_t *counts;
    const ShrinkTile *tiles;
    const void *x;
    int64_t ldx;
    void *y;
    int64_t ldy;
};

hipError_t launch_seg_build(const SegBuildArgs &a, hipStream_t stream);
hipError_t launch_shrink(int dtype, const ApplyArgs &a, int max_tiles, hipStream_t stream);
// grouping and shrink in one launch; batches of at most 1024 rows
constexpr int kFusedMaxRows = 1024;
hipError_t launch_build_shrink(int dtype, const ApplyArgs &a, const SegBuildArgs &sb, int max_tiles,
                               hipStream_t stream);
hipError_t launch_expand(int dtype, const ApplyArgs &a, int max_tiles, hipStream_t stream);
// grouping, shrink and expand in one launch (16-row tiles, one chunk per expand
// workgroup); a.sync: kSyncFlags + max_tiles * kSyncTileInts ints, zeroed at
// creation (per tile: the split flags, then the expand workgroups' counter)
constexpr int kSyncTimeouts = 2, kSyncFlags = 16, kSyncTileInts = 32;
// run expand: tile headers each thread reads (tile bounds up to 512), and a
// unit's fixed cost in 64-byte units
constexpr int kRunHeadersPerThread = 2;
constexpr int kRunUnitFixed = 800;
static_assert(kSyncTileInts > kMaxKSplit, "a tile's flags and counter");
hipError_t launch_build_apply(int dtype, const ApplyArgs &a, const SegBuildArgs &sb, int max_tiles,
                              hipStream_t stream);
// workgroups of build_apply_kernel resident per CU with this much dynamic LDS
int build_apply_wgs_per_cu(int dtype, int lds_bytes);
// shrink and expand of a grouped batch in one launch (same conditions and
// hand-over as launch_build_apply), and its residency per CU
hipError_t launch_apply(int dtype, const ApplyArgs &a, int max_tiles, hipStream_t stream);
int apply_wgs_per_cu(int dtype, int lds_bytes);
// One-launch decode (decode.hip): grouping, shrink and expand of a batch of at
// most kDecodeMaxRows rows over at most kDecodeMaxSlots slots (bf16, one
// slice, rank <= 16), v handed over as tagged 32-bit words.
constexpr int kDecodeMaxRows = 256;
constexpr int kDecodeMaxSlots = 63;
constexpr int kDecodeMaxKs = 8;
// a tile's sync record, after the flags: the epoch of each k-split class (1,
// 2, 4, 8 splits: ints kDecEpoch + log2 ks), then the expand workgroups' counter
constexpr int kDecEpoch = 20, kDecCount = 24;
static_assert(kDecCount < kSyncTileInts && kDecEpoch > kMaxKSplit, "decode state beside the flags");
// tagged v words per tile: one region per k-split class, ks x 16 rows x 16 ranks each
constexpr int kDecodeWordsPerTile = (2 * kDecodeMaxKs - 1) * 16 * 16;
constexpr int kWaitSpinsDefault = 1 << 18;      // polls before a one-launch wait gives up
struct DecodeArgs {
    const int32_t *ids;
    int n;
    int n_slots;
    const int32_t *slot_rank;
    const float *slot_scale;
    const void *A_img;        // operand image of the pool: slot s at s * 16 * k
    const void *B;            // pool, slot s at s * b_slot_stride: [D][rp_s]
    int64_t b_slot_stride;
    int r_max;
    int64_t k;
    int64_t D;
    const void *x;
    int64_t ldx;
    void *y;
    int64_t ldy;
    int ks;                   // k-splits (<= kDecodeMaxKs, (k / 8) % (16 ks) == 0)
    int cpw;                  // 256-column chunks per expand workgroup (1, 2, 4)
    int ncg;                  // expand workgroups per tile: ceil(D / (256 cpw))
    int tiles_bound;          // T = ceil(n / 16) + min(n_slots, n)
    uint32_t *vtag;           // tagged v partials: region of class c at (2^c - 1) * vtag_tiles * 256
                              // words, [ks][tile][16 rows][16 ranks] in it
    int vtag_tiles;           // tile stride of vtag: fixed per segments object, >= T
    int32_t *tile_state;      // per tile kSyncTileInts ints (epoch, counter)
    int32_t *timeouts;        // waits that gave up are counted here (may be null)
    const int32_t *poison;    // nonzero at the start: leave y untouched (may be null)
    int wait_limit;
    // segments object (perm null: not written)
    int32_t *perm;
    int32_t *seg_off;
    int32_t *active;
    int32_t *counts;
    ShrinkTile *tiles;
};
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);
int decode_wgs_per_cu(int ks, int cpw);
// Tiles of one batch never exceed ceil(rows / 16) plus one ragged tile per group.
int max_tiles_for(int64_t n_rows, int n_slots);
int grid_tiles(int64_t n_rows, int n_slots, int sgmv_rows, int dense_min);
int decode_ks(int64_t k);
bool decode_fits(const lora_stack *st, int64_t n_rows, int cpw, int vt_tiles);
DecodeArgs decode_args_for(const lora_stack *st, const int32_t *ids, int64_t n_rows, const void *x,
                           int64_t ldx, void *y, int64_t ldy, int cpw);
bool x_ok(const lora_stack *st, const void *x, int64_t ldx);
bool y_ok(const lora_stack *st, const void *y, int64_t ldy);
lora_status status_of(hipError_t e);
bool device_is_current(int dev);
// Merge of one slot into a dense weight (rows tiled per slice, 64 rows a tile).
struct MergeArgs {
    const void *A;             // the slot's A: [n_slices][r_max][k]
    const void *B;             // the slot's B: [D][rp]
    void *W;                   // [D][ldw], updated in place
    int64_t ldw;
    int64_t k;
    int rank;                  // the slot's true rank
    int rp;                    // its B row pitch (rank rounded up to 8)
    int r_max;
    float s;                   // sign * alpha / rank
    int n_slices;
    int64_t slice_off[LORA_MAX_SLICES + 1];
    int tile0[LORA_MAX_SLICES + 1];   // first row tile of each slice; [n_slices] = total
    int n_cu;                  // compute units of the device (sizes the persistent grid)
};
int merge_row_tiles(int64_t d);
hipError_t launch_merge(int dtype, const MergeArgs &a, hipStream_t stream);
lora_status load_slot(lora_stack *st, int slot, int rank, float alpha, const void *A, const void *B,
                      hipMemcpyKind kind, bool sync, hipStream_t stream);

// Loads of several adapters into free slots by one kernel that reads their A
// and B straight from mapped pinned host memory (device-side pointers).
constexpr int kGatherJobs = 16;
struct GatherJob {
    const void *A;   // [n_slices][rank][k], device-accessible
    const void *B;   // [D][rank], device-accessible
    int slot;
    int rank;
    float scale;     // alpha / rank
    int pad;
};
struct GatherArgs {
    void *A_pool;
    void *A_img;       // the pool's operand image, or null
    void *B_pool;
    int32_t *rank_tab;
    float *scale_tab;
    int64_t k;
    int64_t D;
    int n_slices;
    int r_max;
    int rp_max;
    int esize;
    int n_jobs;
    GatherJob job[kGatherJobs];
};
hipError_t launch_gather_load(const GatherArgs &g, hipStream_t stream);

// The operand image of the A pool, kept beside it for stacks with the MFMA
// path: per (slot, slice, 16-rank chunk) one block of 16 x k elements in which
// the 16-byte granule of rank row 16 jc + m and 8-element k unit u sits at
// granule index 16 u + m (zero for rows at or past r_max).  A matrix-core
// operand of 16 rank rows x 4 consecutive units (lane 16 g + m: row m, unit
// u + g) is then one contiguous kilobyte, where the pool's row-major layout
// spreads it over 16 rows, 64 bytes each.
constexpr int kImgRows = 16;
struct ImageArgs {
    const void *A_pool;
    void *A_img;
    int64_t k;
    int n_slices;
    int r_max;
    int n_jobs;
    int slot[kGatherJobs];
};
// Rebuild the image of the listed slots from their pool regions (bf16).
hipError_t launch_build_image(const ImageArgs &g, hipStream_t stream);
// Record a host-gathered load in the stack's host state (after the launch).
void note_loaded(lora_stack *st, int slot, int rank, float alpha);
hipError_t launch_zero(void *p, size_t bytes, hipStream_t stream);
hipError_t launch_set_slot(int32_t *rank, float *scale, int slot, int r, float s,
                           hipStream_t stream);

}  // namespace lora

struct lora_stack {
    int device;
    lora_dtype dtype;
    int esize;
    int n_slots;
    int r_max;
    int rp_max;               // r_max rounded up to 8
    int64_t k;
    int n_slices;
    int64_t slice_d[LORA_MAX_SLICES];
    int64_t slice_off[LORA_MAX_SLICES + 1];
    int64_t D;
    int64_t max_rows;
    void *A_pool;
    void *A_img;              // operand image of A_pool (stacks with the MFMA path), else null
    void *B_pool;
    int32_t *d_rank;
    float *d_scale;
    float *vpart;
    mutable int n_cu;            // compute units of the device (0: not asked yet)
    mutable int one_launch_wpc;  // build_apply_kernel workgroups resident per CU (-1: not asked yet)
    mutable int apply_wpc;       // apply_kernel workgroups resident per CU (-1: not asked yet)
    std::vector<int> h_rank;
    std::vector<float> h_alpha;
};

struct lora_segments {
    int device;
    int64_t max_rows;
    int n_slots_cap;
    int max_tiles;
    int dense_min;
    int expand_chunks;   // 0: chosen from the shapes
    int32_t *sync;       // one-launch apply state: kSyncFlags + max_tiles * kSyncTileInts ints
    uint32_t *vtag;      // one-launch decode: tagged v partials, kDecodeWordsPerTile per tile
    int vtag_tiles;      // tile bound the decode buffer holds (0: no decode path)
    int wait_limit;      // polls before a one-launch wait gives up
    int32_t *perm;
    int32_t *seg_off;
    int32_t *active;
    int32_t *counts;
    lora::ShrinkTile *tiles;
    int32_t *keys;
    int32_t *chunk;
    int32_t *chunk_bad;
    int4 *binfo;
    // state of the last build
    int built;
    int built_dense_min; // dense_min the tiles were cut with
    int built_sgmv_rows; // dense tile height the tiles were cut with (16 or 64)
    int64_t n_rows;
    int n_slots;
};
