// expand.hip -- add_expand with the per-row merge:
//     y_i[off_q + o] = round(y_i[off_q + o] + scale_s * (B_s v_i)[off_q + o]).
//
// Page "Multi-LoRA Serving: one base, many adapters", section 2 flowchart and
// section 3.4: add_expand computes delta = B v * alpha / r grouped per adapter
// and each row merges y_i = base_i + delta_i; section 3.1: B is d x r.  The sum
// is fp32 and rounded once into the storage type; rows without an adapter and
// columns past D are never written.
//
// Grid: (column chunks of 256, tile bound), over the same tile list as the
// shrink.  Each workgroup loads its tile record (slot, first grouping
// position, row count, path, row indices) and the slot table in one round
// trip, then puts every load of its chunk in flight at once -- the y of its
// rows x 256 columns, the B chunk and the k-split partials of v -- so the
// chunk costs one more round trip before the arithmetic.  v (the sum of the
// partials in split order) and B are staged in dynamically sized LDS; y stays
// in registers.  The column chunks of one tile are consecutive block indices,
// so with 8 | chunks per row every tile of a slot meets a given chunk of B on
// the same XCD.
//
//   SGMV tile (<= 64 rows of a dense group, bf16, 64-aligned slices), MFMA:
//     M = 16 columns, N = 16 rows, K = 32 = 16 ranks of v rounded to bf16
//     ("hi") then the same 16 ranks of the rounding residual ("lo"); the B
//     operand repeats those 16 B values.  hi + lo carries v to about 16
//     significant bits, so B v keeps fp32-level accuracy on bf16 inputs.
//     Inside a wavefront's 64 columns, M-tile mt, index mu is column
//     32 (mt / 2) + 8 (mu / 4) + 4 (mt % 2) + mu % 4, so the accumulators of
//     lane group g land on columns [8 g, 8 g + 8) and [32 + 8 g, 40 + 8 g):
//     each 16-byte y load or store instruction then covers whole 64-byte
//     halves of the rows' 128 bytes (with 16 contiguous columns per lane, each
//     instruction wrote every other 16 bytes of them).  The N-tiles (16 rows each) are done one after the
//     other with four accumulators, which keeps the register count -- and so
//     the number of workgroups resident per CU -- where a streaming kernel
//     needs it.  B sits in LDS as the chunk's contiguous [256 columns][rp]
//     block, copied with 16-byte loads; when that block would not fit beside
//     v, the ranks go through in windows of b_win, one LDS block each.
//   BGMV tile (<= 16 rows), vector ALU: the tile's B columns are staged in LDS
//     in passes (bf16: 8 rank pairs, fp32: 8 ranks); each lane forms the bf16
//     hi/lo pairs of its row's v and accumulates packed bf16 dot products
//     (v_dot2c_f32_bf16), or fp32 FMAs.
//
// The tile code and expand_body live in expand_tiles.h (shared with the
// one-launch kernels); this file holds the expand kernels: expand_kernel (one
// 256-column chunk per workgroup), expand_kernel_bf16_short (its 16-row bf16
// instance, built for six waves per SIMD), expand_stream_kernel (several
// chunks of one tile per workgroup, the next chunk's loads in flight) and
// expand_run_kernel (16-row dense batches: a grid that fits the chip, each
// workgroup a cost-balanced run of chunks with v prepared once per tile).
#include <algorithm>
#include <mutex>
#include <utility>
#include <vector>

#include "device_common.h"
#include "internal.h"
#include "mfma.h"
#include "expand_tiles.h"
#include "group.h"

namespace lora {

namespace {

template <int DT, int MT, bool WO>
__global__ __launch_bounds__(256) void expand_kernel(ApplyArgs a)
{
    expand_body<DT, MT, WO>(a, blockIdx.y, blockIdx.x);
}

// ------------------------------------------- SGMV, several chunks per tile

// Chunks [ch0, ch0 + n_ch) of one 16-row dense tile (bf16, the slot's whole
// rank in one B block).  v of every slice is staged once.  While chunk c is on
// the matrix cores, chunk c + 1's y (registers) and B block (registers,
// written to LDS once every wavefront is done with chunk c's) are in flight;
// the barriers in the loop order LDS only, so those loads cross them.  NG:
// 16-byte B granules per thread and chunk at the stack's widest rank
// (rp_max / 8 rounded up to 2, 4 or 8); a slot of lower rank loads rp / 8.
template <int NG>
__device__ void sgmv_expand_stream(const ApplyArgs &a, const int32_t *rows, int s, int r,
                                   float scale, int p0, int cnt, int ch0, int n_ch, float *vs,
                                   uint16_t *bs)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, m = lane & 15;
    const int rp = (r + 7) & ~7, nj = (r + 15) >> 4, ng = rp >> 3;
    vs = static_cast<float *>(__builtin_assume_aligned(vs, 16));   // 16-byte operand reads
    const bool row_ok = m < cnt;
    const int64_t yrow = (int64_t)rows[min(m, cnt - 1)] * a.ldy;
    const int64_t bslot = (int64_t)s * a.b_slot_stride;
    const int P = v_pitch(a.n_slices, rp);
    int bcolumn[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
        bcolumn[mt] = 64 * wave + 32 * (mt >> 1) + 8 * (m >> 2) + 4 * (mt & 1) + (m & 3);

    // granules of chunk c's contiguous [ncol][rp] B block
    auto n_gran = [&](int c) {
        return (int)min((int64_t)kCols, a.D - (int64_t)(ch0 + c) * kCols) * ng;
    };
    auto load_chunk = [&](int c, Vec8<DT_BF16> &ya, Vec8<DT_BF16> &yb, uint4 (&bg)[NG]) {
        const int64_t c0 = (int64_t)(ch0 + c) * kCols;
        const int64_t cb = c0 + 64 * wave + 8 * g;   // lane's columns: [cb, cb + 8), [cb + 32, cb + 40)
        if (row_ok && cb < a.D) {
            ya.load(a.y, yrow + cb);
            yb.load(a.y, yrow + cb + kHalf);
        }
        const int ngr = n_gran(c);
        const int64_t b0 = bslot + c0 * rp;
#pragma unroll
        for (int i = 0; i < NG; ++i) {
            const int e = i * kCols + (int)threadIdx.x;
            if (i < ng && e < ngr)
                bg[i] = load16(a.B, b0 + 8 * (int64_t)e);
        }
    };
    auto put_b = [&](int c, const uint4 (&bg)[NG]) {
        const int ngr = n_gran(c);
#pragma unroll
        for (int i = 0; i < NG; ++i) {
            const int e = i * kCols + (int)threadIdx.x;
            if (i < ng && e < ngr)
                *reinterpret_cast<uint4 *>(bs + 8 * e) = bg[i];
        }
    };
    auto compute = [&](int c, const Vec8<DT_BF16> &ya, const Vec8<DT_BF16> &yb) {
        const int64_t c0 = (int64_t)(ch0 + c) * kCols;
        const int64_t cb = c0 + 64 * wave + 8 * g;
        if (c0 + 64 * wave >= a.D)
            return;   // (uniform per wavefront: D is whole 64-column blocks)
        const int qq = slice_of(a, c0 + 64 * wave);
        f32x4_t acc[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
            acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        for (int jc = 0; jc < nj; ++jc) {
            const int jo = jc * 16 + 8 * (g & 1);
            // the four B operands read together (clamped address, selected
            // after), ahead of v's reads
            const bool bok = jo < rp;
            const int bo = min(jo, rp - 8);
            uint4 bop[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                bop[mt] = *reinterpret_cast<const uint4 *>(bs + bcolumn[mt] * rp + bo);
            const uint4 vop = v_operand(vs + m * P + qq * rp + jo, row_ok, r - jo, g >= 2);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                acc[mt] = mfma_bf16_16x16x32(keep_if(bok, bop[mt]), vop, acc[mt]);
        }
        if (row_ok) {
            float f[16];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    f[4 * mt + i] = acc[mt][i];
            merge16<DT_BF16>(a, yrow + cb, true, true, ya, yb, scale, f, kHalf);
        }
    };
    // chunk c from (cy, cz) while chunk c + 1 loads into (ny, nz)
    uint4 bg[NG];
    auto step = [&](int c, const Vec8<DT_BF16> &cy, const Vec8<DT_BF16> &cz, Vec8<DT_BF16> &ny,
                    Vec8<DT_BF16> &nz) {
        const bool more = c + 1 < n_ch;
        if (more)
            load_chunk(c + 1, ny, nz, bg);
        compute(c, cy, cz);
        if (more) {
            lds_barrier();   // every wavefront is done with chunk c's B
            put_b(c + 1, bg);
            lds_barrier();
        }
    };

    Vec8<DT_BF16> ya0, yb0, ya1, yb1;
    load_chunk(0, ya0, yb0, bg);
    stage_v(a, p0, cnt, r, 0, a.n_slices, vs);   // one round trip with chunk 0's loads
    put_b(0, bg);
    __syncthreads();
    for (int c = 0; c < n_ch; c += 2) {
        step(c, ya0, yb0, ya1, yb1);
        if (c + 1 < n_ch)
            step(c + 1, ya1, yb1, ya0, yb0);
    }
}

// Several consecutive 256-column chunks of one tile per workgroup (a.cpw of
// them): bf16 batches of 16-row dense tiles whose widest rank fits one B
// block beside v of every slice.  Dynamic LDS as expand_body, with v sized
// for all slices.
template <int NG>
__global__ __launch_bounds__(256) void expand_stream_kernel(ApplyArgs a)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    int32_t *rows = reinterpret_cast<int32_t *>(lds);
    int32_t *srank = reinterpret_cast<int32_t *>(lds + kExpandLdsTable);
    float *sscale = reinterpret_cast<float *>(lds + kExpandLdsTable + 4 * kExpandTableSlots);
    float *vs = reinterpret_cast<float *>(lds + a.lds_v_off);
    unsigned char *bst = lds + a.lds_b_off;
    const int n_chunks = (int)((a.D + kCols - 1) / kCols);
    const int ch0 = (int)blockIdx.x * a.cpw;
    if (ch0 >= n_chunks)
        return;   // (the grid's x extent is padded to a multiple of 8)
    const int n_ch = min(a.cpw, n_chunks - ch0);
    const int t = blockIdx.y;
    const ShrinkTile *T = a.tiles + t;
    const int4 h = *reinterpret_cast<const int4 *>(T);
    const int32_t my_row = threadIdx.x < kSgmvTileRows ? T->rows[threadIdx.x] : 0;
    const int n_tiles = a.counts[kCntSgmv] + a.counts[kCntBgmv];
    const bool table = a.n_slots <= kExpandTableSlots;
    if (table) {
#pragma unroll 1
        for (int e = threadIdx.x; e < a.n_slots; e += kApplyThreads) {
            srank[e] = a.rank[e];
            sscale[e] = a.scale[e];
        }
    }
    if (t >= n_tiles)
        return;
    const int s = h.x, p0 = h.y, cnt = h.z;
    if (threadIdx.x < kSgmvTileRows)
        rows[threadIdx.x] = my_row;
    __syncthreads();
    const int r = table ? srank[s] : a.rank[s];
    const float scale = table ? sscale[s] : a.scale[s];
    if (r == 0)
        return;   // slot emptied since the grouping was built: rows stay untouched
    if (h.w == kTileSgmv && a.mfma_ok) {
        sgmv_expand_stream<NG>(a, rows, s, r, scale, p0, cnt, ch0, n_ch, vs,
                               reinterpret_cast<uint16_t *>(bst));
        return;
    }
    // BGMV tile: chunk by chunk
    for (int c = 0; c < n_ch; ++c) {
        const int64_t c0 = (int64_t)(ch0 + c) * kCols;
        for (int sub = 0; sub < cnt; sub += kBgmvTileRows) {
            bgmv_expand_tile<DT_BF16>(a, rows + sub, s, r, scale, p0 + sub,
                                      min(kBgmvTileRows, cnt - sub), c0, vs,
                                      reinterpret_cast<uint32_t *>(bst));
            __syncthreads();   // LDS is restaged by the next sub-tile
        }
    }
}

// bf16 with 16-row dense tiles (every batch up to 4096 rows) fits 80 registers
// without spilling, so it is built for 6 wavefronts per SIMD: more of these
// latency-bound workgroups per CU keep more loads in flight.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(6, 8)))
void expand_kernel_bf16_short(ApplyArgs a)
{
    expand_body<DT_BF16, 1, false>(a, blockIdx.y, blockIdx.x);
}

// ------------------------------------------------ SGMV, runs of chunks

// s_waitcnt immediates (gfx9 encoding, vmcnt split over bits 3:0 and 15:14):
// this wavefront's LDS accesses drained, or its vector-memory accesses drained
// (global-to-LDS copies included); the other counters are not waited on.
constexpr int kWaitLds = 0xC07F;
constexpr int kWaitVm = 0x0F70;

// The one-chunk expand's work (16-row MFMA tiles, every group dense) on a grid
// that fits the chip at once, organised so that v is prepared once per tile
// rather than once per 256-column chunk.  The units of work are the (tile,
// chunk) pairs in tile-major order; workgroup w takes the contiguous run of
// units whose cumulative cost at their start lies in [w T / G, (w + 1) T / G)
// (T the total, G the grid), so a run crosses few tiles and all runs take
// about the same time.  A unit's cost is a fixed share (its round trips:
// measured per-unit times are mostly fixed) plus its y and B bytes; every
// workgroup computes the costs and their prefix sums itself, in LDS, from the
// tile headers.  For each tile of its run the workgroup stages the tile's v (the
// k-split partials summed in split order, every slice) in LDS once, with the
// first chunk's y and B loads in flight (only the slices the run touches);
// each wavefront turns its slice's v
// into the bf16 hi / lo MFMA operands in registers, and the chunks then only
// stream B (LDS) and y (registers).  Each wavefront copies into LDS and reads
// only its own 64 columns of a B chunk, so past the tile's v the wavefronts
// run their chunks without waiting for each other.  The arithmetic is the one-chunk kernel's
// (same operands, same order), so the results are bit-identical to it.
//
// Dynamic LDS (offsets from the host): the slot table, v of the current tile
// (the slices the run touches), one B chunk [256][rp], and the unit costs and
// their prefix sums (2 tile_bound + 1 ints).
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 8)))
void expand_run_kernel(ApplyArgs a)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    int32_t *srank = reinterpret_cast<int32_t *>(lds + kExpandLdsTable);
    float *sscale = reinterpret_cast<float *>(lds + kExpandLdsTable + 4 * kExpandTableSlots);
    float *vs = reinterpret_cast<float *>(lds + a.lds_v_off);
    uint16_t *bs = reinterpret_cast<uint16_t *>(lds + a.lds_b_off);
    int32_t *cost = reinterpret_cast<int32_t *>(lds + a.lds_order_off);   // [tile_bound]
    int32_t *cum = cost + a.tile_bound;                                   // [tile_bound + 1]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, m = lane & 15;
    const int n_chunks = (int)((a.D + kCols - 1) / kCols);

    // the batch's tile count, the slot table, every tile's (slot, rows) and
    // the record of tile blockIdx.x / chunks (a guess at the first tile of
    // this workgroup's run: reread when wrong), in one round trip (headers
    // past the batch's tiles are read in bounds, unused)
    const int t_first = (int)blockIdx.x / n_chunks;   // < tile_bound: the grid is at most the units' bound
    const int4 h_first = *reinterpret_cast<const int4 *>(a.tiles + t_first);
    const int32_t row_first = a.tiles[t_first].rows[m];
    const int n_tiles = a.counts[kCntSgmv] + a.counts[kCntBgmv];
    int2 th[kRunHeadersPerThread];
#pragma unroll
    for (int i = 0; i < kRunHeadersPerThread; ++i) {
        const int t = tid + i * 256;
        const int4 hd = t < a.tile_bound ? *reinterpret_cast<const int4 *>(a.tiles + t)
                                         : make_int4(0, 0, 0, 0);
        th[i] = make_int2(hd.x, hd.z);
    }
#pragma unroll 1
    for (int e = tid; e < a.n_slots; e += kApplyThreads) {
        srank[e] = a.rank[e];
        sscale[e] = a.scale[e];
    }
    lds_barrier();
    const int n_units = n_tiles * n_chunks;
    // one unit each when they all fit: numbered XCD-major over ceil(units / 8)
    // workgroups per XCD, so each XCD takes one contiguous stretch of units
    // (a tile's chunks and the tiles of a slot share an L2); the rest idle
    int u, u_end;
    {
        const int per = (n_units + 7) >> 3, j = (int)blockIdx.x >> 3;
        u = j < per ? min(((int)blockIdx.x & 7) * per + j, n_units) : n_units;
        u_end = min(u + 1, n_units);
    }
    if (n_units > (int)gridDim.x) {   // (uniform)
        // cost of one unit of each tile, in 64-byte units: a fixed share for
        // the unit's round trips and work (measured: about 50 KB worth), y
        // read and written (16 per row) and the B chunk (8 per rank)
#pragma unroll
        for (int i = 0; i < kRunHeadersPerThread; ++i) {
            const int t = tid + i * 256;
            if (t < n_tiles)
                cost[t] = kRunUnitFixed + 16 * th[i].y + 8 * ((srank[th[i].x] + 7) & ~7);
        }
        lds_barrier();
        // cum[t]: cost of all units of tiles 0 .. t - 1 (wavefront 0)
        if (wave == 0) {
            int carry = 0;
            for (int t0 = 0; t0 < n_tiles; t0 += 64) {
                const int t = t0 + lane;
                const int inc = wave_scan_dpp(t < n_tiles ? cost[t] * n_chunks : 0);
                if (t < n_tiles)
                    cum[t + 1] = carry + inc;
                carry += __builtin_amdgcn_readlane(inc, 63);
            }
            if (lane == 0)
                cum[0] = 0;
        }
        lds_barrier();
        // this workgroup's run: the units whose cumulative cost at their
        // start lies in [w T / G, (w + 1) T / G), with w numbered XCD-major so
        // that the runs of one XCD are one contiguous stretch of tiles: a
        // tile's v partials and the B chunks its slot's tiles share are then
        // read into one L2
        const uint32_t total = (uint32_t)cum[n_tiles];
        const int w = xcd_major((int)blockIdx.x, (int)gridDim.x);
        auto units_below = [&](uint64_t x) -> int {   // units starting below cost x
            if (x >= total)
                return n_units;
            int lo = 0, hi = n_tiles;   // cum[lo] <= x < cum[hi]
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if ((uint32_t)cum[mid] <= x)
                    lo = mid;
                else
                    hi = mid;
            }
            const uint32_t c = (uint32_t)cost[lo];
            return lo * n_chunks + (int)(((uint32_t)x - (uint32_t)cum[lo] + c - 1) / c);
        };
        // floor(w T / G) in 32-bit arithmetic (w <= G < 2^16, so w (T mod G)
        // fits): a 64-bit division by the runtime G would cost a long
        // instruction sequence at every workgroup's start
        const uint32_t G = gridDim.x, q = total / G, rm = total - q * G;
        auto share = [&](uint32_t v) -> uint64_t { return (uint64_t)(v * q + v * rm / G); };
        u = units_below(share((uint32_t)w));
        u_end = units_below(share((uint32_t)w + 1));
    }
    int bcolumn[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
        bcolumn[mt] = 64 * wave + 32 * (mt >> 1) + 8 * (m >> 2) + 4 * (mt & 1) + (m & 3);

    while (u < u_end) {
        // the chunks [c_begin, c_end) of one tile
        const int t = u / n_chunks, c_begin = u - t * n_chunks;
        const int c_end = min(n_chunks, c_begin + (u_end - u));
        u += c_end - c_begin;
        int4 h = h_first;
        int32_t my_row = row_first;
        if (t != t_first) {   // (uniform)
            h = *reinterpret_cast<const int4 *>(a.tiles + t);
            my_row = a.tiles[t].rows[m];
        }
        lds_barrier();   // the slot table (first tile); the last tile's LDS reads are done
        const int s = h.x, p0 = h.y, cnt = h.z;
        const int r = srank[s];
        const float scale = sscale[s];
        if (r == 0)
            continue;   // (uniform) slot emptied since the grouping was built: rows stay untouched
        const int rp = (r + 7) & ~7, nj = (r + 15) >> 4;
        const bool half_last = (rp & 15) != 0;   // the last 16-rank step holds 8 ranks
        // the slices the run's chunks touch
        const int q_lo = slice_of(a, (int64_t)c_begin * kCols);
        const int nq = slice_of(a, min((int64_t)c_end * kCols, a.D) - 1) - q_lo + 1;
        const int P = v_pitch(nq, rp);
        const bool row_ok = m < cnt;
        const int64_t yrow = (int64_t)(row_ok ? my_row : __shfl(my_row, 0)) * a.ldy;
        const int64_t bslot = (int64_t)s * a.b_slot_stride;
        int cur_q = -1;
        uint4 vop[4];
#pragma unroll
        for (int jc = 0; jc < 4; ++jc)
            vop[jc] = make_uint4(0, 0, 0, 0);
        for (int c = c_begin; c < c_end; ++c) {
            const int64_t c0 = (int64_t)c * kCols;
            const int64_t cw = c0 + 64 * wave;        // this wavefront's 64 columns
            const bool in_d = cw < a.D;               // (uniform per wavefront: whole 64-column blocks)
            const int64_t cb = cw + 8 * g;            // lane's columns [cb, cb + 8), [cb + 32, cb + 40)
            Vec8<DT_BF16> y0, y1;
            if (in_d) {
                y0.load(a.y, yrow + cb);
                y1.load(a.y, yrow + cb + kHalf);
            }
            // this wavefront's 64 columns of the chunk's [ncol][rp] B block (one
            // contiguous 128 rp bytes), global -> LDS, 16 bytes a lane, into the
            // part of the block that only this wavefront reads: no workgroup
            // barrier orders B, and the wavefronts do not wait for each other
            // between chunks.  Its LDS reads of the last chunk are done first.
            __builtin_amdgcn_s_waitcnt(kWaitLds);
            if (in_d) {
                const int gpw = rp >> 3;
                const uint16_t *src = static_cast<const uint16_t *>(a.B) + bslot + cw * rp + 8 * lane;
                uint16_t *dst = bs + 64 * wave * rp;
                for (int i = 0; i < gpw; ++i)
                    __builtin_amdgcn_global_load_lds(
                        (const __attribute__((address_space(1))) void *)(src + 512 * i),
                        (__attribute__((address_space(3))) void *)(dst + 512 * i), 16, 0, 0);
            }
            if (c == c_begin) {
                // v of the tile for those slices, summed over the k-splits in
                // split order (its loads in flight with the first chunk's)
                stage_v4(a, p0, cnt, r, q_lo, nq, vs);
                lds_barrier();
            }
            // this wavefront's v operands, rebuilt when its slice changes
            if (in_d) {
                const int q = slice_of(a, cw);
                if (q != cur_q) {
                    cur_q = q;
#pragma unroll
                    for (int jc = 0; jc < 4; ++jc) {
                        const int jo = jc * 16 + 8 * (g & 1);
                        if (jc < nj)
                            vop[jc] = v_operand(vs + m * P + (q - q_lo) * rp + jo, row_ok, r - jo, g >= 2);
                    }
                }
            }
            // this wavefront's B columns landed in LDS, and its y in registers
            // (waited on every path: otherwise the compiler, which does not know
            // in_d to be uniform, drains the last chunk's y stores before the
            // next chunk's loads)
            __builtin_amdgcn_s_waitcnt(kWaitVm);
            if (in_d) {
                f32x4_t acc[4];
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
                    acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int jc = 0; jc < 4; ++jc) {
                    if (jc < nj) {
                        const int jo = jc * 16 + 8 * (g & 1);
                        const int bo = min(jo, rp - 8);
                        uint4 bop[4];
#pragma unroll
                        for (int mt = 0; mt < 4; ++mt)
                            bop[mt] = *reinterpret_cast<const uint4 *>(bs + bcolumn[mt] * rp + bo);
                        // ranks past rp (only in a last step of 8 ranks) read as zero
                        const bool bok = !(half_last && jc == nj - 1) || jo < rp;
#pragma unroll
                        for (int mt = 0; mt < 4; ++mt)
                            acc[mt] = mfma_bf16_16x16x32(keep_if(bok, bop[mt]), vop[jc], acc[mt]);
                    }
                }
                if (row_ok) {
                    float f[16];
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            f[4 * mt + i] = acc[mt][i];
                    merge16<DT_BF16>(a, yrow + cb, true, true, y0, y1, scale, f, kHalf);
                }
            }
        }
    }
}

// Workgroups of expand_run_kernel resident per CU at this dynamic LDS size
// (0 on error), computed once per size.
int run_occupancy(int lds_bytes)
{
    static std::mutex mu;
    static std::vector<std::pair<int, int>> known;
    std::lock_guard<std::mutex> lock(mu);
    for (const auto &e : known)
        if (e.first == lds_bytes)
            return e.second;
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, expand_run_kernel, 256, lds_bytes) != hipSuccess)
        return 0;
    known.emplace_back(lds_bytes, occ);
    return occ;
}

// LDS layout of expand_run_kernel: sets the offsets in b, returns the dynamic
// LDS bytes.
int run_layout(ApplyArgs &b, int max_tiles)
{
    const int rp_max = (b.r_max + 7) & ~7;
    b.tile_bound = max_tiles;
    b.lds_v_off = kExpandLdsTable + 8 * kExpandTableSlots;
    const int v_bytes = (16 * (b.n_slices * rp_max + 4) * 4 + 15) & ~15;
    b.lds_b_off = b.lds_v_off + v_bytes;
    b.lds_order_off = b.lds_b_off + kCols * rp_max * 2;
    return b.lds_order_off + ((4 * (2 * max_tiles + 1) + 15) & ~15);
}

// expand_run_kernel serves bf16 batches of 16-row tiles that are all MFMA
// tiles, with at most 64 ranks (one B chunk in LDS; r_max a multiple of 4 for
// the 16-byte v staging), a slot table that fits LDS and a tile bound its
// setup covers, within the LDS budget.
bool run_fits(const ApplyArgs &a, int max_tiles)
{
    if (!a.all_dense || a.n_slots > kExpandTableSlots || a.r_max > 64 || a.r_max % 4 != 0 ||
        max_tiles > kRunHeadersPerThread * 256)
        return false;
    // the cumulative costs stay below 2^31
    const int64_t n_chunks = (a.D + kCols - 1) / kCols;
    if (n_chunks * max_tiles * (kRunUnitFixed + 16 * 16 + 8 * 64) >= ((int64_t)1 << 31))
        return false;
    ApplyArgs b = a;
    return run_layout(b, max_tiles) <= kExpandLdsMax;
}

}  // namespace

hipError_t launch_expand(int dtype, const ApplyArgs &a, int max_tiles, hipStream_t stream)
{
    if (max_tiles <= 0)
        return hipSuccess;
    const dim3 grid((unsigned)((a.D + kCols - 1) / kCols), max_tiles);
    const bool tall = a.sgmv_rows > kBgmvTileRows;   // 64-row dense tiles
    // B chunks in rank windows: windows outer (more registers, but such a
    // launch is held to two workgroups per CU by its LDS anyway)
    const bool windows = a.b_win < ((a.r_max + 7) & ~7);
    if (dtype == DT_BF16 && a.cpw > 1) {
        // several chunks per workgroup; the x extent is padded to a multiple of
        // 8 so that every tile's workgroup for a given chunk group sits on the
        // same XCD (consecutive block indices go to consecutive XCDs)
        const int n_chunks = (int)((a.D + kCols - 1) / kCols);
        int gx = (n_chunks + a.cpw - 1) / a.cpw;
        if (gx >= 8)
            gx = (gx + 7) & ~7;
        const dim3 sgrid((unsigned)gx, max_tiles);
        const int rp_max = (a.r_max + 7) & ~7;
        if (rp_max <= 16)
            hipLaunchKernelGGL(expand_stream_kernel<2>, sgrid, dim3(256), a.lds_bytes, stream, a);
        else if (rp_max <= 32)
            hipLaunchKernelGGL(expand_stream_kernel<4>, sgrid, dim3(256), a.lds_bytes, stream, a);
        else
            hipLaunchKernelGGL(expand_stream_kernel<8>, sgrid, dim3(256), a.lds_bytes, stream, a);
        return hipGetLastError();
    }
    if (dtype == DT_BF16) {
        if (tall && windows)
            hipLaunchKernelGGL((expand_kernel<DT_BF16, 4, true>), grid, dim3(256), a.lds_bytes, stream, a);
        else if (tall)
            hipLaunchKernelGGL((expand_kernel<DT_BF16, 4, false>), grid, dim3(256), a.lds_bytes, stream, a);
        else {
            // as many workgroups as are resident at once (a multiple of 8), at
            // most one per unit of the tile bound
            ApplyArgs b = a;
            const int lds = run_fits(a, max_tiles) ? run_layout(b, max_tiles) : 0;
            const int occ = lds > 0 ? run_occupancy(lds) : 0;
            const int64_t units = (int64_t)grid.x * max_tiles;
            const int64_t resident = (int64_t)occ * a.n_cu;
            // the one-chunk kernel for stacks of rank <= 32, whose v takes at
            // most two rank steps (measured faster there: q-proj at 256 rows
            // x 100 adapters, rank 16 13.2 -> 8.0 us, rank 32 14.7 -> 10.7 us;
            // 4096 rows up to 6 % faster); runs pay from rank 64 (MLP gate/up
            // 28.4 -> 25.7 us, down 9.5 -> 8.3 us)
            if (occ < 1 || a.n_cu < 1 || a.r_max <= 32) {
                hipLaunchKernelGGL(expand_kernel_bf16_short, grid, dim3(256), a.lds_bytes, stream, a);
            } else {
                int64_t g = std::min<int64_t>(units, resident);
                if (g >= 8)
                    g &= ~(int64_t)7;
                hipLaunchKernelGGL(expand_run_kernel, dim3((unsigned)g), dim3(256), lds, stream, b);
            }
        }
    } else {
        hipLaunchKernelGGL((expand_kernel<DT_F32, 1, false>), grid, dim3(256), a.lds_bytes, stream, a);
    }
    return hipGetLastError();
}

}  // namespace lora
