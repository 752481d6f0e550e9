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
//     16 (mu / 4) + 4 mt + mu % 4, so the accumulators land on the lane's 16
//     contiguous columns.  The N-tiles (16 rows each) are done one after the
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
// instance, built for six waves per SIMD) and expand_stream_kernel (several
// chunks per workgroup, the next chunk's loads in flight).
#include "device_common.h"
#include "internal.h"
#include "mfma.h"
#include "expand_tiles.h"

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
    const bool row_ok = m < cnt;
    const int64_t yrow = (int64_t)rows[min(m, cnt - 1)] * a.ldy;
    const int64_t bslot = (int64_t)s * a.b_slot_stride;
    const int P = v_pitch(a.n_slices, rp);
    int bcolumn[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
        bcolumn[mt] = 64 * wave + 16 * (m >> 2) + 4 * mt + (m & 3);

    // granules of chunk c's contiguous [ncol][rp] B block
    auto n_gran = [&](int c) {
        return (int)min((int64_t)kCols, a.D - (int64_t)(ch0 + c) * kCols) * ng;
    };
    auto load_chunk = [&](int c, Vec8<DT_BF16> &ya, Vec8<DT_BF16> &yb, uint4 (&bg)[NG]) {
        const int64_t c0 = (int64_t)(ch0 + c) * kCols;
        const int64_t cb = c0 + 64 * wave + 16 * g;
        if (row_ok && cb < a.D) {
            ya.load(a.y, yrow + cb);
            yb.load(a.y, yrow + cb + 8);
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
        const int64_t cb = c0 + 64 * wave + 16 * g;
        if (c0 + 64 * wave >= a.D)
            return;   // (uniform per wavefront: D is whole 64-column blocks)
        const int qq = slice_of(a, c0 + 64 * wave);
        f32x4_t acc[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
            acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        for (int jc = 0; jc < nj; ++jc) {
            const int jo = jc * 16 + 8 * (g & 1);
            // 8 ranks of row m: two 16-byte reads (ranks past r masked)
            const float4 *vr = reinterpret_cast<const float4 *>(vs + m * P + qq * rp + jo);
            const float4 va = vr[0], vb = vr[1];
            const float vv[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
            float f[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float v = (row_ok && jo + i < r) ? vv[i] : 0.f;
                f[i] = (g < 2) ? v : v - bf16_lo(pack_bf16x2(v, 0.f));
            }
            uint4 vop;
            vop.x = pack_bf16x2(f[0], f[1]);
            vop.y = pack_bf16x2(f[2], f[3]);
            vop.z = pack_bf16x2(f[4], f[5]);
            vop.w = pack_bf16x2(f[6], f[7]);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const uint4 bop = jo < rp ? *reinterpret_cast<const uint4 *>(bs + bcolumn[mt] * rp + jo)
                                          : make_uint4(0, 0, 0, 0);
                acc[mt] = mfma_bf16_16x16x32(bop, vop, acc[mt]);
            }
        }
        if (row_ok) {
            float f[16];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    f[4 * mt + i] = acc[mt][i];
            merge16<DT_BF16>(a, yrow + cb, true, true, ya, yb, scale, f);
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
        for (int e = threadIdx.x; e < a.n_slots; e += blockDim.x) {
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
        else
            hipLaunchKernelGGL(expand_kernel_bf16_short, grid, dim3(256), a.lds_bytes, stream, a);
    } else {
        hipLaunchKernelGGL((expand_kernel<DT_F32, 1, false>), grid, dim3(256), a.lds_bytes, stream, a);
    }
    return hipGetLastError();
}

}  // namespace lora
