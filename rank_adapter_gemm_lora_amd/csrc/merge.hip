// merge.hip -- folding one adapter into a dense base weight and taking it out
// again: for every output row o (in slice q) and input column i < k,
//
//      W[o][i] <- round(W[o][i] + sign * (alpha / r) * sum_j B[o][j] A_q[j][i]),
//
// one rounding per element from fp32.  Page "LoRA serving: multi-adapter
// dynamic loading", section 1 (merging versus keeping the adapter apart: the
// merged weight W + (alpha/r) B A serves that one adapter at the base model's
// cost, and subtracting the same product restores W).  Page "Multi-LoRA
// Serving", section 3.1: B is d x r, A is r x k.
//
// The pass reads and writes W once and the product has only r terms per
// element, so it is bound by HBM.  W is cut into 64 x 128 tiles that each lie
// inside one slice.  Every load of a tile (the adapter's rows and columns and
// the W tile) is issued before the first use of any of them, so a tile costs
// one round trip before its arithmetic.
//   bf16: the 64 x 128 x r product of a tile runs on the matrix cores, and the
//   fp32 result goes through LDS once more so that W is read and written in
//   16-byte units along its rows.  Weights of fewer than kMergeStreamTiles
//   tiles take one tile per workgroup; larger ones a persistent grid whose
//   workgroups walk runs of tiles with the next tile's loads in flight.
//   fp32: one tile per workgroup on the vector ALUs, in rank chunks of 16.
#include <algorithm>

#include "device_common.h"
#include "internal.h"
#include "mfma.h"

namespace lora {

namespace {

constexpr int kMergeRows = 64;
constexpr int kMergeCols = 128;
constexpr int kMergeThreads = 256;
constexpr int kMergeWgPerCu = 2;     // persistent bf16 workgroups per compute unit
// Weights of at least this many 64 x 128 tiles take the persistent kernel
// (measured: it wins on a 28672 x 4096 weight, 14336 tiles, and loses on a
// 4096 x 4096 one, 2048 tiles, where a workgroup gets too few tiles to pipeline).
constexpr int64_t kMergeStreamTiles = 4096;

__device__ __forceinline__ void merge_tile_origin(const MergeArgs &a, int &q, int64_t &o0)
{
    const int t = (int)blockIdx.y;
    q = 0;
    while (q + 1 < a.n_slices && t >= a.tile0[q + 1])
        ++q;
    o0 = a.slice_off[q] + (int64_t)(t - a.tile0[q]) * kMergeRows;
}

// LDS index (in 16-byte units) of unit u (8 bf16 columns) of staged A row j.
// Rows 8 apart land on different bank groups for the transposed column reads.
__device__ __forceinline__ int a_unit(int j, int u) { return j * 16 + (u ^ (2 * ((j >> 3) & 3))); }

// LDS index (in 16-byte units) of unit u (4 fp32 columns) of product row m.
// The four row groups one accumulator store covers land on distinct banks.
__device__ __forceinline__ int c_unit(int m, int u) { return m * 32 + (u ^ (4 * ((m >> 2) & 3))); }

// A 16-byte unit of zeros: the source of A copies past the rank or past k.
__device__ const uint4 g_merge_zero = {0u, 0u, 0u, 0u};

// bf16, one tile per workgroup (weights of fewer than kMergeStreamTiles tiles):
// NKC chunks of 32 rank values (rank <= 32 * NKC).  The slot's A rows for the
// tile's 128 columns are copied global -> LDS directly (global_load_lds, no
// registers held: they go to the B and W loads instead), row-major with
// XOR-swizzled 16-byte units -- the copy writes LDS lane-linearly, so the
// swizzle is applied to the source units -- and each lane gathers its 8 rank
// values of one column with 2-byte reads; wavefront w owns columns
// 32 w .. + 31 and all 64 rows.
template <int NKC>
__global__ __launch_bounds__(kMergeThreads) void merge_bf16_kernel(MergeArgs a)
{
    __shared__ uint4 lds[2048];   // 32 KB: A rows [32 NKC][128], then the fp32 product [64][128]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int su = tid & 15;                       // 16-byte unit of a tile row
    const int64_t c0 = (int64_t)blockIdx.x * kMergeCols;
    const int64_t scol = c0 + 8 * su;              // first column of this thread's unit
    const bool col_ok = scol < a.k;
    int q;
    int64_t o0;
    merge_tile_origin(a, q, o0);
    const int64_t o_end = a.slice_off[q + 1];
    const uint16_t *A = static_cast<const uint16_t *>(a.A) + (int64_t)q * a.r_max * a.k;
    const uint16_t *B = static_cast<const uint16_t *>(a.B);
    uint16_t *W = static_cast<uint16_t *>(a.W);
    // Every load below reads a clamped, in-bounds address and the value is
    // selected afterwards: no branches around loads, so they all stay in flight.
    const int64_t ccol = col_ok ? scol : a.k - 8;

    // A rows 0 .. 32 NKC - 1 of this column range (rows >= rank read as zero):
    // copy p of wavefront w fills LDS units 64 (4 p + w) .. + 63, i.e. rows
    // 4 (4 p + w) + lane / 16, position lane % 16, which holds unit
    // (lane % 16) ^ swizzle(row) of that row
    {
        const uint16_t *Z = reinterpret_cast<const uint16_t *>(&g_merge_zero);
        const int pu = lane & 15;
#pragma unroll
        for (int p = 0; p < 2 * NKC; ++p) {
            const int j = 4 * (4 * p + wave) + (lane >> 4);
            const int u = pu ^ (2 * ((j >> 3) & 3));
            const int64_t col = c0 + 8 * u;
            const uint16_t *src = (j < a.rank && col < a.k) ? A + (int64_t)j * a.k + col : Z;
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void *)src,
                (__attribute__((address_space(3))) void *)(lds + 64 * (4 * p + wave)), 16, 0, 0);
        }
    }
    // matrix-core row operand: B rows o0 + 16 mb + lane % 16, rank values
    // 32 c + 8 (lane / 16) .. + 7 (the pool pads each row to rp with zeros)
    // (raw values: masked where the matrix cores take them, so no select waits
    // on these loads before the rest are issued)
    uint4 bop[NKC][4];
#pragma unroll
    for (int c = 0; c < NKC; ++c) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int64_t o = o0 + 16 * mb + (lane & 15);
            const int g = 4 * c + (lane >> 4);
            bop[c][mb] = load16(B, min(o, o_end - 1) * a.rp + 8 * min(g, a.rp / 8 - 1));
        }
    }
    // this thread's four W units: rows o0 + tid / 16 + 16 p
    uint4 w[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int64_t o = o0 + (tid >> 4) + 16 * p;
        w[p] = load16(W, min(o, o_end - 1) * a.ldw + ccol);   // unused when out of the tile
    }
    // every load above is issued before anything that uses one (the scheduler
    // would otherwise pull a B mask up and wait for all loads before W's)
    __builtin_amdgcn_sched_barrier(0);

    lds_barrier();   // (waits for the A copies)

    // the tile of B A: wave owns columns 32 wave .. + 31, all 64 rows
    f32x4_t acc[4][2];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
        acc[mb][0] = acc[mb][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const uint16_t *as = reinterpret_cast<const uint16_t *>(lds);
#pragma unroll
    for (int c = 0; c < NKC; ++c) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const int n = 32 * wave + 16 * nb + (lane & 15);
            const int jb = 32 * c + 8 * (lane >> 4);
            uint32_t h[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                h[e] = as[a_unit(jb + e, n >> 3) * 8 + (n & 7)];
            const uint4 col = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                                         h[6] | (h[7] << 16));
            const bool g_ok = 8 * (4 * c + (lane >> 4)) < a.rp;
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                const bool ok = g_ok && o0 + 16 * mb + (lane & 15) < o_end;
                acc[mb][nb] = mfma_bf16_16x16x32(keep_if(ok, bop[c][mb]), col, acc[mb][nb]);
            }
        }
    }
    lds_barrier();   // every wave is done with the A rows

    float *cs = reinterpret_cast<float *>(lds);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const int col = 32 * wave + 16 * nb + (lane & 15);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 16 * mb + 4 * (lane >> 4) + i;
                cs[c_unit(m, col >> 2) * 4 + (col & 3)] = acc[mb][nb][i];
            }
        }
    }
    lds_barrier();

    const float4 *c4 = reinterpret_cast<const float4 *>(lds);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int m = (tid >> 4) + 16 * p;
        const int64_t o = o0 + m;
        if (o >= o_end || !col_ok)
            continue;
        const float4 lo = c4[c_unit(m, 2 * su)], hi = c4[c_unit(m, 2 * su + 1)];
        const float d[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        const uint32_t ww[4] = {w[p].x, w[p].y, w[p].z, w[p].w};
        float f[8];
#pragma unroll
        for (int m2 = 0; m2 < 4; ++m2) {
            f[2 * m2] = fmaf(a.s, d[2 * m2], bf16_lo(ww[m2]));
            f[2 * m2 + 1] = fmaf(a.s, d[2 * m2 + 1], bf16_hi(ww[m2]));
        }
        Vec8<DT_BF16>::store(W, o * a.ldw + scol, f);
    }
}

// Column slab, slice and first row of tile t.  Tiles run slab-major: the row
// tiles of all slices for columns [0, 128), then for [128, 256), ...
__device__ __forceinline__ void merge_tile(const MergeArgs &a, int64_t t, int64_t &c0, int &q, int64_t &o0)
{
    const int rt_total = a.tile0[a.n_slices];
    const int64_t slab = t / rt_total;
    const int rt = (int)(t - slab * rt_total);
    c0 = slab * kMergeCols;
    q = 0;
    while (q + 1 < a.n_slices && rt >= a.tile0[q + 1])
        ++q;
    o0 = a.slice_off[q] + (int64_t)(rt - a.tile0[q]) * kMergeRows;
}

// bf16, large weights: NKC chunks of 32 rank values.  Persistent: each
// workgroup walks a contiguous run of tiles, so consecutive tiles mostly share
// the column slab and slice, and the slot's A for that slab is staged in LDS
// once -- transposed, [128 columns][ranks], so each lane's matrix-core operand
// (8 rank values of one column) is one 16-byte LDS read.  While a tile is
// computed, the next tile's B rows and W are already loading.  Wavefront w owns rows
// 16 w .. 16 w + 15 of a tile and all 128 columns (8 N-blocks), so each B row
// is loaded once.  The fp32 product goes through LDS so W is read and written
// in 256-byte row runs.
template <int NKC>
__global__ __launch_bounds__(kMergeThreads) void merge_bf16_stream_kernel(MergeArgs a)
{
    constexpr int kRp = 32 * NKC + 8;              // A^T row pitch in elements (16-byte pad)
    __shared__ uint4 at_lds[kMergeCols * kRp / 8];  // A^T [128][kRp] bf16
    __shared__ uint4 c_lds[kMergeRows * kMergeCols / 4];   // fp32 product [64][128], swizzled
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int su = tid & 15;                       // 16-byte unit of a tile row
    const uint16_t *B = static_cast<const uint16_t *>(a.B);
    uint16_t *W = static_cast<uint16_t *>(a.W);
    uint16_t *at = reinterpret_cast<uint16_t *>(at_lds);
    float *cs = reinterpret_cast<float *>(c_lds);

    const int64_t n_slabs = (a.k + kMergeCols - 1) / kMergeCols;
    const int64_t T = n_slabs * a.tile0[a.n_slices];
    const int64_t t_begin = (int64_t)blockIdx.x * T / gridDim.x;
    const int64_t t_end = ((int64_t)blockIdx.x + 1) * T / gridDim.x;
    if (t_begin >= t_end)
        return;

    // this thread's four W units of a tile: rows o0 + tid / 16 + 16 p, columns
    // c0 + 8 su .. + 7 (clamped in-bounds addresses; units past the tile unused)
    auto load_w = [&](int64_t c0, int64_t o0, int64_t o_end, uint4 (&w)[4]) {
        const int64_t scol = c0 + 8 * su, ccol = scol < a.k ? scol : a.k - 8;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int64_t o = o0 + (tid >> 4) + 16 * p;
            w[p] = load16(W, min(o, o_end - 1) * a.ldw + ccol);
        }
    };

    // matrix-core row operand of a tile: B rows o0 + 16 wave + lane % 16, rank
    // values 32 c + 8 (lane / 16) .. + 7 (the pool pads each row to rp with zeros)
    auto load_b = [&](int64_t o0, int64_t o_end, uint4 (&bop)[NKC]) {
#pragma unroll
        for (int c = 0; c < NKC; ++c) {
            const int64_t o = o0 + 16 * wave + (lane & 15);
            const int g = 4 * c + (lane >> 4);
            const uint4 v = load16(B, min(o, o_end - 1) * a.rp + 8 * min(g, a.rp / 8 - 1));
            bop[c] = keep_if(o < o_end && 8 * g < a.rp, v);
        }
    };

    int64_t c0, o0;
    int q;
    merge_tile(a, t_begin, c0, q, o0);
    uint4 bop[NKC], w_cur[4];
    load_b(o0, a.slice_off[q + 1], bop);
    load_w(c0, o0, a.slice_off[q + 1], w_cur);
    int64_t staged_c0 = -1;
    int staged_q = -1;

    for (int64_t t = t_begin; t < t_end; ++t) {
        const int64_t o_end = a.slice_off[q + 1];
        // the next tile's B and W, in flight while this one is computed (issued
        // after this tile's, so waiting for this tile's never waits for them)
        int64_t nc0 = c0, no0 = o0;
        int nq = q;
        uint4 b_next[NKC], w_next[4];
        if (t + 1 < t_end) {
            merge_tile(a, t + 1, nc0, nq, no0);
            load_b(no0, a.slice_off[nq + 1], b_next);
            load_w(nc0, no0, a.slice_off[nq + 1], w_next);
        }
        // (uniform) new slab or slice: stage its A rows, transposed
        if (c0 != staged_c0 || q != staged_q) {
            if (staged_q >= 0)
                lds_barrier();   // every wavefront is done with the previous A^T
            const uint16_t *A = static_cast<const uint16_t *>(a.A) + (int64_t)q * a.r_max * a.k;
            const int64_t scol = c0 + 8 * su;
            const bool col_ok = scol < a.k;
            const int64_t ccol = col_ok ? scol : a.k - 8;
            uint4 v[2 * NKC];
#pragma unroll
            for (int p = 0; p < 2 * NKC; ++p) {
                const int j = (tid >> 4) + 16 * p;
                v[p] = keep_if(j < a.rank && col_ok, load16(A, (int64_t)min(j, a.rank - 1) * a.k + ccol));
            }
#pragma unroll
            for (int p = 0; p < 2 * NKC; ++p) {
                const int j = (tid >> 4) + 16 * p;
                const uint32_t wd[4] = {v[p].x, v[p].y, v[p].z, v[p].w};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    at[(8 * su + e) * kRp + j] = (uint16_t)(e & 1 ? wd[e >> 1] >> 16 : wd[e >> 1] & 0xffffu);
            }
            lds_barrier();
            staged_c0 = c0;
            staged_q = q;
        }

        f32x4_t acc[8];
#pragma unroll
        for (int nb = 0; nb < 8; ++nb)
            acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NKC; ++c) {
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
                const uint4 col = *reinterpret_cast<const uint4 *>(
                    at + (16 * nb + (lane & 15)) * kRp + 32 * c + 8 * (lane >> 4));
                acc[nb] = mfma_bf16_16x16x32(bop[c], col, acc[nb]);
            }
        }
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
            const int col = 16 * nb + (lane & 15);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 16 * wave + 4 * (lane >> 4) + i;
                cs[c_unit(m, col >> 2) * 4 + (col & 3)] = acc[nb][i];
            }
        }
        lds_barrier();

        const int64_t scol = c0 + 8 * su;
        const bool col_ok = scol < a.k;
        const float4 *c4 = reinterpret_cast<const float4 *>(c_lds);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int m = (tid >> 4) + 16 * p;
            const int64_t o = o0 + m;
            if (o >= o_end || !col_ok)
                continue;
            const float4 lo = c4[c_unit(m, 2 * su)], hi = c4[c_unit(m, 2 * su + 1)];
            const float d[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            const uint32_t ww[4] = {w_cur[p].x, w_cur[p].y, w_cur[p].z, w_cur[p].w};
            float f[8];
#pragma unroll
            for (int m2 = 0; m2 < 4; ++m2) {
                f[2 * m2] = fmaf(a.s, d[2 * m2], bf16_lo(ww[m2]));
                f[2 * m2 + 1] = fmaf(a.s, d[2 * m2 + 1], bf16_hi(ww[m2]));
            }
            Vec8<DT_BF16>::store(W, o * a.ldw + scol, f);
        }
        lds_barrier();   // the product buffer is rewritten by the next tile

#pragma unroll
        for (int p = 0; p < 4; ++p)
            w_cur[p] = w_next[p];
#pragma unroll
        for (int c = 0; c < NKC; ++c)
            bop[c] = b_next[c];
        c0 = nc0;
        o0 = no0;
        q = nq;
    }
}

// fp32: rank chunks of 16 staged in LDS, 4 rows x 8 columns per thread.
__global__ __launch_bounds__(kMergeThreads) void merge_f32_kernel(MergeArgs a)
{
    __shared__ float4 as[16 * 32];   // 16 rank rows x 128 columns
    __shared__ float bs[64 * 17];    // 64 rows x 16 rank values, padded
    const int tid = threadIdx.x, su = tid & 15;
    const int64_t scol = (int64_t)blockIdx.x * kMergeCols + 8 * su;
    const bool col_ok = scol < a.k;
    int q;
    int64_t o0;
    merge_tile_origin(a, q, o0);
    const int64_t o_end = a.slice_off[q + 1];
    const float *A = static_cast<const float *>(a.A) + (int64_t)q * a.r_max * a.k;
    const float *B = static_cast<const float *>(a.B);
    float *W = static_cast<float *>(a.W);

    float acc[4][8];
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[p][e] = 0.f;
    for (int j0 = 0; j0 < a.rank; j0 += 16) {
        // clamped in-bounds loads, values selected afterwards
        const int jj = j0 + (tid >> 4);
        const bool aok = jj < a.rank && col_ok;
        const float4 *ap = reinterpret_cast<const float4 *>(
            A + (int64_t)min(jj, a.rank - 1) * a.k + (col_ok ? scol : a.k - 8));
        const float4 a0 = ap[0], a1 = ap[1];
        as[(tid >> 4) * 32 + 2 * su] = keep_if(aok, a0);
        as[(tid >> 4) * 32 + 2 * su + 1] = keep_if(aok, a1);
        const int64_t o = o0 + (tid >> 2);
        const float *brow = B + min(o, o_end - 1) * a.rp;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = j0 + 4 * (tid & 3) + e;
            const float v = brow[min(j, a.rank - 1)];
            bs[(tid >> 2) * 17 + 4 * (tid & 3) + e] = (o < o_end && j < a.rank) ? v : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float4 lo = as[j * 32 + 2 * su], hi = as[j * 32 + 2 * su + 1];
            const float av[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const float b = bs[((tid >> 4) + 16 * p) * 17 + j];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    acc[p][e] = fmaf(b, av[e], acc[p][e]);
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int64_t o = o0 + (tid >> 4) + 16 * p;
        if (o >= o_end || !col_ok)
            continue;
        Vec8<DT_F32> wv;
        wv.load(W, o * a.ldw + scol);
        float f[8];
        wv.to_f32(f);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            f[e] = fmaf(a.s, acc[p][e], f[e]);
        Vec8<DT_F32>::store(W, o * a.ldw + scol, f);
    }
}

}  // namespace

int merge_row_tiles(int64_t d) { return (int)((d + kMergeRows - 1) / kMergeRows); }

hipError_t launch_merge(int dtype, const MergeArgs &a, hipStream_t stream)
{
    const dim3 grid((unsigned)((a.k + kMergeCols - 1) / kMergeCols), (unsigned)a.tile0[a.n_slices]);
    const dim3 block(kMergeThreads);
    if (grid.x == 0 || grid.y == 0)
        return hipSuccess;
    if (dtype == DT_F32) {
        hipLaunchKernelGGL(merge_f32_kernel, grid, block, 0, stream, a);
        return hipGetLastError();
    }
    const int64_t tiles = (int64_t)grid.x * grid.y;
    const int nkc = (a.rank + 31) / 32;
    if (tiles < kMergeStreamTiles) {
        switch (nkc) {
        case 1: hipLaunchKernelGGL(merge_bf16_kernel<1>, grid, block, 0, stream, a); break;
        case 2: hipLaunchKernelGGL(merge_bf16_kernel<2>, grid, block, 0, stream, a); break;
        case 3: hipLaunchKernelGGL(merge_bf16_kernel<3>, grid, block, 0, stream, a); break;
        default: hipLaunchKernelGGL(merge_bf16_kernel<4>, grid, block, 0, stream, a); break;
        }
        return hipGetLastError();
    }
    // persistent grid: kMergeWgPerCu workgroups per compute unit of the device,
    // each a run of tiles
    if (a.n_cu < 1)
        return hipErrorInvalidValue;
    const dim3 pgrid((unsigned)std::min<int64_t>(tiles, (int64_t)kMergeWgPerCu * a.n_cu));
    switch (nkc) {
    case 1: hipLaunchKernelGGL(merge_bf16_stream_kernel<1>, pgrid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL(merge_bf16_stream_kernel<2>, pgrid, block, 0, stream, a); break;
    case 3: hipLaunchKernelGGL(merge_bf16_stream_kernel<3>, pgrid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL(merge_bf16_stream_kernel<4>, pgrid, block, 0, stream, a); break;
    }
    return hipGetLastError();
}

}  // namespace lora
