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
// element, so it is bound by HBM.  One workgroup owns a 64 x 128 tile of W that
// lies inside one slice.  Loads are issued adapter first, W last: a load
// counter wait for the adapter data then does not also wait for W, whose
// loads stay in flight while the product is formed.
//   bf16: the 64 x 128 x r product runs on the matrix cores.  The rank rows of
//   A are staged in LDS (XOR-swizzled 16-byte units) so that each lane can read
//   its 8 rank values of one column; the fp32 result goes through LDS once more
//   so that W is read and written in 16-byte runs along its rows.
//   fp32: the same tile on the vector ALUs, in rank chunks of 16.
#include "device_common.h"
#include "internal.h"
#include "mfma.h"

namespace lora {

namespace {

constexpr int kMergeRows = 64;
constexpr int kMergeCols = 128;
constexpr int kMergeThreads = 256;

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
__device__ __forceinline__ int c_unit(int m, int u) { return m * 32 + (u ^ (4 * ((m >> 2) & 3))); }

// bf16: NKC chunks of 32 rank values (rank <= 32 * NKC).
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

    // A rows 0 .. 32 NKC - 1 of this column range (rows >= rank read as zero)
    uint4 ast[2 * NKC];
#pragma unroll
    for (int p = 0; p < 2 * NKC; ++p) {
        const int j = (tid >> 4) + 16 * p;
        const uint4 v = load16(A, (int64_t)min(j, a.rank - 1) * a.k + ccol);
        ast[p] = keep_if(j < a.rank && col_ok, v);
    }
    // matrix-core row operand: B rows o0 + 16 mb + lane % 16, rank values
    // 32 c + 8 (lane / 16) .. + 7 (the pool pads each row to rp with zeros)
    uint4 bop[NKC][4];
#pragma unroll
    for (int c = 0; c < NKC; ++c) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int64_t o = o0 + 16 * mb + (lane & 15);
            const int g = 4 * c + (lane >> 4);
            const uint4 v = load16(B, min(o, o_end - 1) * a.rp + 8 * min(g, a.rp / 8 - 1));
            bop[c][mb] = keep_if(o < o_end && 8 * g < a.rp, v);
        }
    }
    // this thread's four W units: rows o0 + tid / 16 + 16 p
    uint4 w[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int64_t o = o0 + (tid >> 4) + 16 * p;
        w[p] = load16(W, min(o, o_end - 1) * a.ldw + ccol);   // unused when out of the tile
    }

#pragma unroll
    for (int p = 0; p < 2 * NKC; ++p)
        lds[a_unit((tid >> 4) + 16 * p, su)] = ast[p];
    lds_barrier();

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
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
                acc[mb][nb] = mfma_bf16_16x16x32(bop[c][mb], col, acc[mb][nb]);
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
    } else {
        switch ((a.rank + 31) / 32) {
        case 1: hipLaunchKernelGGL(merge_bf16_kernel<1>, grid, block, 0, stream, a); break;
        case 2: hipLaunchKernelGGL(merge_bf16_kernel<2>, grid, block, 0, stream, a); break;
        case 3: hipLaunchKernelGGL(merge_bf16_kernel<3>, grid, block, 0, stream, a); break;
        default: hipLaunchKernelGGL(merge_bf16_kernel<4>, grid, block, 0, stream, a); break;
        }
    }
    return hipGetLastError();
}

}  // namespace lora
