// apply.hip -- add_shrink and add_expand over the row tiles of one batch.
//
// Page "Multi-LoRA Serving: one base, many adapters", section 2 flowchart and
// section 3.4: after the shared base GEMM, add_shrink computes v = A x (rank r)
// and add_expand adds delta = B v * alpha / r, both grouped per adapter, and the
// rows merge y_i = base_i + delta_i.  Section 3.1: B is d x r, A is r x k.
//
// One launch of each step covers every tile of the batch; the grid is sized
// from the row count alone (an upper bound on the number of tiles) and each
// workgroup reads its tile from the plan written by the segment builder, so
// the launch never depends on the adapter mix.  Tiles of a large group (SGMV)
// are served by MFMA code; tiles of a small group (BGMV) by the vector code in
// this file:
//
//   shrink (BGMV): a workgroup takes <= 16 rows of one slot and one k-split.
//     Each wavefront owns up to 4 rows; each lane reads 8 consecutive k of A and
//     x per step (16-byte loads), accumulates 16 rank partials per row with
//     packed bf16 dot products, and a wavefront reduce-scatter folds the 64
//     lanes.  The per-split partial v goes to fp32 scratch, indexed by the
//     row's position in the grouping; the expand sums the splits in order.
//   expand (BGMV): a workgroup takes <= 16 rows of one slot and 512 output
//     columns; v of its rows is staged in LDS (summed over the k-splits), each
//     lane owns 8 consecutive columns, keeps their B values (rank-contiguous in
//     the pool) in registers and walks its rows: y = round(y + scale * B v).
#include "device_common.h"
#include "internal.h"
#include "sgmv.h"

namespace lora {

namespace {

template <int DT>
__device__ void bgmv_shrink_tile(const ApplyArgs &a, int s, int p0, int cnt, int ks)
{
    const int r = a.rank[s];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t g8 = a.k >> 3;                       // 8-element groups along k
    const int64_t gb = g8 * ks / a.ks, ge = g8 * (ks + 1) / a.ks;
    const int SR = a.n_slices * a.r_max;

    int row[4];
    bool rv[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int u = wave + 4 * m;
        rv[m] = u < cnt;
        row[m] = rv[m] ? a.perm[p0 + u] : 0;
    }
    if (!rv[0])
        return;

    for (int q = 0; q < a.n_slices; ++q) {
        for (int j0 = 0; j0 < r; j0 += 16) {
            const int64_t abase = ((int64_t)s * a.n_slices + q) * a.r_max * a.k + (int64_t)j0 * a.k;
            float acc[4][16];
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int jj = 0; jj < 16; ++jj)
                    acc[m][jj] = 0.f;

            for (int64_t g = gb + lane; g < ge; g += 64) {
                Vec8<DT> av[16];
#pragma unroll
                for (int jj = 0; jj < 16; ++jj) {
                    if (j0 + jj < r)
                        av[jj].load(a.A, abase + (int64_t)jj * a.k + g * 8);
                    else
                        av[jj].zero();
                }
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    if (rv[m]) {
                        Vec8<DT> xv;
                        xv.load(a.x, (int64_t)row[m] * a.ldx + g * 8);
#pragma unroll
                        for (int jj = 0; jj < 16; ++jj)
                            acc[m][jj] = av[jj].dot(xv, acc[m][jj]);
                    }
                }
            }

            const int j = (lane >> 2) & 15;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                if (rv[m]) {
                    const float t = wave_reduce_scatter16(acc[m]);
                    if ((lane & 3) == 0 && j0 + j < r)
                        a.vws[((int64_t)ks * a.max_rows + p0 + wave + 4 * m) * SR + q * a.r_max + j0 + j] = t;
                }
            }
        }
    }
}

template <int DT>
__device__ void bgmv_expand_tile(const ApplyArgs &a, int s, int p0, int cnt, int64_t c_begin,
                                 float *vsh)
{
    const int r = a.rank[s];
    const float scale = a.scale[s];
    if (r == 0)
        return;   // slot emptied since the grouping was built: rows stay untouched
    stage_v(a, p0, cnt, r, vsh);
    __syncthreads();

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t c = c_begin + lane * 8;
    if (c >= a.D)
        return;
    int q = 0;
    while (q + 1 < a.n_slices && c >= a.slice_off[q + 1])
        ++q;
    const int rp = (r + 7) & ~7;
    const int Sr = a.n_slices * r;
    const int64_t bbase = (int64_t)s * a.b_slot_stride + c * rp;   // 8 columns x rp, contiguous

    float acc[4][8];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int cc = 0; cc < 8; ++cc)
            acc[m][cc] = 0.f;

    for (int j0 = 0; j0 < r; j0 += 16) {
        float b[8][16];
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                float f[8];
                if (j0 + 8 * h < rp) {
                    Vec8<DT> bv;
                    bv.load(a.B, bbase + (int64_t)cc * rp + j0 + 8 * h);
                    bv.to_f32(f);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        f[e] = 0.f;
                }
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    b[cc][8 * h + e] = f[e];
            }
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int u = wave + 4 * m;
            if (u < cnt) {
                const float *vv = vsh + u * Sr + q * r + j0;
#pragma unroll
                for (int jj = 0; jj < 16; ++jj) {
                    if (j0 + jj < r) {
                        const float vj = vv[jj];
#pragma unroll
                        for (int cc = 0; cc < 8; ++cc)
                            acc[m][cc] = fmaf(b[cc][jj], vj, acc[m][cc]);
                    }
                }
            }
        }
    }

#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int u = wave + 4 * m;
        if (u < cnt) {
            const int64_t yi = (int64_t)a.perm[p0 + u] * a.ldy + c;
            Vec8<DT> yv;
            yv.load(a.y, yi);
            float f[8];
            yv.to_f32(f);
#pragma unroll
            for (int cc = 0; cc < 8; ++cc)
                f[cc] = fmaf(scale, acc[m][cc], f[cc]);
            Vec8<DT>::store(a.y, yi, f);
        }
    }
}

template <int DT>
__global__ __launch_bounds__(256) void shrink_kernel(ApplyArgs a)
{
    const int t = blockIdx.x;
    const int n_sg = a.counts[kCntSgmv];
    const int n_all = n_sg + a.counts[kCntBgmv];
    if (t >= n_all)
        return;
    const int4 tile = a.tiles[t];
    if (tile.w == kTileSgmv && a.mfma_ok) {
        sgmv_shrink_tile<DT>(a, tile.x, tile.y, tile.z, blockIdx.y);
    } else {
        // BGMV tile, or a dense tile of a stack without the MFMA path
        for (int sub = 0; sub < tile.z; sub += kBgmvTileRows)
            bgmv_shrink_tile<DT>(a, tile.x, tile.y + sub, min(kBgmvTileRows, tile.z - sub),
                                 blockIdx.y);
    }
}

template <int DT>
__global__ __launch_bounds__(256) void expand_kernel(ApplyArgs a)
{
    extern __shared__ float vsh[];
    const int t = blockIdx.y;
    const int n_all = a.counts[kCntSgmv] + a.counts[kCntBgmv];
    if (t >= n_all)
        return;
    const int64_t c_begin = (int64_t)blockIdx.x * kExpandCols;
    if (c_begin >= a.D)
        return;
    const int4 tile = a.tiles[t];
    if (tile.w == kTileSgmv && a.mfma_ok) {
        sgmv_expand_tile<DT>(a, tile.x, tile.y, tile.z, c_begin, vsh);
    } else {
        for (int sub = 0; sub < tile.z; sub += kBgmvTileRows) {
            bgmv_expand_tile<DT>(a, tile.x, tile.y + sub, min(kBgmvTileRows, tile.z - sub),
                                 c_begin, vsh);
            __syncthreads();   // vsh is restaged by the next sub-tile
        }
    }
}

}  // namespace

hipError_t launch_shrink(int dtype, const ApplyArgs &a, int max_tiles, hipStream_t stream)
{
    if (max_tiles <= 0)
        return hipSuccess;
    dim3 grid(max_tiles, a.ks);
    if (dtype == DT_BF16)
        hipLaunchKernelGGL(shrink_kernel<DT_BF16>, grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(shrink_kernel<DT_F32>, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_expand(int dtype, const ApplyArgs &a, int max_tiles, hipStream_t stream)
{
    if (max_tiles <= 0)
        return hipSuccess;
    const int col_tiles = (int)((a.D + kExpandCols - 1) / kExpandCols);
    dim3 grid(col_tiles, max_tiles);
    const size_t lds = sizeof(float) * (size_t)kSgmvTileRows * a.n_slices * a.r_max;
    if (dtype == DT_BF16)
        hipLaunchKernelGGL(expand_kernel<DT_BF16>, grid, dim3(256), lds, stream, a);
    else
        hipLaunchKernelGGL(expand_kernel<DT_F32>, grid, dim3(256), lds, stream, a);
    return hipGetLastError();
}

}  // namespace lora
