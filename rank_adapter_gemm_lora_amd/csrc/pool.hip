// pool.hip -- stream-ordered maintenance of the adapter pool: zero-filling a
// slot's region before a load, writing the device slot table (rank, scale) so
// that load -> apply -> evict on one stream need no host sync, loading
// several adapters at once straight from mapped pinned host memory, and
// rebuilding a loaded slot's operand image of A.
#include "internal.h"

namespace lora {

namespace {

__global__ void zero_kernel(uint4 *p, size_t n16)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        p[i] = make_uint4(0, 0, 0, 0);
}

__global__ void set_slot_kernel(int32_t *rank, float *scale, int slot, int r, float s)
{
    if (threadIdx.x == 0) {
        rank[slot] = r;
        scale[slot] = s;
    }
}

// One slot per blockIdx.y.  A: the pool region [n_slices][r_max][k] in 16-byte
// units, rows below the rank copied from the source, the rest zero (k % 8 == 0:
// no unit straddles a row).  B: [D][rp], rp = rank rounded up to 8; with
// rank == rp the region is the source itself, else element by element with
// zeros in the ranks past the rank.  Block 0 of the slot writes the slot table.
__global__ __launch_bounds__(256) void gather_load_kernel(GatherArgs g)
{
    const GatherJob &j = g.job[blockIdx.y];
    const int es = g.esize;
    const int rp = (j.rank + 7) & ~7;
    const int64_t row_elems = g.k, slice_elems = (int64_t)g.r_max * g.k;
    const int64_t a_units = (int64_t)g.n_slices * slice_elems * es / 16;
    const int epu = 16 / es;   // elements per 16-byte unit
    uint4 *adst = reinterpret_cast<uint4 *>(static_cast<char *>(g.A_pool) +
                                            (size_t)j.slot * g.n_slices * slice_elems * es);
    const char *asrc = static_cast<const char *>(j.A);
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < a_units; u += stride) {
        const int64_t e = u * epu;
        const int64_t q = e / slice_elems, rem = e - q * slice_elems;
        const int64_t row = rem / row_elems, col = rem - row * row_elems;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (row < j.rank)
            v = *reinterpret_cast<const uint4 *>(asrc + (((q * j.rank + row) * g.k) + col) * es);
        adst[u] = v;
    }
    char *bdst = static_cast<char *>(g.B_pool) + (size_t)j.slot * g.D * g.rp_max * es;
    const char *bsrc = static_cast<const char *>(j.B);
    if (rp == j.rank) {
        const int64_t b_units = g.D * j.rank * es / 16;
        for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < b_units; u += stride)
            reinterpret_cast<uint4 *>(bdst)[u] = reinterpret_cast<const uint4 *>(bsrc)[u];
    } else {
        const int64_t n = g.D * rp;
        for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += stride) {
            const int64_t o = e / rp, c = e - o * rp;
            if (es == 2) {
                const uint16_t v = c < j.rank ? reinterpret_cast<const uint16_t *>(bsrc)[o * j.rank + c] : 0;
                reinterpret_cast<uint16_t *>(bdst)[e] = v;
            } else {
                const uint32_t v = c < j.rank ? reinterpret_cast<const uint32_t *>(bsrc)[o * j.rank + c] : 0u;
                reinterpret_cast<uint32_t *>(bdst)[e] = v;
            }
        }
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        g.rank_tab[j.slot] = j.rank;
        g.scale_tab[j.slot] = j.scale;
    }
}

// One slot per blockIdx.y: its operand image, granule by granule, from its
// pool region [n_slices][r_max][k] (bf16).  Image granule d of the slot is
// (slice q, rank chunk jc, k unit u, row m) with d = ((q * njm + jc) * ku + u)
// * 16 + m; rows at or past r_max are zero.  Writes are contiguous, reads
// gather 16 rows: a one-time cost per loaded adapter.
__global__ __launch_bounds__(256) void build_image_kernel(ImageArgs g)
{
    const int slot = g.slot[blockIdx.y];
    const int64_t ku = g.k >> 3;
    const int njm = (g.r_max + kImgRows - 1) / kImgRows;
    const int64_t n = (int64_t)g.n_slices * njm * ku * kImgRows;
    const uint16_t *src = static_cast<const uint16_t *>(g.A_pool) + (int64_t)slot * g.n_slices * g.r_max * g.k;
    uint4 *dst = static_cast<uint4 *>(g.A_img) + (int64_t)slot * n;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; d < n; d += stride) {
        const int m = (int)(d & (kImgRows - 1));
        const int64_t rest = d / kImgRows;
        const int64_t u = rest % ku, qj = rest / ku;
        const int jc = (int)(qj % njm), q = (int)(qj / njm);
        const int row = jc * kImgRows + m;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (row < g.r_max)
            v = *reinterpret_cast<const uint4 *>(src + ((int64_t)q * g.r_max + row) * g.k + u * 8);
        dst[d] = v;
    }
}

}  // namespace

hipError_t launch_build_image(const ImageArgs &g, hipStream_t stream)
{
    if (g.n_jobs <= 0 || !g.A_img)
        return hipSuccess;
    hipLaunchKernelGGL(build_image_kernel, dim3(64, g.n_jobs), dim3(256), 0, stream, g);
    return hipGetLastError();
}

hipError_t launch_gather_load(const GatherArgs &g, hipStream_t stream)
{
    if (g.n_jobs <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(gather_load_kernel, dim3(64, g.n_jobs), dim3(256), 0, stream, g);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !g.A_img)
        return e;
    // the image is rebuilt from the pool just written (same stream)
    ImageArgs im{};
    im.A_pool = g.A_pool;
    im.A_img = g.A_img;
    im.k = g.k;
    im.n_slices = g.n_slices;
    im.r_max = g.r_max;
    im.n_jobs = g.n_jobs;
    for (int i = 0; i < g.n_jobs; ++i)
        im.slot[i] = g.job[i].slot;
    return launch_build_image(im, stream);
}

hipError_t launch_zero(void *p, size_t bytes, hipStream_t stream)
{
    const size_t n16 = bytes / 16;   // every pool region is a multiple of 16 bytes
    if (n16 == 0)
        return hipSuccess;
    size_t blocks = (n16 + 255) / 256;
    if (blocks > 4096)
        blocks = 4096;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<uint4 *>(p), n16);
    return hipGetLastError();
}

hipError_t launch_set_slot(int32_t *rank, float *scale, int slot, int r, float s,
                           hipStream_t stream)
{
    hipLaunchKernelGGL(set_slot_kernel, dim3(1), dim3(64), 0, stream, rank, scale, slot, r, s);
    return hipGetLastError();
}

}  // namespace lora
