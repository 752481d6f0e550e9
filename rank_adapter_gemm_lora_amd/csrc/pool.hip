// pool.hip -- stream-ordered maintenance of the adapter pool: zero-filling a
// slot's region before a load, and writing the device slot table (rank,
// scale) so that load -> apply -> evict on one stream need no host sync.
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

}  // namespace

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
