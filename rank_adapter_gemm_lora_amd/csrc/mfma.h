// mfma.h -- gfx950 matrix-core helpers: v_mfma_f32_16x16x32_bf16 on raw 16-byte
// operands.  D[16x16] += A[16x32] * B[32x16] in fp32.  Operand lane l holds row
// (A) or column (B) l % 16 and 8 of the 32 K values; the accumulator lane holds
// D[4 * (l / 16) + i][l % 16], i = 0..3.  Which 8 K values a lane holds does not
// matter for a contraction as long as both operands agree, so callers load 8
// contiguous elements per operand (one 16-byte load).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lora {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma_bf16_16x16x32(uint4 a, uint4 b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint4 load16(const void *base, int64_t elem)
{
    return *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(base) + elem);
}

}  // namespace lora
