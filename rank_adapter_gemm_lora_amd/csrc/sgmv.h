// sgmv.h -- row tiles of large adapter groups on the gfx950 matrix cores.
//
// A tile holds up to 64 rows of one slot (a dense segment: the "segmented"
// grouped GEMM of page "Multi-LoRA Serving: one base, many adapters", section
// 3.2).  Both steps use v_mfma_f32_16x16x32_bf16 (D[16x16] += A[16x32] B[32x16],
// fp32 accumulate).  Operand lanes: lane l holds row/column (l % 16) of its
// operand and 8 of the 32 K values; the accumulator lane holds D[4*(l/16)+i][l%16]
// for i = 0..3.  Which 8 K values a lane holds does not matter for a
// contraction as long as both operands use the same assignment, so every lane
// loads 8 contiguous elements (one 16-byte load) per operand.
//
// shrink: M = rows (4 M-tiles of 16), N = ranks (16 per N-tile, one N-tile per
//   slice and rank chunk), K = k.  The four wavefronts split the workgroup's
//   k-range, so no operand is loaded twice; their partial tiles are summed in
//   LDS in wavefront order and written to the fp32 v scratch.  Each lane walks
//   its k in blocks of 4 x 8 contiguous elements (64 bytes per row per lane).
// expand: M = output columns, N = rows, K = 32 = 16 ranks of v rounded to bf16
//   ("hi") followed by the same 16 ranks of the rounding residual ("lo"); the
//   B operand repeats the 16 B values for both halves.  hi + lo carries v to
//   about 16 significant bits, so the product B v keeps fp32-level accuracy
//   while both MFMA inputs are bf16.  Column-to-lane mapping: inside a 64-column
//   block, M-tile mt, M index mu maps to column 16*(mu/4) + 4*mt + mu%4, which
//   gives each lane 16 contiguous columns of one row for the y read-modify-write.
#pragma once

#include "device_common.h"
#include "internal.h"

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

constexpr int kSgmvNTiles = 4;  // N-tiles (slice, rank chunk) accumulated at once
static_assert(kSgmvNTiles * 64 == 256, "one reduction entry per thread");

// Stage v of the rows at grouping positions [p0, p0 + cnt) into LDS, summed over
// the k-splits in split order: vsh[u * (S * r) + q * r + j].
__device__ inline void stage_v(const ApplyArgs &a, int p0, int cnt, int r, float *vsh)
{
    const int SR = a.n_slices * a.r_max;
    const int Sr = a.n_slices * r;
    const int64_t split_stride = a.max_rows * (int64_t)SR;
    for (int idx = threadIdx.x; idx < cnt * Sr; idx += blockDim.x) {
        const int u = idx / Sr;
        const int rem = idx - u * Sr;
        const int q = rem / r;
        const int j = rem - q * r;
        const float *src = a.vws + (int64_t)(p0 + u) * SR + q * a.r_max + j;
        float sum = 0.f;
        for (int kk = 0; kk < a.ks; ++kk)
            sum += src[kk * split_stride];
        vsh[idx] = sum;
    }
}

template <int DT>
__device__ void sgmv_shrink_tile(const ApplyArgs &a, int s, int p0, int cnt, int ks)
{
    if constexpr (DT == DT_BF16) {
        __shared__ f32x4_t red[4][kSgmvNTiles * 64];   // [wave][tt * 64 + lane]
        const int r = a.rank[s];
        const int nj = (r + 15) >> 4;
        const int NT = a.n_slices * nj;
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int m = lane & 15, g = lane >> 4;
        const int SR = a.n_slices * a.r_max;

        const int64_t g8 = a.k >> 3;
        const int64_t gb = g8 * ks / a.ks, ge = g8 * (ks + 1) / a.ks;
        const int64_t wb = gb + (ge - gb) * wave / 4, we = gb + (ge - gb) * (wave + 1) / 4;
        const int n_mt = (cnt + 15) >> 4;

        int64_t xrow[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int u = min(16 * mt + m, cnt - 1);       // clamp: results of u >= cnt are dropped
            xrow[mt] = (int64_t)a.perm[p0 + u] * a.ldx;
        }

        for (int t0 = 0; t0 < NT; t0 += kSgmvNTiles) {
            int64_t arow[kSgmvNTiles];
            bool aok[kSgmvNTiles];
#pragma unroll
            for (int tt = 0; tt < kSgmvNTiles; ++tt) {
                const int t = t0 + tt;
                const int q = t / nj, jc = t - q * nj;
                const int j = jc * 16 + m;
                aok[tt] = t < NT && j < r;
                arow[tt] = aok[tt] ? (((int64_t)s * a.n_slices + q) * a.r_max + j) * a.k : 0;
            }
            f32x4_t acc[4][kSgmvNTiles];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int tt = 0; tt < kSgmvNTiles; ++tt)
                    acc[mt][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

            for (int64_t u0 = wb; u0 < we; u0 += 16) {
                uint4 xs[4][4], as[kSgmvNTiles][4];
#pragma unroll
                for (int st = 0; st < 4; ++st) {
                    const int64_t unit = u0 + 4 * g + st;
                    const bool ok = unit < we;
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt)
                        xs[mt][st] = (ok && mt < n_mt) ? load16(a.x, xrow[mt] + unit * 8)
                                                      : make_uint4(0, 0, 0, 0);
#pragma unroll
                    for (int tt = 0; tt < kSgmvNTiles; ++tt)
                        as[tt][st] = (ok && aok[tt]) ? load16(a.A, arow[tt] + unit * 8)
                                                     : make_uint4(0, 0, 0, 0);
                }
#pragma unroll
                for (int st = 0; st < 4; ++st)
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt)
                        if (mt < n_mt) {
#pragma unroll
                            for (int tt = 0; tt < kSgmvNTiles; ++tt)
                                acc[mt][tt] = mfma_bf16_16x16x32(xs[mt][st], as[tt][st], acc[mt][tt]);
                        }
            }

            // fixed-order sum of the four k-quarters, one M-tile at a time
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                if (mt >= n_mt)
                    break;
#pragma unroll
                for (int tt = 0; tt < kSgmvNTiles; ++tt)
                    red[wave][tt * 64 + lane] = acc[mt][tt];
                __syncthreads();
                {
                    const int e = threadIdx.x;            // kSgmvNTiles * 64 == 256 entries
                    const f32x4_t v = ((red[0][e] + red[1][e]) + red[2][e]) + red[3][e];
                    const int ln = e & 63, tt = e >> 6;
                    const int t = t0 + tt;
                    const int q = t / nj, jc = t - q * nj;
                    const int j = jc * 16 + (ln & 15);
                    if (t < NT && j < r) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int u = 16 * mt + 4 * (ln >> 4) + i;
                            if (u < cnt)
                                a.vws[((int64_t)ks * a.max_rows + p0 + u) * SR + q * a.r_max + j] = v[i];
                        }
                    }
                }
                __syncthreads();
            }
        }
    }
}

template <int DT>
__device__ void sgmv_expand_tile(const ApplyArgs &a, int s, int p0, int cnt, int64_t c_begin,
                                 float *vsh)
{
    if constexpr (DT == DT_BF16) {
        const int r = a.rank[s];
        const float scale = a.scale[s];
        if (r == 0)
            return;   // slot emptied since the grouping was built: rows stay untouched
        stage_v(a, p0, cnt, r, vsh);
        __syncthreads();

        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int m = lane & 15, g = lane >> 4;
        const int nj = (r + 15) >> 4;
        const int rp = (r + 7) & ~7;
        const int Sr = a.n_slices * r;
        const int64_t bslot = (int64_t)s * a.b_slot_stride;

        for (int half = 0; half < 2; ++half) {
            const int64_t cb = c_begin + 128 * wave + 64 * half;   // 64-column block
            if (cb >= a.D)
                break;
            int q = 0;
            while (q + 1 < a.n_slices && cb >= a.slice_off[q + 1])
                ++q;

            f32x4_t acc[4][4];   // [mt][nt]
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int nt = 0; nt < 4; ++nt)
                    acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

            for (int jc = 0; jc < nj; ++jc) {
                const int jo = jc * 16 + 8 * (g & 1);       // this lane's first rank
                // B operand: v of row (16 nt + m), ranks jo .. jo+7, hi (g < 2) or lo
                uint4 vop[4];
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    const int u = 16 * nt + m;
                    float f[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int j = jo + i;
                        const float v = (u < cnt && j < r) ? vsh[u * Sr + q * r + j] : 0.f;
                        const float hi = __uint_as_float(pack_bf16x2(v, 0.f) << 16);
                        f[i] = (g < 2) ? v : v - hi;
                    }
                    vop[nt].x = pack_bf16x2(f[0], f[1]);
                    vop[nt].y = pack_bf16x2(f[2], f[3]);
                    vop[nt].z = pack_bf16x2(f[4], f[5]);
                    vop[nt].w = pack_bf16x2(f[6], f[7]);
                }
                // A operand: B values of column col(mt, m), ranks jo .. jo+7
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    const int64_t col = cb + 16 * (m >> 2) + 4 * mt + (m & 3);
                    const uint4 bop = (jo < rp) ? load16(a.B, bslot + col * rp + jo)
                                                : make_uint4(0, 0, 0, 0);
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt)
                        acc[mt][nt] = mfma_bf16_16x16x32(bop, vop[nt], acc[mt][nt]);
                }
            }

            // lane (g, m) holds row 16 nt + m, columns cb + 16 g + 4 mt + i
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const int u = 16 * nt + m;
                if (u < cnt) {
                    const int64_t yi = (int64_t)a.perm[p0 + u] * a.ldy + cb + 16 * g;
                    float f[16];
                    Vec8<DT_BF16> y0, y1;
                    y0.load(a.y, yi);
                    y1.load(a.y, yi + 8);
                    float lo8[8], hi8[8];
                    y0.to_f32(lo8);
                    y1.to_f32(hi8);
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        f[i] = lo8[i];
                        f[8 + i] = hi8[i];
                    }
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            f[4 * mt + i] = fmaf(scale, acc[mt][nt][i], f[4 * mt + i]);
                    float o0[8], o1[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        o0[i] = f[i];
                        o1[i] = f[8 + i];
                    }
                    Vec8<DT_BF16>::store(a.y, yi, o0);
                    Vec8<DT_BF16>::store(a.y, yi + 8, o1);
                }
            }
        }
    }
}

}  // namespace lora
