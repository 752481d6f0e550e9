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
// position, row count, path, row indices) in one round trip, issues the y
// loads of its rows x 256 block before anything else (so the HBM round trip
// for y overlaps the v and B staging), and stages v of its rows for the
// slices the chunk touches, summing the shrink's k-split partials in split
// order.  Dense tiles have 16 rows in small batches (more workgroups) and 64
// in large ones (a B chunk then serves 64 rows).
// Lane (g, m) of wavefront w owns the 16 columns c0 + 64 w + 16 g .. + 15 of
// rows m, m + 16, ...  The column chunks of one tile are consecutive block
// indices, so with 8 | chunks per row every tile of a slot meets a given chunk
// of B on the same XCD.
//
//   SGMV tile (<= 64 rows of a dense group, bf16, 64-aligned slices), MFMA:
//     M = 16 columns, N = 16 rows (up to 4 N-tiles), K = 32 = 16 ranks of v
//     rounded to bf16 ("hi") then the same 16 ranks of the rounding residual
//     ("lo"); the B operand repeats those 16 B values and is reused by every
//     N-tile.  hi + lo carries v to about 16 significant bits, so B v keeps
//     fp32-level accuracy on bf16 inputs.  Inside a wavefront's 64 columns,
//     M-tile mt, index mu is column 16 (mu / 4) + 4 mt + mu % 4, so the
//     accumulators land on the lane's 16 contiguous columns.
//   BGMV tile (<= 16 rows), vector ALU: the tile's B columns are staged in LDS
//     as bf16 rank pairs; each lane forms the bf16 hi/lo pairs of its row's v
//     and accumulates packed bf16 dot products (v_dot2c_f32_bf16).
#include "device_common.h"
#include "internal.h"
#include "mfma.h"

namespace lora {

namespace {

constexpr int kPairChunk = 16;                       // rank pairs of B per LDS pass (vector path)
constexpr int kLdsFloats = kExpandVsFloats;          // v staging; the vector path shares it with B
constexpr int kVecVsFloats = kLdsFloats - kPairChunk * kExpandCols;

__device__ __forceinline__ int slice_of(const ApplyArgs &a, int64_t c)
{
    int q = 0;
    while (q + 1 < a.n_slices && c >= a.slice_off[q + 1])
        ++q;
    return q;
}

// bf16 hi / lo parts of two fp32 values, each packed as a bf16 pair.
__device__ __forceinline__ void split_pair(float v0, float v1, uint32_t &hi, uint32_t &lo)
{
    hi = pack_bf16x2(v0, v1);
    lo = pack_bf16x2(v0 - bf16_lo(hi), v1 - bf16_hi(hi));
}

// v of rows [p0, p0 + cnt) for slices [q_lo, q_lo + nq) -> vs[u][qq * r + j],
// the sum of the k-split partials in split order.
__device__ __forceinline__ void stage_v(const ApplyArgs &a, int p0, int cnt, int r, int q_lo,
                                        int nq, float *vs)
{
    const int SR = a.n_slices * a.r_max, pitch = nq * r;
    const int64_t split = a.max_rows * (int64_t)SR;
    const uint32_t m_pitch = div_magic(pitch), m_r = div_magic(r);   // cnt * pitch <= 2^14
    for (int idx = threadIdx.x; idx < cnt * pitch; idx += blockDim.x) {
        const int u = div_small(idx, m_pitch);
        const int rem = idx - u * pitch;
        const int qq = div_small(rem, m_r);
        const int j = rem - qq * r;
        const float *src = a.vpart + (int64_t)(p0 + u) * SR + (q_lo + qq) * a.r_max + j;
        float part[kMaxKSplit];   // every split's load in flight before the first add
#pragma unroll
        for (int kk = 0; kk < kMaxKSplit; ++kk)
            part[kk] = kk < a.ks ? src[kk * split] : 0.f;
        float sum = part[0];
#pragma unroll
        for (int kk = 1; kk < kMaxKSplit; ++kk)
            if (kk < a.ks)
                sum += part[kk];
        vs[idx] = sum;
    }
}

template <int DT>
__device__ __forceinline__ void merge16(const ApplyArgs &a, int64_t yi, bool h0, bool h1,
                                        const Vec8<DT> &y0, const Vec8<DT> &y1, float scale,
                                        const float (&acc)[16])
{
    if (h0) {
        float f[8];
        y0.to_f32(f);
#pragma unroll
        for (int c = 0; c < 8; ++c)
            f[c] = fmaf(scale, acc[c], f[c]);
        Vec8<DT>::store(a.y, yi, f);
    }
    if (h1) {
        float f[8];
        y1.to_f32(f);
#pragma unroll
        for (int c = 0; c < 8; ++c)
            f[c] = fmaf(scale, acc[8 + c], f[c]);
        Vec8<DT>::store(a.y, yi + 8, f);
    }
}

__device__ void sgmv_expand_tile(const ApplyArgs &a, const int32_t *rows, int s, int r, float scale,
                                 int p0, int cnt, int64_t c0, float *vs)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, m = lane & 15;
    const int n_nt = (cnt + 15) >> 4;
    const int64_t cb = c0 + 64 * wave + 16 * g;      // lane's 16 columns
    const bool in_d = cb < a.D;                      // whole 64-column blocks (slices % 64 == 0)

    // y of this lane's rows, in flight from here on
    int64_t yi[4];
    Vec8<DT_BF16> y0[4], y1[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        const int u = 16 * nt + m;
        yi[nt] = (int64_t)rows[min(u, cnt - 1)] * a.ldy + cb;   // rows[0 .. cnt) only
        if (nt < n_nt && u < cnt && in_d) {
            y0[nt].load(a.y, yi[nt]);
            y1[nt].load(a.y, yi[nt] + 8);
        }
    }
    // the first 16 ranks of B for the lane's columns, also in flight
    const int rp = (r + 7) & ~7, nj = (r + 15) >> 4;
    const int64_t bslot = (int64_t)s * a.b_slot_stride;
    const int64_t cbw = c0 + 64 * wave;
    int64_t col[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
        col[mt] = in_d ? cbw + 16 * (m >> 2) + 4 * mt + (m & 3) : 0;
    uint4 bop[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
        bop[mt] = (in_d && 8 * (g & 1) < rp) ? load16(a.B, bslot + col[mt] * rp + 8 * (g & 1))
                                             : make_uint4(0, 0, 0, 0);
    const int q_lo = slice_of(a, c0);
    const int nq = slice_of(a, min(c0 + kExpandCols, a.D) - 1) - q_lo + 1;
    const int pitch = nq * r;
    stage_v(a, p0, cnt, r, q_lo, nq, vs);
    __syncthreads();   // v staged
    if (!in_d)
        return;
    const int qq = slice_of(a, cbw) - q_lo;

    f32x4_t acc[4][4];   // [mt][nt]
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
            acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int jc = 0; jc < nj; ++jc) {
        const int jo = jc * 16 + 8 * (g & 1);
        if (jc > 0) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                bop[mt] = jo < rp ? load16(a.B, bslot + col[mt] * rp + jo) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            if (nt >= n_nt)
                break;
            const int u = 16 * nt + m;
            float f[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int j = jo + i;
                const float v = (u < cnt && j < r) ? vs[u * pitch + qq * r + j] : 0.f;
                f[i] = (g < 2) ? v : v - bf16_lo(pack_bf16x2(v, 0.f));
            }
            uint4 vop;
            vop.x = pack_bf16x2(f[0], f[1]);
            vop.y = pack_bf16x2(f[2], f[3]);
            vop.z = pack_bf16x2(f[4], f[5]);
            vop.w = pack_bf16x2(f[6], f[7]);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                acc[mt][nt] = mfma_bf16_16x16x32(bop[mt], vop, acc[mt][nt]);
        }
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        if (nt >= n_nt)
            break;
        if (16 * nt + m < cnt) {
            float f[16];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    f[4 * mt + i] = acc[mt][nt][i];
            merge16<DT_BF16>(a, yi[nt], true, true, y0[nt], y1[nt], scale, f);
        }
    }
}

// One pass of B for the vector path: the 256 columns' ranks [4 quad .. 4 quad + 3]
// of pass base j0 (bf16: rank pairs 2 (pc + 4 quad) .., fp32: ranks j0 + 4 quad ..),
// as 16-byte words; thread c owns column c0 + c.
template <int DT>
__device__ __forceinline__ uint4 b_word(const ApplyArgs &a, int64_t bslot, int64_t gc, int rp,
                                        int elem0)
{
    if (gc >= a.D || elem0 >= rp)
        return make_uint4(0, 0, 0, 0);
    if constexpr (DT == DT_BF16)
        return load16(a.B, bslot + gc * rp + elem0);
    else
        return *reinterpret_cast<const uint4 *>(reinterpret_cast<const float *>(a.B) + bslot +
                                                gc * rp + elem0);
}

template <int DT>
__device__ void bgmv_expand_tile(const ApplyArgs &a, const int32_t *rows, int s, int r, float scale,
                                 int p0, int cnt, int64_t c0, float *lds)
{
    // per pass: bf16 16 rank pairs (4 words of 4 pairs per column), fp32 16 ranks
    // (4 words of 4 ranks per column)
    constexpr int kWords = 4;
    constexpr int kPassElems = DT == DT_BF16 ? 2 * kPairChunk : 16;
    float *vs = lds;
    uint32_t *bsh = reinterpret_cast<uint32_t *>(lds + kVecVsFloats);   // [word lane][col]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, m = lane & 15;
    const bool row_ok = m < cnt;
    const int64_t cb = c0 + 64 * wave + 16 * g;
    const bool h0 = row_ok && cb < a.D, h1 = row_ok && cb + 8 < a.D;
    const int64_t yi = (int64_t)rows[min(m, cnt - 1)] * a.ldy + cb;   // rows[0 .. cnt) only
    Vec8<DT> y0, y1;
    if (h0)
        y0.load(a.y, yi);
    if (h1)
        y1.load(a.y, yi + 8);

    const int rp = (r + 7) & ~7;
    const int64_t bslot = (int64_t)s * a.b_slot_stride;
    const int64_t gcol = c0 + threadIdx.x;            // the column this thread stages
    constexpr int kElemsPerWord = DT == DT_BF16 ? 8 : 4;
    // the first pass of B in flight while v is staged
    uint4 w[kWords];
#pragma unroll
    for (int q4 = 0; q4 < kWords; ++q4)
        w[q4] = b_word<DT>(a, bslot, gcol, rp, kElemsPerWord * q4);

    const int q_lo = slice_of(a, c0);
    const int nq = slice_of(a, min(c0 + kExpandCols, a.D) - 1) - q_lo + 1;
    stage_v(a, p0, cnt, r, q_lo, nq, vs);
    const int pitch = nq * r;
    const int cl = 64 * wave + 16 * g;               // lane's first column in the chunk
    int qh[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
        qh[hh] = slice_of(a, min(cb + 8 * hh, a.D - 1)) - q_lo;

    float acc[16];
#pragma unroll
    for (int c = 0; c < 16; ++c)
        acc[c] = 0.f;

    for (int j0 = 0; j0 < rp; j0 += kPassElems) {
        if (j0 > 0) {
#pragma unroll
            for (int q4 = 0; q4 < kWords; ++q4)
                w[q4] = b_word<DT>(a, bslot, gcol, rp, j0 + kElemsPerWord * q4);
        }
#pragma unroll
        for (int q4 = 0; q4 < kWords; ++q4) {
            bsh[(4 * q4 + 0) * kExpandCols + threadIdx.x] = w[q4].x;
            bsh[(4 * q4 + 1) * kExpandCols + threadIdx.x] = w[q4].y;
            bsh[(4 * q4 + 2) * kExpandCols + threadIdx.x] = w[q4].z;
            bsh[(4 * q4 + 3) * kExpandCols + threadIdx.x] = w[q4].w;
        }
        __syncthreads();   // v and this pass of B staged
        if constexpr (DT == DT_BF16) {
            const int np = min(kPairChunk, (rp - j0) / 2);
            for (int pp = 0; pp < np; ++pp) {
                const int j = j0 + 2 * pp;
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const float *vr = vs + m * pitch + qh[hh] * r;
                    const float v0 = (row_ok && j < r) ? vr[j] : 0.f;
                    const float v1 = (row_ok && j + 1 < r) ? vr[j + 1] : 0.f;
                    uint32_t hi, lo;
                    split_pair(v0, v1, hi, lo);
                    const uint4 b0 = *reinterpret_cast<const uint4 *>(&bsh[pp * kExpandCols + cl + 8 * hh]);
                    const uint4 b1 = *reinterpret_cast<const uint4 *>(&bsh[pp * kExpandCols + cl + 8 * hh + 4]);
                    const uint32_t bw[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
                    for (int c = 0; c < 8; ++c) {
                        const float t = dot2_bf16(bw[c], hi, acc[8 * hh + c]);
                        acc[8 * hh + c] = dot2_bf16(bw[c], lo, t);
                    }
                }
            }
        } else {
            const float *bf = reinterpret_cast<const float *>(bsh);   // [jj][col]
            for (int jj = 0; jj < 16 && j0 + jj < r; ++jj) {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const float vj = row_ok ? vs[m * pitch + qh[hh] * r + j0 + jj] : 0.f;
#pragma unroll
                    for (int c = 0; c < 8; ++c)
                        acc[8 * hh + c] = fmaf(bf[jj * kExpandCols + cl + 8 * hh + c], vj,
                                               acc[8 * hh + c]);
                }
            }
        }
        __syncthreads();   // bsh is restaged by the next pass
    }
    merge16<DT>(a, yi, h0, h1, y0, y1, scale, acc);
}

template <int DT>
__global__ __launch_bounds__(256) void expand_kernel(ApplyArgs a)
{
    __shared__ __attribute__((aligned(16))) float lds[kLdsFloats];
    __shared__ int32_t rows[kSgmvTileRows];
    __shared__ int32_t srank[LORA_MAX_SLOTS];
    __shared__ float sscale[LORA_MAX_SLOTS];
    const int t = blockIdx.y;
    const ShrinkTile *T = a.tiles + t;
    // header, row indices, counts and the slot table in one round trip
    const int4 h = *reinterpret_cast<const int4 *>(T);
    const int32_t my_row = threadIdx.x < kSgmvTileRows ? T->rows[threadIdx.x] : 0;
    const int n_tiles = a.counts[kCntSgmv] + a.counts[kCntBgmv];
    for (int e = threadIdx.x; e < a.n_slots; e += blockDim.x) {
        srank[e] = a.rank[e];
        sscale[e] = a.scale[e];
    }
    if (t >= n_tiles)
        return;
    const int64_t c0 = (int64_t)blockIdx.x * kExpandCols;
    if (c0 >= a.D)
        return;
    const int s = h.x, p0 = h.y, cnt = h.z;
    if (threadIdx.x < kSgmvTileRows)
        rows[threadIdx.x] = my_row;
    __syncthreads();
    const int r = srank[s];
    const float scale = sscale[s];
    if (r == 0)
        return;   // slot emptied since the grouping was built: rows stay untouched
    if constexpr (DT == DT_BF16) {
        if (h.w == kTileSgmv && a.mfma_ok) {
            sgmv_expand_tile(a, rows, s, r, scale, p0, cnt, c0, lds);
            return;
        }
    }
    // BGMV tile, or a dense tile of a stack without the MFMA path
    for (int sub = 0; sub < cnt; sub += kBgmvTileRows) {
        bgmv_expand_tile<DT>(a, rows + sub, s, r, scale, p0 + sub, min(kBgmvTileRows, cnt - sub),
                             c0, lds);
        __syncthreads();   // LDS is restaged by the next sub-tile
    }
}

}  // namespace

hipError_t launch_expand(int dtype, const ApplyArgs &a, int max_tiles, hipStream_t stream)
{
    if (max_tiles <= 0)
        return hipSuccess;
    const dim3 grid((unsigned)((a.D + kExpandCols - 1) / kExpandCols), max_tiles);
    if (dtype == DT_BF16)
        hipLaunchKernelGGL(expand_kernel<DT_BF16>, grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(expand_kernel<DT_F32>, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace lora
