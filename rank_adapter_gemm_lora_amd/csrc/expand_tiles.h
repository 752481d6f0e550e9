// expand_tiles.h -- the expand's tile code (add_expand with the per-row
// merge), shared by the expand kernels and the one-launch decode kernel.
//
// Page "Multi-LoRA Serving: one base, many adapters", section 2 flowchart and
// section 3.4: add_expand computes delta = B v * alpha / r grouped per adapter
// and each row merges y_i = base_i + delta_i; section 3.1: B is d x r.  The sum
// is fp32 and rounded once into the storage type.
//
// Every tile function takes two hooks, no-ops in the expand kernels: `wait`,
// called after the tile's y and B loads are issued and before v is read (in
// the one-launch kernel, the wait for the shrink workgroups that produce the
// tile's v), and `v_read`, called by every thread once its v loads have
// landed in LDS (there, the tile's expand workgroups count themselves done
// with the tile's flags), which returns whether the tile's y is to be written
// (false when the wait gave up).  COH reads v with device-coherent loads (they bypass the XCD's
// non-coherent L2), for v written by a workgroup of the same launch.
#pragma once

#include "device_common.h"
#include "internal.h"
#include "mfma.h"

namespace lora {

namespace {

struct NoWait {
    __device__ __forceinline__ void operator()() const {}
};

// v_read hook of the expand kernels: every tile's y is written.
struct KeepAll {
    __device__ __forceinline__ bool operator()() const { return true; }
};

constexpr int kCols = kExpandCols;
// MFMA expand: a lane's second 8 columns start kHalf columns after its first
constexpr int kHalf = 32;

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

// LDS row pitch (floats) of the staged v: nq slices of rp8 = round_up(r, 8)
// ranks each, plus 4, so the row pitch is an odd number of 16-byte units and
// the 16 rows that one operand read spans start in 16 distinct bank groups.
__device__ __forceinline__ int v_pitch(int nq, int rp8)
{
    return nq * rp8 + 4;
}

// One element of v: a plain load, or a device-coherent one (relaxed agent
// scope: the load bypasses the non-coherent caches) for v written in the same
// launch by a workgroup that may sit on another XCD.
template <bool COH>
__device__ __forceinline__ float load_v(const float *p)
{
    if constexpr (COH)
        return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        return *p;
}

// v of rows [p0, p0 + cnt) for slices [q_lo, q_lo + nq) ->
// vs[u * v_pitch + qq * rp8 + j] (j < r; ranks r .. rp8 are not written), the
// sum of the KS k-split partials in split order.  Each pass puts 8 loads
// per thread in flight (8 / KS elements, every split of each; 16 splits go in
// two batches of 8) before the first add, so a tile's v costs one round trip
// per pass.  Indexes past the tile are clamped to its last element (read, not
// stored).  NT: the workgroup's thread count when fixed at compile time (the
// 64-row tiles measured faster so), else 0 (read at run time).
template <int KS, bool COH, int NT>
__device__ __forceinline__ void stage_v_ks(const ApplyArgs &a, int p0, int cnt, int r, int q_lo,
                                           int nq, float *vs)
{
    constexpr int kL = KS < 8 ? KS : 8;              // splits per batch of loads
    constexpr int kE = 8 / kL;                       // elements per thread per pass
    const int SR = a.n_slices * a.r_max, pitch = nq * r, total = cnt * pitch;
    const int rp8 = (r + 7) & ~7, P = v_pitch(nq, rp8);
    const int64_t split = a.max_rows * (int64_t)SR;
    const uint32_t m_pitch = div_magic(pitch), m_r = div_magic(r);   // cnt * pitch <= 2^14
    for (int base = 0; base < total; base += kE * (NT > 0 ? NT : (int)blockDim.x)) {
        const float *src[kE];
#pragma unroll
        for (int e = 0; e < kE; ++e) {
            const int idx = min(base + e * (NT > 0 ? NT : (int)blockDim.x) + (int)threadIdx.x, total - 1);
            const int u = div_small(idx, m_pitch);
            const int rem = idx - u * pitch;
            const int qq = div_small(rem, m_r);
            const int j = rem - qq * r;
            src[e] = a.vpart + (int64_t)(p0 + u) * SR + (q_lo + qq) * a.r_max + j;
        }
        float sum[kE];
#pragma unroll
        for (int k0 = 0; k0 < KS; k0 += kL) {
            float part[kE][kL];
#pragma unroll
            for (int e = 0; e < kE; ++e)
#pragma unroll
                for (int kk = 0; kk < kL; ++kk)
                    part[e][kk] = load_v<COH>(src[e] + (k0 + kk) * split);
#pragma unroll
            for (int e = 0; e < kE; ++e)
#pragma unroll
                for (int kk = 0; kk < kL; ++kk)
                    sum[e] = (k0 + kk == 0) ? part[e][0] : sum[e] + part[e][kk];
        }
#pragma unroll
        for (int e = 0; e < kE; ++e) {
            const int idx = base + e * (NT > 0 ? NT : (int)blockDim.x) + (int)threadIdx.x;
            if (idx < total) {
                // (the decomposition again: cheaper than holding it across the loads)
                const int u = div_small(idx, m_pitch);
                const int rem = idx - u * pitch;
                const int qq = div_small(rem, m_r);
                vs[u * P + qq * rp8 + (rem - qq * r)] = sum[e];
            }
        }
    }
}

// stage_v_ks for stacks whose r_max is a multiple of 4 (so every 4-rank
// group of a partial row is 16-byte aligned and inside its slice): thread t
// takes 4-rank groups t, t + 256, ... of the tile's rows x slices, loads the
// group of every split at once (one 16-byte load per split) and sums them in
// split order -- the same sums as stage_v_ks, in one round trip for up to 256
// groups (16 rows of rank 64 in one slice).  Ranks r .. round_up(r, 4) of the
// staged rows hold whatever the partials hold there (never used: the operands
// mask ranks past r).
template <int KS>
__device__ __forceinline__ void stage_v4_ks(const ApplyArgs &a, int p0, int cnt, int r, int q_lo,
                                            int nq, float *vs)
{
    const int g4 = (r + 3) >> 2, per_row = nq * g4, total = cnt * per_row;
    const int SR = a.n_slices * a.r_max;
    const int rp8 = (r + 7) & ~7, P = v_pitch(nq, rp8);
    const int64_t split = a.max_rows * (int64_t)SR;   // floats of one split
    const uint32_t m_row = div_magic(per_row), m_g4 = div_magic(g4);   // total <= 2^14
#pragma unroll 1
    for (int idx = threadIdx.x; idx < total; idx += kApplyThreads) {
        const int u = div_small(idx, m_row);
        const int rem = idx - u * per_row;
        const int qq = div_small(rem, m_g4);
        const int k = rem - qq * g4;
        // (a 32-bit offset from a per-split base, so each load takes its base
        // from scalar registers)
        const uint32_t off = (uint32_t)((p0 + u) * SR + (q_lo + qq) * a.r_max + 4 * k);
        // batches of at most 8 splits (16 splits: two round trips), summed in
        // split order
        constexpr int kL = KS < 8 ? KS : 8;
        float4 sum;
#pragma unroll
        for (int k0 = 0; k0 < KS; k0 += kL) {
            float4 part[kL];
#pragma unroll
            for (int kk = 0; kk < kL; ++kk)
                part[kk] = *reinterpret_cast<const float4 *>(a.vpart + (k0 + kk) * split + off);
#pragma unroll
            for (int kk = 0; kk < kL; ++kk) {
                if (k0 + kk == 0) {
                    sum = part[0];
                } else {
                    sum.x += part[kk].x;
                    sum.y += part[kk].y;
                    sum.z += part[kk].z;
                    sum.w += part[kk].w;
                }
            }
        }
        *reinterpret_cast<float4 *>(vs + u * P + qq * rp8 + 4 * k) = sum;
    }
}

// stage_v_ks by 4-rank groups (r_max a multiple of 4), for kernels with the
// registers to hold a group of 8 splits in flight.
__device__ __forceinline__ void stage_v4(const ApplyArgs &a, int p0, int cnt, int r, int q_lo, int nq,
                                         float *vs)
{
    switch (a.ks) {
    case 1: stage_v4_ks<1>(a, p0, cnt, r, q_lo, nq, vs); break;
    case 2: stage_v4_ks<2>(a, p0, cnt, r, q_lo, nq, vs); break;
    case 4: stage_v4_ks<4>(a, p0, cnt, r, q_lo, nq, vs); break;
    case 8: stage_v4_ks<8>(a, p0, cnt, r, q_lo, nq, vs); break;
    default: stage_v4_ks<16>(a, p0, cnt, r, q_lo, nq, vs); break;
    }
}

template <bool COH = false, int NT = 0>
__device__ __forceinline__ void stage_v(const ApplyArgs &a, int p0, int cnt, int r, int q_lo,
                                        int nq, float *vs)
{
    switch (a.ks) {
    case 1: stage_v_ks<1, COH, NT>(a, p0, cnt, r, q_lo, nq, vs); break;
    case 2: stage_v_ks<2, COH, NT>(a, p0, cnt, r, q_lo, nq, vs); break;
    case 4: stage_v_ks<4, COH, NT>(a, p0, cnt, r, q_lo, nq, vs); break;
    case 8: stage_v_ks<8, COH, NT>(a, p0, cnt, r, q_lo, nq, vs); break;
    default: stage_v_ks<16, COH, NT>(a, p0, cnt, r, q_lo, nq, vs); break;
    }
}

// The expand's MFMA operand of v for one lane: 8 ranks of one row, read from
// LDS at vr (16-byte aligned) as two 16-byte reads, as bf16 hi parts (lo_half
// false) or the bf16 parts of the rounding residuals (true).  Ranks at or past
// n_valid (the rank minus the operand's first rank) and every rank of a row
// past the tile give 0: the mask is applied to the packed words, so the reads
// carry no condition (a select on each loaded value had the compiler split
// them into single-float reads, one behind a branch).
__device__ __forceinline__ uint4 v_operand(const float *vr, bool row_ok, int n_valid, bool lo_half)
{
    const float4 va = reinterpret_cast<const float4 *>(vr)[0];
    const float4 vb = reinterpret_cast<const float4 *>(vr)[1];
    const float vv[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
    uint32_t w[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        uint32_t hi, lo;
        split_pair(vv[2 * p], vv[2 * p + 1], hi, lo);
        const uint32_t mask = ((row_ok & (2 * p < n_valid)) ? 0x0000ffffu : 0u) |
                              ((row_ok & (2 * p + 1 < n_valid)) ? 0xffff0000u : 0u);
        w[p] = (lo_half ? lo : hi) & mask;
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// y at yi (8 columns, acc[0..7]) and yi + off1 (8 columns, acc[8..15]) +=
// scale * acc, rounded once.
template <int DT>
__device__ __forceinline__ void merge16(const ApplyArgs &a, int64_t yi, bool h0, bool h1,
                                        const Vec8<DT> &y0, const Vec8<DT> &y1, float scale,
                                        const float (&acc)[16], int off1 = 8)
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
        Vec8<DT>::store(a.y, yi + off1, f);
    }
}

// ---------------------------------------------------------------- SGMV (MFMA)

// MT: row tiles (16 rows each) of the dense tile height this launch serves (1
// for batches up to 4096 rows, 4 above), so the y registers match the shape.
// WO: rank windows in the outer loop (B staged once per window, all MT row
// tiles accumulated at once), for stacks whose B chunk needs several windows.
template <int MT, bool WO, bool COH = false, class Wait = NoWait, class Done = KeepAll>
__device__ void sgmv_expand_tile(const ApplyArgs &a, const int32_t *rows, int s, int r, float scale,
                                 int p0, int cnt, int64_t c0, float *vs, uint16_t *bs,
                                 Wait wait = Wait(), Done v_read = Done())
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, m = lane & 15;
    const int n_nt = (cnt + 15) >> 4;
    // lane's 16 columns: [cb, cb + 8) and [cb + 32, cb + 40), so that each
    // 16-byte load or store of a row covers one contiguous 64-byte half of the
    // wavefront's 128 bytes of that row
    const int64_t cb = c0 + 64 * wave + 8 * g;
    const bool in_d = cb < a.D;                      // whole 64-column blocks (slices % 64 == 0)
    const int rp = (r + 7) & ~7, nj = (r + 15) >> 4;
    // the host places v at a 16-byte boundary, and every operand read below
    // starts at a multiple of 4 floats: 16-byte LDS reads
    vs = static_cast<float *>(__builtin_assume_aligned(vs, 16));

    // y of this lane's rows
    Vec8<DT_BF16> y0[MT], y1[MT];
#pragma unroll
    for (int nt = 0; nt < MT; ++nt) {
        const int u = 16 * nt + m;
        if (nt < n_nt && u < cnt && in_d) {
            const int64_t yi = (int64_t)rows[u] * a.ldy + cb;
            y0[nt].load(a.y, yi);
            y1[nt].load(a.y, yi + kHalf);
        }
    }
    // the B chunk: columns [c0, c0 + 256) of the slot, ranks [w0, w0 + wl) of
    // each column, as LDS [256][wl] (the whole [256][rp] block when the rank
    // fits one window).  16-byte granules go global -> LDS directly, 16 bytes
    // per lane, no register staging; thread t takes granules t, t + 256, ...
    // The first window is in flight with y while v is staged, so B, v and y
    // share one round trip.  Granules of columns past D are not loaded: those
    // columns are whole 64-column blocks (D % 64 == 0 on this path) whose
    // wavefronts never read B.
    const int64_t bchunk = (int64_t)s * a.b_slot_stride + c0 * rp;
    const int ncol = (int)min((int64_t)kCols, a.D - c0);
    const int n_win = (rp + a.b_win - 1) / a.b_win;
    auto stage_b = [&](int w0) {
        const int gpw = min(a.b_win, rp - w0) >> 3;   // granules per column in the window
        const int n_gran = ncol * gpw;
        const uint32_t m_gpw = div_magic(gpw);
        for (int i = 0; i < gpw; ++i) {
            const int e = i * kCols + threadIdx.x;
            if (e < n_gran) {
                // one window: the chunk is contiguous and granule e sits at 8 e
                const int col = div_small(e, m_gpw), gi = e - col * gpw;
                const int64_t off = n_win == 1 ? 8 * (int64_t)e : (int64_t)col * rp + w0 + 8 * gi;
                __builtin_amdgcn_global_load_lds(
                    (const __attribute__((address_space(1))) void *)(
                        reinterpret_cast<const uint16_t *>(a.B) + bchunk + off),
                    (__attribute__((address_space(3))) void *)(bs + 8 * (i * kCols + 64 * wave)), 16, 0,
                    0);
            }
        }
    };
    stage_b(0);
    const int q_lo = slice_of(a, c0);
    const int nq = slice_of(a, min(c0 + kCols, a.D) - 1) - q_lo + 1;
    const int P = v_pitch(nq, rp);
    wait();
    stage_v<COH, (MT == 4 ? kApplyThreads : 0)>(a, p0, cnt, r, q_lo, nq, vs);
    __syncthreads();   // B (first window) and v staged
    const bool keep = v_read();   // false: the wait gave up, y stays untouched
    const int qq = slice_of(a, c0 + 64 * wave) - q_lo;
    // LDS column of M-tile mt for row m, in units of the window's rank pitch
    int bcolumn[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
        bcolumn[mt] = 64 * wave + 32 * (mt >> 1) + 8 * (m >> 2) + 4 * (mt & 1) + (m & 3);

    if constexpr (WO) {
        // windows outer, N-tiles inner: B is staged once per window, every N-tile's
        // accumulators stay live across the windows
        f32x4_t acc[MT][4];
    #pragma unroll
        for (int nt = 0; nt < MT; ++nt)
    #pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                acc[nt][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        for (int w = 0; w < n_win; ++w) {
            const int w0 = w * a.b_win, wl = min(a.b_win, rp - w0);
            if (w > 0) {              // (uniform) restage: every wavefront is done with the last window
                __syncthreads();
                stage_b(w0);
                __syncthreads();
            }
            if (!in_d)
                continue;             // (uniform per wavefront: D is whole 64-column blocks)
    #pragma unroll
            for (int nt = 0; nt < MT; ++nt) {
                if (nt >= n_nt)
                    continue;         // (uniform) fully unrolled: the accumulators stay in registers
                const int u = 16 * nt + m;
                for (int jc = w0 >> 4; jc < min(nj, (w0 + wl + 15) >> 4); ++jc) {
                    const int jo = jc * 16 + 8 * (g & 1);
                    // the four B operands read together from a clamped in-window
                    // address (ranks past the window selected to zero afterwards),
                    // so the reads overlap instead of each waiting behind a branch,
                    // and ahead of v's reads
                    const bool bok = jo < w0 + wl;
                    const int bo = min(jo - w0, wl - 8);
                    uint4 bop[4];
    #pragma unroll
                    for (int mt = 0; mt < 4; ++mt)
                        bop[mt] = *reinterpret_cast<const uint4 *>(bs + bcolumn[mt] * wl + bo);
                    const uint4 vop = v_operand(vs + u * P + qq * rp + jo, u < cnt, r - jo, g >= 2);
    #pragma unroll
                    for (int mt = 0; mt < 4; ++mt)
                        acc[nt][mt] = mfma_bf16_16x16x32(keep_if(bok, bop[mt]), vop, acc[nt][mt]);
                }
            }
        }
        if (in_d && keep) {
    #pragma unroll
            for (int nt = 0; nt < MT; ++nt) {
                const int u = 16 * nt + m;
                if (nt < n_nt && u < cnt) {
                    float f[16];
    #pragma unroll
                    for (int mt = 0; mt < 4; ++mt)
    #pragma unroll
                        for (int i = 0; i < 4; ++i)
                            f[4 * mt + i] = acc[nt][mt][i];
                    merge16<DT_BF16>(a, (int64_t)rows[u] * a.ldy + cb, true, true, y0[nt], y1[nt], scale,
                                     f, kHalf);
                }
            }
        }
    } else {
        // N-tiles outer: one set of accumulators (fewer registers); B is
        // restaged per window and N-tile, so this order serves stacks whose
        // B chunk fits one window
    #pragma unroll
        for (int nt = 0; nt < MT; ++nt) {
            if (nt >= n_nt)
                continue;   // (uniform) fully unrolled: y0[nt] / y1[nt] stay in registers
            const int u = 16 * nt + m;
            f32x4_t acc[4];
    #pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            for (int w = 0; w < n_win; ++w) {
                const int w0 = w * a.b_win, wl = min(a.b_win, rp - w0);
                if (n_win > 1 && (nt > 0 || w > 0)) {   // (uniform) restage this window
                    __syncthreads();                    // every wavefront is done with the last one
                    stage_b(w0);
                    __syncthreads();
                }
                if (!in_d)
                    continue;
                for (int jc = w0 >> 4; jc < min(nj, (w0 + wl + 15) >> 4); ++jc) {
                    const int jo = jc * 16 + 8 * (g & 1);
                    // B operands as in the window-outer order above
                    const bool bok = jo < w0 + wl;
                    const int bo = min(jo - w0, wl - 8);
                    uint4 bop[4];
    #pragma unroll
                    for (int mt = 0; mt < 4; ++mt)
                        bop[mt] = *reinterpret_cast<const uint4 *>(bs + bcolumn[mt] * wl + bo);
                    const uint4 vop = v_operand(vs + u * P + qq * rp + jo, u < cnt, r - jo, g >= 2);
    #pragma unroll
                    for (int mt = 0; mt < 4; ++mt)
                        acc[mt] = mfma_bf16_16x16x32(keep_if(bok, bop[mt]), vop, acc[mt]);
                }
            }
            if (in_d && u < cnt && keep) {
                float f[16];
    #pragma unroll
                for (int mt = 0; mt < 4; ++mt)
    #pragma unroll
                    for (int i = 0; i < 4; ++i)
                        f[4 * mt + i] = acc[mt][i];
                merge16<DT_BF16>(a, (int64_t)rows[u] * a.ldy + cb, true, true, y0[nt], y1[nt], scale,
                                 f, kHalf);
            }
        }
    }
}

// ------------------------------------------------------------ BGMV (vector)

// One 16-byte word of a B pass: ranks [elem0, elem0 + 8) (bf16) or
// [elem0, elem0 + 4) (fp32) of column gc; zero past D or past rp.
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

template <int DT, bool COH = false, class Wait = NoWait, class Done = KeepAll>
__device__ void bgmv_expand_tile(const ApplyArgs &a, const int32_t *rows, int s, int r, float scale,
                                 int p0, int cnt, int64_t c0, float *vs, uint32_t *bsh,
                                 Wait wait = Wait(), Done v_read = Done())
{
    // a pass: 2 words per column = 8 rank pairs (bf16) or 8 ranks (fp32);
    // bsh[word lane w][column] holds rank pair / rank (pass base + w)
    constexpr int kWords = 2;
    constexpr int kElemsPerWord = DT == DT_BF16 ? 8 : 4;
    constexpr int kPassElems = kWords * kElemsPerWord;
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
    // the first pass of B in flight while v is staged
    uint4 w[kWords];
#pragma unroll
    for (int q4 = 0; q4 < kWords; ++q4)
        w[q4] = b_word<DT>(a, bslot, gcol, rp, kElemsPerWord * q4);

    const int q_lo = slice_of(a, c0);
    const int nq = slice_of(a, min(c0 + kCols, a.D) - 1) - q_lo + 1;
    wait();
    stage_v<COH>(a, p0, cnt, r, q_lo, nq, vs);
    const bool keep = v_read();   // false: the wait gave up, y stays untouched
    const int P = v_pitch(nq, rp);
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
#pragma unroll
        for (int q4 = 0; q4 < kWords; ++q4) {
            bsh[(4 * q4 + 0) * kCols + threadIdx.x] = w[q4].x;
            bsh[(4 * q4 + 1) * kCols + threadIdx.x] = w[q4].y;
            bsh[(4 * q4 + 2) * kCols + threadIdx.x] = w[q4].z;
            bsh[(4 * q4 + 3) * kCols + threadIdx.x] = w[q4].w;
        }
        // v and this pass of B staged.  The barriers order LDS only, so the
        // next pass's B, issued before this pass's arithmetic, stays in flight
        // across them.
        lds_barrier();
        if (j0 + kPassElems < rp) {
#pragma unroll
            for (int q4 = 0; q4 < kWords; ++q4)
                w[q4] = b_word<DT>(a, bslot, gcol, rp, j0 + kPassElems + kElemsPerWord * q4);
        }
        if constexpr (DT == DT_BF16) {
            const int np = min(kPassElems, rp - j0) / 2;
            for (int pp = 0; pp < np; ++pp) {
                const int j = j0 + 2 * pp;
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const float *vr = vs + m * P + qh[hh] * rp;
                    const float v0 = (row_ok && j < r) ? vr[j] : 0.f;
                    const float v1 = (row_ok && j + 1 < r) ? vr[j + 1] : 0.f;
                    uint32_t hi, lo;
                    split_pair(v0, v1, hi, lo);
                    const uint4 b0 = *reinterpret_cast<const uint4 *>(&bsh[pp * kCols + cl + 8 * hh]);
                    const uint4 b1 = *reinterpret_cast<const uint4 *>(&bsh[pp * kCols + cl + 8 * hh + 4]);
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
            for (int jj = 0; jj < kPassElems && j0 + jj < r; ++jj) {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const float vj = row_ok ? vs[m * P + qh[hh] * rp + j0 + jj] : 0.f;
#pragma unroll
                    for (int c = 0; c < 8; ++c)
                        acc[8 * hh + c] = fmaf(bf[jj * kCols + cl + 8 * hh + c], vj,
                                               acc[8 * hh + c]);
                }
            }
        }
        lds_barrier();   // bsh is restaged by the next pass
    }
    merge16<DT>(a, yi, h0 && keep, h1 && keep, y0, y1, scale, acc);
}

// Dynamic LDS: [rows: 64 int][slot table: rank, scale (when n_slots <= 256)]
// [v staging at lds_v_off][B staging at lds_b_off]; the host sizes it.
// Tile t, 256-column chunk `chunk`.  Returns whether the workgroup computed
// the tile (false: no such tile in this batch, a chunk past D, or a slot
// emptied since the grouping).  COH, wait and v_read as the tile functions.
template <int DT, int MT, bool WO, bool COH = false, class Wait = NoWait, class Done = KeepAll>
__device__ __forceinline__ bool expand_body(const ApplyArgs &a, int t, int chunk,
                                            Wait wait = Wait(), Done v_read = Done())
{
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    int32_t *rows = reinterpret_cast<int32_t *>(lds);
    int32_t *srank = reinterpret_cast<int32_t *>(lds + kExpandLdsTable);
    float *sscale = reinterpret_cast<float *>(lds + kExpandLdsTable + 4 * kExpandTableSlots);
    float *vs = reinterpret_cast<float *>(lds + a.lds_v_off);
    unsigned char *bst = lds + a.lds_b_off;
    const ShrinkTile *T = a.tiles + t;
    // header, row indices, counts and the slot table in one round trip
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
        return false;
    const int64_t c0 = (int64_t)chunk * kCols;
    if (c0 >= a.D)
        return false;
    const int s = h.x, p0 = h.y, cnt = h.z;
    if (threadIdx.x < kSgmvTileRows)
        rows[threadIdx.x] = my_row;
    __syncthreads();
    const int r = table ? srank[s] : a.rank[s];
    const float scale = table ? sscale[s] : a.scale[s];
    if (r == 0)
        return false;   // slot emptied since the grouping was built: rows stay untouched
    if constexpr (DT == DT_BF16) {
        if (h.w == kTileSgmv && a.mfma_ok) {
            sgmv_expand_tile<MT, WO, COH>(a, rows, s, r, scale, p0, cnt, c0, vs,
                                          reinterpret_cast<uint16_t *>(bst), wait, v_read);
            return true;
        }
    }
    // BGMV tile, or a dense tile of a stack without the MFMA path
    for (int sub = 0; sub < cnt; sub += kBgmvTileRows) {
        bgmv_expand_tile<DT, COH>(a, rows + sub, s, r, scale, p0 + sub, min(kBgmvTileRows, cnt - sub),
                                  c0, vs, reinterpret_cast<uint32_t *>(bst), wait, v_read);
        __syncthreads();   // LDS is restaged by the next sub-tile
    }
    return true;
}

}  // namespace

}  // namespace lora
