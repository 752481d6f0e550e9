// shrink.hip -- add_shrink: v = A_s x_i for every valid row, every slice.
//
// Page "Multi-LoRA Serving: one base, many adapters", section 2 flowchart and
// section 3.4: add_shrink computes the rank-r product v = A x grouped per
// adapter; section 3.1: A is r x k.  v stays fp32 (it is never rounded to the
// storage type).
//
// Grid: (k-splits, tile bound).  A workgroup reads its tile record (slot, first
// grouping position, row count, path and the row indices) in one load, so the
// only dependent round trip before the x and A loads is that record.  Blocks
// with the same k-split sit on the same XCD when the split count is a multiple
// of 8 (they read the same slice of A).
//
//   BGMV tile (<= 16 rows of one slot): each wavefront owns up to 4 rows and
//     walks them two at a time; each lane reads 8 consecutive k of A and x per
//     step (16-byte loads), accumulates 16 rank partials per row with packed
//     bf16 dot products, and a wavefront reduce-scatter folds the 64 lanes.
//   SGMV tile (<= 64 rows, bf16, MFMA): M = rows (4 M-tiles of 16), N = ranks
//     (one N-tile per slice and 16-rank chunk), K = k; the four wavefronts
//     split the workgroup's k-range so no operand is loaded twice, and their
//     partial tiles are summed in LDS in wavefront order.
//
// Each k-split writes its fp32 partial of v, indexed by split and grouping
// position; the expand sums the splits in split order, so results are
// bit-reproducible.  In the shrink kernels no workgroup waits on another.
//
// The file also holds the launches that put the shrink next to other work:
// build_shrink_kernel (grouping in LDS + shrink), and the two one-launch
// kernels, build_apply_kernel (grouping + shrink + expand) and apply_kernel
// (shrink + expand of a grouped batch), whose expand workgroups wait for the
// shrink workgroups of their tile through per-tile flags (TileSync).
#include "device_common.h"
#include "expand_tiles.h"
#include "group.h"
#include "internal.h"
#include "mfma.h"

namespace lora {

namespace {

constexpr int kNT = 4;    // N-tiles (slice, 16-rank chunk) accumulated at once (SGMV)

// Destination of one split's v for grouping position pos.
__device__ __forceinline__ float *v_out(const ApplyArgs &a, int ks, int pos)
{
    const int SR = a.n_slices * a.r_max;
    return a.vpart + ((int64_t)ks * a.max_rows + pos) * SR;
}

// One element of v: a plain store, or a device-coherent one (relaxed agent
// scope: written through to where every XCD reads it) for a reader in the same
// launch.  Every path stores a partial with its lowest fraction bit cleared
// (the one-launch decode carries its hand-over tag in that bit), so all paths
// sum the same values.
template <bool COH>
__device__ __forceinline__ void put_v(float *p, float x)
{
    x = v_word(x);
    if constexpr (COH)
        __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        *p = x;
}

// Vector (BGMV) shrink of a tile of up to 16 rows, fp32 stacks: wavefront w
// owns rows w, w + 4, w + 8, w + 12, two at a time.
template <int DT, bool COH>
__device__ void bgmv_shrink_tile_pairs(const ApplyArgs &a, const int32_t *rows, int s, int r, int p0,
                                       int cnt, int ks)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t g8 = a.k >> 3;                       // 8-element groups along k
    const int64_t gb = split_begin(g8, ks, a.ks), ge = split_begin(g8, ks + 1, a.ks);

    for (int pair = 0; pair < 2; ++pair) {
        const int u0 = wave + 8 * pair, u1 = u0 + 4;
        if (u0 >= cnt)
            break;
        const bool has1 = u1 < cnt;
        const int64_t x0 = (int64_t)rows[u0] * a.ldx;
        const int64_t x1 = (int64_t)rows[has1 ? u1 : u0] * a.ldx;
        for (int q = 0; q < a.n_slices; ++q) {
            for (int j0 = 0; j0 < r; j0 += 16) {
                const int64_t abase =
                    ((int64_t)s * a.n_slices + q) * a.r_max * a.k + (int64_t)j0 * a.k;
                float acc0[16], acc1[16];
#pragma unroll
                for (int jj = 0; jj < 16; ++jj)
                    acc0[jj] = acc1[jj] = 0.f;
                // A rows j0 .. j0 + 15 of the slot: rows at or past the rank are
                // zero in the pool (load_slot zero-fills), so they are read
                // without a branch and add nothing; rows past r_max repeat the
                // last row (their results are never stored).  Row bases are
                // uniform, so only the lane's k offset lives in a vector register.
#pragma nounroll
                for (int64_t g = gb + lane; g < ge; g += 64) {
                    Vec8<DT> xa, xb;
                    xa.load(a.x, x0 + g * 8);
                    if (has1)
                        xb.load(a.x, x1 + g * 8);
                    else
                        xb.zero();
#pragma unroll
                    for (int jj = 0; jj < 16; ++jj) {
                        const int64_t arow = abase + (int64_t)min(jj, a.r_max - 1 - j0) * a.k;
                        Vec8<DT> av;
                        av.load(a.A, arow + g * 8);
                        acc0[jj] = av.dot(xa, acc0[jj]);
                        acc1[jj] = av.dot(xb, acc1[jj]);
                    }
                }
                const int j = (lane >> 2) & 15;
                const float t0 = wave_reduce_scatter16(acc0);
                if ((lane & 3) == 0 && j0 + j < r)
                    put_v<COH>(v_out(a, ks, p0 + u0) + q * a.r_max + j0 + j, t0);
                if (has1) {
                    const float t1 = wave_reduce_scatter16(acc1);
                    if ((lane & 3) == 0 && j0 + j < r)
                        put_v<COH>(v_out(a, ks, p0 + u1) + q * a.r_max + j0 + j, t1);
                }
            }
        }
    }
}

// Vector (BGMV) shrink of a tile of up to 16 rows, bf16 stacks: wavefront w
// owns rows w, w + 4, w + 8, w + 12, all four in one pass over k, so each A
// granule is loaded once per wavefront (measured: decode on vector tiles
// 17.4 -> 15.7 us per step against the pairs above); fp32 tiles keep the pairs
// (four rows would hold 16 fp32 A granules and 64 sums live).
template <bool COH>
__device__ void bgmv_shrink_tile_quads(const ApplyArgs &a, const int32_t *rows, int s, int r, int p0,
                                       int cnt, int ks)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t g8 = a.k >> 3;                       // 8-element groups along k
    const int64_t gb = split_begin(g8, ks, a.ks), ge = split_begin(g8, ks + 1, a.ks);
    constexpr int kR = kBgmvTileRows / 4;              // rows per wavefront
    if (wave >= cnt)
        return;   // (uniform per wavefront; nothing below synchronises)
    int64_t xr[kR];
    bool has[kR];
#pragma unroll
    for (int i = 0; i < kR; ++i) {
        const int u = wave + 4 * i;
        has[i] = u < cnt;
        xr[i] = (int64_t)rows[has[i] ? u : wave] * a.ldx;   // absent rows: a present row, dropped
    }
    for (int q = 0; q < a.n_slices; ++q) {
        for (int j0 = 0; j0 < r; j0 += 16) {
            const int64_t abase =
                ((int64_t)s * a.n_slices + q) * a.r_max * a.k + (int64_t)j0 * a.k;
            float acc[kR][16];
#pragma unroll
            for (int i = 0; i < kR; ++i)
#pragma unroll
                for (int jj = 0; jj < 16; ++jj)
                    acc[i][jj] = 0.f;
            // A rows j0 .. j0 + 15 of the slot: rows at or past the rank are
            // zero in the pool (load_slot zero-fills), so they are read
            // without a branch and add nothing; rows past r_max repeat the
            // last row (their results are never stored).  Row bases are
            // uniform, so only the lane's k offset lives in a vector register.
#pragma nounroll
            for (int64_t g = gb + lane; g < ge; g += 64) {
                Vec8<DT_BF16> xv[kR];
#pragma unroll
                for (int i = 0; i < kR; ++i)
                    xv[i].load(a.x, xr[i] + g * 8);
#pragma unroll
                for (int jj = 0; jj < 16; ++jj) {
                    const int64_t arow = abase + (int64_t)min(jj, a.r_max - 1 - j0) * a.k;
                    Vec8<DT_BF16> av;
                    av.load(a.A, arow + g * 8);
#pragma unroll
                    for (int i = 0; i < kR; ++i)
                        acc[i][jj] = av.dot(xv[i], acc[i][jj]);
                }
            }
            const int j = (lane >> 2) & 15;
#pragma unroll
            for (int i = 0; i < kR; ++i) {
                if (!has[i])
                    continue;   // (uniform)
                const float t = wave_reduce_scatter16(acc[i]);
                if ((lane & 3) == 0 && j0 + j < r)
                    put_v<COH>(v_out(a, ks, p0 + wave + 4 * i) + q * a.r_max + j0 + j, t);
            }
        }
    }
}

template <int DT, bool COH>
__device__ __forceinline__ void bgmv_shrink_tile(const ApplyArgs &a, const int32_t *rows, int s, int r,
                                                 int p0, int cnt, int ks)
{
    if constexpr (DT == DT_BF16)
        bgmv_shrink_tile_quads<COH>(a, rows, s, r, p0, cnt, ks);
    else
        bgmv_shrink_tile_pairs<DT, COH>(a, rows, s, r, p0, cnt, ks);
}

// 16 zero bytes: the source of operand granules that lie outside the data.
__device__ const uint4 g_zero_granule = {0u, 0u, 0u, 0u};

// Products of one 16-row operand set with NTV N-tiles (slice, 16-rank chunk)
// t0 .. t0 + NTV - 1 of slot s over the k units [wb, we): acc[tt] receives
// the 16 x 16 tile of N-tile t0 + tt (lane (g, m): rows 4 g + i, rank row m).
// xrow is the element offset of this lane's x row (lane m: row m of the set).
// kSt 8-element k groups per lane per step (4 for one N-tile, 2 for kNT: the
// two register buffers, loads of step i + 1 in flight during the MFMAs of step
// i, then fit without spilling).  Every load reads an in-bounds address and
// no branch surrounds a load.  (Measured: branches around the loads, or a
// select of "load or zero" on a runtime tile count, made the compiler drain
// the loads in flight at every step.)
template <int NTV>
__device__ __forceinline__ void shrink_stream(const ApplyArgs &a, int64_t xrow, int s, int r, int nj,
                                              int NT, int t0, int64_t wb, int64_t we,
                                              f32x4_t (&acc)[NTV])
{
    constexpr int kSt = NTV == 1 ? 4 : 2;   // register buffers: 2 x kSt x (1 + NTV) granules
    const int lane = threadIdx.x & 63;
    const int m = lane & 15, g = lane >> 4;
    // A comes from the pool's operand image: the N-tile's block of 16 rank
    // rows, lane (g, m) of unit u at element 128 u + 8 m of the block, so
    // each load instruction reads one contiguous kilobyte (less the rows
    // past r).  Rank rows past r and N-tiles past the last read the zero
    // granule instead (the image holds zeros there too, but reading them
    // would cost bandwidth).
    const int njm = (a.r_max + kImgRows - 1) / kImgRows;
    int64_t arow[NTV];
    bool aok[NTV];
#pragma unroll
    for (int tt = 0; tt < NTV; ++tt) {
        const int t = min(t0 + tt, NT - 1);   // N-tiles past the last repeat it
        const int q = t / nj, jc = t - q * nj;
        aok[tt] = t0 + tt < NT && jc * kImgRows + m < r;
        arow[tt] = ((((int64_t)s * a.n_slices + q) * njm + jc) * kImgRows) * a.k + m * 8;
    }
#pragma unroll
    for (int tt = 0; tt < NTV; ++tt)
        acc[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Granules past the k-range (and of dropped N-tiles) are read from a zero
    // granule: the choice is made on the address, so no select waits on a
    // loaded value and the next step's loads stay in flight while this step's
    // products run.  (The address passes through an empty asm statement,
    // opaque to the optimizer, which would otherwise turn the choice of
    // address back into a branch around the load or a select of two loaded
    // values.)
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    typedef const __attribute__((address_space(1))) u32x4 *G16;   // global: no flat loads
    const uint64_t X = (uint64_t)a.x, Ap = (uint64_t)a.A_img, Z = (uint64_t)&g_zero_granule;
    auto gload = [](uint64_t addr) {
        asm("" : "+v"(addr));
        const u32x4 v = *(G16)addr;
        return make_uint4(v.x, v.y, v.z, v.w);
    };
    auto load_step = [&](int64_t u0, uint4 (&xs)[kSt], uint4 (&as)[NTV][kSt]) {
#pragma unroll
        for (int st = 0; st < kSt; ++st) {
            const int64_t unit = u0 + 4 * st + g;   // lanes g = 0..3: 64 contiguous bytes of a row
            const bool ok = unit < we;
            xs[st] = gload(ok ? X + 2 * (xrow + unit * 8) : Z);
#pragma unroll
            for (int tt = 0; tt < NTV; ++tt)
                as[tt][st] = gload(ok && aok[tt] ? Ap + 2 * (arow[tt] + unit * 128) : Z);
        }
    };
    auto mma_step = [&](const uint4 (&xs)[kSt], const uint4 (&as)[NTV][kSt]) {
#pragma unroll
        for (int st = 0; st < kSt; ++st)
#pragma unroll
            for (int tt = 0; tt < NTV; ++tt)
                acc[tt] = mfma_bf16_16x16x32(xs[st], as[tt][st], acc[tt]);
    };
    // Two register buffers, one step of loads in flight behind the products.
    // No load sits under a condition inside the loop: where a load may or may
    // not have been issued, the wait before a product has to assume it was
    // not, and then waits for the loads in flight too.  The last one or two
    // steps are peeled off instead.
    const int64_t n_steps = (we - wb + 4 * kSt - 1) / (4 * kSt);
    constexpr int kStep = 4 * kSt;   // 8-element units per step
    uint4 xa[kSt], aa[NTV][kSt], xb[kSt], ab[NTV][kSt];
    if (n_steps > 0) {
        load_step(wb, xa, aa);
        int64_t i = 0;
        for (; i + 2 < n_steps; i += 2) {
            load_step(wb + (i + 1) * kStep, xb, ab);
            mma_step(xa, aa);
            load_step(wb + (i + 2) * kStep, xa, aa);
            mma_step(xb, ab);
        }
        if (i + 1 < n_steps) {
            load_step(wb + (i + 1) * kStep, xb, ab);
            mma_step(xa, aa);
            mma_step(xb, ab);
        } else {
            mma_step(xa, aa);
        }
    }
}

// 16-row SGMV tile (batches up to 4096 rows): M = the tile's rows, N = up to
// kNT N-tiles (slice, 16-rank chunk) per pass over the k-range, K = k; the
// four wavefronts split the workgroup's k-range and their partial tiles are
// summed in LDS in wavefront order.  A pass handles NTV N-tiles, a template
// parameter: 1 when the whole rank is one N-tile (rank <= 16, one slice: the
// common decode shape loads nothing it drops), else kNT.
template <bool COH>
__device__ void sgmv_shrink_tile(const ApplyArgs &a, const int32_t *rows, int s, int r, int p0,
                                 int cnt, int ks)
{
    __shared__ f32x4_t red[4][kNT * 64];   // [wave][tt * 64 + lane]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = lane & 15;
    const int64_t xrow = (int64_t)rows[min(m, cnt - 1)] * a.ldx;   // clamp: dropped later
    const int nj = (r + 15) >> 4;
    const int NT = a.n_slices * nj;
    const int64_t g8 = a.k >> 3;
    const int64_t gb = split_begin(g8, ks, a.ks), ge = split_begin(g8, ks + 1, a.ks);
    const int64_t wb = gb + (ge - gb) * wave / 4, we = gb + (ge - gb) * (wave + 1) / 4;

    auto pass = [&](int t0, auto ntv_tag) {
        constexpr int NTV = decltype(ntv_tag)::value;
        f32x4_t acc[NTV];
        shrink_stream<NTV>(a, xrow, s, r, nj, NT, t0, wb, we, acc);
        // fixed-order sum of the four k-quarters
#pragma unroll
        for (int tt = 0; tt < NTV; ++tt)
            red[wave][tt * 64 + lane] = acc[tt];
        __syncthreads();
        {
            const int e = threadIdx.x;            // kNT * 64 == 256 entries
            const int ln = e & 63, tt = e >> 6;
            if (tt < NTV && t0 + tt < NT) {
                const f32x4_t v = ((red[0][e] + red[1][e]) + red[2][e]) + red[3][e];
                const int t = t0 + tt;
                const int q = t / nj, jc = t - q * nj;
                const int j = jc * 16 + (ln & 15);
                if (j < r) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int u = 4 * (ln >> 4) + i;
                        if (u < cnt)
                            put_v<COH>(v_out(a, ks, p0 + u) + q * a.r_max + j, v[i]);
                    }
                }
            }
        }
        __syncthreads();
    };
    for (int t0 = 0; t0 < NT; t0 += kNT) {
        // (uniform) one N-tile (rank <= 16, one slice: the common decode
        // shape) or a full pass; a partial last pass loads its empty N-tiles
        // from the zero granule and drops them
        if (NT - t0 == 1)
            pass(t0, std::integral_constant<int, 1>());
        else
            pass(t0, std::integral_constant<int, kNT>());
    }
}

static_assert(kNT * 64 == 256, "one reduction entry per thread");

// 64-row tiles (batches above 4096 rows).  Each wavefront owns 16 rows of the
// tile over the split's whole k-range, so no cross-wavefront reduction is
// needed.  Blocks of 64 k go global -> LDS directly (global_load_lds, 16 bytes
// per lane, no registers) into a ring of kTallSlots slots, kTallSlots - 1
// blocks ahead of the MFMAs:
//   x: each wavefront copies its 16 rows, instruction i covering rows
//      8 i .. 8 i + 7 with 8 lanes (128 contiguous bytes) per row;
//   A: the workgroup copies the NTV N-tiles' 16 rank rows each, two N-tiles
//      per instruction.
// A slot row is 128 bytes (half the banks), so the XOR swizzle that makes the
// operand reads (16 rows x 16 bytes) conflict-free pairs the row's parity with
// the unit XORed by row / 2; the copy writes LDS lane-linearly, so the swizzle
// is applied to the source addresses.  Every slot is a separate __shared__
// object, named directly in each step, so the compiler can tell which copies a
// read depends on; each wavefront waits for its own copies of the block (an
// explicit count: the blocks still in flight behind it), then one LDS barrier
// makes every wavefront's copies visible and frees the slot read one block
// earlier for the next copy.  Units past the split's k-range read a zero
// granule.  NTV (valid N-tiles of a pass) is a template parameter, so only
// those A rows are copied.  The ring is small enough (48 KB) for three
// workgroups per CU, so a prefill's tiles are all resident at once.
constexpr int kTallSlots = 3;
constexpr int kBlkUnits = 8;   // 8-element k units per block


// s_waitcnt immediate: vector-memory count <= n and no LDS access outstanding (the
// reads of a slot are done before a copy may overwrite it); exports not waited on.
#define LORA_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4))

typedef uint4 TallX[4 * 16 * kBlkUnits];     // [wavefront][row][swizzled unit]
typedef uint4 TallA[kNT * 16 * kBlkUnits];   // [N-tile][rank row][swizzled unit]

template <int NTV>
__device__ __forceinline__ void tall_pass(const ApplyArgs &a, const int64_t (&xsrc)[2], int s, int r,
                                          int p0, int cnt, int ks, int t0, int nj, TallX &xs0,
                                          TallX &xs1, TallX &xs2, TallA &as0, TallA &as1,
                                          TallA &as2)
{
    static_assert(kTallSlots == 3, "the ring below names three slots");
    constexpr int NA = (NTV + 1) / 2;             // A copies per wavefront per block
    constexpr int L = 2 + NA;                     // copies per wavefront per block
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int64_t g8 = a.k >> 3;
    const int64_t gb = split_begin(g8, ks, a.ks), ge = split_begin(g8, ks + 1, a.ks);
    const int nb = (int)((ge - gb + kBlkUnits - 1) / kBlkUnits);
    const uint16_t *X = static_cast<const uint16_t *>(a.x);
    const uint16_t *A = static_cast<const uint16_t *>(a.A);
    const uint16_t *Z = reinterpret_cast<const uint16_t *>(&g_zero_granule);
    // copy lanes: row (lane / 8) of 8, column lane % 8
    const int cr = lane >> 3, cc = lane & 7;
    // A source rows of this thread: rank row jm of N-tile 2 p + th (rows past r
    // repeat row r - 1, N-tiles past NTV read zeros: neither is ever stored)
    const int th = threadIdx.x >> 7, jm = (threadIdx.x >> 3) & 15;
    int64_t asrc[NA];
    bool aval[NA];
#pragma unroll
    for (int p = 0; p < NA; ++p) {
        const int t = t0 + 2 * p + th;
        aval[p] = 2 * p + th < NTV;
        const int q = t / nj, jc = t - q * nj;
        const int j = min(16 * jc + jm, r - 1);
        asrc[p] = aval[p] ? (((int64_t)s * a.n_slices + q) * a.r_max + j) * a.k : 0;
    }
    auto copy = [&](int b, uint4 *xslot, uint4 *aslot) {
        const int64_t u0 = gb + (int64_t)b * kBlkUnits;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            // LDS unit 64 i + lane of this wavefront's rows: row 8 i + cr, column cc
            const int row = 8 * i + cr;
            const int64_t unit = u0 + (cc ^ (row >> 1));
            const uint16_t *src = unit < ge ? X + xsrc[i] + unit * 8 : Z;
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void *)src,
                (__attribute__((address_space(3))) void *)(xslot + 16 * kBlkUnits * wave + 64 * i), 16, 0, 0);
        }
#pragma unroll
        for (int p = 0; p < NA; ++p) {
            // LDS unit 256 p + tid: N-tile 2 p + th, rank row jm, column cc
            const int64_t unit = u0 + (cc ^ (jm >> 1));
            const uint16_t *src = (aval[p] && unit < ge) ? A + asrc[p] + unit * 8 : Z;
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void *)src,
                (__attribute__((address_space(3))) void *)(aslot + 256 * p + 64 * wave), 16, 0, 0);
        }
    };
    f32x4_t acc[NTV];
#pragma unroll
    for (int tt = 0; tt < NTV; ++tt)
        acc[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    auto mma = [&](const uint4 *xslot, const uint4 *aslot) {
        const uint4 *xw = xslot + 16 * kBlkUnits * wave;
#pragma unroll
        for (int st = 0; st < kBlkUnits / 4; ++st) {
            const int unit = 4 * st + g;
            const int col = unit ^ (m >> 1);
            const uint4 xop = xw[m * kBlkUnits + col];
#pragma unroll
            for (int tt = 0; tt < NTV; ++tt) {
                const uint4 aop = aslot[(16 * tt + m) * kBlkUnits + col];
                acc[tt] = mfma_bf16_16x16x32(xop, aop, acc[tt]);
            }
        }
    };
    // block b sits in slot b % 3; step: wait for its copies, barrier (also frees
    // the slot of block b - 1), copy block b + 2 into that slot, MFMAs on block b
    auto step = [&](int b, uint4 *cur_x, uint4 *cur_a, uint4 *nxt_x, uint4 *nxt_a) {
        LORA_WAIT_VM(L);           // block b + 1 may still be in flight
        // a bare barrier: a fence here would wait for every copy in flight.
        // The wait above completed this wavefront's copies of block b; every
        // wavefront consumed its reads of block b - 1 before arriving.
        asm volatile("s_barrier" ::: "memory");
        copy(b + 2, nxt_x, nxt_a);   // (past the last block: zeros, never read)
        mma(cur_x, cur_a);
    };
    copy(0, xs0, as0);
    copy(1, xs1, as1);
    const int nt = nb / 3 * 3;      // whole ring turns, then one or two steps
    for (int b = 0; b < nt; b += 3) {
        step(b, xs0, as0, xs2, as2);
        step(b + 1, xs1, as1, xs0, as0);
        step(b + 2, xs2, as2, xs1, as1);
    }
    // blocks nt and nt + 1 are already in slots 0 and 1 (or zeros past the range)
    if (nb - nt >= 1) {
        LORA_WAIT_VM(L);
        asm volatile("s_barrier" ::: "memory");
        mma(xs0, as0);
    }
    if (nb - nt == 2) {
        LORA_WAIT_VM(0);
        asm volatile("s_barrier" ::: "memory");
        mma(xs1, as1);
    }
    // accumulator lane (g, m): rows 16 wave + 4 g + i, rank row m of each N-tile
#pragma unroll
    for (int tt = 0; tt < NTV; ++tt) {
        const int t = t0 + tt;
        const int q = t / nj, jc = t - q * nj;
        const int j = 16 * jc + m;
        if (j < r) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int u = 16 * wave + 4 * g + i;
                if (u < cnt)
                    v_out(a, ks, p0 + u)[q * a.r_max + j] = v_word(acc[tt][i]);
            }
        }
    }
    LORA_WAIT_VM(0);   // the copies past the last block
    __syncthreads();   // the next pass rewrites every slot
}

__device__ void sgmv_shrink_tile_tall(const ApplyArgs &a, const int32_t *rows, int s, int r,
                                      int p0, int cnt, int ks)
{
    // the ring: three slots, each its own object
    __shared__ TallX xs0, xs1, xs2;
    __shared__ TallA as0, as1, as2;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nj = (r + 15) >> 4;
    const int NT = a.n_slices * nj;
    // x rows of this lane's copies: rows 8 i + lane / 8 of the wavefront's 16
    // (rows past the tile repeat its last row: their outputs are never stored)
    int64_t xsrc[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
        xsrc[i] = (int64_t)rows[min(16 * wave + 8 * i + (lane >> 3), cnt - 1)] * a.ldx;
    for (int t0 = 0; t0 < NT; t0 += kNT) {
        switch (min(kNT, NT - t0)) {   // (uniform)
        case 1: tall_pass<1>(a, xsrc, s, r, p0, cnt, ks, t0, nj, xs0, xs1, xs2, as0, as1, as2); break;
        case 2: tall_pass<2>(a, xsrc, s, r, p0, cnt, ks, t0, nj, xs0, xs1, xs2, as0, as1, as2); break;
        case 3: tall_pass<3>(a, xsrc, s, r, p0, cnt, ks, t0, nj, xs0, xs1, xs2, as0, as1, as2); break;
        default: tall_pass<4>(a, xsrc, s, r, p0, cnt, ks, t0, nj, xs0, xs1, xs2, as0, as1, as2); break;
        }
    }
}

// One tile, its rows already in LDS; r is the slot's rank.
// COH: v stored device-coherent (read in the same launch; 16-row tiles only).
template <int DT, int MT, bool COH = false>
__device__ __forceinline__ void shrink_tile(const ApplyArgs &a, const int32_t *rows, int s, int r,
                                            int p0, int cnt, int path, int ks)
{
    static_assert(!(COH && MT == 4), "coherent v stores: 16-row tiles only");
    if constexpr (DT == DT_BF16) {
        if (path == kTileSgmv && a.mfma_ok) {
            if constexpr (MT == 4)
                sgmv_shrink_tile_tall(a, rows, s, r, p0, cnt, ks);
            else
                sgmv_shrink_tile<COH>(a, rows, s, r, p0, cnt, ks);
            return;
        }
    }
    // BGMV tile, or a dense tile of a stack without the MFMA path
    for (int sub = 0; sub < cnt; sub += kBgmvTileRows)
        bgmv_shrink_tile<DT, COH>(a, rows + sub, s, r, p0 + sub, min(kBgmvTileRows, cnt - sub), ks);
}

// Split ks of tile t.  Returns whether the workgroup computed v (false: no
// such tile in this batch, or a slot emptied since the grouping).
template <int DT, int MT, bool COH = false>
__device__ __forceinline__ bool shrink_body(const ApplyArgs &a, int ks, int t)
{
    __shared__ int32_t rows[kSgmvTileRows];
    __shared__ int32_t rank[LORA_MAX_SLOTS];
    const ShrinkTile *T = a.tiles + t;
    // header, row indices, counts and the slot ranks in one round trip
    const int4 h = *reinterpret_cast<const int4 *>(T);
    const int32_t my_row = threadIdx.x < kSgmvTileRows ? T->rows[threadIdx.x] : 0;
    const int n_tiles = a.counts[kCntSgmv] + a.counts[kCntBgmv];
#pragma unroll 1
    for (int e = threadIdx.x; e < a.n_slots; e += kApplyThreads)
        rank[e] = a.rank[e];
    if (t >= n_tiles)
        return false;
    if (threadIdx.x < kSgmvTileRows)
        rows[threadIdx.x] = my_row;
    __syncthreads();
    const int r = rank[h.x];
    if (r == 0)
        return false;   // slot emptied since the grouping was built: nothing to compute
    shrink_tile<DT, MT, COH>(a, rows, h.x, r, h.y, h.z, h.w, ks);
    return true;
}

template <int DT>
__global__ __launch_bounds__(256) void shrink_kernel(ApplyArgs a)
{
    shrink_body<DT, 1>(a, blockIdx.x, blockIdx.y);
}

// 64-row tiles, held to three wavefronts per SIMD: the tile's 48 KB ring lets
// three workgroups share a CU, and the register budget is kept to match
// (without the bound, small code changes tipped it to two).
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))
void shrink_kernel_tall(ApplyArgs a)
{
    shrink_body<DT_BF16, 4>(a, blockIdx.x, blockIdx.y);
}

// Grouping and shrink in one launch, for small batches.  Every workgroup
// groups the whole batch in LDS (group.h) -- the ids are a few KB, read from
// L2 by all but the first -- and takes its tile from the plan.  The segments
// object receives exactly what the grouping kernel would write: workgroups of
// split 0 store their tile (header and rows) and its stretch of perm,
// workgroup (0, 0) stores seg_off, active, the counts and the rows without an
// adapter.  Those stores come last, after the products, so no barrier waits
// on them.  The expand reads the tiles from memory as usual.
template <int DT>
__global__ __launch_bounds__(256) void build_shrink_kernel(ApplyArgs a, SegBuildArgs sb)
{
    __shared__ GroupLds g;
    __shared__ int wc[2][kGroupPer * kGroupWaves];
    __shared__ int32_t rows[kSgmvTileRows];
    const int ks = blockIdx.x, t = blockIdx.y, tid = threadIdx.x;
    const int N = sb.n_slots;
    const int sg_shift = sb.sgmv_rows == 64 ? 6 : 4;
    int key[kGroupPer], rank[kGroupPer];
    group_hist(sb.ids, (int)sb.n, N, sb.slot_rank, g, key);
    group_scan(g, N, sb.dense_min, sg_shift);
    if (t < g.n_sg + g.n_bg) {
        int s, m;
        locate_tile(g, N, t, s, m);
        const BucketPlan p = bucket_plan(g, s, N, sb.dense_min, sg_shift);
        const int lo = m << p.shift;
        const int cnt = min(1 << p.shift, p.count - lo), p0 = p.first + lo;
        group_rank(key, s, wc[0], rank);
#pragma unroll
        for (int j = 0; j < kGroupPer; ++j) {
            const int u = rank[j] - lo;
            if (rank[j] >= 0 && u >= 0 && u < cnt)
                rows[u] = j * kGroupThreads + tid;
        }
        __syncthreads();
        shrink_tile<DT, 1>(a, rows, s, g.rank[s], p0, cnt, p.path, ks);   // 16-row tiles
        if (ks == 0) {
#pragma unroll
            for (int j = 0; j < kGroupPer; ++j) {
                const int u = rank[j] - lo;
                if (rank[j] >= 0 && u >= 0 && u < cnt) {
                    const int row = j * kGroupThreads + tid;
                    sb.perm[p0 + u] = row;
                    sb.tiles[t].rows[u] = row;
                }
            }
            if (tid == 0)
                *reinterpret_cast<int4 *>(&sb.tiles[t]) = make_int4(s, p0, cnt, p.path);
        }
    }
    if (ks == 0 && t == 0) {
        // rows without an adapter, then seg_off, active and the counts
        group_rank(key, N, wc[1], rank);
#pragma unroll
        for (int j = 0; j < kGroupPer; ++j)
            if (rank[j] >= 0)
                sb.perm[g.seg[N] + rank[j]] = j * kGroupThreads + tid;
        group_store(g, N, sb.seg_off, sb.active, sb.counts);
    }
}

// The handover of one tile's v inside a launch (see build_apply_kernel):
// shrink workgroups publish(), expand workgroups wait() before reading v,
// v_read() once every thread's v is in LDS, and finish() at the end.
struct TileSync {
    int32_t *flag;   // the tile's split flags, then its expand workgroups' counter
    int32_t *timeouts;
    int *gave_up;    // LDS: set when a wavefront's wait gave up (zeroed at kernel start)
    int n_split, n_chunks;
    int wait_limit;  // polls before a wait gives up
    int seen;        // thread 0 of an expand workgroup: the counter before its add

    __device__ TileSync(const ApplyArgs &a, int t, int n_chunks_, int *gave_up_)
        : flag(a.sync + kSyncFlags + t * kSyncTileInts), timeouts(a.sync + kSyncTimeouts),
          gave_up(gave_up_), n_split(a.ks), n_chunks(n_chunks_), wait_limit(a.wait_limit), seen(-1)
    {
    }
    // shrink workgroup of split ks: its device-coherent v stores are issued
    __device__ void publish(int ks) const
    {
        LORA_WAIT_VM(0);   // this wavefront's v stores are acknowledged
        __syncthreads();   // ... and every other wavefront's
        if (threadIdx.x == 0)
            __hip_atomic_store(flag + ks, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // each wavefront polls the split flags itself (no barrier, so loads
    // already issued stay in flight)
    __device__ void wait() const
    {
        const int lane = threadIdx.x & 63;
        for (int spins = 0;; ++spins) {
            const bool ok = lane >= n_split ||
                            __hip_atomic_load(flag + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 1;
            if (__all(ok))
                break;
            if (spins >= wait_limit) {
                if (lane == 0) {
                    __hip_atomic_fetch_add(timeouts, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    *gave_up = 1;
                }
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        // v is read after this point, never hoisted above the poll
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
    // every thread's v is in LDS: count this workgroup done with the flags (the
    // atomic's round trip overlaps the products; its result is used in finish).
    // Returns whether y is to be written: not when any wavefront's wait gave up.
    __device__ bool v_read()
    {
        lds_barrier();
        if (threadIdx.x == 0 && seen < 0)
            seen = __hip_atomic_fetch_add(flag + kMaxKSplit, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return *gave_up == 0;
    }
    // the tile's last expand workgroup to count clears the flags and counter
    // (every other one has finished polling and reading v before it counted)
    __device__ void finish() const
    {
        if (threadIdx.x == 0 && seen == n_chunks - 1) {
            for (int k = 0; k < n_split; ++k)
                __hip_atomic_store(flag + k, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(flag + kMaxKSplit, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
};

// Grouping, shrink and expand in one launch (decode-sized batches of 16-row
// tiles).  The grid is one list of workgroups: first ks x tile-bound shrink
// workgroups (split ks % a.ks of tile b / a.ks, so one split's workgroups share
// an XCD when 8 | ks), then chunks x tile-bound expand workgroups (chunk
// c % n_chunks of tile c / n_chunks).  Every workgroup groups the batch in LDS
// as build_shrink_kernel does, so neither side reads anything the other writes
// except v:
//   shrink  computes its split of the tile's v, stores it device-coherent
//           (written through past the XCD's L2), waits until the stores are
//           acknowledged, then sets the tile's flag for its split to 1;
//   expand  puts its y and B loads in flight, then each wavefront polls the
//           tile's split flags (device-coherent loads) until all are 1, reads
//           v device-coherent, counts itself on the tile's counter and
//           finishes the tile; the tile's last expand workgroup to count
//           clears the tile's flags and counter.
// So every launch starts and ends with all flags zero: a launch (or a replay of
// a captured graph) never sees an earlier launch's flags, and no counter is
// shared by the whole grid (one such counter, bumped by every workgroup,
// measured ~7 us per launch).  Each tile's state sits in its own 128 bytes.
// An expand workgroup waits only on shrink workgroups of lower index, which
// are dispatched before it and wait on nothing, so the waits always end; a
// wait that exceeds a.wait_limit polls (by default well under a second) gives up and counts
// a timeout that lora_get_device_status reports.

template <int DT>
__global__ __launch_bounds__(256) void build_apply_kernel(ApplyArgs a, SegBuildArgs sb, int n_prod,
                                                          int n_chunks)
{
    __shared__ GroupLds g;
    __shared__ int wc[2][kGroupPer * kGroupWaves];
    __shared__ int32_t rows[kSgmvTileRows];
    __shared__ int gave_up;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];   // expand staging
    const int tid = threadIdx.x, b = blockIdx.x;
    const bool prod = b < n_prod;
    const int t = prod ? b >> __builtin_ctz((unsigned)a.ks) : (b - n_prod) / n_chunks;   // (a.ks: a power of two)
    const int ks = prod ? b - t * a.ks : 0;
    const int N = sb.n_slots;
    // a wait of an earlier launch gave up: leave y untouched until the host
    // has read the status (which resets the flags)
    const bool poisoned =
        __hip_atomic_load(a.sync + kSyncTimeouts, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
    if (tid == 0)
        gave_up = 0;   // ordered before any use by the grouping's barriers
    int key[kGroupPer], rank[kGroupPer];
    group_hist(sb.ids, (int)sb.n, N, sb.slot_rank, g, key);
    group_scan(g, N, sb.dense_min, 4);
    if (t < g.n_sg + g.n_bg) {
        int s, m;
        locate_tile(g, N, t, s, m);
        const BucketPlan p = bucket_plan(g, s, N, sb.dense_min, 4);
        const int lo = m << p.shift;
        const int cnt = min(1 << p.shift, p.count - lo), p0 = p.first + lo;
        group_rank(key, s, wc[0], rank);
#pragma unroll
        for (int j = 0; j < kGroupPer; ++j) {
            const int u = rank[j] - lo;
            if (rank[j] >= 0 && u >= 0 && u < cnt)
                rows[u] = j * kGroupThreads + tid;
        }
        __syncthreads();
        const int r = g.rank[s];
        TileSync sy(a, t, n_chunks, &gave_up);
        if (prod) {
            if (!poisoned) {
                shrink_tile<DT, 1, true>(a, rows, s, r, p0, cnt, p.path, ks);
                sy.publish(ks);
            }
            if (ks == 0) {
                // the segments object receives what the grouping kernel writes
#pragma unroll
                for (int j = 0; j < kGroupPer; ++j) {
                    const int u = rank[j] - lo;
                    if (rank[j] >= 0 && u >= 0 && u < cnt) {
                        const int row = j * kGroupThreads + tid;
                        sb.perm[p0 + u] = row;
                        sb.tiles[t].rows[u] = row;
                    }
                }
                if (tid == 0)
                    *reinterpret_cast<int4 *>(&sb.tiles[t]) = make_int4(s, p0, cnt, p.path);
            }
        } else if (!poisoned) {
            const int64_t c0 = (int64_t)(b - n_prod - t * n_chunks) * kCols;
            const float scale = a.scale[s];
            auto wait = [&]() { sy.wait(); };
            auto v_read = [&]() { return sy.v_read(); };
            float *vs = reinterpret_cast<float *>(lds + a.lds_v_off);
            unsigned char *bst = lds + a.lds_b_off;
            bool done = false;
            if constexpr (DT == DT_BF16) {
                if (p.path == kTileSgmv && a.mfma_ok) {
                    sgmv_expand_tile<1, false, true>(a, rows, s, r, scale, p0, cnt, c0, vs,
                                                     reinterpret_cast<uint16_t *>(bst), wait, v_read);
                    done = true;
                }
            }
            if (!done) {
                for (int sub = 0; sub < cnt; sub += kBgmvTileRows) {
                    bgmv_expand_tile<DT, true>(a, rows + sub, s, r, scale, p0 + sub,
                                               min(kBgmvTileRows, cnt - sub), c0, vs,
                                               reinterpret_cast<uint32_t *>(bst), wait, v_read);
                    __syncthreads();   // LDS is restaged by the next sub-tile
                }
            }
            sy.finish();
        }
    }
    if (prod && ks == 0 && t == 0) {
        // rows without an adapter, then seg_off, active and the counts
        group_rank(key, N, wc[1], rank);
#pragma unroll
        for (int j = 0; j < kGroupPer; ++j)
            if (rank[j] >= 0)
                sb.perm[g.seg[N] + rank[j]] = j * kGroupThreads + tid;
        group_store(g, N, sb.seg_off, sb.active, sb.counts);
    }
}

// Shrink and expand of a grouped batch in one launch (lora_apply of a
// decode-sized batch): the same grid and hand-over as build_apply_kernel, with
// the tile records read from the segments object instead of a grouping.
template <int DT>
__global__ __launch_bounds__(256) void apply_kernel(ApplyArgs a, int n_prod, int n_chunks)
{
    __shared__ int gave_up;
    const int b = blockIdx.x;
    // a wait of an earlier launch gave up: leave y untouched until the host
    // has read the status (which resets the flags)
    if (__hip_atomic_load(a.sync + kSyncTimeouts, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0)
        return;
    if (threadIdx.x == 0)
        gave_up = 0;   // ordered before any use by the barriers of the tile code
    if (b < n_prod) {
        const int t = b >> __builtin_ctz((unsigned)a.ks), ks = b - t * a.ks;   // (a.ks: a power of two)
        if (shrink_body<DT, 1, true>(a, ks, t)) {
            const TileSync sy(a, t, n_chunks, &gave_up);
            sy.publish(ks);
        }
    } else {
        const int t = (b - n_prod) / n_chunks, chunk = b - n_prod - t * n_chunks;
        TileSync sy(a, t, n_chunks, &gave_up);
        auto wait = [&]() { sy.wait(); };
        auto v_read = [&]() { return sy.v_read(); };
        if (expand_body<DT, 1, false, true>(a, t, chunk, wait, v_read))
            sy.finish();
    }
}

// The kernels take k-split boundaries with split_begin: the split count
// must be a power of two (choose_ks and decode_ks only produce such).
bool ks_ok(int ks) { return ks >= 1 && ks <= kMaxKSplit && (ks & (ks - 1)) == 0; }

}  // namespace

hipError_t launch_apply(int dtype, const ApplyArgs &a, int max_tiles, hipStream_t stream)
{
    if (max_tiles <= 0 || a.sgmv_rows != kBgmvTileRows || a.cpw != 1 || !ks_ok(a.ks) || !a.sync)
        return hipErrorInvalidValue;
    const int n_chunks = (int)((a.D + kCols - 1) / kCols);
    const int n_prod = a.ks * max_tiles;
    const dim3 grid((unsigned)(n_prod + n_chunks * max_tiles));
    if (dtype == DT_BF16)
        hipLaunchKernelGGL(apply_kernel<DT_BF16>, grid, dim3(256), a.lds_bytes, stream, a, n_prod,
                           n_chunks);
    else
        hipLaunchKernelGGL(apply_kernel<DT_F32>, grid, dim3(256), a.lds_bytes, stream, a, n_prod,
                           n_chunks);
    return hipGetLastError();
}

int apply_wgs_per_cu(int dtype, int lds_bytes)
{
    int n = 0;
    const hipError_t e =
        dtype == DT_BF16
            ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, apply_kernel<DT_BF16>, 256, lds_bytes)
            : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, apply_kernel<DT_F32>, 256, lds_bytes);
    return e == hipSuccess ? n : 0;
}

hipError_t launch_build_apply(int dtype, const ApplyArgs &a, const SegBuildArgs &sb, int max_tiles,
                              hipStream_t stream)
{
    if (max_tiles <= 0 || sb.n > kGroupRows || sb.sgmv_rows != kBgmvTileRows || a.cpw != 1 ||
        !ks_ok(a.ks) || !a.sync)
        return hipErrorInvalidValue;
    const int n_chunks = (int)((a.D + kCols - 1) / kCols);
    const int n_prod = a.ks * max_tiles;
    const dim3 grid((unsigned)(n_prod + n_chunks * max_tiles));
    if (dtype == DT_BF16)
        hipLaunchKernelGGL(build_apply_kernel<DT_BF16>, grid, dim3(256), a.lds_bytes, stream, a, sb,
                           n_prod, n_chunks);
    else
        hipLaunchKernelGGL(build_apply_kernel<DT_F32>, grid, dim3(256), a.lds_bytes, stream, a, sb,
                           n_prod, n_chunks);
    return hipGetLastError();
}

int build_apply_wgs_per_cu(int dtype, int lds_bytes)
{
    int n = 0;
    const hipError_t e =
        dtype == DT_BF16
            ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, build_apply_kernel<DT_BF16>, 256, lds_bytes)
            : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, build_apply_kernel<DT_F32>, 256, lds_bytes);
    return e == hipSuccess ? n : 0;
}

hipError_t launch_shrink(int dtype, const ApplyArgs &a, int max_tiles, hipStream_t stream)
{
    if (max_tiles <= 0)
        return hipSuccess;
    if (!ks_ok(a.ks))
        return hipErrorInvalidValue;
    const dim3 grid(a.ks, max_tiles);
    const bool tall = a.sgmv_rows > kBgmvTileRows;   // 64-row dense tiles
    if (dtype == DT_BF16) {
        if (tall)
            hipLaunchKernelGGL(shrink_kernel_tall, grid, dim3(256), 0, stream, a);
        else
            hipLaunchKernelGGL(shrink_kernel<DT_BF16>, grid, dim3(256), 0, stream, a);
    } else {
        hipLaunchKernelGGL(shrink_kernel<DT_F32>, grid, dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

hipError_t launch_build_shrink(int dtype, const ApplyArgs &a, const SegBuildArgs &sb, int max_tiles,
                               hipStream_t stream)
{
    if (max_tiles <= 0 || sb.n > kGroupRows || sb.sgmv_rows != kBgmvTileRows || !ks_ok(a.ks))
        return hipErrorInvalidValue;
    const dim3 grid(a.ks, max_tiles);
    if (dtype == DT_BF16)
        hipLaunchKernelGGL(build_shrink_kernel<DT_BF16>, grid, dim3(256), 0, stream, a, sb);
    else
        hipLaunchKernelGGL(build_shrink_kernel<DT_F32>, grid, dim3(256), 0, stream, a, sb);
    return hipGetLastError();
}

}  // namespace lora
