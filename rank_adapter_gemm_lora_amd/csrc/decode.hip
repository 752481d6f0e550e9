// decode.hip -- a whole decode-sized batch in one launch: grouping, add_shrink
// and add_expand with the per-row merge.
//
// Page "Multi-LoRA Serving: one base, many adapters", section 2 (per-row
// equation y_i += (alpha/r) B_s A_s x_i; flowchart: group rows by adapter id,
// add_shrink, add_expand, per-row merge), section 3.1 (A is r x k, B is d x r)
// and section 3.2 (one grouped kernel serves the heterogeneous batch); page
// "LoRA hot-loading and adapter routing", batched multi-adapter execution
// (one group of row indices per adapter id, stable order); page "LoRA serving:
// multi-adapter dynamic loading", section 6 (launch shapes that depend on the
// adapter mix break graph replay: the grid here depends on shapes only).
//
// Scope: bf16 stacks of one slice with rank <= 16 whose output width is whole
// 64-column blocks, batches of at most 256 rows (one row per thread) over at
// most 63 slots, and k a multiple of 128 per k-split.  The grid is one list:
//
//   KS x T shrink workgroups (tile t = b / KS, k-split ks = b % KS), then
//   NCG x T expand workgroups (tile t, column group cg of 256 * CPW columns),
//
// with T the tile bound ceil(n / 16) + min(n_slots, n).  Every workgroup
// groups the ids itself (wavefront ballots and DPP scans, two LDS barriers),
// so the only data handed across workgroups is v:
//
//   shrink  x and A of its tile's rows over its k-range on the matrix cores
//           (M = rows, N = ranks, K = k), the four wavefronts' k-quarters
//           summed in LDS in a fixed order, then every (row, rank) partial of
//           the tile -- all 16 rows, whatever the tile's row count -- stored
//           as one 32-bit word (the fp32 value with its lowest fraction bit
//           replaced by a tag bit) with a relaxed device-scope atomic store
//           (written through to where every XCD reads it);
//   expand  y and B of its columns in flight, then each thread polls the KS
//           words of one (row, rank) of v with device-scope atomic loads until
//           every tag bit is the launch's, sums them (tag bits cleared) in
//           split order, and the tile is expanded on the matrix cores (M =
//           columns, N = rows, K = 16 ranks of v's bf16 high part + the same
//           16 of its low part) and merged into y with one rounding.
//
// The words of (tile t, k-split count class c = log2 KS) have fixed addresses
// for the segments object (the tile stride is its allocation bound, not this
// launch's T), written only by launches where tile t is live with KS splits,
// and every such launch rewrites all of them.  The class has an epoch (an int
// per tile and class in the segments object), read by every workgroup of the
// tile at its start; a launch's tag bit is the parity of epoch + 1, and the
// tile's last expand workgroup (found with a per-tile counter) advances the
// epoch.  So when a launch starts, every word of (t, c) carries the parity of
// the epoch it reads, the opposite of what it waits for, and a word is valid
// only once this launch has written it: no flag has to be cleared, and a
// captured graph replays correctly.  Since a word's value and tag travel in
// one atomic access, no fence or store acknowledgement sits between the
// shrink and the expand.  Every path of the library stores v partials with
// that bit cleared, so the paths stay bit-identical.
//
// Before the grouping, shrink workgroups prefetch into L2 the rows and the
// slot weights their k-split will read (the workgroups of one split sit on one
// XCD when KS is a multiple of 8), so the loads issued after the grouping hit
// L2 instead of waiting for HBM.
//
// An expand workgroup waits only on shrink workgroups of lower index, which
// are dispatched before it and wait on nothing, so every wait ends.  As a
// guard the polls are bounded: a workgroup that gives up leaves its rows of y
// untouched and counts a timeout; after that every launch on the segments
// object leaves y untouched (it checks the count at its start) until
// lora_get_device_status reports the timeout and resets the hand-over state.
//
// The allocation-free entry point at the end of this file runs the same
// kernel with its hand-over state in a static device array instead of a
// segments object.
#include <mutex>

#include "device_common.h"
#include "group.h"
#include "internal.h"
#include "mfma.h"

namespace lora {

namespace {

constexpr int kT = 16;   // rows per tile

struct DecLds {
    int cnt[4][kDecodeMaxSlots + 1];   // rows per key in each wavefront (key n_slots: no adapter)
    int nbad[4];
    int rows[kT];                      // the workgroup's tile: row indices
    f32x4_t red[4][64];                // shrink: each wavefront's partial tile
    float vs[kT][kT + 4];              // expand: v of the tile (padded pitch)
    int gave_up;
};

// The grouping of one batch, as every workgroup derives it.
struct DecPlan {
    int key;       // this thread's row: its slot, n_slots (no adapter), -1 (past n)
    int grank;     // rank of the row among the rows of its key, in row order
    int n_tiles;   // tiles of the batch
    int n_valid;   // rows with an adapter
    int n_act;     // slots with rows
    int n_bad;     // ids naming no loaded slot (other than -1)
    int tot_l;     // lane l < n_slots: rows of slot l
    int seg_l;     // lane l < n_slots: first grouping position of slot l
    int apos_l;    // lane l < n_slots: position of slot l in the active list
    int s, m, cnt, p0;   // the workgroup's tile (when t < n_tiles)
};

__device__ __forceinline__ int mbcnt64(uint64_t m)
{
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Group the batch: thread i owns row i.  `id` is ids[i] (or -1 past n) and
// `rk_l` the rank of slot `lane` (any value past n_slots).  Ends with the tile's rows
// in L.rows (for t < n_tiles) and every field of P set.
__device__ __forceinline__ void dec_group(const DecodeArgs &a, int t, int id, int rk_l, DecLds &L,
                                          DecPlan &P)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int N = a.n_slots;
    const bool in = tid < a.n;
    const int rk = __shfl(rk_l, (uint32_t)id < (uint32_t)N ? id : 0);
    const bool valid = in && (uint32_t)id < (uint32_t)N && rk > 0;
    const int key = in ? (valid ? id : N) : -1;
    if (lane <= N)
        L.cnt[wave][lane] = 0;
    if (tid == 0)
        L.gave_up = 0;   // (the expand's flag; ordered before its use by the barriers below)
    // lanes holding this lane's key: one ballot per bit of the 7-bit key code
    // (keys 0 .. 63, 127 past n), each lane keeping the ballot or its
    // complement by its own bit.  Its rank in the wavefront is the count of
    // those below it; the lowest of them stores the count.
    const int code = key >= 0 ? key : 127;
    uint64_t same = ~0ull;
#pragma unroll
    for (int bit = 0; bit < 7; ++bit) {
        const uint64_t bal = __ballot((code >> bit) & 1);
        same &= ((code >> bit) & 1) ? bal : ~bal;
    }
    const int wrank = mbcnt64(same);
    if (key >= 0 && wrank == 0)
        L.cnt[wave][key] = __popcll(same);
    const uint64_t bm = __ballot(in && !valid && id != -1);
    if (lane == 0)
        L.nbad[wave] = __popcll(bm);
    lds_barrier();
    int before = 0;
    if (key >= 0) {
        if (wave > 0) before += L.cnt[0][key];
        if (wave > 1) before += L.cnt[1][key];
        if (wave > 2) before += L.cnt[2][key];
    }
    P.key = key;
    P.grank = before + wrank;
    const bool sl = lane < N;
    const int tot = sl ? L.cnt[0][lane] + L.cnt[1][lane] + L.cnt[2][lane] + L.cnt[3][lane] : 0;
    const int ntl = (tot + kT - 1) >> 4;
    const int act = tot > 0 ? 1 : 0;
    const int inc_t = wave_scan_dpp(ntl), inc_c = wave_scan_dpp(tot), inc_a = wave_scan_dpp(act);
    P.tot_l = tot;
    P.seg_l = inc_c - tot;
    P.apos_l = inc_a - act;
    P.n_tiles = __builtin_amdgcn_readlane(inc_t, 63);
    P.n_valid = __builtin_amdgcn_readlane(inc_c, 63);
    P.n_act = __builtin_amdgcn_readlane(inc_a, 63);
    P.n_bad = L.nbad[0] + L.nbad[1] + L.nbad[2] + L.nbad[3];
    P.s = 0; P.m = 0; P.cnt = 0; P.p0 = 0;
    if (t < P.n_tiles) {
        const int tb = inc_t - ntl;
        const uint64_t hit = __ballot(ntl > 0 && tb <= t && t < tb + ntl);
        const int s = __builtin_ctzll(hit);
        const int m = t - __builtin_amdgcn_readlane(tb, s);
        P.s = s;
        P.m = m;
        P.cnt = min(kT, __builtin_amdgcn_readlane(tot, s) - kT * m);
        P.p0 = __builtin_amdgcn_readlane(P.seg_l, s) + kT * m;
        if (key == s && P.grank >= kT * m && P.grank < kT * m + kT)
            L.rows[P.grank - kT * m] = tid;
    }
    lds_barrier();
}

// Segments object contents, as lora_build_segments writes them: tile t's
// record and its stretch of perm (split-0 shrink workgroups), and from
// workgroup 0 the rows without an adapter, seg_off, active and the counts.
__device__ __forceinline__ void dec_store_segments(const DecodeArgs &a, int t, bool tile_ok,
                                                   bool global, const DecLds &L, const DecPlan &P)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int N = a.n_slots;
    if (tile_ok) {
        if (tid < P.cnt) {
            a.perm[P.p0 + tid] = L.rows[tid];
            a.tiles[t].rows[tid] = L.rows[tid];
        }
        if (tid == 0)
            *reinterpret_cast<int4 *>(&a.tiles[t]) = make_int4(P.s, P.p0, P.cnt, kTileSgmv);
    }
    if (global) {
        if (P.key == N)
            a.perm[P.n_valid + P.grank] = tid;
        if (wave == 0) {
            if (lane < N) {
                a.seg_off[lane] = P.seg_l;
                if (P.tot_l > 0)
                    a.active[P.apos_l] = lane;   // positions [0, n_act)
                if (lane >= P.n_act)
                    a.active[lane] = -1;         // positions [n_act, N): disjoint
            }
            if (lane == N)
                a.seg_off[N] = P.n_valid;
        }
        if (tid == 0) {
            a.counts[kCntValid] = P.n_valid;
            a.counts[kCntActive] = P.n_act;
            a.counts[kCntBad] = P.n_bad;
            a.counts[kCntSgmv] = P.n_tiles;
            a.counts[kCntBgmv] = 0;
        }
    }
}

// A v partial with the launch's tag bit in place of its lowest fraction bit.
__device__ __forceinline__ uint32_t tagged(float v, uint32_t tag)
{
    return (__float_as_uint(v) & ~1u) | tag;
}

// The words of k-split class log2(KS): [ks][tile][16 rows][16 ranks].
template <int KS>
__device__ __forceinline__ uint32_t *class_words(const DecodeArgs &a)
{
    return a.vtag + (int64_t)(KS - 1) * a.vtag_tiles * kT * kT;
}

// Prefetch into L2 (through this XCD) what the k-split's shrink workgroups
// will read: rows [16 t, 16 t + 16) of x and a 1/T share of every slot's A
// over the split's k-range, one 4-byte load per 128-byte line (the L2 line),
// at most one per thread.  In the operand image a slot's k-range is one
// contiguous run of 2 lines per 8-element unit (16 rank rows x 16 bytes; this
// kernel serves r_max <= 16, so each slot is one 16-row block).  Issued after
// every other load of the workgroup's start (vector loads complete in order,
// so waiting for those does not wait for this one) and consumed at the end.
// Threads without a line load the split's first line of x row 0 again.
// Returns the address to load.
template <int KS>
__device__ __forceinline__ const uint32_t *dec_prefetch(const DecodeArgs &a, int t, int ks)
{
    const int tid = threadIdx.x;
    const int64_t g8 = a.k >> 3;
    const int64_t u0 = g8 / KS * ks;            // the split's first 8-element unit
    const int lpr = (int)(g8 / KS) >> 3;        // 128-byte lines per row in the split (>= 2)
    const uint32_t m_lpr = div_magic(lpr);
    const int nx = kT * lpr;
    const int lps = (int)(g8 / KS) * 2;         // image lines of one slot in the split
    const int total = a.n_slots * lps;
    const int per = (total + a.tiles_bound - 1) / a.tiles_bound;
    const uint16_t *X = static_cast<const uint16_t *>(a.x), *A = static_cast<const uint16_t *>(a.A_img);
    const uint16_t *p = X + u0 * 8;
    const int e = tid < nx ? tid : tid - nx;
    if (tid < nx) {
        const int q = div_small(e, m_lpr), rem = e - q * lpr;
        const int row = kT * t + q;
        if (row < a.n)
            p = X + (int64_t)row * a.ldx + (u0 + rem * 8) * 8;
    } else if (e < per && t * per + e < total) {
        const int li = t * per + e, s = li / lps, off = li - s * lps;
        p = A + (int64_t)s * kImgRows * a.k + u0 * 128 + (int64_t)off * 64;
    }
    return reinterpret_cast<const uint32_t *>(p);
}

// Shrink of tile (s, rows) over k-split ks: v partials stored tagged (all 16
// rows; rows past the tile's count repeat its last row).
template <int KS>
__device__ __forceinline__ void dec_shrink(const DecodeArgs &a, int t, int ks, const DecPlan &P,
                                           DecLds &L, uint32_t tag)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int64_t xrow = (int64_t)L.rows[min(m, P.cnt - 1)] * a.ldx;   // rows past cnt: dropped
    // A from the slot's operand image (16 rank rows, zero past the rank):
    // lane (g, m) of unit u at element 128 u + 8 m, one kilobyte per load
    const int64_t arow = (int64_t)P.s * kImgRows * a.k + m * 8;
    const int64_t g8 = a.k >> 3;
    const int64_t wb = g8 / KS * ks + (g8 / KS / 4) * wave;   // this wavefront's k-quarter
    const int steps = (int)(g8 / KS / 16);                    // MFMA steps of 32 k per wavefront
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    constexpr int CH = 4;   // steps per batch of loads
    uint4 xs[CH], as[CH];
    for (int s0 = 0; s0 < steps; s0 += CH) {
#pragma unroll
        for (int st = 0; st < CH; ++st) {
            const int64_t unit = wb + 4 * (s0 + st) + g;
            const bool ok = s0 + st < steps;
            const int64_t cu = ok ? unit : wb + g;   // clamped: in bounds, dropped
            xs[st] = keep_if(ok, load16(a.x, xrow + cu * 8));
            as[st] = keep_if(ok, load16(a.A_img, arow + cu * 128));
        }
#pragma unroll
        for (int st = 0; st < CH; ++st)
            acc = mfma_bf16_16x16x32(xs[st], as[st], acc);
    }
    // accumulator lane (g, m): rows 4 g + i, rank m; fixed-order sum of the quarters
    L.red[wave][lane] = acc;
    lds_barrier();
    const int u = tid >> 4, j = tid & 15;
    const int src = 16 * (u >> 2) + j, i = u & 3;
    const float v = ((L.red[0][src][i] + L.red[1][src][i]) + L.red[2][src][i]) + L.red[3][src][i];
    __hip_atomic_store(class_words<KS>(a) + (((int64_t)ks * a.vtag_tiles + t) * kT + u) * kT + j,
                       tagged(v, tag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Expand of tile (s, rows) over column group cg (CPW quads of 64 columns per
// wavefront).  Once every thread's v is in LDS, thread 0 counts the workgroup
// on the tile's counter at `count` (its previous value into `seen`), so the
// count's round trip overlaps the products and y's merge.  Returns false when
// the wait gave up.
template <int KS, int CPW>
__device__ __forceinline__ bool dec_expand(const DecodeArgs &a, int t, int cg, const DecPlan &P,
                                           DecLds &L, uint32_t tag, float scale, int r, int32_t *count,
                                           int &seen)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int rp = (r + 7) & ~7;
    const int64_t cbase = (int64_t)cg * (256 * CPW) + (int64_t)wave * (64 * CPW);
    const bool row_ok = n < P.cnt;
    const int64_t yrow = (int64_t)L.rows[min(n, P.cnt - 1)] * a.ldy;
    // y: lane (g, n) holds columns qb + 16 g .. + 15 of row n in each quad
    uint4 y0[CPW], y1[CPW];
    uint4 bop[CPW][4];
    const int64_t bslot = (int64_t)P.s * a.b_slot_stride;
    const bool b_ok = 8 * (g & 1) < rp;
    const int b_off = b_ok ? 8 * (g & 1) : 0;
    // every load reads an in-bounds address (quads past D read the last one)
    // and is selected afterwards: no branch around a load
#pragma unroll
    for (int q = 0; q < CPW; ++q) {
        const int64_t qb = cbase + 64 * q;
        const bool in_d = qb < a.D;   // D is whole 64-column blocks
        const int64_t qc = min(qb, a.D - 64);
        const int64_t yi = yrow + qc + 16 * g;
        y0[q] = keep_if(in_d && row_ok, load16(a.y, yi));
        y1[q] = keep_if(in_d && row_ok, load16(a.y, yi + 8));
        // B operand of M-tile mt: row n of the operand is column
        // qb + 16 (n / 4) + 4 mt + n % 4, ranks 8 (g & 1) .. + 7
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int64_t col = qc + 16 * (n >> 2) + 4 * mt + (n & 3);
            bop[q][mt] = keep_if(in_d && b_ok, load16(a.B, bslot + col * rp + b_off));
        }
    }
    // v: thread (u, j) polls the KS words of row u, rank j
    const int u = tid >> 4, j = tid & 15;
    float vsum = 0.f;
    bool gave_up = false;
    if (u < P.cnt) {
        const uint32_t *src = class_words<KS>(a) + ((int64_t)t * kT + u) * kT + j;
        const int64_t stride = (int64_t)a.vtag_tiles * kT * kT;
        auto poll = [&](uint32_t (&w)[KS]) {
#pragma unroll
            for (int k2 = 0; k2 < KS; ++k2)
                w[k2] = __hip_atomic_load(src + k2 * stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        };
        // all KS words carry this launch's tag bit: their sum in split order
        auto ready = [&](const uint32_t (&w)[KS]) {
            bool ok = true;
#pragma unroll
            for (int k2 = 0; k2 < KS; ++k2)
                ok = ok && (w[k2] & 1u) == tag;
            if (ok) {
                float sum = __uint_as_float(w[0] & ~1u);
#pragma unroll
                for (int k2 = 1; k2 < KS; ++k2)
                    sum += __uint_as_float(w[k2] & ~1u);
                vsum = sum;
            }
            return ok;
        };
        // one poll in flight at a time (measured: a second one in flight adds
        // memory traffic that slows the step by 0.7 us)
        for (int spin = 0;; ++spin) {
            uint32_t w[KS];
            poll(w);
            if (ready(w))
                break;
            if (spin >= a.wait_limit) {
                gave_up = true;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    L.vs[u][j] = vsum;
    if (gave_up)
        L.gave_up = 1;
    lds_barrier();
    const bool give_up = L.gave_up != 0;
    // every thread is done with its v words: this workgroup counts itself
    if (tid == 0) {
        if (give_up && a.timeouts)
            __hip_atomic_fetch_add(a.timeouts, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        seen = __hip_atomic_fetch_add(count, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // v operand: row n, K = [16 ranks of hi | the same 16 of lo]; lane group g
    // takes ranks 8 (g & 1) .. + 7 of hi (g < 2) or lo (g >= 2)
    const float4 va = *reinterpret_cast<const float4 *>(&L.vs[n][8 * (g & 1)]);
    const float4 vb = *reinterpret_cast<const float4 *>(&L.vs[n][8 * (g & 1) + 4]);
    const float vv[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
    float f[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float v = row_ok ? vv[i] : 0.f;
        f[i] = g < 2 ? v : v - bf16_lo(pack_bf16x2(v, 0.f));
    }
    uint4 vop;
    vop.x = pack_bf16x2(f[0], f[1]);
    vop.y = pack_bf16x2(f[2], f[3]);
    vop.z = pack_bf16x2(f[4], f[5]);
    vop.w = pack_bf16x2(f[6], f[7]);
#pragma unroll
    for (int q = 0; q < CPW; ++q) {
        const int64_t qb = cbase + 64 * q;
        f32x4_t acc[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
            acc[mt] = mfma_bf16_16x16x32(bop[q][mt], vop, f32x4_t{0.f, 0.f, 0.f, 0.f});
        if (qb < a.D && row_ok && !give_up) {
            // accumulator lane (g, n): columns qb + 16 g + 4 mt + i of row n
            float o[16];
            const uint32_t yw[8] = {y0[q].x, y0[q].y, y0[q].z, y0[q].w, y1[q].x, y1[q].y, y1[q].z, y1[q].w};
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int c = 4 * mt + i;
                    const float yin = (c & 1) ? bf16_hi(yw[c >> 1]) : bf16_lo(yw[c >> 1]);
                    o[c] = fmaf(scale, acc[mt][i], yin);
                }
            uint4 s0, s1;
            s0.x = pack_bf16x2(o[0], o[1]);   s0.y = pack_bf16x2(o[2], o[3]);
            s0.z = pack_bf16x2(o[4], o[5]);   s0.w = pack_bf16x2(o[6], o[7]);
            s1.x = pack_bf16x2(o[8], o[9]);   s1.y = pack_bf16x2(o[10], o[11]);
            s1.z = pack_bf16x2(o[12], o[13]); s1.w = pack_bf16x2(o[14], o[15]);
            uint16_t *yp = static_cast<uint16_t *>(a.y) + yrow + qb + 16 * g;
            *reinterpret_cast<uint4 *>(yp) = s0;
            *reinterpret_cast<uint4 *>(yp + 8) = s1;
        }
    }
    return !give_up;
}

template <int KS, int CPW>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a)
{
    __shared__ DecLds L;
    const int tid = threadIdx.x, lane = tid & 63;
    const int b = blockIdx.x;
    // (KS is the launch's a.ks: divisions by it are shifts, not the long
    // integer division sequence a runtime divisor costs at every workgroup's start)
    const int n_prod = KS * a.tiles_bound;
    const bool prod = b < n_prod;
    const int t = prod ? b / KS : (b - n_prod) / a.ncg;
    const int part = prod ? b - t * KS : b - n_prod - t * a.ncg;   // k-split or column group
    // everything that depends on nothing, in one batch of loads (the prefetch
    // last: it is the one left in flight)
    const int id = a.ids[min(tid, a.n - 1)];   // (rows past n: key -1 below)
    const int rk_l = a.slot_rank[min(lane, a.n_slots - 1)];
    const float sc_l = a.slot_scale[min(lane, a.n_slots - 1)];
    int32_t *st = a.tile_state + t * kSyncTileInts;
    constexpr int kClass = KS == 1 ? 0 : KS == 2 ? 1 : KS == 4 ? 2 : 3;   // log2 KS
    const int epoch = __hip_atomic_load(st + kDecEpoch + kClass, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int poisoned =
        a.poison ? __hip_atomic_load(a.poison, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
    // (every workgroup issues the load, expand workgroups at the ids, so the
    // count of loads in flight is the same on every path)
    const uint32_t pf = *(prod ? dec_prefetch<KS>(a, t, part) : reinterpret_cast<const uint32_t *>(a.ids));
    DecPlan P;
    dec_group(a, t, id, rk_l, L, P);
    const bool tile_ok = t < P.n_tiles;
    const uint32_t tag = ((uint32_t)epoch + 1u) & 1u;
    if (prod) {
        if (tile_ok && poisoned == 0)
            dec_shrink<KS>(a, t, part, P, L, tag);
        if (a.perm)
            dec_store_segments(a, t, tile_ok && part == 0, b == 0, L, P);
    } else if (tile_ok && poisoned == 0) {
        const int r = __shfl(rk_l, P.s);
        const float scale = __shfl(sc_l, P.s);
        int seen = -1;
        dec_expand<KS, CPW>(a, t, part, P, L, tag, scale, r, st + kDecCount, seen);
        // every expand workgroup of the tile counted itself once done with its
        // v: the last to count advances the tile's epoch
        if (tid == 0) {
            if (seen == a.ncg - 1) {
                __hip_atomic_store(st + kDecCount, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(st + kDecEpoch + kClass, epoch + 1, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
    asm volatile("; prefetched word %0" ::"v"(pf));   // keeps the prefetch load, consumed here
}

}  // namespace

template <int KS>
hipError_t launch_decode_ks(const DecodeArgs &a, dim3 grid, hipStream_t stream)
{
    switch (a.cpw) {
    case 1: hipLaunchKernelGGL((decode_kernel<KS, 1>), grid, dim3(256), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((decode_kernel<KS, 2>), grid, dim3(256), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((decode_kernel<KS, 4>), grid, dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream)
{
    if (a.n < 1 || a.n > kDecodeMaxRows || a.n_slots < 1 || a.n_slots > kDecodeMaxSlots || a.r_max > 16 ||
        a.ks < 1 || a.ks > kDecodeMaxKs || (a.ks & (a.ks - 1)) != 0 || (a.k >> 3) % (16 * a.ks) != 0 ||
        a.D % 64 != 0 ||
        a.tiles_bound < 1 || a.tiles_bound > a.vtag_tiles || !a.vtag || !a.tile_state)
        return hipErrorInvalidValue;
    const int n_prod = a.ks * a.tiles_bound;
    const dim3 grid((unsigned)(n_prod + a.ncg * a.tiles_bound));
    switch (a.ks) {
    case 1: return launch_decode_ks<1>(a, grid, stream);
    case 2: return launch_decode_ks<2>(a, grid, stream);
    case 4: return launch_decode_ks<4>(a, grid, stream);
    case 8: return launch_decode_ks<8>(a, grid, stream);
    default: return hipErrorInvalidValue;
    }
}

int decode_wgs_per_cu(int ks, int cpw)
{
    int n = 0;
    hipError_t e = hipErrorInvalidValue;
#define LORA_DEC_OCC(K, C) \
    if (ks == K && cpw == C) \
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_kernel<K, C>, 256, 0);
    LORA_DEC_OCC(1, 1) LORA_DEC_OCC(1, 2) LORA_DEC_OCC(1, 4)
    LORA_DEC_OCC(2, 1) LORA_DEC_OCC(2, 2) LORA_DEC_OCC(2, 4)
    LORA_DEC_OCC(4, 1) LORA_DEC_OCC(4, 2) LORA_DEC_OCC(4, 4)
    LORA_DEC_OCC(8, 1) LORA_DEC_OCC(8, 2) LORA_DEC_OCC(8, 4)
#undef LORA_DEC_OCC
    return e == hipSuccess ? n : 0;
}

}  // namespace lora

// ---------------------------------------------------------------------------
// lora_build_apply_noalloc: the one-launch decode with its hand-over state
// (per-tile epochs and counters, then the tagged v words) in `scratch`, a
// static device array every call on a GPU shares, so the call allocates
// nothing.  The array starts zeroed (static storage) and every launch leaves
// the counters zero; epochs only grow, and a tagged word from an earlier call
// never matches a later call's tag.

namespace lora {

namespace {

constexpr int kNoAllocTiles = kDecodeMaxRows / 16 + kDecodeMaxSlots;   // tile bound of any eligible batch
constexpr size_t kNoAllocStateBytes = (size_t)kNoAllocTiles * kSyncTileInts * sizeof(int32_t);
constexpr size_t kNoAllocStateAligned = (kNoAllocStateBytes + 255) / 256 * 256;
constexpr size_t kNoAllocVtagBytes = (size_t)kDecodeWordsPerTile * kNoAllocTiles * sizeof(uint32_t);
constexpr size_t kNoAllocScratchBytes = kNoAllocStateAligned + kNoAllocVtagBytes;   // 1,223,680 bytes
static_assert(kNoAllocScratchBytes == 1223680, "the size the header states");

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kNoAllocMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kNoAllocMaxDevices];   // device address of `scratch`, per device

// The device address of this device's copy of `scratch` (looked up once per
// device, with that device current).
hipError_t scratch_of(int dev, void **out)
{
    if (dev < 0 || dev >= kNoAllocMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (!ptr)
            return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

}  // namespace lora

extern "C" lora_status lora_build_apply_noalloc(const lora_stack *st, void *y, int64_t ldy, const void *x,
                                                int64_t ldx, const int32_t *ids, int64_t n_rows,
                                                int32_t *timeouts, void *stream)
{
    using namespace lora;
    if (!st || n_rows < 0 || (n_rows > 0 && !ids) || (reinterpret_cast<uintptr_t>(ids) & 3u) != 0 ||
        (reinterpret_cast<uintptr_t>(timeouts) & 3u) != 0 || !device_is_current(st->device))
        return LORA_E_ARG;
    if (n_rows == 0)
        return LORA_OK;
    if (!x_ok(st, x, ldx) || !y_ok(st, y, ldy))
        return LORA_E_ARG;
    if (n_rows > kDecodeMaxRows || !decode_fits(st, n_rows, 1, kNoAllocTiles))
        return LORA_E_UNSUPPORTED;
    void *base = nullptr;
    const lora_status ls = status_of(scratch_of(st->device, &base));
    if (ls != LORA_OK)
        return ls;
    DecodeArgs a = decode_args_for(st, ids, n_rows, x, ldx, y, ldy, 1);
    a.tile_state = static_cast<int32_t *>(base);
    a.vtag = reinterpret_cast<uint32_t *>(static_cast<unsigned char *>(base) + kNoAllocStateAligned);
    a.vtag_tiles = kNoAllocTiles;
    a.timeouts = timeouts;
    a.poison = nullptr;
    return status_of(launch_decode(a, reinterpret_cast<hipStream_t>(stream)));
}
