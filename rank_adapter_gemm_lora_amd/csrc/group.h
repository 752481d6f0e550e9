// group.h -- grouping of a batch of at most kGroupRows rows by adapter slot,
// done by one workgroup entirely in LDS: the bucket histogram, its scan (the
// group offsets and the tile plan) and the rank of each row inside its bucket.
//
// Page "LoRA hot-loading and adapter routing", batched multi-adapter execution
// section: the rows of a batch are processed as one group per adapter id, in a
// stable order.  Bucket n_slots holds the rows without a valid adapter (id -1,
// an id outside [0, n_slots), or a slot that holds no adapter).
//
// Thread t of the workgroup owns rows t, t + 256, t + 512 and t + 768, so each
// id load is one coalesced access and index order is (row block, wavefront,
// lane).  The rank of a row among the rows of one bucket is then a ballot and a
// masked bit count inside the wavefront plus a prefix over 16 (row block,
// wavefront) counts: no sort, no serial loop over rows.
#pragma once

#include "device_common.h"
#include "internal.h"

namespace lora {

constexpr int kGroupThreads = 256;
constexpr int kGroupPer = 4;                              // rows per thread
constexpr int kGroupRows = kGroupThreads * kGroupPer;     // 1024 rows at most
constexpr int kGroupBuckets = LORA_MAX_SLOTS + 1;
constexpr int kGroupWaves = kGroupThreads / 64;
static_assert(kGroupRows == kFusedMaxRows, "the fused launch groups one batch per workgroup");

struct GroupLds {
    int hist[kGroupBuckets];   // rows per bucket
    int seg[kGroupBuckets];    // exclusive scan of hist: group offsets
    int bsg[kGroupBuckets];    // first SGMV tile of each slot
    int bbg[kGroupBuckets];    // first BGMV tile of each slot, not counting the SGMV tiles
    int apos[kGroupBuckets];   // position of each slot in the active list
    int rank[kGroupBuckets];   // slot ranks (0: no adapter)
    int4 tmp[kGroupWaves];
    int n_sg, n_bg, n_act, n_bad;
};

// Where one bucket's rows go: tiles of 2^shift rows starting at tile0.
struct BucketPlan {
    int count, first, tile0, shift, path;
};

__device__ __forceinline__ BucketPlan bucket_plan(const GroupLds &g, int b, int N, int dense_min,
                                                  int sg_shift)
{
    BucketPlan p;
    p.count = g.hist[b];
    p.first = g.seg[b];
    const bool dense = b < N && p.count >= dense_min;
    p.tile0 = dense ? g.bsg[b] : g.n_sg + g.bbg[b];
    p.shift = dense ? sg_shift : 4;
    p.path = dense ? kTileSgmv : kTileBgmv;
    return p;
}

// Keys and histogram.  key[j] = slot of row j * 256 + tid when it holds a valid
// adapter, N when it does not, -1 past the end of the batch.  Counts the bad ids
// into g.n_bad and keeps the slot ranks in g.rank.  Ends with the histogram
// complete in LDS.
__device__ __forceinline__ void group_hist(const int32_t *ids, int n, int N, const int32_t *slot_rank,
                                           GroupLds &g, int (&key)[kGroupPer])
{
    const int tid = threadIdx.x;
    int32_t id[kGroupPer];
#pragma unroll
    for (int j = 0; j < kGroupPer; ++j) {
        const int i = j * kGroupThreads + tid;
        id[j] = i < n ? ids[i] : -1;
    }
    for (int e = tid; e <= N; e += kGroupThreads) {
        g.hist[e] = 0;
        g.rank[e] = e < N ? slot_rank[e] : 0;
    }
    if (tid == 0)
        g.n_bad = 0;
    __syncthreads();
    // all table lookups first, then the atomics
    int look[kGroupPer];
#pragma unroll
    for (int j = 0; j < kGroupPer; ++j)
        look[j] = g.rank[(uint32_t)id[j] < (uint32_t)N ? id[j] : 0];   // clamped: in bounds
    int bad = 0;
#pragma unroll
    for (int j = 0; j < kGroupPer; ++j) {
        const int i = j * kGroupThreads + tid;
        const bool in = i < n;
        const bool valid = (uint32_t)id[j] < (uint32_t)N && look[j] > 0;
        bad += (in && !valid && id[j] != -1) ? 1 : 0;
        key[j] = in ? (valid ? id[j] : N) : -1;
    }
#pragma unroll
    for (int j = 0; j < kGroupPer; ++j)
        if (key[j] >= 0)
            atomicAdd(&g.hist[key[j]], 1);
    if (bad)
        atomicAdd(&g.n_bad, bad);
    __syncthreads();
}

// Inclusive scan over a wavefront with DPP moves: shifts by 1, 2, 4, 8 inside
// each row of 16 lanes, then the row-15 and row-31 broadcasts carry the row
// totals forward.  Lanes whose source falls outside the row read 0.
__device__ __forceinline__ int wave_scan_dpp(int x)
{
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15 -> rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31 -> rows 2, 3
    return x;
}

// Scan of the buckets: group offsets, the SGMV and BGMV tile bases of every
// slot and the positions in the active list, all into LDS, from g.hist.
__device__ __forceinline__ void group_scan(GroupLds &g, int N, int dense_min, int sg_shift)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int NB = N + 1;
    int4 carry = make_int4(0, 0, 0, 0);
    // one pass covers 4 buckets per thread; with few slots wavefront 0 alone
    // scans them and no barrier is needed inside the pass
    const bool one_wave = NB <= 256;
    const int per_pass = one_wave ? 256 : 4 * kGroupThreads;
    for (int e0 = 0; e0 < NB; e0 += per_pass) {
        const bool part = !one_wave || wave == 0;
        int4 v[4];   // (rows, active, SGMV tiles, BGMV tiles) per bucket
        int4 sum = make_int4(0, 0, 0, 0);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e = e0 + 4 * tid + u;
            v[u] = make_int4(0, 0, 0, 0);
            if (part && e < NB) {
                const int c = g.hist[e];
                v[u].x = c;
                if (e < N && c > 0) {
                    const bool dn = c >= dense_min;
                    v[u].y = 1;
                    v[u].z = dn ? (c + (1 << sg_shift) - 1) >> sg_shift : 0;
                    v[u].w = dn ? 0 : (c + kBgmvTileRows - 1) >> 4;
                }
            }
            sum.x += v[u].x; sum.y += v[u].y; sum.z += v[u].z; sum.w += v[u].w;
        }
        const int4 inc = make_int4(wave_scan_dpp(sum.x), wave_scan_dpp(sum.y), wave_scan_dpp(sum.z),
                                   wave_scan_dpp(sum.w));
        int4 base = make_int4(0, 0, 0, 0), tot;
        if (!one_wave) {
            if (lane == 63)
                g.tmp[wave] = inc;
            __syncthreads();
            tot = make_int4(0, 0, 0, 0);
#pragma unroll
            for (int u = 0; u < kGroupWaves; ++u) {
                const int4 t = g.tmp[u];
                if (u < wave) {
                    base.x += t.x; base.y += t.y; base.z += t.z; base.w += t.w;
                }
                tot.x += t.x; tot.y += t.y; tot.z += t.z; tot.w += t.w;
            }
            __syncthreads();
        } else {
            tot = make_int4(__builtin_amdgcn_readlane(inc.x, 63), __builtin_amdgcn_readlane(inc.y, 63),
                            __builtin_amdgcn_readlane(inc.z, 63), __builtin_amdgcn_readlane(inc.w, 63));
        }
        int4 ex = make_int4(carry.x + base.x + inc.x - sum.x, carry.y + base.y + inc.y - sum.y,
                            carry.z + base.z + inc.z - sum.z, carry.w + base.w + inc.w - sum.w);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e = e0 + 4 * tid + u;
            if (part && e < NB) {
                g.seg[e] = ex.x;
                g.apos[e] = ex.y;
                g.bsg[e] = ex.z;
                g.bbg[e] = ex.w;
            }
            ex.x += v[u].x; ex.y += v[u].y; ex.z += v[u].z; ex.w += v[u].w;
        }
        carry.x += tot.x; carry.y += tot.y; carry.z += tot.z; carry.w += tot.w;
    }
    if (tid == 0) {
        g.n_act = carry.y;
        g.n_sg = carry.z;
        g.n_bg = carry.w;
    }
    __syncthreads();
}

// seg_off, active (with its -1 tail) and the counts, from the LDS plan.
__device__ __forceinline__ void group_store(const GroupLds &g, int N, int32_t *seg_off,
                                            int32_t *active, int32_t *counts)
{
    for (int e = threadIdx.x; e <= N; e += kGroupThreads) {
        seg_off[e] = g.seg[e];
        if (e < N && g.hist[e] > 0)
            active[g.apos[e]] = e;
        if (e >= g.n_act && e < N)
            active[e] = -1;
    }
    if (threadIdx.x == 0) {
        counts[kCntValid] = g.seg[N];
        counts[kCntActive] = g.n_act;
        counts[kCntBad] = g.n_bad;
        counts[kCntSgmv] = g.n_sg;
        counts[kCntBgmv] = g.n_bg;
    }
}

// Rank of each of this thread's rows among the rows of bucket b, in index
// order; -1 for rows of other buckets.  `wc` is LDS scratch of 16 ints that no
// other call may use until this one has returned in every thread.
__device__ __forceinline__ void group_rank(const int (&key)[kGroupPer], int b, int *wc,
                                           int (&rank)[kGroupPer])
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint64_t m[kGroupPer];
#pragma unroll
    for (int j = 0; j < kGroupPer; ++j)
        m[j] = __ballot(key[j] == b);
    if (lane == 0) {
#pragma unroll
        for (int j = 0; j < kGroupPer; ++j)
            wc[j * kGroupWaves + wave] = __popcll(m[j]);
    }
    __syncthreads();
    int run = 0;
#pragma unroll
    for (int j = 0; j < kGroupPer; ++j) {
        int before = run;
#pragma unroll
        for (int w = 0; w < kGroupWaves; ++w) {
            const int c = wc[j * kGroupWaves + w];
            before += w < wave ? c : 0;
            run += c;
        }
        const unsigned below =
            __builtin_amdgcn_mbcnt_hi((unsigned)(m[j] >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m[j], 0u));
        rank[j] = key[j] == b ? before + (int)below : -1;
    }
}

// Slot and index inside the slot's tiles of tile t (t < n_sg + n_bg).
__device__ __forceinline__ void locate_tile(const GroupLds &g, int N, int t, int &s, int &m)
{
    const bool sg = t < g.n_sg;
    const int *base = sg ? g.bsg : g.bbg;
    const int v = sg ? t : t - g.n_sg;
    // last slot s with base[s] <= v whose bucket holds tiles of this kind; the
    // bases are nondecreasing, slots without such tiles share the next one's base
    int lo = 0, hi = N;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (base[mid] <= v)
            lo = mid;
        else
            hi = mid;
    }
    s = lo;
    m = v - base[lo];
}

}  // namespace lora
