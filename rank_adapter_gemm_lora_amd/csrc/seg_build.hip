// seg_build.hip -- group the rows of a batch by adapter slot, on the device,
// and write the work lists of the shrink and expand kernels.
//
// Page "LoRA hot-loading and adapter routing", batched multi-adapter execution
// section: the batch is processed as one group of row indices per adapter id;
// page "Multi-LoRA Serving: one base, many adapters", section 2 flowchart:
// grouping the rows by their adapter id comes before add_shrink / add_expand.
//
// The grouping is a stable counting sort with n_slots + 1 buckets (bucket
// n_slots collects the rows without a valid adapter).  Two layouts: one
// workgroup per bucket for batches of at most 1024 rows (group.h), and a
// chunked count / scan / place for larger ones.  Launch shapes depend only on
// n and the slot count, never on the ids.
#include "device_common.h"
#include "group.h"
#include "internal.h"

namespace lora {

namespace {

// ---------------------------------------------------------------------------
// Larger batches: a chunked counting sort in three launches over chunks of 256
// rows (one row per thread).
//   count: each chunk's histogram over the buckets (and its bad ids); the row
//          keys are kept for the placement.
//   scan:  one workgroup turns the chunk histograms into, per bucket, the
//          exclusive prefix over chunks (in place), the group offsets, the tile
//          plan, the active list and the counts, and writes every tile header.
//   place: each chunk puts its rows at group offset + chunk prefix + rank among
//          the chunk's earlier rows of the same bucket, so the order inside a
//          group is the row order: the sort is stable.
// Every launch's shape depends only on n and the slot count.

constexpr int kChunk = kChunkRows;

__device__ __forceinline__ int chunk_key(const SegBuildArgs &a, int64_t i, int N, int &bad)
{
    if (i >= a.n)
        return -1;
    const int32_t id = a.ids[i];
    const bool in_range = (uint32_t)id < (uint32_t)N;
    const bool valid = in_range && a.slot_rank[in_range ? id : 0] > 0;
    bad = (!valid && id != -1) ? 1 : 0;
    return valid ? id : N;
}

__global__ __launch_bounds__(kChunk) void seg_count_kernel(SegBuildArgs a)
{
    __shared__ int hist[kGroupBuckets];
    __shared__ int nbad;
    const int N = a.n_slots, NB = N + 1, c = blockIdx.x, tid = threadIdx.x;
    const int64_t i = (int64_t)c * kChunk + tid;
    int bad = 0;
    const int key = chunk_key(a, i, N, bad);
    for (int e = tid; e < NB; e += kChunk)
        hist[e] = 0;
    if (tid == 0)
        nbad = 0;
    __syncthreads();
    if (key >= 0) {
        atomicAdd(&hist[key], 1);
        a.keys[i] = key;
    }
    if (bad)
        atomicAdd(&nbad, 1);
    __syncthreads();
    for (int e = tid; e < NB; e += kChunk)
        a.chunk[(int64_t)c * NB + e] = hist[e];
    if (tid == 0)
        a.chunk_bad[c] = nbad;
}

__global__ __launch_bounds__(kGroupThreads) void seg_scan_kernel(SegBuildArgs a, int n_chunks)
{
    __shared__ GroupLds g;
    const int N = a.n_slots, NB = N + 1, tid = threadIdx.x;
    const int sg_shift = a.sgmv_rows == 64 ? 6 : 4;
    // per bucket: exclusive prefix over the chunks (written back) and the
    // total.  tpb threads (a power of two inside one wavefront) share a bucket,
    // each taking a run of consecutive chunks; their sums are scanned across
    // the group with shuffles.  Loads go out in batches of kBat.
    constexpr int kBat = 16;
    int tpb = 1;
    while (tpb < 64 && 2 * tpb * NB <= kGroupThreads)
        tpb *= 2;
    const int per = (n_chunks + tpb - 1) / tpb;
    for (int b0 = 0; b0 < NB; b0 += kGroupThreads / tpb) {
        const int b = b0 + tid / tpb, sub = tid % tpb;
        const bool act = b < NB;
        const int c_begin = min(sub * per, n_chunks), c_end = min(c_begin + per, n_chunks);
        int32_t *col = a.chunk + (act ? b : 0);
        int v[kBat];
        int local = 0;
        for (int c0 = c_begin; c0 < c_end; c0 += kBat) {
#pragma unroll
            for (int j = 0; j < kBat; ++j)
                v[j] = (act && c0 + j < c_end) ? col[(int64_t)(c0 + j) * NB] : 0;
#pragma unroll
            for (int j = 0; j < kBat; ++j)
                local += v[j];
        }
        int incl = local;
        for (int o = 1; o < tpb; o <<= 1) {
            const int y = __shfl_up(incl, o, tpb);
            if (sub >= o)
                incl += y;
        }
        int run = incl - local;
        for (int c0 = c_begin; c0 < c_end; c0 += kBat) {
            if (c_end - c_begin > kBat) {   // values of this batch no longer in registers
#pragma unroll
                for (int j = 0; j < kBat; ++j)
                    v[j] = (act && c0 + j < c_end) ? col[(int64_t)(c0 + j) * NB] : 0;
            }
#pragma unroll
            for (int j = 0; j < kBat; ++j) {
                if (act && c0 + j < c_end) {
                    col[(int64_t)(c0 + j) * NB] = run;
                    run += v[j];
                }
            }
        }
        if (act && sub == tpb - 1)
            g.hist[b] = incl;
    }
    if (tid == 0)
        g.n_bad = 0;
    __syncthreads();
    int bad = 0;
    for (int c = tid; c < n_chunks; c += kGroupThreads)
        bad += a.chunk_bad[c];
    if (bad)
        atomicAdd(&g.n_bad, bad);
    group_scan(g, N, a.dense_min, sg_shift);   // ends with a barrier
    group_store(g, N, a.seg_off, a.active, a.counts);
    // per bucket: group offset, first tile, tile shift, path
    for (int b = tid; b < NB; b += kGroupThreads) {
        const BucketPlan p = bucket_plan(g, b, N, a.dense_min, sg_shift);
        a.binfo[b] = make_int4(p.first, p.tile0, p.shift, p.path);
    }
    for (int t = tid; t < g.n_sg + g.n_bg; t += kGroupThreads) {
        int s, m;
        locate_tile(g, N, t, s, m);
        const BucketPlan p = bucket_plan(g, s, N, a.dense_min, sg_shift);
        const int lo = m << p.shift;
        *reinterpret_cast<int4 *>(&a.tiles[t]) =
            make_int4(s, p.first + lo, min(1 << p.shift, p.count - lo), p.path);
    }
}

__global__ __launch_bounds__(kChunk) void seg_place_kernel(SegBuildArgs a)
{
    __shared__ int run[kGroupBuckets];
    __shared__ int4 info[kGroupBuckets];
    const int N = a.n_slots, NB = N + 1, c = blockIdx.x, tid = threadIdx.x;
    const int wave = tid >> 6;
    const int64_t i = (int64_t)c * kChunk + tid;
    const int key = i < a.n ? a.keys[i] : -1;
    for (int e = tid; e < NB; e += kChunk) {
        const int4 bi = a.binfo[e];
        info[e] = bi;
        run[e] = bi.x + a.chunk[(int64_t)c * NB + e];
    }
    // rank among the wavefront's lanes with the same key, one distinct key at
    // a time (the lowest lane still unplaced names the next key)
    int rank = 0, count = 0;
    uint64_t left = __ballot(key >= 0);
    while (left) {
        const int k0 = __builtin_amdgcn_readlane(key, (int)__builtin_ctzll(left));
        const uint64_t m = __ballot(key == k0);
        if (key == k0) {
            rank = (int)__builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
            count = __popcll(m);
        }
        left &= ~m;
    }
    __syncthreads();   // run and info ready
    // wavefronts in row order: read the running position, then the key's first
    // lane advances it (inside a wavefront every read precedes the write)
    int pos = -1;
    for (int w = 0; w < kChunk / 64; ++w) {
        if (wave == w && key >= 0) {
            pos = run[key] + rank;
            if (rank == 0)
                run[key] += count;
        }
        __syncthreads();
    }
    if (key >= 0) {
        a.perm[pos] = (int32_t)i;
        if (key < N) {
            const int4 bi = info[key];
            const int p = pos - bi.x;
            a.tiles[bi.y + (p >> bi.z)].rows[p & ((1 << bi.z) - 1)] = (int32_t)i;
        }
    }
}

// ---------------------------------------------------------------------------
// Batches of at most kGroupRows rows: one workgroup per bucket again, but every
// row sits in a register of its own thread (group.h), so the ranks inside a
// bucket come from ballots instead of a block scan per chunk, and each bucket's
// workgroup writes the headers of its own tiles.
__global__ __launch_bounds__(kGroupThreads) void seg_build_small_kernel(SegBuildArgs a)
{
    __shared__ GroupLds g;
    __shared__ int wc[kGroupPer * kGroupWaves];
    const int b = blockIdx.x, N = a.n_slots, tid = threadIdx.x;
    const int sg_shift = a.sgmv_rows == 64 ? 6 : 4;
    int key[kGroupPer];
    group_hist(a.ids, (int)a.n, N, a.slot_rank, g, key);
    group_scan(g, N, a.dense_min, sg_shift);
    int rank[kGroupPer];
    group_rank(key, b, wc, rank);
    const BucketPlan p = bucket_plan(g, b, N, a.dense_min, sg_shift);
    const int mask = (1 << p.shift) - 1;
#pragma unroll
    for (int j = 0; j < kGroupPer; ++j) {
        if (rank[j] >= 0) {
            const int row = j * kGroupThreads + tid;
            a.perm[p.first + rank[j]] = row;
            if (b < N)
                a.tiles[p.tile0 + (rank[j] >> p.shift)].rows[rank[j] & mask] = row;
        }
    }
    if (b < N) {
        const int nt = (p.count + mask) >> p.shift;
        for (int m = tid; m < nt; m += kGroupThreads)
            *reinterpret_cast<int4 *>(&a.tiles[p.tile0 + m]) =
                make_int4(b, p.first + (m << p.shift), min(1 << p.shift, p.count - (m << p.shift)),
                          p.path);
    }
    if (b == 0)
        group_store(g, N, a.seg_off, a.active, a.counts);
}

}  // namespace

hipError_t launch_seg_build(const SegBuildArgs &a, hipStream_t stream)
{
    if (a.n <= kGroupRows) {
        hipLaunchKernelGGL(seg_build_small_kernel, dim3(a.n_slots + 1), dim3(kGroupThreads), 0,
                           stream, a);
        return hipGetLastError();
    }
    const int n_chunks = (int)((a.n + kChunk - 1) / kChunk);
    hipLaunchKernelGGL(seg_count_kernel, dim3(n_chunks), dim3(kChunk), 0, stream, a);
    hipLaunchKernelGGL(seg_scan_kernel, dim3(1), dim3(kGroupThreads), 0, stream, a, n_chunks);
    hipLaunchKernelGGL(seg_place_kernel, dim3(n_chunks), dim3(kChunk), 0, stream, a);
    return hipGetLastError();
}

}  // namespace lora
