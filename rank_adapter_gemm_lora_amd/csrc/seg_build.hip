// seg_build.hip -- group the rows of a batch by adapter slot, on the device,
// and write the work lists of the shrink and expand kernels.
//
// Page "LoRA hot-loading and adapter routing", batched multi-adapter execution
// section: the batch is processed as one group of row indices per adapter id;
// page "Multi-LoRA Serving: one base, many adapters", section 2 flowchart:
// grouping the rows by their adapter id comes before add_shrink / add_expand.
//
// The grouping is a stable counting sort with n_slots + 1 buckets (bucket
// n_slots collects the rows without a valid adapter); the kernel below says
// how it is laid out on the GPU.  The launch shape depends only on the slot
// count, never on the ids.
#include "device_common.h"
#include "group.h"
#include "internal.h"

namespace lora {

namespace {

// Last index s in [0, n) with base[s] <= v (base nondecreasing, base[0] <= v).
__device__ __forceinline__ int upper_slot(const int *base, int n, int v)
{
    int lo = 0, hi = n;   // answer in [lo, hi)
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (base[mid] <= v)
            lo = mid;
        else
            hi = mid;
    }
    return lo;
}

// ---------------------------------------------------------------------------
// One workgroup per bucket.  Every workgroup reads all ids and the slot table,
// builds the bucket histogram and its scan in LDS (cheap at these sizes), then
// writes only the rows of its own bucket.  Rows are taken in chunks of
// kParRows, thread t owning rows [kParPer t, kParPer (t + 1)) of a chunk, so a
// block scan of per-thread match counts (plus the count carried from earlier
// chunks) gives every row its rank in index order: the sort is stable.
// Workgroup 0 also writes seg_off, active, counts and the tile headers.  All
// workgroups run at once and none waits on another.

constexpr int kParThreads = 256;
constexpr int kParPer = 16;                           // rows per thread per chunk
constexpr int kParRows = kParThreads * kParPer;       // 4096 rows per chunk
constexpr int kParBuckets = LORA_MAX_SLOTS + 1;

// Exclusive scan of one int4 per thread (component-wise) over 256 threads.
__device__ int4 scan256x4(int4 v, int4 *tmp, int4 *total)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int4 x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int4 y = make_int4(__shfl_up(x.x, o), __shfl_up(x.y, o), __shfl_up(x.z, o),
                                 __shfl_up(x.w, o));
        if (lane >= o) {
            x.x += y.x; x.y += y.y; x.z += y.z; x.w += y.w;
        }
    }
    if (lane == 63)
        tmp[w] = x;
    __syncthreads();
    int4 base = make_int4(0, 0, 0, 0), tot = make_int4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int4 t = tmp[u];
        if (u < w) {
            base.x += t.x; base.y += t.y; base.z += t.z; base.w += t.w;
        }
        tot.x += t.x; tot.y += t.y; tot.z += t.z; tot.w += t.w;
    }
    *total = tot;
    __syncthreads();
    return make_int4(base.x + x.x - v.x, base.y + x.y - v.y, base.z + x.z - v.z, base.w + x.w - v.w);
}

// ids of rows [r0, r0 + kParPer) (-1 past the batch end).
__device__ __forceinline__ void load_ids(const SegBuildArgs &a, int64_t r0, int32_t (&id)[kParPer])
{
#pragma unroll
    for (int j = 0; j < kParPer; ++j)
        id[j] = r0 + j < a.n ? a.ids[r0 + j] : -1;
}

// Bucket key of row i with id `id`: the slot when it holds an adapter, n_slots
// otherwise, -1 past the batch end.  Branch-free: the table lookup is always
// made, at a clamped (in-bounds) index.
__device__ __forceinline__ int row_key(int64_t i, int64_t n, int32_t id, int N, const uint8_t *ok,
                                       int &bad)
{
    const bool in = i < n;
    const bool in_range = (uint32_t)id < (uint32_t)N;
    const int look = ok[in_range ? id : 0];
    const bool valid = in_range && look != 0;
    bad += (in && !valid && id != -1) ? 1 : 0;
    return in ? (valid ? id : N) : -1;
}

__global__ __launch_bounds__(kParThreads) void seg_build_kernel(SegBuildArgs a)
{
    __shared__ int hist[kParBuckets];    // rows per bucket
    __shared__ int seg[kParBuckets];     // seg_off
    __shared__ int bsg[kParBuckets];     // first SGMV tile of each slot
    __shared__ int bbg[kParBuckets];     // first BGMV tile (without the SGMV count)
    __shared__ uint8_t ok[kParBuckets];
    __shared__ int4 tmp[4];

    const int b = blockIdx.x;            // the bucket this workgroup places
    const int N = a.n_slots, NB = N + 1;
    const int tid = threadIdx.x;
    const int64_t n = a.n;
    const int sg_shift = a.sgmv_rows == 64 ? 6 : 4;   // dense tiles: 16 or 64 rows

    // the first chunk's ids in flight while the slot table is copied to LDS;
    // a one-chunk batch keeps them in registers for both passes
    int32_t id0[kParPer];
    load_ids(a, (int64_t)tid * kParPer, id0);
    for (int e = tid; e < NB; e += kParThreads) {
        hist[e] = 0;
        ok[e] = (e < N && a.slot_rank[e] > 0) ? 1 : 0;
    }
    __syncthreads();

    // histogram; runs of equal keys are merged inside the thread; the next
    // chunk's ids are in flight while this one is counted
    int bad = 0;
    int32_t idn[kParPer];
#pragma unroll
    for (int j = 0; j < kParPer; ++j)
        idn[j] = id0[j];
    for (int64_t c0 = 0; c0 < n; c0 += kParRows) {
        const int64_t r0 = c0 + (int64_t)tid * kParPer;
        int32_t id[kParPer];
#pragma unroll
        for (int j = 0; j < kParPer; ++j)
            id[j] = idn[j];
        if (c0 + kParRows < n)
            load_ids(a, r0 + kParRows, idn);
        int run_key = -1, run_len = 0;
#pragma unroll
        for (int j = 0; j < kParPer; ++j) {
            const int key = row_key(r0 + j, n, id[j], N, ok, bad);
            if (key != run_key) {
                if (run_len > 0)
                    atomicAdd(&hist[run_key], run_len);
                run_key = key;
                run_len = 0;
            }
            run_len += key >= 0 ? 1 : 0;
        }
        if (run_len > 0)
            atomicAdd(&hist[run_key], run_len);
    }
    __syncthreads();

    // scan of the buckets, 4 per thread per pass: (rows, SGMV tiles, BGMV tiles, active)
    int4 carry = make_int4(0, 0, 0, 0);
    for (int e0 = 0; e0 < NB; e0 += 4 * kParThreads) {
        int4 v4[4];
        int4 sum = make_int4(0, 0, 0, 0);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e = e0 + 4 * tid + u;
            v4[u] = make_int4(0, 0, 0, 0);
            if (e < NB) {
                const int c = hist[e];
                v4[u].x = c;
                if (e < N && c > 0) {
                    const bool dn = c >= a.dense_min;
                    v4[u].y = dn ? (c + (1 << sg_shift) - 1) >> sg_shift : 0;
                    v4[u].z = dn ? 0 : (c + kBgmvTileRows - 1) >> 4;
                    v4[u].w = 1;
                }
            }
            sum.x += v4[u].x; sum.y += v4[u].y; sum.z += v4[u].z; sum.w += v4[u].w;
        }
        int4 tot;
        int4 ex = scan256x4(sum, tmp, &tot);
        ex.x += carry.x; ex.y += carry.y; ex.z += carry.z; ex.w += carry.w;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e = e0 + 4 * tid + u;
            if (e < NB) {
                seg[e] = ex.x;
                bsg[e] = ex.y;
                bbg[e] = ex.z;
                if (b == 0) {
                    a.seg_off[e] = ex.x;
                    if (v4[u].w)
                        a.active[ex.w] = e;
                }
            }
            ex.x += v4[u].x; ex.y += v4[u].y; ex.z += v4[u].z; ex.w += v4[u].w;
        }
        carry.x += tot.x; carry.y += tot.y; carry.z += tot.z; carry.w += tot.w;
    }
    __syncthreads();
    const int n_sg = carry.y, n_bg = carry.z;

    // this bucket's rows, in index order
    const bool dense = b < N && hist[b] >= a.dense_min;
    const int tile0 = dense ? bsg[b] : n_sg + bbg[b];
    const int shift = dense ? sg_shift : 4;
    const int mask = (1 << shift) - 1;
    int placed = 0, bad_w = 0;
    if (n > kParRows)
        load_ids(a, (int64_t)tid * kParPer, idn);       // second pass from chunk 0 again
    for (int64_t c0 = 0; c0 < n; c0 += kParRows) {
        const int64_t r0 = c0 + (int64_t)tid * kParPer;
        int32_t id[kParPer];
#pragma unroll
        for (int j = 0; j < kParPer; ++j)
            id[j] = n > kParRows ? idn[j] : id0[j];
        if (c0 + kParRows < n)
            load_ids(a, r0 + kParRows, idn);
        int key[kParPer];
        int mine = 0;
#pragma unroll
        for (int j = 0; j < kParPer; ++j) {
            key[j] = row_key(r0 + j, n, id[j], N, ok, bad_w);
            mine += key[j] == b ? 1 : 0;
        }
        int4 tot;
        int rk = placed + scan256x4(make_int4(mine, 0, 0, 0), tmp, &tot).x;
        placed += tot.x;
#pragma unroll
        for (int j = 0; j < kParPer; ++j) {
            if (key[j] == b) {
                a.perm[seg[b] + rk] = (int32_t)(r0 + j);
                if (b < N)
                    a.tiles[tile0 + (rk >> shift)].rows[rk & mask] = (int32_t)(r0 + j);
                ++rk;
            }
        }
    }

    if (b != 0)
        return;
    // workgroup 0: the rest of the active list, counts, tile headers
    int4 bt;
    (void)scan256x4(make_int4(bad, 0, 0, 0), tmp, &bt);
    for (int e = carry.w + tid; e < N; e += kParThreads)
        a.active[e] = -1;
    if (tid == 0) {
        a.counts[kCntValid] = seg[N];
        a.counts[kCntActive] = carry.w;
        a.counts[kCntBad] = bt.x;
        a.counts[kCntSgmv] = n_sg;
        a.counts[kCntBgmv] = n_bg;
    }
    for (int t = tid; t < n_sg + n_bg; t += kParThreads) {
        int s, m, sh;
        if (t < n_sg) {
            s = upper_slot(bsg, N, t);
            m = t - bsg[s];
            sh = sg_shift;
        } else {
            s = upper_slot(bbg, N, t - n_sg);
            m = t - n_sg - bbg[s];
            sh = 4;
        }
        const int c = hist[s];
        *reinterpret_cast<int4 *>(&a.tiles[t]) =
            make_int4(s, seg[s] + (m << sh), min(1 << sh, c - (m << sh)),
                      t < n_sg ? kTileSgmv : kTileBgmv);
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
    if (a.n <= kGroupRows)
        hipLaunchKernelGGL(seg_build_small_kernel, dim3(a.n_slots + 1), dim3(kGroupThreads), 0,
                           stream, a);
    else
        hipLaunchKernelGGL(seg_build_kernel, dim3(a.n_slots + 1), dim3(kParThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace lora
