// seg_build.hip -- group the rows of a batch by adapter slot, on the device.
//
// Page "LoRA hot-loading and adapter routing", batched multi-adapter execution
// section: the batch is processed as one group of row indices per adapter id;
// page "Multi-LoRA Serving: one base, many adapters", section 2 flowchart:
// "group rows by adapter id" precedes add_shrink / add_expand.
//
// The grouping is a stable counting sort with n_slots + 1 buckets (bucket
// n_slots collects rows without a valid adapter), done by ONE workgroup of 1024
// threads so that the result is bit-exact and no atomic decides an order:
//   1. histogram (LDS atomics only add counts, which is order-free);
//   2. exclusive scan -> seg_off;
//   3. active-slot list and the tile plan (SGMV tiles first, then BGMV tiles);
//   4. stable scatter, 1024 rows per pass: inside a wavefront a row's rank among
//      equal keys comes from a ballot of the lanes below it; across the 16
//      wavefronts of the pass, per-key counts are prefix-summed in wave order;
//      across passes a running offset per key carries on.
// The launch shape never depends on the ids.
#include "device_common.h"
#include "internal.h"

namespace lora {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

// Exclusive scan of one int per thread across the workgroup; *total receives
// the sum.  tmp: LDS scratch of at least kWaves + 1 ints.
__device__ int block_exclusive_scan(int v, int *tmp, int *total)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int y = __shfl_up(x, o);
        if (lane >= o)
            x += y;
    }
    if (lane == 63)
        tmp[w] = x;
    __syncthreads();
    if (w == 0) {
        int t = lane < kWaves ? tmp[lane] : 0;
        int s = t;
#pragma unroll
        for (int o = 1; o < kWaves; o <<= 1) {
            int y = __shfl_up(s, o);
            if (lane >= o)
                s += y;
        }
        if (lane < kWaves)
            tmp[lane] = s - t;
        if (lane == kWaves - 1)
            tmp[kWaves] = s;
    }
    __syncthreads();
    int excl = tmp[w] + x - v;
    *total = tmp[kWaves];
    __syncthreads();
    return excl;
}

__device__ __forceinline__ bool routed(int32_t id, int n_slots, const int32_t *rank)
{
    return id >= 0 && id < n_slots && rank[id] > 0;
}

__global__ __launch_bounds__(kThreads) void seg_build_kernel(SegBuildArgs a)
{
    extern __shared__ int smem[];
    const int NB = a.n_slots + 1;                 // buckets: slots, then "no adapter"
    const int NBp = (NB + 3) & ~3;
    int *hist = smem;                             // [NB] counts, later per-pass totals
    int *run = hist + NBp;                        // [NB] running start of each bucket
    int *tmp = run + NBp;                         // [kWaves + 1] scan scratch
    int *misc = tmp + 32;                         // [4]
    uint16_t *wcnt = reinterpret_cast<uint16_t *>(misc + 4);  // [kWaves][NB]

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t n = a.n;

    for (int e = tid; e < NB; e += kThreads)
        hist[e] = 0;
    if (tid == 0)
        misc[0] = 0;
    __syncthreads();

    // 1. histogram
    int bad = 0;
    for (int64_t i = tid; i < n; i += kThreads) {
        int32_t id = a.ids[i];
        bool ok = routed(id, a.n_slots, a.slot_rank);
        atomicAdd(&hist[ok ? id : a.n_slots], 1);
        bad += (!ok && id != -1);
    }
    if (bad)
        atomicAdd(&misc[0], bad);
    __syncthreads();

    // 2. exclusive scan of the buckets -> run[], seg_off[]
    int carry = 0;
    for (int e0 = 0; e0 < NB; e0 += kThreads) {
        int e = e0 + tid;
        int v = e < NB ? hist[e] : 0;
        int total;
        int ex = block_exclusive_scan(v, tmp, &total);
        if (e < NB) {
            run[e] = carry + ex;
            a.seg_off[e] = carry + ex;
        }
        carry += total;
    }
    __syncthreads();

    // 3. active slots and the tile plan; one thread per slot
    {
        int act_carry = 0, sg_carry = 0, bg_carry = 0;
        int n_sgmv_total = 0;
        // first pass: SGMV tile total (SGMV tiles are stored first)
        for (int s0 = 0; s0 < a.n_slots; s0 += kThreads) {
            int s = s0 + tid;
            int c = s < a.n_slots ? hist[s] : 0;
            bool dense = a.sgmv_ok && c >= a.dense_min;
            int nt = (c > 0 && dense) ? (c + kSgmvTileRows - 1) / kSgmvTileRows : 0;
            int total;
            (void)block_exclusive_scan(nt, tmp, &total);
            n_sgmv_total += total;
        }
        for (int s0 = 0; s0 < a.n_slots; s0 += kThreads) {
            int s = s0 + tid;
            int c = s < a.n_slots ? hist[s] : 0;
            bool dense = a.sgmv_ok && c >= a.dense_min;
            int nsg = (c > 0 && dense) ? (c + kSgmvTileRows - 1) / kSgmvTileRows : 0;
            int nbg = (c > 0 && !dense) ? (c + kBgmvTileRows - 1) / kBgmvTileRows : 0;
            int tot_a, tot_s, tot_b;
            int pa = block_exclusive_scan(c > 0 ? 1 : 0, tmp, &tot_a);
            int ps = block_exclusive_scan(nsg, tmp, &tot_s);
            int pb = block_exclusive_scan(nbg, tmp, &tot_b);
            if (s < a.n_slots) {
                if (c > 0)
                    a.active[act_carry + pa] = s;
                int start = run[s];
                for (int m = 0; m < nsg; ++m) {
                    int rows = min(kSgmvTileRows, c - m * kSgmvTileRows);
                    a.tiles[sg_carry + ps + m] =
                        make_int4(s, start + m * kSgmvTileRows, rows, kTileSgmv);
                }
                for (int m = 0; m < nbg; ++m) {
                    int rows = min(kBgmvTileRows, c - m * kBgmvTileRows);
                    a.tiles[n_sgmv_total + bg_carry + pb + m] =
                        make_int4(s, start + m * kBgmvTileRows, rows, kTileBgmv);
                }
            }
            act_carry += tot_a;
            sg_carry += tot_s;
            bg_carry += tot_b;
        }
        for (int s = act_carry + tid; s < a.n_slots; s += kThreads)
            a.active[s] = -1;
        if (tid == 0) {
            a.counts[kCntValid] = run[a.n_slots];
            a.counts[kCntActive] = act_carry;
            a.counts[kCntBad] = misc[0];
            a.counts[kCntSgmv] = sg_carry;
            a.counts[kCntBgmv] = bg_carry;
        }
    }
    __syncthreads();

    // 4. stable scatter, one row per thread per pass
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int64_t base = 0; base < n; base += kThreads) {
        for (int e = tid; e < kWaves * NB; e += kThreads)
            wcnt[e] = 0;
        __syncthreads();

        const int64_t i = base + tid;
        const bool in = i < n;
        int key = a.n_slots;
        if (in) {
            int32_t id = a.ids[i];
            key = routed(id, a.n_slots, a.slot_rank) ? id : a.n_slots;
        }
        // rank of this row among the equal keys of its wavefront, lanes below it
        uint64_t pending = __ballot(in);
        int my_rank = 0;
        while (pending) {
            const int leader = __ffsll((unsigned long long)pending) - 1;
            const int k0 = __shfl(key, leader);
            const uint64_t m = __ballot(in && key == k0);
            if (in && key == k0)
                my_rank = __popcll(m & below);
            if (lane == leader)
                wcnt[w * NB + k0] = (uint16_t)__popcll(m);
            pending &= ~m;
        }
        __syncthreads();

        // per key: prefix over the wavefronts of this pass, and the pass total
        for (int e = tid; e < NB; e += kThreads) {
            int p = 0;
#pragma unroll
            for (int ww = 0; ww < kWaves; ++ww) {
                int c = wcnt[ww * NB + e];
                wcnt[ww * NB + e] = (uint16_t)p;
                p += c;
            }
            hist[e] = p;
        }
        __syncthreads();

        if (in)
            a.perm[run[key] + wcnt[w * NB + key] + my_rank] = (int32_t)i;
        __syncthreads();

        for (int e = tid; e < NB; e += kThreads)
            run[e] += hist[e];
        __syncthreads();
    }
}

}  // namespace

size_t seg_build_lds_bytes(int n_slots)
{
    const int NB = n_slots + 1;
    const int NBp = (NB + 3) & ~3;
    return sizeof(int) * (2 * NBp + 32 + 4) + sizeof(uint16_t) * (size_t)kWaves * NB;
}

hipError_t launch_seg_build(const SegBuildArgs &a, hipStream_t stream)
{
    hipLaunchKernelGGL(seg_build_kernel, dim3(1), dim3(kThreads), seg_build_lds_bytes(a.n_slots),
                       stream, a);
    return hipGetLastError();
}

}  // namespace lora
