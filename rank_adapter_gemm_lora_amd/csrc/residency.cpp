// residency.cpp -- the adapter lifecycle around one stack: a host tier of
// registered adapters in pinned memory, GPU residency of up to n_slots of them
// with least-recently-used eviction, and the mapping of a batch's per-row
// adapter ids to slot ids.
//
// Page "LoRA hot-loading and adapter routing", adapter-lifecycle section: an
// adapter is loaded when a request first uses it, after its rank is checked
// against the engine's limit; when more adapters are loaded than the limit
// allows, the one used least recently is unloaded and must be loaded again on
// its next use.  Page "Multi-LoRA Serving: one base, many adapters", section
// 3.2: adapters stay resident in GPU memory, with an optional CPU-side cache
// for the cold ones; max_loras bounds the distinct adapters one batch can run
// together, max_cpu_loras the CPU cache; section 6: a batch that references
// more distinct adapters than max_loras cannot run in one step.  Page "LoRA
// serving: multi-adapter dynamic loading", section 4: loading copies A and B
// to the GPU, unloading is immediate.
//
// A manager created without a stack plans only: it takes the same decisions
// (hits, loads, evictions, slot ids) and moves no data, for schedulers that
// simulate admission and for tests of the policy on a machine without a GPU.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

#include "internal.h"

namespace {

struct HostEntry {
    int rank = 0;
    float alpha = 0.f;
    void *A = nullptr;        // pinned, mapped [n_slices][rank][k]
    void *B = nullptr;        // pinned, mapped [D][rank]
    void *dA = nullptr;       // their device-side addresses
    void *dB = nullptr;
    uint64_t last = 0;        // tick of the last batch that used it (or its registration)
    int slot = -1;            // GPU slot holding it, -1 when not resident
    hipEvent_t copied = nullptr;   // completes when the last load from A, B has been consumed
    bool pending = false;
};

lora_status hip_status(hipError_t e)
{
    if (e == hipSuccess)
        return LORA_OK;
    (void)hipGetLastError();
    return e == hipErrorOutOfMemory ? LORA_E_NOMEM : LORA_E_HIP;
}

}  // namespace

struct lora_residency {
    lora_stack *st = nullptr;   // null: plan only
    int n_slots = 0, r_max = 0, max_cpu = 0;
    int64_t k = 0, D = 0;
    int n_slices = 0, esize = 0;
    uint64_t tick = 0;
    std::unordered_map<int64_t, HostEntry> host;
    std::vector<int64_t> slot_adapter;   // adapter held by each slot, -1 = empty
    int64_t stats[LORA_RES_NSTATS] = {};
};

namespace {

// Wait for the copies that read an entry's pinned buffers, then free them.
lora_status release_entry(HostEntry &e)
{
    lora_status rc = LORA_OK;
    if (e.copied) {
        if (e.pending)
            rc = hip_status(hipEventSynchronize(e.copied));
        (void)hipEventDestroy(e.copied);
        e.copied = nullptr;
    }
    if (e.A)
        (void)hipHostFree(e.A);
    if (e.B)
        (void)hipHostFree(e.B);
    e.A = e.B = nullptr;
    return rc;
}

// Free a slot in stream order (plan mode: bookkeeping only).
lora_status evict(lora_residency *m, int slot, void *stream)
{
    const int64_t id = m->slot_adapter[slot];
    if (id < 0)
        return LORA_OK;
    if (m->st) {
        const lora_status rc = lora_evict_slot(m->st, slot, stream);
        if (rc != LORA_OK)
            return rc;
    }
    auto it = m->host.find(id);
    if (it != m->host.end())
        it->second.slot = -1;
    m->slot_adapter[slot] = -1;
    m->stats[LORA_RES_EVICTIONS] += 1;
    return LORA_OK;
}

// Put registered adapters into free slots: bookkeeping first, then one
// gather kernel per kGatherJobs adapters that reads them straight from the
// pinned host tier and writes the pool and the slot table, in stream order.
lora_status load_all(lora_residency *m, const std::vector<std::pair<int, int64_t>> &todo,
                     void *stream)
{
    for (const auto &t : todo) {
        HostEntry &e = m->host.at(t.second);
        e.slot = t.first;
        m->slot_adapter[t.first] = t.second;
        m->stats[LORA_RES_LOADS] += 1;
        m->stats[LORA_RES_BYTES_LOADED] += (int64_t)e.rank * (m->n_slices * m->k + m->D) * m->esize;
    }
    if (!m->st || todo.empty())
        return LORA_OK;
    lora_stack *st = m->st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    for (size_t b = 0; b < todo.size(); b += lora::kGatherJobs) {
        lora::GatherArgs g;
        std::memset(&g, 0, sizeof g);
        g.A_pool = st->A_pool;
        g.A_img = st->A_img;
        g.B_pool = st->B_pool;
        g.rank_tab = st->d_rank;
        g.scale_tab = st->d_scale;
        g.k = st->k;
        g.D = st->D;
        g.n_slices = st->n_slices;
        g.r_max = st->r_max;
        g.rp_max = st->rp_max;
        g.esize = st->esize;
        const size_t n = std::min(todo.size() - b, (size_t)lora::kGatherJobs);
        g.n_jobs = (int)n;
        for (size_t i = 0; i < n; ++i) {
            const HostEntry &e = m->host.at(todo[b + i].second);
            g.job[i].A = e.dA;
            g.job[i].B = e.dB;
            g.job[i].slot = todo[b + i].first;
            g.job[i].rank = e.rank;
            g.job[i].scale = e.alpha / (float)e.rank;   // the slot table's value, as in a load
        }
        lora_status rc = hip_status(lora::launch_gather_load(g, s));
        if (rc != LORA_OK)
            return rc;
        for (size_t i = 0; i < n; ++i) {
            HostEntry &e = m->host.at(todo[b + i].second);
            lora::note_loaded(st, todo[b + i].first, e.rank, e.alpha);
            rc = hip_status(hipEventRecord(e.copied, s));
            if (rc != LORA_OK)
                return rc;
            e.pending = true;
        }
    }
    return LORA_OK;
}

// Free a slot for an adapter about to be loaded into it: bookkeeping only (the
// load overwrites the slot's pool region and table entry in stream order).
void displace(lora_residency *m, int slot)
{
    const int64_t id = m->slot_adapter[slot];
    if (id < 0)
        return;
    auto it = m->host.find(id);
    if (it != m->host.end())
        it->second.slot = -1;
    m->slot_adapter[slot] = -1;
    m->stats[LORA_RES_EVICTIONS] += 1;
}

// Follow direct calls on the stack made since the last batch: a slot the
// caller loaded becomes the caller's; a slot the caller emptied (evicted, or
// never the manager's) becomes usable; an adapter whose slot the caller
// evicted is no longer resident.
void follow_stack(lora_residency *m)
{
    if (!m->st)
        return;
    for (int sl = 0; sl < m->n_slots; ++sl) {
        const bool loaded = m->st->h_rank[sl] != 0;
        const int64_t a = m->slot_adapter[sl];
        if (a == -1 && loaded) {
            m->slot_adapter[sl] = -2;
        } else if (a == -2 && !loaded) {
            m->slot_adapter[sl] = -1;
        } else if (a >= 0 && !loaded) {
            auto it = m->host.find(a);
            if (it != m->host.end())
                it->second.slot = -1;
            m->slot_adapter[sl] = -1;
        }
    }
}

}  // namespace

extern "C" {

lora_status lora_residency_create(lora_residency **out, lora_stack *st, int n_slots, int r_max,
                                  int64_t k, int n_slices, const int64_t *slice_d,
                                  lora_dtype dtype, int max_cpu_adapters)
{
    if (!out)
        return LORA_E_ARG;
    *out = nullptr;
    if (max_cpu_adapters < 1)
        return LORA_E_ARG;
    lora_residency *m = new (std::nothrow) lora_residency;
    if (!m)
        return LORA_E_NOMEM;
    if (st) {
        m->st = st;
        m->n_slots = st->n_slots;
        m->r_max = st->r_max;
        m->k = st->k;
        m->n_slices = st->n_slices;
        m->D = st->D;
        m->esize = st->esize;
    } else {
        if (n_slots < 1 || n_slots > LORA_MAX_SLOTS || r_max < 1 || r_max > LORA_MAX_RANK || k < 1 ||
            n_slices < 1 || n_slices > LORA_MAX_SLICES || !slice_d ||
            (dtype != LORA_F32 && dtype != LORA_BF16)) {
            delete m;
            return LORA_E_ARG;
        }
        m->n_slots = n_slots;
        m->r_max = r_max;
        m->k = k;
        m->n_slices = n_slices;
        for (int q = 0; q < n_slices; ++q) {
            if (slice_d[q] < 1) {
                delete m;
                return LORA_E_ARG;
            }
            m->D += slice_d[q];
        }
        m->esize = dtype == LORA_F32 ? 4 : 2;
    }
    m->max_cpu = max_cpu_adapters;
    m->slot_adapter.assign(m->n_slots, -1);
    if (st) {
        // slots the caller already filled stay the caller's: never handed out
        for (int sl = 0; sl < m->n_slots; ++sl)
            if (st->h_rank[sl] != 0)
                m->slot_adapter[sl] = -2;
    }
    *out = m;
    return LORA_OK;
}

lora_status lora_residency_destroy(lora_residency *m)
{
    if (!m)
        return LORA_OK;
    lora_status rc = LORA_OK;
    for (auto &kv : m->host) {
        const lora_status r = release_entry(kv.second);
        if (rc == LORA_OK)
            rc = r;
    }
    delete m;
    return rc;
}

lora_status lora_residency_register(lora_residency *m, int64_t adapter_id, int rank, float alpha,
                                    const void *A, const void *B)
{
    if (!m || adapter_id < 0 || !A || !B || !std::isfinite(alpha))
        return LORA_E_ARG;
    if (rank < 1 || rank > m->r_max)
        return LORA_E_RANK;
    if (m->host.count(adapter_id))
        return LORA_E_OCCUPIED;
    if ((int)m->host.size() >= m->max_cpu) {
        // drop the least recently used adapter that is not on the GPU
        auto victim = m->host.end();
        for (auto it = m->host.begin(); it != m->host.end(); ++it) {
            if (it->second.slot >= 0)
                continue;
            if (victim == m->host.end() || it->second.last < victim->second.last ||
                (it->second.last == victim->second.last && it->first < victim->first))
                victim = it;
        }
        if (victim == m->host.end())
            return LORA_E_CAPACITY;
        const lora_status rc = release_entry(victim->second);
        m->host.erase(victim);
        m->stats[LORA_RES_HOST_DROPS] += 1;
        if (rc != LORA_OK)
            return rc;
    }
    HostEntry e;
    e.rank = rank;
    e.alpha = alpha;
    e.last = ++m->tick;   // a registration counts as a use
    if (m->st) {
        const size_t a_bytes = (size_t)m->n_slices * rank * m->k * m->esize;
        const size_t b_bytes = (size_t)m->D * rank * m->esize;
        lora_status rc = hip_status(hipHostMalloc(&e.A, a_bytes, hipHostMallocMapped));
        if (rc == LORA_OK)
            rc = hip_status(hipHostMalloc(&e.B, b_bytes, hipHostMallocMapped));
        if (rc == LORA_OK)
            rc = hip_status(hipHostGetDevicePointer(&e.dA, e.A, 0));
        if (rc == LORA_OK)
            rc = hip_status(hipHostGetDevicePointer(&e.dB, e.B, 0));
        if (rc == LORA_OK)
            rc = hip_status(hipEventCreateWithFlags(&e.copied, hipEventDisableTiming));
        if (rc != LORA_OK) {
            release_entry(e);
            return rc;
        }
        std::memcpy(e.A, A, a_bytes);
        std::memcpy(e.B, B, b_bytes);
    }
    m->host.emplace(adapter_id, e);
    return LORA_OK;
}

lora_status lora_residency_unregister(lora_residency *m, int64_t adapter_id, void *stream)
{
    if (!m)
        return LORA_E_ARG;
    auto it = m->host.find(adapter_id);
    if (it == m->host.end())
        return LORA_E_NOT_FOUND;
    if (it->second.slot >= 0) {
        const lora_status rc = evict(m, it->second.slot, stream);
        if (rc != LORA_OK)
            return rc;
    }
    const lora_status rc = release_entry(it->second);
    m->host.erase(it);
    return rc;
}

lora_status lora_residency_map_batch(lora_residency *m, const int64_t *row_adapter, int64_t n_rows,
                                     int32_t *ids_out, void *stream)
{
    if (!m || n_rows < 0 || (n_rows > 0 && (!row_adapter || !ids_out)))
        return LORA_E_ARG;
    follow_stack(m);
    // the batch's distinct adapters, in order of first use; checked before any change
    std::vector<int64_t> distinct;
    std::unordered_map<int64_t, int> seen;
    for (int64_t i = 0; i < n_rows; ++i) {
        const int64_t id = row_adapter[i];
        if (id == -1)
            continue;
        if (id < 0)
            return LORA_E_ARG;
        if (seen.emplace(id, 1).second) {
            if (!m->host.count(id))
                return LORA_E_NOT_FOUND;
            distinct.push_back(id);
        }
    }
    int usable = 0;
    for (int64_t a : m->slot_adapter)
        usable += a != -2;
    if ((int)distinct.size() > usable)
        return LORA_E_CAPACITY;

    const uint64_t now = ++m->tick;
    for (int64_t id : distinct) {
        HostEntry &e = m->host.at(id);
        e.last = now;
        if (e.slot >= 0)
            m->stats[LORA_RES_HITS] += 1;
    }
    std::vector<std::pair<int, int64_t>> todo;   // (slot, adapter) to load
    for (int64_t id : distinct) {
        HostEntry &e = m->host.at(id);
        if (e.slot >= 0)
            continue;
        // an empty slot (lowest index), else the least recently used slot
        // whose adapter this batch does not use (ties: lowest index)
        int slot = -1;
        for (int sl = 0; sl < m->n_slots && slot < 0; ++sl)
            if (m->slot_adapter[sl] == -1)
                slot = sl;
        if (slot < 0) {
            uint64_t best = 0;
            for (int sl = 0; sl < m->n_slots; ++sl) {
                const int64_t a = m->slot_adapter[sl];
                if (a < 0 || seen.count(a))
                    continue;
                const uint64_t last = m->host.at(a).last;
                if (slot < 0 || last < best) {
                    slot = sl;
                    best = last;
                }
            }
            displace(m, slot);
            if (m->st)
                m->st->h_rank[slot] = 0;
        }
        m->slot_adapter[slot] = id;   // taken: not handed out twice in this batch
        todo.emplace_back(slot, id);
    }
    const lora_status rc = load_all(m, todo, stream);
    if (rc != LORA_OK)
        return rc;
    for (int64_t i = 0; i < n_rows; ++i) {
        const int64_t id = row_adapter[i];
        ids_out[i] = id == -1 ? -1 : m->host.at(id).slot;
    }
    return LORA_OK;
}

lora_status lora_residency_slot_of(const lora_residency *m, int64_t adapter_id, int *slot)
{
    if (!m || !slot)
        return LORA_E_ARG;
    auto it = m->host.find(adapter_id);
    if (it == m->host.end())
        return LORA_E_NOT_FOUND;
    *slot = it->second.slot;
    return LORA_OK;
}

lora_status lora_residency_stats(const lora_residency *m, int64_t *stats)
{
    if (!m || !stats)
        return LORA_E_ARG;
    for (int i = 0; i < LORA_RES_NSTATS; ++i)
        stats[i] = m->stats[i];
    stats[LORA_RES_HOST_ENTRIES] = (int64_t)m->host.size();
    int res = 0;
    for (int64_t a : m->slot_adapter)
        res += a >= 0;
    stats[LORA_RES_RESIDENT] = res;
    return LORA_OK;
}

}  // extern "C"
