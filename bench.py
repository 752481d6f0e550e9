"""Benchmark of one multi-adapter LoRA layer step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is the whole hot path over one batch, one lora_build_apply call: group
the rows by adapter, shrink (v = A x), expand (y += scale B v).  Decode-sized
batches run it as one kernel (decode_kernel, or build_apply_kernel for shapes
the decode kernel does not serve); other batches of up to 1024 rows take two
(grouping fused into the shrink, then the expand), larger ones three or five
(grouping, shrink, expand).
Inputs are resident in HBM before the timed region.  Steps rotate through
independent buffer sets (stack + ids + x + y) totalling >= 512 MB so that the
256 MB MALL cannot serve them: every step reads its weights and rows from HBM.

One JSON line goes to stdout:
  value      LoRA-applied tokens/s (valid rows per second over the timed steps)
  roofline   the dominant kernel's algorithmic bytes per launch over its mean
             launch duration (that kernel launched K times back to back on the
             rotating sets, HIP events on the launch stream), against the
             8 TB/s HBM peak and against the achievable ceiling (a plain copy
             kernel moving the same bytes in one launch, timed in the same run:
             ceiling_gbs, frac_of_ceiling); traffic = HBM bytes per launch from
             rocprofv3 FETCH_SIZE/WRITE_SIZE (scaled by a copy-kernel
             calibration) when the committed measurement for the workload
             (profiles/traffic.json) matches the current kernel sources, else null
  cpu_baseline  the CPU oracle on the host cores on a bounded sample

Other modes: --all (every workload, lines to --out); --merge (lora_merge_slot
on named projections, one line each); --sweep (adapter count x rank against the
base GEMM of the same layer); --residency (adapter load bandwidth from the
pinned host tier, decode steps under Zipf adapter churn); --copy-probe (plain copy
kernel at each workload's step size and at 2 GiB: the achievable HBM ceiling);
--copy-calib MB (a plain copy of known size, the calibration run for the PMC
byte counters); --pmc-summary (fold two rocprofv3 --pmc runs and their
calibration runs into bytes per launch; --traffic-update stores them as the
workload's entry of profiles/traffic.json).
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
ROTATE_BYTES = 512 << 20       # 2x the 256 MB MALL
DEFAULT_WORKLOAD = "decode_bgmv"
KERNEL_SOURCES = ("seg_build.hip", "shrink.hip", "expand.hip", "expand_tiles.h", "group.h",
                  "mfma.h", "device_common.h", "internal.h", "decode.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ----------------------------------------------------------------- accounting

def accounting(p) -> dict:
    """Algorithmic bytes and flops of one step (what the method must move):
    each valid row's x read once, each valid row's y read and written once, the
    live A and B of every slot the batch references read once at true rank."""
    b = p.elem_bytes
    ok = np.array([0 <= s < p.n_slots and p.ranks[s] > 0 for s in p.ids], bool)
    n_valid = int(ok.sum())
    slots = np.unique(p.ids[ok])
    live_a = sum(int(p.ranks[s]) * p.n_slices * p.k for s in slots) * b
    live_b = sum(int(p.ranks[s]) * p.D for s in slots) * b
    x_bytes = n_valid * p.k * b
    y_bytes = 2 * n_valid * p.D * b
    flops = sum(2 * int(p.ranks[s]) * (p.n_slices * p.k + p.D) + p.D for s in p.ids[ok])
    shrink_flops = sum(2 * int(p.ranks[s]) * p.n_slices * p.k for s in p.ids[ok])
    # ids, the slot table and the grouping's outputs are metadata and are not
    # counted (seg_build alone is priced by its ids and segments bytes)
    return dict(n_valid=n_valid, distinct_slots=int(slots.size),
                bytes=dict(shrink=x_bytes + live_a, expand=y_bytes + live_b,
                           seg_build=8 * p.n_rows + 4 * (p.n_slots + 1),
                           build_shrink=x_bytes + live_a,
                           build_apply=x_bytes + y_bytes + live_a + live_b,
                           apply=x_bytes + y_bytes + live_a + live_b,
                           total=x_bytes + y_bytes + live_a + live_b),
                flops=dict(total=int(flops), shrink=int(shrink_flops), build_apply=int(flops),
                           apply=int(flops),
                           build_shrink=int(shrink_flops), expand=int(flops - shrink_flops)))


# what each launch count of lora_build_apply (lora_build_apply_plan) runs
STEP_KERNELS = {1: ("build_apply",), 2: ("build_shrink", "expand"),
                3: ("seg_build", "shrink", "expand"), 5: ("seg_build", "shrink", "expand")}


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "rank_adapter_gemm_lora_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def committed_traffic(workload: str):
    """HBM bytes per launch of this workload's kernels from the committed
    counter summary (one entry per workload), if the entry was taken on the
    current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f).get(workload)
    except (OSError, ValueError, AttributeError):
        return None
    if not t or t.get("kernel_sources") != kernel_source_hash():
        return None
    return t


# ----------------------------------------------------------------- GPU side

class BufferSet:
    """One independent copy of the stack, ids, x and y of a workload."""

    def __init__(self, p, lb, torch, dev, stream, dA, dB, dense_min, expand_chunks=None):
        dt = lb.LORA_BF16 if p.dtype == "bf16" else lb.LORA_F32
        self.stack = lb.lora_stack_create(dt, p.n_slots, p.r_max, p.k, p.slice_d, p.n_rows)
        self.seg = lb.lora_segments_create(p.n_rows, p.n_slots)
        if dense_min is not None:
            lb.lora_segments_set_dense_min(self.seg, dense_min)
        if expand_chunks is not None:
            lb.lora_segments_set_expand_chunks(self.seg, expand_chunks)
        for s in range(p.n_slots):
            if p.ranks[s] > 0:
                lb.lora_load_slot(self.stack, s, int(p.ranks[s]), float(p.alphas[s]),
                                  dA[s].data_ptr(), dB[s].data_ptr(), False, stream)
        raw = torch.int16 if p.dtype == "bf16" else torch.float32
        self.ids = torch.from_numpy(p.ids).to(dev)
        self.x = torch.from_numpy(p.x.view(np.int16) if p.dtype == "bf16" else p.x).to(dev)
        self.y = torch.from_numpy(p.y.view(np.int16) if p.dtype == "bf16" else p.y).to(dev)
        assert self.x.dtype == raw and self.y.dtype == raw

    def close(self, lb):
        lb.lora_segments_destroy(self.seg)
        lb.lora_stack_destroy(self.stack)


def set_bytes(p) -> int:
    b = p.elem_bytes
    rp = (p.r_max + 7) // 8 * 8
    pool = p.n_slots * (p.n_slices * p.r_max * p.k + p.D * rp) * b
    return pool + p.x.nbytes + p.y.nbytes + p.ids.nbytes


def run_gpu(p, steps: int, warmup: int, rotate: bool = True, dense_min=None, expand_chunks=None,
            graph: bool = True) -> dict:
    import torch
    from rank_adapter_gemm_lora_amd import binding as lb

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream(dev)        # default priority
    sh = stream.cuda_stream
    raw = (lambda a: a.view(np.int16)) if p.dtype == "bf16" else (lambda a: a)
    dA = [None if p.ranks[s] == 0 else torch.from_numpy(raw(np.ascontiguousarray(p.A[s]))).to(dev)
          for s in range(p.n_slots)]
    dB = [None if p.ranks[s] == 0 else torch.from_numpy(raw(np.ascontiguousarray(p.B[s]))).to(dev)
          for s in range(p.n_slots)]
    torch.cuda.synchronize()               # staged weights complete before other streams read them
    n_sets = max(2, math.ceil(ROTATE_BYTES / set_bytes(p))) if rotate else 1
    n_sets = min(n_sets, 4096)
    with torch.cuda.stream(stream):
        sets = [BufferSet(p, lb, torch, dev, sh, dA, dB, dense_min, expand_chunks)
                for _ in range(n_sets)]
    torch.cuda.synchronize()
    del dA, dB

    def build(bs):
        lb.lora_build_segments(bs.stack, bs.ids.data_ptr(), p.n_rows, bs.seg, sh)

    def shrink(bs):
        lb.lora_add_shrink(bs.stack, bs.x.data_ptr(), p.ldx, bs.seg, sh)

    def build_shrink(bs):
        lb.lora_build_shrink(bs.stack, bs.x.data_ptr(), p.ldx, bs.ids.data_ptr(), p.n_rows,
                             bs.seg, sh)

    def expand(bs):
        lb.lora_add_expand(bs.stack, bs.y.data_ptr(), p.ldy, bs.seg, sh)

    def apply(bs):
        lb.lora_apply(bs.stack, bs.y.data_ptr(), p.ldy, bs.x.data_ptr(), p.ldx, bs.seg, sh)

    def step(bs):
        lb.lora_build_apply(bs.stack, bs.y.data_ptr(), p.ldy, bs.x.data_ptr(), p.ldx,
                            bs.ids.data_ptr(), p.n_rows, bs.seg, sh)

    for i in range(warmup):
        step(sets[i % n_sets])
    torch.cuda.synchronize()

    # the step: K passes of the whole path, one buffer set each, events only
    # around the region
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        step(sets[(warmup + i) % n_sets])
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = start.elapsed_time(stop)

    # each kernel alone: K back-to-back launches over the rotating sets (every
    # set already holds its segments and v, so each launch does its full work);
    # mean launch duration = region time / K, events only at the region's ends.
    # The split path's grouping and shrink are timed too, for comparison.
    # With a one-launch step, the two-launch path's kernels (build_shrink,
    # expand) are timed for comparison as well.
    # lora_apply on the grouped sets ("apply": one launch or shrink + expand) is
    # timed as well: the call a model makes per projection after one grouping.
    fns = dict(seg_build=build, shrink=shrink, build_shrink=build_shrink, expand=expand,
               build_apply=step, apply=apply)
    n_launch = lb.lora_build_apply_plan(sets[0].stack, p.n_rows, sets[0].seg)
    step_k = STEP_KERNELS[n_launch]
    extra = ("build_shrink", "expand", "seg_build", "shrink", "apply") if n_launch == 1 else \
        ("seg_build", "shrink", "apply")
    names = list(step_k) + [k for k in extra if k not in step_k]
    per = {}
    for name in names:
        fn = fns[name]
        for i in range(min(warmup, n_sets)):
            fn(sets[i % n_sets])
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(steps):
            fn(sets[i % n_sets])
        e1.record(stream)
        torch.cuda.synchronize()
        per[name] = e0.elapsed_time(e1) * 1e3 / steps
    # the same step replayed from HIP graphs (one captured per buffer set): the
    # launch shapes depend only on the batch shape, so a graph serves any mix
    graph_ms = graph_chain_ms = None
    if graph:
        graphs = []
        for bs in sets:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                step(bs)
            graphs.append(g)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            # every graph replayed once (a graph's first replay costs more),
            # then the warm-up count
            for i in range(n_sets + warmup):
                graphs[i % n_sets].replay()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(steps):
                graphs[(warmup + i) % n_sets].replay()
            e1.record(stream)
        torch.cuda.synchronize()
        graph_ms = e0.elapsed_time(e1) / steps
        del graphs
        # one graph holding a pass over every buffer set (one step each), as a
        # serving loop captures many layers per graph: the graph launch cost is
        # shared by the steps it holds
        chain = torch.cuda.CUDAGraph()
        with torch.cuda.graph(chain, stream=stream):
            for bs in sets:
                step(bs)
        torch.cuda.synchronize()
        reps = max(2, steps // n_sets)
        with torch.cuda.stream(stream):
            chain.replay()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(reps):
                chain.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        graph_chain_ms = e0.elapsed_time(e1) / (reps * n_sets)
        del chain
    n_bgmv, n_sgmv = lb.lora_segments_tile_counts(sets[0].seg, sh)
    for bs in sets:
        bs.close(lb)
    torch.cuda.synchronize()
    return dict(wall_s=wall, gpu_ms=gpu_ms, n_sets=n_sets, set_bytes=set_bytes(p),
                kernel_us=per, step_kernels=step_k, tiles=dict(bgmv=n_bgmv, sgmv=n_sgmv),
                graph_ms=graph_ms,
                graph_chain_ms=graph_chain_ms)


# ----------------------------------------------------------------- CPU oracle

def host_cpu() -> dict:
    """The host's CPU model and core counts: threads this process may run on
    (its affinity mask) and CPUs online (os.cpu_count)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        visible = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        visible = os.cpu_count() or 1
    return dict(model=model, cores_visible=visible, cpus_online=os.cpu_count() or 1)


def run_cpu_baseline(p, acct, budget_s: float = 10.0, budget_1t_s: float = 3.0) -> dict:
    """The oracle as it stands: OpenMP over rows on up to 16 host threads for
    ~budget_s, then one thread for ~budget_1t_s; full passes of the batch."""
    import oracle
    threads = max(1, min(16, host_cpu()["cores_visible"]))
    ranks = p.ranks

    def passes(n_threads, budget):
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.build_segments(p.ids, p.n_slots, ranks)
            oracle.apply_rows(p.dtype, p.k, p.slice_d, ranks, p.alphas, p.A, p.B, p.ids, p.x, p.y,
                              n_threads=n_threads)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return reps, el

    reps, el = passes(threads, budget_s)
    reps1, el1 = passes(1, budget_1t_s)
    host = host_cpu()
    return dict(value=acct["n_valid"] * reps / el, unit="tokens/s", cores=threads, kind="oracle",
                host_cores_visible=host["cores_visible"], host_cpus_online=host["cpus_online"],
                cpu_model=host["model"],
                sample=f"{reps} full passes of the {p.name} batch ({p.n_rows} rows, "
                       f"{acct['n_valid']} with an adapter): segments + fp64 apply, "
                       f"{el:.1f} s, OpenMP over rows",
                value_1_thread=acct["n_valid"] * reps1 / el1)


# ----------------------------------------------------------------- modes

def bench_workload(name, steps, warmup, rotate=True, cpu=True, dense_min=None,
                   expand_chunks=None) -> dict:
    from rank_adapter_gemm_lora_amd import synth
    p = synth.make_workload(name)
    acct = accounting(p)
    log(f"[bench] {name}: {p.note}; valid rows {acct['n_valid']}, "
        f"algorithmic bytes {acct['bytes']['total'] / 1e6:.2f} MB/step")
    g = run_gpu(p, steps, warmup, rotate=rotate, dense_min=dense_min, expand_chunks=expand_chunks)
    # the same step on one buffer set, cache-resident (MALL / L2 served, not HBM)
    warm = run_gpu(p, steps, warmup, rotate=False, dense_min=dense_min, expand_chunks=expand_chunks,
                   graph=False) if rotate else g
    ms = g["gpu_ms"] / steps
    ku = g["kernel_us"]
    dom = max(g["step_kernels"], key=lambda k: ku[k])
    achieved = acct["bytes"][dom] / (ku[dom] * 1e-6) / 1e9
    traffic = committed_traffic(name)
    # the achievable ceiling: a plain copy moving the same bytes in one launch
    ceil = copy_probe((acct["bytes"][dom],), reps=max(20, steps))[0]
    roof = dict(kernel=dom, bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS,
                unit="GB/s", frac=round(achieved / HBM_PEAK_GBS, 4),
                traffic=(traffic["per_launch_bytes"].get(dom) if traffic else None),
                algorithmic_bytes_per_launch=acct["bytes"][dom],
                mean_launch_us=round(ku[dom], 3),
                ceiling_gbs=ceil["gbs"], frac_of_ceiling=round(achieved / ceil["gbs"], 4),
                ceiling_note=f"plain device copy moving {ceil['bytes_moved']} bytes per launch "
                             f"(HBM-cold rotation), {ceil['mean_us']} us")
    line = {
        "metric": "LoRA-applied tokens/s per layer + achieved HBM GB/s (% of MI355X peak)",
        "value": round(acct["n_valid"] * steps / (g["gpu_ms"] * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": p.dtype, "data": "synthetic (seeded, HBM-cold rotation)" if rotate else
        "synthetic (seeded, warm: cache-served, not HBM)",
        "config": {"workload": name, "rows": p.n_rows, "valid_rows": acct["n_valid"],
                   "k": p.k, "slices": p.slice_d, "slots": p.n_slots, "r_max": p.r_max,
                   "ranks": sorted({int(r) for r in p.ranks if r > 0}),
                   "distinct_slots": acct["distinct_slots"], "buffer_sets": g["n_sets"],
                   "parallelism": "single GPU"},
        "step_hbm_gbs": round(acct["bytes"]["total"] / (ms * 1e-3) / 1e9, 1),
        "step_hbm_frac": round(acct["bytes"]["total"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "step_kernels": list(g["step_kernels"]),
        "kernel_us": {k: round(v, 3) for k, v in ku.items()},
        "kernel_gbs": {k: round(acct["bytes"][k] / (ku[k] * 1e-6) / 1e9, 1)
                       for k in ku if k != "seg_build"},
        "mfma_util": {k: round(acct["flops"][k] / (ku[k] * 1e-6) / 1e12
                               / MFMA_BF16_PEAK_TFLOPS, 5) for k in ku if k != "seg_build"},
        "tiles": g["tiles"],
        "roofline": roof,
        "host_wall_ms_per_step": round(g["wall_s"] * 1e3 / steps, 4),
        "warm_ms_per_step": round(warm["gpu_ms"] / steps, 5),
        "warm_note": "one buffer set, cache-served (not HBM)",
        "graph_ms_per_step": (round(g["graph_ms"], 5) if g["graph_ms"] is not None else None),
        "graph_tokens_per_s": (round(acct["n_valid"] / (g["graph_ms"] * 1e-3), 1)
                               if g["graph_ms"] is not None else None),
        "graph_chain_ms_per_step": (round(g["graph_chain_ms"], 5)
                                    if g["graph_chain_ms"] is not None else None),
        "graph_chain_steps": g["n_sets"] if g["graph_chain_ms"] is not None else None,
    }
    if cpu:
        line["cpu_baseline"] = run_cpu_baseline(p, acct)
    return line


MERGE_CASES = {
    # name: (k, slice widths, rank)
    "merge_q_proj_r16": (4096, [4096], 16),
    "merge_q_proj_r64": (4096, [4096], 64),
    "merge_q_proj_r128": (4096, [4096], 128),
    "merge_fused_qkv_r16": (4096, [4096, 1024, 1024], 16),
    "merge_gate_up_r64": (4096, [14336, 14336], 64),
}


def bench_merge(name, steps, warmup, cpu=True) -> dict:
    """lora_merge_slot on bf16 weights of a named projection: each call reads
    and writes the whole weight once (plus the slot's factors).  Calls alternate
    merge and unmerge over weight copies totalling >= 512 MB (HBM-cold)."""
    import torch
    from rank_adapter_gemm_lora_amd import binding as lb
    from rank_adapter_gemm_lora_amd import synth

    k, slice_d, rank = MERGE_CASES[name]
    D = sum(slice_d)
    p = synth.make_random(0, n_rows=1, k=k, slice_d=slice_d, n_slots=1, ranks=[rank],
                          r_max=rank, dtype="bf16")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream(dev)
    sh = stream.cuda_stream
    w_bytes = D * k * 2
    n_w = max(2, math.ceil(ROTATE_BYTES / w_bytes))
    W0 = torch.from_numpy(synth.make_base_weight(1, D, k, "bf16").view(np.int16)).to(dev)
    Ws = [W0.clone() for _ in range(n_w)]
    del W0
    dA = torch.from_numpy(np.ascontiguousarray(p.A[0]).view(np.int16)).to(dev)
    dB = torch.from_numpy(np.ascontiguousarray(p.B[0]).view(np.int16)).to(dev)
    torch.cuda.synchronize()
    st = lb.lora_stack_create(lb.LORA_BF16, 1, rank, k, slice_d, 1)
    lb.lora_load_slot(st, 0, rank, 32.0, dA.data_ptr(), dB.data_ptr(), False, sh)

    def call(i):
        lb.lora_merge_slot(st, 0, Ws[i % n_w].data_ptr(), k, 1 if (i // n_w) % 2 == 0 else -1, sh)

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        call(warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    lb.lora_stack_destroy(st)
    rp = (rank + 7) // 8 * 8
    byts = 2 * w_bytes + (len(slice_d) * rank * k + D * rp) * 2
    flops = 2 * D * k * rank
    gbs = byts / (us * 1e-6) / 1e9
    line = {
        "metric": "merge: weight bytes moved per second (read + write) by lora_merge_slot",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "us_per_merge": round(us, 3), "higher_is_better": True, "dtype": "bf16",
        "data": "synthetic (seeded, HBM-cold rotation)",
        "config": {"workload": name, "k": k, "slices": slice_d, "rank": rank,
                   "weight_copies": n_w},
        "roofline": {"kernel": "merge_bf16_kernel", "bound": "hbm", "achieved": round(gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": None, "algorithmic_bytes_per_launch": byts,
                     "mean_launch_us": round(us, 3)},
        "mfma_util": round(flops / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 5),
    }
    if cpu:
        import oracle
        threads = max(1, min(16, os.cpu_count() or 1))
        n_rows = min(D, 256)
        Wh = synth.make_base_weight(1, D, k, "bf16")
        reps, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 5.0:
            oracle.merge("bf16", k, [n_rows], rank, 32.0, p.A[0][:1], p.B[0][:n_rows], Wh[:n_rows],
                         1, n_threads=threads)
            reps += 1
        el = time.perf_counter() - t0
        cpu_bytes = (2 * n_rows * k + rank * k + n_rows * rp) * 2
        line["cpu_baseline"] = {"value": round(cpu_bytes * reps / el / 1e9, 3), "unit": "GB/s",
                                "cores": threads, "kind": "oracle",
                                "sample": f"{reps} oracle merges of the first {n_rows} rows "
                                          f"of slice 0 in {el:.1f} s"}
    return line


SWEEP_ADAPTERS = (1, 4, 16, 100)
SWEEP_RANKS = (8, 16, 32, 64, 128)
SWEEP_ROWS = (256, 4096)
SWEEP_K = 4096


def sweep_problem(n_rows, n_adapters, rank, seed=0):
    """q-proj 4096 -> 4096, bf16, every row routed, ids uniform over the adapters."""
    from rank_adapter_gemm_lora_amd import synth
    return synth.make_random(seed, n_rows=n_rows, k=SWEEP_K, slice_d=[SWEEP_K], n_slots=n_adapters,
                             ranks=[rank] * n_adapters, r_max=rank, dtype="bf16", alpha=32.0,
                             name=f"sweep_n{n_rows}_a{n_adapters}_r{rank}")


def time_base_gemm(n_rows, steps, warmup) -> float:
    """Mean time (us) of the shared base projection y = x W^T (torch's GEMM,
    bf16, 4096 x 4096) over W and x copies totalling >= 512 MB."""
    import torch
    from rank_adapter_gemm_lora_amd import synth
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(dev)
    w = torch.from_numpy(synth.make_base_weight(3, SWEEP_K, SWEEP_K, "bf16").view(np.int16))
    w = w.to(dev).view(torch.bfloat16)
    x = torch.randn((n_rows, SWEEP_K), generator=torch.Generator().manual_seed(5)).to(dev)
    x = x.to(torch.bfloat16)
    per = w.numel() * 2 + x.numel() * 2 + n_rows * SWEEP_K * 2
    n = max(2, math.ceil(ROTATE_BYTES / per))
    ws = [w.clone() for _ in range(n)]
    xs = [x.clone() for _ in range(n)]
    ys = [torch.empty((n_rows, SWEEP_K), dtype=torch.bfloat16, device=dev) for _ in range(n)]
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for i in range(warmup):
            torch.matmul(xs[i % n], ws[i % n].t(), out=ys[i % n])
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            torch.matmul(xs[i % n], ws[i % n].t(), out=ys[i % n])
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / steps


def bench_sweep(steps, warmup, out=None, md=None) -> list:
    """Adapter count x rank sweep of one q-proj LoRA layer (lora_build_apply,
    HBM-cold rotation) against the base GEMM of the same layer on the same GPU."""
    lines = []
    for n_rows in SWEEP_ROWS:
        base_us = time_base_gemm(n_rows, steps, warmup)
        log(f"[sweep] base GEMM n={n_rows}: {base_us:.2f} us")
        for n_ad in SWEEP_ADAPTERS:
            for rank in SWEEP_RANKS:
                p = sweep_problem(n_rows, n_ad, rank)
                acct = accounting(p)
                g = run_gpu(p, steps, warmup, rotate=True, graph=False)
                us = g["gpu_ms"] * 1e3 / steps
                line = {"metric": "sweep: one LoRA q-proj layer vs its base GEMM",
                        "config": {"workload": p.name, "rows": n_rows, "adapters": n_ad,
                                   "rank": rank, "k": SWEEP_K, "d": SWEEP_K},
                        "lora_us": round(us, 3), "base_gemm_us": round(base_us, 3),
                        "relative_throughput": round(base_us / (base_us + us), 4),
                        "lora_hbm_gbs": round(acct["bytes"]["total"] / (us * 1e-6) / 1e9, 1),
                        "distinct_slots": acct["distinct_slots"],
                        "kernel_us": {k: round(v, 3) for k, v in g["kernel_us"].items()},
                        "tiles": g["tiles"]}
                lines.append(line)
                emit(line, out)
    if md:
        with open(md, "w") as f:
            f.write("# One q-proj LoRA layer against its base GEMM (MI355X, bf16, HBM-cold rotation)\n\n"
                    f"Command: `python3 bench.py --sweep --steps {steps} --warmup {warmup} --sweep-md <file>`\n"
                    "(LoRA step = one lora_build_apply; base = torch's bf16 GEMM of the same shape)\n")
            f.write(sweep_markdown(lines))
    return lines


def sweep_markdown(lines) -> str:
    rows = sorted({l["config"]["rows"] for l in lines})
    out = []
    for n in rows:
        sel = [l for l in lines if l["config"]["rows"] == n]
        base = sel[0]["base_gemm_us"]
        out.append(f"\n### {n} rows, q-proj 4096 -> 4096 bf16; base GEMM {base:.2f} us\n")
        out.append("LoRA step time in us (relative throughput base / (base + LoRA)):\n")
        ranks = sorted({l["config"]["rank"] for l in sel})
        out.append("| adapters | " + " | ".join(f"r={r}" for r in ranks) + " |")
        out.append("|---|" + "---|" * len(ranks))
        for a in sorted({l["config"]["adapters"] for l in sel}):
            cells = []
            for r in ranks:
                l = next(l for l in sel if l["config"]["adapters"] == a and l["config"]["rank"] == r)
                cells.append(f"{l['lora_us']:.1f} ({l['relative_throughput'] * 100:.0f}%)")
            out.append(f"| {a} | " + " | ".join(cells) + " |")
    return "\n".join(out) + "\n"


def bench_residency(steps, warmup, out=None) -> list:
    """Adapter residency on the decode projection (4096 -> 4096, bf16, rank 16,
    16 GPU slots, 200 registered adapters in the pinned host tier):
    (1) host -> HBM load bandwidth: batches of 16 adapters none of which is
        resident, so every map_batch call loads 16 adapters (GPU time of the
        copies, HIP events on the stream);
    (2) decode steps under Zipf(1.1) adapter churn: each step maps a batch of
        256 rows over 16 adapters drawn Zipf without replacement, then runs
        lora_build_apply; mean step time, hit rate and loads per step against
        the same steps with every adapter already resident."""
    import torch
    from rank_adapter_gemm_lora_amd import binding as lb
    from rank_adapter_gemm_lora_amd import synth

    k, D, rank, n_slots, n_ad, n_rows = 4096, 4096, 16, 16, 200, 256
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream(dev)
    sh = stream.cuda_stream
    rng = np.random.default_rng(0)
    st = lb.lora_stack_create(lb.LORA_BF16, n_slots, rank, k, [D], n_rows)
    seg = lb.lora_segments_create(n_rows, n_slots)
    m = lb.lora_residency_create(st, n_ad)
    ad_bytes = rank * (k + D) * 2
    for aid in range(n_ad):
        A = synth.f32_to_bf16_bits(rng.standard_normal((1, rank, k), dtype=np.float32) * 0.02)
        B = synth.f32_to_bf16_bits(rng.standard_normal((D, rank), dtype=np.float32) * 0.02)
        lb.lora_residency_register(m, aid, rank, 32.0, A.ctypes.data, B.ctypes.data)
    lines = []

    # (1) cold loads: 16 fresh adapters per call
    groups = [list(range(i, i + n_slots)) for i in range(0, n_ad - n_slots + 1, n_slots)]
    for g in groups[:2]:
        lb.lora_residency_map_batch(m, g, sh)
    torch.cuda.synchronize()
    s0 = lb.lora_residency_stats(m)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    calls = 0
    for rep in range(max(1, steps // len(groups))):
        for g in groups[2:] + groups[:2]:
            lb.lora_residency_map_batch(m, g, sh)
            calls += 1
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    s1 = lb.lora_residency_stats(m)
    loads = s1["loads"] - s0["loads"]
    byts = s1["bytes_loaded"] - s0["bytes_loaded"]
    gpu_s = e0.elapsed_time(e1) * 1e-3
    line = {"metric": "residency: adapter load bandwidth, pinned host tier -> HBM",
            "value": round(byts / gpu_s / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
            "loads": loads, "bytes_per_load": ad_bytes, "us_per_load": round(gpu_s * 1e6 / loads, 2),
            "host_wall_us_per_load": round(wall * 1e6 / loads, 2), "map_calls": calls,
            "config": {"workload": "residency_cold_loads", "k": k, "d": D, "rank": rank,
                       "slots": n_slots, "registered": n_ad}}
    lines.append(line)
    emit(line, out)

    # (2) Zipf churn vs all-resident steps
    x = torch.from_numpy(synth._normal(rng, (n_rows, k), 1.0, "bf16").view(np.int16)).to(dev)
    y = torch.from_numpy(synth._normal(rng, (n_rows, D), 1.0, "bf16").view(np.int16)).to(dev)
    p = synth.zipf_probs(n_ad, 1.1)
    batches = []
    for _ in range(steps):
        use = rng.choice(n_ad, size=n_slots, replace=False, p=p)
        batches.append(rng.choice(use, size=n_rows).astype(np.int64))
    ids_dev = torch.empty(n_rows, dtype=torch.int32, device=dev)
    pinned = torch.empty(n_rows, dtype=torch.int32, pin_memory=True)

    def step(rows):
        ids = lb.lora_residency_map_batch(m, rows, sh)
        pinned.numpy()[:] = ids
        with torch.cuda.stream(stream):
            ids_dev.copy_(pinned, non_blocking=True)
        lb.lora_build_apply(st, y.data_ptr(), D, x.data_ptr(), k, ids_dev.data_ptr(), n_rows, seg, sh)
        stream.synchronize()   # the pinned staging buffer is reused by the next step

    for rows in batches[:warmup]:
        step(rows)
    s0 = lb.lora_residency_stats(m)
    t0 = time.perf_counter()
    for rows in batches:
        step(rows)
    churn = (time.perf_counter() - t0) / len(batches)
    s1 = lb.lora_residency_stats(m)
    # the same loop with one fixed resident set: no loads
    hot = batches[0]
    step(hot)
    t0 = time.perf_counter()
    for _ in batches:
        step(hot)
    resident = (time.perf_counter() - t0) / len(batches)
    uses = (s1["hits"] - s0["hits"]) + (s1["loads"] - s0["loads"])
    line = {"metric": "residency: decode step under Zipf(1.1) adapter churn (host wall, map + upload + apply)",
            "value": round(churn * 1e6, 2), "unit": "us/step", "higher_is_better": False,
            "n_gpus": 1, "steps": len(batches),
            "all_resident_us_per_step": round(resident * 1e6, 2),
            "hit_rate": round((s1["hits"] - s0["hits"]) / max(1, uses), 4),
            "loads_per_step": round((s1["loads"] - s0["loads"]) / len(batches), 3),
            "config": {"workload": "residency_zipf_churn", "rows": n_rows, "k": k, "d": D,
                       "rank": rank, "slots": n_slots, "registered": n_ad,
                       "adapters_per_batch": n_slots}}
    lines.append(line)
    emit(line, out)
    torch.cuda.synchronize()
    lb.lora_residency_destroy(m)
    lb.lora_segments_destroy(seg)
    lb.lora_stack_destroy(st)
    return lines


def copy_probe(moved=(7_626_752, 2 << 30), reps: int = 50) -> list:
    """A plain device copy (torch's copy kernel) moving each of ``moved`` bytes
    per launch (half read, half written), rotated over buffers totalling
    >= 512 MB so the MALL cannot serve them: the achievable HBM rate of one
    streaming launch of that size, launch overhead included, to set beside the
    8 TB/s paper peak."""
    import torch
    dev = torch.device("cuda:0")
    out = []
    for total in moved:
        nbytes = max(256, total // 2 // 256 * 256)
        n_buf = max(2, math.ceil(ROTATE_BYTES / (2 * nbytes)))
        src = [torch.empty(nbytes // 2, dtype=torch.int16, device=dev).fill_(1) for _ in range(n_buf)]
        dst = [torch.empty_like(s) for s in src]
        for i in range(n_buf + 5):
            dst[i % n_buf].copy_(src[i % n_buf])
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            dst[i % n_buf].copy_(src[i % n_buf])
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        out.append(dict(bytes_moved=2 * nbytes, mean_us=round(us, 3),
                        gbs=round(2 * nbytes / (us * 1e-6) / 1e9, 1)))
        del src, dst
        torch.cuda.empty_cache()
    return out


def copy_calibration(mbytes: int, reps: int = 20):
    """A plain device copy of ``mbytes`` MB, ``reps`` times: the calibration
    kernel for the PMC byte counters (it reads and writes exactly that much)."""
    import torch
    dev = torch.device("cuda:0")
    n = (mbytes << 20) // 2
    src = torch.ones(n, dtype=torch.int16, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()


def _counter_per_dispatch(d: str, counter: str) -> dict:
    """Median value of ``counter`` per dispatch, by kernel name, from a
    rocprofv3 --pmc output directory (csv)."""
    import csv
    vals = {}
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                key = (row["Kernel_Name"], row.get("Dispatch_Id", row.get("Correlation_Id", "")))
                vals.setdefault(row["Kernel_Name"], {}).setdefault(key[1], 0.0)
                vals[row["Kernel_Name"]][key[1]] += float(row["Counter_Value"])
    return {k: float(np.median(list(v.values()))) for k, v in vals.items()}


def pmc_summary(fetch_dir, write_dir, cal_fetch_dir, cal_write_dir, copy_mb, workload) -> dict:
    """HBM bytes per launch of each kernel from two rocprofv3 --pmc runs
    (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each scaled by what the
    same counter reads for a plain copy of copy_mb MB (read copy_mb, wrote copy_mb)."""
    fetch = _counter_per_dispatch(fetch_dir, "FETCH_SIZE")
    write = _counter_per_dispatch(write_dir, "WRITE_SIZE")
    cf = _counter_per_dispatch(cal_fetch_dir, "FETCH_SIZE")
    cw = _counter_per_dispatch(cal_write_dir, "WRITE_SIZE")
    copy_bytes = copy_mb << 20

    def biggest(d):
        return max(d.values()) if d else None

    f_scale = copy_bytes / (biggest(cf) * 1024.0) if cf else None
    w_scale = copy_bytes / (biggest(cw) * 1024.0) if cw else None
    # kernel functions behind each timed name (the grouping has a small-batch
    # and a chunked variant)
    names = {"seg_build": ("seg_build_kernel", "seg_build_small_kernel"),
             "shrink": ("shrink_kernel", "shrink_kernel_tall"),
             "build_shrink": ("build_shrink_kernel",),
             "build_apply": ("decode_kernel", "build_apply_kernel"),
             "apply": ("apply_kernel",),
             "expand": ("expand_kernel", "expand_kernel_bf16_short", "expand_stream_kernel",
                        "expand_run_kernel")}

    def bare(kname):
        head = kname.replace("(anonymous namespace)", "").split("(")[0].split("<")[0]
        return head.split("::")[-1].strip()

    per, raw = {}, {}
    for k, keys in names.items():
        fb = next((v for n, v in fetch.items() if bare(n) in keys), None)
        wb = next((v for n, v in write.items() if bare(n) in keys), None)
        if fb is None and wb is None:
            continue
        raw[k] = {"fetch_kib": fb, "write_kib": wb}
        if fb is None or wb is None or f_scale is None or w_scale is None:
            per[k] = None
        else:
            per[k] = int(round(fb * 1024.0 * f_scale + wb * 1024.0 * w_scale))
    return dict(workload=workload, kernel_sources=kernel_source_hash(), copy_mb=copy_mb,
                fetch_scale=f_scale, write_scale=w_scale, raw_per_dispatch=raw,
                per_launch_bytes=per)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--all", action="store_true", help="bench every workload")
    ap.add_argument("--out", default=None, help="also append JSON lines to this file")
    ap.add_argument("--warm", action="store_true", help="no buffer rotation (cache-served)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--dense-min", type=int, default=None, help="SGMV threshold (rows per group)")
    ap.add_argument("--expand-chunks", type=int, default=None,
                    help="256-column chunks per expand workgroup (lora_segments_set_expand_chunks)")
    ap.add_argument("--merge", action="store_true",
                    help="bench lora_merge_slot on the named projections instead")
    ap.add_argument("--sweep", action="store_true",
                    help="adapter count x rank sweep against the base GEMM")
    ap.add_argument("--sweep-md", default=None, help="also write the sweep as a markdown table")
    ap.add_argument("--residency", action="store_true",
                    help="adapter load bandwidth and Zipf churn through the residency manager")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--copy-calib", type=int, default=None, metavar="MB",
                    help="only run a plain device copy of MB megabytes (PMC calibration)")
    ap.add_argument("--pmc-summary", nargs=4,
                    metavar=("FETCH_DIR", "WRITE_DIR", "CAL_FETCH_DIR", "CAL_WRITE_DIR"))
    ap.add_argument("--copy-mb", type=int, default=256)
    ap.add_argument("--traffic-update", action="store_true",
                    help="with --pmc-summary: store the result as --workload's entry of "
                         "profiles/traffic.json")
    args = ap.parse_args(argv)

    if args.pmc_summary:
        res = pmc_summary(*args.pmc_summary, args.copy_mb, args.workload)
        print(json.dumps(res, indent=1))
        if args.traffic_update:
            try:
                with open(TRAFFIC_FILE) as f:
                    table = json.load(f)
            except (OSError, ValueError):
                table = {}
            table[args.workload] = res
            with open(TRAFFIC_FILE, "w") as f:
                json.dump(table, f, indent=1, sort_keys=True)
                f.write("\n")
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path "
              f"(rows shard with no exchange; see the design notes). --gpus {args.gpus} "
              "is not supported.", file=sys.stderr)
        return 2
    if "RANK" in os.environ and os.environ.get("WORLD_SIZE", "1") != "1":
        print("bench.py runs on one GPU only", file=sys.stderr)
        return 2
    if args.copy_calib is not None:
        copy_calibration(args.copy_calib)
        return 0
    if args.copy_probe:
        from rank_adapter_gemm_lora_amd import synth
        sizes = {n: accounting(synth.make_workload(n))["bytes"]["total"]
                 for n in ("decode_bgmv", "mlp_down", "mlp_gate_up", "many_adapter", "prefill_sgmv")}
        res = copy_probe(tuple(sizes.values()) + (2 << 30,))
        for r, n in zip(res, list(sizes) + ["2 GiB"]):
            r["size_of"] = n
        print(json.dumps({"copy_probe": res}))
        return 0

    if args.residency:
        bench_residency(args.steps, args.warmup, args.out)
        return 0
    if args.sweep:
        bench_sweep(args.steps, args.warmup, args.out, args.sweep_md)
        return 0
    if args.merge:
        for i, name in enumerate(MERGE_CASES):
            emit(bench_merge(name, args.steps, args.warmup, cpu=not args.no_cpu and i == 0),
                 args.out)
        return 0
    names = ["tiny_ref", "decode_bgmv", "prefill_sgmv", "mlp_gate_up", "mlp_down",
             "many_adapter", "many_adapter_tp4", "mlp_down_tp4"] if args.all else [args.workload]
    lines = {}
    for name in names:
        line = bench_workload(name, args.steps, args.warmup, rotate=not args.warm,
                              cpu=not args.no_cpu and (not args.all or name == DEFAULT_WORKLOAD),
                              dense_min=args.dense_min, expand_chunks=args.expand_chunks)
        lines[name] = line
        emit(line, args.out)
    if "mlp_gate_up" in lines and "mlp_down" in lines:
        # one MLP layer: the gate/up stack then the down stack on the same batch
        gu, dn = lines["mlp_gate_up"], lines["mlp_down"]
        ms = gu["ms_per_step"] + dn["ms_per_step"]
        rows = gu["config"]["valid_rows"]
        emit({"metric": gu["metric"], "value": round(rows / (ms * 1e-3), 1), "unit": "tokens/s",
              "ms_per_step": round(ms, 5), "config": {"workload": "mlp_layer (gate/up + down)",
                                                      "valid_rows": rows}}, args.out)
        emit(bench_mlp_layer_one_grouping(args.steps, args.warmup), args.out)
    return 0


def bench_mlp_layer_one_grouping(steps: int, warmup: int) -> dict:
    """One MLP layer as a serving loop runs it: the batch is grouped once
    (inside the gate/up shrink, lora_build_shrink) and the down projection
    reuses those segments (page "LoRA hot-loading and adapter routing", batched
    multi-adapter execution: the groups are formed once per batch).  Per step:
    lora_build_shrink + lora_add_expand on the gate/up stack, then
    lora_add_shrink + lora_add_expand on the down stack with the same segments
    object, over rotating buffer sets of both workloads."""
    import torch
    from rank_adapter_gemm_lora_amd import binding as lb
    from rank_adapter_gemm_lora_amd import synth

    pg, pd = synth.make_workload("mlp_gate_up"), synth.make_workload("mlp_down")
    assert (pg.ids == pd.ids).all() and pg.n_slots == pd.n_slots and pg.n_rows == pd.n_rows
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream(dev)
    sh = stream.cuda_stream

    def staged(p):
        raw = (lambda a: a.view(np.int16)) if p.dtype == "bf16" else (lambda a: a)
        dA = [None if p.ranks[s] == 0 else torch.from_numpy(raw(np.ascontiguousarray(p.A[s]))).to(dev)
              for s in range(p.n_slots)]
        dB = [None if p.ranks[s] == 0 else torch.from_numpy(raw(np.ascontiguousarray(p.B[s]))).to(dev)
              for s in range(p.n_slots)]
        return dA, dB

    (gA, gB), (dA, dB) = staged(pg), staged(pd)
    torch.cuda.synchronize()
    n_sets = max(2, math.ceil(ROTATE_BYTES / (set_bytes(pg) + set_bytes(pd))))
    with torch.cuda.stream(stream):
        sets = [(BufferSet(pg, lb, torch, dev, sh, gA, gB, None),
                 BufferSet(pd, lb, torch, dev, sh, dA, dB, None)) for _ in range(n_sets)]
    torch.cuda.synchronize()
    del gA, gB, dA, dB

    def layer(pair):
        g, d = pair
        lb.lora_build_shrink(g.stack, g.x.data_ptr(), pg.ldx, g.ids.data_ptr(), pg.n_rows, g.seg, sh)
        lb.lora_add_expand(g.stack, g.y.data_ptr(), pg.ldy, g.seg, sh)
        lb.lora_add_shrink(d.stack, d.x.data_ptr(), pd.ldx, g.seg, sh)
        lb.lora_add_expand(d.stack, d.y.data_ptr(), pd.ldy, g.seg, sh)

    for i in range(warmup):
        layer(sets[i % n_sets])
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(steps):
        layer(sets[(warmup + i) % n_sets])
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    for g, d in sets:
        g.close(lb)
        d.close(lb)
    rows = int((pg.ids >= 0).sum())
    return {"metric": "LoRA-applied tokens/s per layer", "value": round(rows / (ms * 1e-3), 1),
            "unit": "tokens/s", "ms_per_step": round(ms, 5), "steps": steps, "warmup": warmup,
            "config": {"workload": "mlp_layer (gate/up + down, one grouping)", "valid_rows": rows,
                       "buffer_sets": n_sets}}


def emit(line, out):
    s = json.dumps(line)
    print(s, flush=True)
    if out:
        with open(out, "a") as f:
            f.write(s + "\n")


if __name__ == "__main__":
    sys.exit(main())
