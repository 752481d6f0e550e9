"""GPU behaviour of the C ABI beyond the named workloads: edge shapes, bad ids,
errors, slot hot-swap in stream order, determinism and the invariances the
per-row definition implies (bit-exact on the GPU)."""
import numpy as np
import pytest
import torch

import oracle
from rank_adapter_gemm_lora_amd import binding as lb
from rank_adapter_gemm_lora_amd import synth
from gpu_helpers import GpuRun, check_against_oracle, note

pytestmark = pytest.mark.gpu

PATHS = {"bgmv": 1 << 30, "sgmv": 1, "auto": None}


def _run_and_check(p, dense_min=None, what="", **kw):
    run = GpuRun(p, dense_min=dense_min, **kw)
    try:
        run.build()
        run.apply()
        y = run.y_host()
        seg = run.segments()
        n_bad = lb.lora_get_device_status(run.seg, run.stream)
    finally:
        run.close()
    ref = oracle.build_segments(p.ids, p.n_slots, p.ranks)
    for key in ("perm", "seg_off", "active", "counts"):
        np.testing.assert_array_equal(seg[key], ref[key], err_msg=f"{what} {key}")
    assert n_bad == ref["counts"][2]
    check_against_oracle(p, y, what=what)
    return y


EDGE_CASES = {
    # name: make_random kwargs
    "k8_d8_rank1": dict(n_rows=5, k=8, slice_d=[8], n_slots=2, ranks=[1, 1], r_max=1),
    "ragged_slices": dict(n_rows=70, k=40, slice_d=[72, 8, 64], n_slots=3, ranks=[3, 16, 9],
                          r_max=16, p_none=0.2),
    "rank128": dict(n_rows=40, k=256, slice_d=[128], n_slots=2, ranks=[128, 100], r_max=128),
    "mixed_ranks_slices": dict(n_rows=200, k=512, slice_d=[256, 128], n_slots=6,
                               ranks=[8, 16, 32, 64, 5, 0], r_max=64, p_none=0.1),
    "many_rows_pass": dict(n_rows=5000, k=64, slice_d=[64], n_slots=37,
                           ranks=[16] * 37, r_max=16, p_none=0.05),
    "max_slots": dict(n_rows=3000, k=64, slice_d=[64], n_slots=1024, ranks=[8] * 1024,
                      r_max=8, p_none=0.1),
    "single_row": dict(n_rows=1, k=128, slice_d=[64], n_slots=1, ranks=[16], r_max=16),
    # rank windows of the MFMA expand: B of a 256-column chunk does not fit
    # LDS beside v in one piece (64-row tiles above 4096 rows: 48-rank windows)
    "rank128_tall": dict(n_rows=4500, k=256, slice_d=[256], n_slots=2, ranks=[128, 100],
                         r_max=128, p_none=0.05),
    "rank128_slices": dict(n_rows=300, k=128, slice_d=[192, 64], n_slots=2, ranks=[128, 72],
                           r_max=128),
    # long k at a small batch: 16 k-splits (the v partials summed in two batches)
    "ks16_long_k": dict(n_rows=100, k=8192, slice_d=[512], n_slots=4, ranks=[16, 8, 32, 64],
                        r_max=64, p_none=0.1),
    # the most slices a stack takes, ragged and unaligned (slices * r_max = 256)
    "max_slices": dict(n_rows=300, k=96, slice_d=[64, 8, 16, 128, 64, 24, 8, 200], n_slots=3,
                       ranks=[32, 7, 1], r_max=32, p_none=0.1),
    # both sides of the switch to 64-row dense tiles
    "rows4096": dict(n_rows=4096, k=128, slice_d=[128], n_slots=3, ranks=[16, 16, 8], r_max=16),
    "rows4097": dict(n_rows=4097, k=128, slice_d=[128], n_slots=3, ranks=[16, 16, 8], r_max=16),
    # 64-row dense tiles below 4096 rows: a wide output at r_max >= 32
    "tall_wide_d": dict(n_rows=1100, k=256, slice_d=[8192], n_slots=4, ranks=[32, 16, 8, 32],
                        r_max=32, p_none=0.05),
    # the run expand (16-row dense tiles, r_max 64) on grids smaller than one
    # workgroup per XCD: one 256-column chunk, then two
    "run_one_chunk": dict(n_rows=20, k=64, slice_d=[256], n_slots=2, ranks=[64, 40], r_max=64),
    "run_two_chunks": dict(n_rows=40, k=128, slice_d=[448, 64], n_slots=3, ranks=[64, 64, 33],
                           r_max=64, p_none=0.1),
}


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", list(EDGE_CASES))
def test_edge_shapes(case, dtype):
    kw = dict(EDGE_CASES[case])
    p = synth.make_random(7, dtype=dtype, name=case, **kw)
    for path, dm in PATHS.items():
        note(f"edge {case} {dtype} {path}")
        _run_and_check(p, dense_min=dm, what=f"{case}/{dtype}/{path}")


def test_zero_rows_and_all_none():
    p = synth.make_random(3, n_rows=64, k=64, slice_d=[64], n_slots=4, ranks=[16] * 4, r_max=16)
    note("zero rows")
    run = GpuRun(p)
    try:
        run.build(n_rows=0)
        run.apply()
        y = run.y_host()
        seg = run.segments()
    finally:
        run.close()
    np.testing.assert_array_equal(y, p.y)
    assert list(seg["counts"]) == [0, 0, 0]
    note("all none")
    p.ids[:] = -1
    _run_and_check(p, what="all-none")


def test_bad_ids_counted_and_untouched():
    p = synth.make_random(5, n_rows=300, k=128, slice_d=[128], n_slots=6,
                          ranks=[16, 16, 0, 16, 8, 16], r_max=16, p_none=0.1)
    p.ids[::7] = 2          # empty slot
    p.ids[3::11] = 6        # == n_slots
    p.ids[5::13] = -9       # negative, not -1
    p.ids[9::17] = 1 << 20  # far out of range
    for path, dm in PATHS.items():
        note(f"bad ids {path}")
        _run_and_check(p, dense_min=dm, what=f"bad-ids/{path}")


def test_load_from_device_source():
    p = synth.make_random(9, n_rows=100, k=256, slice_d=[128, 64], n_slots=3,
                          ranks=[16, 7, 32], r_max=32, p_none=0.2)
    note("device-source load")
    _run_and_check(p, load_from_device=True, what="device-load")


def test_errors():
    p = synth.make_random(1, n_rows=16, k=64, slice_d=[64], n_slots=3, ranks=[8, 0, 8], r_max=16)
    note("error paths")
    run = GpuRun(p)
    A = np.zeros((1, 17, 64), np.uint16)
    B = np.zeros((64, 17), np.uint16)
    try:
        def status(fn, *a):
            with pytest.raises(lb.LoraError) as e:
                fn(*a)
            return e.value.status
        assert status(lb.lora_load_slot, run.stack, 1, 17, 1.0, A.ctypes.data, B.ctypes.data,
                      True, run.stream) == lb.LORA_E_RANK
        assert status(lb.lora_load_slot, run.stack, 1, 0, 1.0, A.ctypes.data, B.ctypes.data,
                      True, run.stream) == lb.LORA_E_RANK
        assert status(lb.lora_load_slot, run.stack, 3, 8, 1.0, A.ctypes.data, B.ctypes.data,
                      True, run.stream) == lb.LORA_E_SLOT
        assert status(lb.lora_load_slot, run.stack, -1, 8, 1.0, A.ctypes.data, B.ctypes.data,
                      True, run.stream) == lb.LORA_E_SLOT
        assert status(lb.lora_load_slot, run.stack, 0, 8, 1.0, A.ctypes.data, B.ctypes.data,
                      True, run.stream) == lb.LORA_E_OCCUPIED
        assert status(lb.lora_load_slot, run.stack, 1, 8, float("nan"), A.ctypes.data,
                      B.ctypes.data, True, run.stream) == lb.LORA_E_ARG
        assert status(lb.lora_evict_slot, run.stack, 1, run.stream) == lb.LORA_E_EMPTY
        assert status(lb.lora_evict_slot, run.stack, 5, run.stream) == lb.LORA_E_SLOT
        # apply before any build
        assert status(lb.lora_apply, run.stack, run.y.data_ptr(), p.ldy, run.x.data_ptr(),
                      p.ldx, run.seg, run.stream) == lb.LORA_E_ARG
        run.build()
        assert status(lb.lora_apply, run.stack, run.y.data_ptr(), p.ldy, run.x.data_ptr(),
                      p.ldx - 8, run.seg, run.stream) == lb.LORA_E_ARG
        assert status(lb.lora_apply, run.stack, run.y.data_ptr() + 2, p.ldy, run.x.data_ptr(),
                      p.ldx, run.seg, run.stream) == lb.LORA_E_ARG
        assert status(lb.lora_build_segments, run.stack, run.ids.data_ptr(), p.n_rows + 1,
                      run.seg, run.stream) == lb.LORA_E_ARG
        # rank / alpha bookkeeping and the r(d + k) parameter count
        r, a, n = lb.lora_slot_info(run.stack, 0)
        assert (r, a) == (8, float(p.alphas[0]))
        assert n == oracle.param_count(8, p.k, p.slice_d)
        assert lb.lora_slot_info(run.stack, 1) == (0, 0.0, 0)
        # nothing above changed y
        torch.cuda.synchronize()
        np.testing.assert_array_equal(run.y_host(), p.y)
    finally:
        run.close()


def test_hot_swap_in_stream_order():
    """load -> build -> apply -> evict -> load other weights -> build -> apply,
    all enqueued on one stream with no host synchronisation in between."""
    p = synth.make_random(21, n_rows=200, k=256, slice_d=[256], n_slots=4, ranks=[16] * 4,
                          r_max=32, p_none=0.1)
    note("hot swap")
    run = GpuRun(p)
    try:
        run.build()
        run.apply()
        y1 = run.y.clone()
        # swap slot 2 for an adapter of another rank and alpha
        lb.lora_evict_slot(run.stack, 2, run.stream)
        swap = synth.make_random(23, n_rows=1, k=256, slice_d=[256], n_slots=1, ranks=[24],
                                 r_max=32)
        A2, B2 = swap.A[0], swap.B[0]
        run.load(2, A2, B2, 12.0, from_device=True)
        # evict slot 3 entirely: its rows become bad ids in the next build
        lb.lora_evict_slot(run.stack, 3, run.stream)
        run.build()
        run.apply()
        y2 = run.y_host()
        y1h = y1.cpu().numpy().view(np.uint16)
    finally:
        run.close()
    check_against_oracle(p, y1h, what="before swap")
    p2 = synth.Problem(**{**p.__dict__})
    p2.A = list(p.A)
    p2.B = list(p.B)
    p2.A[2], p2.B[2] = A2, B2
    p2.A[3] = p2.B[3] = None
    p2.ranks = p.ranks.copy()
    p2.ranks[2], p2.ranks[3] = 24, 0
    p2.alphas = p.alphas.copy()
    p2.alphas[2] = 12.0
    p2.y = y1h
    check_against_oracle(p2, y2, what="after swap")


SHRINK_SWAPS = {
    # multi-slice stack on the matrix-core path: rank 64 -> 8 and 64 -> 40 (not a
    # multiple of 16) in slots whose operand image held the larger adapters
    "mfma_two_slices": dict(n_rows=300, k=256, slice_d=[128, 192], n_slots=3, ranks=[64, 64, 32],
                            r_max=64, swaps={0: 8, 1: 40}),
    # decode-kernel shape (one slice, r_max 16, <= 256 rows): the kernel reads all
    # 16 rank rows of a slot's image, so rows past a smaller rank must be zero
    "decode_rank16_to_4": dict(n_rows=200, k=512, slice_d=[512], n_slots=4, ranks=[16] * 4,
                               r_max=16, swaps={1: 4, 2: 12}),
}


@pytest.mark.parametrize("mode", ["split", "build_apply"])
@pytest.mark.parametrize("case", list(SHRINK_SWAPS))
def test_reload_smaller_rank_clears_operand_rows(case, mode):
    """Evict and reload slots with a smaller rank in stream order; the rank rows
    the earlier adapters held must read as zero afterwards (pool and image).
    build_apply runs the decode kernel on the decode shape."""
    c = dict(SHRINK_SWAPS[case])
    swaps = c.pop("swaps")
    p = synth.make_random(41, dtype="bf16", p_none=0.05, **c)
    note(f"reload smaller rank {case} {mode}")
    run = GpuRun(p)

    def step():
        if mode == "split":
            run.build()
            run.apply()
        else:
            run.build_apply()

    try:
        step()
        y1 = run.y.clone()
        new = {}
        for slot, rank in swaps.items():
            q = synth.make_random(43 + slot, n_rows=1, k=p.k, slice_d=p.slice_d, n_slots=1,
                                  ranks=[rank], r_max=p.r_max, dtype="bf16")
            lb.lora_evict_slot(run.stack, slot, run.stream)
            run.load(slot, q.A[0], q.B[0], 3.0 + slot, from_device=True)
            new[slot] = (q.A[0], q.B[0], rank)
        step()
        y2 = run.y_host()
        y1h = y1.cpu().numpy().view(np.uint16)
    finally:
        run.close()
    check_against_oracle(p, y1h, what=f"{case} before reload")
    p2 = synth.Problem(**{**p.__dict__})
    p2.A, p2.B = list(p.A), list(p.B)
    p2.ranks, p2.alphas = p.ranks.copy(), p.alphas.copy()
    for slot, (A2, B2, rank) in new.items():
        p2.A[slot], p2.B[slot] = A2, B2
        p2.ranks[slot] = rank
        p2.alphas[slot] = 3.0 + slot
    p2.y = y1h
    check_against_oracle(p2, y2, what=f"{case} after reload")


def test_evicted_after_build_leaves_rows_untouched():
    p = synth.make_random(31, n_rows=120, k=128, slice_d=[128], n_slots=3, ranks=[16] * 3,
                          r_max=16)
    for path, dm in PATHS.items():
        note(f"evict after build {path}")
        run = GpuRun(p, dense_min=dm)
        try:
            run.build()
            lb.lora_evict_slot(run.stack, 1, run.stream)
            run.apply()
            y = run.y_host()
        finally:
            run.close()
        ranks = p.ranks.copy()
        ranks[1] = 0
        check_against_oracle(p, y, ranks=ranks, what=f"evict-after-build/{path}")


@pytest.mark.parametrize("name", ["decode_bgmv", "mlp_down", "many_adapter"])
def test_deterministic_and_invariant(name):
    """Same inputs -> same bits; permuting rows or relabelling slots permutes
    or preserves the output bit for bit (a row's arithmetic never depends on
    its position or its neighbours)."""
    p = synth.make_workload(name)
    for path, dm in PATHS.items():
        note(f"invariance {name} {path}")

        def run_once(q):
            r = GpuRun(q, dense_min=dm)
            try:
                r.build()
                r.apply()
                return r.y_host()
            finally:
                r.close()

        y0 = run_once(p)
        np.testing.assert_array_equal(run_once(p), y0)
        perm = np.random.default_rng(0).permutation(p.n_rows)
        pp = synth.Problem(**{**p.__dict__})
        pp.ids, pp.x, pp.y = p.ids[perm].copy(), p.x[perm].copy(), p.y[perm].copy()
        np.testing.assert_array_equal(run_once(pp), y0[perm])
        sigma = np.random.default_rng(1).permutation(p.n_slots)
        inv = np.argsort(sigma)
        ps = synth.Problem(**{**p.__dict__})
        ps.ids = np.array([sigma[s] if s >= 0 else s for s in p.ids], np.int32)
        ps.ranks, ps.alphas = p.ranks[inv].copy(), p.alphas[inv].copy()
        ps.A = [p.A[j] for j in inv]
        ps.B = [p.B[j] for j in inv]
        np.testing.assert_array_equal(run_once(ps), y0)


def test_shrink_expand_split_equals_apply():
    p = synth.make_workload("decode_bgmv")
    note("split shrink/expand")
    r1 = GpuRun(p)
    r2 = GpuRun(p)
    try:
        r1.build()
        r1.apply()
        r2.build()
        lb.lora_add_shrink(r2.stack, r2.x.data_ptr(), p.ldx, r2.seg, r2.stream)
        lb.lora_add_expand(r2.stack, r2.y.data_ptr(), p.ldy, r2.seg, r2.stream)
        np.testing.assert_array_equal(r1.y_host(), r2.y_host())
    finally:
        r1.close()
        r2.close()


SEG_CASES = [(1, 1), (63, 3), (64, 3), (65, 3), (1000, 100), (1024, 8), (1025, 8),
             (1024, 1024), (2048, 254), (2049, 254), (2048, 255), (2048, 256), (700, 300),
             (4097, 10), (9000, 7)]


@pytest.mark.parametrize("n,n_slots", SEG_CASES)
def test_segments_across_builders(n, n_slots):
    """Both segment builders (the one-workgroup grouping up to 1024 rows, the
    chunked one beyond) give the oracle's grouping bit for bit, bad ids
    included, and the tile plan the policy asks for."""
    rng = np.random.default_rng(n * 7 + n_slots)
    ranks = np.full(n_slots, 8, np.int32)
    ranks[rng.random(n_slots) < 0.1] = 0
    p = synth.make_random(3, n_rows=n, k=8, slice_d=[8], n_slots=n_slots, ranks=ranks, r_max=8,
                          ids=rng.integers(-2, n_slots + 2, size=n).astype(np.int32))
    note(f"segments n={n} slots={n_slots}")
    for dm in (1, 16, 1 << 30):
        run = GpuRun(p, dense_min=dm)
        try:
            run.build()
            got = run.segments()
            nb, ns = lb.lora_segments_tile_counts(run.seg, run.stream)
        finally:
            run.close()
        ref = oracle.build_segments(p.ids, p.n_slots, p.ranks)
        for key in ("perm", "seg_off", "active", "counts"):
            np.testing.assert_array_equal(got[key], ref[key], err_msg=f"{key} dense_min={dm}")
        cnt = np.diff(ref["seg_off"])
        dense = cnt >= dm
        tile = 16 if n <= 4096 else 64
        assert ns == int(np.sum((cnt[dense] + tile - 1) // tile))
        assert nb == int(np.sum((cnt[~dense & (cnt > 0)] + 15) // 16))


@pytest.mark.parametrize("build_with", ["narrow", "wide"])
def test_segments_shared_across_stacks(build_with):
    """One grouping per batch serves every projection (page "LoRA hot-loading
    and adapter routing", batched multi-adapter execution: the row groups are
    formed once per batch).  At 2000 rows a rank-8 q-proj stack cuts dense
    groups into 16-row tiles and a rank-64 stack with a wide output into
    64-row tiles; segments built with either stack are applied with both, and
    each result matches the oracle for its own stack (the apply follows the
    tile height the segments were built with)."""
    n, n_slots = 2000, 6
    ids = synth.make_random(7, n_rows=n, k=64, slice_d=[64], n_slots=n_slots,
                            ranks=[8] * n_slots, r_max=8, p_none=0.1).ids
    narrow = synth.make_random(11, n_rows=n, k=512, slice_d=[512], n_slots=n_slots,
                               ranks=[8, 4, 8, 8, 1, 8], r_max=8, ids=ids)
    wide = synth.make_random(12, n_rows=n, k=512, slice_d=[4608], n_slots=n_slots,
                             ranks=[64, 32, 16, 64, 8, 40], r_max=64, ids=ids)
    ra, rb = GpuRun(narrow), GpuRun(wide)
    try:
        builder = ra if build_with == "narrow" else rb
        note(f"shared segments: built with the {build_with} stack")
        builder.build()
        for run, p in ((ra, narrow), (rb, wide)):
            lb.lora_apply(run.stack, run.y.data_ptr(), p.ldy, run.x.data_ptr(), p.ldx, builder.seg,
                          run.stream)
            check_against_oracle(p, run.y_host(), what=f"{p.slice_d} on {build_with} segments")
    finally:
        ra.close()
        rb.close()


def test_tall_batch_with_vector_tiles():
    """Above 4096 rows dense groups take 64-row tiles; with dense_min above the
    smaller groups' sizes those groups take 16-row vector tiles in the same
    batch, so the launch grids keep the 16-row tile bound (the 64-row bound
    holds only when every group is dense)."""
    n_slots = 6
    probs = np.array([0.5, 0.3, 0.17, 0.015, 0.01, 0.005])
    p = synth.make_random(21, n_rows=4500, k=256, slice_d=[256], n_slots=n_slots,
                          ranks=[16, 8, 16, 4, 16, 8], r_max=16, id_probs=probs, p_none=0.02,
                          name="tall_mixed")
    counts = np.bincount(p.ids[p.ids >= 0], minlength=n_slots)
    dense_min = 200
    assert (counts >= dense_min).any() and ((counts > 0) & (counts < dense_min)).any(), counts
    for dt in ("bf16", "f32"):
        q = p if dt == "bf16" else synth.make_random(21, n_rows=4500, k=256, slice_d=[256],
                                                     n_slots=n_slots, ranks=[16, 8, 16, 4, 16, 8],
                                                     r_max=16, id_probs=probs, p_none=0.02,
                                                     dtype="f32", name="tall_mixed")
        note(f"tall batch with vector tiles, {dt}")
        _run_and_check(q, dense_min=dense_min, what=f"tall_mixed/{dt}")
