"""lora_build_apply: grouping and apply in one call.

For small batches the grouping runs inside the shrink kernel; the call must
leave the same segments as lora_build_segments (bit for bit, checked against
the oracle), give bit-identical y to lora_build_segments + lora_apply (the
products run the same tile code on the same tile plan), and pass the oracle's
float gate.  Larger batches, and an empty one, take the two-call path; the
ragged cases cover both sides of that switch.
"""
import numpy as np
import pytest
import torch

import oracle
from rank_adapter_gemm_lora_amd import binding as lb
from rank_adapter_gemm_lora_amd import synth
from gpu_helpers import GpuRun, check_against_oracle, note, sample_rows

pytestmark = pytest.mark.gpu

PATHS = {"auto": None, "bgmv": 1 << 30, "sgmv": 1}
WORKLOADS = ("tiny_ref", "decode_bgmv", "mlp_gate_up", "mlp_down", "many_adapter")


def _seg_equal(got, p, what):
    ref = oracle.build_segments(p.ids, p.n_slots, p.ranks)
    for key in ("perm", "seg_off", "active", "counts"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=f"{what} {key}")


def _fused_vs_split(p, dm, what):
    """(y, segments, tile counts) of build_apply and of build + apply."""
    out = []
    for fused in (True, False):
        run = GpuRun(p, dense_min=dm)
        try:
            if fused:
                run.build_apply()
            else:
                run.build()
                run.apply()
            y = run.y_host()
            seg = run.segments()
            tc = lb.lora_segments_tile_counts(run.seg, run.stream)
            lb.lora_get_device_status(run.seg, run.stream)   # raises if a wait timed out
        finally:
            run.close()
        out.append((y, seg, tc))
    (yf, sf, tf), (ys, ss, ts) = out
    np.testing.assert_array_equal(yf, ys, err_msg=f"{what}: fused y differs from split y")
    assert tf == ts, what
    _seg_equal(sf, p, what)
    return yf


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("name", WORKLOADS)
def test_build_apply_workloads(name, path):
    p = synth.make_workload(name)
    note(f"build_apply {name} path={path} n={p.n_rows}")
    y = _fused_vs_split(p, PATHS[path], f"{name}/{path}")
    check_against_oracle(p, y, what=f"{name}/{path}/fused")


RAGGED = [(1, 1), (15, 2), (16, 2), (17, 2), (200, 300), (255, 9), (256, 9), (257, 9),
          (1000, 100), (1023, 5), (1024, 5), (1024, 1024), (1025, 5), (1500, 40)]


@pytest.mark.parametrize("n,n_slots", RAGGED)
def test_build_apply_ragged(n, n_slots):
    """Row counts around the wavefront, tile and 1024-row limits, bad ids,
    empty slots; bf16 and fp32."""
    rng = np.random.default_rng(1000 + n + n_slots)
    ranks = np.full(n_slots, 16, np.int32)
    ranks[rng.random(n_slots) < 0.15] = 0
    ids = rng.integers(-2, n_slots + 2, size=n).astype(np.int32)
    for dtype in ("bf16", "f32"):
        p = synth.make_random(11, n_rows=n, k=128, slice_d=[64, 64], n_slots=n_slots,
                              ranks=ranks, r_max=16, dtype=dtype, ids=ids)
        for path, dm in PATHS.items():
            note(f"build_apply ragged n={n} slots={n_slots} {dtype} {path}")
            y = _fused_vs_split(p, dm, f"n={n}/{dtype}/{path}")
            check_against_oracle(p, y, what=f"n={n}/{dtype}/{path}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_build_apply_ks16_mixed_ranks(dtype):
    """Long k at a small batch: 16 k-splits, so each tile's expand workgroups
    wait on 16 shrink workgroups' flags in the one-launch kernel; mixed ranks
    up to 64 and two slices."""
    p = synth.make_random(23, n_rows=100, k=8192, slice_d=[512, 256], n_slots=4,
                          ranks=[16, 8, 32, 64], r_max=64, p_none=0.1, dtype=dtype)
    for path, dm in PATHS.items():
        note(f"build_apply ks16 {dtype} {path}")
        y = _fused_vs_split(p, dm, f"ks16/{dtype}/{path}")
        check_against_oracle(p, y, what=f"ks16/{dtype}/{path}")


def test_build_apply_empty_and_errors():
    p = synth.make_random(5, n_rows=32, k=64, slice_d=[64], n_slots=3, ranks=[8, 8, 8], r_max=8)
    run = GpuRun(p, max_rows=32)
    try:
        note("build_apply empty batch")
        run.build_apply(n_rows=0)
        seg = lb.lora_segments_download(run.seg, 0, p.n_slots, run.stream)
        assert list(seg["counts"]) == [0, 0, 0]
        assert list(seg["seg_off"]) == [0] * (p.n_slots + 1)
        assert list(seg["active"]) == [-1] * p.n_slots
        np.testing.assert_array_equal(run.y_host(), p.y)
        note("build_apply errors")
        with pytest.raises(lb.LoraError) as e:
            run.build_apply(n_rows=33)                      # beyond max_rows
        assert e.value.status == lb.LORA_E_ARG
        with pytest.raises(lb.LoraError) as e:
            lb.lora_build_apply(run.stack, run.y.data_ptr(), p.ldy, 0, p.ldx,
                                run.ids.data_ptr(), 32, run.seg, run.stream)   # null x
        assert e.value.status == lb.LORA_E_ARG
        with pytest.raises(lb.LoraError) as e:
            lb.lora_build_apply(run.stack, run.y.data_ptr(), p.ldy, run.x.data_ptr() + 2, p.ldx,
                                run.ids.data_ptr(), 32, run.seg, run.stream)   # misaligned x
        assert e.value.status == lb.LORA_E_ARG
        # nothing was enqueued by the failed calls: y is still the input
        np.testing.assert_array_equal(run.y_host(), p.y)
    finally:
        run.close()


def test_build_apply_repeated_layers():
    """One grouping per batch, then the call repeated on new x/y (the layers of
    a model): each result matches the oracle for its own inputs."""
    base = synth.make_workload("decode_bgmv")
    run = GpuRun(base)
    try:
        for layer in range(3):
            p = synth.make_random(200 + layer, n_rows=base.n_rows, k=base.k, slice_d=base.slice_d,
                                  n_slots=base.n_slots, ranks=base.ranks, r_max=base.r_max,
                                  ids=base.ids, dtype=base.dtype)
            p.A, p.B, p.alphas = base.A, base.B, base.alphas
            note(f"build_apply layer {layer}")
            run.x.copy_(torch.from_numpy(p.x.view(np.int16)).to(run.device))
            run.y.copy_(torch.from_numpy(p.y.view(np.int16)).to(run.device))
            run.build_apply()
            check_against_oracle(p, run.y_host(), what=f"layer {layer}")
    finally:
        run.close()


@pytest.mark.parametrize("name", ["decode_bgmv", "tiny_ref"])
def test_build_apply_back_to_back(name):
    """Ten one-launch calls in a row on one stream, no host synchronisation
    between them (each on a fresh copy of the base y, alternating two adapter
    mixes): every launch opens a new epoch, so none may consume the v of an
    earlier one.  The last call's y matches the oracle, its segments are
    exact, and no wait timed out."""
    base = synth.make_workload(name)
    other = base.ids.copy()[::-1].copy()
    run = GpuRun(base)
    try:
        y0 = run.y.clone()
        ids = [torch.from_numpy(base.ids).to(run.device), torch.from_numpy(other).to(run.device)]
        note(f"back-to-back build_apply {name}")
        for i in range(10):
            run.ids.copy_(ids[i % 2], non_blocking=True)
            run.y.copy_(y0, non_blocking=True)
            run.build_apply()
        p = synth.make_random(0, n_rows=base.n_rows, k=base.k, slice_d=base.slice_d,
                              n_slots=base.n_slots, ranks=base.ranks, r_max=base.r_max,
                              ids=other, dtype=base.dtype)
        p.A, p.B, p.alphas, p.x, p.y = base.A, base.B, base.alphas, base.x, base.y
        check_against_oracle(p, run.y_host(), what=f"{name} back-to-back")
        _seg_equal(run.segments(), p, f"{name} back-to-back")
        lb.lora_get_device_status(run.seg, run.stream)
    finally:
        run.close()


APPLY_CASES = {
    "decode_bgmv": lambda: synth.make_workload("decode_bgmv"),
    "tiny_ref": lambda: synth.make_workload("tiny_ref"),
    "mixed_ranks": lambda: synth.make_random(31, n_rows=200, k=512, slice_d=[256, 128], n_slots=6,
                                             ranks=[8, 16, 32, 64, 5, 0], r_max=64, p_none=0.1),
    "ks16": lambda: synth.make_random(23, n_rows=100, k=8192, slice_d=[512, 256], n_slots=4,
                                      ranks=[16, 8, 32, 64], r_max=64, p_none=0.1),
    "rows3000": lambda: synth.make_random(3, n_rows=3000, k=512, slice_d=[512], n_slots=8,
                                          ranks=[16] * 8, r_max=16, p_none=0.1),
}


@pytest.mark.parametrize("case", list(APPLY_CASES))
def test_apply_one_launch_matches_two(case):
    """lora_apply of a grouped batch (one launch where the grid fits the chip)
    gives the same bits as lora_add_shrink + lora_add_expand (two launches),
    on dense and vector tiles, and passes the oracle's gate."""
    p = APPLY_CASES[case]()
    for path, dm in PATHS.items():
        note(f"apply one launch {case} {path}")
        ys = []
        for one in (True, False):
            run = GpuRun(p, dense_min=dm)
            try:
                run.build()
                if one:
                    run.apply()
                else:
                    lb.lora_add_shrink(run.stack, run.x.data_ptr(), p.ldx, run.seg, run.stream)
                    lb.lora_add_expand(run.stack, run.y.data_ptr(), p.ldy, run.seg, run.stream)
                ys.append(run.y_host())
                lb.lora_get_device_status(run.seg, run.stream)
            finally:
                run.close()
        np.testing.assert_array_equal(ys[0], ys[1], err_msg=f"{case}/{path}")
        rows = sample_rows(p, 256) if p.n_rows > 1000 else None
        check_against_oracle(p, ys[0], rows=rows, what=f"apply {case}/{path}")


def test_apply_back_to_back_and_graph():
    """One grouping, then lora_apply ten times in a row on one stream with no
    host synchronisation (each on a fresh copy of the base y), then the same
    call captured in a HIP graph and replayed: every result matches the
    oracle and no wait timed out."""
    p = synth.make_workload("decode_bgmv")
    run = GpuRun(p)
    try:
        run.build()
        y0 = run.y.clone()
        note("apply back-to-back")
        for _ in range(10):
            run.y.copy_(y0, non_blocking=True)
            run.apply()
        check_against_oracle(p, run.y_host(), what="apply back-to-back")
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        note("apply graph capture")
        with torch.cuda.graph(graph):
            lb.lora_apply(run.stack, run.y.data_ptr(), p.ldy, run.x.data_ptr(), p.ldx, run.seg,
                          torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        for rep in range(3):
            run.y.copy_(y0)
            torch.cuda.synchronize()
            note(f"apply graph replay {rep}")
            graph.replay()
            torch.cuda.synchronize()
            check_against_oracle(p, run.y_host(), what=f"apply replay {rep}")
        del graph
        lb.lora_get_device_status(run.seg, run.stream)
    finally:
        run.close()


def test_build_apply_plan():
    """Launch counts of lora_build_apply from the host query: one kernel for
    decode batches (the decode kernel up to 63 slots of rank <= 16, so 16
    adapters at 256 rows too), two where no one-launch grid fits the chip
    (rank 128, whose LDS holds one workgroup per CU), three or five for larger
    batches; the query changes nothing."""
    cases = {
        "decode_bgmv": (synth.make_workload("decode_bgmv"), 1),
        "mlp_gate_up": (synth.make_workload("mlp_gate_up"), 2),
        "many_adapter": (synth.make_workload("many_adapter"), 3),
        "16_adapters": (synth.make_random(3, n_rows=256, k=4096, slice_d=[4096], n_slots=16,
                                          ranks=[16] * 16, r_max=16), 1),
        "rank128": (synth.make_random(3, n_rows=256, k=4096, slice_d=[4096], n_slots=1,
                                      ranks=[128], r_max=128), 2),
        "rows3000": (synth.make_random(3, n_rows=3000, k=512, slice_d=[512], n_slots=8,
                                       ranks=[16] * 8, r_max=16), 5),
    }
    # the one-launch rule compares grids with what the chip holds at once: the
    # counts below are those of a whole MI355X (256 CUs); a partitioned device
    # only gets the checks that do not depend on the CU count
    whole_chip = torch.cuda.get_device_properties(0).multi_processor_count == 256
    for name, (p, want) in cases.items():
        note(f"build_apply plan {name}")
        run = GpuRun(p)
        try:
            run.build()
            before = run.segments()
            got = lb.lora_build_apply_plan(run.stack, p.n_rows, run.seg)
            if whole_chip or want > 2:
                assert got == want, name
            else:
                assert got in (1, 2), name
            assert lb.lora_build_apply_plan(run.stack, 0, run.seg) == 1
            after = run.segments()
            for key in before:
                np.testing.assert_array_equal(after[key], before[key], err_msg=f"{name} {key}")
            with pytest.raises(lb.LoraError) as e:
                lb.lora_build_apply_plan(run.stack, run.max_rows + 1, run.seg)
            assert e.value.status == lb.LORA_E_ARG
        finally:
            run.close()


GRAPH_CASES = {
    # name: (rows, k, output width, launches lora_build_apply makes)
    "one_launch": (256, 512, 512, 1),        # the decode kernel
    "two_launches": (512, 4096, 4096, 2),    # grouping inside the shrink, then the expand
    "five_launches": (3000, 512, 512, 5),    # chunked grouping, shrink, expand
}


@pytest.mark.parametrize("case", list(GRAPH_CASES))
def test_build_apply_graph_replay_any_mix(case):
    """The launch shapes depend only on the batch shape, so one captured HIP
    graph of lora_build_apply serves every adapter mix: replays with new ids
    (and a fresh base y) each match the oracle, segments included.  The new
    inputs are copied in eagerly between replays, with synchronisations.  The
    cases cover every launch layout of the call (the plan query confirms it)."""
    n_rows, k, d, launches = GRAPH_CASES[case]
    base = synth.make_random(41, n_rows=n_rows, k=k, slice_d=[d], n_slots=8, ranks=[16] * 8,
                             r_max=16, p_none=1 / 9)
    run = GpuRun(base)
    try:
        got = lb.lora_build_apply_plan(run.stack, base.n_rows, run.seg)
        if torch.cuda.get_device_properties(0).multi_processor_count == 256 or launches > 2:
            assert got == launches, (case, got)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        note(f"graph capture of lora_build_apply, {case}")
        with torch.cuda.graph(graph):
            lb.lora_build_apply(run.stack, run.y.data_ptr(), base.ldy, run.x.data_ptr(), base.ldx,
                                run.ids.data_ptr(), base.n_rows, run.seg,
                                torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        rng = np.random.default_rng(7)
        for rep in range(4):
            ids = rng.integers(-1, base.n_slots, size=base.n_rows).astype(np.int32)
            if rep == 3:
                ids[:] = 2   # one dense group
            p = synth.make_random(41, n_rows=n_rows, k=k, slice_d=[d], n_slots=8,
                                  ranks=[16] * 8, r_max=16, ids=ids)
            p.A, p.B, p.alphas, p.x, p.y = base.A, base.B, base.alphas, base.x, base.y
            run.ids.copy_(torch.from_numpy(ids).to(run.device))
            run.y.copy_(torch.from_numpy(base.y.view(np.int16)).to(run.device))
            torch.cuda.synchronize()
            note(f"graph replay {rep}, {case}")
            graph.replay()
            torch.cuda.synchronize()
            check_against_oracle(p, run.y_host(), what=f"replay {rep}")
            _seg_equal(lb.lora_segments_download(run.seg, p.n_rows, p.n_slots, run.stream), p,
                       f"replay {rep}")
            lb.lora_get_device_status(run.seg, run.stream)
        del graph
    finally:
        run.close()


def _untouched_or_correct(p, y_out, what):
    """Rows without an adapter and columns past D bitwise untouched; every
    element of a valid row either bitwise untouched or within the gate's
    per-element bound (4 bf16 ulps at max(|yref|, 2^-8 max|yref|)) of the
    oracle.  Returns the fraction of valid-row elements left untouched."""
    from oracle import compare
    from gpu_helpers import oracle_rows, valid_mask
    ok = valid_mask(p)
    np.testing.assert_array_equal(y_out[~ok], p.y[~ok], err_msg=f"{what}: rows without adapter")
    np.testing.assert_array_equal(y_out[:, p.D:], p.y[:, p.D:], err_msg=f"{what}: padding columns")
    sel = np.nonzero(ok)[0]
    ref = oracle_rows(p, rows=sel)
    got = compare.to_f64(y_out[sel, :p.D], p.dtype)
    same = y_out[sel, :p.D] == p.y[sel, :p.D]
    floor = compare.ULP_FLOOR_FRACTION * np.max(np.abs(ref))
    ulps = np.abs(got - ref) / compare.ulp_of(np.maximum(np.abs(ref), floor), p.dtype)
    bad = ~same & ~(ulps <= compare.BF16_MAX_ULP)
    assert not bad.any(), f"{what}: {int(bad.sum())} elements neither untouched nor correct"
    return float(same.mean())


WAIT_GUARD_CASES = {
    # name: (tile policy, call)
    "decode_kernel": (None, "build_apply"),          # lora_build_apply, the decode kernel
    "build_apply_kernel": (1 << 30, "build_apply"),  # vector tiles: the general one-launch kernel
    "apply_kernel": (None, "apply"),                 # lora_apply of a grouped batch
}


@pytest.mark.parametrize("case", list(WAIT_GUARD_CASES))
def test_wait_guard_leaves_y_untouched(case):
    """The one-launch hand-over's bounded wait, forced to give up from the host
    (a wait limit of 0 polls: each expand wavefront checks once, before its
    shrink workgroups can have finished; every kernel still exits normally).
    Rows of a tile whose wait gave up stay bitwise untouched, the rest are
    correct; the next call on the object, made before the status is read,
    leaves y wholly untouched; lora_get_device_status reports LORA_E_HIP and
    resets the hand-over state, after which a call with the default limit
    matches the oracle and reports no error."""
    dm, call = WAIT_GUARD_CASES[case]
    p = synth.make_workload("decode_bgmv")
    run = GpuRun(p, dense_min=dm)
    try:
        y0 = run.y.clone()
        assert lb.lora_build_apply_plan(run.stack, p.n_rows, run.seg) == 1   # one kernel
        if call == "apply":
            run.build()
        fn = run.build_apply if call == "build_apply" else run.apply
        lb.lora_segments_set_wait_limit(run.seg, 0)
        note(f"wait guard {case}: limit 0")
        fn()
        frac = _untouched_or_correct(p, run.y_host(), f"{case} first call")
        run.y.copy_(y0)
        torch.cuda.synchronize()
        note(f"wait guard {case}: call before the status is read")
        fn()
        y2 = run.y_host()
        with pytest.raises(lb.LoraError) as e:
            lb.lora_get_device_status(run.seg, run.stream)
        assert e.value.status == lb.LORA_E_HIP, case
        np.testing.assert_array_equal(y2, p.y, err_msg=f"{case}: call after a timeout wrote y")
        note(f"wait guard {case}: {frac:.2f} of the first call's elements untouched")
        lb.lora_segments_set_wait_limit(run.seg, 1 << 18)
        run.y.copy_(y0)
        torch.cuda.synchronize()
        fn()
        check_against_oracle(p, run.y_host(), what=f"{case} after the reset")
        assert lb.lora_get_device_status(run.seg, run.stream) == 0   # no bad ids, no timeout
        with pytest.raises(lb.LoraError):
            lb.lora_segments_set_wait_limit(run.seg, -1)
    finally:
        run.close()
