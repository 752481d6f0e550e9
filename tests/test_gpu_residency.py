"""GPU behaviour of the residency manager: batches of rows naming adapters by
id, mapped to slots (loads and LRU evictions in stream order on the batch's
stream, no host synchronisation in between), then applied with
lora_build_apply; every batch's output is gated against the oracle applying
each row's own adapter.  Page "LoRA hot-loading and adapter routing",
adapter-lifecycle section; page "Multi-LoRA Serving: one base, many
adapters", sections 3.2 and 6."""
import numpy as np
import pytest
import torch

import oracle
from oracle import compare
from rank_adapter_gemm_lora_amd import binding as lb
from rank_adapter_gemm_lora_amd import synth
from gpu_helpers import ORACLE_THREADS, _dev_raw, _host_raw, note

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _adapters(dtype, n, k, slice_d, ranks, seed):
    """n adapters (A, B, alpha) drawn like the workloads' slots."""
    p = synth.make_random(seed, n_rows=1, k=k, slice_d=slice_d, n_slots=n, ranks=ranks,
                          r_max=max(ranks), dtype=dtype, alpha=32.0)
    return p.A, p.B, [32.0] * n


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_batches_through_residency_match_oracle(dtype):
    k, slice_d, n_slots, r_max = 256, [128, 64], 4, 32
    n_ad = 10
    ranks = [8, 16, 32, 4, 16, 24, 8, 32, 12, 16]
    A, B, alphas = _adapters(dtype, n_ad, k, slice_d, ranks, seed=21)
    stream = torch.cuda.current_stream(DEV).cuda_stream
    dt = lb.LORA_BF16 if dtype == "bf16" else lb.LORA_F32
    n_rows = 96
    st = lb.lora_stack_create(dt, n_slots, r_max, k, slice_d, n_rows)
    seg = lb.lora_segments_create(n_rows, n_slots)
    m = lb.lora_residency_create(st, 2 * n_slots)   # host tier smaller than the adapter set
    rng = np.random.default_rng(5)

    def registered(aid):
        try:
            lb.lora_residency_slot_of(m, int(aid))
            return True
        except lb.LoraError:
            return False

    try:
        for b in range(12):
            # the scheduler's batch: at most n_slots distinct adapters, each
            # (re-)registered if the host tier does not hold it (admitting one
            # may drop another non-resident one, so repeat until all are in)
            use = rng.choice(n_ad, size=int(rng.integers(1, n_slots + 1)), replace=False)
            for _ in range(2 * n_slots):
                missing = [int(a) for a in use if not registered(a)]
                if not missing:
                    break
                aid = missing[0]
                lb.lora_residency_register(m, aid, ranks[aid], alphas[aid],
                                           np.ascontiguousarray(A[aid]).ctypes.data,
                                           np.ascontiguousarray(B[aid]).ctypes.data)
            assert all(registered(a) for a in use)
            rows = rng.choice(use, size=n_rows).astype(np.int64)
            rows[rng.random(n_rows) < 0.1] = -1
            note(f"residency {dtype} batch {b} adapters {sorted(use.tolist())}")
            ids = lb.lora_residency_map_batch(m, rows, stream)
            x = synth.make_random(100 + b, n_rows=n_rows, k=k, slice_d=slice_d, n_slots=1,
                                  ranks=[1], r_max=1, dtype=dtype).x
            y0 = synth.make_random(200 + b, n_rows=n_rows, k=k, slice_d=slice_d, n_slots=1,
                                   ranks=[1], r_max=1, dtype=dtype).y
            dx, dy = _dev_raw(x, DEV), _dev_raw(y0, DEV)
            dids = torch.from_numpy(ids).to(DEV)
            lb.lora_build_apply(st, dy.data_ptr(), y0.shape[1], dx.data_ptr(), k, dids.data_ptr(),
                                n_rows, seg, stream)
            y = _host_raw(dy, dtype)
            # the oracle applies each row's own adapter, by adapter index
            ok = rows >= 0
            ref = oracle.apply_rows(dtype, k, slice_d, ranks, alphas, A, B,
                                    np.where(ok, rows, -1).astype(np.int32), x, y0,
                                    rows=np.nonzero(ok)[0], n_threads=ORACLE_THREADS)
            np.testing.assert_array_equal(y[~ok], y0[~ok])
            compare.check(y[ok][:, :sum(slice_d)], ref, dtype, f"residency batch {b}")
            for aid in use:
                assert lb.lora_residency_slot_of(m, int(aid)) == ids[rows == aid][0]
        s = lb.lora_residency_stats(m)
        assert s["loads"] >= n_slots and s["evictions"] > 0 and s["resident"] <= n_slots
    finally:
        torch.cuda.synchronize(DEV)
        lb.lora_residency_destroy(m)
        lb.lora_segments_destroy(seg)
        lb.lora_stack_destroy(st)


def test_caller_slots_are_kept_and_unregister_evicts():
    k, slice_d = 64, [64]
    A, B, alphas = _adapters("bf16", 3, k, slice_d, [8, 8, 8], seed=4)
    stream = torch.cuda.current_stream(DEV).cuda_stream
    st = lb.lora_stack_create(lb.LORA_BF16, 3, 8, k, slice_d, 8)
    lb.lora_load_slot(st, 1, 8, 32.0, np.ascontiguousarray(A[0]).ctypes.data,
                      np.ascontiguousarray(B[0]).ctypes.data, True, stream)
    m = lb.lora_residency_create(st, 4)
    try:
        for aid in (10, 11, 12):
            lb.lora_residency_register(m, aid, 8, 32.0, np.ascontiguousarray(A[aid - 10]).ctypes.data,
                                       np.ascontiguousarray(B[aid - 10]).ctypes.data)
        note("residency caller slots")
        ids = lb.lora_residency_map_batch(m, [10, 11, 10], stream)
        assert sorted(set(ids.tolist())) == [0, 2]        # slot 1 belongs to the caller
        with pytest.raises(lb.LoraError) as e:
            lb.lora_residency_map_batch(m, [10, 11, 12], stream)
        assert e.value.status == lb.LORA_E_CAPACITY
        lb.lora_residency_unregister(m, 10, stream)
        assert lb.lora_slot_info(st, 1)[0] == 8            # untouched
        assert lb.lora_residency_map_batch(m, [12], stream).tolist() == [ids[0]]
        with pytest.raises(lb.LoraError) as e:
            lb.lora_residency_map_batch(m, [10], stream)
        assert e.value.status == lb.LORA_E_NOT_FOUND
        torch.cuda.synchronize(DEV)
    finally:
        lb.lora_residency_destroy(m)
        lb.lora_stack_destroy(st)


def test_direct_stack_calls_are_followed():
    k, slice_d = 64, [64]
    A, B, alphas = _adapters("bf16", 3, k, slice_d, [8, 8, 8], seed=6)
    stream = torch.cuda.current_stream(DEV).cuda_stream
    st = lb.lora_stack_create(lb.LORA_BF16, 3, 8, k, slice_d, 8)
    m = lb.lora_residency_create(st, 8)
    ptr = lambda a: np.ascontiguousarray(a).ctypes.data
    try:
        for aid in range(3):
            lb.lora_residency_register(m, aid, 8, 32.0, ptr(A[aid]), ptr(B[aid]))
        note("residency follows direct stack calls")
        # the caller takes slot 0 after the manager was created
        lb.lora_load_slot(st, 0, 8, 32.0, ptr(A[0]), ptr(B[0]), True, stream)
        with pytest.raises(lb.LoraError) as e:
            lb.lora_residency_map_batch(m, [0, 1, 2], stream)
        assert e.value.status == lb.LORA_E_CAPACITY
        ids = lb.lora_residency_map_batch(m, [1, 2], stream)
        assert sorted(ids.tolist()) == [1, 2]
        # the caller evicts one of the manager's slots: that adapter is reloaded on use
        lb.lora_evict_slot(st, int(ids[0]), stream)
        assert lb.lora_residency_map_batch(m, [1], stream).tolist() == [int(ids[0])]
        assert lb.lora_slot_info(st, int(ids[0]))[0] == 8
        # the caller frees slot 0: three distinct adapters fit again
        lb.lora_evict_slot(st, 0, stream)
        assert sorted(lb.lora_residency_map_batch(m, [0, 1, 2], stream).tolist()) == [0, 1, 2]
        torch.cuda.synchronize(DEV)
    finally:
        lb.lora_residency_destroy(m)
        lb.lora_stack_destroy(st)
