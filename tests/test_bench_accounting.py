"""The benchmark's algorithmic byte and flop counts (the numerators of every
reported GB/s and roofline fraction), checked on the CPU against figures
worked out by hand from the per-row formula: each valid row's x read once,
its y read and written once, the live A and B of every referenced slot read
once at its true rank; flops 2 r (S k + D) + D per valid row."""
import numpy as np
import pytest

import bench
from rank_adapter_gemm_lora_amd import synth


def _valid(p):
    return np.array([0 <= s < p.n_slots and p.ranks[s] > 0 for s in p.ids], bool)


def test_decode_bytes_by_hand():
    p = synth.make_workload("decode_bgmv")
    ok = _valid(p)
    n = int(ok.sum())
    assert n == 225                               # seed 0: 31 of 256 rows have no adapter
    assert sorted(np.unique(p.ids[ok]).tolist()) == list(range(8))
    a = bench.accounting(p)
    x = n * 4096 * 2
    y = n * 4096 * 2 * 2
    live = 8 * 16 * (4096 + 4096) * 2                 # every slot referenced, rank 16
    assert (x, y, live) == (1_843_200, 3_686_400, 2_097_152)
    assert a["bytes"]["total"] == x + y + live == 7_626_752
    assert a["bytes"]["apply"] == 7_626_752
    # ids, slot table and segments are metadata, not algorithmic bytes
    assert a["bytes"]["build_apply"] == 7_626_752
    assert a["bytes"]["build_shrink"] == x + 8 * 16 * 4096 * 2
    assert a["bytes"]["shrink"] == x + 8 * 16 * 4096 * 2
    assert a["bytes"]["expand"] == y + 8 * 16 * 4096 * 2
    assert a["flops"]["total"] == n * (2 * 16 * (4096 + 4096) + 4096)


def test_mixed_rank_bytes_use_true_ranks():
    """The MLP gate/up stack pads ranks {8, 16, 32, 64} to 64; the count uses
    each referenced slot's true rank, never the padding."""
    p = synth.make_workload("mlp_gate_up")
    ok = _valid(p)
    n = int(ok.sum())
    assert n == 512 - 102
    slots = np.unique(p.ids[ok])
    ranks = [8, 16, 32, 64]
    live_a = sum(ranks[s % 4] * 2 * 4096 for s in slots) * 2      # two slices of A
    live_b = sum(ranks[s % 4] * 28672 for s in slots) * 2
    a = bench.accounting(p)
    assert a["bytes"]["shrink"] == n * 4096 * 2 + live_a
    assert a["bytes"]["expand"] == n * 28672 * 2 * 2 + live_b
    padded = len(slots) * 64 * (2 * 4096 + 28672) * 2
    assert live_a + live_b < padded


@pytest.mark.parametrize("n_launch,kernels", [(1, ("build_apply",)),
                                              (2, ("build_shrink", "expand")),
                                              (3, ("seg_build", "shrink", "expand")),
                                              (5, ("seg_build", "shrink", "expand"))])
def test_step_kernel_labels(n_launch, kernels):
    """The kernels bench.py times for each launch count lora_build_apply_plan
    can report; every label has a byte count to price it."""
    assert bench.STEP_KERNELS[n_launch] == kernels
    a = bench.accounting(synth.make_workload("tiny_ref"))
    for k in kernels:
        assert k in a["bytes"]
