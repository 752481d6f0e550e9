"""GPU parity of lora_merge_slot: folding one slot's adapter into a dense base
weight (sign +1) and taking it out again (sign -1), against the oracle's
fp64 merged weight.

Page "LoRA serving: multi-adapter dynamic loading", section 1 (merge versus a
separate adapter); page "Multi-LoRA Serving", section 3.1 (shapes of B and A).

Gate: the same float gate as the apply path (bf16 rel-L2 <= 2e-3 and <= 4 ulps,
fp32 rel-L2 <= 1e-5), and for bf16 at most 1 ulp: every element is one
rounding of an fp32 value whose only other error is the fp32 sum of r exact
products.  Columns >= k of W must come back bit-identical.
"""
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


class MergeRig:
    """A stack with slots loaded from a synthetic problem (device-side loads, so
    the merge reads the pool in stream order right after the copies)."""

    def __init__(self, dtype, k, slice_d, ranks, r_max, seed=0, alpha=32.0):
        self.p = synth.make_random(seed, n_rows=1, k=k, slice_d=slice_d, n_slots=len(ranks),
                                   ranks=ranks, r_max=r_max, dtype=dtype, alpha=alpha)
        self.stream = torch.cuda.current_stream(DEV).cuda_stream
        dt = lb.LORA_BF16 if dtype == "bf16" else lb.LORA_F32
        self.stack = lb.lora_stack_create(dt, len(ranks), r_max, k, slice_d, 1)
        self._keep = []
        for s, r in enumerate(ranks):
            if r > 0:
                dA, dB = _dev_raw(self.p.A[s], DEV), _dev_raw(self.p.B[s], DEV)
                self._keep += [dA, dB]
                lb.lora_load_slot(self.stack, s, int(r), float(self.p.alphas[s]), dA.data_ptr(),
                                  dB.data_ptr(), False, self.stream)

    def merge(self, slot, W_host, sign=1, times=1):
        """Merged copy of W_host (raw dtype) after ``times`` calls."""
        dW = _dev_raw(W_host, DEV)
        for _ in range(times):
            lb.lora_merge_slot(self.stack, slot, dW.data_ptr(), W_host.shape[1], sign, self.stream)
        torch.cuda.synchronize(DEV)
        return _host_raw(dW, self.p.dtype)

    def ref(self, slot, W_host, sign=1, rows=None):
        """Oracle merged weight, for every row or for the sorted row sample ``rows``."""
        p = self.p
        if rows is None:
            return oracle.merge(p.dtype, p.k, p.slice_d, int(p.ranks[slot]), float(p.alphas[slot]),
                                p.A[slot], p.B[slot], W_host, sign, n_threads=ORACLE_THREADS)
        # rows of different slices are independent: merge the sampled rows as
        # a smaller problem with the same A and the sampled rows of B and W
        off = np.concatenate([[0], np.cumsum(p.slice_d)])
        sub_d = [int(np.sum((rows >= off[q]) & (rows < off[q + 1]))) for q in range(len(p.slice_d))]
        keep = [q for q in range(len(sub_d)) if sub_d[q] > 0]
        A = p.A[slot][keep]
        return oracle.merge(p.dtype, p.k, [sub_d[q] for q in keep], int(p.ranks[slot]),
                            float(p.alphas[slot]), A, p.B[slot][rows], W_host[rows], sign,
                            n_threads=ORACLE_THREADS)

    def close(self):
        torch.cuda.synchronize(DEV)
        lb.lora_stack_destroy(self.stack)


def _gate(got, ref, dtype, what):
    m = compare.check(got, ref, dtype, what)
    if dtype == "bf16":
        assert m["max_ulp"] <= 1.0 + 1e-9, f"{what}: {m}"
    return m


CASES = {
    # name: (k, slice_d, ranks, r_max, pad)
    "ragged_slices": (200, [48, 16, 24], [3, 16, 9], 16, 24),
    "rank_chunks": (136, [72, 64], [1, 8, 31, 33, 64, 65, 100, 128], 128, 8),
    "r_max_40": (256, [40, 88], [40, 17], 40, 0),
    "k8_d8": (8, [8], [1], 1, 8),
    "multi_tile": (1032, [200, 136], [16, 64], 64, 16),
}


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", list(CASES))
def test_merge_matches_oracle(case, dtype):
    k, slice_d, ranks, r_max, pad = CASES[case]
    rig = MergeRig(dtype, k, slice_d, ranks, r_max, seed=3)
    try:
        D = sum(slice_d)
        for s in range(len(ranks)):
            W = synth.make_base_weight(100 + s, D, k, dtype, pad=pad)
            for sign in (1, -1):
                note(f"merge {case} {dtype} slot {s} rank {ranks[s]} sign {sign}")
                got = rig.merge(s, W, sign)
                np.testing.assert_array_equal(got[:, k:], W[:, k:], err_msg="columns >= k changed")
                _gate(got[:, :k], rig.ref(s, W, sign), dtype, f"{case}/{dtype}/slot{s}/{sign:+d}")
    finally:
        rig.close()


# the projections of the named workloads, merged at full size; large weights
# are checked on a row sample (first and last row of every slice included)
WORKLOAD_MERGES = {
    "q_proj_4096_r16": (4096, [4096], [16, 16], 16, None),
    "fused_qkv_r16": (4096, [4096, 1024, 1024], [16], 16, None),
    "gate_up_r64": (4096, [14336, 14336], [64, 8], 64, 600),
    "up_8192_28672_r16": (8192, [28672], [16], 16, 300),
    # >= 4096 tiles (the persistent kernel) with ragged slabs, slices and rank
    "ragged_stream_r40": (136, [131000, 72], [40], 40, 600),
}


@pytest.mark.parametrize("case", list(WORKLOAD_MERGES))
def test_merge_workload_shapes(case):
    k, slice_d, ranks, r_max, n_sample = WORKLOAD_MERGES[case]
    rig = MergeRig("bf16", k, slice_d, ranks, r_max, seed=5)
    try:
        D = sum(slice_d)
        W = synth.make_base_weight(7, D, k, "bf16")
        slot = len(ranks) - 1
        note(f"merge workload {case} slot {slot}")
        got = rig.merge(slot, W, 1)
        if n_sample is None:
            rows = None
            sel = got
        else:
            rng = np.random.default_rng(1)
            off = np.cumsum([0] + slice_d)
            rows = set(rng.choice(D, size=n_sample, replace=False).tolist())
            for q in range(len(slice_d)):
                rows.update([int(off[q]), int(off[q + 1] - 1)])
            rows = np.array(sorted(rows), np.int64)
            sel = got[rows]
        _gate(sel, rig.ref(slot, W, 1, rows=rows), "bf16", case)
    finally:
        rig.close()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_merge_then_unmerge_restores(dtype):
    """Unmerge after merge gives W back up to the two roundings (<= 1 ulp each,
    counted at the larger of |W| and |W'|), at the decode projection's size."""
    rig = MergeRig(dtype, 4096, [4096], [16], 16, seed=9)
    try:
        W = synth.make_base_weight(11, 4096, 4096, dtype)
        dW = _dev_raw(W, DEV)
        note(f"merge+unmerge {dtype}")
        lb.lora_merge_slot(rig.stack, 0, dW.data_ptr(), 4096, 1, rig.stream)
        torch.cuda.synchronize(DEV)
        mid = compare.to_f64(_host_raw(dW, dtype), dtype)
        lb.lora_merge_slot(rig.stack, 0, dW.data_ptr(), 4096, -1, rig.stream)
        back = compare.to_f64(_host_raw(dW, dtype), dtype)
        w0 = compare.to_f64(W, dtype)
        assert np.abs(mid - w0).max() > 0, "merge changed nothing"
        mag = np.maximum(np.abs(w0), np.abs(mid))
        ulps = np.abs(back - w0) / compare.ulp_of(mag, dtype)
        assert ulps.max() <= 2.0 + 1e-9, ulps.max()
    finally:
        rig.close()


def test_merge_is_deterministic_and_repeats():
    """The same merge on the same input gives bit-identical results."""
    rig = MergeRig("bf16", 512, [256, 128], [32], 32, seed=13)
    try:
        W = synth.make_base_weight(17, 384, 512, "bf16")
        note("merge determinism")
        a = rig.merge(0, W, 1)
        b = rig.merge(0, W, 1)
        np.testing.assert_array_equal(a, b)
    finally:
        rig.close()


def test_merge_errors():
    rig = MergeRig("bf16", 64, [64], [8, 0], 8, seed=2)
    try:
        W = torch.zeros((64, 72), dtype=torch.int16, device=DEV)
        ptr = W.data_ptr()
        st = rig.stack

        def status(slot, w, ldw, sign):
            try:
                lb.lora_merge_slot(st, slot, w, ldw, sign, rig.stream)
                return lb.LORA_OK
            except lb.LoraError as e:
                return e.status

        note("merge errors")
        assert status(1, ptr, 72, 1) == 5        # empty slot
        assert status(-1, ptr, 72, 1) == 3
        assert status(2, ptr, 72, 1) == 3
        assert status(0, ptr, 72, 0) == 1        # sign
        assert status(0, ptr, 72, 2) == 1
        assert status(0, ptr, 56, 1) == 1        # ldw < k
        assert status(0, ptr, 68, 1) == 1        # ldw not a multiple of 8
        assert status(0, ptr + 2, 72, 1) == 1    # misaligned
        assert status(0, 0, 72, 1) == 1          # null
        torch.cuda.synchronize(DEV)
        assert int(W.abs().sum()) == 0, "a rejected call wrote W"
        lb.lora_evict_slot(st, 0, rig.stream)
        assert status(0, ptr, 72, 1) == 5        # evicted
    finally:
        rig.close()
