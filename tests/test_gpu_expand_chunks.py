"""The expand with several 256-column chunks per workgroup (the launch shape
lora_segments_set_expand_chunks picks): every chunk count gives the same bits
as one chunk per workgroup, and the oracle's result within the float gate.
Covers ragged last chunk groups, slices that end inside a group, mixed ranks
(one, two and eight 16-byte B granules per thread), an empty slot, vector
(BGMV) tiles inside the several-chunk kernel, and shapes where the knob is
ignored (64-row tiles, fp32)."""
import numpy as np
import pytest

from rank_adapter_gemm_lora_amd import binding as lb
from rank_adapter_gemm_lora_amd import synth
from gpu_helpers import GpuRun, check_against_oracle, note

pytestmark = pytest.mark.gpu

CASES = {
    # two slices of 1280 + 1536 columns: 11 chunks, a slice boundary inside a chunk group
    "rank16_two_slices": dict(n_rows=300, k=256, slice_d=[1280, 1536], n_slots=9,
                              ranks=[16] * 9, r_max=16, p_none=0.1),
    # r_max 64: eight granules per thread; ranks 5 and 8 load fewer; slot 5 empty
    "mixed_ranks": dict(n_rows=260, k=192, slice_d=[1024, 640], n_slots=6,
                        ranks=[8, 16, 32, 64, 5, 0], r_max=64, p_none=0.15),
    # r_max 24: four granules per thread, three used
    "rank24": dict(n_rows=130, k=128, slice_d=[2304], n_slots=3, ranks=[24, 24, 9],
                   r_max=24),
    # 64-row dense tiles: the knob is ignored
    "rows4097": dict(n_rows=4097, k=128, slice_d=[512], n_slots=3, ranks=[16, 16, 8], r_max=16),
}
CHUNKS = [1, 2, 3, 5, 16]


def _y(p, chunks, dense_min):
    run = GpuRun(p, dense_min=dense_min, expand_chunks=chunks)
    try:
        run.build()
        run.apply()
        return run.y_host()
    finally:
        run.close()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", list(CASES))
def test_expand_chunks_bit_identical(case, dtype):
    p = synth.make_random(11, dtype=dtype, name=case, **CASES[case])
    for dm in (1, 1 << 30):   # dense (MFMA) tiles, then vector tiles
        note(f"expand chunks {case} {dtype} dense_min={dm}")
        y1 = _y(p, 1, dm)
        check_against_oracle(p, y1, what=f"{case}/{dtype}/dm{dm}/chunks1")
        for c in CHUNKS[1:] + [0]:
            yc = _y(p, c, dm)
            np.testing.assert_array_equal(yc, y1, err_msg=f"{case} {dtype} dm={dm} chunks={c}")


def test_expand_chunks_rejects_bad_values():
    p = synth.make_random(3, dtype="bf16", name="knob", n_rows=8, k=64, slice_d=[64],
                          n_slots=2, ranks=[4, 4], r_max=4)
    run = GpuRun(p)
    try:
        for bad in (-1, 17):
            with pytest.raises(lb.LoraError) as e:
                lb.lora_segments_set_expand_chunks(run.seg, bad)
            assert e.value.status == lb.LORA_E_ARG
        lb.lora_segments_set_expand_chunks(run.seg, 0)
    finally:
        run.close()
