"""GPU parity at the corners of the adapter-count x rank sweep (one q-proj
layer 4096 -> 4096, bf16, every row routed, ids uniform over the adapters):
the sweep times these shapes, so they are held to the same gate as the named
workloads.  Page "LoRA serving: multi-adapter dynamic loading", section on
relative throughput with many adapters; page "Multi-LoRA Serving", section
3.1 (cost linear in the rank)."""
import pytest

from rank_adapter_gemm_lora_amd import synth
from gpu_helpers import GpuRun, check_against_oracle, note, sample_rows

pytestmark = pytest.mark.gpu

CORNERS = [
    # rows, adapters, rank
    (256, 1, 8),
    (256, 100, 128),
    (256, 16, 64),
    (4096, 1, 128),
    (4096, 100, 8),
    (4096, 4, 32),
]


@pytest.mark.parametrize("n_rows,n_adapters,rank", CORNERS)
def test_sweep_corner(n_rows, n_adapters, rank):
    p = synth.make_random(0, n_rows=n_rows, k=4096, slice_d=[4096], n_slots=n_adapters,
                          ranks=[rank] * n_adapters, r_max=rank, dtype="bf16", alpha=32.0)
    note(f"sweep corner rows {n_rows} adapters {n_adapters} rank {rank}")
    run = GpuRun(p)
    try:
        run.build_apply()
        y = run.y_host()
    finally:
        run.close()
    check_against_oracle(p, y, rows=sample_rows(p, 384), what=f"sweep {n_rows}/{n_adapters}/{rank}")
