"""The seeded workload generator: determinism, shapes, id distributions, and the
bf16 rounding it applies (checked against torch's own conversion)."""
import numpy as np
import pytest
import torch

from rank_adapter_gemm_lora_amd import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1e-40, -1e-40, 3.4e38, -3.4e38, np.inf, -np.inf,
                                  1.00390625, 1.01171875, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8],
                                 np.float32)])
    ours = synth.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    nan = synth.f32_to_bf16_bits(np.array([np.nan], np.float32))
    assert np.isnan(synth.bf16_bits_to_f32(nan))[0]
    back = synth.bf16_bits_to_f32(ours[:1000])
    np.testing.assert_array_equal(back, torch.from_numpy(a[:1000]).to(torch.bfloat16).float().numpy())


@pytest.mark.parametrize("name", ["tiny_ref", "decode_bgmv", "mlp_down"])
def test_deterministic(name):
    p1 = synth.make_workload(name, seed=0)
    p2 = synth.make_workload(name, seed=0)
    for f in ("ids", "x", "y"):
        np.testing.assert_array_equal(getattr(p1, f), getattr(p2, f))
    for s in range(p1.n_slots):
        np.testing.assert_array_equal(p1.A[s], p2.A[s])
        np.testing.assert_array_equal(p1.B[s], p2.B[s])
    p3 = synth.make_workload(name, seed=1)
    assert not np.array_equal(p1.x, p3.x)


def test_tiny_ref_shape():
    p = synth.make_workload("tiny_ref")
    assert (p.dtype, p.n_rows, p.k, p.D, p.n_slots, p.r_max) == ("f32", 8, 256, 256, 3, 8)
    assert set(np.unique(p.ids)) <= {-1, 0, 1, 2}
    assert p.x.dtype == np.float32 and p.A[0].shape == (1, 8, 256) and p.B[0].shape == (256, 8)
    assert np.all(p.alphas == 16)
    assert abs(float(np.std(p.y)) - 0.02) < 0.005


def test_decode_shape():
    p = synth.make_workload("decode_bgmv")
    assert (p.dtype, p.n_rows, p.k, p.D, p.n_slots, p.r_max) == ("bf16", 256, 4096, 4096, 8, 16)
    assert p.ids.min() >= -1 and p.ids.max() <= 7
    assert 0 < np.sum(p.ids == -1) < 60
    a = synth.bf16_bits_to_f32(p.A[3])
    assert abs(float(a.std()) - 0.02) < 0.001


def test_mlp_pair_shares_ids():
    up = synth.make_workload("mlp_gate_up")
    down = synth.make_workload("mlp_down")
    np.testing.assert_array_equal(up.ids, down.ids)
    assert np.sum(up.ids == -1) == 102
    assert up.slice_d == [14336, 14336] and up.k == 4096 and up.r_max == 64
    assert down.slice_d == [4096] and down.k == 14336
    assert list(up.ranks[:4]) == [8, 16, 32, 64]
    assert up.A[3].shape == (2, 64, 4096) and up.B[0].shape == (28672, 8)


@pytest.mark.slow
def test_prefill_and_many_adapter_shapes():
    p = synth.make_workload("prefill_sgmv")
    assert p.slice_d == [4096, 1024, 1024] and p.n_slots == 4
    assert 64 * 64 <= p.n_rows <= 64 * 1024 and np.all(p.ids >= 0)
    # requests are packed in order: ids change at most 63 times
    assert np.count_nonzero(np.diff(p.ids)) <= 63
    m = synth.make_workload("many_adapter")
    assert m.n_slots == 100 and m.n_rows == 1024 and m.D == 28672 and m.k == 8192
    counts = np.bincount(m.ids, minlength=100)
    assert counts[0] == counts.max() and counts[0] > 150


def test_zipf_probs():
    p = synth.zipf_probs(4, 1.2)
    np.testing.assert_allclose(p.sum(), 1.0)
    np.testing.assert_allclose(p[0] / p[1], 2 ** 1.2)


def test_strides_keep_data():
    p = synth.make_workload("tiny_ref")
    q = synth.with_strides(p, 8, 16)
    assert q.ldx == p.k + 8 and q.ldy == p.D + 16
    np.testing.assert_array_equal(q.x[:, :p.k], p.x)
    np.testing.assert_array_equal(q.y[:, :p.D], p.y)


def test_tensor_parallel_shares_cut_the_full_workload():
    """The one-GPU shares are cuts of the full workloads, nothing redrawn:
    columns [0, D/4) of the up-projection, input columns [0, k/4) of the
    down-projection."""
    full, share = synth.make_workload("many_adapter"), synth.make_workload("many_adapter_tp4")
    assert share.slice_d == [7168] and share.k == full.k
    np.testing.assert_array_equal(share.y, full.y[:, :7168])
    np.testing.assert_array_equal(share.x, full.x)
    for s in (0, 57, 99):
        np.testing.assert_array_equal(share.B[s], full.B[s][:7168])
        np.testing.assert_array_equal(share.A[s], full.A[s])
    full, share = synth.make_workload("mlp_down"), synth.make_workload("mlp_down_tp4")
    assert share.k == 3584 and share.slice_d == full.slice_d
    np.testing.assert_array_equal(share.x, full.x[:, :3584])
    np.testing.assert_array_equal(share.y, full.y)
    for s in (0, 3, 15):
        np.testing.assert_array_equal(share.A[s], full.A[s][:, :, :3584])
        np.testing.assert_array_equal(share.B[s], full.B[s])
    np.testing.assert_array_equal(share.ids, full.ids)
