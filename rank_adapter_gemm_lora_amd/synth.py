"""Seeded synthetic workloads for multi-adapter LoRA apply.

This module only draws random inputs and stores them in the library's dtypes;
it contains none of the method's arithmetic.  The same host buffers feed the
HIP library (tests, bench) and the CPU oracle (tests), so both see identical
bits.

Drawing recipe (numpy PCG64, seed 0 unless stated), in this fixed order:
request lengths (prefill only), adapter ids, x, A (slot-major, then slice,
each [r_s, k]), B (slot-major, each [D, r_s]), y.  Normals are drawn as fp32
``standard_normal * std`` and, for bf16 workloads, rounded to bf16 with
round-to-nearest-even.  "Zipf(a) over N slots" means p_s proportional to
(s + 1)**-a for s in [0, N) (slot 0 is the hottest), drawn with ``rng.choice``.

The named workloads follow the shapes the pages discuss: one adapter shelf with
several resident adapters, one integer id per row with "none" meaning the base
model (page "Multi-LoRA Serving: one base, many adapters", section 2), rank-r
adapters on q/k/v and MLP projections (page "LoRA hot-loading and adapter
routing", weight-structure section) and a rank cap that sizes the slots
(Multi-LoRA page, section 3.2).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import List, Optional

import numpy as np

WORKLOADS = ("tiny_ref", "decode_bgmv", "prefill_sgmv", "mlp_gate_up", "mlp_down",
             "many_adapter")
# One GPU's share of a projection under 4-way tensor parallelism (the whole
# workload's inputs cut, nothing redrawn): the column-parallel up-projection
# keeps the first D/4 output columns; the row-parallel down-projection keeps
# the first k/4 input columns (its v would then be summed across GPUs).
SHARD_WORKLOADS = ("many_adapter_tp4", "mlp_down_tp4")


def f32_to_bf16_bits(a) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even, NaN kept quiet."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = ((u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16))
    out = rounded.astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = ((u[nan] >> np.uint64(16)) | np.uint64(0x0040)).astype(np.uint16)
    return out


def bf16_bits_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


@dataclass
class Problem:
    """One stack (one projection) and one batch of rows."""
    name: str
    dtype: str                  # "f32" or "bf16"
    k: int
    slice_d: List[int]
    n_slots: int
    r_max: int
    ranks: np.ndarray           # int32 [n_slots], 0 = empty slot
    alphas: np.ndarray          # float32 [n_slots]
    ids: np.ndarray             # int32 [n_rows], -1 = none
    x: np.ndarray               # [n_rows, ldx]  float32, or uint16 bf16 bits
    y: np.ndarray               # [n_rows, ldy]  base output, same dtype
    A: List[Optional[np.ndarray]] = field(default_factory=list)  # per slot [S, r_s, k]
    B: List[Optional[np.ndarray]] = field(default_factory=list)  # per slot [D, r_s]
    note: str = ""

    @property
    def n_rows(self) -> int:
        return int(self.ids.shape[0])

    @property
    def n_slices(self) -> int:
        return len(self.slice_d)

    @property
    def D(self) -> int:
        return int(sum(self.slice_d))

    @property
    def ldx(self) -> int:
        return int(self.x.shape[1])

    @property
    def ldy(self) -> int:
        return int(self.y.shape[1])

    @property
    def np_dtype(self):
        return np.float32 if self.dtype == "f32" else np.uint16

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


def _normal(rng, shape, std, dtype):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a = a * np.float32(std)
    return a if dtype == "f32" else f32_to_bf16_bits(a)


def zipf_probs(n: int, a: float) -> np.ndarray:
    w = (np.arange(1, n + 1, dtype=np.float64)) ** (-a)
    return w / w.sum()


def _draw_factors(rng, dtype, ranks, k, slice_d, std_a, std_b):
    S, D = len(slice_d), int(sum(slice_d))
    A = [(_normal(rng, (S, int(r), k), std_a, dtype) if r > 0 else None) for r in ranks]
    B = [(_normal(rng, (D, int(r)), std_b, dtype) if r > 0 else None) for r in ranks]
    return A, B


def make_random(seed: int, n_rows: int, k: int, slice_d, n_slots: int, ranks, r_max: int,
                dtype: str = "bf16", alpha=32.0, id_probs=None, p_none: float = 0.0,
                ids=None, std_x=1.0, std_ab=0.02, std_y=1.0, pad_x: int = 0, pad_y: int = 0,
                name: str = "random") -> Problem:
    """A generic seeded problem: ids drawn from ``id_probs`` (uniform by default)
    with a fraction ``p_none`` of none rows, unless ``ids`` is given."""
    rng = np.random.default_rng(seed)
    ranks = np.asarray(ranks, dtype=np.int32)
    assert ranks.shape == (n_slots,)
    if ids is None:
        if id_probs is None:
            id_probs = np.full(n_slots, 1.0 / n_slots)
        ids = rng.choice(n_slots, size=n_rows, p=id_probs).astype(np.int32)
        if p_none > 0:
            none = rng.random(n_rows) < p_none
            ids[none] = -1
    ids = np.asarray(ids, dtype=np.int32)
    D = int(sum(slice_d))
    x = _normal(rng, (n_rows, k + pad_x), std_x, dtype)
    A, B = _draw_factors(rng, dtype, ranks, k, slice_d, std_ab, std_ab)
    y = _normal(rng, (n_rows, D + pad_y), std_y, dtype)
    alphas = np.broadcast_to(np.asarray(alpha, np.float32), (n_slots,)).astype(np.float32)
    return Problem(name, dtype, k, list(slice_d), n_slots, r_max, ranks, alphas, ids, x, y, A, B)


def _tiny_ref(seed):
    # 8 rows, k = d = 256, rank 8, 3 slots + none, fp32, alpha 16,
    # ids uniform over {none, 0, 1, 2}; x ~ N(0,1); A, B, y ~ N(0, 0.02).
    rng = np.random.default_rng(seed)
    ids = rng.integers(-1, 3, size=8).astype(np.int32)
    x = _normal(rng, (8, 256), 1.0, "f32")
    ranks = np.full(3, 8, np.int32)
    A, B = _draw_factors(rng, "f32", ranks, 256, [256], 0.02, 0.02)
    y = _normal(rng, (8, 256), 0.02, "f32")
    return Problem("tiny_ref", "f32", 256, [256], 3, 8, ranks, np.full(3, 16.0, np.float32),
                   ids, x, y, A, B, note="8 rows, 256->256, r=8, 3 slots + none, fp32")


def _decode_bgmv(seed):
    # 256 decode rows, q-proj 4096 -> 4096, rank 16, 8 slots, ids uniform over
    # {none, 0..7}, bf16, x ~ N(0,1), A, B ~ N(0, 0.02), y ~ N(0,1), alpha 32.
    rng = np.random.default_rng(seed)
    ids = rng.integers(-1, 8, size=256).astype(np.int32)
    x = _normal(rng, (256, 4096), 1.0, "bf16")
    ranks = np.full(8, 16, np.int32)
    A, B = _draw_factors(rng, "bf16", ranks, 4096, [4096], 0.02, 0.02)
    y = _normal(rng, (256, 4096), 1.0, "bf16")
    return Problem("decode_bgmv", "bf16", 4096, [4096], 8, 16, ranks,
                   np.full(8, 32.0, np.float32), ids, x, y, A, B,
                   note="256 rows x 1 token, 4096->4096, r=16, 8 slots + none, bf16")


def _prefill_sgmv(seed):
    # 64 requests with lengths U{64..1024}, packed in request order; fused QKV
    # 4096 -> 4096/1024/1024; rank 16; 4 slots; Zipf(1.2) adapter per request.
    rng = np.random.default_rng(seed)
    lengths = rng.integers(64, 1025, size=64)
    req_ids = rng.choice(4, size=64, p=zipf_probs(4, 1.2)).astype(np.int32)
    ids = np.repeat(req_ids, lengths).astype(np.int32)
    n = ids.shape[0]
    x = _normal(rng, (n, 4096), 1.0, "bf16")
    ranks = np.full(4, 16, np.int32)
    slice_d = [4096, 1024, 1024]
    A, B = _draw_factors(rng, "bf16", ranks, 4096, slice_d, 0.02, 0.02)
    y = _normal(rng, (n, sum(slice_d)), 1.0, "bf16")
    return Problem("prefill_sgmv", "bf16", 4096, slice_d, 4, 16, ranks,
                   np.full(4, 32.0, np.float32), ids, x, y, A, B,
                   note=f"64 requests, {n} tokens, fused QKV 4096->4096/1024/1024, r=16, "
                        "4 slots, Zipf(1.2)")


def _mlp_pair(seed):
    # 512 decode rows, exactly 102 none rows at seeded positions, the other 410
    # uniform over 16 slots; slot s has rank [8,16,32,64][s % 4], slots padded
    # to r_max = 64; alpha 32.  Stack 1: gate/up 4096 -> 2 x 14336; stack 2:
    # down 14336 -> 4096 with fresh x and y.
    rng = np.random.default_rng(seed)
    order = rng.permutation(512)
    ids = np.full(512, -1, np.int32)
    routed = np.sort(order[102:])
    ids[routed] = rng.integers(0, 16, size=routed.shape[0]).astype(np.int32)
    ranks = np.array([[8, 16, 32, 64][s % 4] for s in range(16)], np.int32)
    alphas = np.full(16, 32.0, np.float32)
    x1 = _normal(rng, (512, 4096), 1.0, "bf16")
    A1, B1 = _draw_factors(rng, "bf16", ranks, 4096, [14336, 14336], 0.02, 0.02)
    y1 = _normal(rng, (512, 28672), 1.0, "bf16")
    x2 = _normal(rng, (512, 14336), 1.0, "bf16")
    A2, B2 = _draw_factors(rng, "bf16", ranks, 14336, [4096], 0.02, 0.02)
    y2 = _normal(rng, (512, 4096), 1.0, "bf16")
    up = Problem("mlp_gate_up", "bf16", 4096, [14336, 14336], 16, 64, ranks, alphas, ids,
                 x1, y1, A1, B1, note="512 rows (102 none), gate/up 4096->2x14336, ranks "
                                      "{8,16,32,64} padded to 64, 16 slots")
    down = Problem("mlp_down", "bf16", 14336, [4096], 16, 64, ranks, alphas, ids.copy(),
                   x2, y2, A2, B2, note="512 rows (102 none), down 14336->4096, ranks "
                                        "{8,16,32,64} padded to 64, 16 slots")
    return up, down


def _many_adapter(seed):
    # 1024 decode rows, up-proj 8192 -> 28672, 100 resident slots of rank 16,
    # Zipf(1.1) ids, no none rows, bf16, alpha 32.
    rng = np.random.default_rng(seed)
    ids = rng.choice(100, size=1024, p=zipf_probs(100, 1.1)).astype(np.int32)
    x = _normal(rng, (1024, 8192), 1.0, "bf16")
    ranks = np.full(100, 16, np.int32)
    A, B = _draw_factors(rng, "bf16", ranks, 8192, [28672], 0.02, 0.02)
    y = _normal(rng, (1024, 28672), 1.0, "bf16")
    return Problem("many_adapter", "bf16", 8192, [28672], 100, 16, ranks,
                   np.full(100, 32.0, np.float32), ids, x, y, A, B,
                   note="1024 rows, 8192->28672, 100 slots r=16, Zipf(1.1)")


def tp_share(p: Problem, degree: int, mode: str) -> Problem:
    """One GPU's share of ``p`` under ``degree``-way tensor parallelism:
    mode "column" keeps the first d_q / degree columns of every slice (B rows,
    y columns), mode "row" the first k / degree input columns (x, A)."""
    if mode == "column":
        keep = [d // degree for d in p.slice_d]
        cols = np.concatenate([off + np.arange(kq) for off, kq in
                               zip(np.cumsum([0] + list(p.slice_d[:-1])), keep)])
        B = [None if b is None else np.ascontiguousarray(b[cols]) for b in p.B]
        y = np.ascontiguousarray(p.y[:, cols])
        return replace(p, name=f"{p.name}_tp{degree}", slice_d=keep, B=B, y=y,
                       note=p.note + f"; column share 1/{degree}: D = {sum(keep)}")
    if mode == "row":
        k = p.k // degree
        A = [None if a is None else np.ascontiguousarray(a[:, :, :k]) for a in p.A]
        x = np.ascontiguousarray(p.x[:, :k])
        return replace(p, name=f"{p.name}_tp{degree}", k=k, A=A, x=x,
                       note=p.note + f"; row share 1/{degree}: k = {k}")
    raise ValueError(mode)


def make_workload(name: str, seed: int = 0) -> Problem:
    """One of the named workloads (see WORKLOADS and SHARD_WORKLOADS)."""
    if name == "many_adapter_tp4":
        return tp_share(_many_adapter(seed), 4, "column")
    if name == "mlp_down_tp4":
        return tp_share(_mlp_pair(seed)[1], 4, "row")
    if name == "tiny_ref":
        return _tiny_ref(seed)
    if name == "decode_bgmv":
        return _decode_bgmv(seed)
    if name == "prefill_sgmv":
        return _prefill_sgmv(seed)
    if name == "mlp_gate_up":
        return _mlp_pair(seed)[0]
    if name == "mlp_down":
        return _mlp_pair(seed)[1]
    if name == "many_adapter":
        return _many_adapter(seed)
    raise KeyError(name)


def with_strides(p: Problem, pad_x: int, pad_y: int, seed: int = 1) -> Problem:
    """Copy of ``p`` whose x and y rows carry extra trailing columns (ldx > k,
    ldy > D) filled with seeded values that must come back untouched."""
    rng = np.random.default_rng(seed)
    n = p.n_rows
    x = np.empty((n, p.k + pad_x), p.np_dtype)
    x[:, :p.k] = p.x[:, :p.k]
    x[:, p.k:] = _normal(rng, (n, pad_x), 1.0, p.dtype)
    y = np.empty((n, p.D + pad_y), p.np_dtype)
    y[:, :p.D] = p.y[:, :p.D]
    y[:, p.D:] = _normal(rng, (n, pad_y), 1.0, p.dtype)
    return replace(p, x=x, y=y, name=p.name + f"+ld({pad_x},{pad_y})")


def make_base_weight(seed: int, D: int, k: int, dtype: str = "bf16", std: float = 0.02,
                     pad: int = 0) -> np.ndarray:
    """A seeded dense base weight [D, k + pad] (row = output feature), N(0, std),
    for the merge path; the pad columns must come back untouched."""
    rng = np.random.default_rng(seed)
    return _normal(rng, (D, k + pad), std, dtype)


def subset_rows(p: Problem, n: int) -> Problem:
    """The first n rows of ``p`` (same adapters)."""
    return replace(p, ids=p.ids[:n].copy(), x=p.x[:n].copy(), y=p.y[:n].copy(),
                   name=p.name + f"[:{n}]")
