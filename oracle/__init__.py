"""Plain CPU fp64 reference ("the oracle") for multi-adapter LoRA apply.

TEST INFRASTRUCTURE ONLY: tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package; the library in
``rank_adapter_gemm_lora_amd`` never does.  The arithmetic lives in
``lora_oracle.c`` (plain loops, IEEE double); this module only compiles it with
gcc and marshals numpy arrays into it.

Functions follow the pages:

* :func:`build_segments` -- group rows by adapter id (page "LoRA hot-loading and
  adapter routing", batched multi-adapter execution section; page "Multi-LoRA
  Serving: one base, many adapters", section 2 flowchart "group rows by adapter
  id").  Stable counting sort; rows without a valid adapter go last.
* :func:`apply_rows` -- y_i + (alpha/r) * B_a (A_a x_i) per row, in double
  (Multi-LoRA page, section 2 per-row equation and section 3.1 LoRA math).
* :func:`apply_grouped` -- the same result computed the way the hot-loading
  page's batched-execution section runs a batch: the rows are gathered into
  one group per adapter id, each group's inputs go through the adapter's two
  factors as whole matrices (numpy matmul in double), and the scaled delta is
  added into the group's rows of the base output.  A second algorithm for the
  same quantity, used to pin :func:`apply_rows`.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lora_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

F32, BF16 = 0, 1


def build(out_path: str = _LIB_PATH, src: str = _SRC, extra_flags=()) -> str:
    """Compile the oracle with gcc (-O2, OpenMP over rows) into ``out_path``."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", *extra_flags,
           src, "-o", out_path + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(out_path + ".tmp", out_path)
    return out_path


def _bind(lib):
    P = ctypes.c_void_p
    i64 = ctypes.c_int64
    lib.oracle_build_segments.restype = ctypes.c_int
    lib.oracle_build_segments.argtypes = [P, i64, ctypes.c_int, P, P, P, P, P]
    lib.oracle_apply_rows.restype = ctypes.c_int
    lib.oracle_apply_rows.argtypes = [ctypes.c_int, i64, ctypes.c_int, P, ctypes.c_int, P, P,
                                      P, P, P, P, P, P, i64, P, i64, P, i64, P, ctypes.c_int]
    lib.oracle_merge.restype = ctypes.c_int
    lib.oracle_merge.argtypes = [ctypes.c_int, i64, ctypes.c_int, P, ctypes.c_int, ctypes.c_double,
                                 P, P, P, i64, ctypes.c_int, P, ctypes.c_int]
    lib.oracle_param_count.restype = ctypes.c_int64
    lib.oracle_param_count.argtypes = [ctypes.c_int, i64, ctypes.c_int, P]
    return lib


def load(path: str | None = None):
    """Load (building first if absent) the oracle shared library."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build()
            _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def build_segments(ids, n_slots: int, slot_rank, lib=None) -> dict:
    """Group rows by slot.  Returns dict(perm, seg_off, active, counts)."""
    lib = lib or load()
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    rank = np.ascontiguousarray(slot_rank, dtype=np.int32)
    assert rank.shape == (n_slots,)
    n = ids.shape[0]
    perm = np.empty(max(n, 1), np.int32)
    seg_off = np.empty(n_slots + 1, np.int32)
    active = np.empty(n_slots, np.int32)
    counts = np.empty(3, np.int32)
    rc = lib.oracle_build_segments(_ptr(ids), n, n_slots, _ptr(rank), _ptr(perm),
                                   _ptr(seg_off), _ptr(active), _ptr(counts))
    if rc != 0:
        raise ValueError("oracle_build_segments: bad argument")
    return dict(perm=perm[:n], seg_off=seg_off, active=active, counts=counts)


def param_count(rank: int, k: int, slice_d, lib=None) -> int:
    """Parameters of one adapter on one stack: r * (n_slices * k + D)."""
    lib = lib or load()
    sd = np.ascontiguousarray(slice_d, dtype=np.int64)
    return int(lib.oracle_param_count(int(rank), int(k), len(sd), _ptr(sd)))


def _cat(parts, dtype):
    """Concatenate per-slot factor arrays; empty slots contribute nothing."""
    offs = np.zeros(len(parts), np.int64)
    flat = []
    pos = 0
    for s, p in enumerate(parts):
        offs[s] = pos
        if p is not None:
            a = np.ascontiguousarray(p, dtype=dtype).reshape(-1)
            flat.append(a)
            pos += a.size
    cat = np.concatenate(flat) if flat else np.zeros(1, dtype)
    return cat, offs


def apply_rows(dtype: str, k: int, slice_d, slot_rank, slot_alpha, A, B, ids, x, y_in,
               rows=None, n_threads: int = 1, lib=None) -> np.ndarray:
    """fp64 adapted output of the selected rows, shape [n_sel, D].

    ``A[s]`` is slot s's shrink factor [n_slices, r_s, k] and ``B[s]`` its expand
    factor [D, r_s] (None for an empty slot).  x [n, ldx] and y_in [n, ldy] hold
    float32 values, or bf16 bit patterns as uint16 when ``dtype == "bf16"``.
    """
    lib = lib or load()
    code = {"f32": F32, "bf16": BF16}[dtype]
    npdt = np.float32 if code == F32 else np.uint16
    slice_d = np.ascontiguousarray(slice_d, dtype=np.int64)
    rank = np.ascontiguousarray(slot_rank, dtype=np.int32)
    alpha = np.ascontiguousarray(slot_alpha, dtype=np.float64)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    x = np.ascontiguousarray(x, dtype=npdt)
    y_in = np.ascontiguousarray(y_in, dtype=npdt)
    n_slots = rank.shape[0]
    D = int(slice_d.sum())
    for s in range(n_slots):
        if rank[s] > 0:
            assert A[s].shape == (len(slice_d), rank[s], k), (s, A[s].shape)
            assert B[s].shape == (D, rank[s]), (s, B[s].shape)
    A_cat, A_off = _cat([A[s] if rank[s] > 0 else None for s in range(n_slots)], npdt)
    B_cat, B_off = _cat([B[s] if rank[s] > 0 else None for s in range(n_slots)], npdt)
    if rows is None:
        n_sel = ids.shape[0]
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        n_sel = rows_arr.shape[0]
    out = np.empty((max(n_sel, 1), D), np.float64)
    rc = lib.oracle_apply_rows(code, k, len(slice_d), _ptr(slice_d), n_slots, _ptr(rank),
                               _ptr(alpha), _ptr(A_cat), _ptr(A_off), _ptr(B_cat), _ptr(B_off),
                               _ptr(ids), _ptr(x), x.shape[1], _ptr(y_in), y_in.shape[1],
                               _ptr(rows_arr), n_sel, _ptr(out), int(n_threads))
    if rc != 0:
        raise ValueError("oracle_apply_rows: bad argument")
    return out[:n_sel]


def merge(dtype: str, k: int, slice_d, rank: int, alpha: float, A, B, W, sign: int = 1,
          n_threads: int = 1, lib=None) -> np.ndarray:
    """fp64 merged (sign +1) or unmerged (sign -1) weight, shape [D, k].

    ``A`` is the slot's shrink factor [n_slices, rank, k], ``B`` its expand
    factor [D, rank], ``W`` the base weight [D, ldw]; float32 values, or bf16
    bit patterns as uint16 when ``dtype == "bf16"``.
    """
    lib = lib or load()
    code = {"f32": F32, "bf16": BF16}[dtype]
    npdt = np.float32 if code == F32 else np.uint16
    slice_d = np.ascontiguousarray(slice_d, dtype=np.int64)
    D = int(slice_d.sum())
    A = np.ascontiguousarray(A, dtype=npdt)
    B = np.ascontiguousarray(B, dtype=npdt)
    W = np.ascontiguousarray(W, dtype=npdt)
    assert A.shape == (len(slice_d), rank, k), A.shape
    assert B.shape == (D, rank), B.shape
    assert W.shape[0] == D and W.shape[1] >= k, W.shape
    out = np.empty((D, k), np.float64)
    rc = lib.oracle_merge(code, k, len(slice_d), _ptr(slice_d), int(rank), float(alpha), _ptr(A),
                          _ptr(B), _ptr(W), W.shape[1], int(sign), _ptr(out), int(n_threads))
    if rc != 0:
        raise ValueError("oracle_merge: bad argument")
    return out


def apply_grouped(dtype: str, k: int, slice_d, slot_rank, slot_alpha, A, B, ids, x, y_in) -> np.ndarray:
    """fp64 adapted output of every row, shape [n, D], grouped per adapter.

    Page "LoRA hot-loading and adapter routing", batched multi-adapter
    execution section: one group of row indices per adapter id in the batch;
    for each group the inputs are gathered, passed through the adapter's
    shrink and expand factors, scaled by alpha / r and added into those rows of
    the base output; rows without an adapter (id -1, or an id naming no loaded
    adapter) keep the base output.  Arguments as :func:`apply_rows` (bf16 as
    uint16 bit patterns); x [n, >= k], y_in [n, >= D].
    """
    from .compare import to_f64
    slice_d = [int(d) for d in slice_d]
    D = sum(slice_d)
    n = len(ids)
    xf = to_f64(np.asarray(x)[:, :k], dtype)
    out = to_f64(np.asarray(y_in)[:, :D], dtype).copy()
    groups = {}
    for i in range(n):
        s = int(ids[i])
        if 0 <= s < len(slot_rank) and int(slot_rank[s]) > 0:
            groups.setdefault(s, []).append(i)
    for s, rows in groups.items():
        r = int(slot_rank[s])
        scale = float(slot_alpha[s]) / r
        a = to_f64(np.asarray(A[s]), dtype).reshape(len(slice_d), r, k)
        b = to_f64(np.asarray(B[s]), dtype).reshape(D, r)
        xg = xf[rows]                        # the group's inputs, [n_g, k]
        off = 0
        for q, d in enumerate(slice_d):
            v = xg @ a[q].T                  # shrink: [n_g, r]
            out[rows, off:off + d] += scale * (v @ b[off:off + d].T)   # expand, scaled
            off += d
    return out
