"""ctypes binding of include/lora.h -- argument marshalling only.

Every function has the name of the C entry point it calls.  Pointers are plain
integers (e.g. ``tensor.data_ptr()``), streams are ``hipStream_t`` values as
integers (``torch.cuda.current_stream().cuda_stream``) or None for the default
stream.  A non-OK status raises :class:`LoraError`.  There is no fallback: if
the HIP library has not been built, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

from .build import LIB_PATH

LORA_F32, LORA_BF16 = 0, 1
LORA_OK, LORA_E_ARG, LORA_E_RANK, LORA_E_SLOT, LORA_E_OCCUPIED, LORA_E_EMPTY = 0, 1, 2, 3, 4, 5
LORA_E_NOMEM, LORA_E_HIP, LORA_E_BAD_IDS, LORA_E_UNSUPPORTED = 6, 7, 8, 9
LORA_E_CAPACITY, LORA_E_NOT_FOUND = 10, 11
RES_STATS = ("hits", "loads", "evictions", "host_drops", "bytes_loaded", "host_entries",
             "resident")
STATUS_NAMES = {0: "LORA_OK", 1: "LORA_E_ARG", 2: "LORA_E_RANK", 3: "LORA_E_SLOT",
                4: "LORA_E_OCCUPIED", 5: "LORA_E_EMPTY", 6: "LORA_E_NOMEM", 7: "LORA_E_HIP",
                8: "LORA_E_BAD_IDS", 9: "LORA_E_UNSUPPORTED", 10: "LORA_E_CAPACITY",
                11: "LORA_E_NOT_FOUND"}

# Every symbol include/lora.h declares, in header order.
EXPORTS = ("lora_stack_create", "lora_stack_destroy", "lora_load_slot", "lora_evict_slot",
           "lora_slot_info", "lora_merge_slot", "lora_segments_create", "lora_segments_destroy",
           "lora_segments_set_dense_min", "lora_segments_set_expand_chunks",
           "lora_segments_set_wait_limit",
           "lora_build_segments", "lora_add_shrink",
           "lora_add_expand", "lora_apply", "lora_build_shrink", "lora_build_apply",
           "lora_build_apply_noalloc", "lora_build_apply_plan",
           "lora_residency_create", "lora_residency_destroy", "lora_residency_register",
           "lora_residency_unregister", "lora_residency_map_batch", "lora_residency_slot_of",
           "lora_residency_stats",
           "lora_segments_download",
           "lora_get_device_status",
           "lora_segments_tile_counts", "lora_status_string")

_lock = threading.Lock()
_lib = None


class LoraError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        self.where = where
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} "
                         f"({_status_text(status)})")


def _status_text(status: int) -> str:
    try:
        return load().lora_status_string(status).decode()
    except Exception:  # pragma: no cover - library not loadable
        return "?"


def load(path: str | None = None):
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        # another build of the same library (the host-sanitized CPU test build)
        p = path or os.environ.get("RANK_ADAPTER_GEMM_LORA_LIB") or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(f"HIP library not built: {p} is missing "
                               "(run `python -m rank_adapter_gemm_lora_amd.build`)")
        # torch's wheel carries its own HIP runtime: load it first so the
        # library binds to that one (opened before torch, it binds to the
        # system runtime, and its allocations then fail)
        import torch  # noqa: F401
        lib = ctypes.CDLL(p)
        P, I, I64, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
        PP = ctypes.POINTER(ctypes.c_void_p)
        sig = {
            "lora_stack_create": [PP, I, I, I, I64, I, P, I64],
            "lora_stack_destroy": [P],
            "lora_load_slot": [P, I, I, F, P, P, I, P],
            "lora_evict_slot": [P, I, P],
            "lora_slot_info": [P, I, P, P, P],
            "lora_merge_slot": [P, I, P, I64, I, P],
            "lora_segments_create": [PP, I64, I],
            "lora_segments_destroy": [P],
            "lora_segments_set_dense_min": [P, I],
            "lora_segments_set_expand_chunks": [P, I],
            "lora_segments_set_wait_limit": [P, I],
            "lora_build_segments": [P, P, I64, P, P],
            "lora_add_shrink": [P, P, I64, P, P],
            "lora_add_expand": [P, P, I64, P, P],
            "lora_apply": [P, P, I64, P, I64, P, P],
            "lora_build_shrink": [P, P, I64, P, I64, P, P],
            "lora_build_apply": [P, P, I64, P, I64, P, I64, P, P],
            "lora_build_apply_noalloc": [P, P, I64, P, I64, P, I64, P, P],
            "lora_build_apply_plan": [P, I64, P, P],
            "lora_residency_create": [PP, P, I, I, I64, I, P, I, I],
            "lora_residency_destroy": [P],
            "lora_residency_register": [P, I64, I, F, P, P],
            "lora_residency_unregister": [P, I64, P],
            "lora_residency_map_batch": [P, P, I64, P, P],
            "lora_residency_slot_of": [P, I64, P],
            "lora_residency_stats": [P, P],
            "lora_segments_download": [P, P, P, P, P, P],
            "lora_get_device_status": [P, P, P],
            "lora_segments_tile_counts": [P, P, P, P],
        }
        for name, args in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        lib.lora_status_string.argtypes = [ctypes.c_int]
        lib.lora_status_string.restype = ctypes.c_char_p
        if path is None:
            _lib = lib
        return lib


def _check(status: int, where: str):
    if status != LORA_OK:
        raise LoraError(status, where)


def _stream(stream):
    return None if stream is None else ctypes.c_void_p(int(stream))


def lora_stack_create(dtype: int, n_slots: int, r_max: int, k: int, slice_d, max_rows: int):
    sd = (ctypes.c_int64 * len(slice_d))(*[int(d) for d in slice_d])
    out = ctypes.c_void_p()
    _check(load().lora_stack_create(ctypes.byref(out), int(dtype), int(n_slots), int(r_max),
                                    int(k), len(slice_d), ctypes.cast(sd, ctypes.c_void_p),
                                    int(max_rows)), "lora_stack_create")
    return out


def lora_stack_destroy(stack):
    _check(load().lora_stack_destroy(stack), "lora_stack_destroy")


def lora_load_slot(stack, slot: int, rank: int, alpha: float, A: int, B: int,
                   src_is_host: bool = False, stream=None):
    _check(load().lora_load_slot(stack, int(slot), int(rank), float(alpha), ctypes.c_void_p(A),
                                 ctypes.c_void_p(B), 1 if src_is_host else 0, _stream(stream)),
           "lora_load_slot")


def lora_evict_slot(stack, slot: int, stream=None):
    _check(load().lora_evict_slot(stack, int(slot), _stream(stream)), "lora_evict_slot")


def lora_slot_info(stack, slot: int):
    """(rank, alpha, live_params) of one slot."""
    r, a, p = ctypes.c_int(), ctypes.c_float(), ctypes.c_int64()
    _check(load().lora_slot_info(stack, int(slot), ctypes.byref(r), ctypes.byref(a),
                                 ctypes.byref(p)), "lora_slot_info")
    return r.value, a.value, p.value


def lora_merge_slot(stack, slot: int, W: int, ldw: int, sign: int = 1, stream=None):
    _check(load().lora_merge_slot(stack, int(slot), ctypes.c_void_p(W), int(ldw), int(sign),
                                  _stream(stream)), "lora_merge_slot")


def lora_segments_create(max_rows: int, n_slots: int):
    out = ctypes.c_void_p()
    _check(load().lora_segments_create(ctypes.byref(out), int(max_rows), int(n_slots)),
           "lora_segments_create")
    return out


def lora_segments_destroy(seg):
    _check(load().lora_segments_destroy(seg), "lora_segments_destroy")


def lora_segments_set_dense_min(seg, m_min: int):
    _check(load().lora_segments_set_dense_min(seg, int(m_min)), "lora_segments_set_dense_min")


def lora_segments_set_expand_chunks(seg, chunks: int):
    _check(load().lora_segments_set_expand_chunks(seg, int(chunks)),
           "lora_segments_set_expand_chunks")


def lora_segments_set_wait_limit(seg, polls: int):
    _check(load().lora_segments_set_wait_limit(seg, int(polls)), "lora_segments_set_wait_limit")


def lora_build_segments(stack, ids: int, n_rows: int, seg, stream=None):
    _check(load().lora_build_segments(stack, ctypes.c_void_p(ids), int(n_rows), seg,
                                      _stream(stream)), "lora_build_segments")


def lora_add_shrink(stack, x: int, ldx: int, seg, stream=None):
    _check(load().lora_add_shrink(stack, ctypes.c_void_p(x), int(ldx), seg, _stream(stream)),
           "lora_add_shrink")


def lora_add_expand(stack, y: int, ldy: int, seg, stream=None):
    _check(load().lora_add_expand(stack, ctypes.c_void_p(y), int(ldy), seg, _stream(stream)),
           "lora_add_expand")


def lora_apply(stack, y: int, ldy: int, x: int, ldx: int, seg, stream=None):
    _check(load().lora_apply(stack, ctypes.c_void_p(y), int(ldy), ctypes.c_void_p(x), int(ldx),
                             seg, _stream(stream)), "lora_apply")


def lora_build_shrink(stack, x: int, ldx: int, ids: int, n_rows: int, seg, stream=None):
    _check(load().lora_build_shrink(stack, ctypes.c_void_p(x), int(ldx), ctypes.c_void_p(ids),
                                    int(n_rows), seg, _stream(stream)), "lora_build_shrink")


def lora_build_apply(stack, y: int, ldy: int, x: int, ldx: int, ids: int, n_rows: int, seg,
                     stream=None):
    _check(load().lora_build_apply(stack, ctypes.c_void_p(y), int(ldy), ctypes.c_void_p(x),
                                   int(ldx), ctypes.c_void_p(ids), int(n_rows), seg,
                                   _stream(stream)), "lora_build_apply")


def lora_build_apply_noalloc(stack, y: int, ldy: int, x: int, ldx: int, ids: int, n_rows: int,
                             timeouts: int = 0, stream=None):
    _check(load().lora_build_apply_noalloc(stack, ctypes.c_void_p(y), int(ldy), ctypes.c_void_p(x),
                                           int(ldx), ctypes.c_void_p(ids), int(n_rows),
                                           ctypes.c_void_p(timeouts or None), _stream(stream)),
           "lora_build_apply_noalloc")


def lora_build_apply_plan(stack, n_rows: int, seg) -> int:
    """Kernel launches a lora_build_apply of n_rows makes (host only)."""
    n = ctypes.c_int32()
    _check(load().lora_build_apply_plan(stack, int(n_rows), seg, ctypes.byref(n)),
           "lora_build_apply_plan")
    return n.value


def lora_segments_download(seg, n_rows: int, n_slots: int, stream=None):
    """Host copies: dict(perm, seg_off, active, counts)."""
    import numpy as np
    perm = np.empty(max(n_rows, 1), np.int32)
    seg_off = np.empty(n_slots + 1, np.int32)
    active = np.empty(n_slots, np.int32)
    counts = np.empty(3, np.int32)
    _check(load().lora_segments_download(seg, perm.ctypes.data, seg_off.ctypes.data,
                                         active.ctypes.data, counts.ctypes.data, _stream(stream)),
           "lora_segments_download")
    return dict(perm=perm[:n_rows], seg_off=seg_off, active=active, counts=counts)


def lora_get_device_status(seg, stream=None) -> int:
    """Number of bad ids in the last build (LORA_E_BAD_IDS is not raised)."""
    n = ctypes.c_int64()
    st = load().lora_get_device_status(seg, ctypes.byref(n), _stream(stream))
    if st not in (LORA_OK, LORA_E_BAD_IDS):
        raise LoraError(st, "lora_get_device_status")
    return n.value


def lora_segments_tile_counts(seg, stream=None):
    """(BGMV tiles, SGMV tiles) of the last build."""
    b, s = ctypes.c_int32(), ctypes.c_int32()
    _check(load().lora_segments_tile_counts(seg, ctypes.byref(b), ctypes.byref(s),
                                            _stream(stream)), "lora_segments_tile_counts")
    return b.value, s.value


def lora_residency_create(stack, max_cpu_adapters: int, n_slots: int = 0, r_max: int = 0,
                          k: int = 0, slice_d=(), dtype: int = LORA_BF16):
    """With a stack the shape arguments are ignored; stack=None plans only."""
    sd = (ctypes.c_int64 * max(1, len(slice_d)))(*[int(d) for d in slice_d])
    out = ctypes.c_void_p()
    _check(load().lora_residency_create(ctypes.byref(out), stack, int(n_slots), int(r_max), int(k),
                                        len(slice_d), ctypes.cast(sd, ctypes.c_void_p) if slice_d
                                        else None, int(dtype), int(max_cpu_adapters)),
           "lora_residency_create")
    return out


def lora_residency_destroy(m):
    _check(load().lora_residency_destroy(m), "lora_residency_destroy")


def lora_residency_register(m, adapter_id: int, rank: int, alpha: float, A: int, B: int):
    _check(load().lora_residency_register(m, int(adapter_id), int(rank), float(alpha),
                                          ctypes.c_void_p(A), ctypes.c_void_p(B)),
           "lora_residency_register")


def lora_residency_unregister(m, adapter_id: int, stream=None):
    _check(load().lora_residency_unregister(m, int(adapter_id), _stream(stream)),
           "lora_residency_unregister")


def lora_residency_map_batch(m, row_adapter, stream=None):
    """row_adapter: int64 sequence (-1 = none) -> numpy int32 slot ids."""
    import numpy as np
    ra = np.ascontiguousarray(row_adapter, dtype=np.int64)
    ids = np.empty(ra.shape[0], np.int32)
    _check(load().lora_residency_map_batch(m, ra.ctypes.data, ra.shape[0], ids.ctypes.data,
                                           _stream(stream)), "lora_residency_map_batch")
    return ids


def lora_residency_slot_of(m, adapter_id: int) -> int:
    v = ctypes.c_int(0)
    _check(load().lora_residency_slot_of(m, int(adapter_id), ctypes.byref(v)),
           "lora_residency_slot_of")
    return v.value


def lora_residency_stats(m) -> dict:
    a = (ctypes.c_int64 * len(RES_STATS))()
    _check(load().lora_residency_stats(m, ctypes.cast(a, ctypes.c_void_p)), "lora_residency_stats")
    return dict(zip(RES_STATS, list(a)))


def lora_status_string(status: int) -> str:
    return load().lora_status_string(int(status)).decode()
