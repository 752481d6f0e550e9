"""The C-ABI library loads and exports every symbol include/lora.h declares,
and rejects bad host arguments before touching the GPU (runs without one)."""
import ctypes
import os
import re

import pytest

from rank_adapter_gemm_lora_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "lora.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(lora_\w+)\s*\(", src, flags=re.M)


def test_header_lists_the_binding_exports():
    declared = _declared()
    assert len(declared) == len(set(declared))
    assert tuple(declared) == binding.EXPORTS


def test_library_exports_every_symbol():
    lib = ctypes.CDLL(binding.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name


def test_status_strings():
    for s in range(12):
        assert binding.lora_status_string(s) not in ("", "unknown status")
    assert binding.lora_status_string(99) == "unknown status"


@pytest.mark.parametrize("args,status", [
    ((binding.LORA_BF16, 0, 16, 4096, [4096], 8), binding.LORA_E_ARG),        # no slots
    ((binding.LORA_BF16, 4, 0, 4096, [4096], 8), binding.LORA_E_ARG),         # rank cap 0
    ((binding.LORA_BF16, 4, 16, 4100, [4096], 8), binding.LORA_E_ARG),        # k % 8
    ((binding.LORA_BF16, 4, 16, 4096, [4092], 8), binding.LORA_E_ARG),        # slice % 8
    ((binding.LORA_BF16, 4, 16, 4096, [4096], 0), binding.LORA_E_ARG),        # max_rows
    ((7, 4, 16, 4096, [4096], 8), binding.LORA_E_ARG),                        # dtype
    ((binding.LORA_BF16, 2000, 16, 4096, [4096], 8), binding.LORA_E_UNSUPPORTED),
    ((binding.LORA_BF16, 4, 256, 4096, [4096], 8), binding.LORA_E_UNSUPPORTED),
    ((binding.LORA_BF16, 4, 64, 4096, [1024] * 5, 8), binding.LORA_E_UNSUPPORTED),
])
def test_create_rejects_bad_shapes_on_host(args, status):
    with pytest.raises(binding.LoraError) as e:
        binding.lora_stack_create(*args)
    assert e.value.status == status


def test_null_handles_rejected_on_host():
    lib = binding.load()
    assert lib.lora_stack_destroy(None) == binding.LORA_OK
    assert lib.lora_segments_destroy(None) == binding.LORA_OK
    assert lib.lora_load_slot(None, 0, 1, 1.0, None, None, 0, None) == binding.LORA_E_ARG
    assert lib.lora_evict_slot(None, 0, None) == binding.LORA_E_ARG
    assert lib.lora_slot_info(None, 0, None, None, None) == binding.LORA_E_ARG
    assert lib.lora_segments_set_dense_min(None, 4) == binding.LORA_E_ARG
    assert lib.lora_segments_set_expand_chunks(None, 2) == binding.LORA_E_ARG
    assert lib.lora_build_apply_plan(None, 8, None, None) == binding.LORA_E_ARG
    assert lib.lora_build_segments(None, None, 0, None, None) == binding.LORA_E_ARG
    assert lib.lora_apply(None, None, 8, None, 8, None, None) == binding.LORA_E_ARG
    assert lib.lora_add_shrink(None, None, 8, None, None) == binding.LORA_E_ARG
    assert lib.lora_add_expand(None, None, 8, None, None) == binding.LORA_E_ARG
    assert lib.lora_segments_download(None, None, None, None, None, None) == binding.LORA_E_ARG
    assert lib.lora_get_device_status(None, None, None) == binding.LORA_E_ARG
    assert lib.lora_segments_tile_counts(None, None, None, None) == binding.LORA_E_ARG
    out = ctypes.c_void_p()
    assert lib.lora_segments_create(ctypes.byref(out), 0, 4) == binding.LORA_E_ARG
    assert lib.lora_segments_create(None, 8, 4) == binding.LORA_E_ARG
