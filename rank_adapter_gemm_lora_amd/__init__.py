"""MI355X-native multi-adapter LoRA apply.

The compute lives in a C-ABI HIP library (include/lora.h, sources in csrc/);
:mod:`.binding` marshals arguments into it (same function names), and
:mod:`.synth` draws seeded synthetic workloads.  PyTorch, where callers use
it, only provides device memory and streams.
"""
from .binding import (EXPORTS, LORA_BF16, LORA_F32, LoraError, lora_add_expand,  # noqa: F401
                      lora_add_shrink, lora_apply, lora_build_apply, lora_build_segments,
                      lora_build_shrink,
                      lora_evict_slot,
                      lora_get_device_status, lora_load_slot, lora_segments_create,
                      lora_segments_destroy, lora_segments_download, lora_segments_set_dense_min,
                      lora_segments_tile_counts, lora_slot_info, lora_merge_slot, lora_stack_create,
                      lora_stack_destroy, lora_status_string, lora_residency_create,
                      lora_residency_destroy, lora_residency_register, lora_residency_unregister,
                      lora_residency_map_batch, lora_residency_slot_of, lora_residency_stats)
