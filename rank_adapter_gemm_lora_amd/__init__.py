"""MI355X-native multi-adapter LoRA apply (placeholder until the binding lands)."""
