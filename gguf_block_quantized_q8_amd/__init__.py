"""GGUF block-quantized matmul on MI355X (placeholder during bring-up)."""
