"""MI355X (gfx950) exact attention: FlashAttention-2 forward and backward on HIP."""
