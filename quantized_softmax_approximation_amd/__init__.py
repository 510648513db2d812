"""Quantized-softmax attention forward for MI355X (gfx950)."""
