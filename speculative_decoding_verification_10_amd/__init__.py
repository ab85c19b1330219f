"""Batched verify step of speculative decoding on AMD Instinct MI355X (gfx950)."""
