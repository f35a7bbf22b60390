"""Blockwise causal attention with RoPE and a packing mask for MI355X (gfx950)."""
