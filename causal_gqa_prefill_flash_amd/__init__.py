"""Causal GQA prefill and varlen SDPA for MI355X (gfx950)."""
