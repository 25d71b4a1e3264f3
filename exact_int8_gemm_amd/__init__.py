"""Exact, batch-invariant int8 linear layer for MI355X (gfx950)."""
