"""Paged KV cache decode path for MI355X (gfx950)."""
