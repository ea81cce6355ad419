"""Exact tiled attention for MI355X (gfx950)."""
