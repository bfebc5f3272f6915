"""Continuous-batching decode forward step for AMD MI355X (gfx950)."""
