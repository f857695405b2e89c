"""MI355X (gfx950) fused HSTU attention forward: Python binding placeholder."""
