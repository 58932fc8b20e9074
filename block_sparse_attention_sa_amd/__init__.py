"""Block-sparse attention forward for MI355X (gfx950)."""
