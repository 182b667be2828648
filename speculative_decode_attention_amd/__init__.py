"""Block-verify decode attention over an int8 paged KV cache, for MI355X (gfx950)."""
