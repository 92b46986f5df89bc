"""lsv: dense non-causal varlen BF16 attention forward for MI355X (gfx950)."""
