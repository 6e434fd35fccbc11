"""1.5-entmax attention with a per-row threshold, hand-written HIP for gfx950."""
