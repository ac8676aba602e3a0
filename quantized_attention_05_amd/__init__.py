"""libsattn: SageAttention-style quantized attention for video DiTs, hand-written HIP for MI355X (gfx950)."""
