"""exact_attention_33_amd: fused exact-attention forward for MI355X (gfx950)."""
