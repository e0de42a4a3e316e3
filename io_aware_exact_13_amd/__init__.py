"""MI355X-native fused exact attention forward (HIP, gfx950)."""
