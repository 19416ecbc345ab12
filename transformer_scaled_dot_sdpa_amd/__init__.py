"""MI355X-native scaled dot-product attention forward (HIP, gfx950)."""
