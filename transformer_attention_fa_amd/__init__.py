"""MI355X-native exact attention: tiled prefill and split-KV decode (HIP, gfx950)."""
