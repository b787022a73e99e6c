"""MI355X-native Qwen3 decoder-layer forward (HIP kernels for gfx950 behind a C ABI)."""
