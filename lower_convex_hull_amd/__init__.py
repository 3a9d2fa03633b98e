"""MI355X-native batched weighted isotonic regression (gfx950 HIP kernels behind a C ABI)."""
