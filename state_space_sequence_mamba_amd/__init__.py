"""MI355X-native Mamba-2 SSD chunked scan (gfx950 HIP kernels behind a C ABI)."""
