"""MI355X-native MoE token dispatch and combine (gfx950 HIP kernels behind a C ABI)."""
