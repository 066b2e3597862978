"""MI355X-native SparseFlashAttentionGrad (gfx950 HIP kernels behind a C ABI)."""
