"""Paged KV-cache decode path for MI355X (gfx950): HIP kernels behind a C ABI."""
