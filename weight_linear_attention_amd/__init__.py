"""MI355X (gfx950) fast-weight delta-rule linear attention with DPFP projection.

The compute path is libfwa.so (hand-written HIP kernels behind the C ABI in include/fwa.h);
`weight_linear_attention_amd.fwa` is its Python binding.  Importing this package loads nothing
heavy; `from weight_linear_attention_amd import fwa` binds the library on first use.
"""
__all__ = ["fwa", "synthetic", "build"]
