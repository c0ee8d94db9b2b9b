"""Column-sparse cross-step delta for diffusion transformers on MI355X (gfx950).

The compute lives in ``libchipmunk.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/chipmunk.h``); ``dynamic_column_sparse_amd.lib`` is its
ctypes binding and ``dynamic_column_sparse_amd.layers`` keeps the per-layer
device state for a sampler loop.  Import ``lib`` explicitly: importing this
package alone does not load the library.
"""
__all__ = ["lib", "layers", "build"]
