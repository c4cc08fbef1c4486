"""MI355X-native CARVE chunk-parallel layer (HIP kernels for gfx950 behind a C ABI): forward
pass, backward pass and decode step.

`chunk_fwd`, `chunk_bwd`, `recurrent_step` and `recurrent_ref_shapes` are imported lazily so that the input
generator (`workloads`) and the build script work without torch or the
compiled library.
"""

__all__ = ["chunk_fwd", "chunk_bwd", "recurrent_step", "recurrent_ref_shapes"]


def __getattr__(name):
    if name in __all__:
        from . import api
        return getattr(api, name)
    raise AttributeError(name)
