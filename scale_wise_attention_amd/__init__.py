"""Next-scale (scale-wise) attention for visual-autoregressive generation on MI355X.

The compute lives in ``libvarattn.so`` (HIP kernels for gfx950 behind a C ABI
declared in ``include/var_attn.h``).  ``scale_wise_attention_amd.api`` is a
thin ctypes binding over it; it is imported lazily so that the seeded input
generators in ``scale_wise_attention_amd.inputs`` stay importable without the
native library.
"""

__all__ = ["api", "inputs"]


def __getattr__(name):
    if name == "api":
        from . import api
        return api
    if name == "inputs":
        from . import inputs
        return inputs
    raise AttributeError(name)
