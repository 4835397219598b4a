"""Next-scale (scale-wise) attention for visual-autoregressive generation on MI355X.

The compute lives in ``libvarattn.so`` (HIP kernels for gfx950 behind the C ABI
declared in ``include/var_attn.h``).  Submodules:

* ``scale_wise_attention_amd.api``    -- thin ctypes binding over the library
  (loads it on import; raises if it has not been built).
* ``scale_wise_attention_amd.inputs`` -- seeded synthetic inputs; importable
  without the native library.
* ``scale_wise_attention_amd.build``  -- builds the library with hipcc.

Import the submodule you need explicitly (``from scale_wise_attention_amd import api``).
"""
