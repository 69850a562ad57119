"""MI355X-native MLX-affine quantized row product (weight-only low-bit GEMV
for decode windows of 1-16 activation rows).

The product lives in a C-ABI shared library of hand-written HIP kernels for
gfx950 (``csrc/``, declared in ``include/qgemv.h``); ``qgemv`` is its thin
ctypes binding.  ``synth`` draws seeded synthetic inputs.
"""

from . import synth  # noqa: F401

__all__ = ["synth", "qgemv"]


def __getattr__(name):
    if name == "qgemv":
        from . import qgemv as mod
        return mod
    raise AttributeError(name)
