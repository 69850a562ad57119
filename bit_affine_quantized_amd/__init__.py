"""MI355X-native MLX-affine quantized row product (weight-only low-bit GEMV
for decode windows of 1-16 activation rows).

The product lives in a C-ABI shared library of hand-written HIP kernels for
gfx950 (``csrc/``, declared in ``include/qgemv.h``); ``qgemv`` is its thin
ctypes binding (``from bit_affine_quantized_amd import qgemv``).  ``synth``
draws seeded synthetic inputs.
"""
