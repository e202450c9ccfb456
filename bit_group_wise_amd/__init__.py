"""bit_group_wise_amd: 4-bit group-wise weight quantization on MI355X (gfx950).

The compute path is the C-ABI library ``libq4.so`` (hand-written HIP kernels,
declared in ``include/q4.h``); ``bit_group_wise_amd.q4`` is its thin ctypes
binding.  Importing this package loads nothing; ``bit_group_wise_amd.q4``
loads the library on first use and raises if it has not been built.
"""
