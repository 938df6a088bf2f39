"""Tree-masked speculative verification on AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library libsvt.so (HIP kernels, see
include/svt.h); `svt` is its thin Python binding.
"""
from . import svt  # noqa: F401
