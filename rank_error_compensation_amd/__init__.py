"""MI355X (gfx950) inference path of group-shared low-rank quantisation-error correction.

The compute lives in libglowq.so (HIP kernels behind the C ABI of include/glowq.h);
``glowq`` is its thin ctypes binding.  Build with ``python -m rank_error_compensation_amd.build``.
"""
from . import glowq  # noqa: F401
