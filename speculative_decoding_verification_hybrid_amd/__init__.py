"""Tree-verification attention (Hybrid Tree Attention) for MI355X.

The kernels live in ``libhta.so`` (HIP, gfx950) behind the C ABI of
``include/hta.h``; :mod:`.hta` is the thin ctypes binding with the same
function names.
"""

from . import hta  # noqa: F401
