"""paged_kv_amd -- quantized flash-attention forward for MI355X (gfx950).

The compute lives in the HIP library ``libattnq.so`` (C ABI declared in
``include/attnq.h``); ``paged_kv_amd.api`` is a thin ctypes binding with the
same entry-point names.  Importing this package does not load the library;
the first call does, and fails loudly if it has not been built
(``python -m paged_kv_amd.build``).
"""
from . import api  # noqa: F401
from .api import *  # noqa: F401,F403
