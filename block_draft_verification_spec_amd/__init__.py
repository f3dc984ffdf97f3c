"""Block speculative verification on MI355X (gfx950).

The computation runs in the HIP library ``libspecverify.so`` behind the C ABI
of ``include/spec_verify.h``; ``binding`` is its thin ctypes binding.
"""

from . import binding  # noqa: F401
from .binding import (  # noqa: F401
    gdn_verify_commit, spec_accept, spec_verify_attention, spec_verify_step)
