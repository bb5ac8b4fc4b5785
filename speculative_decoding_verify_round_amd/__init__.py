"""MI355X-native speculative-decoding verify round.

The hot path (verify forward, fused LM-head statistics, acceptance, commit)
is hand-written HIP for gfx950 in libspecverify.so behind the C ABI declared
in include/spec_verify.h; `binding` exposes those calls under the same names
and `runtime` holds device buffers in torch tensors.  There is no CPU path:
calls raise if the library is not built.
"""
from . import binding  # noqa: F401
from .binding import LIB_PATH, load_library  # noqa: F401
