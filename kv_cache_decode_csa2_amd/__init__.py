"""CSA2 decode hot path on MI355X (gfx950): HIP kernels behind the C ABI of
include/csa2.h, bound here with ctypes under the same names."""
from .binding import *  # noqa: F401,F403
from .binding import EXPORTS, LIB_PATH, load  # noqa: F401
