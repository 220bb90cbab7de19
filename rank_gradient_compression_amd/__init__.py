"""PowerSGD bucket compression for MI355X (gfx950): a C-ABI HIP library
(libpowersgd.so, declared in include/powersgd.h) and its thin Python binding."""
from .powersgd import (POWERSGD_BF16, POWERSGD_F16, POWERSGD_F32, PowerSGDError,
                       PowerSGDState, PreparedViews, load_library, powersgd_batched_side)

__all__ = ["POWERSGD_BF16", "POWERSGD_F16", "POWERSGD_F32", "PowerSGDError", "PowerSGDState",
           "PreparedViews", "load_library", "powersgd_batched_side"]
