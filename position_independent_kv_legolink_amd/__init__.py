"""piclink: the link step of position-independent KV caching on MI355X (gfx950).

Python face of libpiclink.so (include/piclink.h). The library must be built
(``__graft_entry__.build()``); nothing here falls back to another
implementation.
"""
from .binding import (DTYPES, STATIC_SCRATCH_BYTES, LinkRequest, Plan, PicError, Store, link_attend,
                      link_attend_static, link_decode, lib)

__all__ = ["DTYPES", "STATIC_SCRATCH_BYTES", "LinkRequest", "Plan", "PicError", "Store", "link_attend",
           "link_attend_static", "link_decode", "lib"]
