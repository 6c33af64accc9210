"""piclink: the link step of position-independent KV caching on MI355X (gfx950).

Python face of libpiclink.so (include/piclink.h). The library must be built
(``__graft_entry__.build()``); nothing here falls back to another
implementation.
"""
from .binding import (DTYPES, STATIC_SCRATCH_BYTES, LinkRequest, Model, Plan, PicError, Store,
                      forward_workspace_bytes, lib, linear, link_attend, link_attend_layer, link_attend_static,
                      link_decode, link_forward, rmsnorm)

__all__ = ["DTYPES", "STATIC_SCRATCH_BYTES", "LinkRequest", "Model", "Plan", "PicError", "Store",
           "forward_workspace_bytes", "lib", "linear", "link_attend", "link_attend_layer", "link_attend_static",
           "link_decode", "link_forward", "rmsnorm"]
