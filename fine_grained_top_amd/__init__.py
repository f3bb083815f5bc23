"""libspattn: selective sparse attention on MI355X (gfx950).

The compute path is the HIP library ``libspattn.so`` (C ABI declared in
``include/spattn.h``); ``fine_grained_top_amd.spattn`` is its thin Python
binding. Import the binding explicitly; this package init loads nothing.
"""
__all__ = ["inputs", "metrics", "spattn"]
