"""libsmoe: routed-expert MoE layer over a speculative window, HIP for MI355X.

The HIP library (libsmoe.so, built from csrc/ with hipcc for gfx950) does
all of the work; this package is its thin Python binding (`_lib`, same
names as the C entry points) and a layer runner that sequences the calls
(`layer.DeviceLayer`). Importing the binding fails loudly if the library
has not been built.
"""

import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libsmoe.so")


def lib():
    """Import and return the ctypes binding (loads libsmoe.so)."""
    from . import _lib
    return _lib
