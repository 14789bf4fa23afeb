"""Content-adaptive block-sparse attention (ASA / ASA_G) for MI355X: the forward layer, its
backward, alternative block selection and estimation, and BSA query pruning.

The computation lives in libdbs.so (hand-written HIP for gfx950, C ABI in
include/dbs.h); this package holds the ctypes binding (`ops`, one wrapper per
entry point) and a layer helper (`layer.AsaLayer`) that chains the calls.
"""
from . import ops  # noqa: F401
from ._lib import DbsError, LIB_PATH, lib  # noqa: F401

__all__ = ["ops", "lib", "LIB_PATH", "DbsError"]
