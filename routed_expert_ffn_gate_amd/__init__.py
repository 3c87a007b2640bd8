"""MI355X-native MoE routing-and-balancing hot path (libmoelb).

``moelb`` is the ctypes binding of the HIP library (same entry-point names as
``include/moelb.h``); ``layer`` strings the entry points into one layer step.
"""
from . import moelb  # noqa: F401
from .moelb import MoelbError, lib  # noqa: F401

__all__ = ["moelb", "MoelbError", "lib"]
