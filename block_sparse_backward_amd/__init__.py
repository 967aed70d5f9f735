"""LazyFlash-style attention on MI355X (gfx950): dense tiled forward, gradient-
mass-budgeted query-block selection, and a backward over the kept blocks only.

The compute lives in the HIP library ``liblazyflash.so`` (C ABI declared in
``include/lazyflash.h``); ``binding`` marshals torch tensors into it.
"""
__all__ = ["binding", "synth"]
