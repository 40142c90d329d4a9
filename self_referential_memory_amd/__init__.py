"""MI355X-native forward pass of the stabilised SRNL operator (four routes,
row/column-aligned chunks, channel-scale fusion).

The compute path is the HIP library ``libsrnl.so`` (C ABI declared in
``include/srnl.h``); :mod:`self_referential_memory_amd.srnl` is the thin
ctypes binding over it. Importing this package does not load the library.
"""
__all__ = ["srnl", "synth"]
