"""MI355X-native HISA hierarchical indexer and flat DSA indexer.

The compute path is the HIP library ``libhisa.so`` built from ``csrc/``
(C-ABI declared in ``include/hisa.h``); ``hisa`` is its thin ctypes binding.
Importing the package loads nothing; the library is opened on first use and
a missing library raises instead of falling back to anything else.
"""
__all__ = ["hisa", "synth"]
