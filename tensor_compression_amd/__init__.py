"""MI355X-native KVTC-style transform coding of transformer KV caches.

The coded path lives in ``libkvtc.so`` (HIP kernels for gfx950 behind a C
ABI, declared in ``include/kvtc.h``); :mod:`tensor_compression_amd.kvtc` is
the thin ctypes binding.  Importing this package loads nothing: the library
is opened on first use, and the binding raises if it is missing.
"""
__all__ = ["kvtc", "synth"]
