"""Tiered KV-cache decode hot path for AMD Instinct MI355X (gfx950).

The compute lives in ``libtkv.so`` (hand-written HIP behind a C ABI declared in
``include/tkv.h``); :mod:`tiered_kv_cache_amd.tkv` is its Python binding and
:mod:`tiered_kv_cache_amd.driver` the decode state machine built on it.  Importing
this package loads nothing; the library is opened on first use.
"""
__version__ = "0.1.0"
