"""KIVI grouped KV-cache codec for AMD MI355X (gfx950).

The codec runs in hand-written HIP kernels behind the C ABI of ``libkivi``
(declared in ``include/kivi.h``); this package is the thin Python binding
over it.
"""
