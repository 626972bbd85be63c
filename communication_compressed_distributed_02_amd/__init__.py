"""1-bit Adam's compression-phase step on MI355X (gfx950).

The product is the C-ABI library libob_adam.so (include/ob_adam.h); this
package holds its sources (csrc/), its build script and the thin ctypes
binding (ob_adam.py).  Import the binding explicitly:

    from communication_compressed_distributed_02_amd import ob_adam
"""
