"""FlashLoop lazy-update loop attention for MI355X (gfx950).

The GPU work sits in ``libflashloop.so`` (hand-written HIP kernels behind a
C ABI, declared in ``include/flashloop.h``); ``sparse_attention_kv_amd.fl``
is the thin ctypes binding with the same entry-point names.  Importing this
package loads nothing; the binding loads the library on first use and raises
if it is missing.
"""
__all__ = ["synth", "fl"]
