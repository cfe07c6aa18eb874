"""SLA2 sparse-linear attention forward for MI355X (gfx950).

The compute path is the HIP library ``libsla2.so`` behind a C ABI
(``include/sla2.h``); ``sparse_linear_attention_amd.sla2`` is a thin ctypes
binding over it (argument marshalling only).  Importing this package does not
load the library; the first call through the binding does, and fails loudly if
it is missing.
"""
__all__ = ["inputs", "sla2"]
