"""prefill_decode_amd: POD-style fused prefill+decode attention for MI355X.

The library ``libpod_attn.so`` (HIP, gfx950) is loaded on first use by
:mod:`prefill_decode_amd.binding`; importing this package loads nothing, so
host-only modules (``inputs``) import without the library.
"""

__all__ = ["binding", "inputs"]
