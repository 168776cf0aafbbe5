"""NF4 + double-quantized QLoRA frozen-base linear layer for AMD MI355X (gfx950).

The compute path lives in ``libqlora.so`` (hand-written HIP kernels behind a
C ABI, declared in ``include/qlora.h``); ``bit_nf4_quantized_qlora_amd.qlora``
is the thin ctypes binding with the same call names.  Importing this package
does not load the library; importing ``.qlora`` does, and fails loudly if it
has not been built.
"""
__all__ = ["inputs"]
