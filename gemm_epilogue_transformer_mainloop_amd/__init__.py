"""MI355X-native CODA GEMM-epilogue path: bf16 MFMA GEMMs whose epilogues carry
the non-attention Transformer-block work, exposed through the C-ABI library
``libcoda.so`` and a thin ctypes binding (``coda``).

Importing the package is cheap; the HIP library is loaded on first use of
``gemm_epilogue_transformer_mainloop_amd.coda``.
"""

__all__ = ["coda", "synth"]
