"""MI355X (gfx950) exact attention: tiled forward with online softmax and the
recomputing training backward, behind a C ABI (``include/fa.h``).

Importing the package loads nothing; the HIP library is loaded on the first
call of ``fa_fwd``/``fa_bwd`` and the call fails loudly when it is missing.
"""
