"""MI355X (gfx950) draft correction for block-diffusion drafters.

The hot path is libcorrector.so: hand-written HIP kernels behind a C-ABI
(``include/corrector.h``).  ``draft_correction_amd.corrector`` is a thin ctypes
binding with the same call names; ``draft_correction_amd.device`` moves
NumPy inputs to device tensors in the layout the library reads.
Importing this package loads nothing; the binding loads the library on first
use and raises if it has not been built.
"""

__all__ = ["corrector", "device", "build"]
