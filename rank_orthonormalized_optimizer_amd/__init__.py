"""MI355X-native Dion optimizer step: gfx950 HIP kernels behind a C ABI.

Dion ("Dion: Distributed Orthonormalized Updates", reviewed on rivista.ai in
"Dion e la fine del monopolio di Adam negli optimizer AI distribuiti")
orthonormalizes only the top-r directions of each 2-D weight's update by one
amortized power-iteration step with QR/Cholesky, and keeps the rest in an
error-feedback momentum.  This package is the thin Python face of the C ABI:
torch supplies device memory and the current stream, and every step of the
computation runs in the library's kernels.  1-D parameters (biases, norms) are
not Dion's: ``group_matrices`` rejects them, and ``adamw_step_`` / ``lion_step_``
(or ``MixedDion``, which routes every parameter) update them with the library's
element-wise AdamW or Lion, as the page describes.
"""
from __future__ import annotations

from ._lib import (BF16, EXPORTS, F32, FLAG_F64, FLAG_HOUSEHOLDER, FLAG_NONFINITE, FLAG_SHIFTED,  # noqa: F401
                   OPT_EXACT_PRODUCTS, OPT_FORCE_F32, OPT_FORCE_F64, OPT_HOUSEHOLDER, OPT_SPECTRAL_SHIFT,
                   OPT_STICKY_F64, DionError, adamw_step_raw, lambda_max_raw, lambda_max_workspace_size, lion_step_raw, load,
                   step_batched_raw, strerror, version, workspace_size)
from .api import (DionStack, GraphedStep, MixedDion, StickyF64Hint, adamw_step_, group_matrices,  # noqa: F401
                  lambda_max_, lion_step_, step_)
