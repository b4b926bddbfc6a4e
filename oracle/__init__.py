"""fp64 CPU oracle of the Dion step: TEST INFRASTRUCTURE ONLY.

Only tests/, the package smoke check and the benchmark's CPU-baseline leg may
import it; the library never does.  ``dion_oracle`` is the fp64 step (LAPACK
Householder QR); ``mp_reference`` is a 50-digit step (modified Gram-Schmidt)
for tiny inputs, used to pin the fp64 step.
"""
from .dion_oracle import (accumulate, column_normalize, dion_step, dion_step_batched,  # noqa: F401
                          error_feedback, power_step, project_back, thin_qr_positive,
                          update_scale, weight_update)
