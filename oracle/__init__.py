"""CPU oracle for the SSD scan: float64, plain, slow.  Test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import anything from this package; the product path never does.
"""
from .ssd_oracle import softplus, silu, head_groups, ssd_recurrence, ssd_step_ref, ssd_quadratic  # noqa: F401
from . import ssd_stages, conv1d, gated_norm  # noqa: F401
