"""CPU oracle of the MoE feed-forward path.  Test infrastructure only: imported by the tests, the
smoke check and the benchmark's CPU-baseline leg, never by the product path."""
from . import moe_oracle  # noqa: F401
