"""CPU oracle of the routed MoE FFN layer -- test infrastructure only.

Importable by the tests, the smoke check and the benchmark's CPU-baseline leg;
never by the product path.  See ``moe_oracle`` for what it computes."""
from .moe_oracle import *  # noqa: F401,F403
from . import moe_oracle  # noqa: F401
