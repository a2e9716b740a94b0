"""CPU oracle for the W4A16 path (test infrastructure only; the product path
never imports it)."""
from .w4a16_ref import *  # noqa: F401,F403
from .w4a16_ref import GROUP, QMAX, QMAX8, REL_L2_TOL, ELEM_TOL  # noqa: F401
