"""CPU oracle for the fused MoE expert layer -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the bench's CPU-baseline leg import this
package; the HIP library and its Python binding never do.
"""
from .ref import *  # noqa: F401,F403
