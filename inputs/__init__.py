"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This package holds none of the method's arithmetic: it only draws random
numbers (numpy PCG64) and casts fp32 draws to bf16 with torch's own CPU cast.
"""

from .gen import *  # noqa: F401,F403
