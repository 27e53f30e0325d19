"""Seeded synthetic inputs for absorbed-MLA decode.

This package only draws random numbers and encodes them into the byte layouts the
library reads (bf16 bits, FP8 E4M3 codes, packed E2M1 + E4M3 scales, page pools and
block tables).  It holds none of the decode arithmetic: it serves both the float64
oracle and the HIP library, which never import each other.
"""

from .gen import *  # noqa: F401,F403
