"""fp64 CPU oracle for the block-sparse attention path.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the CPU
baseline leg of the benchmark, never by the library's product path.  It
shares no code with the HIP library.
"""

from .msa_oracle import *  # noqa: F401,F403
