"""fp64 CPU oracle (test infrastructure only; never imported by the GPU
library).  See lsa_oracle for the definitions and their sources."""
from .lsa_oracle import *  # noqa: F401,F403
