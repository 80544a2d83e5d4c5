"""fp64 CPU oracle for packed gated-delta-rule prefill, checkpoints, conv and
decode.  Test infrastructure only: the tests, the smoke check and the CPU
baseline leg of the benchmark use it; the library never does."""
from .gdn_oracle import *  # noqa: F401,F403
