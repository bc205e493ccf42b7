"""CPU oracle for Cut Cross-Entropy: test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this package.
The GPU library never calls it and shares no code with it."""
from .cce_oracle import *  # noqa: F401,F403
