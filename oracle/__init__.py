"""Float64 CPU oracle (test infrastructure only; see ``paged_oracle``)."""
from .paged_oracle import *  # noqa: F401,F403
