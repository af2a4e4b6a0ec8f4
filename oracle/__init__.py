"""Float64 CPU oracle for the looped nGPT forward pass.

Test infrastructure: imported only by tests/, the smoke check and the benchmark's CPU
baseline leg. It shares no code with the HIP library and does not import it.
"""
from .dory_oracle import *  # noqa: F401,F403
from . import mxfp8  # noqa: F401
from . import vocab  # noqa: F401
from . import nvfp4  # noqa: F401
from . import speculative  # noqa: F401
