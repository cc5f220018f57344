"""CPU oracle for adaptive block-sparse video attention (routing + plan + attention).

TEST INFRASTRUCTURE ONLY.  Plain, slow NumPy float64 code written from the
method's description; it shares no code with the HIP library.  Only the test
suite, the smoke check and the bench's CPU-baseline leg may import it; the
product path never does.
"""

from .fva_oracle import *  # noqa: F401,F403
from . import fva_balance as balance  # noqa: F401
from . import fva_gsrs as gsrs  # noqa: F401
