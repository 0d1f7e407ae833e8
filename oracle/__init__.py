"""Plain, slow CPU oracle for the collective KV-cache reuse path.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the package smoke check and
the CPU-baseline leg of the benchmark may import anything under ``oracle/``.
The product path (the HIP library and its Python binding) never calls it and
must fail loudly when its compiled library is missing.
"""

from .tdx_oracle import *  # noqa: F401,F403
from .round_oracle import round_plan, segments  # noqa: F401
from . import paged_oracle as paged  # noqa: F401
