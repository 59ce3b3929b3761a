"""CPU oracle for query-guided KV selection.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only the test suite, the smoke check and the
CPU-baseline leg of the benchmark use it.  It shares no code with the HIP
library (no kernels, headers, helpers, tables or constant generators).

Everything here is a plain, slow, fp64 restatement of what the source pages
define; see ``kvsel_oracle`` for the functions and the passage each follows.
"""

from .kvsel_oracle import *  # noqa: F401,F403
