"""CPU oracle for OLMo 3 per-layer hybrid (sliding / full) causal attention.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously correct
statement of what the attention path computes.  Only the test suite, the
smoke check and the benchmark's CPU-baseline leg may import it.  The product
path (the HIP library and its Python binding) never imports, calls or links
anything here, and nothing here imports the product path.

Parity unpinned (shared conventions the pages do not fix, see the module
docstring of ``olmo3_oracle``): the RoPE rotation sign beyond the complex
multiplication convention, the contiguous GQA head grouping, the YaRN ramp
parameters and the 1/sqrt(d) softmax scale.
"""

from .olmo3_oracle import *  # noqa: F401,F403
from .olmo3_oracle import __all__  # noqa: F401
