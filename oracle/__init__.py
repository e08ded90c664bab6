"""CPU oracle for exact softmax attention (fp64 numpy).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
CPU-baseline leg of the benchmark, never by the library or its binding.  It
shares no code with the GPU path.
"""

from .attention import (  # noqa: F401
    allowed_mask,
    attention_backward,
    attention_forward,
    backward_preprocess,
)
from .philox import (  # noqa: F401
    dropout_scale,
    dropout_threshold,
    keep_mask,
    philox4x32_10,
)
