"""CPU fp64 oracle for exact attention (forward and training backward).

TEST INFRASTRUCTURE. Only the test-suite, the package smoke check and the
benchmark's CPU-baseline leg import this package; the product path (the HIP
library and its Python binding) never does, and this package imports nothing
from the product.

Pages cited in this package:
  [Training-FA]  "Как работает FlashAttention для training (не только
                 inference)?" -- aivaro.ru/en/answers/474
  [Week-13]      "Неделя 13. GPU и FlashAttention" --
                 snula.amonoc.com/course/ru/week-13.html
  [FA-guide]     "FlashAttention: IO Farkındalığı ile Hızlı ve Bellek
                 Açısından Verimli Tam Dikkat" (reading guide to arXiv
                 2205.14135) -- xyznot.com/tr/paper/2205.14135
"""

from .attention import (  # noqa: F401
    MASK_BLOCK,
    keep_matrix,
    forward,
    backward,
    forward_backward,
    forward_rows,
    query_rows,
    key_rows,
    kept_pairs,
)
from . import dropout  # noqa: F401
from .online import (  # noqa: F401
    merge_stats,
    tiled_forward_rescaled,
    tiled_forward_deferred,
)
from . import decode  # noqa: F401
from . import gqa  # noqa: F401
from . import fp8  # noqa: F401
