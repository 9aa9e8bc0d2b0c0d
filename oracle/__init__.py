"""fp64 CPU oracle for exact attention -- test infrastructure only.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never does, and this
package imports nothing from it.
"""

from .attention import (  # noqa: F401
    attention_probs,
    causal_visible,
    kv_head,
    ref_bwd,
    ref_decode,
    ref_decode_paged,
    ref_fwd,
    ref_fwd_rows,
    ref_fwd_tiled,
    ref_merge_partials,
)
from .fp8 import (  # noqa: F401
    E4M3_MAX,
    e4m3_decode,
    e4m3_round,
    fp8_dequantize,
)
