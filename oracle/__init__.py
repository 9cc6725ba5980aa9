"""CPU oracle for split-KV decode attention (fp64, NumPy).

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the
HIP library and imports nothing from it.

Every function here is pinned by the CPU tests in ``tests/test_oracle.py``
against facts fixed outside this code (the worked example printed on the
FlashAttention capstone page, closed forms, brute force, an independent
library). The one result left "parity unpinned" is the GPU's own fp32
rounding at 128K tokens, which no closed form fixes; only the tolerance
applies there.
"""

from .attention import (  # noqa: F401
    as_f64,
    attention_row,
    block_stats,
    decode_attention,
    decode_attention_multi,
    decode_partials,
    logical_kv,
    merge_partials,
    merge_two,
    online_softmax_row,
    split_bounds,
)
from .fp8 import decode_e4m3, e4m3_value  # noqa: F401
