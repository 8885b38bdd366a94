"""FP64 CPU oracle for paged-FP8 MLA decode.

Test infrastructure only: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import it; the HIP library and its binding never do, and
this package imports nothing from them.  Every function is pinned by tests in
``tests/test_oracle_*.py`` (see the module docstring of ``mla_oracle`` for the
definitions and the readings it follows).
"""

from .mla_oracle import (  # noqa: F401
    E4M3FN_TABLE,
    attention_rows,
    bf16_round,
    decode,
    decode_ragged,
    decode_range,
    e4m3fn_value,
    gather_dequant,
    merge_partials,
    resolve,
)
from .kv_append import FP8_MAX, append_kv, e4m3fn_round, quantize_row  # noqa: F401
from .unquantized import decode_unquantized, gather_rows  # noqa: F401
