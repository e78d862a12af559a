"""CPU oracle for MLRA decode attention (test infrastructure, not product code).

Plain, slow, float64 NumPy / pure-Python implementations of what the decode
path computes, written from the method's description. Only the tests, the
smoke check and the CPU-baseline leg of the benchmark may import this
package; the product (the HIP library and its Python binding) never does.
It shares no code with the HIP path: both take their inputs from the seeded
generator, which holds none of the method's arithmetic.

Parity status of every function is listed in ``oracle/mlra_oracle.py``,
``oracle/append_oracle.py`` and ``oracle/out_proj_oracle.py``.
"""
from .mlra_oracle import (  # noqa: F401
    paged_gather,
    visible_length,
    mlra_decode,
    mlra_decode_bruteforce,
    mlra_expanded,
    mla_expanded,
)
from .append_oracle import (  # noqa: F401
    rope_rotate,
    round_to_bf16_f64,
    cache_append,
)
from .out_proj_oracle import (  # noqa: F401
    absorb_weights,
    out_projection,
)
