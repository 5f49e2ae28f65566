"""fp64 CPU oracle for the KDA decode recurrence (test infrastructure only).

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
import this package; the HIP library neither imports nor links it.
"""
from .kda_oracle import (  # noqa: F401
    DEFAULT_L2_EPS,
    GATE_LOWER_BOUND,
    GATE_SOFTPLUS,
    STATE_K_FIRST,
    STATE_V_FIRST,
    decay,
    decode_tile,
    delta_write,
    gate,
    kda_decode,
    kda_decode_conv,
    l2_normalize,
    read,
    round_to_bf16,
    short_conv,
    sigmoid,
    silu,
    softplus,
    write_strength,
)
