"""Seeded synthetic inputs shared by the oracle side and the device side.

This package holds no attention, softmax, allocation or scatter arithmetic.
It only draws random numbers and describes workloads as data:

* ``draws``      -- seeded N(0,1) draws rounded to the storage dtype
                    (fp32 as-is, bf16 by round-to-nearest-even), returned as
                    raw bit patterns plus exact float64 values; free-list
                    permutations.
* ``workloads``  -- the benchmark / parity workloads as lists of allocator
                    operations (add, append, fork, decode) with their shapes.

Both the oracle-driven tests and the HIP path consume exactly these values,
so inputs are identical on both sides by construction.
"""

from .draws import (  # noqa: F401
    BF16,
    F32,
    bits_to_f64,
    f32_to_bf16_bits,
    free_order,
    normal_bits,
    token_rows,
)
from .workloads import WORKLOADS, Workload, get_workload  # noqa: F401
