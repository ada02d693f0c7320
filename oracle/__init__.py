"""CPU oracle of the routed-MoE call: plain, slow, float64, written from the pages.

TEST INFRASTRUCTURE ONLY. Only tests/, the smoke check and the benchmark's
CPU-baseline leg may import this package. The product path (the HIP library
and its Python binding) never imports, calls or links it, and the oracle
shares no code with that path.

Parity pins: every function here is pinned in tests/test_oracle_*.py against
format definitions, an independent library (torch's float8/bf16 casts), closed
forms, brute force and invariants; see the header of each module.
"""

from . import formats, moe  # noqa: F401
