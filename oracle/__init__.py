"""CPU oracle of the Engram lookup -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The library path never calls it, and it imports nothing
from the library.
"""
from .engram_oracle import (  # noqa: F401
    DEFAULT_HASH_SEED,
    BLOCK,
    E4M3_TABLE,
    E8M0_TABLE,
    SCALE_FORMATS,
    N_HEADS,
    N_MODULES,
    N_SUB,
    ORDERS,
    ROW_BYTES,
    ROWS_PER_MODULE,
    WINDOW,
    dedup,
    e4m3_value,
    e8m0_value,
    gather_reduce,
    gather_rows,
    gather_weighted,
    hash_addresses,
    lookup,
    multipliers,
    row_scales,
    splitmix64,
    sub_index,
    windows,
)
