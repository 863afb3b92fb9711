"""CPU oracle for exact Lloyd k-means (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
package.  The k-means library never imports it, and it imports nothing from
the library.
"""
from .oracle import (  # noqa: F401
    DTYPES, assign, decode, emeans, fit, lib, load_library, near_tie, num_threads, objective, objective_bits,
    optimal_1d, round_to, update, update_bits, using_library,
)
