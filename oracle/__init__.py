"""CPU oracle for the jagged HSTU encoder (test infrastructure only).

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import this
package; the product path never does. ``hstu_oracle`` is the float64 NumPy
definition of the layer stack; ``brute`` re-derives it with scalar Python loops
for tiny inputs.
"""
from .hstu_oracle import (MacCounter, OracleCache, attention_user, count_macs, encode,  # noqa: F401
                          jagged_offsets, layer_user, normalize_rows, pack_uih, round_bf16, score_head,
                          sigmoid, silu,
                          user_positions, NORM_EPS)
