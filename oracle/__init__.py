"""fp64 CPU oracle for the CSA2 layer -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg use
this package; the HIP library never imports or calls it.
"""
from .csa2_oracle import *  # noqa: F401,F403
from .csa2_oracle import (FULL, REINDEX, REUSE, attend, block_pool, decode_bf16,
                          decode_e4m3, dequant, full_row_scores, group_query,
                          index_scores, inverse_rope, layer_query, pool_records,
                          pool_row_scores, rope_rotate, sink_softmax, top_k,
                          visible_records, window_positions)
