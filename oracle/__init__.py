"""fp64 CPU oracle (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this
package.  The HIP library never calls it and shares no code with it.
"""
from .relpos_oracle import (ALL_MECHS, MECHS, Params, allowed_mask, backward, backward_head,
                            backward_chunk, backward_head_chunked, bias_rows, finish_chunks,
                            dq_rows, forward, forward_rows, index_maps, scores_rows, t5_bucket,
                            row_chunks, sum_chunks, t5_bucket_by_offset, table_shapes,
                            txl_rows)

__all__ = ["ALL_MECHS", "MECHS", "Params", "allowed_mask", "backward", "backward_head",
           "backward_chunk", "backward_head_chunked", "bias_rows", "finish_chunks",
           "dq_rows", "forward", "forward_rows", "index_maps", "scores_rows", "t5_bucket",
           "row_chunks", "sum_chunks", "t5_bucket_by_offset", "table_shapes", "txl_rows"]
