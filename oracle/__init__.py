"""CPU oracle of the H2O chunk step -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never does.
"""
from .h2o_oracle import (attention_chunk, attention_chunk_backward, score_accumulate,
                         evict_select, kv_scatter, h2o_step, snapkv_keep,
                         snapkv_compact, quantize_rows_int8, dequantize_rows_int8,
                         attention_chunk_q8, kv_scatter_q8, h2o_step_q8)

__all__ = ["attention_chunk", "attention_chunk_backward", "score_accumulate",
           "evict_select", "kv_scatter", "h2o_step", "snapkv_keep", "snapkv_compact",
           "quantize_rows_int8", "dequantize_rows_int8", "attention_chunk_q8", "kv_scatter_q8",
           "h2o_step_q8"]
