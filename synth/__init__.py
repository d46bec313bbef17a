"""Seeded synthetic inputs shared by the oracle tests, the HIP parity tests
and the benchmark.  Holds no arithmetic of the method itself."""
from .workloads import (WORKLOADS, Workload, Chunk, CacheState, gen_chunk,
                        empty_state, prefilled_state, steady_state, partial_state, to_bf16,
                        bf16_bits_to_f32, chunk_start)

__all__ = ["WORKLOADS", "Workload", "Chunk", "CacheState", "gen_chunk",
           "empty_state", "prefilled_state", "steady_state", "partial_state", "to_bf16",
           "bf16_bits_to_f32", "chunk_start"]
