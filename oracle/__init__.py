"""fp64 CPU oracle for the paged / ragged attention hot path.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg, never by the library. See ``oracle.ref``.
"""
from .ref import (MASK_BLOCK_CAUSAL, MASK_CAUSAL, MASK_NONE, attend, gather_pages,  # noqa: F401
                  merge_states, paged_attention, ragged_attention, request_lengths,
                  run_workload, to_f64, visible)
