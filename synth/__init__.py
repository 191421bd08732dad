"""Seeded synthetic workloads for the MSA forward path.

This module only draws random inputs and describes the workload shapes; it holds
none of the method's arithmetic. Both the CPU oracle's tests and the HIP path's
tests/benchmark take their inputs from here, so that the two sides read the very
same bits.

Recipe (fixed generation order q_idx, k_idx, stripes, Q, K, V from one seeded
torch.Generator on the target device):

* q_idx ``[B, N, Hkv, Di]`` and k_idx ``[B, N, Di]``: integers drawn uniformly
  from {-4, ..., 4}, stored in the workload's dtype. Integer values keep every
  index score exact in fp32 (|score| <= Di * 4 * 7 < 2**24), which makes the block
  selection a well-defined integer problem on both sides.
* Optional long-range stripes: round(frac * nb) key blocks chosen without
  replacement get +bias added to every component of k_idx for all Bk of their
  tokens (so a learned indexer's "stripe" pattern shows up in the selection).
* Q ``[B, N, Hq, D]``, K and V ``[B, N, Hkv, D]``: standard normal, drawn in fp32
  and rounded to the workload dtype (round-to-nearest-even for bf16).
* Decode batches: caches of capacity N per sequence drawn as above, one new
  query per sequence, cached lengths uniform on [1, N] (``make_decode_inputs``).
"""
from .configs import CONFIGS, DECODE_CONFIGS, Workload, get_workload
from .inputs import (make_inputs, make_decode_inputs, make_grad_output, make_row_weights, sample_rows,
                     uniform_rows, edge_positions, to_fp4_e2m1)

__all__ = ["CONFIGS", "DECODE_CONFIGS", "Workload", "get_workload", "make_inputs", "make_decode_inputs",
           "make_grad_output", "make_row_weights",
           "sample_rows", "uniform_rows",
           "edge_positions", "to_fp4_e2m1"]
