"""Seeded synthetic inputs shared by the CPU oracle, the tests and the bench.

Holds input generation only (random values, step streams, workload shapes),
none of the ring method's arithmetic.
"""

from .configs import (ACCEPT_SHARES, WORKLOADS, Workload, accepted_counts,
                      commit_stream, context_rows, fused_features, n_warmup_steps,
                      noise_inputs, projection_weights, start_positions, T_K, T_V)

__all__ = ["ACCEPT_SHARES", "WORKLOADS", "Workload", "accepted_counts",
           "commit_stream", "context_rows", "fused_features", "n_warmup_steps",
           "noise_inputs", "projection_weights", "start_positions", "T_K", "T_V"]
