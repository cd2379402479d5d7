"""CPU oracle of the draft-KV ring step: TEST INFRASTRUCTURE ONLY.

Plain, slow, fp64 (or fp32-accumulated) numpy code that states what the ring
step computes, used to check the device path.  Only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may import
it.  It shares no code with the device path (``draft_model_kv_amd``), and
neither imports the other; both read their inputs from ``workload``.
"""

from .ring_oracle import (BULK_CHUNK, FullCache, Geometry, Plan, RingStep,
                          SlotHistory, align_up, attend, geometry, mask_full,
                          noise_positions, plan_step, ring_bytes, rope,
                          rope_inv_freq, rope_rows_f16)

__all__ = ["BULK_CHUNK", "FullCache", "Geometry", "Plan", "RingStep",
           "SlotHistory", "align_up", "attend", "geometry", "mask_full",
           "noise_positions", "plan_step", "ring_bytes", "rope",
           "rope_inv_freq", "rope_rows_f16"]
