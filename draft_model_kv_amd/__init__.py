"""Draft-KV ring of a block-diffusion speculative decoder, MI355X-native.

The ring path (append with absolute RoPE, window mask, masked GQA attention
of the noise block, and the new rows' K/V projected from a feature mirror)
runs in HIP kernels for gfx950 behind the C ABI declared in
include/ring_kv.h; ``draft_model_kv_amd.ring`` is its Python binding.
"""

from .ring import (Ring, RingConfig, RingError, RingGeometry, RingKvWeights, RingPlan,
                   make_config, ring_attn, ring_attn_noalloc, ring_begin_step, ring_begin_step_batch,
                   ring_begin_step_deferred, ring_begin_step_mirror, ring_begin_step_mirror_registered,
                   ring_set_kv_weights,
                   ring_describe, ring_free, ring_init, ring_last_error, ring_mirror_write,
                   ring_mirror_write_deferred,
                   ring_plan_from_state, ring_plan_step, ring_query_geometry, ring_read_mask,
                   ring_read_mask_swa, ring_read_rows, ring_read_slot_pos, ring_read_state,
                   ring_profile_enable, ring_profile_read, ring_profile_floor,
                   ring_profile_floor_timeouts, RING_KERNEL_STEP, RING_KERNEL_ATTN,
                   RING_KERNEL_MERGE, RING_KERNEL_PROJ, RING_KERNEL_FLOOR, RING_FLOOR_EMPTY,
                   RING_FLOOR_READ, RING_FLOOR_PARTIALS, RING_FLOOR_LAST_ARRIVER,
                   RING_FLOOR_BARRIER, RING_FLOOR_TWO_LAUNCH, RING_FLOOR_HOLD,
                   RING_FLOOR_MATRIX_MATH, RING_FLOOR_VECTOR_MATH, RING_FLOOR_PROJ_READ,
                   RING_FLOOR_READ_LOCKSTEP, RING_FLOOR_SHARED_TILES, ring_profile_stamps,
                   RING_STAMPS_ATTN,
                   RING_STAMPS_MERGE, RING_STAMPS_PROJ, RING_STAMP_WAVES, RING_STAMP_WORDS)

__all__ = ["Ring", "RingConfig", "RingError", "RingGeometry", "RingKvWeights", "RingPlan",
           "make_config", "ring_attn", "ring_attn_noalloc", "ring_begin_step", "ring_begin_step_batch",
           "ring_begin_step_deferred",
           "ring_begin_step_mirror", "ring_begin_step_mirror_registered", "ring_set_kv_weights",
           "ring_describe", "ring_free", "ring_init", "ring_last_error", "ring_mirror_write",
           "ring_mirror_write_deferred",
           "ring_plan_from_state", "ring_plan_step", "ring_query_geometry", "ring_read_mask",
           "ring_read_mask_swa", "ring_read_rows", "ring_read_slot_pos", "ring_read_state",
           "ring_profile_enable", "ring_profile_read", "ring_profile_floor",
           "ring_profile_floor_timeouts", "RING_KERNEL_STEP", "RING_KERNEL_ATTN",
           "RING_KERNEL_MERGE", "RING_KERNEL_PROJ", "RING_KERNEL_FLOOR", "RING_FLOOR_EMPTY",
           "RING_FLOOR_READ", "RING_FLOOR_PARTIALS", "RING_FLOOR_LAST_ARRIVER",
           "RING_FLOOR_BARRIER", "RING_FLOOR_TWO_LAUNCH", "RING_FLOOR_HOLD",
           "RING_FLOOR_MATRIX_MATH", "RING_FLOOR_VECTOR_MATH", "RING_FLOOR_PROJ_READ",
           "RING_FLOOR_READ_LOCKSTEP", "RING_FLOOR_SHARED_TILES", "ring_profile_stamps",
           "RING_STAMPS_ATTN",
           "RING_STAMPS_MERGE", "RING_STAMPS_PROJ", "RING_STAMP_WAVES", "RING_STAMP_WORDS"]
