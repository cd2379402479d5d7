// ring_kernels.h -- launch interface between the host runtime and the HIP
// kernels of the draft-KV ring (internal to the library).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ring_layout.h"

#define RING_MAX_SEQ_INTERNAL 64

namespace ringkv {

// One begin_step launch: appends rows [row0, row0 + n_rows) of the step's new
// rows (bulk chunk or fold-in) plus, for a fold-in, n_pad pad rows to the
// trash slot; when do_mask != 0 it also rebuilds slot_pos, the mask and the
// noise RoPE table of the sequence.
struct StepArgs {
  const uint16_t* k_new;     // [n_layer][n_new][kv_row] F16, K not rotated
  const uint16_t* v_new;     // same shape
  uint16_t* kring;           // this sequence's K tiles [n_layer][n_head_kv][n_tiles][4096]
  uint16_t* vring;
  int32_t* slot_pos;         // [cap]
  uint16_t* mask;            // [q_len][kv_total]
  uint16_t* mask_swa;        // [q_len][kv_total] sliding-window mask, or nullptr
  double* rope_noise;        // [q_len][64][2] (cos, sin) at committed + i
  float* rope_q;             // [q_len][64][2] the same values rounded to fp32
  const double* inv_freq;    // [64] theta_i
  int64_t start;             // first new position
  int32_t start_mod;         // start % cap
  int64_t committed;
  int64_t lo;
  int64_t swa_lo;            // committed - min(swa_window, win)
  int32_t n_new;             // rows per layer in k_new / v_new
  int32_t row0;              // first new row this launch appends
  int32_t n_rows;            // real rows this launch appends
  int32_t n_pad;             // pad rows (fold-in only)
  int32_t cap, q_len, kv_total, n_head_kv, n_layer, trash_slot, n_tiles;
  int32_t do_mask;
  uint64_t layer_skip;       // bit l set: no rows for layer l in this launch
  // Rows from projected features instead of k_new / v_new (proj != nullptr):
  // row i of this launch is the sum over the n_ds d-slices of
  // proj[layer][ds][i][0 .. 2 kv_row) (K raw, then V), K normalised per KV
  // head (RMS with eps, times k_norm[layer][dim]) before its rotation.
  const float* proj;         // [n_layer][n_ds][kProjRows][2 * kv_row]
  const float* k_norm;       // [n_layer][128]
  double eps;
  int32_t n_ds;
};

// Fold-in steps of several sequences in one append launch: the fields of
// StepArgs that differ between sequences, per sequence.  Every sequence takes
// blocks_per_seq work-groups (a_step rows of every layer, then the index
// blocks), so that a work-group finds its sequence by one division.
// Positions are below 2^31.
constexpr int kStepBatch = 16;
struct StepBatchArgs {
  StepArgs a;                        // shared geometry; base pointers of sequence 0
  int64_t seq_stride;                // halves between sequences in kring / vring
  int32_t slot_stride;               // int32 per sequence in slot_pos
  int32_t blocks_per_seq;
  int32_t a_step;                    // rows per layer of a fold-in (new rows, then pad rows)
  int32_t n_seq;                     // sequences of this launch, 1..kStepBatch
  int32_t seq[kStepBatch];           // ring sequence index
  int32_t start[kStepBatch];         // first new position
  int32_t start_mod[kStepBatch];     // its slot
  int32_t n_new[kStepBatch];         // new rows (0..a_step)
  int32_t committed[kStepBatch];
  int32_t lo[kStepBatch];
  int32_t swa_lo[kStepBatch];
  uint64_t k_new[kStepBatch];        // [n_layer][n_new][kv_row] F16, not rotated
  uint64_t v_new[kStepBatch];
};

// Projection of new rows' K and V from fused features (one launch projects
// at most kProjRows rows of every layer): raw K and V, in fp32, per d-slice
// of kProjSlice feature dimensions, into the scratch the step kernel reads.
constexpr int kProjRows = 64;
constexpr int kProjSlice = 256;
constexpr int kProjMaxKvHeads = 16;   // KV heads a ring with a feature mirror may have
struct ProjArgs {
  const uint16_t* mirror;    // this sequence's fused features [cap][d_model] F16, slot p % cap
  // A deferred mirror write carried out by this launch, or nullptr: the
  // features of its rows [n_rows][d_model] F16 (row i at position pos0 + i),
  // read from here instead of the mirror and stored into the mirror
  // (mirror_w, the same array) by the work-groups of layer 0, head part 0.
  const uint16_t* feat;
  uint16_t* mirror_w;
  const uint16_t* wk;        // [n_layer][kv_row][d_model] F16 (packed: the packed K and V weights)
  const uint16_t* wv;        // [n_layer][kv_row][d_model] F16 (packed: unused)
  int32_t packed;            // weights in the kernel's load order (pack_weights below)
  float* scratch;            // [n_layer][n_ds][kProjRows][2 * kv_row]
  int64_t pos0;              // position of this launch's row 0
  int32_t slot0;             // its mirror slot, pos0 % cap
  int32_t n_rows;            // rows of this launch, 1..kProjRows
  int32_t cap, d_model, kv_row, n_head_kv, n_layer, n_ds;
  // recip32() of the row tiles, n_ds and 4 n_head_kv (half head parts; set
  // by launch_project)
  uint64_t rcp_n_rt, rcp_n_ds, rcp_n_hh;
};

// Projection weights in the projection kernel's load order: for each work-group
// block (layer, head part hp = K head 0..n_head_kv-1 then V head, d-slice ds,
// wave w) 16 KiB [blk 0..3][j 0..3][lane 0..63][e 0..7] holding
//   W[head row 32 w + lane % 32][dim 256 ds + 64 blk + 32 (lane / 32) + 8 j + e]
// of wk (hp < n_head_kv) or wv, so that each of the wave's 16 loads of 16 B
// per lane reads 1 KiB of consecutive bytes.  Blocks in (layer, hp, ds, w)
// order; the whole is 2 n_layer kv_row d_model halves, as wk and wv.
struct PackArgs {
  const uint16_t* wk;        // [n_layer][kv_row][d_model] F16
  const uint16_t* wv;
  uint16_t* packed;
  int64_t n_chunks;          // 16-byte chunks of the packed weights
  int32_t d_model, kv_row, n_head_kv, n_ds;
};

// Sequences' deferred fold-in steps, carried out by the next attention
// launch of each layer (the fused launch): this layer's new rows, and the
// window the attention sees.  Positions are below 2^31.  Per-sequence fields
// are arrays of kFusedMaxSeq, so that a kernel fetches each with one
// lane-indexed load (lane i holds sequence i % kFusedMaxSeq, a power of two
// at most 64).
constexpr int kFusedMaxSeq = 16;
struct FusedSeqs {
  uint64_t k_new[kFusedMaxSeq];      // this layer's K rows [n_new][kv_row] F16, not rotated, or 0
  uint64_t v_new[kFusedMaxSeq];      // this layer's V rows
  int32_t start[kFusedMaxSeq];       // first new position
  int32_t start_mod[kFusedMaxSeq];   // its slot
  int32_t n_new[kFusedMaxSeq];       // new rows this launch appends for this layer (0: none)
  int32_t committed[kFusedMaxSeq];   // noise positions committed + i
  int32_t lo[kFusedMaxSeq];          // this layer's visible ring positions: [lo, committed)
};

// Quotients by a launch constant d without a division: with
// recip32(d) = ceil(2^32 / d), floor(n / d) = (n * recip32(d)) >> 32 for every
// n with n * d <= 2^32 (the excess n * (recip32(d) - 2^32 / d) / 2^32 stays
// below 1 / d, so it never carries into the integer part).
inline uint64_t recip32(uint32_t d) { return ((uint64_t(1) << 32) + d - 1) / d; }
// floor(n / d) from r = recip32(d), exact for n * d <= 2^32.
__host__ __device__ inline uint32_t quot32(uint32_t n, uint64_t r) {
  return (uint32_t)(((uint64_t)n * r) >> 32);
}

// One ring_attn launch over every sequence of the ring for one layer.
struct AttnArgs {
  uint16_t* kring;           // ring base (all sequences and layers)
  uint16_t* vring;
  const uint16_t* mask;      // [n_seq][q_len][kv_total]
  const double* rope_noise;  // [n_seq][q_len][64][2]
  const float* rope_q;       // [n_seq][q_len][64][2] the same values rounded to fp32
  const uint16_t* q;         // [n_seq][q_len][n_head][128]
  const uint16_t* k_noise;   // [n_seq][q_len][kv_row]
  const uint16_t* v_noise;
  float* out;                // [n_seq][q_len][n_head][128]
  uint16_t* part_acc;        // [n_seq * n_head_kv][n_split][mpad][128] F16: each split's
                             // output normalised by its sum (fragment order)
  float* part_ml;            // [n_seq * n_head_kv][n_split][mpad][2] its (max, sum)
  int64_t seq_stride;        // halves between sequences in kring / vring
  int64_t layer_offset;      // halves from a sequence's base to this layer
  int64_t head_stride;       // halves between KV heads (n_tiles * 4096)
  int32_t n_seq, n_head, n_head_kv, group, q_len, m, cap, kv_total, n_tiles;
  int32_t n_split;
  int32_t n_rb;              // work-groups per (sequence, head, split), one per block of
                             // 32 query rows (one-block kernel; 1 for the others)
  int32_t ring_tiles;        // tiles holding ring slots: ceil(cap / 32)
  // recip32() of the launch's divisors n_split * n_rb, n_rb, n_head_kv,
  // n_split and group, filled in by launch_attn / launch_attn_fused.
  uint64_t rcp_per_unit, rcp_n_rb, rcp_n_head_kv, rcp_n_split, rcp_group;
  // Visible ring tiles of each sequence: vis_count tiles from vis_first on,
  // circularly modulo ring_tiles (the window's slots, slot = position % cap).
  int32_t vis_first[RING_MAX_SEQ_INTERNAL];
  int32_t vis_count[RING_MAX_SEQ_INTERNAL];
  // Cross-split merge inside the launch (kernels whose waves stream several
  // tiles, 2..kInKernelMergeMaxSplits splits): one ticket counter per
  // (sequence x KV head, row block), zero before the launch and left zero by
  // it; nullptr: the partials are merged by launch_merge.  (Last, so that
  // the other fields keep their kernel-argument offsets.)
  uint32_t* tickets;
};

// The fused launch: the attention's arguments plus the deferred steps.  It
// appends the step's rows of this layer and writes their slot_pos entries;
// the masks and the noise RoPE table are rebuilt later, by an append launch
// without rows, before anything reads them (the fused launch does not).
struct FusedAttnArgs {
  AttnArgs a;
  int32_t swa_layer;         // this layer attends with the sliding-window mask
  int32_t n_attn_blocks;     // work-groups of the launch
  int32_t slot_stride;       // int32 per sequence in slot_pos
  double theta[64];          // theta_i, fetched by lane at kernel entry
  int32_t* slot_pos;         // [n_seq][slot_stride]
  FusedSeqs fs;
};

struct MergeArgs {
  const uint16_t* part_acc;  // F16 normalised split outputs (see AttnArgs)
  const float* part_ml;
  float* out;
  int32_t n_units, n_split, n_head, n_head_kv, group, q_len, m, mpad;
  // recip32() of the work-groups per unit, n_head_kv and group, filled in
  // by launch_merge.
  uint64_t rcp_per_unit, rcp_n_head_kv, rcp_group;
};

// Profiling-only floor launches (ring_floor.hip): the attention's grid and
// tile order with a trivial consumer, optionally its partial stores and an
// in-kernel cross-split merge.  Kinds as in ring_floor.hip.
struct FloorArgs {
  const uint16_t* kring;
  const uint16_t* vring;
  int64_t seq_stride, layer_offset, head_stride;
  uint16_t* part_acc;        // the ring's split partials, [unit][split][n_rb * 32][128] F16
  float* part_ml;            // [unit][split][n_rb * 32][2]
  int64_t part_bytes;        // bytes of part_acc (below 2^31 for kinds 3 and 4)
  float* out;                // profiling buffer, [unit * n_rb][32 * 128] fp32
  uint32_t* counter;         // [unit * n_rb] tickets
  uint32_t* err;             // bounded-wait timeouts
  uint32_t epoch;            // kind 4: launches of that kind since the counters were zeroed
  int32_t n_seq, n_head_kv, n_split, n_rb, ring_tiles;
  int32_t rotate;            // the attention's tile walk starts per (unit, split): its waves stream several tiles
  uint64_t rcp_per_unit, rcp_n_rb, rcp_n_head_kv, rcp_n_split;
  int32_t vis_first[RING_MAX_SEQ_INTERNAL];
  int32_t vis_count[RING_MAX_SEQ_INTERNAL];
};

// Floor of the projection launch of a decode step (ring_profile_floor kind
// 9): its grid for one 32-row tile and its weight loads, a trivial consumer.
struct ProjFloorArgs {
  const uint16_t* wpack;     // registered weights, packed (ProjArgs.wk with packed = 1)
  float* out;                // one word per wave
  int32_t n_layer, n_head_kv, n_ds;
  uint64_t rcp_n_ds, rcp_n_hh;  // recip32 of n_ds and 4 n_head_kv (set by the launcher)
};

// t0 / t1: optional events bound to the dispatch (start and end of the
// kernel itself), or nullptr.
hipError_t launch_step(const StepArgs& a, hipStream_t s, hipEvent_t t0, hipEvent_t t1);
hipError_t launch_step_batch(const StepBatchArgs& b, hipStream_t s, hipEvent_t t0, hipEvent_t t1);
hipError_t launch_attn(const AttnArgs& a, hipStream_t s, hipEvent_t t0, hipEvent_t t1);
// Whether launch_attn / launch_attn_fused pick the kernel whose waves attend
// at most one ring tile each (at most 4 tiles per split); that kernel ignores
// a.tickets and always leaves the merge to launch_merge.
bool attn_short_waves(const AttnArgs& a);
constexpr int kInKernelMergeMaxSplits = 16;
// The fused launch: appends and index work of a.fs[] plus the attention.
hipError_t launch_attn_fused(const FusedAttnArgs& f, hipStream_t s, hipEvent_t t0, hipEvent_t t1);
hipError_t launch_merge(const MergeArgs& a, hipStream_t s, hipEvent_t t0, hipEvent_t t1);
hipError_t launch_project(const ProjArgs& a, hipStream_t s, hipEvent_t t0, hipEvent_t t1);
hipError_t launch_floor_proj(const ProjFloorArgs& a, hipStream_t s, hipEvent_t t0, hipEvent_t t1);
hipError_t launch_pack_weights(const PackArgs& a, hipStream_t s);
hipError_t launch_fill_u16(uint16_t* p, uint16_t value, int64_t n, hipStream_t s);

// The static split-partial array of ring_attn_noalloc (ring_kernels.hip):
// its size, the call that resolves its address on `device` (which must be
// current; once per device, thread-safe), and that address (nullptr until
// resolved).
constexpr size_t kStaticScratchBytes = size_t(16) << 20;
hipError_t resolve_static_scratch(int device);
void* static_scratch(int device);
hipError_t launch_floor(const FloorArgs& a, int kind, hipStream_t s, hipEvent_t t0, hipEvent_t t1);

// Per-wave timestamps (profiling build only: the library compiled with
// RING_WAVE_STAMPS, libringkv_stamps.so).  Each wave of the attention, merge
// and projection kernels records the device's constant-rate clock
// (s_memrealtime) at fixed points of its work, and its hardware placement,
// in region `kernel` of a static device array: kStampWords 64-bit words per
// wave (kStampPhases stamps, HW_ID, XCC_ID), wave index = work-group index x
// waves per work-group + wave.  In the product build the kernels record
// nothing and stamps_address returns hipErrorNotSupported.
constexpr int kStampRegions = 3;   // attention (plain and fused), merge, projection
constexpr int kStampWaves = 8192;
constexpr int kStampPhases = 8;
constexpr int kStampWords = kStampPhases + 2;
hipError_t stamps_address(void** ptr);
// Work-groups of the floor kernel that fit the device at once (0 on error).
int floor_resident_blocks();

}  // namespace ringkv
