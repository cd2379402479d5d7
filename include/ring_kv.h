/*
 * ring_kv.h -- C ABI of the DFlash2 draft-KV ring for AMD Instinct MI355X (gfx950).
 *
 * The draft model's K/V cache is a fixed-size circular buffer: the row of
 * absolute position p lives in slot p % cap, K is rotated (RoPE) at its
 * absolute position, and explicit 0 / -inf masks select the window of the last
 * `cap` committed positions.  Attention over the ring is then equal to
 * attention over a full cache restricted to that window.
 *   Source: page "DFLASH2_RING_PORT.md" (DFlash2 draft KV-ring port to
 *   llama.cpp), TL;DR and section 1 ("what the ring does in Luce"): 1.1
 *   geometry, 1.2 mod-cap slot map, 1.3 window and step start, 1.4 attention
 *   masks, 1.5 fixed-topology step, 1.6 driver, 1.7 equivalence and memory.
 *
 * Conventions
 *   - Every call returns RING_OK (0) or a negative RING_E* code and never
 *     aborts; ring_last_error() gives a message for the calling thread.
 *   - Arguments are validated before any device work: a failed call leaves
 *     the ring unchanged.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Device work is enqueued asynchronously on it; device pointers passed in
 *     must stay valid until the stream has passed that work.
 *   - A ring_t may be used by one host thread at a time.
 *   - F16 means IEEE binary16; every device buffer is in the ring's device
 *     memory (the device that was current at ring_init).
 */
#ifndef RING_KV_H
#define RING_KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RING_OK       0
#define RING_EINVAL  (-1)  /* bad argument or unsupported shape               */
#define RING_ERANGE  (-2)  /* sequence, layer or position out of range        */
#define RING_ENOMEM  (-3)  /* allocation failed or workspace too small        */
#define RING_EDEVICE (-4)  /* HIP runtime error                               */
#define RING_ESTATE  (-5)  /* call does not match the ring's state            */

/* Largest number of sequences one ring may hold (their windows travel as
 * kernel arguments). */
#define RING_MAX_SEQ 64

/* Shapes of one ring (all sequences and layers share them).
 *   cap        ring capacity in context slots (last `cap` positions), >= 1
 *   q_len      noise-block length, the draft's block size (8 on the page), 1..32
 *   n_head     query heads; n_head_kv KV heads; n_head % n_head_kv == 0 and
 *              q_len * n_head / n_head_kv <= 64
 *   head_dim   must be 128
 *   n_layer    draft layers, each with its own K and V ring (>= 1)
 *   n_seq      independent sequences, 1..RING_MAX_SEQ
 *   rope_base  RoPE base (theta_i = rope_base^(-2i/head_dim)), > 1
 *   swa_window sliding-window layers (page 1 section 1.4, mask_swa): each
 *              step also builds their mask, whose window is the last
 *              eff_win = min(swa_window, win) committed positions (anchored
 *              at committed for every noise row) and whose noise block is
 *              causal (noise row i sees noise slots j <= i).  0 = no such
 *              layers; else >= 1, and swa_layers must be non-zero.
 *   swa_layers bit l set: layer l attends with that mask; only bits below
 *              min(n_layer, 64) may be set; 0 when swa_window is 0.
 *   d_model    width of the fused feature vector the draft's K/V projection
 *              reads (the page's notes on the port: Luce keeps a mirror of
 *              the target's features whose capacity is the ring's, and
 *              begin_step computes the new rows' K/V from it).  0 = no
 *              feature mirror; else a multiple of 256, at most 65536, and
 *              then n_head_kv <= 16.                                        */
typedef struct ring_config {
  int32_t cap;
  int32_t q_len;
  int32_t n_head;
  int32_t n_head_kv;
  int32_t head_dim;
  int32_t n_layer;
  int32_t n_seq;
  float rope_base;
  int32_t swa_window;   /* sliding-window layers' window; 0 = none        */
  uint64_t swa_layers;  /* bit l set: layer l is a sliding-window layer   */
  int32_t d_model;      /* fused feature width of the mirror; 0 = none    */
} ring_config;

/* Derived geometry (section 1.1 of the page):
 *   a_step     = 2 * q_len + 2, rows one fold-in step appends (real + pad)
 *   trash_slot = cap + q_len, destination of pad rows
 *   kv_total   = align_up(cap + q_len + 1, 32), rows per ring
 *   kv_row     = head_dim * n_head_kv, F16 values per row
 *   kv_bytes_per_layer  K plus V bytes of one (sequence, layer) ring
 *   workspace_bytes     device bytes ring_init needs when the caller
 *                       provides the workspace (with a feature mirror this
 *                       includes the mirror, the projection scratch and room
 *                       for the registered weights, ring_set_kv_weights)    */
typedef struct ring_geometry {
  int32_t a_step;
  int32_t trash_slot;
  int32_t kv_total;
  int32_t kv_row;
  int64_t kv_bytes_per_layer;
  int64_t workspace_bytes;
} ring_geometry;

/* Plan of one begin_step (section 1.3 of the page):
 *   win = min(committed, cap), lo = committed - win,
 *   start = max(next_pos, lo), n_new = committed - start; rows for positions
 *   [start, committed) are appended.  bulk != 0 when n_new > a_step: the rows
 *   go in n_chunks chunks of at most 1024 rows in ascending position;
 *   otherwise they are folded into one fixed a_step-row append whose pad rows
 *   target trash_slot.  After a rewind that dropped window rows the ring no
 *   longer holds, start = lo (the whole window is appended again).          */
typedef struct ring_plan {
  int64_t committed;
  int64_t win;
  int64_t lo;
  int64_t start;
  int64_t n_new;
  int32_t bulk;
  int32_t n_chunks;
} ring_plan;

typedef struct ring ring_t;

/* Pure host: validate `cfg` and fill `out`.  Errors: RING_EINVAL. */
int ring_query_geometry(const ring_config* cfg, ring_geometry* out);

/* Create a ring on the current HIP device.
 *   workspace        device buffer of at least workspace_bytes, 256-byte
 *                    aligned, owned by the caller (must outlive ring_free); or
 *                    NULL to let the library allocate (and free) it.
 *   workspace_bytes  size of `workspace` (ignored when it is NULL)
 * Enqueues on `stream`: zeroing of every K/V ring row (empty slots are read
 * by the attention and must be finite, section 1.1), slot_pos = -1 for every
 * slot, and the index state of committed = 0 for every sequence.
 * Errors: RING_EINVAL (cfg, alignment), RING_ENOMEM (too small / allocation),
 * RING_EDEVICE.  On error *out is left NULL and nothing stays allocated.     */
int ring_init(const ring_config* cfg, void* workspace, size_t workspace_bytes,
              void* stream, ring_t** out);

/* Pure host: the plan the next ring_begin_step(seq, committed) would run.
 * `ap_rows` (nullable) receives, for a fold-in plan, the a_step destination
 * rows: (start + i) % cap for i < n_new, then trash_slot.  For a bulk plan it
 * receives nothing.  Errors: RING_ERANGE (seq, committed).                  */
int ring_plan_step(const ring_t* r, int32_t seq, int64_t committed,
                   ring_plan* out, int32_t* ap_rows);

/* Pure host, no ring needed: the same plan from an explicit state.
 *   next_pos  committed count of the sequence's previous step (0 at first)
 *   held_lo   lo of the previous step (0 at first): the ring then holds
 *             exactly positions [held_lo, next_pos)
 * Errors: RING_EINVAL (cfg, state), RING_ERANGE (committed).                */
int ring_plan_from_state(const ring_config* cfg, int64_t next_pos, int64_t held_lo,
                         int64_t committed, ring_plan* out, int32_t* ap_rows);

/* Append the newly committed rows of sequence `seq` and rebuild its mask.
 *   committed  committed positions after this step (0 <= committed and
 *              committed + q_len <= 2^31 - 1)
 *   k_new      device F16 [n_layer][n_rows][kv_row]: K rows of positions
 *              [start, committed) in ascending order, NOT yet rotated
 *   v_new      device F16, same shape: V rows
 *   n_rows     must equal the plan's n_new (may be 0; then k_new/v_new may
 *              be NULL)
 * Device work (section 1.2-1.4): K rotated at its absolute position p and
 * written with V to slot p % cap of every layer's ring; pad rows of a fold-in
 * write zeros to trash_slot; slot_pos[p % cap] = p; the F16 mask
 * [q_len][kv_total] of the sequence becomes 0 (0x0000) for ring slots with
 * lo <= slot_pos < committed and for the q_len noise slots, -inf (0xFC00)
 * elsewhere; with sliding-window layers their mask too (0 for ring slots
 * with committed - eff_win <= slot_pos < committed, noise slot cap + j for
 * noise rows i >= j); the RoPE table of the noise positions committed + i is
 * rebuilt.
 * Errors: RING_ERANGE, RING_ESTATE (n_rows != n_new), RING_EINVAL (NULL),
 * RING_EDEVICE.                                                             */
int ring_begin_step(ring_t* r, int32_t seq, int64_t committed,
                    const void* k_new, const void* v_new, int64_t n_rows,
                    void* stream);

/* ring_begin_step deferred into the attention launches (fused step).  Same
 * arguments, plan, checks and result as ring_begin_step.  For a fold-in plan
 * nothing is enqueued here: the next ring_attn of each layer appends that
 * layer's rows itself (and attends them as keys of their own, not through
 * the ring tiles that hold their slots) and writes their slot_pos entries,
 * all in its one launch; the masks and the noise RoPE table, which that
 * launch does not read, are rebuilt by an append launch without rows before
 * anything reads them (a plain attention launch, ring_read_mask*, an append
 * of the sequence).  Pad rows are not written (the trash slot keeps its
 * zeros).  k_new and v_new must therefore stay
 * valid until every layer's ring_attn has been enqueued and the stream has
 * passed them.  Whatever a deferred step still owes (layers whose attention
 * has not run) is appended by the ordinary append kernel on the ring's last
 * stream before any other call that needs it: a begin_step of the same
 * sequence and the ring_read_* inspection calls.  A bulk plan, and rings
 * with more than 16 sequences or 64 layers, append right away as
 * ring_begin_step does.
 * Errors: as ring_begin_step.                                               */
int ring_begin_step_deferred(ring_t* r, int32_t seq, int64_t committed,
                             const void* k_new, const void* v_new, int64_t n_rows,
                             void* stream);

/* ring_begin_step for n distinct sequences at once (the batched decode, where
 * every sequence commits its own accepted tokens each step; section 1.3's
 * plan is per sequence).  Entry i is the call
 *   ring_begin_step(r, seqs[i], committed[i], k_new[i], v_new[i], n_rows[i])
 * with host arrays of n entries (the row pointers are device addresses).
 * The result is that of those n calls; the fold-in plans among them are
 * appended together, up to 16 sequences per launch of one append kernel,
 * and bulk plans append as ring_begin_step does.  Every entry is checked
 * before anything is enqueued, so a rejected call changes nothing.
 *   n  0..n_seq (0: nothing to do)
 * Errors: RING_ERANGE (n, a seq, a committed), RING_EINVAL (NULL array or
 * rows, a sequence listed twice), RING_ESTATE (an n_rows != n_new),
 * RING_EDEVICE.                                                             */
int ring_begin_step_batch(ring_t* r, int32_t n, const int32_t* seqs,
                          const int64_t* committed, const void* const* k_new,
                          const void* const* v_new, const int64_t* n_rows,
                          void* stream);

/* ---- New rows from fused features (feature mirror + K/V projection) ----
 * The page's notes on the port describe Luce's begin_step: the draft keeps a
 * mirror of the target's fused feature vectors with the ring's capacity
 * (section 1.6: the ring capacity is the mirror's), and the context K/V of
 * each new position are computed from it per layer as the shallow injection
 * wk/wv @ fused + k_norm + rope (the test log's list of refuted hypotheses,
 * item 4).  Both need a ring created with d_model > 0.                      */

/* Projection weights of every layer, device memory:
 *   wk, wv   F16 [n_layer][kv_row][d_model] (output dim first, feature dim
 *            contiguous), 16-byte aligned
 *   k_norm   F32 [n_layer][head_dim], the learned weight of the K norm
 *   eps      epsilon of the K norm (>= 0)
 * For a position p with fused features f: k = wk f, v = wv f; each KV head's
 * 128 values of k are divided by sqrt(mean of their squares + eps) and
 * multiplied by k_norm; K is then rotated at p (the ring's RoPE) and both are
 * rounded once to F16.  The products accumulate in fp32 on the matrix cores;
 * norm and rotation are done in fp64.                                       */
typedef struct ring_kv_weights {
  const void* wk;
  const void* wv;
  const float* k_norm;
  float eps;
} ring_kv_weights;

/* Store the fused features of positions [pos0, pos0 + n) of sequence `seq`
 * in its mirror: position p goes to mirror slot p % cap (when n > cap only
 * the last cap rows can stay and only those are copied).
 *   features  device F16 [n][d_model]
 * The mirror then holds, for each slot, the position last written to it.
 * Errors: RING_ESTATE (no mirror), RING_ERANGE (seq, positions),
 * RING_EINVAL (NULL), RING_EDEVICE.                                         */
int ring_mirror_write(ring_t* r, int32_t seq, int64_t pos0, int64_t n,
                      const void* features, void* stream);

/* ring_mirror_write whose copy is left to the next projection of the
 * sequence: the same checks and result, but the rows stay in the caller's
 * buffer until then.  When the sequence's next ring_begin_step_mirror
 * projects exactly positions [pos0, pos0 + n) in one launch (a decode step:
 * n = n_new <= 64), that launch reads their features from `features` and
 * also writes them into the mirror, so the step has one launch fewer; any
 * other call that needs them first (another mirror write of the sequence,
 * a begin_step_mirror of other rows) copies them as ring_mirror_write does,
 * on its own stream.  `features` must stay valid and unchanged until that
 * happens.  Errors: as ring_mirror_write.                                   */
int ring_mirror_write_deferred(ring_t* r, int32_t seq, int64_t pos0, int64_t n,
                               const void* features, void* stream);

/* Register the projection weights of every layer once (the draft model's
 * wk / wv and k_norm are constant: the page's test log, item 4 of the list
 * of refuted hypotheses, names the projection as the shallow injection
 * wk/wv @ fused + k_norm + rope).  The library copies wk and wv into its
 * workspace in the order the projection kernel loads them (each wave's
 * 16-byte loads then read consecutive bytes), and k_norm and eps beside
 * them; ring_begin_step_mirror with w == NULL then projects through this copy
 * with the same arithmetic and results as through the caller's weights.  A
 * later call replaces the registered weights.  The copy is enqueued on
 * `stream`; the caller's buffers must stay valid until the stream has passed
 * it.  Errors: RING_ESTATE (no mirror), RING_EINVAL (NULL, alignment, eps),
 * RING_EDEVICE.                                                             */
int ring_set_kv_weights(ring_t* r, const ring_kv_weights* w, void* stream);

/* ring_begin_step with the new rows computed from the mirror: the same plan
 * (positions [start, committed)), every one of which the mirror must hold
 * (else RING_ESTATE before any device work: after a rewind that re-appends
 * the whole window, write the positions the mirror lost again), projected
 * through `w` for every layer as described above (w == NULL: through the
 * weights registered with ring_set_kv_weights) and appended like
 * ring_begin_step's rows (pads, slot_pos, masks and noise RoPE table alike).
 * Errors: RING_ESTATE (no mirror, position missing, w == NULL with no
 * weights registered), RING_ERANGE, RING_EINVAL (NULL weight pointers,
 * alignment, eps), RING_EDEVICE.                                            */
int ring_begin_step_mirror(ring_t* r, int32_t seq, int64_t committed,
                           const ring_kv_weights* w, void* stream);

/* Masked GQA attention of the noise block of every sequence over its ring
 * (one draft layer), section 1.4 masks: the full mask with the noise block
 * visible both ways, or for a sliding-window layer its mask, reading only
 * the ring tiles that hold its window.
 *   q        device F16 [n_seq][q_len][n_head][head_dim], not yet rotated;
 *            query row i sits at absolute position committed + i
 *   k_noise  device F16 [n_seq][q_len][kv_row], noise K, not yet rotated
 *   v_noise  device F16 [n_seq][q_len][kv_row]
 *   out      device F32 [n_seq][q_len][n_head][head_dim]
 * Query head h reads KV head h / (n_head / n_head_kv); scores are scaled by
 * 1/sqrt(head_dim).  The rotated noise K and V are also written to ring rows
 * cap + j of this layer.  Uses each sequence's state from its last
 * begin_step.  Errors: RING_ERANGE (layer), RING_EINVAL (NULL), RING_EDEVICE.
 * The attention is split over ring tiles (split-K) and the splits' partials
 * are merged by a second launch.  Tuning switches, read by ring_init from
 * the environment: RING_ATTN_SPLITS=n forces n splits (1..64);
 * RING_ATTN_ROW_BLOCKS=0 keeps both 32-query blocks of a KV head in one
 * work-group; RING_ATTN_MERGE=kernel merges the splits inside the attention
 * launch where its waves stream several tiles and it has at most 16 splits
 * (the work-group that finishes last merges; counters in the workspace). */
int ring_attn(ring_t* r, int32_t layer, const void* q, const void* k_noise,
              const void* v_noise, float* out, void* stream);

/* ring_attn for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments, checks, kernels and results as ring_attn, but the split
 * partials of the attention (each split's output normalised by its softmax
 * sum in F16, and fp32 (max, sum) pairs, for a launch with more than one
 * split) go to a static array of 16 MiB in the
 * library's device code instead of the ring's workspace.  The call allocates
 * and frees nothing; ring_init resolves the array's address once per device.
 * Every call on one GPU shares that GPU's array: two calls whose work
 * overlaps on the device (different streams, not ordered) race on it, so
 * order them on one stream.  Launches whose partials need more than 16 MiB
 * (n_seq x n_head_kv x splits x 32 or 64 query rows x 264 B) are refused.
 * Errors: as ring_attn, and RING_EINVAL when the partials exceed the array. */
int ring_attn_noalloc(ring_t* r, int32_t layer, const void* q, const void* k_noise,
                      const void* v_noise, float* out, void* stream);

/* Synchronise the ring's last stream and release what the library
 * allocated.  A caller-owned workspace is not freed.  NULL is accepted.    */
int ring_free(ring_t* r);

/* Message of the calling thread's last failed call ("" if none).  The
 * pointer stays valid until the thread's next ring_* call.                  */
const char* ring_last_error(void);

/* One-line summary in the style of the Luce log line (cap, kv_total, a_step,
 * layers, F16 cache MiB) written to buf (always NUL-terminated).           */
int ring_describe(const ring_t* r, char* buf, size_t len);

/* ---- Inspection (synchronous: waits for the device; for tests/tools) ---- */

/* slot_pos of sequence `seq`, int32 [cap], -1 for never-written slots.     */
int ring_read_slot_pos(const ring_t* r, int32_t seq, int32_t* host_out);

/* Mask of sequence `seq`, F16 bit patterns uint16 [q_len][kv_total].        */
int ring_read_mask(const ring_t* r, int32_t seq, uint16_t* host_out);

/* Sliding-window mask of sequence `seq` (same layout); RING_ESTATE when the
 * ring has no sliding-window layers.                                        */
int ring_read_mask_swa(const ring_t* r, int32_t seq, uint16_t* host_out);

/* Rows [slot0, slot0 + n) of the (seq, layer) ring, converted from the
 * device layout to plain rows: F16 bit patterns [n][kv_row] for K (rotated)
 * and for V.  Either output may be NULL.                                    */
int ring_read_rows(const ring_t* r, int32_t seq, int32_t layer, int32_t slot0,
                   int32_t n, uint16_t* k_out, uint16_t* v_out);

/* Host-side state of sequence `seq`: next_pos (= committed of its last step)
 * and held_lo (= that step's lo).                                           */
int ring_read_state(const ring_t* r, int32_t seq, int64_t* next_pos,
                    int64_t* held_lo);

/* ---- Profiling ----
 * Kernel kinds: RING_KERNEL_STEP (append + mask launches of ring_begin_step
 * and ring_begin_step_mirror), RING_KERNEL_ATTN (attention launch of
 * ring_attn), RING_KERNEL_MERGE (cross-split merge launch of ring_attn,
 * absent when one split suffices), RING_KERNEL_PROJ (projection launches of
 * ring_begin_step_mirror), RING_KERNEL_FLOOR (ring_profile_floor).          */
#define RING_KERNEL_STEP  0
#define RING_KERNEL_ATTN  1
#define RING_KERNEL_MERGE 2
#define RING_KERNEL_PROJ  3
#define RING_KERNEL_FLOOR 4

/* Time the next `max_launches` launches of each kernel kind with HIP events
 * bound to the dispatch itself (kernel start to kernel end, no launch gaps).
 * 0 turns profiling off.  Errors: RING_EINVAL, RING_EDEVICE.               */
int ring_profile_enable(ring_t* r, int32_t max_launches);

/* Wait for the timed launches of `kernel` to finish, report how many there
 * were and their summed duration in milliseconds, and start counting anew.
 * Errors: RING_EINVAL, RING_EDEVICE.                                        */
int ring_profile_read(ring_t* r, int32_t kernel, int32_t* n_launches, double* total_ms);

/* ---- Floors of the attention launch (profiling only) ----
 * What bounds one ring_attn launch of `layer` on this hardware, measured with
 * the attention's own launch shape: the same grid (one work-group of four
 * waves per sequence, KV head, split and 32-query block), the same
 * work-group order (a KV head's splits on one XCD) and the same ring tiles
 * per wave from each sequence's window at its last begin_step, with a
 * trivial consumer in place of the attention's arithmetic:
 *   RING_FLOOR_EMPTY         a kernel that returns at once (launch + drain)
 *   RING_FLOOR_READ          every visible K and V tile loaded once with the
 *                            attention's 16-byte loads, folded by xor
 *   RING_FLOOR_PARTIALS      RING_FLOOR_READ plus the 8 KiB F16 split
 *                            partial (and its fp32 max/sum pairs) each
 *                            work-group of the attention stores
 *   RING_FLOOR_TWO_LAUNCH    RING_FLOOR_PARTIALS, then the ring's own merge
 *                            launch over those partials: the data movement
 *                            of ring_attn's two launches (timed as two
 *                            RING_KERNEL_FLOOR launches)
 *   RING_FLOOR_MATRIX_MATH   RING_FLOOR_READ plus, per tile and wave, the
 *                            attention's contractions on the matrix cores:
 *                            16 v_mfma_f32_32x32x16_f16 for the scores (query
 *                            as two F16 halves) and 8 for P V, on the loaded
 *                            K and V fragments
 *   RING_FLOOR_VECTOR_MATH   RING_FLOOR_READ plus the same 393,216 products
 *                            per tile and wave on the vector unit (v_dot2),
 *                            the other side of the matrix-core A/B
 *   RING_FLOOR_PROJ_READ     the projection launch of ring_begin_step_mirror
 *                            for one 32-row tile instead (page's notes on the
 *                            port: the new rows' K/V come from the feature
 *                            mirror through the draft's wk and wv): its grid
 *                            of two-wave work-groups, each wave loading its
 *                            16 KiB of the registered (packed) weights of
 *                            every layer as the projection does, folded by
 *                            xor; `layer` is only range-checked.  Needs
 *                            ring_set_kv_weights first (else RING_ESTATE)
 *   RING_FLOOR_READ_LOCKSTEP RING_FLOOR_READ with every work-group walking
 *                            its split's tiles from the split's first one
 *                            (the attention starts each walk at an offset of
 *                            its own when its waves stream several tiles;
 *                            this kind times the walk without it)
 *   RING_FLOOR_HOLD          one wave that sleeps for about 14 ms (a bounded
 *                            loop) and reads nothing: launches queued behind
 *                            it then run back to back on the device, however
 *                            slowly the host submits them (not timed)
 *   RING_FLOOR_LAST_ARRIVER  RING_FLOOR_PARTIALS with the cross-split merge
 *                            in the same launch: partials stored write-through
 *                            at device scope, one atomic ticket per
 *                            work-group, and the work-group with the last
 *                            ticket of its (sequence, head) sums every
 *                            split's partial
 *   RING_FLOOR_BARRIER       RING_FLOOR_PARTIALS with a bounded barrier per
 *                            (sequence, head): every work-group waits for all
 *                            tickets of its head (at most 2^20 polls, then it
 *                            counts a timeout and goes on), then sums its
 *                            share of every split's partial
 *   RING_FLOOR_SHARED_TILES  (rings with 64 queries per KV head, whose two
 *                            32-query blocks the attention gives work-groups
 *                            of their own, each reading every tile) one read
 *                            of each visible tile for both blocks: a
 *                            work-group of eight waves per (unit, split),
 *                            with as many splits as the attention's grid has
 *                            work-groups per head; each pair of waves copies
 *                            its tile's K and V into LDS with direct
 *                            global-to-LDS loads (two stages, one barrier per
 *                            tile) and both run the attention's 24 matrix
 *                            ops on them, one per query block
 * These launches read the ring but change none of its state or outputs (the
 * split partials are scratch; the sums go to a buffer of their own, which
 * the first floor launch allocates and ring_free releases).  Deferred steps
 * are appended first.  They run on `stream`; ring_profile_enable /
 * ring_profile_read time them as RING_KERNEL_FLOOR.
 * Errors: RING_ERANGE (layer), RING_EINVAL (kind; a launch with one split
 * for the kinds with partials; RING_FLOOR_BARRIER when the grid does not fit the
 * device at once; RING_FLOOR_SHARED_TILES on a ring without two query-block
 * work-groups per head), RING_ENOMEM, RING_EDEVICE.                         */
#define RING_FLOOR_EMPTY        0
#define RING_FLOOR_READ         1
#define RING_FLOOR_PARTIALS     2
#define RING_FLOOR_LAST_ARRIVER 3
#define RING_FLOOR_BARRIER      4
#define RING_FLOOR_TWO_LAUNCH    5
#define RING_FLOOR_HOLD          6
#define RING_FLOOR_MATRIX_MATH   7
#define RING_FLOOR_VECTOR_MATH   8
#define RING_FLOOR_PROJ_READ     9
#define RING_FLOOR_READ_LOCKSTEP 10
#define RING_FLOOR_SHARED_TILES  11
int ring_profile_floor(ring_t* r, int32_t layer, int32_t kind, void* stream);

/* Number of RING_FLOOR_BARRIER waits that ended by their poll limit rather
 * than by the last ticket (synchronous; 0 when no floor launch ran).        */
int ring_profile_floor_timeouts(ring_t* r, uint32_t* timeouts);

/* ---- Per-wave timestamps (profiling build only) ----
 * The library built with RING_WAVE_STAMPS (libringkv_stamps.so, same sources)
 * has every wave of the attention, merge and projection kernels read the
 * device's constant-rate clock (s_memrealtime) at fixed points of its work
 * and store the readings, with its hardware placement, in a static device
 * array: per region, RING_STAMP_WAVES waves of RING_STAMP_WORDS uint64
 * words, wave index = work-group index x waves per work-group + wave:
 *   words 0..7  the clock at the wave's points (below), 8 HW_ID, 9 XCC_ID
 *   RING_STAMPS_ATTN   (ring_attn's attention launch, plain or fused):
 *                      0 entry, 1 work-group mapped, 2 first tile's loads
 *                      issued, 3 queries built and first extra rows staged
 *                      (past the barrier), 4 extra key rows attended, 5 ring
 *                      tiles attended, 6 the waves' blocks exchanged through
 *                      LDS, 7 output or partial stored (issued)
 *   RING_STAMPS_MERGE  (its merge launch): 0 entry, 1 mapped, 2 loads
 *                      issued, 3 partials in, 4 past the LDS exchange,
 *                      5 and 6 unused (zero), 7 end
 *   RING_STAMPS_PROJ   (ring_begin_step_mirror's projection): 0 entry,
 *                      1 mapped, 2 feature and weight loads issued,
 *                      3 features staged, 4 matrix-core products issued,
 *                      5 and 6 unused, 7 slice sums stored (issued)
 * Each launch overwrites the entries of its waves; words of waves that did
 * not run keep what was there (zero after a clear).  This call waits for the
 * device, copies the first min(max_waves, RING_STAMP_WAVES) waves of
 * `region` to `host` (max_waves x RING_STAMP_WORDS uint64), then zeroes the
 * region if `clear`; *clock_khz (if not NULL) gets the clock's rate.
 * Errors: RING_EINVAL (region, max_waves, host NULL with max_waves > 0),
 * RING_ESTATE (the product library, built without stamps), RING_EDEVICE. */
#define RING_STAMPS_ATTN  0
#define RING_STAMPS_MERGE 1
#define RING_STAMPS_PROJ  2
#define RING_STAMP_WAVES  8192
#define RING_STAMP_WORDS  10
int ring_profile_stamps(ring_t* r, int32_t region, uint64_t* host, int32_t max_waves,
                        int32_t clear, int32_t* clock_khz);

#ifdef __cplusplus
}
#endif

#endif /* RING_KV_H */
