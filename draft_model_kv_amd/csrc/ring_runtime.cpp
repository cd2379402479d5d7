// ring_runtime.cpp -- host side of the draft-KV ring C ABI (include/ring_kv.h).
//
// Owns the per-sequence step state (next_pos, held_lo, committed), plans each
// begin_step (page "DFLASH2_RING_PORT.md", section 1.3), carves the device
// workspace and enqueues the kernels of ring_kernels.hip on the caller's
// stream.  Arguments are validated before any device work.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "ring_kernels.h"
#include "ring_kv.h"

using namespace ringkv;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return RING_OK;
}

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

struct Layout {
  int32_t n_tiles = 0, m = 0, mpad = 0, group = 0, n_split = 1;
  bool n_split_forced = false;
  // attention work-groups per (sequence, head, split): one per 32 query rows
  // (RING_ATTN_ROW_BLOCKS=0: one work-group holds both blocks of m > 32)
  int32_t n_rb = 1;
  int64_t seq_stride = 0;  // halves per sequence in the K (or V) ring
  size_t off_k = 0, off_v = 0, off_slot = 0, off_mask = 0, off_mask_swa = 0, off_rope = 0,
         off_ropeq = 0, off_freq = 0;
  size_t off_pacc = 0, off_pml = 0, total = 0;
  size_t off_ticket = 0;                  // in-launch merge tickets, one per (seq x head, row block)
  int32_t n_ds = 0;                       // d-slices of the projection
  int64_t slot_stride = 0;                // int32 per sequence in slot_pos (cap padded)
  size_t off_mirror = 0, off_proj = 0;    // feature mirror, projection scratch
  size_t off_wpack = 0, off_knorm = 0;    // registered weights (packed), their k_norm
};

constexpr int kMaxSplits = 64;  // each merge wave holds up to 16 splits in registers

// Splits of the ring tiles per (sequence, KV head): enough work-groups to
// cover the 256 compute units, and about 8 tiles per wave read from HBM
// (the n_rb work-groups of a split read the same tiles, the later ones from
// L2), but at least one 32-slot tile per wave.  Measured (one work-group
// per compute unit): 16 ring sequences of 4096 slots attend 15% faster at 4
// splits than at 2 (16 tiles per wave); one 32768-slot ring with two query
// blocks 17% faster at 16 splits than at 32 and 30% faster than at 8.
// RING_ATTN_SPLITS (1..64) overrides the choice, for tuning and tests; the
// override also holds for launches whose windows are narrower.
bool splits_forced() {
  const char* env = std::getenv("RING_ATTN_SPLITS");
  return env && std::atoi(env) >= 1;
}

int32_t choose_splits(const ring_config& c, int32_t n_rb) {
  const int n_groups = c.n_seq * c.n_head_kv * n_rb;
  const int ring_tiles = (c.cap + kTile - 1) / kTile;
  int s = std::max(1, (256 + n_groups - 1) / n_groups);
  s = std::max(s, (ring_tiles + 32 * n_rb - 1) / (32 * n_rb));
  s = std::min(s, std::max(1, (ring_tiles + 3) / 4));
  if (const char* env = std::getenv("RING_ATTN_SPLITS")) {
    const int v = std::atoi(env);
    if (v >= 1) s = v;
  }
  return std::min(s, kMaxSplits);
}

int validate(const ring_config* c) {
  if (!c) return fail(RING_EINVAL, "config is NULL");
  if (c->cap < 1 || c->cap > (1 << 26)) return fail(RING_EINVAL, "cap %d out of [1, 2^26]", c->cap);
  if (c->q_len < 1 || c->q_len > 32) return fail(RING_EINVAL, "q_len %d out of [1, 32]", c->q_len);
  if (c->head_dim != kHeadDim)
    return fail(RING_EINVAL, "head_dim %d unsupported (must be %d)", c->head_dim, kHeadDim);
  if (c->n_head_kv < 1 || c->n_head < 1 || c->n_head % c->n_head_kv != 0)
    return fail(RING_EINVAL, "n_head %d must be a positive multiple of n_head_kv %d", c->n_head,
                c->n_head_kv);
  if (c->n_head_kv > 64) return fail(RING_EINVAL, "n_head_kv %d > 64", c->n_head_kv);
  if (c->q_len * (c->n_head / c->n_head_kv) > kMaxM)
    return fail(RING_EINVAL, "q_len * n_head / n_head_kv = %d exceeds %d",
                c->q_len * (c->n_head / c->n_head_kv), kMaxM);
  if (c->n_layer < 1 || c->n_layer > 1024) return fail(RING_EINVAL, "n_layer %d out of [1, 1024]", c->n_layer);
  if (c->n_seq < 1 || c->n_seq > RING_MAX_SEQ)
    return fail(RING_EINVAL, "n_seq %d out of [1, %d]", c->n_seq, RING_MAX_SEQ);
  if (!(c->rope_base > 1.0f) || !std::isfinite(c->rope_base))
    return fail(RING_EINVAL, "rope_base must be finite and > 1");
  if (c->swa_window < 0) return fail(RING_EINVAL, "swa_window %d < 0", c->swa_window);
  if ((c->swa_window == 0) != (c->swa_layers == 0))
    return fail(RING_EINVAL, "swa_window and swa_layers must both be zero or both non-zero");
  if (c->n_layer < 64 && (c->swa_layers >> c->n_layer) != 0)
    return fail(RING_EINVAL, "swa_layers names a layer >= n_layer %d", c->n_layer);
  if (c->d_model < 0 || c->d_model > 65536 || c->d_model % kProjSlice != 0)
    return fail(RING_EINVAL, "d_model %d must be a multiple of %d in [0, 65536]", c->d_model,
                kProjSlice);
  if (c->d_model > 0 && c->n_head_kv > kProjMaxKvHeads)
    return fail(RING_EINVAL, "a feature mirror supports at most %d KV heads", kProjMaxKvHeads);
  return RING_OK;
}

void geometry_of(const ring_config& c, ring_geometry* g, Layout* L) {
  g->a_step = 2 * c.q_len + 2;
  g->trash_slot = c.cap + c.q_len;
  g->kv_total = (int32_t)align_up((int64_t)c.cap + c.q_len + 1, 32);
  g->kv_row = c.head_dim * c.n_head_kv;
  g->kv_bytes_per_layer = 2ll * g->kv_row * g->kv_total * 2;

  L->n_tiles = g->kv_total / kTile;
  L->group = c.n_head / c.n_head_kv;
  L->m = c.q_len * L->group;
  L->mpad = L->m <= 32 ? 32 : 64;
  {
    const char* env = std::getenv("RING_ATTN_ROW_BLOCKS");
    const bool row_blocks = !(env && std::atoi(env) == 0);
    L->n_rb = row_blocks ? L->mpad / 32 : 1;
  }
  L->n_split = choose_splits(c, L->n_rb);
  L->n_split_forced = splits_forced();
  L->seq_stride = (int64_t)c.n_layer * c.n_head_kv * L->n_tiles * kTileHalves;
  size_t off = 0;
  auto take = [&off](size_t bytes) {
    const size_t o = off;
    off = (size_t)align_up((int64_t)(off + bytes), 256);
    return o;
  };
  const size_t ring_bytes = (size_t)c.n_seq * L->seq_stride * 2;
  L->off_k = take(ring_bytes);
  L->off_v = take(ring_bytes);
  // slot_pos rows padded to 64 entries, so that 16-byte loads of four slots
  // stay aligned and inside the sequence's row
  L->slot_stride = align_up(c.cap, 64);
  L->off_slot = take((size_t)c.n_seq * L->slot_stride * 4);
  L->off_mask = take((size_t)c.n_seq * c.q_len * g->kv_total * 2);
  L->off_mask_swa = take(c.swa_window > 0 ? (size_t)c.n_seq * c.q_len * g->kv_total * 2 : 0);
  L->off_rope = take((size_t)c.n_seq * c.q_len * 64 * 2 * 8);
  L->off_ropeq = take((size_t)c.n_seq * c.q_len * 64 * 2 * 4);
  L->off_freq = take(64 * 8);
  const size_t n_part = L->n_split > 1 ? (size_t)c.n_seq * c.n_head_kv * L->n_split * L->mpad : 0;
  L->off_pacc = take(n_part * kHeadDim * 2);
  L->off_pml = take(n_part * 2 * 4);
  L->off_ticket = take(L->n_split > 1 ? (size_t)c.n_seq * c.n_head_kv * L->n_rb * 4 : 0);
  L->n_ds = c.d_model / kProjSlice;
  L->off_mirror = take((size_t)c.n_seq * c.cap * c.d_model * 2);
  L->off_proj = take((size_t)c.n_layer * L->n_ds * kProjRows * 2 * g->kv_row * 4);
  // registered projection weights (ring_set_kv_weights): wk and wv packed in
  // the projection kernel's load order, and k_norm
  L->off_wpack = take((size_t)c.n_layer * 2 * g->kv_row * c.d_model * 2);
  L->off_knorm = take(c.d_model > 0 ? (size_t)c.n_layer * kHeadDim * 4 : 0);
  L->total = off;
  g->workspace_bytes = (int64_t)L->total;
}

struct Plan {
  int64_t win, lo, start, n_new;
  bool bulk;
};

// Section 1.3: win = min(committed, cap), lo = committed - win,
// start = max(next_pos, lo); after a rewind that lost window rows the whole
// window is appended again (start = lo).
Plan plan_of(int64_t cap, int64_t a_step, int64_t committed, int64_t next_pos, int64_t held_lo) {
  Plan p;
  p.win = std::min(committed, cap);
  p.lo = committed - p.win;
  if (p.lo < held_lo) p.start = p.lo;
  else p.start = std::max(std::min(next_pos, committed), p.lo);
  p.n_new = committed - p.start;
  p.bulk = p.n_new > a_step;
  return p;
}

}  // namespace

// A sequence's deferred fold-in step (ring_begin_step_deferred): its rows are
// appended, layer by layer, by the next attention launch of each layer, and
// the first such launch also rebuilds the index state.
// A sequence's deferred mirror write (ring_mirror_write_deferred): the rows
// of positions [pos0, pos0 + n) are still in the caller's buffer.
struct MirrorPending {
  bool active = false;
  int64_t pos0 = 0, n = 0;
  const uint16_t* features = nullptr;
};

struct Pending {
  bool active = false;
  const uint16_t* k = nullptr;  // [n_layer][n_new][kv_row] F16, not rotated
  const uint16_t* v = nullptr;
  int64_t start = 0, n_new = 0, committed = 0, lo = 0, swa_lo = 0;
  uint64_t layers_left = 0;     // bit l: layer l's rows are not appended yet
  bool index_left = false;      // slot_pos, masks and RoPE table not rebuilt yet
};

struct ring {
  ring_config cfg{};
  ring_geometry geo{};
  Layout L;
  int device = 0;
  bool owns_ws = false;
  uint8_t* ws = nullptr;
  uint16_t* kring = nullptr;
  uint16_t* vring = nullptr;
  int32_t* slot_pos = nullptr;
  uint16_t* mask = nullptr;
  uint16_t* mask_swa = nullptr;  // sliding-window layers' mask, or nullptr
  double* rope_noise = nullptr;
  float* rope_q = nullptr;
  double* inv_freq = nullptr;
  uint16_t* part_acc = nullptr;
  float* part_ml = nullptr;
  // ticket counters of the in-launch cross-split merge (zero between
  // launches), or nullptr; used only with RING_ATTN_MERGE=kernel
  uint32_t* tickets = nullptr;
  bool merge_in_launch = false;
  uint16_t* mirror = nullptr;   // fused features [n_seq][cap][d_model], or nullptr
  float* proj = nullptr;        // projection scratch
  uint16_t* wpack = nullptr;    // registered weights, packed (ring_set_kv_weights)
  float* knorm = nullptr;       // their k_norm [n_layer][head_dim]
  float weights_eps = 0.0f;
  bool weights_set = false;
  std::vector<int64_t> next_pos, held_lo, committed;
  std::vector<std::vector<int64_t>> mirror_pos;  // per sequence: position in each mirror slot, -1 empty
                                                 // (a deferred write's rows included)
  std::vector<MirrorPending> mirror_pending;      // per sequence
  std::vector<Pending> pending;                   // per sequence
  // per sequence: slot_pos is current but the masks and the noise RoPE table
  // still hold an earlier step's (a fused launch wrote the new rows' slot_pos
  // entries and left the rest for an index-only append launch, which runs
  // before anything reads them: a plain attention launch or a mask read)
  std::vector<uint8_t> index_owed;
  std::vector<double> inv_freq_host;
  hipStream_t last_stream = nullptr;
  // profiling: per kernel kind, event pairs (start, end) and how many are used
  int32_t prof_max = 0;
  std::vector<hipEvent_t> prof_ev[5];
  int32_t prof_used[5] = {0, 0, 0, 0, 0};
  // profiling-only floor launches (ring_profile_floor): counters, timeout
  // count and output of the in-kernel merge variants, allocated on first use
  uint8_t* floor_buf = nullptr;
  int32_t floor_last_kind = -1;
  uint32_t floor_epoch = 0;
};

namespace {

int use_device(const ring* r) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return fail(RING_EDEVICE, "hipGetDevice failed");
  if (cur != r->device && hipSetDevice(r->device) != hipSuccess)
    return fail(RING_EDEVICE, "hipSetDevice(%d) failed", r->device);
  return RING_OK;
}

StepArgs step_args(ring* r, int32_t seq) {
  StepArgs a{};
  a.kring = r->kring + seq * r->L.seq_stride;
  a.vring = r->vring + seq * r->L.seq_stride;
  a.slot_pos = r->slot_pos + (int64_t)seq * r->L.slot_stride;
  a.mask = r->mask + (int64_t)seq * r->cfg.q_len * r->geo.kv_total;
  a.mask_swa = r->mask_swa ? r->mask_swa + (int64_t)seq * r->cfg.q_len * r->geo.kv_total : nullptr;
  a.rope_noise = r->rope_noise + (int64_t)seq * r->cfg.q_len * 128;
  a.rope_q = r->rope_q + (int64_t)seq * r->cfg.q_len * 128;
  a.inv_freq = r->inv_freq;
  a.cap = r->cfg.cap;
  a.q_len = r->cfg.q_len;
  a.kv_total = r->geo.kv_total;
  a.n_head_kv = r->cfg.n_head_kv;
  a.n_layer = r->cfg.n_layer;
  a.trash_slot = r->geo.trash_slot;
  a.n_tiles = r->L.n_tiles;
  return a;
}

// Next free (start, end) event pair for a launch of `kind`, or nullptrs.
void next_events(ring* r, int kind, hipEvent_t* t0, hipEvent_t* t1) {
  *t0 = *t1 = nullptr;
  if (r->prof_used[kind] < r->prof_max) {
    *t0 = r->prof_ev[kind][2 * r->prof_used[kind]];
    *t1 = r->prof_ev[kind][2 * r->prof_used[kind] + 1];
    ++r->prof_used[kind];
  }
}

void destroy_events(ring* r) {
  for (auto& v : r->prof_ev) {
    for (hipEvent_t e : v) (void)hipEventDestroy(e);
    v.clear();
  }
  r->prof_max = 0;
  for (int32_t& u : r->prof_used) u = 0;
}

int check_launch(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(RING_EDEVICE, "%s: %s", what, hipGetErrorString(e));
  return RING_OK;
}

// Carry out what a deferred step of `seq` still owes (rows of the layers
// whose attention has not run, the index state) with the ordinary append
// kernel, on the ring's last stream.
int flush_seq(ring* r, int32_t seq) {
  Pending& p = r->pending[seq];
  if (!p.active) return RING_OK;
  if (p.layers_left || p.index_left) {
    StepArgs a = step_args(r, seq);
    a.k_new = p.k;
    a.v_new = p.v;
    a.start = p.start;
    a.start_mod = (int32_t)(p.start % r->cfg.cap);
    a.committed = p.committed;
    a.lo = p.lo;
    a.swa_lo = p.swa_lo;
    a.n_new = (int32_t)p.n_new;
    a.row0 = 0;
    a.n_rows = (int32_t)p.n_new;
    a.n_pad = r->geo.a_step - (int32_t)p.n_new;
    a.do_mask = (p.index_left || r->index_owed[seq]) ? 1 : 0;
    a.layer_skip = ~p.layers_left;
    hipEvent_t t0, t1;
    next_events(r, RING_KERNEL_STEP, &t0, &t1);
    if (int e = check_launch(launch_step(a, r->last_stream, t0, t1), "deferred append"))
      return e;
    if (a.do_mask) r->index_owed[seq] = 0;
  }
  p = Pending{};
  return RING_OK;
}

// Rebuild the masks and the noise RoPE table of `seq` from its slot_pos and
// state if a fused launch left them owed: an append launch with no rows.
int flush_index(ring* r, int32_t seq) {
  if (!r->index_owed[seq]) return RING_OK;
  StepArgs a = step_args(r, seq);
  const int64_t c = r->committed[seq];
  const int64_t win = std::min<int64_t>(c, r->cfg.cap);
  a.start = c;
  a.start_mod = (int32_t)(c % r->cfg.cap);
  a.committed = c;
  a.lo = r->held_lo[seq];
  a.swa_lo = c - std::min<int64_t>(r->cfg.swa_window, win);
  a.n_new = 0;
  a.row0 = 0;
  a.n_rows = 0;
  a.n_pad = 0;
  a.do_mask = 1;
  hipEvent_t t0, t1;
  next_events(r, RING_KERNEL_STEP, &t0, &t1);
  if (int e = check_launch(launch_step(a, r->last_stream, t0, t1), "index rebuild")) return e;
  r->index_owed[seq] = 0;
  return RING_OK;
}

// Everything deferred steps still owe, for every sequence.
int flush_all(ring* r) {
  for (int32_t seq = 0; seq < r->cfg.n_seq; ++seq) {
    if (int e = flush_seq(r, seq)) return e;
    if (int e = flush_index(r, seq)) return e;
  }
  return RING_OK;
}

}  // namespace

extern "C" {

int ring_query_geometry(const ring_config* cfg, ring_geometry* out) {
  if (int e = validate(cfg)) return e;
  if (!out) return fail(RING_EINVAL, "out is NULL");
  Layout L;
  geometry_of(*cfg, out, &L);
  return ok();
}

int ring_init(const ring_config* cfg, void* workspace, size_t workspace_bytes, void* stream,
              ring_t** out) {
  if (!out) return fail(RING_EINVAL, "out is NULL");
  *out = nullptr;
  if (int e = validate(cfg)) return e;
  ring* r = new (std::nothrow) ring();
  if (!r) return fail(RING_ENOMEM, "host allocation failed");
  r->cfg = *cfg;
  geometry_of(*cfg, &r->geo, &r->L);
  if (workspace) {
    if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0) {
      delete r;
      return fail(RING_EINVAL, "workspace must be 256-byte aligned");
    }
    if (workspace_bytes < r->L.total) {
      delete r;
      return fail(RING_ENOMEM, "workspace of %zu bytes < %zu needed", workspace_bytes, r->L.total);
    }
  }
  if (hipGetDevice(&r->device) != hipSuccess) {
    delete r;
    return fail(RING_EDEVICE, "no HIP device");
  }
  // device address of ring_attn_noalloc's static partials on this device
  if (hipError_t e = resolve_static_scratch(r->device); e != hipSuccess) {
    delete r;
    return fail(RING_EDEVICE, "static scratch of device %d: %s", r->device, hipGetErrorString(e));
  }
  if (workspace) {
    r->ws = static_cast<uint8_t*>(workspace);
  } else {
    void* p = nullptr;
    if (hipMalloc(&p, r->L.total) != hipSuccess) {
      (void)hipGetLastError();
      delete r;
      return fail(RING_ENOMEM, "hipMalloc of %zu bytes failed", r->L.total);
    }
    r->ws = static_cast<uint8_t*>(p);
    r->owns_ws = true;
  }
  r->kring = reinterpret_cast<uint16_t*>(r->ws + r->L.off_k);
  r->vring = reinterpret_cast<uint16_t*>(r->ws + r->L.off_v);
  r->slot_pos = reinterpret_cast<int32_t*>(r->ws + r->L.off_slot);
  r->mask = reinterpret_cast<uint16_t*>(r->ws + r->L.off_mask);
  r->rope_noise = reinterpret_cast<double*>(r->ws + r->L.off_rope);
  if (cfg->swa_window > 0) r->mask_swa = reinterpret_cast<uint16_t*>(r->ws + r->L.off_mask_swa);
  r->rope_q = reinterpret_cast<float*>(r->ws + r->L.off_ropeq);
  r->inv_freq = reinterpret_cast<double*>(r->ws + r->L.off_freq);
  r->part_acc = reinterpret_cast<uint16_t*>(r->ws + r->L.off_pacc);
  r->part_ml = reinterpret_cast<float*>(r->ws + r->L.off_pml);
  if (r->L.n_split > 1) r->tickets = reinterpret_cast<uint32_t*>(r->ws + r->L.off_ticket);
  {
    // RING_ATTN_MERGE=kernel: merge the splits inside the attention launch
    // where it applies (measured no faster than the merge launch on the
    // wide rings: the coherent partial stores, the ticket and the last
    // arriver's loads cost the attention as much as the launch it saves)
    const char* env = std::getenv("RING_ATTN_MERGE");
    r->merge_in_launch = env && std::strcmp(env, "kernel") == 0;
  }
  if (cfg->d_model > 0) {
    r->mirror = reinterpret_cast<uint16_t*>(r->ws + r->L.off_mirror);
    r->proj = reinterpret_cast<float*>(r->ws + r->L.off_proj);
    r->wpack = reinterpret_cast<uint16_t*>(r->ws + r->L.off_wpack);
    r->knorm = reinterpret_cast<float*>(r->ws + r->L.off_knorm);
    r->mirror_pos.assign(cfg->n_seq, std::vector<int64_t>(cfg->cap, -1));
    r->mirror_pending.assign(cfg->n_seq, MirrorPending{});
  }
  r->pending.assign(cfg->n_seq, Pending{});
  r->index_owed.assign(cfg->n_seq, 0);
  r->next_pos.assign(cfg->n_seq, 0);
  r->held_lo.assign(cfg->n_seq, 0);
  r->committed.assign(cfg->n_seq, 0);
  r->inv_freq_host.resize(64);
  for (int i = 0; i < 64; ++i)
    r->inv_freq_host[i] = std::pow((double)cfg->rope_base, -2.0 * i / (double)kHeadDim);

  hipStream_t s = static_cast<hipStream_t>(stream);
  r->last_stream = s;
  const size_t ring_bytes = (size_t)cfg->n_seq * r->L.seq_stride * 2;
  hipError_t e = hipMemsetAsync(r->kring, 0, ring_bytes, s);
  if (e == hipSuccess) e = hipMemsetAsync(r->vring, 0, ring_bytes, s);
  if (e == hipSuccess) e = hipMemsetAsync(r->slot_pos, 0xFF, (size_t)cfg->n_seq * r->L.slot_stride * 4, s);
  if (e == hipSuccess && r->tickets)
    e = hipMemsetAsync(r->tickets, 0, (size_t)cfg->n_seq * cfg->n_head_kv * r->L.n_rb * 4, s);
  if (e == hipSuccess)
    e = launch_fill_u16(r->mask, 0xFC00u, (int64_t)cfg->n_seq * cfg->q_len * r->geo.kv_total, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(r->inv_freq, r->inv_freq_host.data(), 64 * sizeof(double),
                       hipMemcpyHostToDevice, s);
  // Index state of committed = 0: nothing visible but the noise block.
  for (int32_t seq = 0; seq < cfg->n_seq && e == hipSuccess; ++seq) {
    StepArgs a = step_args(r, seq);
    a.do_mask = 1;
    e = launch_step(a, s, nullptr, nullptr);
  }
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    const int code = fail(RING_EDEVICE, "ring_init device work failed: %s", hipGetErrorString(e));
    if (r->owns_ws) (void)hipFree(r->ws);
    delete r;
    return code;
  }
  *out = r;
  return ok();
}

namespace {
void fill_plan(const ring_config& c, int32_t a_step, int32_t trash_slot, int64_t committed,
               int64_t next_pos, int64_t held_lo, ring_plan* out, int32_t* ap_rows) {
  const Plan p = plan_of(c.cap, a_step, committed, next_pos, held_lo);
  out->committed = committed;
  out->win = p.win;
  out->lo = p.lo;
  out->start = p.start;
  out->n_new = p.n_new;
  out->bulk = p.bulk ? 1 : 0;
  out->n_chunks = p.bulk ? (int32_t)((p.n_new + kBulkChunk - 1) / kBulkChunk) : 0;
  if (ap_rows && !p.bulk) {
    for (int i = 0; i < a_step; ++i)
      ap_rows[i] = i < p.n_new ? (int32_t)((p.start + i) % c.cap) : trash_slot;
  }
}
}  // namespace

int ring_plan_from_state(const ring_config* cfg, int64_t next_pos, int64_t held_lo,
                         int64_t committed, ring_plan* out, int32_t* ap_rows) {
  if (int e = validate(cfg)) return e;
  if (!out) return fail(RING_EINVAL, "out is NULL");
  if (next_pos < 0 || held_lo < 0 || held_lo > next_pos || next_pos - held_lo > cfg->cap)
    return fail(RING_EINVAL, "state next_pos %lld / held_lo %lld is not one a ring can be in",
                (long long)next_pos, (long long)held_lo);
  if (committed < 0 || committed + cfg->q_len > INT32_MAX)
    return fail(RING_ERANGE, "committed %lld out of range", (long long)committed);
  fill_plan(*cfg, 2 * cfg->q_len + 2, cfg->cap + cfg->q_len, committed, next_pos, held_lo, out,
            ap_rows);
  return ok();
}

int ring_plan_step(const ring_t* r, int32_t seq, int64_t committed, ring_plan* out,
                   int32_t* ap_rows) {
  if (!r || !out) return fail(RING_EINVAL, "NULL argument");
  if (seq < 0 || seq >= r->cfg.n_seq) return fail(RING_ERANGE, "seq %d out of range", seq);
  if (committed < 0 || committed + r->cfg.q_len > INT32_MAX)
    return fail(RING_ERANGE, "committed %lld out of range", (long long)committed);
  fill_plan(r->cfg, r->geo.a_step, r->geo.trash_slot, committed, r->next_pos[seq],
            r->held_lo[seq], out, ap_rows);
  return ok();
}

namespace {
// Checks of one begin_step call; *out gets its plan.
int check_step(const ring* r, int32_t seq, int64_t committed, const void* k_new,
               const void* v_new, int64_t n_rows, Plan* out) {
  if (seq < 0 || seq >= r->cfg.n_seq) return fail(RING_ERANGE, "seq %d out of range", seq);
  if (committed < 0 || committed + r->cfg.q_len > INT32_MAX)
    return fail(RING_ERANGE, "committed %lld out of range", (long long)committed);
  const Plan p = plan_of(r->cfg.cap, r->geo.a_step, committed, r->next_pos[seq], r->held_lo[seq]);
  if (n_rows != p.n_new)
    return fail(RING_ESTATE, "n_rows %lld != planned n_new %lld (start %lld)", (long long)n_rows,
                (long long)p.n_new, (long long)p.start);
  if (p.n_new > 0 && (!k_new || !v_new)) return fail(RING_EINVAL, "k_new / v_new is NULL");
  *out = p;
  return RING_OK;
}

// State after an append whose last launch rebuilt the index state.
void set_state(ring* r, int32_t seq, int64_t committed, const Plan& p) {
  r->next_pos[seq] = committed;
  r->held_lo[seq] = p.lo;
  r->committed[seq] = committed;
  r->index_owed[seq] = 0;
}

// The append launches of one checked step (bulk chunks or the fold-in).
int append_now(ring* r, int32_t seq, int64_t committed, const Plan& p, const void* k_new,
               const void* v_new, hipStream_t s) {
  StepArgs a = step_args(r, seq);
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.start = p.start;
  a.start_mod = (int32_t)(p.start % r->cfg.cap);
  a.committed = committed;
  a.lo = p.lo;
  a.swa_lo = committed - std::min<int64_t>(r->cfg.swa_window, p.win);
  a.n_new = (int32_t)p.n_new;
  if (p.bulk) {
    for (int64_t row0 = 0; row0 < p.n_new; row0 += kBulkChunk) {
      a.row0 = (int32_t)row0;
      a.n_rows = (int32_t)std::min<int64_t>(kBulkChunk, p.n_new - row0);
      a.n_pad = 0;
      a.do_mask = row0 + kBulkChunk >= p.n_new;
      hipEvent_t t0, t1;
      next_events(r, RING_KERNEL_STEP, &t0, &t1);
      if (int e = check_launch(launch_step(a, s, t0, t1), "bulk append")) return e;
    }
  } else {
    a.row0 = 0;
    a.n_rows = (int32_t)p.n_new;
    a.n_pad = r->geo.a_step - (int32_t)p.n_new;
    a.do_mask = 1;
    hipEvent_t t0, t1;
    next_events(r, RING_KERNEL_STEP, &t0, &t1);
    if (int e = check_launch(launch_step(a, s, t0, t1), "fold-in append")) return e;
  }
  set_state(r, seq, committed, p);
  return RING_OK;
}
}  // namespace

int ring_begin_step(ring_t* r, int32_t seq, int64_t committed, const void* k_new,
                    const void* v_new, int64_t n_rows, void* stream) {
  if (!r) return fail(RING_EINVAL, "ring is NULL");
  Plan p;
  if (int e = check_step(r, seq, committed, k_new, v_new, n_rows, &p)) return e;
  if (int e = use_device(r)) return e;
  if (int e = flush_seq(r, seq)) return e;
  hipStream_t s = static_cast<hipStream_t>(stream);
  r->last_stream = s;
  if (int e = append_now(r, seq, committed, p, k_new, v_new, s)) return e;
  return ok();
}

int ring_begin_step_batch(ring_t* r, int32_t n, const int32_t* seqs, const int64_t* committed,
                          const void* const* k_new, const void* const* v_new,
                          const int64_t* n_rows, void* stream) {
  if (!r) return fail(RING_EINVAL, "ring is NULL");
  if (n < 0 || n > r->cfg.n_seq)
    return fail(RING_ERANGE, "n %d out of [0, n_seq %d]", n, r->cfg.n_seq);
  if (n == 0) return ok();
  if (!seqs || !committed || !k_new || !v_new || !n_rows)
    return fail(RING_EINVAL, "NULL array argument");
  std::vector<Plan> plans((size_t)n);
  std::vector<uint8_t> listed((size_t)r->cfg.n_seq, 0);
  for (int32_t i = 0; i < n; ++i) {
    if (int e = check_step(r, seqs[i], committed[i], k_new[i], v_new[i], n_rows[i], &plans[i]))
      return e;
    if (listed[seqs[i]]++) return fail(RING_EINVAL, "seq %d listed twice", seqs[i]);
  }
  if (int e = use_device(r)) return e;
  for (int32_t i = 0; i < n; ++i)
    if (int e = flush_seq(r, seqs[i])) return e;
  hipStream_t s = static_cast<hipStream_t>(stream);
  r->last_stream = s;

  StepBatchArgs b{};
  b.a = step_args(r, 0);
  b.a.do_mask = 1;
  b.seq_stride = r->L.seq_stride;
  b.slot_stride = r->L.slot_stride;
  b.a_step = r->geo.a_step;
  b.blocks_per_seq = r->geo.a_step * r->cfg.n_layer + (r->geo.kv_total + 255) / 256;
  int32_t members[kStepBatch];
  auto launch = [&]() -> int {
    if (b.n_seq == 0) return RING_OK;
    hipEvent_t t0, t1;
    next_events(r, RING_KERNEL_STEP, &t0, &t1);
    if (int e = check_launch(launch_step_batch(b, s, t0, t1), "batched fold-in append")) return e;
    for (int32_t j = 0; j < b.n_seq; ++j) {
      const int32_t i = members[j];
      set_state(r, seqs[i], committed[i], plans[i]);
    }
    b.n_seq = 0;
    return RING_OK;
  };
  for (int32_t i = 0; i < n; ++i) {
    const Plan& p = plans[i];
    if (p.bulk) {
      if (int e = append_now(r, seqs[i], committed[i], p, k_new[i], v_new[i], s)) return e;
      continue;
    }
    const int32_t j = b.n_seq++;
    members[j] = i;
    b.seq[j] = seqs[i];
    b.start[j] = (int32_t)p.start;
    b.start_mod[j] = (int32_t)(p.start % r->cfg.cap);
    b.n_new[j] = (int32_t)p.n_new;
    b.committed[j] = (int32_t)committed[i];
    b.lo[j] = (int32_t)p.lo;
    b.swa_lo[j] = (int32_t)(committed[i] - std::min<int64_t>(r->cfg.swa_window, p.win));
    b.k_new[j] = reinterpret_cast<uint64_t>(k_new[i]);
    b.v_new[j] = reinterpret_cast<uint64_t>(v_new[i]);
    if (b.n_seq == kStepBatch)
      if (int e = launch()) return e;
  }
  if (int e = launch()) return e;
  return ok();
}

int ring_begin_step_deferred(ring_t* r, int32_t seq, int64_t committed, const void* k_new,
                             const void* v_new, int64_t n_rows, void* stream) {
  if (!r) return fail(RING_EINVAL, "ring is NULL");
  if (seq < 0 || seq >= r->cfg.n_seq) return fail(RING_ERANGE, "seq %d out of range", seq);
  if (committed < 0 || committed + r->cfg.q_len > INT32_MAX)
    return fail(RING_ERANGE, "committed %lld out of range", (long long)committed);
  const Plan p = plan_of(r->cfg.cap, r->geo.a_step, committed, r->next_pos[seq], r->held_lo[seq]);
  // Bulk appends and rings beyond what one fused launch carries append now.
  // (Rings whose attention waves stream several tiles are fused too: since
  // the fused launch tests each slot's visibility with one window test on
  // slot_pos, its tile pass costs what the plain one's does — a 32768-slot
  // window 29.4-29.9 against 29.3 us — and the append launch it saves is
  // the gain.)
  if (p.bulk || r->cfg.n_seq > kFusedMaxSeq || r->cfg.n_layer > 64)
    return ring_begin_step(r, seq, committed, k_new, v_new, n_rows, stream);
  if (n_rows != p.n_new)
    return fail(RING_ESTATE, "n_rows %lld != planned n_new %lld (start %lld)", (long long)n_rows,
                (long long)p.n_new, (long long)p.start);
  if (p.n_new > 0 && (!k_new || !v_new)) return fail(RING_EINVAL, "k_new / v_new is NULL");
  if (int e = use_device(r)) return e;
  if (int e = flush_seq(r, seq)) return e;
  r->last_stream = static_cast<hipStream_t>(stream);
  Pending& d = r->pending[seq];
  d.active = true;
  d.k = static_cast<const uint16_t*>(k_new);
  d.v = static_cast<const uint16_t*>(v_new);
  d.start = p.start;
  d.n_new = p.n_new;
  d.committed = committed;
  d.lo = p.lo;
  d.swa_lo = committed - std::min<int64_t>(r->cfg.swa_window, p.win);
  d.layers_left = r->cfg.n_layer == 64 ? ~0ull : ((1ull << r->cfg.n_layer) - 1);
  d.index_left = true;
  r->next_pos[seq] = committed;
  r->held_lo[seq] = p.lo;
  r->committed[seq] = committed;
  return ok();
}

namespace {
int check_mirror_write(const ring* r, int32_t seq, int64_t pos0, int64_t n, const void* features) {
  if (!r) return fail(RING_EINVAL, "ring is NULL");
  if (!r->mirror) return fail(RING_ESTATE, "the ring has no feature mirror (d_model = 0)");
  if (seq < 0 || seq >= r->cfg.n_seq) return fail(RING_ERANGE, "seq %d out of range", seq);
  if (pos0 < 0 || n < 0 || pos0 + n + r->cfg.q_len > INT32_MAX)
    return fail(RING_ERANGE, "positions [%lld, %lld) out of range", (long long)pos0,
                (long long)(pos0 + n));
  if (n > 0 && !features) return fail(RING_EINVAL, "features is NULL");
  return RING_OK;
}

// Only the last cap rows of a write can stay: earlier ones share their slots
// with later ones.  Returns the first position that stays.
int64_t mirror_first_kept(const ring* r, int64_t pos0, int64_t n) {
  return pos0 + std::max<int64_t>(0, n - r->cfg.cap);
}

// Copy the rows of positions [pos0, pos0 + n) (features row i = position
// pos0 + i) into sequence seq's mirror, slot p % cap.
int mirror_copy(ring* r, int32_t seq, int64_t pos0, int64_t n, const void* features,
                hipStream_t s) {
  const int64_t cap = r->cfg.cap, d = r->cfg.d_model;
  const int64_t first = mirror_first_kept(r, pos0, n), m = pos0 + n - first;
  const int64_t s0 = first % cap;
  const int64_t piece1 = std::min<int64_t>(m, cap - s0);
  const uint8_t* src = static_cast<const uint8_t*>(features) + (first - pos0) * d * 2;
  uint16_t* base = r->mirror + (int64_t)seq * cap * d;
  hipError_t e = hipMemcpyAsync(base + s0 * d, src, (size_t)(piece1 * d * 2),
                                hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess && m > piece1)
    e = hipMemcpyAsync(base, src + piece1 * d * 2, (size_t)((m - piece1) * d * 2),
                       hipMemcpyDeviceToDevice, s);
  if (e != hipSuccess) return fail(RING_EDEVICE, "mirror copy: %s", hipGetErrorString(e));
  return RING_OK;
}

// Positions [first kept, pos0 + n) are held by the mirror (or will be, once
// a deferred write lands).
void mirror_record(ring* r, int32_t seq, int64_t pos0, int64_t n) {
  std::vector<int64_t>& mp = r->mirror_pos[seq];
  for (int64_t p = mirror_first_kept(r, pos0, n); p < pos0 + n; ++p) mp[p % r->cfg.cap] = p;
}

// A deferred mirror write of seq still owed, copied now on stream s.
int flush_mirror(ring* r, int32_t seq, hipStream_t s) {
  MirrorPending& m = r->mirror_pending[seq];
  if (!m.active) return RING_OK;
  const MirrorPending w = m;
  if (int e = mirror_copy(r, seq, w.pos0, w.n, w.features, s)) return e;
  m = MirrorPending{};
  return RING_OK;
}
}  // namespace

int ring_mirror_write(ring_t* r, int32_t seq, int64_t pos0, int64_t n, const void* features,
                      void* stream) {
  if (int e = check_mirror_write(r, seq, pos0, n, features)) return e;
  if (n == 0) return ok();
  if (int e = use_device(r)) return e;
  hipStream_t s = static_cast<hipStream_t>(stream);
  r->last_stream = s;
  // an earlier deferred write lands first (a later write to its slots wins)
  if (int e = flush_mirror(r, seq, s)) return e;
  if (int e = mirror_copy(r, seq, pos0, n, features, s)) return e;
  mirror_record(r, seq, pos0, n);
  return ok();
}

int ring_mirror_write_deferred(ring_t* r, int32_t seq, int64_t pos0, int64_t n,
                               const void* features, void* stream) {
  if (int e = check_mirror_write(r, seq, pos0, n, features)) return e;
  if (n == 0) return ok();
  if (int e = use_device(r)) return e;
  hipStream_t s = static_cast<hipStream_t>(stream);
  r->last_stream = s;
  if (int e = flush_mirror(r, seq, s)) return e;
  MirrorPending& m = r->mirror_pending[seq];
  m.active = true;
  m.pos0 = pos0;
  m.n = n;
  m.features = static_cast<const uint16_t*>(features);
  mirror_record(r, seq, pos0, n);
  return ok();
}

namespace {
int check_weights(const ring_kv_weights* w) {
  if (!w || !w->wk || !w->wv || !w->k_norm) return fail(RING_EINVAL, "weights are NULL");
  if (((reinterpret_cast<uintptr_t>(w->wk) | reinterpret_cast<uintptr_t>(w->wv)) & 15) ||
      (reinterpret_cast<uintptr_t>(w->k_norm) & 3))
    return fail(RING_EINVAL, "wk / wv must be 16-byte and k_norm 4-byte aligned");
  if (!(w->eps >= 0.0f) || !std::isfinite(w->eps)) return fail(RING_EINVAL, "eps must be finite and >= 0");
  return RING_OK;
}
}  // namespace

int ring_set_kv_weights(ring_t* r, const ring_kv_weights* w, void* stream) {
  if (!r) return fail(RING_EINVAL, "ring is NULL");
  if (!r->mirror) return fail(RING_ESTATE, "the ring has no feature mirror (d_model = 0)");
  if (int e = check_weights(w)) return e;
  if (int e = use_device(r)) return e;
  hipStream_t s = static_cast<hipStream_t>(stream);
  r->last_stream = s;
  PackArgs pk{};
  pk.wk = static_cast<const uint16_t*>(w->wk);
  pk.wv = static_cast<const uint16_t*>(w->wv);
  pk.packed = r->wpack;
  pk.n_chunks = (int64_t)r->cfg.n_layer * 2 * r->geo.kv_row * r->cfg.d_model / 8;
  pk.d_model = r->cfg.d_model;
  pk.kv_row = r->geo.kv_row;
  pk.n_head_kv = r->cfg.n_head_kv;
  pk.n_ds = r->L.n_ds;
  if (int e = check_launch(launch_pack_weights(pk, s), "weight packing")) return e;
  if (hipMemcpyAsync(r->knorm, w->k_norm, (size_t)r->cfg.n_layer * kHeadDim * 4,
                     hipMemcpyDeviceToDevice, s) != hipSuccess)
    return fail(RING_EDEVICE, "k_norm copy failed");
  r->weights_eps = w->eps;
  r->weights_set = true;
  return ok();
}

int ring_begin_step_mirror(ring_t* r, int32_t seq, int64_t committed, const ring_kv_weights* w,
                           void* stream) {
  if (!r) return fail(RING_EINVAL, "ring is NULL");
  if (!r->mirror) return fail(RING_ESTATE, "the ring has no feature mirror (d_model = 0)");
  if (seq < 0 || seq >= r->cfg.n_seq) return fail(RING_ERANGE, "seq %d out of range", seq);
  if (committed < 0 || committed + r->cfg.q_len > INT32_MAX)
    return fail(RING_ERANGE, "committed %lld out of range", (long long)committed);
  if (!w && !r->weights_set)
    return fail(RING_ESTATE, "no weights given and none registered (ring_set_kv_weights)");
  if (w) {
    if (int e = check_weights(w)) return e;
  }
  const Plan p = plan_of(r->cfg.cap, r->geo.a_step, committed, r->next_pos[seq], r->held_lo[seq]);
  const std::vector<int64_t>& mp = r->mirror_pos[seq];
  for (int64_t q = p.start; q < committed; ++q)
    if (mp[q % r->cfg.cap] != q)
      return fail(RING_ESTATE, "position %lld is not in the feature mirror (write it first)",
                  (long long)q);
  if (int e = use_device(r)) return e;
  if (int e = flush_seq(r, seq)) return e;
  hipStream_t s = static_cast<hipStream_t>(stream);
  r->last_stream = s;
  // A deferred mirror write of exactly this step's rows (one projection
  // launch) is carried out by that launch; any other is copied first.
  MirrorPending& mw = r->mirror_pending[seq];
  const bool fuse_write = mw.active && p.n_new > 0 && p.n_new <= kProjRows &&
                          mw.pos0 == p.start && mw.n == p.n_new;
  if (!fuse_write) {
    if (int e = flush_mirror(r, seq, s)) return e;
  }

  StepArgs a = step_args(r, seq);
  a.start = p.start;
  a.start_mod = (int32_t)(p.start % r->cfg.cap);
  a.committed = committed;
  a.lo = p.lo;
  a.swa_lo = committed - std::min<int64_t>(r->cfg.swa_window, p.win);
  a.n_new = (int32_t)p.n_new;
  a.proj = r->proj;
  a.k_norm = w ? w->k_norm : r->knorm;
  a.eps = (double)(w ? w->eps : r->weights_eps);
  a.n_ds = r->L.n_ds;
  ProjArgs pa{};
  pa.mirror = r->mirror + (int64_t)seq * r->cfg.cap * r->cfg.d_model;
  if (fuse_write) {
    pa.feat = mw.features;
    pa.mirror_w = r->mirror + (int64_t)seq * r->cfg.cap * r->cfg.d_model;
  }
  pa.wk = w ? static_cast<const uint16_t*>(w->wk) : r->wpack;
  pa.wv = w ? static_cast<const uint16_t*>(w->wv) : nullptr;
  pa.packed = w ? 0 : 1;
  pa.scratch = r->proj;
  pa.cap = r->cfg.cap;
  pa.d_model = r->cfg.d_model;
  pa.kv_row = r->geo.kv_row;
  pa.n_head_kv = r->cfg.n_head_kv;
  pa.n_layer = r->cfg.n_layer;
  pa.n_ds = r->L.n_ds;
  // Rows go in launches of at most kProjRows (projection, then the append
  // that normalises, rotates and stores them); a fold-in is one such pair
  // with its pad rows, and the last pair of a step also rebuilds the mask.
  int64_t row0 = 0;
  do {
    const int32_t n = (int32_t)std::min<int64_t>(kProjRows, p.n_new - row0);
    pa.pos0 = p.start + row0;
    pa.slot0 = (int32_t)(pa.pos0 % r->cfg.cap);
    pa.n_rows = n;
    hipEvent_t t0, t1;
    if (n > 0) {
      next_events(r, RING_KERNEL_PROJ, &t0, &t1);
      if (int e = check_launch(launch_project(pa, s, t0, t1), "projection")) return e;
    }
    a.row0 = (int32_t)row0;
    a.n_rows = n;
    a.n_pad = p.bulk ? 0 : r->geo.a_step - n;
    a.do_mask = row0 + n >= p.n_new;
    next_events(r, RING_KERNEL_STEP, &t0, &t1);
    if (int e = check_launch(launch_step(a, s, t0, t1), "append from features")) return e;
    row0 += n;
  } while (row0 < p.n_new);
  if (fuse_write) mw = MirrorPending{};
  set_state(r, seq, committed, p);
  return ok();
}

namespace {
// The attention launch of `layer` over every sequence of the ring, without
// its tensors: ring geometry, each sequence's visible tiles (from its state
// of the last begin_step) and the split count.  Returns n_split.
int32_t attn_geometry(const ring* r, int32_t layer, AttnArgs* out, bool* swa_out) {
  AttnArgs a{};
  a.kring = r->kring;
  a.vring = r->vring;
  a.mask = r->mask;
  a.rope_noise = r->rope_noise;
  a.rope_q = r->rope_q;
  a.part_acc = r->part_acc;
  a.part_ml = r->part_ml;
  a.seq_stride = r->L.seq_stride;
  a.head_stride = (int64_t)r->L.n_tiles * kTileHalves;
  a.layer_offset = (int64_t)layer * r->cfg.n_head_kv * a.head_stride;
  a.n_seq = r->cfg.n_seq;
  a.n_head = r->cfg.n_head;
  a.n_head_kv = r->cfg.n_head_kv;
  a.group = r->L.group;
  a.q_len = r->cfg.q_len;
  a.m = r->L.m;
  a.cap = r->cfg.cap;
  a.kv_total = r->geo.kv_total;
  a.n_tiles = r->L.n_tiles;
  a.n_split = r->L.n_split;
  a.n_rb = 1;
  const int64_t cap = r->cfg.cap;
  const int32_t ring_tiles = (int32_t)((cap + kTile - 1) / kTile);
  a.ring_tiles = ring_tiles;
  const bool swa = layer < 64 && ((r->cfg.swa_layers >> layer) & 1u);
  if (swa) a.mask = r->mask_swa;
  int32_t max_count = 0;
  for (int i = 0; i < r->cfg.n_seq; ++i) {
    // Visible positions [committed - w, committed) sit in slots from
    // (committed - w) % cap on, circularly: w = win for full layers,
    // min(swa_window, win) for sliding-window layers.  (A deferred step's
    // new rows, which a fused launch attends as extra keys, need no tiles.)
    const int64_t c = r->committed[i];
    const int64_t win = std::min<int64_t>(c, cap);
    const int64_t w = swa ? std::min<int64_t>(r->cfg.swa_window, win) : win;
    int32_t first = 0, count = 0;
    if (w > 0 && w < win) {
      const int64_t s0 = (c - w) % cap, s1 = s0 + w;  // slot range [s0, s1), s1 may pass cap
      first = (int32_t)(s0 / kTile);
      const int64_t end_tile = (std::min<int64_t>(s1, cap) + kTile - 1) / kTile;
      count = (int32_t)(end_tile - first);
      if (s1 > cap) count += (int32_t)((s1 - cap + kTile - 1) / kTile);
      if (count > ring_tiles) first = 0, count = ring_tiles;
    } else if (w > 0) {
      count = (int32_t)((win + kTile - 1) / kTile);  // slots [0, win)
    }
    a.vis_first[i] = first;
    a.vis_count[i] = count;
    max_count = std::max(max_count, count);
  }
  // Splits for this launch: as many as give every wave at least one tile of
  // the widest window, at most the ring's (partial buffers are sized for it).
  const int32_t n_split = r->L.n_split_forced
                              ? r->L.n_split
                              : std::max(1, std::min(r->L.n_split, (max_count + 3) / 4));
  a.n_split = n_split;
  *out = a;
  if (swa_out) *swa_out = swa;
  return n_split;
}
}  // namespace

namespace {
// Checks of a ring_attn call (before any device work).
int check_attn(const ring* r, int32_t layer, const void* q, const void* k_noise,
               const void* v_noise, const float* out) {
  if (!r) return fail(RING_EINVAL, "ring is NULL");
  if (layer < 0 || layer >= r->cfg.n_layer) return fail(RING_ERANGE, "layer %d out of range", layer);
  if (!q || !k_noise || !v_noise || !out) return fail(RING_EINVAL, "NULL tensor pointer");
  const uintptr_t al = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_noise) |
                       reinterpret_cast<uintptr_t>(v_noise) | reinterpret_cast<uintptr_t>(out);
  if (al & 15) return fail(RING_EINVAL, "q, k_noise, v_noise and out must be 16-byte aligned");
  return RING_OK;
}

// Bytes of the split partials (F16 normalised outputs, then (max, sum) pairs 256-byte
// aligned) of a launch with n_split splits.
size_t partial_bytes(const ring* r, int32_t n_split, size_t* ml_offset) {
  const size_t rows = (size_t)r->cfg.n_seq * r->cfg.n_head_kv * n_split * r->L.mpad;
  const size_t acc = (size_t)align_up((int64_t)(rows * kHeadDim * 2), 256);
  if (ml_offset) *ml_offset = acc;
  return acc + rows * 2 * 4;
}

// The attention launches of a checked call, split partials in part_acc /
// part_ml (sized for the launch's splits).
int attn_launch(ring* r, int32_t layer, const void* q, const void* k_noise, const void* v_noise,
                float* out, void* stream, uint16_t* part_acc, float* part_ml) {
  if (int e = use_device(r)) return e;
  hipStream_t s = static_cast<hipStream_t>(stream);
  r->last_stream = s;

  AttnArgs a;
  bool swa = false;
  const int32_t n_split = attn_geometry(r, layer, &a, &swa);
  a.part_acc = part_acc;
  a.part_ml = part_ml;
  a.q = static_cast<const uint16_t*>(q);
  a.k_noise = static_cast<const uint16_t*>(k_noise);
  a.v_noise = static_cast<const uint16_t*>(v_noise);
  a.out = out;
  const int64_t cap = r->cfg.cap;
  const uint64_t bit = layer < 64 ? (1ull << layer) : 0;
  // With RING_ATTN_MERGE=kernel, the cross-split merge inside the attention
  // launch (a last-arriver merge per sequence x head and row block) where
  // the waves stream several tiles and the splits are few; else (default)
  // the merge launch below.
  a.n_rb = r->L.n_rb;
  const bool merge_in_launch = r->merge_in_launch && r->tickets && n_split > 1 &&
                               n_split <= kInKernelMergeMaxSplits && !attn_short_waves(a);
  if (merge_in_launch) a.tickets = r->tickets;
  hipEvent_t t0, t1;
  next_events(r, RING_KERNEL_ATTN, &t0, &t1);
  // Deferred steps owing this layer's rows or the index state: one fused
  // launch appends and rebuilds them and attends.
  bool fuse = false;
  for (const Pending& p : r->pending) fuse |= p.active && (p.layers_left & bit);
  if (fuse) {
    FusedAttnArgs f{};
    f.a = a;
    f.a.n_rb = r->L.n_rb;
    f.swa_layer = swa ? 1 : 0;
    f.n_attn_blocks = r->cfg.n_seq * r->cfg.n_head_kv * n_split * r->L.n_rb;
    f.slot_stride = (int32_t)r->L.slot_stride;
    f.slot_pos = r->slot_pos;
    const int64_t kv_row = r->geo.kv_row;
    for (int i = 0; i < 64; ++i) f.theta[i] = r->inv_freq_host[i];
    FusedSeqs& fs = f.fs;
    for (int i = 0; i < r->cfg.n_seq; ++i) {
      const Pending& p = r->pending[i];
      const int64_t c = r->committed[i];
      const int64_t win = std::min<int64_t>(c, cap);
      fs.committed[i] = (int32_t)c;
      fs.lo[i] = (int32_t)(c - (swa ? std::min<int64_t>(r->cfg.swa_window, win) : win));
      if (!p.active) continue;
      fs.start[i] = (int32_t)p.start;
      fs.start_mod[i] = (int32_t)(p.start % cap);
      if ((p.layers_left & bit) && p.n_new > 0) {
        fs.k_new[i] = reinterpret_cast<uint64_t>(p.k + (int64_t)layer * p.n_new * kv_row);
        fs.v_new[i] = reinterpret_cast<uint64_t>(p.v + (int64_t)layer * p.n_new * kv_row);
        fs.n_new[i] = (int32_t)p.n_new;
      }
    }
    if (int e = check_launch(launch_attn_fused(f, s, t0, t1), "ring_attn (fused step)")) return e;
    for (int32_t i = 0; i < r->cfg.n_seq; ++i) {
      Pending& p = r->pending[i];
      if (!p.active) continue;
      p.layers_left &= ~bit;
      if (p.index_left) {
        // slot_pos of the new rows is written; the masks and table are owed
        p.index_left = false;
        r->index_owed[i] = 1;
      }
      if (!p.layers_left) p = Pending{};
    }
  } else {
    // a plain launch reads the masks and the noise RoPE table
    for (int32_t i = 0; i < r->cfg.n_seq; ++i)
      if (int e = flush_index(r, i)) return e;
    a.n_rb = r->L.n_rb;
    if (int e = check_launch(launch_attn(a, s, t0, t1), "ring_attn")) return e;
  }
  if (n_split > 1 && !merge_in_launch) {
    MergeArgs m{};
    m.part_acc = part_acc;
    m.part_ml = part_ml;
    m.out = out;
    m.n_units = r->cfg.n_seq * r->cfg.n_head_kv;
    m.n_split = n_split;
    m.n_head = r->cfg.n_head;
    m.n_head_kv = r->cfg.n_head_kv;
    m.group = r->L.group;
    m.q_len = r->cfg.q_len;
    m.m = r->L.m;
    m.mpad = r->L.mpad;
    next_events(r, RING_KERNEL_MERGE, &t0, &t1);
    if (int e = check_launch(launch_merge(m, s, t0, t1), "ring_attn merge")) return e;
  }
  return ok();
}
}  // namespace

int ring_attn(ring_t* r, int32_t layer, const void* q, const void* k_noise, const void* v_noise,
              float* out, void* stream) {
  if (int e = check_attn(r, layer, q, k_noise, v_noise, out)) return e;
  return attn_launch(r, layer, q, k_noise, v_noise, out, stream, r->part_acc, r->part_ml);
}

int ring_attn_noalloc(ring_t* r, int32_t layer, const void* q, const void* k_noise,
                      const void* v_noise, float* out, void* stream) {
  if (int e = check_attn(r, layer, q, k_noise, v_noise, out)) return e;
  AttnArgs a;
  const int32_t n_split = attn_geometry(r, layer, &a, nullptr);
  size_t ml_off = 0;
  const size_t need = n_split > 1 ? partial_bytes(r, n_split, &ml_off) : 0;
  if (need > kStaticScratchBytes)
    return fail(RING_EINVAL,
                "ring_attn_noalloc: this launch's split partials need %zu bytes, more than the "
                "%zu of the static scratch (%d sequences x %d KV heads x %d splits); use ring_attn",
                need, kStaticScratchBytes, r->cfg.n_seq, r->cfg.n_head_kv, n_split);
  uint8_t* base = static_cast<uint8_t*>(static_scratch(r->device));
  if (!base) return fail(RING_EDEVICE, "static scratch of device %d is not resolved", r->device);
  return attn_launch(r, layer, q, k_noise, v_noise, out, stream, reinterpret_cast<uint16_t*>(base),
                     reinterpret_cast<float*>(base + ml_off));
}


namespace {
// Bytes of the floor buffer: counters, the timeout count, then the output.
size_t floor_counter_bytes(const ring* r) {
  return (size_t)align_up((int64_t)r->cfg.n_seq * r->cfg.n_head_kv * r->L.n_rb * 4, 256);
}
size_t floor_out_bytes(const ring* r) {
  // the attention floors' sums, or one word per wave of the projection floor
  const size_t attn = (size_t)r->cfg.n_seq * r->cfg.n_head_kv * r->L.n_rb * 32 * kHeadDim * 4;
  const size_t proj = (size_t)r->cfg.n_layer * 4 * r->cfg.n_head_kv * r->L.n_ds * 2 * 4;
  return std::max(attn, proj);
}
}  // namespace

int ring_profile_floor(ring_t* r, int32_t layer, int32_t kind, void* stream) {
  if (!r) return fail(RING_EINVAL, "ring is NULL");
  if (layer < 0 || layer >= r->cfg.n_layer) return fail(RING_ERANGE, "layer %d out of range", layer);
  if (kind < RING_FLOOR_EMPTY || kind > RING_FLOOR_SHARED_TILES)
    return fail(RING_EINVAL, "floor kind %d out of range", kind);
  if (kind == RING_FLOOR_SHARED_TILES && r->L.n_rb != 2)
    return fail(RING_EINVAL, "the shared-tile floor needs a ring with two 32-query blocks per "
                "KV head in work-groups of their own");
  if (kind == RING_FLOOR_PROJ_READ && !r->weights_set)
    return fail(RING_ESTATE, "the projection floor reads registered weights (ring_set_kv_weights)");
  if (kind == RING_FLOOR_HOLD) {
    if (int e = use_device(r)) return e;
    hipStream_t s = static_cast<hipStream_t>(stream);
    r->last_stream = s;
    FloorArgs none{};
    return check_launch(launch_floor(none, kind, s, nullptr, nullptr), "floor hold launch")
               ? RING_EDEVICE : ok();
  }
  if (kind == RING_FLOOR_PROJ_READ) {
    if (int e = use_device(r)) return e;
    hipStream_t s = static_cast<hipStream_t>(stream);
    r->last_stream = s;
    if (!r->floor_buf) {
      void* p = nullptr;
      if (hipMalloc(&p, floor_counter_bytes(r) + 256 + floor_out_bytes(r)) != hipSuccess) {
        (void)hipGetLastError();
        return fail(RING_ENOMEM, "floor buffer allocation failed");
      }
      r->floor_buf = static_cast<uint8_t*>(p);
      r->floor_last_kind = -1;
    }
    ProjFloorArgs f{};
    f.wpack = r->wpack;
    f.out = reinterpret_cast<float*>(r->floor_buf + floor_counter_bytes(r) + 256);
    f.n_layer = r->cfg.n_layer;
    f.n_head_kv = r->cfg.n_head_kv;
    f.n_ds = r->L.n_ds;
    hipEvent_t t0, t1;
    next_events(r, RING_KERNEL_FLOOR, &t0, &t1);
    if (int e = check_launch(launch_floor_proj(f, s, t0, t1), "projection floor launch")) return e;
    return ok();
  }
  if (r->L.n_rb * 32 != r->L.mpad)
    return fail(RING_EINVAL, "floor launches need one work-group per 32-query block");
  AttnArgs a;
  const int32_t n_split = attn_geometry(r, layer, &a, nullptr);
  const size_t part_bytes =
      (size_t)r->cfg.n_seq * r->cfg.n_head_kv * r->L.n_split * r->L.mpad * kHeadDim * 2;
  const bool with_partials = kind == RING_FLOOR_PARTIALS || kind == RING_FLOOR_LAST_ARRIVER ||
                             kind == RING_FLOOR_BARRIER || kind == RING_FLOOR_TWO_LAUNCH;
  if (with_partials && n_split < 2)
    return fail(RING_EINVAL, "this launch has one split: there are no partials to store");
  const bool ticketed = kind == RING_FLOOR_LAST_ARRIVER || kind == RING_FLOOR_BARRIER;
  if (ticketed && part_bytes >= (size_t(1) << 31))
    return fail(RING_EINVAL, "partials of %zu bytes exceed a buffer descriptor's range", part_bytes);
  const int64_t grid = (int64_t)r->cfg.n_seq * r->cfg.n_head_kv * n_split * r->L.n_rb;
  if (kind == RING_FLOOR_BARRIER && grid > floor_resident_blocks())
    return fail(RING_EINVAL, "%lld work-groups do not fit the device at once: no barrier",
                (long long)grid);
  if (int e = use_device(r)) return e;
  if (int e = flush_all(r)) return e;
  hipStream_t s = static_cast<hipStream_t>(stream);
  r->last_stream = s;
  const size_t cb = floor_counter_bytes(r);
  if (!r->floor_buf) {
    void* p = nullptr;
    if (hipMalloc(&p, cb + 256 + floor_out_bytes(r)) != hipSuccess) {
      (void)hipGetLastError();
      return fail(RING_ENOMEM, "floor buffer allocation failed");
    }
    r->floor_buf = static_cast<uint8_t*>(p);
    r->floor_last_kind = -1;
  }
  if (ticketed && kind != r->floor_last_kind) {
    // tickets count from zero for a series of one kind
    if (hipMemsetAsync(r->floor_buf, 0, cb + 256, s) != hipSuccess)
      return fail(RING_EDEVICE, "floor counter reset failed");
    r->floor_epoch = 0;
  }
  FloorArgs f{};
  f.kring = a.kring;
  f.vring = a.vring;
  f.seq_stride = a.seq_stride;
  f.layer_offset = a.layer_offset;
  f.head_stride = a.head_stride;
  f.part_acc = r->part_acc;
  f.part_ml = r->part_ml;
  f.part_bytes = (int64_t)part_bytes;
  f.counter = reinterpret_cast<uint32_t*>(r->floor_buf);
  f.err = reinterpret_cast<uint32_t*>(r->floor_buf + cb);
  f.out = reinterpret_cast<float*>(r->floor_buf + cb + 256);
  f.epoch = r->floor_epoch;
  f.n_seq = a.n_seq;
  f.n_head_kv = a.n_head_kv;
  f.n_split = n_split;
  f.n_rb = r->L.n_rb;
  if (kind == RING_FLOOR_SHARED_TILES) {
    // as many splits as the attention's grid has work-groups per head, each
    // one work-group for both query blocks
    f.n_split = n_split * r->L.n_rb;
    f.n_rb = 1;
  }
  f.ring_tiles = a.ring_tiles;
  for (int i = 0; i < RING_MAX_SEQ_INTERNAL; ++i) {
    f.vis_first[i] = a.vis_first[i];
    f.vis_count[i] = a.vis_count[i];
  }
  {
    AttnArgs sa = a;
    sa.n_split = n_split;
    f.rotate = attn_short_waves(sa) || kind == RING_FLOOR_READ_LOCKSTEP ? 0 : 1;
  }
  hipEvent_t t0, t1;
  next_events(r, RING_KERNEL_FLOOR, &t0, &t1);
  const int fk = kind == RING_FLOOR_TWO_LAUNCH    ? RING_FLOOR_PARTIALS
                 : kind == RING_FLOOR_READ_LOCKSTEP ? RING_FLOOR_READ
                                                    : kind;
  if (int e = check_launch(launch_floor(f, fk, s, t0, t1), "floor launch")) return e;
  if (kind == RING_FLOOR_TWO_LAUNCH) {
    // the ring's own merge launch over those partials, into the floor buffer
    MergeArgs m{};
    m.part_acc = r->part_acc;
    m.part_ml = r->part_ml;
    m.out = f.out;
    m.n_units = r->cfg.n_seq * r->cfg.n_head_kv;
    m.n_split = n_split;
    m.n_head = r->cfg.n_head;
    m.n_head_kv = r->cfg.n_head_kv;
    m.group = r->L.group;
    m.q_len = r->cfg.q_len;
    m.m = r->L.m;
    m.mpad = r->L.mpad;
    next_events(r, RING_KERNEL_FLOOR, &t0, &t1);
    if (int e = check_launch(launch_merge(m, s, t0, t1), "floor merge launch")) return e;
  }
  r->floor_last_kind = kind;
  if (kind == RING_FLOOR_BARRIER) ++r->floor_epoch;
  return ok();
}

int ring_profile_floor_timeouts(ring_t* r, uint32_t* timeouts) {
  if (!r || !timeouts) return fail(RING_EINVAL, "NULL argument");
  *timeouts = 0;
  if (!r->floor_buf) return ok();
  if (int e = use_device(r)) return e;
  if (hipStreamSynchronize(r->last_stream) != hipSuccess ||
      hipMemcpy(timeouts, r->floor_buf + floor_counter_bytes(r), 4, hipMemcpyDeviceToHost) !=
          hipSuccess)
    return fail(RING_EDEVICE, "reading the floor timeout count failed");
  return ok();
}

int ring_free(ring_t* r) {
  if (!r) return ok();
  int code = RING_OK;
  if (use_device(r) == RING_OK) {
    if (hipStreamSynchronize(r->last_stream) != hipSuccess)
      code = fail(RING_EDEVICE, "stream synchronisation failed in ring_free");
    if (r->owns_ws && hipFree(r->ws) != hipSuccess)
      code = fail(RING_EDEVICE, "hipFree failed");
    if (r->floor_buf && hipFree(r->floor_buf) != hipSuccess)
      code = fail(RING_EDEVICE, "hipFree failed");
    destroy_events(r);
  } else {
    code = RING_EDEVICE;
  }
  delete r;
  if (code == RING_OK) return ok();
  return code;
}

const char* ring_last_error(void) { return g_err.c_str(); }

int ring_describe(const ring_t* r, char* buf, size_t len) {
  if (!r || !buf || len == 0) return fail(RING_EINVAL, "NULL argument");
  const double mib = (double)r->cfg.n_layer * r->geo.kv_bytes_per_layer / (1024.0 * 1024.0);
  const int n = snprintf(buf, len,
                         "[draft-kv] ring: cap=%d kv_total=%d a_step=%d layers=%d seqs=%d f16 cache "
                         "%.1f MiB per seq, splits=%d",
                         r->cfg.cap, r->geo.kv_total, r->geo.a_step, r->cfg.n_layer, r->cfg.n_seq,
                         mib, r->L.n_split);
  if (r->cfg.d_model > 0 && n > 0 && (size_t)n < len) {
    const size_t used = strlen(buf);
    snprintf(buf + used, len - used, ", feature mirror d_model=%d", r->cfg.d_model);
  }
  if (r->cfg.swa_window > 0 && n > 0 && (size_t)n < len)
    snprintf(buf + strlen(buf), len - strlen(buf), ", swa_window=%d swa_layers=0x%llx",
             r->cfg.swa_window,
             (unsigned long long)r->cfg.swa_layers);
  return ok();
}

int ring_read_slot_pos(const ring_t* r, int32_t seq, int32_t* host_out) {
  if (!r || !host_out) return fail(RING_EINVAL, "NULL argument");
  if (seq < 0 || seq >= r->cfg.n_seq) return fail(RING_ERANGE, "seq %d out of range", seq);
  if (int e = use_device(r)) return e;
  if (int e = flush_all(const_cast<ring*>(r))) return e;
  if (hipDeviceSynchronize() != hipSuccess) return fail(RING_EDEVICE, "device synchronisation failed");
  if (hipMemcpy(host_out, r->slot_pos + (int64_t)seq * r->L.slot_stride, (size_t)r->cfg.cap * 4,
                hipMemcpyDeviceToHost) != hipSuccess)
    return fail(RING_EDEVICE, "hipMemcpy failed");
  return ok();
}

int ring_read_mask(const ring_t* r, int32_t seq, uint16_t* host_out) {
  if (!r || !host_out) return fail(RING_EINVAL, "NULL argument");
  if (seq < 0 || seq >= r->cfg.n_seq) return fail(RING_ERANGE, "seq %d out of range", seq);
  if (int e = use_device(r)) return e;
  if (int e = flush_all(const_cast<ring*>(r))) return e;
  if (hipDeviceSynchronize() != hipSuccess) return fail(RING_EDEVICE, "device synchronisation failed");
  const size_t n = (size_t)r->cfg.q_len * r->geo.kv_total;
  if (hipMemcpy(host_out, r->mask + (int64_t)seq * n, n * 2, hipMemcpyDeviceToHost) != hipSuccess)
    return fail(RING_EDEVICE, "hipMemcpy failed");
  return ok();
}

int ring_read_mask_swa(const ring_t* r, int32_t seq, uint16_t* host_out) {
  if (!r || !host_out) return fail(RING_EINVAL, "NULL argument");
  if (seq < 0 || seq >= r->cfg.n_seq) return fail(RING_ERANGE, "seq %d out of range", seq);
  if (!r->mask_swa) return fail(RING_ESTATE, "the ring has no sliding-window layers");
  if (int e = use_device(r)) return e;
  if (int e = flush_all(const_cast<ring*>(r))) return e;
  if (hipDeviceSynchronize() != hipSuccess) return fail(RING_EDEVICE, "device synchronisation failed");
  const size_t n = (size_t)r->cfg.q_len * r->geo.kv_total;
  if (hipMemcpy(host_out, r->mask_swa + (int64_t)seq * n, n * 2, hipMemcpyDeviceToHost) != hipSuccess)
    return fail(RING_EDEVICE, "hipMemcpy failed");
  return ok();
}

int ring_read_rows(const ring_t* r, int32_t seq, int32_t layer, int32_t slot0, int32_t n,
                   uint16_t* k_out, uint16_t* v_out) {
  if (!r) return fail(RING_EINVAL, "ring is NULL");
  if (seq < 0 || seq >= r->cfg.n_seq) return fail(RING_ERANGE, "seq %d out of range", seq);
  if (layer < 0 || layer >= r->cfg.n_layer) return fail(RING_ERANGE, "layer %d out of range", layer);
  if (n < 0 || slot0 < 0 || (int64_t)slot0 + n > r->geo.kv_total)
    return fail(RING_ERANGE, "slots [%d, %d) out of [0, %d)", slot0, slot0 + n, r->geo.kv_total);
  if (n == 0) return ok();
  if (int e = use_device(r)) return e;
  if (int e = flush_all(const_cast<ring*>(r))) return e;
  if (hipDeviceSynchronize() != hipSuccess) return fail(RING_EDEVICE, "device synchronisation failed");
  const int t0 = slot0 / kTile, t1 = (slot0 + n - 1) / kTile + 1;
  const int64_t head_stride = (int64_t)r->L.n_tiles * kTileHalves;
  const int kv_row = r->geo.kv_row;
  std::vector<uint16_t> buf((size_t)(t1 - t0) * kTileHalves);
  for (int which = 0; which < 2; ++which) {
    uint16_t* dst = which == 0 ? k_out : v_out;
    if (!dst) continue;
    const uint16_t* base = (which == 0 ? r->kring : r->vring) + seq * r->L.seq_stride +
                           (int64_t)layer * r->cfg.n_head_kv * head_stride;
    for (int h = 0; h < r->cfg.n_head_kv; ++h) {
      if (hipMemcpy(buf.data(), base + h * head_stride + (int64_t)t0 * kTileHalves,
                    buf.size() * 2, hipMemcpyDeviceToHost) != hipSuccess)
        return fail(RING_EDEVICE, "hipMemcpy failed");
      for (int i = 0; i < n; ++i) {
        const int slot = slot0 + i;
        const uint16_t* tile = buf.data() + (int64_t)(slot / kTile - t0) * kTileHalves;
        for (int d = 0; d < kHeadDim; ++d) {
          const int off = which == 0 ? k_frag_index(slot % kTile, d) : v_frag_index(slot % kTile, d);
          dst[(int64_t)i * kv_row + h * kHeadDim + d] = tile[off];
        }
      }
    }
  }
  return ok();
}

int ring_read_state(const ring_t* r, int32_t seq, int64_t* next_pos, int64_t* held_lo) {
  if (!r || !next_pos || !held_lo) return fail(RING_EINVAL, "NULL argument");
  if (seq < 0 || seq >= r->cfg.n_seq) return fail(RING_ERANGE, "seq %d out of range", seq);
  *next_pos = r->next_pos[seq];
  *held_lo = r->held_lo[seq];
  return ok();
}

int ring_profile_enable(ring_t* r, int32_t max_launches) {
  if (!r || max_launches < 0 || max_launches > (1 << 20))
    return fail(RING_EINVAL, "bad ring or max_launches");
  if (int e = use_device(r)) return e;
  if (hipStreamSynchronize(r->last_stream) != hipSuccess)
    return fail(RING_EDEVICE, "stream synchronisation failed");
  destroy_events(r);
  for (auto& v : r->prof_ev) {
    v.resize(2 * (size_t)max_launches, nullptr);
    for (auto& e : v) {
      if (hipEventCreate(&e) != hipSuccess) {
        e = nullptr;
        destroy_events(r);
        return fail(RING_EDEVICE, "hipEventCreate failed");
      }
    }
  }
  r->prof_max = max_launches;
  return ok();
}

int ring_profile_read(ring_t* r, int32_t kernel, int32_t* n_launches, double* total_ms) {
  if (!r || !n_launches || !total_ms || kernel < 0 || kernel > RING_KERNEL_FLOOR)
    return fail(RING_EINVAL, "bad argument");
  if (int e = use_device(r)) return e;
  double total = 0.0;
  const int n = r->prof_used[kernel];
  for (int i = 0; i < n; ++i) {
    float ms = 0.0f;
    hipEvent_t t0 = r->prof_ev[kernel][2 * i], t1 = r->prof_ev[kernel][2 * i + 1];
    if (hipEventSynchronize(t1) != hipSuccess || hipEventElapsedTime(&ms, t0, t1) != hipSuccess)
      return fail(RING_EDEVICE, "event timing failed");
    total += ms;
  }
  r->prof_used[kernel] = 0;
  *n_launches = n;
  *total_ms = total;
  return ok();
}

static_assert(RING_STAMP_WAVES == kStampWaves && RING_STAMP_WORDS == kStampWords &&
                  RING_STAMPS_PROJ + 1 == kStampRegions,
              "stamp layout of the header and the kernels");

int ring_profile_stamps(ring_t* r, int32_t region, uint64_t* host, int32_t max_waves,
                        int32_t clear, int32_t* clock_khz) {
  if (!r || region < 0 || region >= kStampRegions || max_waves < 0 ||
      (max_waves > 0 && !host))
    return fail(RING_EINVAL, "bad argument");
  if (int e = use_device(r)) return e;
  void* base = nullptr;
  if (stamps_address(&base) != hipSuccess || !base)
    return fail(RING_ESTATE, "library built without wave stamps (libringkv_stamps.so has them)");
  if (hipDeviceSynchronize() != hipSuccess)
    return fail(RING_EDEVICE, "device synchronisation failed");
  const size_t words = (size_t)kStampWaves * kStampWords;
  uint64_t* dev = reinterpret_cast<uint64_t*>(base) + (size_t)region * words;
  const size_t n = (size_t)std::min(max_waves, kStampWaves) * kStampWords;
  if (n && hipMemcpy(host, dev, n * 8, hipMemcpyDeviceToHost) != hipSuccess)
    return fail(RING_EDEVICE, "stamp copy failed");
  if (clear && (hipMemset(dev, 0, words * 8) != hipSuccess || hipDeviceSynchronize() != hipSuccess))
    return fail(RING_EDEVICE, "stamp clear failed");
  if (clock_khz) {
    int khz = 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, r->device) != hipSuccess)
      return fail(RING_EDEVICE, "clock rate query failed");
    *clock_khz = khz;
  }
  return ok();
}

}  // extern "C"
