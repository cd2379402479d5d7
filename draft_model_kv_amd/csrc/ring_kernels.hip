// ring_kernels.hip -- HIP kernels of the draft-KV ring for gfx950 (MI355X).
//
//   k_ring_step   begin_step: mod-cap append of new K/V rows with RoPE at
//                 their absolute positions (bulk chunk or fixed-shape
//                 fold-in with pad rows to the trash slot), then slot_pos,
//                 the 0/-inf window mask and the noise RoPE table.
//                 Page "DFLASH2_RING_PORT.md", sections 1.1-1.4.
//                 k_ring_step_batch: the fold-in steps of several sequences
//                 in one launch.
//   k_ring_attn   masked GQA attention of the q_len noise queries over the
//                 ring, split-K over 32-slot ring tiles, matrix-core QK^T and
//                 PV, online softmax, per-workgroup merge of its waves; the
//                 noise rows are rotated, stored to ring rows cap + r and
//                 attended one per wave.
//   k_ring_merge  cross-split merge of the partial (max, sum, acc) triples.
#include "ring_kernels.h"

#include <math.h>

#include <mutex>

namespace ringkv {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kNegInf = -__builtin_inff();

// Global-memory pointers for rows that arrive as integer addresses: loads
// through a generic pointer become flat loads, and a flat load in flight
// makes the compiler wait for every other load before the next use of any.
typedef const __attribute__((address_space(1))) uint16_t gcu16;
typedef __attribute__((address_space(1))) uint16_t gu16;
typedef _Float16 half4 __attribute__((ext_vector_type(4)));

// Per-wave timestamps of the profiling build (RING_WAVE_STAMPS): stamp p is
// the device clock when the wave passes point p of its work (the scheduler
// keeps every instruction on its side of the point); flush stores the
// stamps, HW_ID and XCC_ID of the wave with lane 0's vector stores.  In the
// product build both are empty.
#ifdef RING_WAVE_STAMPS
__device__ uint64_t g_wave_stamps[kStampRegions * kStampWaves * kStampWords];
struct WaveStamps {
  uint64_t t[kStampPhases];
  __device__ WaveStamps() {
#pragma unroll
    for (int p = 0; p < kStampPhases; ++p) t[p] = 0;
    t[0] = __builtin_amdgcn_s_memrealtime();
  }
  __device__ inline void at(int p) {
    __builtin_amdgcn_sched_barrier(0);
    t[p] = __builtin_amdgcn_s_memrealtime();
    __builtin_amdgcn_sched_barrier(0);
  }
  __device__ inline void flush(int region, uint32_t wave_gid) {
    at(kStampPhases - 1);
    if (wave_gid >= (uint32_t)kStampWaves || (threadIdx.x & 63) != 0) return;
    uint64_t* d = g_wave_stamps + ((size_t)region * kStampWaves + wave_gid) * kStampWords;
#pragma unroll
    for (int p = 0; p < kStampPhases; ++p) d[p] = t[p];
    d[kStampPhases] = __builtin_amdgcn_s_getreg(4 | (31 << 11));       // HW_ID
    d[kStampPhases + 1] = __builtin_amdgcn_s_getreg(20 | (3 << 11));   // XCC_ID, bits 3:0
  }
};
#else
struct WaveStamps {
  __device__ inline void at(int) {}
  __device__ inline void flush(int, uint32_t) {}
};
#endif

hipError_t stamps_address(void** ptr) {
#ifdef RING_WAVE_STAMPS
  return hipGetSymbolAddress(ptr, HIP_SYMBOL(g_wave_stamps));
#else
  *ptr = nullptr;
  return hipErrorNotSupported;
#endif
}

// 2^x with the hardware instruction: about 1 ulp for normal results; results
// below 2^-126 flush to zero and 2^-inf = 0.  Softmax weights that small
// change no output at the precision that is kept.
__device__ inline float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
// sin and cos of an angle x (radians, fp64): x is reduced to the nearest
// whole turn in fp64 (|x| < 2^31 here, so the reduction loses at most about
// 2e-7 rad), and the remaining fraction of a turn (|f| <= 1/2), rounded to
// fp32, goes to the hardware sine and cosine, which take their argument in
// turns (measured on gfx950 over [-1/2, 1/2] against fp64: at most 1.25e-7
// absolute error, below the fp32 sincosf of f * 2 pi at 2.1e-7).
__device__ inline void sincos_turns_f32(double x, float& s, float& c) {
  const double turns = x * 0.15915494309189533577;  // 1 / (2 pi)
  const float f = (float)(turns - rint(turns));
  s = __builtin_amdgcn_sinf(f);
  c = __builtin_amdgcn_cosf(f);
}

// sin and cos (fp64) of a rotary angle x = p * theta (|x| < 2^31): x less
// the nearest whole number of turns, with 2 pi split into two doubles (Cody
// and Waite, "Software Manual for the Elementary Functions", 1980) and each
// product taken off by one fused multiply-add (error below 1e-15 for
// |x| < 2^31), then the library sincos of the reduced angle, |r| <= pi, which
// needs none of its long argument reduction.
__device__ inline void sincos_angle(double x, double* s, double* c) {
  const double k = rint(x * 0.15915494309189535);       // 1 / (2 pi)
  double r = fma(-k, 6.283185307179586, x);             // 2 pi, leading double
  r = fma(-k, 2.4492935982947064e-16, r);               // 2 pi, the rest
  sincos(r, s, c);
}

// log2(e) / sqrt(128): folds the 1/sqrt(head_dim) score scale and the
// change of base for exp2 into the query.
constexpr double kQScale = 1.4426950408889634074 / 11.313708498984760390;

// ---------------------------------------------------------------------------
// F16 helpers
// ---------------------------------------------------------------------------
__device__ inline double f16_to_f64(uint16_t b) {
  return (double)__builtin_bit_cast(_Float16, b);
}

// binary64 -> binary16 with a single rounding to nearest even.  Rounds to
// binary32 with round-to-odd first, then to binary16 with the hardware's
// round-to-nearest-even: binary32 carries 24 >= 11 + 2 significand bits, so
// the two roundings equal one (Boldo and Melquiond, "Emulation of FMA and
// correctly rounded sums: proved algorithms using rounding to odd", IEEE
// Trans. Computers 57(4), 2008).
__device__ inline uint16_t f64_to_f16_rne(double x) {
  float f = (float)x;
  const double back = (double)f;
  if (back != x) {
    uint32_t b = __builtin_bit_cast(uint32_t, f);
    if (fabs(back) > fabs(x)) b -= 1;  // round-to-nearest went away from zero
    b |= 1u;                           // truncation with the sticky bit set
    f = __builtin_bit_cast(float, b);
  }
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// Work-group barrier that orders LDS only: global loads and stores issued
// before it stay in flight (a full __syncthreads() would first wait for all of
// them).  No kernel here passes data between waves through global memory.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Rotate the pair (x, y) by the angle whose cosine and sine are (c, s); no
// contraction so the products round as written.
__device__ inline void rot_pair(double x, double y, double c, double s,
                                double& xr, double& yr) {
#pragma clang fp contract(off)
  xr = x * c - y * s;
  yr = y * c + x * s;
}

// Index state of one sequence after a step, one work-group of 256 threads per
// 256 slots (block mblk): slot_pos of the new slots, the 0 / -inf window mask
// (and the sliding-window mask), and in block 0 the cos / sin table of the
// noise positions committed + i.
// Slot s of the index state, given its slot_pos before the step (sp, read
// by the caller; anything for s >= cap).
__device__ inline void index_slot(const StepArgs& a, int s, int64_t sp) {
  if (s >= a.kv_total) return;
  bool vis, vis_swa = false;
  if (s < a.cap) {
    int d = s - a.start_mod;  // offset of slot s from the first new slot, mod cap
    if (d < 0) d += a.cap;
    if (d < a.n_new) {
      sp = a.start + d;
      a.slot_pos[s] = (int32_t)sp;
    }
    vis = sp >= a.lo && sp < a.committed;
    vis_swa = sp >= a.swa_lo && sp < a.committed;
  } else {
    vis = s < a.cap + a.q_len;  // noise slots: visible to every noise row
  }
  const uint16_t mv = vis ? 0x0000u : 0xFC00u;
  for (int i = 0; i < a.q_len; ++i) a.mask[(int64_t)i * a.kv_total + s] = mv;
  if (a.mask_swa) {
    // sliding-window layers: the window above; noise slot cap + j visible to
    // noise rows i >= j only
    for (int i = 0; i < a.q_len; ++i) {
      const bool v = s < a.cap ? vis_swa : (s - a.cap <= i);
      a.mask_swa[(int64_t)i * a.kv_total + s] = v ? 0x0000u : 0xFC00u;
    }
  }
}

__device__ inline void index_block(const StepArgs& a, int mblk, int t) {
  if (mblk == 0) {
    // cos / sin of the noise positions committed + i, for every frequency.
    for (int item = t; item < a.q_len * 64; item += 256) {
      const int i = item >> 6, f = item & 63;
      double sn, cs;
      sincos_angle((double)(a.committed + i) * a.inv_freq[f], &sn, &cs);
      a.rope_noise[2 * item] = cs;
      a.rope_noise[2 * item + 1] = sn;
      a.rope_q[2 * item] = (float)cs;
      a.rope_q[2 * item + 1] = (float)sn;
    }
  }
  const int s = mblk * 256 + t;
  index_slot(a, s, s < a.cap ? a.slot_pos[s] : 0);
}

// ---------------------------------------------------------------------------
// begin_step: append + slot_pos + mask + noise RoPE table
// ---------------------------------------------------------------------------
// Work-group blk of one sequence's launch: rows first (n_rows + n_pad of
// every layer), then the index blocks.
__device__ inline void step_block(const StepArgs& a, const int blk) {
  const int t = threadIdx.x;
  const int rows_per_layer = a.n_rows + a.n_pad;
  const int n_row_blocks = rows_per_layer * a.n_layer;
  const int kv_row = a.n_head_kv * kHeadDim;
  const int64_t head_stride = (int64_t)a.n_tiles * kTileHalves;
  const int64_t layer_stride = head_stride * a.n_head_kv;

  if (blk < n_row_blocks) {
    // One row (one position, all KV heads of one layer) per work-group.
    __shared__ double2 cs_row[64];  // (cos, sin) of p * theta_f
    const int layer = blk / rows_per_layer;
    if (layer < 64 && ((a.layer_skip >> layer) & 1u)) return;
    const int i = blk - layer * rows_per_layer;
    const bool pad = i >= a.n_rows;
    // Every pad row is the same zero row for the same trash slot: the first
    // pad block writes it and the others have nothing to add (many blocks
    // storing to one row's cache lines at once queue behind each other).
    if (pad && i != a.n_rows) return;
    int slot;
    int64_t p = 0;
    gcu16* ksrc = nullptr;
    gcu16* vsrc = nullptr;
    if (!pad) {
      const int idx = a.row0 + i;
      p = a.start + idx;
      slot = (int)(p % a.cap);
      if (!a.proj) {
        ksrc = (gcu16*)a.k_new + ((int64_t)layer * a.n_new + idx) * kv_row;
        vsrc = (gcu16*)a.v_new + ((int64_t)layer * a.n_new + idx) * kv_row;
      }
      if (t < 64) {
        double sn, cs;
        sincos_angle((double)p * a.inv_freq[t], &sn, &cs);
        cs_row[t] = make_double2(cs, sn);
      }
    } else {
      slot = a.trash_slot;
    }
    // Row from projected features: the sum of the d-slices (fixed order) of
    // every column, K then V, staged in LDS; all loads of a thread in flight
    // together.
    __shared__ float raw[2 * kProjMaxKvHeads * kHeadDim];
    if (a.proj && !pad) {
      const int n4 = 2 * kv_row / 4;
      const int64_t ds4 = (int64_t)kProjRows * 2 * kv_row / 4;
      const float4* pr =
          (const float4*)(a.proj + ((int64_t)layer * a.n_ds * kProjRows + i) * 2 * kv_row);
#pragma unroll 2
      for (int c = t; c < n4; c += 256) {
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
        for (int ds = 0; ds < a.n_ds; ++ds) {
          const float4 v = pr[ds * ds4 + c];
          acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
        }
        ((float4*)raw)[c] = acc;
      }
    }
    lds_barrier();
    const int s_t = slot & (kTile - 1);
    const int64_t tile_off = (int64_t)(slot >> 5) * kTileHalves;
    uint16_t* kl = a.kring + layer * layer_stride + tile_off;
    uint16_t* vl = a.vring + layer * layer_stride + tile_off;
    for (int item = t; item < a.n_head_kv * 64; item += 256) {
      const int h = item >> 6, f = item & 63;
      uint16_t* kd = kl + h * head_stride;
      uint16_t* vd = vl + h * head_stride;
      if (pad) {
        kd[k_frag_index(s_t, f)] = 0;
        kd[k_frag_index(s_t, f + 64)] = 0;
        vd[v_frag_index(s_t, f)] = 0;
        vd[v_frag_index(s_t, f + 64)] = 0;
      } else if (a.proj) {
        // Scale K to unit RMS over its KV head (the 64 lanes of this wave
        // hold head h, two dims each) times k_norm, rotate, round once to F16.
        const float xs = raw[h * kHeadDim + f], ys = raw[h * kHeadDim + f + 64];
        const float vxs = raw[kv_row + h * kHeadDim + f], vys = raw[kv_row + h * kHeadDim + f + 64];
        double x = xs, y = ys;
        double ss = x * x + y * y;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
        const double inv = 1.0 / sqrt(ss / (double)kHeadDim + a.eps);
        x = x * inv * (double)a.k_norm[layer * kHeadDim + f];
        y = y * inv * (double)a.k_norm[layer * kHeadDim + f + 64];
        const double2 cs = cs_row[f];
        double xr, yr;
        rot_pair(x, y, cs.x, cs.y, xr, yr);
        kd[k_frag_index(s_t, f)] = f64_to_f16_rne(xr);
        kd[k_frag_index(s_t, f + 64)] = f64_to_f16_rne(yr);
        vd[v_frag_index(s_t, f)] = __builtin_bit_cast(uint16_t, (_Float16)vxs);
        vd[v_frag_index(s_t, f + 64)] = __builtin_bit_cast(uint16_t, (_Float16)vys);
      } else {
        const double x = f16_to_f64(ksrc[h * kHeadDim + f]);
        const double y = f16_to_f64(ksrc[h * kHeadDim + f + 64]);
        const double2 cs = cs_row[f];
        double xr, yr;
        rot_pair(x, y, cs.x, cs.y, xr, yr);
        kd[k_frag_index(s_t, f)] = f64_to_f16_rne(xr);
        kd[k_frag_index(s_t, f + 64)] = f64_to_f16_rne(yr);
        vd[v_frag_index(s_t, f)] = vsrc[h * kHeadDim + f];
        vd[v_frag_index(s_t, f + 64)] = vsrc[h * kHeadDim + f + 64];
      }
    }
    return;
  }
  if (!a.do_mask) return;
  index_block(a, blk - n_row_blocks, t);
}

__global__ __launch_bounds__(256) void k_ring_step(StepArgs a) { step_block(a, blockIdx.x); }

// Fold-in steps of b.n_seq sequences: blocks_per_seq work-groups each.
__global__ __launch_bounds__(256) void k_ring_step_batch(StepBatchArgs b) {
  const int j = blockIdx.x / b.blocks_per_seq;
  const int blk = blockIdx.x - j * b.blocks_per_seq;
  StepArgs a = b.a;
  const int64_t seq = b.seq[j];
  a.kring += seq * b.seq_stride;
  a.vring += seq * b.seq_stride;
  a.slot_pos += seq * b.slot_stride;
  const int64_t mask_stride = (int64_t)a.q_len * a.kv_total;
  a.mask += seq * mask_stride;
  if (a.mask_swa) a.mask_swa += seq * mask_stride;
  a.rope_noise += seq * a.q_len * 128;
  a.rope_q += seq * a.q_len * 128;
  a.k_new = reinterpret_cast<const uint16_t*>(b.k_new[j]);
  a.v_new = reinterpret_cast<const uint16_t*>(b.v_new[j]);
  a.start = b.start[j];
  a.start_mod = b.start_mod[j];
  a.committed = b.committed[j];
  a.lo = b.lo[j];
  a.swa_lo = b.swa_lo[j];
  a.n_new = b.n_new[j];
  a.row0 = 0;
  a.n_rows = a.n_new;
  a.n_pad = b.a_step - a.n_new;
  step_block(a, blk);
}

// ---------------------------------------------------------------------------
// ring_attn
// ---------------------------------------------------------------------------
__device__ inline f32x16 mfma32(half8 a, half8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ inline float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ inline float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// Query fragments (B operand of S^T = K Q^T): query block mb, chunk c, lane.
// Kept in registers (QL false) or read from LDS at each use (QL true: two
// query blocks, or waves that attend one tile).
template <int MB, bool QL = (MB > 1)>
struct QFrag {
  static constexpr bool kLds = QL;
  half8 hi[kLds ? 1 : MB][kLds ? 1 : 8];
  half8 lo[kLds ? 1 : MB][kLds ? 1 : 8];
};

// Additive mask of a tile from its mask words (plain launch): accumulator
// row j = 4 jj + u of query block mb takes mw[mb][2 jj + (u >> 1)], two F16
// per word, the low half for even u.
template <int MB>
struct MaskWords {
  const uint32_t (&mw)[MB][8];
  __device__ inline void operator()(int mb, f32x16& s) const {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t w = mw[mb][2 * (j >> 2) + ((j & 3) >> 1)];
      s[j] += (j & 1) ? f16_hi(w) : f16_lo(w);
    }
  }
};

// Visibility of a tile from its slot_pos (fused launch): slot s is visible
// when its position p lies in [lo, hi), tested as (unsigned)(p - lo) < span
// with span = hi - lo; a hidden slot's score becomes -inf.  When the launch
// attends the step's new rows as extra keys, hi is their first position
// `start`, which hides their slots whatever the tile's load finds there: the
// new rows' positions (written by another wave of this launch) are >= start,
// and an older occupant of such a slot lies below lo (evicted: position
// start + j - cap < committed - cap <= lo) or at or above start (a rolled-back
// row).  Otherwise hi = committed.  sp[jj] holds slots 8 jj + 4 hl + 0..3,
// accumulator rows j = 4 jj + 0..3.
struct SlotVis {
  const int4 (&sp)[4];
  uint32_t lo, span;
  __device__ static inline int pos(const int4& v, int u) {
    return u == 0 ? v.x : u == 1 ? v.y : u == 2 ? v.z : v.w;
  }
  __device__ inline void operator()(int, f32x16& s) const {
#pragma unroll
    for (int j = 0; j < 16; ++j)
      s[j] = (uint32_t)pos(sp[j >> 2], j & 3) - lo < span ? s[j] : kNegInf;
  }
};

// One 32-slot tile: S^T = K Q^T (Q as hi + lo F16), mask, online softmax,
// O^T += V^T P^T.
//   kc, vc   K and V chunks (fragment order, see ring_layout.h)
//   mask     MaskWords or SlotVis, applied to S^T of each query block
//   limit    rows r >= limit of this tile are hidden (-inf)
template <int MB, bool QL, class Mask>
__device__ inline void attend_tile(const half8 (&kc)[8], const half8 (&vc)[8],
                                   const Mask& mask, int limit, int hl,
                                   const QFrag<MB, QL>& q, const half8* q_lds, int lane,
                                   float (&m_run)[MB], float (&l_run)[MB],
                                   f32x16 (&o)[MB][4]) {
  // Query fragments from LDS: the lane index passes through an empty asm
  // statement at every tile, so the compiler cannot hoist the LDS reads out
  // of the tile loop (held in registers, two query blocks' fragments take
  // 128 VGPRs and push the accumulators to scratch).
  int qln = lane;
  if constexpr (QL) asm volatile("" : "+v"(qln));
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    f32x16 s = {};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      half8 qh, ql;
      if constexpr (QL) {
        qh = q_lds[((mb * 2 + 0) * 8 + c) * 64 + qln];
        ql = q_lds[((mb * 2 + 1) * 8 + c) * 64 + qln];
      } else {
        qh = q.hi[mb][c];
        ql = q.lo[mb][c];
      }
      s = mfma32(kc[c], qh, s);
      s = mfma32(kc[c], ql, s);
    }
    float mx = kNegInf;
    mask(mb, s);
    if (limit < kTile) {  // ragged tile: rows r >= limit are not ring slots
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = 8 * (j >> 2) + 4 * hl + (j & 3);
        if (r >= limit) s[j] = kNegInf;
      }
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[j]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_old = m_run[mb];
    const float mnew = fmaxf(m_old, mx);
    float alpha = 1.0f;
    float ls = 0.0f;
    if (mnew == kNegInf) {
#pragma unroll
      for (int j = 0; j < 16; ++j) s[j] = 0.0f;
    } else {
      alpha = exp2_hw(m_run[mb] - mnew);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        s[j] = exp2_hw(s[j] - mnew);
        ls += s[j];
      }
    }
    ls += __shfl_xor(ls, 32);
    l_run[mb] = l_run[mb] * alpha + ls;
    m_run[mb] = mnew;
    half8 pb0, pb1;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pb0[e] = (_Float16)s[e];
      pb1[e] = (_Float16)s[8 + e];
    }
    // Rescale the accumulators only when some query's running max moved
    // (never on a wave's first tile, whose accumulators are still zero).
    if (__any(alpha != 1.0f && m_old != kNegInf)) {
#pragma unroll
      for (int b = 0; b < 4; ++b) o[mb][b] *= alpha;
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      o[mb][b] = mfma32(vc[2 * b], pb0, o[mb][b]);
      o[mb][b] = mfma32(vc[2 * b + 1], pb1, o[mb][b]);
    }
  }
}

// A fused launch's per-sequence fields of one sequence (wave-uniform).
struct FusedLane {
  uint64_t k_new, v_new;
  int start, start_mod, n_new, committed, lo;
};

// Fetch them for every sequence at kernel entry, lane i holding sequence
// i % kFusedMaxSeq (one vector load per field, issued together), then pick
// sequence `seq` with readlane once it is known.
struct FusedLaneVec {
  uint64_t k_new, v_new;
  int start, start_mod, n_new, committed, lo;
  double theta;   // theta of frequency lane
};

__device__ inline FusedLaneVec fused_fetch(const FusedAttnArgs& f) {
  const int i = threadIdx.x & (kFusedMaxSeq - 1);
  FusedLaneVec v;
  v.k_new = f.fs.k_new[i];
  v.v_new = f.fs.v_new[i];
  v.start = f.fs.start[i];
  v.start_mod = f.fs.start_mod[i];
  v.n_new = f.fs.n_new[i];
  v.committed = f.fs.committed[i];
  v.lo = f.fs.lo[i];
  v.theta = f.theta[threadIdx.x & 63];
  return v;
}

__device__ inline uint64_t readlane64(uint64_t x, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)x, l);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(x >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

__device__ inline FusedLane fused_pick(const FusedLaneVec& v, int seq) {
  FusedLane u;
  u.k_new = readlane64(v.k_new, seq);
  u.v_new = readlane64(v.v_new, seq);
  u.start = __builtin_amdgcn_readlane(v.start, seq);
  u.start_mod = __builtin_amdgcn_readlane(v.start_mod, seq);
  u.n_new = __builtin_amdgcn_readlane(v.n_new, seq);
  u.committed = __builtin_amdgcn_readlane(v.committed, seq);
  u.lo = __builtin_amdgcn_readlane(v.lo, seq);
  return u;
}

// What a fused launch tells the attention body about its sequence's
// deferred step (unused in a plain launch).
struct FusedCtx {
  gcu16* k_new;             // this layer's new K rows, at this KV head's column
  gcu16* v_new;
  int32_t* slot_pos;        // the sequence's slot_pos row (the new rows' entries are
                            // written by the waves that store those rows)
  double invf;              // theta of frequency `lane`
  int kv_row;
  int start, start_mod, n_new, committed, lo, cap;
  int swa;                  // sliding-window layer: causal noise block
};

// Work-group: NW waves for one (sequence, KV head, split).  Every split
// runs the same body; the q_len noise rows of a (sequence, head) are spread
// one per wave over its waves, so no wave carries more than one ring tile
// plus one noise row when the tiles divide evenly.
//
// Order of work (memory latency is the cost on a 4096-slot ring, so every
// load is issued as early as its inputs allow):
//   1. loads for the query build, for the wave's extra key row (a noise row,
//      or in a fused launch one of the step's new rows) and for its first
//      ring tile;
//   2. the work-group rotates/scales/splits the queries into LDS, and a wave
//      that owns an extra row rotates it (fp64, one rounding to F16), stores
//      it to its ring row and stages it in LDS; one barrier;
//   3. that wave folds the row into its online softmax (dot products on the
//      vector unit, P V on the matrix core) while its ring tile is still in
//      flight (a fused launch's tile pass hides the new slots, which it
//      attends this way);
//   4. each wave streams its ring tiles;
//   5. waves merge through LDS; the work-group writes its output or partial.
// Every global load of the fast path is issued unconditionally from an
// in-bounds (clamped) address and selected afterwards: the compiler can then
// wait for each group of loads alone instead of draining all of them at a
// control-flow join.
// SHARE: the merge buffer reuses the prologue bytes (a work-group small
// enough for two per CU).
template <int MB, int NW, bool FUSED = false, bool SHARE = false>
struct AttnShape {
  static constexpr int MP = MB * 32;               // padded queries
  static constexpr int NT = NW * 64;               // threads
  static constexpr int kQBytes = MB * 2 * 8 * 64 * 16;
  static constexpr int kRowBytes = NW * 2 * kHeadDim * 2;  // one K and one V row per wave
  static constexpr int kMergeBytes = MB * 4 * NW * 4 * 64 * 16;  // reduce-scatter buffer
  // fp32 (cos, sin) of the noise positions, [q_len <= 32][64][2]: read by the
  // query build only, so it shares bytes with the merge buffer (written after
  // the query build's barrier).
  static constexpr int kRopeOffset = kQBytes + kRowBytes;
  static constexpr int kRopeBytes = 32 * 64 * 2 * 4;  // = 4 passes of NT float4
  static_assert(kRopeBytes == 4 * NT * 16, "rope passes fill the table bytes");
  // The query fragments and the noise-row buffers live until a wave's tile
  // loop ends.  With one query block the merge buffer has bytes of its own,
  // so a wave writes it as soon as its own loop ends; with two it reuses the
  // prologue bytes behind a barrier that every wave reaches after its loop.
  static constexpr bool kOwnMergeBytes = !SHARE && kQBytes + kRowBytes + kMergeBytes <= 96 * 1024;
  static constexpr int kMergeOffset = kOwnMergeBytes ? kQBytes + kRowBytes : 0;
  static constexpr int kLdsBytes =
      kOwnMergeBytes ? kQBytes + kRowBytes + kMergeBytes
                     : (kQBytes + kRowBytes > kMergeBytes ? kQBytes + kRowBytes : kMergeBytes);
  static_assert(kRopeOffset + kRopeBytes <= kLdsBytes, "rope table fits the merge bytes");
  static constexpr int kTotalLds = kLdsBytes;
};

// One extra key row of this wave's (sequence, head), already loaded: lane f
// holds K and V at dims f and f + 64, (cos, sin) of frequency f at the row's
// position (plain launch), and the mask word of its query in each query
// block.  Extra row e < q_len is noise row e; in a fused launch, extra row
// q_len + j is the step's new row j of this layer (position start + j).
template <int MB>
struct NoiseRow {
  uint16_t kx, ky, vx, vy;
  double2 cs;
  uint16_t mask[MB];
};

template <int MB, bool FUSED>
__device__ __forceinline__ void load_noise_row(const AttnArgs& a, const FusedCtx& fx, int seq,
                                               int g, int r, const uint16_t* mask_seq,
                                               const unsigned (&qrow)[MB], int lane,
                                               NoiseRow<MB>& nr) {
  const int kv_row = a.n_head_kv * kHeadDim;
  if constexpr (FUSED) {
    // noise row r, or new row r - q_len (loaded from a pointer picked
    // without a branch, so that the load is not sunk behind later ones);
    // (cos, sin) are computed where the row is attended
    const bool is_new = r >= a.q_len;
    const int j = r - a.q_len;
    gcu16* kb = is_new ? fx.k_new + (int64_t)j * kv_row
                       : (gcu16*)a.k_noise + ((int64_t)seq * a.q_len + r) * kv_row + g * kHeadDim;
    gcu16* vb = is_new ? fx.v_new + (int64_t)j * kv_row
                       : (gcu16*)a.v_noise + ((int64_t)seq * a.q_len + r) * kv_row + g * kHeadDim;
    nr.kx = kb[lane];
    nr.ky = kb[lane + 64];
    nr.vx = vb[lane];
    nr.vy = vb[lane + 64];
    nr.cs = make_double2(0.0, 0.0);
    // the noise block is visible to every query, or causal in a sliding-
    // window layer; a new row (a committed position) is visible when it lies
    // in the layer's window [lo, committed)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      nr.mask[mb] = is_new ? (fx.start + j >= fx.lo ? 0x0000u : 0xFC00u)
                           : ((fx.swa && (unsigned)r > qrow[mb]) ? 0xFC00u : 0x0000u);
    return;
  } else {
    const int64_t ro = ((int64_t)seq * a.q_len + r) * kv_row + g * kHeadDim;
    nr.kx = a.k_noise[ro + lane];
    nr.ky = a.k_noise[ro + lane + 64];
    nr.vx = a.v_noise[ro + lane];
    nr.vy = a.v_noise[ro + lane + 64];
    nr.cs = *(const double2*)(a.rope_noise + (((int64_t)seq * a.q_len + r) * 64 + lane) * 2);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) nr.mask[mb] = mask_seq[qrow[mb] * a.kv_total + a.cap + r];
  }
}

// Rotate extra row r at its position (fp64, one rounding to F16), store it
// to its ring row (noise row r: row cap + r; new row j: slot (start + j) %
// cap) and stage it in the wave's own LDS row buffer.  It needs neither the
// queries nor the tiles, so a wave does it while its tile is in flight,
// before the work-group's query barrier.
template <int MB, bool FUSED>
__device__ __forceinline__ void stage_extra_row(const AttnArgs& a, const FusedCtx& fx,
                                                const NoiseRow<MB>& nr, int r, uint16_t* kh,
                                                uint16_t* vh, uint16_t* rowk, uint16_t* rowv,
                                                int lane, bool store_row, bool store_slot_pos) {
  double2 cs = nr.cs;
  int slot = a.cap + r;  // ring row of this layer and head
  if constexpr (FUSED) {
    const int j = r - a.q_len;
    int pos = fx.committed + r;
    if (j >= 0) {
      pos = fx.start + j;
      slot = fx.start_mod + j;
      if (slot >= fx.cap) slot -= fx.cap;
    }
    sincos_angle((double)pos * fx.invf, &cs.y, &cs.x);
  }
  double xr, yr;
  rot_pair(f16_to_f64(nr.kx), f16_to_f64(nr.ky), cs.x, cs.y, xr, yr);
  const uint16_t kx = f64_to_f16_rne(xr), ky = f64_to_f16_rne(yr);
  if constexpr (FUSED) {
    // a new row's slot now holds its position (the tile pass of this launch
    // hides the new slots whatever slot_pos says)
    if (store_slot_pos && r >= a.q_len && lane == 0) fx.slot_pos[slot] = fx.start + (r - a.q_len);
  }
  if (store_row) {
    uint16_t* kt = kh + (int64_t)(slot >> 5) * kTileHalves;
    uint16_t* vt = vh + (int64_t)(slot >> 5) * kTileHalves;
    kt[k_frag_index(slot & 31, lane)] = kx;
    kt[k_frag_index(slot & 31, lane + 64)] = ky;
    vt[v_frag_index(slot & 31, lane)] = nr.vx;
    vt[v_frag_index(slot & 31, lane + 64)] = nr.vy;
  }
  // the row in LDS, private to this wave
  rowk[lane] = kx;
  rowk[lane + 64] = ky;
  rowv[lane] = nr.vx;
  rowv[lane + 64] = nr.vy;
}

// Fold the staged extra row into the wave's running softmax as one more
// key.  S = Q k on the vector unit (dot products of the hi and lo query
// fragments with the F16 key); the P V update is one matrix op per 32-dim
// block with the row as slot 0 of a V fragment.
template <int MB, bool QL>
__device__ __forceinline__ void attend_extra_row(const NoiseRow<MB>& nr, const uint16_t* rowk,
                                                 const uint16_t* rowv, int lane, int hl, int col,
                                                 const QFrag<MB, QL>& q, const half8* q_lds,
                                                 float (&m_run)[MB], float (&l_run)[MB],
                                                 f32x16 (&o)[MB][4]) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  typedef _Float16 half2v __attribute__((ext_vector_type(2)));
  half8 kd[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) kd[c] = *(const half8*)(rowk + 16 * c + 8 * hl);
  // V fragment with the row at slot 0: lanes 0..31, element 0, dim 32 b + col
  uint16_t vd[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) vd[b] = rowv[32 * b + col];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // four chains keep the unit busy
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      half8 qh, ql;
      if constexpr (QL) {
        qh = q_lds[((mb * 2 + 0) * 8 + c) * 64 + lane];
        ql = q_lds[((mb * 2 + 1) * 8 + c) * 64 + lane];
      } else {
        qh = q.hi[mb][c];
        ql = q.lo[mb][c];
      }
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const half2v kk = {kd[c][e], kd[c][e + 1]};
        acc[e >> 1] = __builtin_amdgcn_fdot2((half2v){qh[e], qh[e + 1]}, kk, acc[e >> 1], false);
        acc[e >> 1] = __builtin_amdgcn_fdot2((half2v){ql[e], ql[e + 1]}, kk, acc[e >> 1], false);
      }
    }
    const float dot = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    const float sc = dot + __shfl_xor(dot, 32) +
                     (float)__builtin_bit_cast(_Float16, nr.mask[mb]);
    const float m_old = m_run[mb];
    const float mnew = fmaxf(m_old, sc);
    float alpha = 1.0f, p = 0.0f;
    if (mnew != kNegInf) {
      alpha = exp2_hw(m_old - mnew);
      p = exp2_hw(sc - mnew);
    }
    l_run[mb] = l_run[mb] * alpha + p;
    m_run[mb] = mnew;
    if (__any(alpha != 1.0f && m_old != kNegInf)) {
#pragma unroll
      for (int b = 0; b < 4; ++b) o[mb][b] *= alpha;
    }
    half8 pb = {};
    pb[0] = hl == 0 ? (_Float16)p : (_Float16)0.0f;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      half8 vf = {};
      vf[0] = hl == 0 ? __builtin_bit_cast(_Float16, vd[b]) : (_Float16)0.0f;
      o[mb][b] = mfma32(vf, pb, o[mb][b]);
    }
  }
}

// Merge of the NW waves of a work-group by reduce-scatter over the four
// 32-dim blocks of O^T, and the store of the result.  Wave W keeps block W and
// hands the other three, unscaled, to their owners through LDS (same fragment
// order, so lane l reads what lane l of the other wave wrote), together with
// its running (max, sum) per query.  After one barrier each lane owns query
// n = 32 mb + col: it forms the work-group's (mx, lt), weighs every wave's
// block by 2^(m - mx) (and by 1 / lt when this is the only split) and stores
// its block of the output or partial: lane (col, hl) holds dims
// 32 W + 8 jj + 4 hl + 0..3 of query 32 mb + col; rows past m are padding.
// A wave-uniform value made opaque to the compiler (it can neither re-load
// nor re-compute it later, so it stays in SGPRs).
__device__ inline uint64_t keep_sgpr(uint64_t v) {
  uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  asm volatile("" : "+s"(lo), "+s"(hi));
  return ((uint64_t)hi << 32) | lo;
}
__device__ inline int keep_sgpr(int v) {
  v = __builtin_amdgcn_readfirstlane(v);
  asm volatile("" : "+s"(v));
  return v;
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Buffer accesses with device-scope coherence on gfx950: cache policy sc1
// (a store writes through to memory, a load is coherent across the XCDs'
// L2 caches); word 3 of a raw gfx9 buffer descriptor, 32-bit data format.
constexpr int kScDevice = 16;
__device__ inline __amdgpu_buffer_rsrc_t dev_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}
typedef __attribute__((address_space(1))) float gfloat;
typedef __attribute__((address_space(1))) f32x2 gf32x2;
typedef __attribute__((address_space(1))) f32x4 gf32x4;
typedef __attribute__((address_space(1))) half4 ghalf4;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// What the store of a work-group's result needs: its output rows (one split)
// or its partial slot, and the query geometry.
struct EpilogueArgs {
  gfloat* out_unit;
  gu16* pacc;
  gfloat* pml;
  bool one_split;
  bool coherent;  // the partial is stored with device-scope coherence for the
                  // in-launch merge (last_arriver_merge)
  int m, group, n_head;
  int row0;  // first query row of this work-group's block(s)
};

template <int MB, int NW, int W, bool SHARE>
__device__ __forceinline__ void merge_store(const EpilogueArgs& a, unsigned char* lds,
                                            float (*sm_m)[MB * 32], float (*sm_l)[MB * 32],
                                            const float (&m_run)[MB], const float (&l_run)[MB],
                                            const f32x16 (&o)[MB][4], int lane, WaveStamps& st) {
  using S = AttnShape<MB, NW, false, SHARE>;
  const int hl = lane >> 5, col = lane & 31;
  // [mb][block][writer][jj][lane]
  float4* xbuf = reinterpret_cast<float4*>(lds + S::kMergeOffset);
  if constexpr (!S::kOwnMergeBytes) lds_barrier();  // every wave is past its loop
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    if (hl == 0) {
      sm_m[W][mb * 32 + col] = m_run[mb];
      sm_l[W][mb * 32 + col] = l_run[mb];
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      if (b == W) continue;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        xbuf[(((mb * 4 + b) * NW + W) * 4 + jj) * 64 + lane] =
            make_float4(o[mb][b][4 * jj], o[mb][b][4 * jj + 1], o[mb][b][4 * jj + 2],
                        o[mb][b][4 * jj + 3]);
    }
  }
  lds_barrier();
  st.at(6);  // the waves' blocks exchanged through LDS
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int nl = mb * 32 + col;   // row within the work-group's block(s)
    const int n = a.row0 + nl;      // query row
    float mw_[NW], lw_[NW];
    float4 blk[NW][4];
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      mw_[w] = sm_m[w][nl];
      lw_[w] = sm_l[w][nl];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        if (w == W)
          blk[w][jj] = make_float4(o[mb][W][4 * jj], o[mb][W][4 * jj + 1], o[mb][W][4 * jj + 2],
                                   o[mb][W][4 * jj + 3]);
        else
          blk[w][jj] = xbuf[(((mb * 4 + W) * NW + w) * 4 + jj) * 64 + lane];
      }
    }
    float mx = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, mw_[w]);
    // A wave that saw no visible key has m = -inf and l = 0.
    float sw[NW], lt = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float e = exp2_hw(mw_[w] - mx);
      sw[w] = mw_[w] == kNegInf ? 0.0f : e;
      lt += sw[w] * lw_[w];
    }
    float4 v[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float4 u = blk[w][jj];
        acc.x += sw[w] * u.x; acc.y += sw[w] * u.y; acc.z += sw[w] * u.z; acc.w += sw[w] * u.w;
      }
      v[jj] = acc;
    }
    if (a.one_split) {
      // lt > 0: the noise rows are visible to every query.
      const float inv = 1.0f / lt;
      if (n < a.m) {
        const unsigned i = n / a.group, hh = n - i * a.group;
        gfloat* dst = a.out_unit + (i * a.n_head + hh) * kHeadDim + 32 * W + 4 * hl;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          *(gf32x4*)(dst + 8 * jj) = f32x4{v[jj].x * inv, v[jj].y * inv, v[jj].z * inv,
                                           v[jj].w * inv};
      }
    } else {
      // partial in fragment order [mb][block][jj][lane], four F16 per lane:
      // the work-group's output normalised by its sum (zeros where no key
      // of this split is visible to the query, lt = 0), and (max, sum) in
      // fp32; each store instruction writes 512 B contiguous.
      const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
      half4 hv[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        hv[jj] = half4{(_Float16)(v[jj].x * inv), (_Float16)(v[jj].y * inv),
                       (_Float16)(v[jj].z * inv), (_Float16)(v[jj].w * inv)};
      if (a.coherent) {
        const __amdgpu_buffer_rsrc_t ra = dev_rsrc((const uint16_t*)a.pacc, MB * 32 * kHeadDim * 2);
        const __amdgpu_buffer_rsrc_t rm = dev_rsrc((const float*)a.pml, MB * 32 * 2 * 4);
        if (W == 0 && hl == 0 && n < a.m)
          __builtin_amdgcn_raw_buffer_store_b64(f32x2{mx, lt}, rm, nl * 8, 0, kScDevice);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, hv[jj]), ra,
                                                (((mb * 4 + W) * 4 + jj) * 64 + lane) * 8, 0,
                                                kScDevice);
      } else {
        if (W == 0 && hl == 0 && n < a.m) *(gf32x2*)(a.pml + nl * 2) = f32x2{mx, lt};
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          *(ghalf4*)(a.pacc + (((mb * 4 + W) * 4 + jj) * 64 + lane) * 4) = hv[jj];
      }
    }
  }
}

// Cross-split merge inside the launch (the kernels whose waves stream
// several tiles, with 2..kInKernelMergeMaxSplits splits): every work-group
// has stored its partial and (max, sum) pairs with device-scope coherence;
// once those stores are complete it draws a ticket from the counter of its
// (sequence x KV head, row block), and the work-group that draws the last
// one resets the counter and merges every split's partial into the output
// as k_ring_merge does: M = max_t m_t, a_t = 2^(m_t - M) l_t, out =
// sum_t a_t o_t / sum_t a_t for the normalised split outputs o_t (a split
// without a visible key has m = -inf, l = 0).  Thread x holds group f =
// 256 i + x of four values of the work-group's partial, i < 4 MB, in its
// fragment order [mb][block][jj][lane]; KB splits' loads are in flight at
// a time and merged online.
template <int MB>
__device__ __forceinline__ void last_arriver_merge(const AttnArgs& a, const EpilogueArgs& ep, int unit,
                                                   int rb) {
  constexpr int MP = MB * 32, NF = 4 * MB, KB = MB == 1 ? 8 : 4;
  __shared__ uint32_t ticket;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's partial stores are done
  __syncthreads();
  uint32_t* cnt = a.tickets + unit * a.n_rb + rb;
  if (threadIdx.x == 0)
    ticket = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  // (the ticket through an SGPR: compared with it, n_split must not be
  // replaced by a value the compiler takes for a per-lane one)
  if (__builtin_amdgcn_readfirstlane(ticket) + 1 != (uint32_t)a.n_split) return;
  if (threadIdx.x == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // split t's partial rows start split_rows * t rows after split 0's;
  // descriptors in SGPRs (the values are wave-uniform)
  const int split_rows = keep_sgpr(MP * a.n_rb);
  const int64_t row00 = (int64_t)unit * a.n_split * split_rows + rb * MP;
  const uint32_t span = (uint32_t)keep_sgpr((a.n_split - 1) * split_rows + MP);
  const __amdgpu_buffer_rsrc_t ra = dev_rsrc(
      (const uint16_t*)keep_sgpr((uint64_t)(a.part_acc + row00 * kHeadDim)), span * kHeadDim * 2);
  const __amdgpu_buffer_rsrc_t rm = dev_rsrc(
      (const float*)keep_sgpr((uint64_t)(a.part_ml + row00 * 2)), span * 2 * 4);
  const int x = threadIdx.x, ln = x & 63, col = ln & 31;
  float M[MB], L[MB];
  f32x4 O[NF];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) { M[mb] = kNegInf; L[mb] = 0.0f; }
#pragma unroll
  for (int i = 0; i < NF; ++i) O[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int tb = 0; tb < a.n_split; tb += KB) {
    f32x2 ml[KB][MB];
    half4 v[KB][NF];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const uint32_t t = (uint32_t)min(tb + u, a.n_split - 1);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        ml[u][mb] = __builtin_amdgcn_raw_buffer_load_b64(
            rm, (t * split_rows + mb * 32 + col) * 8, 0, kScDevice);
#pragma unroll
      for (int i = 0; i < NF; ++i)
        v[u][i] = __builtin_bit_cast(half4, __builtin_amdgcn_raw_buffer_load_b64(
            ra, (t * split_rows * kHeadDim + (i * 256 + x) * 4) * 2, 0, kScDevice));
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      float mx = M[mb];
#pragma unroll
      for (int u = 0; u < KB; ++u)
        if (tb + u < a.n_split) mx = fmaxf(mx, ml[u][mb].x);
      // rescale what the earlier batches summed (nothing yet: M = -inf)
      const float so = M[mb] == kNegInf ? 0.0f : exp2_hw(M[mb] - mx);
      L[mb] *= so;
#pragma unroll
      for (int k = 0; k < 4; ++k) O[4 * mb + k] *= so;
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        const float e = exp2_hw(ml[u][mb].x - mx);
        const float w = (tb + u < a.n_split && ml[u][mb].x != kNegInf) ? e * ml[u][mb].y : 0.0f;
        L[mb] += w;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const half4 h = v[u][4 * mb + k];
          O[4 * mb + k] += w * f32x4{(float)h.x, (float)h.y, (float)h.z, (float)h.w};
        }
      }
      M[mb] = mx;
    }
  }
#pragma unroll
  for (int i = 0; i < NF; ++i) {
    const int f = i * 256 + x, mb = i >> 2, b = (f >> 8) & 3, jj = (f >> 6) & 3, hl = ln >> 5;
    const int n = rb * MP + mb * 32 + col;  // query row
    if (n < a.m) {
      // L > 0: the noise rows are visible to every query.
      const float inv = 1.0f / L[mb];
      const unsigned q = quot32(n, a.rcp_group), hh = n - q * a.group;
      gfloat* dst = ep.out_unit + (q * a.n_head + hh) * kHeadDim + 32 * b + 8 * jj + 4 * hl;
      *(gf32x4*)dst = O[i] * inv;
    }
  }
}

// SHORT: every wave attends at most one ring tile.  Then nothing is fetched
// ahead, the query fragments are read from LDS at each use instead of held in
// registers, and the work-group shares its merge bytes with the prologue, so
// that two work-groups fit one CU.
template <int MB, int NW, int RP, bool FUSED, bool SHORT>
__device__ __forceinline__ void attn_body(const AttnArgs& a, const FusedAttnArgs* fa,
                                          const FusedLane& fl, double theta_lane, int unit,
                                          int split, int row0, int vis_first, int vis_count,
                                          unsigned char* lds, float (*sm_m)[MB * 32],
                                          float (*sm_l)[MB * 32], WaveStamps& st) {
  constexpr bool QL = MB > 1 || SHORT;
  constexpr bool SHARE = SHORT;
  using S = AttnShape<MB, NW, FUSED, SHARE>;
  constexpr int MP = S::MP, NT = S::NT;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hl = lane >> 5;
  const int col = lane & 31;

  const int seq = quot32(unit, a.rcp_n_head_kv);
  const int g = unit - seq * a.n_head_kv;
  const float* ropeq = a.rope_q + (int64_t)seq * a.q_len * 128;
  const uint16_t* mask_seq = a.mask + (int64_t)seq * a.q_len * a.kv_total;

  // Ring tiles of this split: logical tiles [t0, t1) of the vis_count
  // visible ones; logical tile k is ring tile (vis_first + k) mod ring_tiles.
  const int nvt = vis_count;
  const int per = quot32(nvt + a.n_split - 1, a.rcp_n_split);
  const int t0 = min(nvt, split * per);
  const int t1 = min(nvt, t0 + per);
  // Waves that stream several tiles walk their split's range from a start
  // of its own, a multiple of 4 tiles set by (unit, split): logical tile k
  // is taken as t0 + (k - t0 + rot) mod n, so each wave keeps its number of
  // tiles, while the work-groups' concurrent streams no longer sit at one
  // common offset of every head's K and V (where they contend in the DRAM:
  // a 16-sequence ring read 12 % slower in lockstep).
  int rot = 0;
  if constexpr (!SHORT) {
    const int n = t1 - t0;
    if (n > 0) rot = ((unit * 5 + split * 3) * 4) % n;
  }
  auto ring_tile = [&](int k) {
    int j = k + rot;
    if (j >= t1) j -= t1 - t0;
    const int t = vis_first + j;
    return t >= a.ring_tiles ? t - a.ring_tiles : t;
  };
  uint16_t* kh = a.kring + seq * a.seq_stride + a.layer_offset + g * a.head_stride;
  uint16_t* vh = a.vring + seq * a.seq_stride + a.layer_offset + g * a.head_stride;
  // Fused launch: this sequence's deferred step (new rows of this layer,
  // window) and theta of frequency `lane`.
  FusedCtx fx{};
  if constexpr (FUSED) {
    const int kv_row = a.n_head_kv * kHeadDim;
    fx.k_new = fl.k_new ? (gcu16*)fl.k_new + g * kHeadDim : nullptr;
    fx.v_new = fl.v_new ? (gcu16*)fl.v_new + g * kHeadDim : nullptr;
    fx.slot_pos = fa->slot_pos + (int64_t)seq * fa->slot_stride;
    fx.invf = theta_lane;
    fx.kv_row = kv_row;
    fx.start = fl.start;
    fx.start_mod = fl.start_mod;
    fx.n_new = fl.n_new;
    fx.committed = fl.committed;
    fx.lo = fl.lo;
    fx.cap = a.cap;
    fx.swa = fa->swa_layer;
  }
  // The destinations and the few integers the store needs are computed
  // up front and pass through an empty asm statement that redefines them, so the
  // compiler keeps them in SGPRs instead of re-loading kernel arguments in
  // the epilogue (a scalar memory round trip); stores then go through
  // global-address-space pointers.
  uint64_t out_unit = (uint64_t)(a.out + ((int64_t)seq * a.q_len * a.n_head + g * a.group) * kHeadDim);
  // partial rows [row0, row0 + MP) of the split's n_rb * MP
  const int64_t prow = ((int64_t)unit * a.n_split + split) * (MP * a.n_rb) + row0;
  uint64_t pacc = (uint64_t)(a.part_acc + prow * kHeadDim);  // F16
  uint64_t pml = (uint64_t)(a.part_ml + prow * 2);
  const EpilogueArgs ep{(gfloat*)keep_sgpr(out_unit), (gu16*)keep_sgpr(pacc),
                        (gfloat*)keep_sgpr(pml), keep_sgpr(a.n_split == 1) != 0,
                        !SHORT && keep_sgpr(a.n_split > 1 && a.tickets != nullptr) != 0,
                        keep_sgpr(a.m), keep_sgpr(a.group), keep_sgpr(a.n_head),
                        keep_sgpr(row0)};

  // Noise rows of this wave: r = rank, rank + W, ... with W the waves of the
  // (sequence, head); rank counts from the last wave of the last split, whose
  // tile share is the smallest.
  const int n_waves = a.n_split * NW;
  const int rank = n_waves - 1 - (split * NW + wave);

  // Query row (noise position index) of this lane's query in block mb.
  unsigned qrow[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int n = row0 + mb * 32 + col;
    qrow[mb] = n < a.m ? quot32(n, a.rcp_group) : 0;
  }

  // ---- 1a. loads for the query build: the sequence's (cos, sin) table once
  //      per work-group (q_len * 32 float4, staged through LDS), then per
  //      thread item = (mb, chunk pair c, lane ln) the query halves x = dims
  //      16c + 8h + e and y = the same dims + 64.
  //      RP passes of one float4 per thread cover q_len <= RP * NT / 32; a
  //      pass past the table re-reads its last float4 (one line for the wave).
  //      (Fused launch: the table is computed here from theta, loaded now,
  //      after the other loads are issued.)
  float4 rope_v[RP];
  double2 rope_th[RP];
#pragma unroll
  for (int k = 0; k < RP; ++k) {
    const int o = min((int)threadIdx.x + k * NT, a.q_len * 32 - 1);
    if constexpr (FUSED) {
      const int f0 = (2 * o) & 63;
      rope_th[k] = make_double2(__shfl(theta_lane, f0), __shfl(theta_lane, f0 + 1));
    } else {
      rope_v[k] = ((const float4*)ropeq)[o];
    }
  }
  half8 qx[MB], qy[MB];
  unsigned qfreq[MB];  // float4 index of (cos, sin) of frequency 16c + 8h at query row i
  const uint16_t* qseq = a.q + ((int64_t)seq * a.q_len * a.n_head + g * a.group) * kHeadDim;
#pragma unroll
  for (int k = 0; k < MB; ++k) {
    const int item = threadIdx.x + k * NT;
    const int c = (item >> 6) & 3, ln = item & 63;
    const int n = min(row0 + (item >> 8) * 32 + (ln & 31), a.m - 1), h2 = ln >> 5;
    const unsigned i = quot32(n, a.rcp_group), hh = n - i * a.group;
    const unsigned qo = (i * a.n_head + hh) * kHeadDim + 16 * c + 8 * h2;
    qx[k] = *(const half8*)(qseq + qo);
    qy[k] = *(const half8*)(qseq + qo + 64);
    qfreq[k] = (i * 64 + 16 * c + 8 * h2) / 2;
  }

  // ---- 1b. the wave's first extra key row: noise rows, then (fused
  //      launch) the step's new rows of this layer (a wave without one
  //      loads the last row and ignores it).
  const int n_extra = a.q_len + (FUSED ? fx.n_new : 0);
  NoiseRow<MB> nr;
  load_noise_row<MB, FUSED>(a, fx, seq, g, min(rank, n_extra - 1), mask_seq, qrow, lane, nr);

  // ---- 1c. the wave's first ring tile (a wave without tiles loads its
  //      split's last tile again and ignores it).
  // (Fused launch: the slot_pos of the tile's slots instead of the mask,
  //  spv[jj] = slots 8 jj + 4 (lane / 32) + 0..3.)
  auto load_tile = [&](int tile, half8 (&kc)[8], half8 (&vc)[8], uint32_t (&mw)[MB][8],
                       int4 (&spv)[4]) {
    // K, then the mask words (or slot_pos), then V: loads return in issue
    // order, so S = Q K^T and the softmax can run while V is in flight.
    const half8* kt = (const half8*)(kh + (int64_t)tile * kTileHalves);
    const half8* vt = (const half8*)(vh + (int64_t)tile * kTileHalves);
#pragma unroll
    for (int c = 0; c < 8; ++c) kc[c] = kt[c * 64 + lane];
    if constexpr (FUSED) {
      const int4* sp = (const int4*)(fx.slot_pos + tile * kTile + 4 * hl);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) spv[jj] = sp[2 * jj];
    } else {
      const uint16_t* mt = mask_seq + tile * kTile;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const unsigned mo = qrow[mb] * a.kv_total + 4 * hl;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const uint2 w = *(const uint2*)(mt + mo + 8 * jj);
          mw[mb][2 * jj] = w.x;
          mw[mb][2 * jj + 1] = w.y;
        }
      }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) vc[c] = vt[c * 64 + lane];
  };
  int tile = t0 + wave;
  const int tile_last = max(t1 - 1, 0);
  half8 kc[8], vc[8];
  uint32_t mw[MB][8];
  int4 spv[4];
  load_tile(ring_tile(min(tile, tile_last)), kc, vc, mw, spv);
  st.at(2);  // the first tile's loads issued
  // ---- 2. queries: rotate at committed + i, scale by log2(e)/sqrt(d),
  //      split into hi + lo F16 (fragment order [mb][hi/lo][chunk][lane]);
  //      queries past q_len * group are zero.
  float4* rope_lds = reinterpret_cast<float4*>(lds + S::kRopeOffset);
  if constexpr (FUSED) {
    // (cos, sin) of frequencies f0, f0 + 1 at noise position committed + i,
    // entry o = items 2o, 2o + 1 of [q_len][64], for the query rotation only:
    // the angle reduced modulo a turn in fp64, then the hardware sine and
    // cosine of the fraction (at most about 4e-7 rad in all, the order of
    // the 2^-22 relative precision that the hi + lo F16 split of a query keeps)
#pragma unroll
    for (int k = 0; k < RP; ++k) {
      const int o = min((int)threadIdx.x + k * NT, a.q_len * 32 - 1);
      const double pos = (double)(fx.committed + ((2 * o) >> 6));
      float s0, c0, s1, c1;
      sincos_turns_f32(pos * rope_th[k].x, s0, c0);
      sincos_turns_f32(pos * rope_th[k].y, s1, c1);
      rope_v[k] = make_float4(c0, s0, c1, s1);
    }
  }
  // unconditional: entries past the table hold copies of its last float4
  // and are never read (a conditional store would let the compiler sink the
  // load into the branch and wait for every load in flight there)
#pragma unroll
  for (int k = 0; k < RP; ++k) rope_lds[threadIdx.x + k * NT] = rope_v[k];
  lds_barrier();
  float4 qcs[MB][4];  // (cos, sin) pairs of frequencies 16c + 8h + e, e = 0..7
#pragma unroll
  for (int k = 0; k < MB; ++k)
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) qcs[k][e2] = rope_lds[qfreq[k] + e2];
  half8* q_lds = reinterpret_cast<half8*>(lds);
#pragma unroll
  for (int k = 0; k < MB; ++k) {
    const int item = threadIdx.x + k * NT;
    const int mb = item >> 8, c = (item >> 6) & 3, ln = item & 63;
    const bool valid = row0 + mb * 32 + (ln & 31) < a.m;
    half8 xh, xl, yh, yl;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      float xr[2], yr[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float cs = u ? qcs[k][e >> 1].z : qcs[k][e >> 1].x;
        const float sn = u ? qcs[k][e >> 1].w : qcs[k][e >> 1].y;
        const float x = valid ? (float)qx[k][e + u] : 0.0f;
        const float y = valid ? (float)qy[k][e + u] : 0.0f;
        xr[u] = (x * cs - y * sn) * (float)kQScale;
        yr[u] = (y * cs + x * sn) * (float)kQScale;
      }
      // hi = x rounded toward zero to F16, lo = the rest rounded likewise:
      // hi + lo carries about 22 significant bits of x.
      const auto xhp = __builtin_amdgcn_cvt_pkrtz(xr[0], xr[1]);
      const auto yhp = __builtin_amdgcn_cvt_pkrtz(yr[0], yr[1]);
      const auto xlp = __builtin_amdgcn_cvt_pkrtz(xr[0] - (float)xhp[0], xr[1] - (float)xhp[1]);
      const auto ylp = __builtin_amdgcn_cvt_pkrtz(yr[0] - (float)yhp[0], yr[1] - (float)yhp[1]);
      xh[e] = xhp[0]; xh[e + 1] = xhp[1];
      yh[e] = yhp[0]; yh[e + 1] = yhp[1];
      xl[e] = xlp[0]; xl[e + 1] = xlp[1];
      yl[e] = ylp[0]; yl[e + 1] = ylp[1];
    }
    q_lds[((mb * 2 + 0) * 8 + c) * 64 + ln] = xh;
    q_lds[((mb * 2 + 0) * 8 + c + 4) * 64 + ln] = yh;
    q_lds[((mb * 2 + 1) * 8 + c) * 64 + ln] = xl;
    q_lds[((mb * 2 + 1) * 8 + c + 4) * 64 + ln] = yl;
  }
  // ---- 2b. the wave's first extra key row, rotated, stored and staged
  //      before the barrier (its loads were issued with the queries').
  uint16_t* rowk = reinterpret_cast<uint16_t*>(lds + S::kQBytes) + wave * 2 * kHeadDim;
  uint16_t* rowv = rowk + kHeadDim;
  const bool store_rows = row0 == 0;  // one row block stores the rotated rows
  const bool store_sp = store_rows && g == 0;  // and KV head 0 their slot_pos entries
  if (rank < n_extra)
    stage_extra_row<MB, FUSED>(a, fx, nr, rank, kh, vh, rowk, rowv, lane, store_rows, store_sp);
  lds_barrier();
  st.at(3);  // queries built, the first extra rows staged

  QFrag<MB, QL> qf;
  if constexpr (!QL) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        qf.hi[mb][c] = q_lds[((mb * 2 + 0) * 8 + c) * 64 + lane];
        qf.lo[mb][c] = q_lds[((mb * 2 + 1) * 8 + c) * 64 + lane];
      }
  }

  float m_run[MB], l_run[MB];
  f32x16 o[MB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    m_run[mb] = kNegInf;
    l_run[mb] = 0.0f;
#pragma unroll
    for (int b = 0; b < 4; ++b) o[mb][b] = f32x16{};
  }

  // ---- 3. extra key rows (noise rows, and a fused launch's new rows).
  if (rank < n_extra) {
    attend_extra_row<MB, QL>(nr, rowk, rowv, lane, hl, col, qf, q_lds, m_run, l_run, o);
    for (int r = rank + n_waves; r < n_extra; r += n_waves) {
      load_noise_row<MB, FUSED>(a, fx, seq, g, r, mask_seq, qrow, lane, nr);
      stage_extra_row<MB, FUSED>(a, fx, nr, r, kh, vh, rowk, rowv, lane, store_rows, store_sp);
      attend_extra_row<MB, QL>(nr, rowk, rowv, lane, hl, col, qf, q_lds, m_run, l_run, o);
    }
  }
  st.at(4);  // extra key rows attended

  // Attend ring tile rt with its mask words (plain launch) or with the
  // visibility of its slots from their slot_pos (fused launch).
  auto attend = [&](int rt, const half8 (&kc)[8], const half8 (&vc)[8],
                    const uint32_t (&mw)[MB][8], const int4 (&spv)[4]) {
    const int limit = a.cap - rt * kTile;
    if constexpr (FUSED) {
      const int hi = fx.n_new > 0 ? fx.start : fx.committed;
      const SlotVis vis{spv, (uint32_t)fx.lo, (uint32_t)(hi - fx.lo)};
      attend_tile<MB, QL>(kc, vc, vis, limit, hl, qf, q_lds, lane, m_run, l_run, o);
    } else {
      attend_tile<MB, QL>(kc, vc, MaskWords<MB>{mw}, limit, hl, qf, q_lds, lane, m_run, l_run, o);
    }
  };

  // ---- 4. ring tiles.  One query block: the next tile's loads are issued
  //      before the current tile is processed (two tiles in registers); two
  //      query blocks have no room for that.  (Two tiles ahead, through three
  //      rotating register buffers, measured slower on long waves.)
  constexpr bool kPrefetch = !SHORT;
  if constexpr (kPrefetch) {
    // every tile but the wave's last one: its successor is fetched first
    while (tile + NW < t1) {
      half8 kn[8], vn[8];
      uint32_t mn[MB][8];
      int4 spn[4];
      load_tile(ring_tile(tile + NW), kn, vn, mn, spn);
      attend(ring_tile(tile), kc, vc, mw, spv);
#pragma unroll
      for (int c = 0; c < 8; ++c) { kc[c] = kn[c]; vc[c] = vn[c]; }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < 8; ++j) mw[mb][j] = mn[mb][j];
      if constexpr (FUSED) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) spv[jj] = spn[jj];
      }
      tile += NW;
    }
    if (tile < t1) attend(ring_tile(tile), kc, vc, mw, spv);
  } else if constexpr (SHORT) {
    // at most NW tiles per split: at most one per wave
    if (tile < t1) attend(ring_tile(tile), kc, vc, mw, spv);
  } else {
    while (tile < t1) {
      const int next = tile + NW;
      attend(ring_tile(tile), kc, vc, mw, spv);
      if (next < t1) load_tile(ring_tile(next), kc, vc, mw, spv);
      tile = next;
    }
  }
  st.at(5);  // ring tiles attended

  // ---- 5./6. merge the waves and store: a copy of the code per wave, so
  //      that the wave's own accumulator block is picked at compile time.
  static_assert(NW == 4, "one 32-dim output block per wave");
  if (wave == 0)
    merge_store<MB, NW, 0, SHARE>(ep, lds, sm_m, sm_l, m_run, l_run, o, lane, st);
  else if (wave == 1)
    merge_store<MB, NW, 1, SHARE>(ep, lds, sm_m, sm_l, m_run, l_run, o, lane, st);
  else if (wave == 2)
    merge_store<MB, NW, 2, SHARE>(ep, lds, sm_m, sm_l, m_run, l_run, o, lane, st);
  else
    merge_store<MB, NW, 3, SHARE>(ep, lds, sm_m, sm_l, m_run, l_run, o, lane, st);
  if constexpr (!SHORT) {
    if (ep.coherent) last_arriver_merge<MB>(a, ep, unit, row0 / MP);
  }
}

template <int MB, int NW, int RP, bool FUSED, bool SHORT>
__device__ __forceinline__ void attn_entry(const AttnArgs& a, const FusedAttnArgs* fa) {
  using S = AttnShape<MB, NW, FUSED, SHORT>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[S::kTotalLds];
  __shared__ float sm_m[NW][S::MP];
  __shared__ float sm_l[NW][S::MP];
  WaveStamps st;
  // Work-group -> (sequence, KV head, split).  Work-groups are handed to the
  // eight XCDs round-robin; keep every split of one (sequence, head) on one XCD.
  // Every argument the body reads is fetched here in one batch: left to
  // itself the compiler loads each field where it is first used, and each
  // uniform branch in between then costs a full memory round trip before the
  // first ring load can issue.  vis_first[] and vis_count[] come in as one
  // lane-indexed vector load each and are picked by sequence below.
  const int firstv = a.vis_first[threadIdx.x & 63];
  const int countv = a.vis_count[threadIdx.x & 63];
  FusedLaneVec fv{};
  if constexpr (FUSED) {
    fv = fused_fetch(*fa);
    asm volatile("" ::"v"(fv.k_new), "v"(fv.v_new), "v"(fv.start), "v"(fv.start_mod),
                 "v"(fv.n_new), "v"(fv.committed), "v"(fv.lo), "v"(fv.theta),
                 "s"(fa->slot_pos), "s"(fa->slot_stride), "s"(fa->swa_layer));
  }
  asm volatile("" ::"s"(a.kring), "s"(a.vring), "s"(a.mask), "s"(a.rope_noise), "s"(a.rope_q),
               "s"(a.q),
               "s"(a.k_noise), "s"(a.v_noise), "s"(a.out), "s"(a.part_acc), "s"(a.part_ml),
               "s"(a.seq_stride), "s"(a.layer_offset), "s"(a.head_stride), "s"(a.n_seq),
               "s"(a.n_head), "s"(a.n_head_kv), "s"(a.group), "s"(a.q_len), "s"(a.m),
               "s"(a.cap), "s"(a.kv_total), "s"(a.n_split), "s"(a.n_rb), "s"(a.ring_tiles),
               "s"(a.rcp_per_unit), "s"(a.rcp_n_rb), "s"(a.rcp_n_head_kv), "s"(a.rcp_n_split),
               "s"(a.rcp_group), "v"(firstv), "v"(countv));
  // (the row blocks of one split follow each other, on the same XCD, so
  // that the second read of a tile finds it in that XCD's L2)
  const int n_units = a.n_seq * a.n_head_kv;
  const int per_unit = a.n_split * a.n_rb;
  int unit, r;
  if ((n_units & 7) == 0) {
    const int xcd = blockIdx.x & 7, k = blockIdx.x >> 3;
    const int q = quot32(k, a.rcp_per_unit);
    unit = (q << 3) + xcd;
    r = k - q * per_unit;
  } else {
    unit = quot32(blockIdx.x, a.rcp_per_unit);
    r = blockIdx.x - unit * per_unit;
  }
  const int split = quot32(r, a.rcp_n_rb);
  const int rb = r - split * a.n_rb;
  const int seq = quot32(unit, a.rcp_n_head_kv);
  FusedLane fl{};
  if constexpr (FUSED) fl = fused_pick(fv, seq);
  st.at(1);  // work-group mapped (kernel arguments in registers)
  attn_body<MB, NW, RP, FUSED, SHORT>(a, fa, fl, fv.theta, unit, split, rb * S::MP,
                               __builtin_amdgcn_readlane(firstv, seq),
                               __builtin_amdgcn_readlane(countv, seq), lds, sm_m, sm_l, st);
  st.flush(0, blockIdx.x * NW + (threadIdx.x >> 6));
}

template <int MB, int NW, int RP, bool SHORT>
__global__ __launch_bounds__(NW * 64, SHORT ? 2 : 1) void k_ring_attn(AttnArgs a) {
  attn_entry<MB, NW, RP, false, SHORT>(a, nullptr);
}

// The fused launch: the attention work-groups (same mapping as k_ring_attn),
// which also append the step's new rows of this layer (K rotated at its
// position, V) and write their slot_pos entries.
template <int MB, int NW, int RP, bool SHORT>
__global__ __launch_bounds__(NW * 64, SHORT ? 2 : 1) void k_ring_attn_fused(FusedAttnArgs f) {
  attn_entry<MB, NW, RP, true, SHORT>(f.a, &f);
}

// ---------------------------------------------------------------------------
// Cross-split merge: out = sum_t a_t o_t / sum_t a_t with a_t = l_t
// 2^(m_t - M), M = max_t m_t, for the splits' outputs o_t normalised by their
// sums l_t (stored F16).  The partials are in the attention's fragment order
// [unit][split][mb][block b][jj][lane] of four F16, lane = query col + 32 hl
// holding dims 32 b + 8 jj + 4 hl + 0..3.  One work-group per (unit, mb, b,
// jj): wave w merges splits w, w + 4, ... (each split's four values of a
// lane are one contiguous 512 B row of the wave and the merge is lane-local,
// every load of the wave in flight together), then wave 0 combines the four
// partial merges through LDS and writes the output.
// ---------------------------------------------------------------------------
template <int KMAX>
__global__ __launch_bounds__(256) void k_ring_merge(MergeArgs a) {
  __shared__ float sM[4][64], sL[4][64];
  __shared__ float4 sO[4][64];
  WaveStamps st;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // (unit, item) of this work-group; the items of a unit run on the XCD
  // whose attention work-groups wrote its partials (same mapping), so the
  // partials are read from that XCD's L2
  const int per_unit = (a.mpad / 32) * 16;
  int unit, f;
  if ((a.n_units & 7) == 0) {
    const int xcd = blockIdx.x & 7, k = blockIdx.x >> 3;
    const int q = quot32(k, a.rcp_per_unit);
    unit = (q << 3) + xcd;
    f = k - q * per_unit;
  } else {
    unit = quot32(blockIdx.x, a.rcp_per_unit);
    f = blockIdx.x - unit * per_unit;
  }
  const int mb = f >> 4, b = (f >> 2) & 3, jj = f & 3;
  const int col = lane & 31, hl = lane >> 5;
  const int n = mb * 32 + col;
  const int64_t ml_step = (int64_t)a.mpad * 2, acc_step = (int64_t)a.mpad * kHeadDim;
  const float* ml = a.part_ml + (int64_t)unit * a.n_split * ml_step + n * 2;
  const uint16_t* acc = a.part_acc + (int64_t)unit * a.n_split * acc_step + (f * 64 + lane) * 4;

  float2 mlv[KMAX];
  half4 u[KMAX];
  st.at(1);  // work-group mapped
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    const int t = min(wave + 4 * k, a.n_split - 1);
    mlv[k] = *(const float2*)(ml + t * ml_step);
    u[k] = *(const half4*)(acc + t * acc_step);
  }
  st.at(2);  // partial loads issued
  // Take every load as one batch: the reductions below start from a value
  // that the empty asm statements make depend on every loaded register, so
  // the scheduler cannot interleave them with the loads.
  float mx = kNegInf;
#pragma unroll
  for (int k = 0; k < KMAX; ++k)
    asm volatile("" : "+v"(mx) : "v"(mlv[k].x), "v"(mlv[k].y), "v"(__builtin_bit_cast(u32x2, u[k])));
  st.at(3);  // partials in
#pragma unroll
  for (int k = 0; k < KMAX; ++k)
    if (wave + 4 * k < a.n_split) mx = fmaxf(mx, mlv[k].x);
  // A split that saw no visible key has m = -inf and l = 0.
  float L = 0.0f;
  float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    // a split's output is stored normalised: its weight is 2^(m - mx) l
    const float e = exp2_hw(mlv[k].x - mx);
    const float w = (wave + 4 * k < a.n_split && mlv[k].x != kNegInf) ? e * mlv[k].y : 0.0f;
    L += w;
    O.x += w * (float)u[k].x; O.y += w * (float)u[k].y;
    O.z += w * (float)u[k].z; O.w += w * (float)u[k].w;
  }
  sM[wave][lane] = mx;
  sL[wave][lane] = L;
  sO[wave][lane] = O;
  lds_barrier();
  st.at(4);  // the waves' sums exchanged through LDS
  if (wave != 0) {
    st.flush(1, blockIdx.x * 4 + wave);
    return;
  }
  float M = kNegInf;
#pragma unroll
  for (int w = 0; w < 4; ++w) M = fmaxf(M, sM[w][lane]);
  float Lt = 0.0f;
  float4 Ot = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float mw = sM[w][lane];
    const float e = exp2_hw(mw - M);
    const float s = mw == kNegInf ? 0.0f : e;
    const float4 ow = sO[w][lane];
    Lt += s * sL[w][lane];
    Ot.x += s * ow.x; Ot.y += s * ow.y; Ot.z += s * ow.z; Ot.w += s * ow.w;
  }
  if (n < a.m) {
    // Lt > 0: the noise rows are visible to every query.
    const float inv = 1.0f / Lt;
    Ot.x *= inv; Ot.y *= inv; Ot.z *= inv; Ot.w *= inv;
    const int seq = quot32(unit, a.rcp_n_head_kv), g = unit - seq * a.n_head_kv;
    const int i = quot32(n, a.rcp_group), hh = n - i * a.group;
    float* dst = a.out + (((int64_t)seq * a.q_len + i) * a.n_head + g * a.group + hh) * kHeadDim;
    *(float4*)(dst + 32 * b + 8 * jj + 4 * hl) = Ot;
  }
  st.flush(1, blockIdx.x * 4 + wave);
}

// ---------------------------------------------------------------------------
// Projection of new rows from fused features: raw = W f for W = wk and wv of
// every layer, on the matrix cores, one d-slice per work-group.
//   Work-group (layer, half of head part hp, d-slice ds, 32-row tile rt):
//   hp < n_head_kv is K head hp, else V head hp - n_head_kv; its two waves
//   compute 32 output dims each, [32 pw, 32 pw + 32) with pw = 2 half +
//   wave, for the tile's rows over the slice's 256 feature dims (two-wave
//   work-groups: 1280 at 5 layers of 8 KV heads and d_model 2048, five per
//   compute unit, where 640 of four waves leave half the compute units three
//   and half two; 8.7 against 8.9 us in isolation, within the run-to-run
//   spread in the step).  The slice of the 32 feature rows is
//   staged in LDS by each work-group (rows past n_rows repeat the last row
//   and are never stored).  The sum over d is
//   order-free, so each lane takes 64 contiguous bytes of its W row and of
//   its feature row per 64-d block: MFMA step j of a block pairs, for both
//   operands, dims 64 blk + 32 (lane / 32) + 8 j + e.
// ---------------------------------------------------------------------------
template <bool PACKED>
__global__ __launch_bounds__(128) void k_ring_project(ProjArgs a) {
  constexpr int kRowStride = kProjSlice / 8 + 1;  // half8 per staged row (+1: no bank conflicts)
  __shared__ half8 f_lds[32 * kRowStride];
  WaveStamps st;
  // every argument fetched in one batch at entry (see attn_entry)
  asm volatile("" ::"s"(a.mirror), "s"(a.feat), "s"(a.wk), "s"(a.wv), "s"(a.scratch), "s"(a.slot0),
               "s"(a.n_rows), "s"(a.cap), "s"(a.d_model), "s"(a.kv_row), "s"(a.n_head_kv),
               "s"(a.n_ds), "s"(a.rcp_n_rt), "s"(a.rcp_n_ds), "s"(a.rcp_n_hh));
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_rt = (a.n_rows + 31) >> 5;
  // work-group -> (layer, half head part, d-slice, row tile) by quotients
  // with host-computed reciprocals (no integer division); the two waves of
  // half hh & 1 of head part hh >> 1 compute its output dims
  // 64 (hh & 1) + 32 wave + 0..31
  const uint32_t b0 = blockIdx.x;
  const uint32_t b1 = quot32(b0, a.rcp_n_rt);
  const int rt = (int)(b0 - b1 * n_rt);
  const uint32_t b2 = quot32(b1, a.rcp_n_ds);
  const int ds = (int)(b1 - b2 * a.n_ds);
  const int n_hp = 2 * a.n_head_kv, n_hh = 2 * n_hp;
  const int layer = (int)quot32(b2, a.rcp_n_hh);
  const int hh = (int)(b2 - layer * n_hh);
  const int hp = hh >> 1;
  const int pw = 2 * (hh & 1) + wave;  // the wave's 32 output dims of the head part
  const int r0 = rt * 32;
  const int d0 = ds * kProjSlice;
  st.at(1);  // work-group mapped

  // features of the tile's rows, first (loads return in issue order, and
  // the LDS staging needs them): 32 rows x 32 chunks of 16 B, 8 per thread;
  // row i sits in mirror slot (slot0 + i) % cap (slot0 < cap, i < 64), or,
  // for a deferred mirror write, at row i of a.feat (the source picked
  // without a branch, so that the loads issue together)
  half8 fv[8];
  int fslot[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int c = threadIdx.x + 128 * k;
    const int row = c >> 5, dc = c & 31;
    const int i = min(r0 + row, a.n_rows - 1);
    // slot0 < cap and i < 64: one subtraction unless cap < 64
    int slot = a.slot0 + i;
    if (slot >= a.cap) slot -= a.cap;
    if (slot >= a.cap) slot %= a.cap;
    fslot[k] = slot;
    const uint16_t* src = a.feat ? a.feat + (int64_t)i * a.d_model + d0 + 8 * dc
                                 : a.mirror + (int64_t)slot * a.d_model + d0 + 8 * dc;
    fv[k] = *(const half8*)src;
  }

  // weights: row 32 w + lane % 32 of the head part, 4 blocks x 64 B (dims
  // 64 blk + 32 (lane / 32) + 8 j + e of the slice); packed weights hold the
  // wave's 16 KiB in exactly this load order.  The loads are issued in the
  // order the matrix ops use them (a scheduling barrier after each): loads
  // return in issue order, so each op waits only for its own weights and
  // the chain runs while the later ones arrive (left to itself the compiler
  // issued the first op's weights fifteenth, and the chain waited for all).
  half8 wa[4][4];
  if constexpr (PACKED) {
    const half8* wp = (const half8*)a.wk +
                      ((((int64_t)layer * n_hp + hp) * a.n_ds + ds) * 4 + pw) * 1024;
#pragma unroll
    for (int blk = 0; blk < 4; ++blk)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        wa[blk][j] = wp[(blk * 4 + j) * 64 + lane];
        __builtin_amdgcn_sched_barrier(0);
      }
  } else {
    const bool is_v = hp >= a.n_head_kv;
    const int head = is_v ? hp - a.n_head_kv : hp;
    const uint16_t* wrow = (is_v ? a.wv : a.wk) +
                           ((int64_t)layer * a.kv_row + head * kHeadDim + 32 * pw + (lane & 31)) *
                               a.d_model +
                           d0 + 32 * (lane >> 5);
#pragma unroll
    for (int blk = 0; blk < 4; ++blk)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        wa[blk][j] = *(const half8*)(wrow + blk * 64 + 8 * j);
        __builtin_amdgcn_sched_barrier(0);
      }
  }
  // every weight load is issued before the wait for the features
  __builtin_amdgcn_sched_barrier(0);
  st.at(2);  // feature and weight loads issued
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int c = threadIdx.x + 128 * k;
    f_lds[(c >> 5) * kRowStride + (c & 31)] = fv[k];
  }
  // a deferred mirror write: the work-groups of layer 0, head part 0 (one
  // per d-slice and row tile) store the rows' features into their slots
  if (a.feat && layer == 0 && hh == 0) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int c = threadIdx.x + 128 * k;
      if (r0 + (c >> 5) < a.n_rows)
        *(half8*)(a.mirror_w + (int64_t)fslot[k] * a.d_model + d0 + 8 * (c & 31)) = fv[k];
    }
  }
  lds_barrier();
  st.at(3);  // features staged in LDS

  f32x16 acc = {};
  const half8* frow = f_lds + (lane & 31) * kRowStride + 4 * (lane >> 5);
#pragma unroll
  for (int blk = 0; blk < 4; ++blk)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = mfma32(wa[blk][j], frow[blk * 8 + j], acc);
  st.at(4);  // matrix-core products issued

  // acc[r] = raw[out dim 8 (r / 4) + 4 (lane / 32) + r % 4][row lane % 32]
  const int n = r0 + (lane & 31);
  if (n < a.n_rows) {
    float* dst = a.scratch +
                 (((int64_t)layer * a.n_ds + ds) * kProjRows + n) * 2 * a.kv_row +
                 hp * kHeadDim + 32 * pw + 4 * (lane >> 5);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *(float4*)(dst + 8 * q) = make_float4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2],
                                            acc[4 * q + 3]);
  }
  st.flush(2, blockIdx.x * 2 + wave);
}

// Weights into the projection's load order (PackArgs): one 16-byte chunk
// per thread, read from its row of wk or wv, written contiguously.
__global__ __launch_bounds__(256) void k_ring_pack_weights(PackArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= a.n_chunks) return;
  const int lane = (int)(i & 63);
  int64_t t = i >> 6;
  const int j = (int)(t & 3);
  t >>= 2;
  const int blk = (int)(t & 3);
  t >>= 2;
  const int w = (int)(t & 3);
  t >>= 2;
  const int ds = (int)(t % a.n_ds);
  t /= a.n_ds;
  const int n_hp = 2 * a.n_head_kv;
  const int hp = (int)(t % n_hp);
  const int64_t layer = t / n_hp;
  const bool is_v = hp >= a.n_head_kv;
  const int head = is_v ? hp - a.n_head_kv : hp;
  const int64_t row = layer * a.kv_row + head * kHeadDim + 32 * w + (lane & 31);
  const int64_t col = (int64_t)ds * kProjSlice + 64 * blk + 32 * (lane >> 5) + 8 * j;
  const uint16_t* src = (is_v ? a.wv : a.wk) + row * a.d_model + col;
  *(half8*)(a.packed + i * 8) = *(const half8*)src;
}

__global__ void k_fill_u16(uint16_t* p, uint16_t value, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = value;
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_step(const StepArgs& a, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  const int row_blocks = (a.n_rows + a.n_pad) * a.n_layer;
  const int mask_blocks = a.do_mask ? (a.kv_total + 255) / 256 : 0;
  const int grid = row_blocks + mask_blocks;
  if (grid == 0) return hipSuccess;
  hipExtLaunchKernelGGL(k_ring_step, dim3(grid), dim3(256), 0, s, t0, t1, 0, a);
  return hipGetLastError();
}

hipError_t launch_step_batch(const StepBatchArgs& b, hipStream_t s, hipEvent_t t0,
                             hipEvent_t t1) {
  const int grid = b.n_seq * b.blocks_per_seq;
  if (grid == 0) return hipSuccess;
  hipExtLaunchKernelGGL(k_ring_step_batch, dim3(grid), dim3(256), 0, s, t0, t1, 0, b);
  return hipGetLastError();
}

// The reciprocals of an attention launch's divisors; false if a quotient
// could be inexact (a dividend times its divisor above 2^32).
static bool set_attn_recips(AttnArgs& a) {
  const uint64_t lim = uint64_t(1) << 32;
  const uint64_t per_unit = (uint64_t)a.n_split * a.n_rb;
  const uint64_t grid = (uint64_t)a.n_seq * a.n_head_kv * per_unit;
  if (a.n_split < 1 || a.n_rb < 1 || a.n_head_kv < 1 || a.group < 1 || grid * per_unit > lim ||
      (uint64_t)a.n_seq * a.n_head_kv * a.n_head_kv > lim ||
      (uint64_t)(a.ring_tiles + a.n_split) * a.n_split > lim ||
      (uint64_t)(a.m + 32 * a.n_rb) * a.group > lim)
    return false;
  a.rcp_per_unit = recip32((uint32_t)per_unit);
  a.rcp_n_rb = recip32(a.n_rb);
  a.rcp_n_head_kv = recip32(a.n_head_kv);
  a.rcp_n_split = recip32(a.n_split);
  a.rcp_group = recip32(a.group);
  return true;
}

// Whether every wave of the launch attends at most one ring tile (the widest
// window's tiles over n_split splits of 4 waves).
bool attn_short_waves(const AttnArgs& a) {
  int max_count = 0;
  for (int i = 0; i < a.n_seq && i < RING_MAX_SEQ_INTERNAL; ++i)
    max_count = max_count > a.vis_count[i] ? max_count : a.vis_count[i];
  const int per_split = (max_count + a.n_split - 1) / a.n_split;
  return per_split <= 4;
}

hipError_t launch_attn(const AttnArgs& args, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  AttnArgs a = args;
  if (!set_attn_recips(a)) return hipErrorInvalidValue;
  const int grid = a.n_seq * a.n_head_kv * a.n_split * a.n_rb;
  // rope table passes: one float4 per thread covers q_len <= 8
  const bool one_pass = a.q_len <= 8;
  const bool sw = attn_short_waves(a);
  // one query block per work-group: m <= 32, or one work-group per row block
  if (a.m <= 32 || a.n_rb > 1) {
    if (one_pass && sw)
      hipExtLaunchKernelGGL((k_ring_attn<1, 4, 1, true>), dim3(grid), dim3(256), 0, s, t0, t1, 0, a);
    else if (one_pass)
      hipExtLaunchKernelGGL((k_ring_attn<1, 4, 1, false>), dim3(grid), dim3(256), 0, s, t0, t1, 0, a);
    else if (sw)
      hipExtLaunchKernelGGL((k_ring_attn<1, 4, 4, true>), dim3(grid), dim3(256), 0, s, t0, t1, 0, a);
    else
      hipExtLaunchKernelGGL((k_ring_attn<1, 4, 4, false>), dim3(grid), dim3(256), 0, s, t0, t1, 0, a);
  } else {
    if (one_pass)
      hipExtLaunchKernelGGL((k_ring_attn<2, 4, 1, false>), dim3(grid), dim3(256), 0, s, t0, t1, 0, a);
    else
      hipExtLaunchKernelGGL((k_ring_attn<2, 4, 4, false>), dim3(grid), dim3(256), 0, s, t0, t1, 0, a);
  }
  return hipGetLastError();
}

hipError_t launch_attn_fused(const FusedAttnArgs& args, hipStream_t s, hipEvent_t t0,
                             hipEvent_t t1) {
  FusedAttnArgs f = args;
  if (!set_attn_recips(f.a)) return hipErrorInvalidValue;
  const AttnArgs& a = f.a;
  const int grid = f.n_attn_blocks;
  const bool one_pass = a.q_len <= 8;
  const bool sw = attn_short_waves(a);
  if (a.m <= 32 || a.n_rb > 1) {
    if (one_pass && sw)
      hipExtLaunchKernelGGL((k_ring_attn_fused<1, 4, 1, true>), dim3(grid), dim3(256), 0, s, t0, t1, 0, f);
    else if (one_pass)
      hipExtLaunchKernelGGL((k_ring_attn_fused<1, 4, 1, false>), dim3(grid), dim3(256), 0, s, t0, t1, 0, f);
    else if (sw)
      hipExtLaunchKernelGGL((k_ring_attn_fused<1, 4, 4, true>), dim3(grid), dim3(256), 0, s, t0, t1, 0, f);
    else
      hipExtLaunchKernelGGL((k_ring_attn_fused<1, 4, 4, false>), dim3(grid), dim3(256), 0, s, t0, t1, 0, f);
  } else {
    if (one_pass)
      hipExtLaunchKernelGGL((k_ring_attn_fused<2, 4, 1, false>), dim3(grid), dim3(256), 0, s, t0, t1, 0, f);
    else
      hipExtLaunchKernelGGL((k_ring_attn_fused<2, 4, 4, false>), dim3(grid), dim3(256), 0, s, t0, t1, 0, f);
  }
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& args, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  MergeArgs a = args;
  const uint64_t per_unit = (uint64_t)(a.mpad / 32) * 16;
  if (a.n_head_kv < 1 || a.group < 1 || per_unit < 1 ||
      (uint64_t)a.n_units * per_unit * per_unit > (uint64_t(1) << 32) ||
      (uint64_t)a.n_units * a.n_head_kv > (uint64_t(1) << 32) ||
      (uint64_t)a.mpad * a.group > (uint64_t(1) << 32))
    return hipErrorInvalidValue;
  a.rcp_per_unit = recip32((uint32_t)per_unit);
  a.rcp_n_head_kv = recip32(a.n_head_kv);
  a.rcp_group = recip32(a.group);
  const dim3 grid(a.n_units * (a.mpad / 32) * 16), block(256);
  const int per_wave = (a.n_split + 3) / 4;  // splits per wave (n_split <= 64)
  if (per_wave <= 1) {
    hipExtLaunchKernelGGL(k_ring_merge<1>, grid, block, 0, s, t0, t1, 0, a);
  } else if (per_wave <= 2) {
    hipExtLaunchKernelGGL(k_ring_merge<2>, grid, block, 0, s, t0, t1, 0, a);
  } else if (per_wave <= 4) {
    hipExtLaunchKernelGGL(k_ring_merge<4>, grid, block, 0, s, t0, t1, 0, a);
  } else if (per_wave <= 8) {
    hipExtLaunchKernelGGL(k_ring_merge<8>, grid, block, 0, s, t0, t1, 0, a);
  } else {
    hipExtLaunchKernelGGL(k_ring_merge<16>, grid, block, 0, s, t0, t1, 0, a);
  }
  return hipGetLastError();
}

hipError_t launch_project(const ProjArgs& args, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  if (args.n_rows <= 0) return hipSuccess;
  ProjArgs a = args;
  // work-groups of two waves, one per half head part (1280 for 5 layers
  // of 8 KV heads and 8 slices: five per compute unit)
  const uint32_t n_rt = (a.n_rows + 31) / 32, n_hh = 4 * a.n_head_kv;
  const uint64_t grid = (uint64_t)a.n_layer * n_hh * a.n_ds * n_rt;
  // every quotient exact: dividend times divisor at most 2^32
  if (grid * n_rt > (uint64_t(1) << 32) || grid > (uint64_t(1) << 31)) return hipErrorInvalidValue;
  a.rcp_n_rt = recip32(n_rt);
  a.rcp_n_ds = recip32(a.n_ds);
  a.rcp_n_hh = recip32(n_hh);
  if (a.packed)
    hipExtLaunchKernelGGL(k_ring_project<true>, dim3((unsigned)grid), dim3(128), 0, s, t0, t1, 0, a);
  else
    hipExtLaunchKernelGGL(k_ring_project<false>, dim3((unsigned)grid), dim3(128), 0, s, t0, t1, 0, a);
  return hipGetLastError();
}

hipError_t launch_pack_weights(const PackArgs& a, hipStream_t s) {
  if (a.n_chunks <= 0) return hipSuccess;
  const int64_t grid = (a.n_chunks + 255) / 256;
  hipLaunchKernelGGL(k_ring_pack_weights, dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fill_u16(uint16_t* p, uint16_t value, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t grid = (n + 255) / 256;
  hipLaunchKernelGGL(k_fill_u16, dim3((unsigned)grid), dim3(256), 0, s, p, value, n);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Split partials of ring_attn_noalloc: one array per device, in the code
// object's static data, shared by every call on that device (it keeps the
// last call's contents; nothing in it needs to start at zero, since each call
// writes every partial it reads).  Host code takes its device address from
// hipGetSymbolAddress, resolved once per device at ring_init; the array's
// name itself is a host-side stand-in and is never passed to a kernel.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t resolve_static_scratch(int device) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  if (g_scratch_ptr[device]) return hipSuccess;
  void* ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  g_scratch_ptr[device] = ptr;
  return hipSuccess;
}

void* static_scratch(int device) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return device >= 0 && device < kMaxDevices ? g_scratch_ptr[device] : nullptr;
}

}  // namespace ringkv
