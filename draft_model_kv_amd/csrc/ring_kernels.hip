// ring_kernels.hip -- HIP kernels of the draft-KV ring for gfx950 (MI355X).
//
//   k_ring_step   begin_step: mod-cap append of new K/V rows with RoPE at
//                 their absolute positions (bulk chunk or fixed-shape
//                 fold-in with pad rows to the trash slot), then slot_pos,
//                 the 0/-inf window mask and the noise RoPE table.
//                 Page "DFLASH2_RING_PORT.md", sections 1.1-1.4.
//   k_ring_attn   masked GQA attention of the q_len noise queries over the
//                 ring, split-K over 32-slot ring tiles, matrix-core QK^T and
//                 PV, online softmax, per-workgroup merge of its waves.
//   k_ring_merge  cross-split merge of the partial (max, sum, acc) triples.
#include "ring_kernels.h"

#include <math.h>

namespace ringkv {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kNegInf = -__builtin_inff();
// log2(e) / sqrt(128): folds the 1/sqrt(head_dim) score scale and the
// change of base for exp2 into the query.
constexpr double kQScale = 1.4426950408889634074 / 11.313708498984760390;

// ---------------------------------------------------------------------------
// F16 helpers
// ---------------------------------------------------------------------------
__device__ inline double f16_to_f64(uint16_t b) {
  return (double)__builtin_bit_cast(_Float16, b);
}

// binary64 -> binary16, one rounding, round to nearest even (subnormals and
// overflow to infinity included).
__device__ inline uint16_t f64_to_f16_rne(double x) {
  const uint64_t b = __builtin_bit_cast(uint64_t, x);
  const uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  const int exp = (int)((b >> 52) & 0x7FF);
  const uint64_t man = b & ((1ull << 52) - 1);
  if (exp == 0x7FF) return sign | 0x7C00u | (man ? 0x200u : 0u);
  if (exp == 0) return sign;  // binary64 subnormal: far below binary16 range
  const int e = exp - 1023;
  if (e > 15) return sign | 0x7C00u;
  const uint64_t full = man | (1ull << 52);
  const int shift = (e >= -14) ? 42 : 28 - e;
  if (shift > 62) return sign;
  uint64_t q = full >> shift;
  const uint64_t rem = full & ((1ull << shift) - 1);
  const uint64_t halfway = 1ull << (shift - 1);
  if (rem > halfway || (rem == halfway && (q & 1))) ++q;
  if (e >= -14) {
    int he = e + 15;
    if (q == 2048) { q = 1024; ++he; }
    if (he >= 31) return sign | 0x7C00u;
    return sign | (uint16_t)(he << 10) | (uint16_t)(q & 0x3FF);
  }
  return sign | (uint16_t)q;  // subnormal; q == 1024 is the smallest normal
}

// Rotate the pair (x, y) by the angle whose cosine and sine are (c, s); no
// contraction so the products round as written.
__device__ inline void rot_pair(double x, double y, double c, double s,
                                double& xr, double& yr) {
#pragma clang fp contract(off)
  xr = x * c - y * s;
  yr = y * c + x * s;
}

// ---------------------------------------------------------------------------
// begin_step: append + slot_pos + mask + noise RoPE table
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_ring_step(StepArgs a) {
  const int t = threadIdx.x;
  const int rows_per_layer = a.n_rows + a.n_pad;
  const int n_row_blocks = rows_per_layer * a.n_layer;
  const int blk = blockIdx.x;
  const int kv_row = a.n_head_kv * kHeadDim;
  const int64_t head_stride = (int64_t)a.n_tiles * kTileHalves;
  const int64_t layer_stride = head_stride * a.n_head_kv;

  if (blk < n_row_blocks) {
    const int layer = blk / rows_per_layer;
    const int i = blk - layer * rows_per_layer;
    const bool pad = i >= a.n_rows;
    int slot;
    int64_t p = 0;
    const uint16_t* ksrc = nullptr;
    const uint16_t* vsrc = nullptr;
    if (!pad) {
      const int idx = a.row0 + i;
      p = a.start + idx;
      slot = (int)(p % a.cap);
      ksrc = a.k_new + ((int64_t)layer * a.n_new + idx) * kv_row;
      vsrc = a.v_new + ((int64_t)layer * a.n_new + idx) * kv_row;
    } else {
      slot = a.trash_slot;
    }
    const int s_t = slot & (kTile - 1);
    const int64_t tile_off = (int64_t)(slot >> 5) * kTileHalves;
    uint16_t* kl = a.kring + layer * layer_stride + tile_off;
    uint16_t* vl = a.vring + layer * layer_stride + tile_off;
    // item = (head, two neighbouring rotation pairs)
    for (int item = t; item < a.n_head_kv * 32; item += 256) {
      const int h = item >> 5;
      const int f0 = (item & 31) * 2;
      uint16_t* kd = kl + h * head_stride;
      uint16_t* vd = vl + h * head_stride;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int f = f0 + u;
        if (pad) {
          kd[k_frag_index(s_t, f)] = 0;
          kd[k_frag_index(s_t, f + 64)] = 0;
          vd[v_frag_index(s_t, f)] = 0;
          vd[v_frag_index(s_t, f + 64)] = 0;
        } else {
          const double x = f16_to_f64(ksrc[h * kHeadDim + f]);
          const double y = f16_to_f64(ksrc[h * kHeadDim + f + 64]);
          double sn, cs;
          sincos((double)p * a.inv_freq[f], &sn, &cs);
          double xr, yr;
          rot_pair(x, y, cs, sn, xr, yr);
          kd[k_frag_index(s_t, f)] = f64_to_f16_rne(xr);
          kd[k_frag_index(s_t, f + 64)] = f64_to_f16_rne(yr);
          vd[v_frag_index(s_t, f)] = vsrc[h * kHeadDim + f];
          vd[v_frag_index(s_t, f + 64)] = vsrc[h * kHeadDim + f + 64];
        }
      }
    }
    return;
  }
  if (!a.do_mask) return;

  const int mblk = blk - n_row_blocks;
  if (mblk == 0) {
    // cos / sin of the noise positions committed + i, for every frequency.
    for (int item = t; item < a.q_len * 64; item += 256) {
      const int i = item >> 6, f = item & 63;
      double sn, cs;
      sincos((double)(a.committed + i) * a.inv_freq[f], &sn, &cs);
      a.rope_noise[2 * item] = cs;
      a.rope_noise[2 * item + 1] = sn;
    }
  }
  const int s = mblk * 256 + t;
  if (s >= a.kv_total) return;
  bool vis;
  if (s < a.cap) {
    int64_t sp = a.slot_pos[s];
    const int64_t d = ((int64_t)s - a.start % a.cap + a.cap) % a.cap;
    if (d < a.n_new) {
      sp = a.start + d;
      a.slot_pos[s] = (int32_t)sp;
    }
    vis = sp >= a.lo && sp < a.committed;
  } else {
    vis = s < a.cap + a.q_len;  // noise slots: visible to every noise row
  }
  const uint16_t mv = vis ? 0x0000u : 0xFC00u;
  for (int i = 0; i < a.q_len; ++i) a.mask[(int64_t)i * a.kv_total + s] = mv;
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
// Kept in registers for one query block, read from LDS for two.
template <int MB>
struct QFrag {
  static constexpr bool kLds = MB > 1;
  half8 hi[kLds ? 1 : MB][kLds ? 1 : 8];
  half8 lo[kLds ? 1 : MB][kLds ? 1 : 8];
};

// One 32-slot tile: S^T = K Q^T (Q as hi + lo F16), additive mask, online
// softmax, O^T += V^T P^T.
//   kc, vc   K and V chunks (fragment order, see ring_layout.h)
//   mw       mask of accumulator rows j = 4 jj + u, two F16 per word:
//            mw[mb][2 jj + (u >> 1)], low half for even u
//   limit    rows r >= limit of this tile are hidden (-inf)
template <int MB>
__device__ inline void attend_tile(const half8 (&kc)[8], const half8 (&vc)[8],
                                   const uint32_t (&mw)[MB][8], int limit, int hl,
                                   const QFrag<MB>& q, const half8* q_lds, int lane,
                                   float (&m_run)[MB], float (&l_run)[MB],
                                   f32x16 (&o)[MB][4]) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    f32x16 s = {};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      half8 qh, ql;
      if constexpr (QFrag<MB>::kLds) {
        qh = q_lds[((mb * 2 + 0) * 8 + c) * 64 + lane];
        ql = q_lds[((mb * 2 + 1) * 8 + c) * 64 + lane];
      } else {
        qh = q.hi[mb][c];
        ql = q.lo[mb][c];
      }
      s = mfma32(kc[c], qh, s);
      s = mfma32(kc[c], ql, s);
    }
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t w = mw[mb][2 * (j >> 2) + ((j & 3) >> 1)];
      float b = (j & 1) ? f16_hi(w) : f16_lo(w);
      const int r = 8 * (j >> 2) + 4 * hl + (j & 3);
      if (r >= limit) b = kNegInf;
      s[j] += b;
      mx = fmaxf(mx, s[j]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(m_run[mb], mx);
    float alpha = 1.0f;
    float ls = 0.0f;
    if (mnew == kNegInf) {
#pragma unroll
      for (int j = 0; j < 16; ++j) s[j] = 0.0f;
    } else {
      alpha = exp2f(m_run[mb] - mnew);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        s[j] = exp2f(s[j] - mnew);
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
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      o[mb][b] *= alpha;
      o[mb][b] = mfma32(vc[2 * b], pb0, o[mb][b]);
      o[mb][b] = mfma32(vc[2 * b + 1], pb1, o[mb][b]);
    }
  }
}

template <int MB, int NW>
__global__ __launch_bounds__(NW * 64) void k_ring_attn(AttnArgs a) {
  constexpr int MP = MB * 32;
  constexpr int OS = 132;  // LDS row stride (floats) of the merged output
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int hl = lane >> 5;
  const int col = lane & 31;

  // Work-group -> (sequence, KV head, split).  Work-groups are handed to the
  // eight XCDs round-robin; keep every split of one (sequence, head) on one XCD.
  const int n_units = a.n_seq * a.n_head_kv;
  int unit, split;
  if ((n_units & 7) == 0) {
    const int xcd = blockIdx.x & 7, k = blockIdx.x >> 3;
    unit = ((k / a.n_split) << 3) + xcd;
    split = k % a.n_split;
  } else {
    unit = blockIdx.x / a.n_split;
    split = blockIdx.x % a.n_split;
  }
  const int seq = unit / a.n_head_kv;
  const int g = unit - seq * a.n_head_kv;
  const int kv_row = a.n_head_kv * kHeadDim;
  const double* rope = a.rope_noise + (int64_t)seq * a.q_len * 128;
  const uint16_t* mask_seq = a.mask + (int64_t)seq * a.q_len * a.kv_total;

  // ---- ring tiles of this split (visible ring slots are [0, win)); start
  //      their loads before anything else.
  const int win = a.win[seq];
  const int nvt = (win + kTile - 1) / kTile;
  const int per = (nvt + a.n_split - 1) / a.n_split;
  const int t0 = min(nvt, split * per);
  const int t1 = min(nvt, t0 + per);
  const uint16_t* kh = a.kring + seq * a.seq_stride + a.layer_offset + g * a.head_stride;
  const uint16_t* vh = a.vring + seq * a.seq_stride + a.layer_offset + g * a.head_stride;

  // Query row (noise position index) of this lane's query in block mb.
  int qrow[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int n = mb * 32 + col;
    qrow[mb] = n < a.m ? n / a.group : 0;
  }

  auto load_tile = [&](int tile, half8 (&kc)[8], half8 (&vc)[8], uint32_t (&mw)[MB][8]) {
    const half8* kt = (const half8*)(kh + (int64_t)tile * kTileHalves);
    const half8* vt = (const half8*)(vh + (int64_t)tile * kTileHalves);
#pragma unroll
    for (int c = 0; c < 8; ++c) kc[c] = kt[c * 64 + lane];
#pragma unroll
    for (int c = 0; c < 8; ++c) vc[c] = vt[c * 64 + lane];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const uint16_t* mr = mask_seq + (int64_t)qrow[mb] * a.kv_total + tile * kTile + 4 * hl;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const uint2 w = *(const uint2*)(mr + 8 * jj);
        mw[mb][2 * jj] = w.x;
        mw[mb][2 * jj + 1] = w.y;
      }
    }
  };

  int tile = t0 + wave;
  half8 kc[8], vc[8];
  uint32_t mw[MB][8];
  if (tile < t1) load_tile(tile, kc, vc, mw);

  // ---- queries of this KV head's group, rotated at committed + i, scaled by
  //      log2(e)/sqrt(head_dim), split into hi + lo F16; built once per
  //      work-group in LDS (fragment order: [mb][hi/lo][chunk][lane]).
  __shared__ half8 q_lds[MB * 2 * 8 * 64];
  for (int item = threadIdx.x; item < MB * 4 * 64; item += NW * 64) {
    const int mb = item / 256, c = (item >> 6) & 3, ln = item & 63;
    const int n = mb * 32 + (ln & 31), h2 = ln >> 5;
    const bool valid = n < a.m;
    const int i = valid ? n / a.group : 0;
    const int hh = valid ? n - i * a.group : 0;
    const uint16_t* qp =
        a.q + (((int64_t)seq * a.q_len + i) * a.n_head + g * a.group + hh) * kHeadDim;
    half8 x = half8{}, y = half8{};
    if (valid) {
      x = *(const half8*)(qp + 16 * c + 8 * h2);
      y = *(const half8*)(qp + 16 * (c + 4) + 8 * h2);
    }
    half8 xh, xl, yh, yl;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int f = 16 * c + 8 * h2 + e;
      const double cs = rope[(i * 64 + f) * 2], sn = rope[(i * 64 + f) * 2 + 1];
      double xr, yr;
      rot_pair((double)x[e], (double)y[e], cs, sn, xr, yr);
      xr *= kQScale;
      yr *= kQScale;
      xh[e] = (_Float16)(float)xr;
      yh[e] = (_Float16)(float)yr;
      xl[e] = (_Float16)(float)(xr - (double)xh[e]);
      yl[e] = (_Float16)(float)(yr - (double)yh[e]);
    }
    q_lds[((mb * 2 + 0) * 8 + c) * 64 + ln] = xh;
    q_lds[((mb * 2 + 0) * 8 + c + 4) * 64 + ln] = yh;
    q_lds[((mb * 2 + 1) * 8 + c) * 64 + ln] = xl;
    q_lds[((mb * 2 + 1) * 8 + c + 4) * 64 + ln] = yl;
  }
  __syncthreads();
  QFrag<MB> qf;
  if constexpr (!QFrag<MB>::kLds) {
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

  // One query block: the next tile's loads are issued before the current
  // tile is processed (two tiles in registers).  Two query blocks have no
  // room for that; their next load follows the current tile.
  constexpr bool kPrefetch = MB == 1;
  while (tile < t1) {
    const int next = tile + NW;
    if constexpr (kPrefetch) {
      half8 kn[8], vn[8];
      uint32_t mn[MB][8];
      if (next < t1) load_tile(next, kn, vn, mn);
      attend_tile<MB>(kc, vc, mw, a.cap - tile * kTile, hl, qf, q_lds, lane, m_run, l_run, o);
      if (next < t1) {
#pragma unroll
        for (int c = 0; c < 8; ++c) { kc[c] = kn[c]; vc[c] = vn[c]; }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int j = 0; j < 8; ++j) mw[mb][j] = mn[mb][j];
      }
    } else {
      attend_tile<MB>(kc, vc, mw, a.cap - tile * kTile, hl, qf, q_lds, lane, m_run, l_run, o);
      if (next < t1) load_tile(next, kc, vc, mw);
    }
    tile = next;
  }

  // ---- noise block: rows r < q_len of k_noise / v_noise at committed + r,
  //      visible to every query (split 0, the wave with the fewest tiles).
  if (split == 0 && wave == (t1 - t0) % NW) {
    const uint16_t* knb = a.k_noise + (int64_t)seq * a.q_len * kv_row + g * kHeadDim;
    const uint16_t* vnb = a.v_noise + (int64_t)seq * a.q_len * kv_row + g * kHeadDim;
    const bool rv = col < a.q_len;
    const int r = rv ? col : 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      half8 x = half8{}, y = half8{};
      if (rv) {
        x = *(const half8*)(knb + (int64_t)r * kv_row + 16 * c + 8 * hl);
        y = *(const half8*)(knb + (int64_t)r * kv_row + 16 * (c + 4) + 8 * hl);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int f = 16 * c + 8 * hl + e;
        const double cs = rope[(r * 64 + f) * 2], sn = rope[(r * 64 + f) * 2 + 1];
        double xr, yr;
        rot_pair((double)x[e], (double)y[e], cs, sn, xr, yr);
        kc[c][e] = __builtin_bit_cast(_Float16, f64_to_f16_rne(xr));
        kc[c + 4][e] = __builtin_bit_cast(_Float16, f64_to_f16_rne(yr));
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int b = j >> 1, ks = j & 1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int slot = 16 * ks + 8 * (e >> 2) + 4 * hl + (e & 3);
        vc[j][e] = slot < a.q_len
                       ? __builtin_bit_cast(_Float16, vnb[(int64_t)slot * kv_row + 32 * b + col])
                       : (_Float16)0.0f;
      }
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const uint16_t* mr = mask_seq + (int64_t)qrow[mb] * a.kv_total + a.cap;
#pragma unroll
      for (int w2 = 0; w2 < 8; ++w2) {
        const int r0 = 8 * (w2 >> 1) + 4 * hl + 2 * (w2 & 1);
        const uint32_t lo = r0 < a.q_len ? mr[r0] : 0xFC00u;
        const uint32_t hi = r0 + 1 < a.q_len ? mr[r0 + 1] : 0xFC00u;
        mw[mb][w2] = lo | (hi << 16);
      }
    }
    attend_tile<MB>(kc, vc, mw, a.q_len, hl, qf, q_lds, lane, m_run, l_run, o);

    // Rotated noise rows into ring rows cap + r of this layer.
    uint16_t* khw = a.kring + seq * a.seq_stride + a.layer_offset + g * a.head_stride;
    uint16_t* vhw = a.vring + seq * a.seq_stride + a.layer_offset + g * a.head_stride;
    if (rv) {
      const int slot = a.cap + col;
      uint16_t* kt = khw + (int64_t)(slot >> 5) * kTileHalves;
#pragma unroll
      for (int c = 0; c < 8; ++c)
        *(half8*)(kt + k_frag_index(slot & 31, 16 * c + 8 * hl)) = kc[c];
    }
    for (int rr = 0; rr < a.q_len; ++rr) {
      const int slot = a.cap + rr;
      uint16_t* vt = vhw + (int64_t)(slot >> 5) * kTileHalves;
      vt[v_frag_index(slot & 31, lane)] = vnb[(int64_t)rr * kv_row + lane];
      vt[v_frag_index(slot & 31, lane + 64)] = vnb[(int64_t)rr * kv_row + lane + 64];
    }
  }

  // ---- merge the waves of this work-group through LDS (fixed wave order).
  __shared__ float sm_m[NW][MP];
  __shared__ float sm_l[NW][MP];
  __shared__ float sm_ml[MP][2];
  __shared__ float sm_o[MP * OS];
  if (hl == 0) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      sm_m[wave][mb * 32 + col] = m_run[mb];
      sm_l[wave][mb * 32 + col] = l_run[mb];
    }
  }
  __syncthreads();
  float scale[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int n = mb * 32 + col;
    float mx = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, sm_m[w][n]);
    float lt = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w)
      lt += sm_m[w][n] == kNegInf ? 0.0f : sm_l[w][n] * exp2f(sm_m[w][n] - mx);
    scale[mb] = m_run[mb] == kNegInf ? 0.0f : exp2f(m_run[mb] - mx);
    if (wave == 0 && hl == 0) {
      sm_ml[n][0] = mx;
      sm_ml[n][1] = lt;
    }
  }
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    if (wave == w) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int n = mb * 32 + col;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            float4* dst = (float4*)&sm_o[n * OS + 32 * b + 8 * jj + 4 * hl];
            float4 v = make_float4(o[mb][b][4 * jj] * scale[mb], o[mb][b][4 * jj + 1] * scale[mb],
                                   o[mb][b][4 * jj + 2] * scale[mb], o[mb][b][4 * jj + 3] * scale[mb]);
            if (w != 0) {
              const float4 u = *dst;
              v.x += u.x; v.y += u.y; v.z += u.z; v.w += u.w;
            }
            *dst = v;
          }
        }
      }
    }
    __syncthreads();
  }

  // ---- write the final output (one split) or this split's partial.
  for (int item = threadIdx.x; item < a.m * 32; item += NW * 64) {
    const int n = item >> 5, d4 = item & 31;
    float4 v = *(const float4*)&sm_o[n * OS + 4 * d4];
    if (a.n_split == 1) {
      const float inv = 1.0f / sm_ml[n][1];
      v.x *= inv; v.y *= inv; v.z *= inv; v.w *= inv;
      const int i = n / a.group, hh = n - i * a.group;
      float* dst = a.out + (((int64_t)seq * a.q_len + i) * a.n_head + g * a.group + hh) * kHeadDim;
      *(float4*)(dst + 4 * d4) = v;
    } else {
      const int64_t pbase = ((int64_t)unit * a.n_split + split) * MP + n;
      *(float4*)(a.part_acc + pbase * kHeadDim + 4 * d4) = v;
      if (d4 == 0) {
        a.part_ml[pbase * 2] = sm_ml[n][0];
        a.part_ml[pbase * 2 + 1] = sm_ml[n][1];
      }
    }
  }
}
// ---------------------------------------------------------------------------
// Cross-split merge: out = sum_t acc_t 2^(m_t - M) / sum_t l_t 2^(m_t - M).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_ring_merge(MergeArgs a) {
  const int64_t item = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)a.n_units * a.m * 32;
  if (item >= total) return;
  const int d4 = (int)(item & 31);
  const int64_t un = item >> 5;
  const int n = (int)(un % a.m);
  const int unit = (int)(un / a.m);
  const float* ml = a.part_ml + ((int64_t)unit * a.n_split * a.mpad + n) * 2;
  const float* acc = a.part_acc + ((int64_t)unit * a.n_split * a.mpad + n) * kHeadDim + 4 * d4;
  float mx = kNegInf;
  for (int t = 0; t < a.n_split; ++t) mx = fmaxf(mx, ml[(int64_t)t * a.mpad * 2]);
  float lt = 0.0f;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int t = 0; t < a.n_split; ++t) {
    const float mt = ml[(int64_t)t * a.mpad * 2];
    if (mt == kNegInf) continue;
    const float w = exp2f(mt - mx);
    lt += ml[(int64_t)t * a.mpad * 2 + 1] * w;
    const float4 u = *(const float4*)(acc + (int64_t)t * a.mpad * kHeadDim);
    v.x += w * u.x; v.y += w * u.y; v.z += w * u.z; v.w += w * u.w;
  }
  const float inv = 1.0f / lt;
  v.x *= inv; v.y *= inv; v.z *= inv; v.w *= inv;
  const int seq = unit / a.n_head_kv, g = unit - seq * a.n_head_kv;
  const int i = n / a.group, hh = n - i * a.group;
  float* dst = a.out + (((int64_t)seq * a.q_len + i) * a.n_head + g * a.group + hh) * kHeadDim;
  *(float4*)(dst + 4 * d4) = v;
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

hipError_t launch_attn(const AttnArgs& a, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  const int grid = a.n_seq * a.n_head_kv * a.n_split;
  if (a.m <= 32) {
    hipExtLaunchKernelGGL((k_ring_attn<1, 4>), dim3(grid), dim3(256), 0, s, t0, t1, 0, a);
  } else {
    hipExtLaunchKernelGGL((k_ring_attn<2, 4>), dim3(grid), dim3(256), 0, s, t0, t1, 0, a);
  }
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  const int64_t total = (int64_t)a.n_units * a.m * 32;
  const int grid = (int)((total + 255) / 256);
  hipExtLaunchKernelGGL(k_ring_merge, dim3(grid), dim3(256), 0, s, t0, t1, 0, a);
  return hipGetLastError();
}

hipError_t launch_fill_u16(uint16_t* p, uint16_t value, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t grid = (n + 255) / 256;
  hipLaunchKernelGGL(k_fill_u16, dim3((unsigned)grid), dim3(256), 0, s, p, value, n);
  return hipGetLastError();
}

}  // namespace ringkv
