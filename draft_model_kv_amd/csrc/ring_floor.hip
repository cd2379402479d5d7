// ring_floor.hip -- profiling-only kernels that measure what bounds the
// attention launch of a ring (ring_profile_floor in include/ring_kv.h).
//
// Each one runs on the attention's own grid: one work-group of four waves per
// (sequence, KV head, split, row block), the same XCD-pinned work-group order
// and the same tiles per wave (tile t0 + wave, t0 + wave + 4, ... of the
// ring's visible window, the walk started at the attention's offset per
// unit and split), but with a trivial consumer instead of the softmax:
//   kind 0  empty kernel (launch and drain only)
//   kind 1  every visible K and V tile loaded once (16-byte loads per lane,
//           the attention's fragment order and tile walk) and folded by xor;
//           with FloorArgs.rotate = 0 (the host's lockstep kind) every
//           work-group walks its split's tiles from the first one
//   kind 2  kind 1, then the work-group's 8 KiB F16 split partial and its
//           fp32 (max, sum) pairs stored where the attention stores them
//   kind 3  kind 2 with an in-kernel cross-split merge by the last arriver:
//           partials stored with device-scope coherence (sc1, write-through),
//           the stores waited for, one atomic ticket per work-group on a
//           counter per (sequence, head, row block); the work-group that
//           draws the last ticket loads every split's partial (sc1, eight
//           splits' loads in flight at a time) and writes their sum
//   kind 4  kind 2 with a bounded barrier instead: every work-group of a
//           (sequence, head, row block) waits for all its splits' tickets
//           (at most 2^20 polls with s_sleep, then an error count), then
//           sums its 1/n_split slice of every split's partial (loads
//           batched as in kind 3)
//   kind 5  (host side) kind 2, then the ring's own merge launch over those
//           partials
//   kind 7  kind 1 plus, per tile, the attention's matrix-core contractions
//           on the loaded K and V fragments: 16 v_mfma_f32_32x32x16_f16 for
//           S^T = K Q^T with Q as hi + lo F16, 8 for O^T += V^T P^T (query
//           fragments are stand-ins; the products are what is timed)
//   kind 8  kind 1 plus the same 393,216 products per tile and wave on the
//           vector unit (v_dot2_f32_f16), for the matrix-core A/B
//   kind 9  the projection launch of a decode step instead (one 32-row tile):
//           its grid of two-wave work-groups, each wave loading its 16 KiB of
//           the packed weights as the projection does (16 loads of 1 KiB),
//           folded by xor
//   kind 6  one wave that sleeps for several milliseconds (a bounded loop of
//           s_sleep): the host queues a batch of launches behind it, so that
//           their back-to-back time on the device is not bounded by how fast
//           the host submits them
// The merges sum partials without the softmax weights: these kernels time
// data movement and synchronisation, not the attention's arithmetic.
#include "ring_kernels.h"

namespace ringkv {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ inline f32x16 floor_mfma(half8 a, half8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Cache-policy bits of the buffer instructions on gfx950: sc1 = device scope
// (stores write through to memory, loads are coherent across the XCDs' L2s).
constexpr int kPolicySc1 = 16;
// Word 3 of a raw buffer descriptor on gfx9 parts (32-bit data format).
constexpr int kBufferWord3 = 0x00020000;

__device__ inline __amdgpu_buffer_rsrc_t floor_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, kBufferWord3);
}

template <int KIND>
__global__ __launch_bounds__(256) void k_ring_floor(FloorArgs a) {
  if constexpr (KIND == 0) {
    return;
  } else {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
    const int g = unit - seq * a.n_head_kv;
    const int nvt = a.vis_count[seq];
    const int first = a.vis_first[seq];
    const int per = quot32(nvt + a.n_split - 1, a.rcp_n_split);
    const int t0 = min(nvt, split * per);
    const int t1 = min(nvt, t0 + per);
    const uint16_t* kh = a.kring + seq * a.seq_stride + a.layer_offset + g * a.head_stride;
    const uint16_t* vh = a.vring + seq * a.seq_stride + a.layer_offset + g * a.head_stride;
    u32x4 x = {0u, 0u, 0u, 0u};
    // kinds 7 and 8: the attention's tile contractions on the loaded tiles,
    // with the query fragments stand-ins built from the lane index
    f32x16 acc[4] = {};
    float vacc[8] = {};
    half8 qh, ql;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qh[e] = (_Float16)(0.01f * (float)(lane + e));
      ql[e] = (_Float16)(1e-4f * (float)(lane - e));
    }
    // the attention's tile walk: a start of its own per (unit, split) when
    // its waves stream several tiles
    const int n = t1 - t0;
    const int rot = a.rotate && n > 0 ? ((unit * 5 + split * 3) * 4) % n : 0;
    for (int t = t0 + wave; t < t1; t += 4) {
      int j = t + rot;
      if (j >= t1) j -= n;
      int rt = first + j;
      if (rt >= a.ring_tiles) rt -= a.ring_tiles;
      const u32x4* kt = (const u32x4*)(kh + (int64_t)rt * kTileHalves);
      const u32x4* vt = (const u32x4*)(vh + (int64_t)rt * kTileHalves);
      u32x4 kc[8], vc[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) kc[c] = kt[c * 64 + lane];
#pragma unroll
      for (int c = 0; c < 8; ++c) vc[c] = vt[c * 64 + lane];
      if constexpr (KIND == 7) {
        // 16 matrix ops for S^T = K Q^T (Q as hi + lo), 8 for O^T += V^T P^T
        f32x16 sacc = {};
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          sacc = floor_mfma(__builtin_bit_cast(half8, kc[c]), qh, sacc);
          sacc = floor_mfma(__builtin_bit_cast(half8, kc[c]), ql, sacc);
        }
        half8 p0, p1;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p0[e] = (_Float16)sacc[e];
          p1[e] = (_Float16)sacc[8 + e];
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          acc[b] = floor_mfma(__builtin_bit_cast(half8, vc[2 * b]), p0, acc[b]);
          acc[b] = floor_mfma(__builtin_bit_cast(half8, vc[2 * b + 1]), p1, acc[b]);
        }
      } else if constexpr (KIND == 8) {
        // the same 393,216 products per wave on the vector unit: for each of
        // the 32 queries, its hi and lo halves against the lane's 64 K
        // halves (2 x 32 v_dot2), and 32 v_dot2 against its 64 V halves
        typedef _Float16 half2v __attribute__((ext_vector_type(2)));
#pragma unroll 4
        for (int n = 0; n < 32; ++n) {
          const half8 qa = qh * (_Float16)(float)n, qb = ql * (_Float16)(float)n;
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const half8 kk = __builtin_bit_cast(half8, kc[c]);
            const half8 vv = __builtin_bit_cast(half8, vc[c]);
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
              const half2v k2 = {kk[e], kk[e + 1]}, v2 = {vv[e], vv[e + 1]};
              vacc[(e >> 1)] = __builtin_amdgcn_fdot2((half2v){qa[e], qa[e + 1]}, k2, vacc[e >> 1], false);
              vacc[4 + (e >> 1)] = __builtin_amdgcn_fdot2((half2v){qb[e], qb[e + 1]}, k2, vacc[4 + (e >> 1)], false);
              vacc[(e >> 1)] = __builtin_amdgcn_fdot2((half2v){qa[e + 1], qb[e]}, v2, vacc[e >> 1], false);
            }
          }
        }
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) x ^= kc[c] ^ vc[c];
      }
    }
    if constexpr (KIND == 7 || KIND == 8) {
      float r = 0.0f;
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int j = 0; j < 16; ++j) r += acc[b][j];
#pragma unroll
      for (int i = 0; i < 8; ++i) r += vacc[i];
      x.x = __builtin_bit_cast(uint32_t, r);
    }
    if constexpr (KIND == 1 || KIND == 7 || KIND == 8) {
      // one word per wave keeps every load live
      uint32_t w = x.x ^ x.y ^ x.z ^ x.w;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) w ^= __shfl_xor(w, off);
      if (lane == 0) a.out[blockIdx.x * 4 + wave] = (float)(w & 0xFFFFu);
      return;
    } else {
      // the split partial: 32 rows x 128 dims F16 where the attention puts
      // the partial of (unit, split, row block), and its fp32 (max, sum) pairs
      const f32x4 v = {(float)(x.x & 0xFFu), (float)(x.y & 0xFFu), (float)(x.z & 0xFFu), 1.0f};
      const int64_t prow = ((int64_t)(unit * a.n_split + split) * a.n_rb + rb) * 32;
      const uint32_t pbytes = (uint32_t)a.part_bytes;
      const __amdgpu_buffer_rsrc_t pr = floor_rsrc(a.part_acc, pbytes);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const half4 h = {(_Float16)(v.x + i), (_Float16)(v.y + i), (_Float16)(v.z + i),
                         (_Float16)(v.w + i)};
        const uint32_t off = (uint32_t)((prow * kHeadDim + (i * 256 + threadIdx.x) * 4) * 2);
        if constexpr (KIND == 2)
          *(half4*)(a.part_acc + prow * kHeadDim + (i * 256 + threadIdx.x) * 4) = h;
        else
          __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, h), pr, off, 0, kPolicySc1);
      }
      if (threadIdx.x < 32) *(float2*)(a.part_ml + (prow + threadIdx.x) * 2) = make_float2(v.x, 1.0f);
      if constexpr (KIND == 2) return;
      // every partial store of the work-group has completed (device scope)
      // before its ticket is drawn
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      __shared__ uint32_t ticket;
      uint32_t* cnt = a.counter + unit * a.n_rb + rb;
      if (threadIdx.x == 0)
        ticket = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      const int64_t base_row = ((int64_t)unit * a.n_split * a.n_rb + rb) * 32;  // split 0
      const int64_t split_f4 = (int64_t)a.n_rb * 32 * kHeadDim / 4;            // between splits
      float* outp = a.out + ((int64_t)unit * a.n_rb + rb) * 32 * kHeadDim;
      // group idx of four values of split t's partial, as fp32 (sc1 load;
      // past the buffer: zero)
      auto load_f4 = [&](int t, int idx) {
        const uint32_t off = (uint32_t)(((base_row * kHeadDim / 4) + t * split_f4 + idx) * 8);
        const half4 h = __builtin_bit_cast(half4, __builtin_amdgcn_raw_buffer_load_b64(pr, off, 0, kPolicySc1));
        return f32x4{(float)h.x, (float)h.y, (float)h.z, (float)h.w};
      };
      // sum over splits t = t_first, t_first + t_step, ... < n_split of float4
      // idx: eight loads in flight at a time, issued before any is added
      auto sum_splits = [&](int t_first, int t_step, int idx) {
        f32x4 o = {};
        for (int tb = t_first; tb < a.n_split; tb += 8 * t_step) {
          f32x4 ld[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) ld[u] = load_f4(min(tb + u * t_step, a.n_split - 1), idx);
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (tb + u * t_step < a.n_split) o += ld[u];
        }
        return o;
      };
      if constexpr (KIND == 3) {
        if (ticket + 1 != (uint32_t)a.n_split) return;
        if (threadIdx.x == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // the four float4 of each thread: 32 loads in flight per batch
        f32x4 o[4] = {};
        for (int tb = 0; tb < a.n_split; tb += 8) {
          f32x4 ld[8][4];
#pragma unroll
          for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              ld[u][i] = load_f4(min(tb + u, a.n_split - 1), i * 256 + threadIdx.x);
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (tb + u < a.n_split)
#pragma unroll
              for (int i = 0; i < 4; ++i) o[i] += ld[u][i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) *(f32x4*)(outp + (i * 256 + threadIdx.x) * 4) = o[i];
      } else {
        // KIND 4: every split's ticket is in (tickets count up from
        // epoch * n_split; the counter is never reset), bounded wait
        if (threadIdx.x == 0) {
          const uint32_t target = (a.epoch + 1u) * (uint32_t)a.n_split;
          int n = 0;
          while ((int32_t)(__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) -
                           target) < 0) {
            __builtin_amdgcn_s_sleep(1);
            if (++n > (1 << 20)) {
              __hip_atomic_fetch_add(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              break;
            }
          }
        }
        __syncthreads();
        // slice `split` of the 1024 float4 of a partial
        const int sf = (1024 + a.n_split - 1) / a.n_split;
        __shared__ f32x4 red[256];
        if (sf >= 256) {
          for (int i = threadIdx.x; i < sf; i += 256) {
            const int idx = split * sf + i;
            if (idx >= 1024) break;
            *(f32x4*)(outp + idx * 4) = sum_splits(0, 1, idx);
          }
        } else {
          const int groups = 256 / sf;
          const int grp = threadIdx.x / sf, e = threadIdx.x - grp * sf;
          const int idx = min(split * sf + e, 1023);
          f32x4 o = {};
          if (grp < groups) o = sum_splits(grp, groups, idx);
          red[threadIdx.x] = o;
          __syncthreads();
          if (grp == 0 && split * sf + e < 1024) {
            f32x4 s = red[e];
            for (int j = 1; j < groups; ++j) s += red[j * sf + e];
            *(f32x4*)(outp + idx * 4) = s;
          }
        }
      }
    }
  }
}

// kind 11: one read of every visible tile for both 32-query blocks of a KV
// head.  A work-group of eight waves per (unit, split): wave w = 4 qb + p;
// pair p (waves p and 4 + p) takes the split's tiles t0 + p, t0 + p + 4, ...
// Wave p copies the tile's K and wave 4 + p its V into LDS with direct
// global-to-LDS loads (1 KiB per instruction), two stages; after one barrier
// per tile both waves read K and V from LDS and run the attention's 24
// matrix ops on them (query fragments stand-ins), while the pair's next tile
// is already on its way into the other stage.  Every wave of the
// work-group passes the same number of barriers (the split's largest tile
// count per pair).
__global__ __launch_bounds__(512) void k_ring_floor_pair(FloorArgs a) {
  typedef __attribute__((address_space(3))) void lds_void;
  typedef const __attribute__((address_space(1))) void gvoid;
  __shared__ __attribute__((aligned(16))) u32x4 stage[2][4][2][512];  // 128 KiB
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int p = wave & 3, qb = wave >> 2;
  const int n_units = a.n_seq * a.n_head_kv;
  const int per_unit = a.n_split;
  int unit, split;
  if ((n_units & 7) == 0) {
    const int xcd = blockIdx.x & 7, k = blockIdx.x >> 3;
    const int q = quot32(k, a.rcp_per_unit);
    unit = (q << 3) + xcd;
    split = k - q * per_unit;
  } else {
    unit = quot32(blockIdx.x, a.rcp_per_unit);
    split = blockIdx.x - unit * per_unit;
  }
  const int seq = quot32(unit, a.rcp_n_head_kv);
  const int g = unit - seq * a.n_head_kv;
  const int nvt = a.vis_count[seq];
  const int first = a.vis_first[seq];
  const int per = quot32(nvt + a.n_split - 1, a.rcp_n_split);
  const int t0 = min(nvt, split * per);
  const int t1 = min(nvt, t0 + per);
  const int n = t1 - t0;
  const int rot = a.rotate && n > 0 ? ((unit * 5 + split * 3) * 4) % n : 0;
  const uint16_t* base = (qb == 0 ? a.kring : a.vring) + seq * a.seq_stride + a.layer_offset +
                         g * a.head_stride;
  auto ring_tile = [&](int k) {
    int j = k + rot;
    if (j >= t1) j -= n;
    int rt = first + j;
    return rt >= a.ring_tiles ? rt - a.ring_tiles : rt;
  };
  // this wave's half (K or V) of tile k into stage st
  auto copy_in = [&](int k, int st) {
    const uint16_t* src = base + (int64_t)ring_tile(k) * kTileHalves;
#pragma unroll
    for (int c = 0; c < 8; ++c)
      __builtin_amdgcn_global_load_lds((gvoid*)(src + c * 512 + lane * 8),
                                       (lds_void*)&stage[st][p][qb][c * 64], 16, 0, 0);
  };
  const int trips = (n + 3) >> 2;
  f32x16 acc[4] = {};
  half8 qh, ql;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    qh[e] = (_Float16)(0.01f * (float)(lane + e));
    ql[e] = (_Float16)(1e-4f * (float)(lane - e));
  }
  if (p < n) copy_in(t0 + p, 0);
  for (int i = 0; i < trips; ++i) {
    const int k = t0 + p + 4 * i;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (k + 4 < t1) copy_in(k + 4, (i + 1) & 1);
    if (k < t1) {
      const int st = i & 1;
      half8 kc[8], vc[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        kc[c] = __builtin_bit_cast(half8, stage[st][p][0][c * 64 + lane]);
        vc[c] = __builtin_bit_cast(half8, stage[st][p][1][c * 64 + lane]);
      }
      f32x16 sacc = {};
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        sacc = floor_mfma(kc[c], qh, sacc);
        sacc = floor_mfma(kc[c], ql, sacc);
      }
      half8 p0, p1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p0[e] = (_Float16)sacc[e];
        p1[e] = (_Float16)sacc[8 + e];
      }
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        acc[b] = floor_mfma(vc[2 * b], p0, acc[b]);
        acc[b] = floor_mfma(vc[2 * b + 1], p1, acc[b]);
      }
    }
  }
  float r = 0.0f;
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int j = 0; j < 16; ++j) r += acc[b][j];
  if (lane == 0) a.out[blockIdx.x * 8 + wave] = r;
}

// 4096 sleeps of 64 x 127 clocks each: about 14 ms at 2.4 GHz
__global__ __launch_bounds__(64) void k_ring_floor_hold() {
  for (int i = 0; i < 4096; ++i) __builtin_amdgcn_s_sleep(127);
}

hipError_t launch_floor(const FloorArgs& args, int kind, hipStream_t s, hipEvent_t t0,
                        hipEvent_t t1) {
  if (kind == 6) {
    hipExtLaunchKernelGGL(k_ring_floor_hold, dim3(1), dim3(64), 0, s, t0, t1, 0);
    return hipGetLastError();
  }
  if (kind == 11) {
    // one work-group of eight waves per (unit, split); a.n_split counts the
    // splits of this grid, a.n_rb must be 1
    FloorArgs a = args;
    const uint64_t grid = (uint64_t)a.n_seq * a.n_head_kv * a.n_split;
    if (a.n_split < 1 || a.n_rb != 1 || grid * a.n_split > (uint64_t(1) << 32) ||
        (uint64_t)(a.ring_tiles + a.n_split) * a.n_split > (uint64_t(1) << 32))
      return hipErrorInvalidValue;
    a.rcp_per_unit = recip32((uint32_t)a.n_split);
    a.rcp_n_rb = recip32(1);
    a.rcp_n_head_kv = recip32(a.n_head_kv);
    a.rcp_n_split = recip32(a.n_split);
    hipExtLaunchKernelGGL(k_ring_floor_pair, dim3((unsigned)grid), dim3(512), 0, s, t0, t1, 0, a);
    return hipGetLastError();
  }
  FloorArgs a = args;
  const uint64_t per_unit = (uint64_t)a.n_split * a.n_rb;
  const uint64_t grid = (uint64_t)a.n_seq * a.n_head_kv * per_unit;
  if (a.n_split < 1 || a.n_rb < 1 || grid * per_unit > (uint64_t(1) << 32) ||
      (uint64_t)(a.ring_tiles + a.n_split) * a.n_split > (uint64_t(1) << 32))
    return hipErrorInvalidValue;
  a.rcp_per_unit = recip32((uint32_t)per_unit);
  a.rcp_n_rb = recip32(a.n_rb);
  a.rcp_n_head_kv = recip32(a.n_head_kv);
  a.rcp_n_split = recip32(a.n_split);
  const dim3 g((unsigned)grid), b(256);
  switch (kind) {
    case 0: hipExtLaunchKernelGGL(k_ring_floor<0>, g, b, 0, s, t0, t1, 0, a); break;
    case 1: hipExtLaunchKernelGGL(k_ring_floor<1>, g, b, 0, s, t0, t1, 0, a); break;
    case 2: hipExtLaunchKernelGGL(k_ring_floor<2>, g, b, 0, s, t0, t1, 0, a); break;
    case 3: hipExtLaunchKernelGGL(k_ring_floor<3>, g, b, 0, s, t0, t1, 0, a); break;
    case 4: hipExtLaunchKernelGGL(k_ring_floor<4>, g, b, 0, s, t0, t1, 0, a); break;
    case 7: hipExtLaunchKernelGGL(k_ring_floor<7>, g, b, 0, s, t0, t1, 0, a); break;
    case 8: hipExtLaunchKernelGGL(k_ring_floor<8>, g, b, 0, s, t0, t1, 0, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

__global__ __launch_bounds__(128) void k_ring_floor_proj(ProjFloorArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // work-group -> (layer, half head part hh, d-slice), the projection's order
  const uint32_t b1 = blockIdx.x;
  const uint32_t b2 = quot32(b1, a.rcp_n_ds);
  const int ds = (int)(b1 - b2 * a.n_ds);
  const int n_hh = 4 * a.n_head_kv, n_hp = 2 * a.n_head_kv;
  const int layer = (int)quot32(b2, a.rcp_n_hh);
  const int hh = (int)(b2 - layer * n_hh);
  const int pw = 2 * (hh & 1) + wave;
  const u32x4* wp = (const u32x4*)a.wpack +
                    ((((int64_t)layer * n_hp + (hh >> 1)) * a.n_ds + ds) * 4 + pw) * 1024;
  u32x4 w[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) w[i] = wp[i * 64 + lane];
  u32x4 x = w[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) x ^= w[i];
  uint32_t v = x.x ^ x.y ^ x.z ^ x.w;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v ^= __shfl_xor(v, off);
  if (lane == 0) a.out[blockIdx.x * 2 + wave] = (float)(v & 0xFFFFu);
}

hipError_t launch_floor_proj(const ProjFloorArgs& args, hipStream_t s, hipEvent_t t0,
                             hipEvent_t t1) {
  ProjFloorArgs a = args;
  const uint32_t n_hh = 4 * a.n_head_kv;
  const uint64_t grid = (uint64_t)a.n_layer * n_hh * a.n_ds;
  if (a.n_ds < 1 || grid * a.n_ds > (uint64_t(1) << 32) || grid > (uint64_t(1) << 31))
    return hipErrorInvalidValue;
  a.rcp_n_ds = recip32(a.n_ds);
  a.rcp_n_hh = recip32(n_hh);
  hipExtLaunchKernelGGL(k_ring_floor_proj, dim3((unsigned)grid), dim3(128), 0, s, t0, t1, 0, a);
  return hipGetLastError();
}

int floor_resident_blocks() {
  int dev = 0, per_cu = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_ring_floor<4>, 256, 0) != hipSuccess)
    return 0;
  return per_cu * prop.multiProcessorCount;
}

}  // namespace ringkv
