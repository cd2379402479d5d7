// ring_layout.h -- device layout of the K/V rings (host and device code).
//
// A ring of one (sequence, layer) holds kv_total slots of kv_row = n_head_kv *
// 128 F16 values.  In device memory each KV head's slots are cut into tiles of
// 32 slots (8 KiB per tile for K, 8 KiB for V), and each tile is stored in the
// operand order of the gfx950 matrix instruction v_mfma_f32_32x32x16_f16, so
// that the attention kernel loads every operand with one coalesced 16-byte
// load per lane and no LDS transpose:
//
//   K tile, chunk c (0..7), lane l (0..63), element e (0..7):
//       K[slot = l % 32][dim = 16 c + 8 (l / 32) + e]
//     -- the A operand of S^T = K Q^T for dims [16c, 16c + 16).
//   V tile, chunk j = 2 b + ks (b: 32-dim block 0..3, ks: 16-slot step 0..1):
//       V[slot = 16 ks + 8 (e / 4) + 4 (l / 32) + e % 4][dim = 32 b + l % 32]
//     -- the A operand of O^T = V^T P^T.  The slot order inside a 16-slot step
//        matches the rows of the S^T accumulator that lane l holds, so the
//        softmax weights feed the PV product straight from registers.
//
// Element (chunk, lane, e) sits at halves offset (chunk * 64 + lane) * 8 + e.
// Tiles are ordered [seq][layer][kv head][tile].
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define RING_HD __host__ __device__
#else
#define RING_HD
#endif

namespace ringkv {

constexpr int kTile = 32;                       // slots per tile
constexpr int kHeadDim = 128;                   // supported head_dim
constexpr int kTileHalves = kTile * kHeadDim;   // 4096 F16 = 8 KiB
constexpr int kBulkChunk = 1024;                // rows per bulk append chunk
constexpr int kMaxM = 64;                       // q_len * group supported

// Offset (in halves) inside a K tile of slot s_t (0..31), head dim d (0..127).
RING_HD inline int k_frag_index(int s_t, int d) {
  const int c = d >> 4, h = (d >> 3) & 1, e = d & 7;
  return ((c << 6) + (h << 5) + s_t) * 8 + e;
}

// Offset (in halves) inside a V tile of slot s_t (0..31), head dim d (0..127).
RING_HD inline int v_frag_index(int s_t, int d) {
  const int b = d >> 5, n = d & 31;
  const int ks = s_t >> 4, r = s_t & 15;
  const int e = ((r >> 3) << 2) | (r & 3);
  const int h = (r >> 2) & 1;
  return ((((b << 1) | ks) << 6) + (h << 5) + n) * 8 + e;
}

}  // namespace ringkv
