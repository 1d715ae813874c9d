// ra_pos.h -- position and mask algebra shared by the host planner and the device kernels.
//
// Global positions: query row i at q_off + i*s, key t at k_off + t*s (s = 1 for the
// contiguous layout, s = P for the striped one).  The causal rule k <= q ("Ring
// Attention：把超长序列沿设备环流动", Causal section) becomes
//     k_off + t*s <= q_off + i*s   <=>   t - i <= (q_off - k_off)/s   <=>   t <= i + diag,
// diag = floor((q_off - k_off) / s), because t - i is an integer.  Every mask and skip
// decision in the library is a comparison against that one shifted diagonal, so the host
// planner and the kernels cannot disagree.
//
// Tiles: a query tile holds rows [i0, i1), a key tile keys [t0, t1).  It is EMPTY when its
// best pair (last row, first key) is masked, FULL when its worst pair (first row, last key)
// is allowed, PARTIAL otherwise (the page's strictly-future / diagonal-crossing / unmasked
// rule, applied per tile as well as per block).
#pragma once

#include <stdint.h>

#if defined(__HIPCC__) || defined(__HIP__)
#define RA_HD __host__ __device__ __forceinline__
#else
#define RA_HD static inline
#endif

namespace ra {

enum : int { TILE_EMPTY = 0, TILE_FULL = 1, TILE_PARTIAL = 2 };

RA_HD int64_t floor_div(int64_t a, int64_t b) {  // b > 0
  int64_t q = a / b;
  return (a % b != 0 && a < 0) ? q - 1 : q;
}

// diag for a block, clamped to [-(n_q + 1), n_k + 1]: outside that range every decision
// over i in [0, n_q), t in [0, n_k) is already "nothing" or "everything", so the clamp
// changes none of them and lets the kernels work in int32.
RA_HD int32_t diag_shift(int causal, int64_t q_off, int64_t k_off, int32_t s, int32_t n_q,
                         int32_t n_k) {
  if (!causal) return n_k + 1;
  int64_t d = floor_div(q_off - k_off, (int64_t)s);
  if (d > (int64_t)n_k + 1) d = (int64_t)n_k + 1;
  if (d < -(int64_t)n_q - 1) d = -(int64_t)n_q - 1;
  return (int32_t)d;
}

// Keys of the block visible to row i: t in [0, keys_visible).
RA_HD int32_t keys_visible(int32_t i, int32_t diag, int32_t n_k) {
  int64_t c = (int64_t)i + diag + 1;
  if (c < 0) c = 0;
  if (c > n_k) c = n_k;
  return (int32_t)c;
}

// Key tiles of width bk that query tile [i0, i1) must visit: tiles [0, tiles_live).
RA_HD int32_t tiles_live(int32_t i0, int32_t i1, int32_t diag, int32_t n_k, int32_t bk) {
  (void)i0;
  if (i1 <= i0) return 0;
  int32_t n = keys_visible(i1 - 1, diag, n_k);
  return (n + bk - 1) / bk;
}

// Leading key tiles that are FULL for every row of [i0, i1): tiles [0, tiles_full).
RA_HD int32_t tiles_full(int32_t i0, int32_t i1, int32_t diag, int32_t n_k, int32_t bk) {
  if (i1 <= i0) return 0;
  int32_t n = keys_visible(i0, diag, n_k);
  if (n == n_k) return (n_k + bk - 1) / bk;
  return n / bk;
}

RA_HD int classify_tile(int32_t i0, int32_t i1, int32_t t0, int32_t t1, int32_t diag) {
  if (i1 <= i0 || t1 <= t0) return TILE_EMPTY;
  if ((int64_t)t0 > (int64_t)(i1 - 1) + diag) return TILE_EMPTY;
  if ((int64_t)(t1 - 1) <= (int64_t)i0 + diag) return TILE_FULL;
  return TILE_PARTIAL;
}

}  // namespace ra
