// Band geometry of causal sliding-window attention, shared by the kernels and by
// the host-side tile enumerator that the tests compare with the mask definition.
//
// Mask ("Autoresearch 深度教程" §5.2.2: every layer passes a (W, 0) window to
// FlashAttention-3, i.e. W keys to the left of the query and none to the right):
//   key j is visible to query i  iff  0 <= i - j <= W   (W < 0: no left bound)
// and both i and j lie inside the sequence [0, T).
#pragma once

#if defined(__HIPCC__)
#define SW_HD __host__ __device__ __forceinline__
#else
#define SW_HD inline
#endif

namespace swattn {

// Tile classes for a (query rows) x (key rows) block.
enum TileClass : int { TILE_EMPTY = 0, TILE_PARTIAL = 1, TILE_FULL = 2 };

SW_HD int imin(int a, int b) { return a < b ? a : b; }
SW_HD int imax(int a, int b) { return a > b ? a : b; }

// Window normalised so that "no bound" is a value no distance reaches.
SW_HD int eff_window(int T, int window) { return (window < 0 || window >= T) ? T : window; }

SW_HD bool visible(int i, int j, int T, int W) {
  // W already normalised by eff_window
  return i < T && j < T && j <= i && i - j <= W;
}

// Keys visible to at least one query row of [q_lo, q_hi] (clamped to [0, T)).
// Returns false when there is none.
SW_HD bool kv_range(int q_lo, int q_hi, int T, int W, int* kv_lo, int* kv_hi) {
  q_hi = imin(q_hi, T - 1);
  if (q_lo > q_hi) return false;
  *kv_lo = imax(0, q_lo - W);
  *kv_hi = q_hi;
  return true;
}

// Queries that see at least one key of [kv_lo, kv_hi].
SW_HD bool q_range(int kv_lo, int kv_hi, int T, int W, int* q_lo, int* q_hi) {
  kv_hi = imin(kv_hi, T - 1);
  if (kv_lo > kv_hi) return false;
  *q_lo = kv_lo;
  long long hi = (long long)kv_hi + W;
  *q_hi = hi > (long long)(T - 1) ? T - 1 : (int)hi;
  return true;
}

// Class of the block of queries [q_lo, q_hi] x keys [kv_lo, kv_hi] (unclamped
// bounds: rows or keys past T count as invisible).
SW_HD int tile_class(int q_lo, int q_hi, int kv_lo, int kv_hi, int T, int W) {
  // empty: every key right of every query, or every key beyond the window
  int qh = imin(q_hi, T - 1), kh = imin(kv_hi, T - 1);
  if (q_lo > qh || kv_lo > kh) return TILE_EMPTY;
  if (kv_lo > qh) return TILE_EMPTY;
  if (q_lo - kh > W) return TILE_EMPTY;
  // full: inside the sequence, all keys left of (or at) all queries, all within W
  if (q_hi < T && kv_hi < T && kv_hi <= q_lo && q_hi - kv_lo <= W) return TILE_FULL;
  return TILE_PARTIAL;
}

// Schedule of the persistent dK/dV kernels.  The n8 key tiles of one XCD's
// range (consecutive tiles of its (batch, head) slices, nkt per slice) go to
// its g8 workgroups in rounds of g8 consecutive tiles; in round i workgroup s
// takes tile i g8 + x, or none past the range (-1).  x = (s + 7 i) mod g8
// rotates the light tiles of the causal tail through the workgroups: when the
// number of rounds R is a multiple of nkt (and nkt divides g8), every
// workgroup meets every tile position of a slice equally often.  Otherwise,
// with R even, round i >= R / 2 takes the mirror g8 - 1 - x of round i - R / 2:
// mirrored positions of a causal band have band lengths that sum to about a
// constant, so each workgroup's pairs of rounds carry about equal work.
// mirror_from() is the first mirrored round (the number of rounds when none
// is); the launcher computes it and passes it to the kernels, which compile the
// mirrored schedule only when some round is mirrored.
SW_HD int mirror_from(int g8, int n8, int nkt) {
  const int rounds = (n8 + g8 - 1) / g8;
  return ((rounds & 1) == 0 && rounds % nkt != 0) ? rounds / 2 : rounds;
}
SW_HD int schedule_tile(int i, int s, int g8, int n8, int half) {
  if (i * g8 >= n8) return -1;
  const bool m = i >= half;
  const int x0 = (s + 7 * (m ? i - half : i)) % g8;
  const int r = i * g8 + (m ? g8 - 1 - x0 : x0);
  return r < n8 ? r : -1;
}

SW_HD int persistent_tile(int i, int s, int g8, int n8, int nkt) {
  return schedule_tile(i, s, g8, n8, mirror_from(g8, n8, nkt));
}

}  // namespace swattn
