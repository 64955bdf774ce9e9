// Integer tile schedule of the varlen attention kernel, shared by the device
// code and the host entry points (the host copy is exported so the schedule
// can be checked against brute force on the CPU).
//
// Visibility rule (the pages name causal and window_size but do not define
// them for Lq != Lk; this is the bottom-right reading): query row i of a
// segment with Lq queries and Lk keys sits at key position p = i + Lk - Lq;
// key j is visible when lo(i) <= j <= hi(i) with
//     lo(i) = window_left  >= 0 ? max(0, p - window_left)        : 0
//     hi(i) = causal              ? min(Lk - 1, p)
//           : window_right >= 0   ? min(Lk - 1, p + window_right) : Lk - 1
// Both bounds grow by at most one per row, so the rows that see at least one
// key form a contiguous range and their key intervals overlap or touch: the
// keys a block of rows needs form one contiguous range of tiles.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define VA_HD __host__ __device__ __forceinline__
#else
#define VA_HD inline
#endif

namespace va {

struct RowBounds {
  int64_t lo;
  int64_t hi;
};

VA_HD int64_t imin64(int64_t a, int64_t b) { return a < b ? a : b; }
VA_HD int64_t imax64(int64_t a, int64_t b) { return a > b ? a : b; }

// Floor division for a possibly negative numerator and a positive divisor.
VA_HD int64_t floor_div(int64_t a, int64_t b) {
  int64_t q = a / b;
  return (a % b != 0 && a < 0) ? q - 1 : q;
}

VA_HD RowBounds row_bounds(int64_t i, int64_t Lq, int64_t Lk, int causal, int wl, int wr) {
  const int64_t p = i + Lk - Lq;
  RowBounds r;
  r.lo = wl >= 0 ? imax64(0, p - wl) : 0;
  r.hi = Lk - 1;
  if (causal)
    r.hi = imin64(r.hi, p);
  else if (wr >= 0)
    r.hi = imin64(r.hi, p + wr);
  return r;
}

struct TileRange {
  int32_t kt_begin, kt_end;      // key tiles visited
  int32_t full_begin, full_end;  // tiles that need no mask (subset of the above)
};

// Schedule for rows [r0, r1) (0 <= r0 < r1 <= Lq) and key tiles of bn keys.
VA_HD TileRange tile_range(int64_t Lq, int64_t Lk, int64_t r0, int64_t r1, int causal, int wl,
                           int wr, int bn) {
  TileRange t;
  t.kt_begin = t.kt_end = t.full_begin = t.full_end = 0;
  if (Lk <= 0 || r1 <= r0) return t;
  const int64_t off = Lk - Lq;
  // Rows that see >= 1 key: p >= -right_reach and p <= Lk - 1 + wl.
  int64_t first = r0, last = r1 - 1;
  const bool right_bounded = causal || wr >= 0;
  const int64_t right_reach = causal ? 0 : wr;
  if (right_bounded) first = imax64(first, -right_reach - off);
  if (wl >= 0) last = imin64(last, Lk - 1 + wl - off);
  if (first > last) return t;
  const int64_t lo_first = row_bounds(first, Lq, Lk, causal, wl, wr).lo;
  const int64_t hi_last = row_bounds(last, Lq, Lk, causal, wl, wr).hi;
  t.kt_begin = (int32_t)(lo_first / bn);
  t.kt_end = (int32_t)(hi_last / bn + 1);
  // A tile needs no mask when every row of the block sees all of it: the
  // largest lo (last row) is <= the tile start and the smallest hi (first
  // row) is >= the tile end.  Empty rows (hi < lo) make this impossible.
  const int64_t lo_max = row_bounds(r1 - 1, Lq, Lk, causal, wl, wr).lo;
  const int64_t hi_min = row_bounds(r0, Lq, Lk, causal, wl, wr).hi;
  int64_t fb = floor_div(lo_max + bn - 1, bn);
  int64_t fe = floor_div(hi_min + 1, bn);
  fb = imax64(fb, t.kt_begin);
  fe = imin64(fe, t.kt_end);
  if (fb >= fe) {
    fb = fe = t.kt_begin;
  }
  t.full_begin = (int32_t)fb;
  t.full_end = (int32_t)fe;
  return t;
}

// ---------------------------------------------------------------------------
// Workgroup -> (segment, head, q-tile).
//
// The hardware dispatches workgroup w to XCD w % 8 (8 XCDs, each with its own
// L2).  Work is grouped by (segment b, head h), g = b * heads + h, each group
// owning n_qt q-tiles that stream the same K/V.  Groups are dealt round-robin
// over the XCDs (group g -> XCD g % 8) so every XCD gets the same mix of
// segments, and the q-tiles of one group sit next to each other in their
// XCD's dispatch order so they run together and share that XCD's L2.
// The grid is padded to a multiple of 8 groups; padding blocks get valid = 0.
struct WorkUnit {
  int32_t b, h, qt;
  int32_t valid;
};

VA_HD int64_t grid_blocks(int64_t batch, int64_t heads, int64_t n_qt) {
  const int64_t groups = batch * heads;
  return 8 * ((groups + 7) / 8) * n_qt;
}

VA_HD WorkUnit decode_block(int64_t w, int64_t batch, int64_t heads, int64_t n_qt, int causal) {
  const int64_t x = w & 7, k = w >> 3;
  const int64_t gl = k / n_qt, qi = k % n_qt;
  const int64_t g = gl * 8 + x;
  WorkUnit u;
  u.valid = g < batch * heads;
  u.b = (int32_t)(g / heads);
  u.h = (int32_t)(g % heads);
  // Causal: the last q-tiles of a segment see the most keys; start them first.
  u.qt = (int32_t)(causal ? n_qt - 1 - qi : qi);
  return u;
}

}  // namespace va
