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

// Division by a run-time constant without a divide: q = floor(n / d) for
// 0 <= n < 2^31 as (umulhi(n, mul) + n) >> shift, with 2^shift >= d and
// 2^32 + mul = ceil(2^(32 + shift) / d).  (Exact: writing
// (2^32 + mul) d = 2^(32 + shift) + e with 0 <= e < d <= 2^shift, the
// product n (2^32 + mul) / 2^(32 + shift) exceeds n / d by n e / (d 2^(32 +
// shift)) < 1 / d, too little to reach the next integer; n < 2^31 keeps
// umulhi(n, mul) + n below 2^32.)  The host computes the multipliers once
// per launch; the kernel's work-unit decode then costs a multiply and a
// shift per division instead of a division routine.
struct FastDiv {
  uint32_t d, mul, shift;
};

VA_HD FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  uint32_t s = 0;
  while (((uint64_t)1 << s) < (uint64_t)d) ++s;
  const uint64_t m = (((uint64_t)1 << (32 + s)) + d - 1) / d;
  f.d = d;
  f.mul = (uint32_t)(m - ((uint64_t)1 << 32));
  f.shift = s;
  return f;
}

VA_HD uint32_t fdiv(uint32_t n, FastDiv f) {
  const uint32_t t = (uint32_t)(((uint64_t)n * f.mul) >> 32);
  return (t + n) >> f.shift;
}

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

// Schedule for rows [r0, r1) (0 <= r0 < r1 <= Lq) and key tiles of bn keys,
// the segment's keys starting at key key_off of the tiled range (0 unless
// several short segments share one workgroup's keys).
VA_HD TileRange tile_range(int64_t Lq, int64_t Lk, int64_t r0, int64_t r1, int causal, int wl,
                           int wr, int bn, int64_t key_off = 0) {
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
  const int64_t lo_first = key_off + row_bounds(first, Lq, Lk, causal, wl, wr).lo;
  const int64_t hi_last = key_off + row_bounds(last, Lq, Lk, causal, wl, wr).hi;
  t.kt_begin = (int32_t)(lo_first / bn);
  t.kt_end = (int32_t)(hi_last / bn + 1);
  // A tile needs no mask when every row of the block sees all of it: the
  // largest lo (last row) is <= the tile start and the smallest hi (first
  // row) is >= the tile end.  Empty rows (hi < lo) make this impossible.
  const int64_t lo_max = key_off + row_bounds(r1 - 1, Lq, Lk, causal, wl, wr).lo;
  const int64_t hi_min = key_off + row_bounds(r0, Lq, Lk, causal, wl, wr).hi;
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

// Split-KV: the split-th of num_splits runs of ceil(n / num_splits) tiles of
// a visit range of n tiles (the last runs may be short or empty), with its
// unmasked sub-range.  num_splits == 1 returns t unchanged.
VA_HD TileRange split_range(TileRange t, int split, int num_splits) {
  if (num_splits <= 1) return t;
  const int32_t n = t.kt_end - t.kt_begin;
  const int32_t per = (n + num_splits - 1) / num_splits;
  TileRange r;
  r.kt_begin = (int32_t)imin64(t.kt_begin + (int64_t)split * per, t.kt_end);
  r.kt_end = (int32_t)imin64((int64_t)r.kt_begin + per, t.kt_end);
  r.full_begin = (int32_t)imin64(imax64(t.full_begin, r.kt_begin), r.kt_end);
  r.full_end = (int32_t)imin64(imax64(t.full_end, r.kt_begin), r.kt_end);
  if (r.full_begin >= r.full_end) r.full_begin = r.full_end = r.kt_begin;
  return r;
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
//
// Within an XCD, workgroups are dispatched strictly in order, and the k-th
// one (k = w >> 3) always goes to shader engine (k + c) % 4 for some c: when
// the next workgroup's engine has no free CU, dispatch waits even if other
// engines are idle.  Workgroups of unequal cost should therefore share each
// engine evenly.  Runs of q-tiles in cost order (causal q-tiles, or groups
// dealt longest first) are dealt in a snake over aligned quads of k: every
// odd quad is reversed (k -> k ^ 3), so no engine always gets the costliest
// workgroup of each quad.
struct WorkUnit {
  int32_t b, h, qt;
  int32_t valid;
};

// Short segments share a workgroup of four waves of rows_per_wave query
// rows: with every segment at most rows_per_wave queries long, four
// consecutive segments (one wave each); at most twice that, two (two waves
// each); otherwise one.  The group of P segments then takes the place of a
// segment in the dealing below (segment index = group index, one q-tile),
// and its keys, consecutive in memory, are the workgroup's keys.
VA_HD int32_t segments_per_block(int64_t max_seqlen_q, int64_t rows_per_wave) {
  return max_seqlen_q <= rows_per_wave ? 4 : (max_seqlen_q <= 2 * rows_per_wave ? 2 : 1);
}

// How a workgroup's four waves are filled when segments are that short:
// with grouped KV heads whose group size is a multiple of P, the P slots take
// P query heads of one KV head over the same segment (kPackHeads: every K/V
// tile staged feeds all of them, and the segment's rows and tiles are those
// of an unpacked unit); otherwise P consecutive segments of one head
// (kPackSegments).  The workgroup's unit is then (segment, group of P query
// heads) or (group of P segments, head), one q-tile.
enum PackMode : int32_t { kPackNone = 0, kPackSegments = 1, kPackHeads = 2 };

VA_HD int32_t pack_mode(int64_t max_seqlen_q, int64_t rows_per_wave, int64_t heads, int64_t heads_k) {
  const int32_t pk = segments_per_block(max_seqlen_q, rows_per_wave);
  if (pk == 1) return kPackNone;
  return (heads_k > 0 && heads % heads_k == 0 && (heads / heads_k) % pk == 0) ? kPackHeads : kPackSegments;
}

// Workgroups of a launch: (segment, head group) groups dealt over the 8
// XCDs, each holding n_per workgroups (its heads' q-tiles).
VA_HD int64_t grid_blocks(int64_t batch, int64_t hgroups, int64_t n_per) {
  const int64_t groups = batch * hgroups;
  return 8 * ((groups + 7) / 8) * n_per;
}

// Head groups.  With head dims of 72 or 80 a head's row of Q, K, V or O
// (144 / 160 bytes) shares 128-byte lines with its neighbours, so heads
// dealt to different XCDs make every XCD's L2 fetch those lines again
// (measured: 1.6x the algorithmic bytes fetched on the 256- and 64-token
// ViT windows).  The dealing below therefore keeps 2^hs adjacent heads of a
// segment together, 2^hs x (row bytes) being a whole number of lines: their
// workgroups go to one XCD, one q-tile of each head after the other, so they
// run together and share those lines in its L2.  hs = 0 for grouped KV
// heads (whose own dealing keeps a KV head's query heads together) and
// where the rows are line-aligned already.
VA_HD int32_t head_group_shift(int32_t d_qk, int32_t d_v, int32_t heads, int32_t heads_k, int32_t in_bytes) {
  if (heads_k != heads) return 0;
  for (int32_t s = 0; s <= 3; ++s) {
    const int32_t hg = 1 << s;
    if (heads % hg != 0) break;
    if ((hg * d_qk * in_bytes) % 128 == 0 && (hg * d_v * in_bytes) % 128 == 0 && (hg * d_v * 2) % 128 == 0)
      return s;
  }
  return 0;
}

// One-wave workgroups of short segments (a segment's rows are one unit
// per head) deal more heads together: all of a segment's heads (up to 16)
// on one XCD, so that XCD reads the segment's rows of Q, K, V and O whole
// rather than four XCDs reading interleaved pieces of them (measured 3%
// faster on 700 windows of 64 tokens, 16 heads, d 80), as long as the
// batch still gives every XCD at least 8 groups; never fewer heads than
// head_group_shift asks for.
VA_HD int32_t short_head_group_shift(int32_t d_qk, int32_t d_v, int32_t heads, int32_t heads_k, int64_t batch,
                                     int32_t in_bytes) {
  int32_t s = head_group_shift(d_qk, d_v, heads, heads_k, in_bytes);
  if (heads_k != heads) return s;
  while (s < 4 && heads % (2 << s) == 0 && batch * (heads >> (s + 1)) >= 64) ++s;
  return s;
}

// The quad snake over an XCD's dispatch index k (of k_count per XCD); a
// trailing partial quad keeps its order.
VA_HD uint32_t snake_quads(uint32_t k, uint32_t k_count) {
  return ((k >> 2) & 1u) && (k | 3u) < k_count ? k ^ 3u : k;
}

// 32-bit arithmetic: the launch checks that the grid fits in int32.
// `hgroups` is the dealt head count over 2^hs (head groups, see
// head_group_shift) and `n_per` the workgroups per group (q-tiles per
// segment times 2^hs), both as FastDivs.  Within a group the order is
// q-tile major: q-tile 0 of its 2^hs heads, then q-tile 1, ...
VA_HD WorkUnit decode_block(uint32_t w, uint32_t batch, FastDiv hgroups, FastDiv n_per, uint32_t hs, int causal) {
  const uint32_t groups = batch * hgroups.d;
  const uint32_t x = w & 7u;
  const uint32_t k = snake_quads(w >> 3, (groups + 7u) / 8u * n_per.d);
  const uint32_t gl = fdiv(k, n_per), local = k - gl * n_per.d;
  const uint32_t g = gl * 8u + x;
  const uint32_t qi = local >> hs, n_qt = n_per.d >> hs;
  WorkUnit u;
  u.valid = g < groups;
  u.b = (int32_t)fdiv(g, hgroups);
  u.h = (int32_t)(((g - (uint32_t)u.b * hgroups.d) << hs) + (local & ((1u << hs) - 1u)));
  // Causal: the last q-tiles of a segment see the most keys; start them first.
  u.qt = (int32_t)(causal ? n_qt - 1u - qi : qi);
  return u;
}

// Longest-first dealing.  On a batch of segments of different lengths,
// dealing in packing order can leave a long segment's workgroups for last,
// running alone at the end.  When the batch has at most kLptMaxBatch segments
// and they are not all alike, the segments are instead ranked by key length,
// longest first (ties in packing order), groups are dealt round-robin over
// the XCDs in that order (group r * heads + h -> XCD (r * heads + h) % 8 for
// the segment of rank r), and each group contributes only its real q-tiles
// (ceil(Lq / block_m)), adjacent in its XCD's dispatch order.  The kernel
// computes this from cu_seqlens (one lane per segment); decode_block_lpt is
// the host reference.
constexpr int kLptMaxBatch = 64;

// Grouped KV heads.  With heads_k KV heads shared by heads query heads
// (heads a multiple of heads_k), query head h reads KV head h / (heads /
// heads_k): consecutive query heads share a KV head.  The schedule deals
// groups by a dealing index d, not by the query head directly: d runs over
// the KV heads fastest, so the query heads of one KV head have dealing
// indices congruent modulo heads_k and, when heads_k is a multiple of 8
// (groups being dealt over the 8 XCDs by d), all run on one XCD and read
// that KV head through its L2 (with heads_k = 4, on two).  Without grouping
// (heads_k == heads) d is the query head.
// heads_k as a FastDiv, group = heads / heads_k.
VA_HD int32_t query_head(int32_t d, FastDiv heads_k, int32_t group) {
  const int32_t dq = (int32_t)fdiv((uint32_t)d, heads_k);
  return (d - dq * (int32_t)heads_k.d) * group + dq;
}

// The heads (or head groups) of the segment of rank r dealt to XCD x are
// h0, h0 + 8, ...
VA_HD int32_t xcd_first_head(int32_t r, int32_t heads, int32_t x) {
  return (x - (int32_t)(((int64_t)r * heads) % 8) + 8) % 8;
}
VA_HD int32_t xcd_head_count(int32_t h0, int32_t heads) { return h0 < heads ? (heads - 1 - h0) / 8 + 1 : 0; }

// Whether longest-first dealing applies to segments with these lengths.
inline bool lpt_applies(int32_t batch, const int32_t* lq, const int32_t* lk) {
  if (batch > kLptMaxBatch) return false;
  for (int32_t i = 1; i < batch; ++i)
    if (lq[i] != lq[0] || lk[i] != lk[0]) return true;
  return false;
}

// Host reference of the kernel's longest-first mapping (quadratic in batch).
inline WorkUnit decode_block_lpt(int64_t w, int32_t batch, int32_t heads, int32_t block_m, int32_t n_qt,
                                 int causal, const int32_t* lq, const int32_t* lk, int32_t hs = 0,
                                 bool pair = false) {
  const int32_t x = (int32_t)(w & 7);
  const int32_t hgroups = heads >> hs;
  const int64_t k = snake_quads((uint32_t)(w >> 3), (uint32_t)(grid_blocks(batch, hgroups, (int64_t)n_qt << hs) / 8));
  int64_t pre = 0;
  for (int32_t r = 0; r < batch; ++r) {
    int32_t i = 0;  // the segment of rank r
    for (; i < batch; ++i) {
      int32_t rank = 0;
      for (int32_t j = 0; j < batch; ++j) rank += (lk[j] > lk[i] || (lk[j] == lk[i] && j < i)) ? 1 : 0;
      if (rank == r) break;
    }
    const int32_t nqt1 = (lq[i] + block_m - 1) / block_m;
    const int32_t nqt = pair ? (nqt1 + 1) / 2 : nqt1;  // q-tiles, or pairs of them
    const int64_t per = (int64_t)nqt << hs;  // workgroups of one head group of this segment
    const int32_t h0 = xcd_first_head(r, hgroups, x);
    const int64_t n = (int64_t)xcd_head_count(h0, hgroups) * per;
    if (k < pre + n) {
      const int64_t local = k - pre, grp = local / per, rem = local - grp * per, qi = rem >> hs;
      WorkUnit u;
      u.valid = 1;
      u.b = i;
      u.h = (int32_t)(((h0 + 8 * grp) << hs) + (rem & ((1 << hs) - 1)));
      u.qt = (int32_t)(causal ? nqt - 1 - qi : qi);
      return u;
    }
    pre += n;
  }
  WorkUnit u;
  u.valid = 0;
  u.b = u.h = u.qt = -1;
  return u;
}

}  // namespace va
