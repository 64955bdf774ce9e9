// Short segments: one wavefront per (segment, head, block of 64 query rows).
//
// Segments of at most 64 queries (windowed ViT attention with 64-patch
// windows, say) are one wave's rows each, and their keys a few 32-key tiles.
// The four-wave kernel can only give such a segment one wave of a shared
// workgroup: the workgroup then streams four segments' keys behind common
// barriers, and in each tile step only the wave whose segment owns the tile
// computes.  Here each wave is a work unit of its own, which streams its
// segment's keys and meets no barrier:
//
//   K tile: HBM -> registers directly.  The A operand of S^T = K Q^T on
//       v_mfma_f32_32x32x16_bf16 is, per lane, 16 contiguous bytes of one key
//       row (key l % 32, head dims 16 c + 8 (l / 32) ...), so it needs no
//       LDS staging.  Rows past the segment's keys read as zero.
//   V tile: HBM -> one of two private LDS stages by direct-to-LDS loads, for
//       the transposing reads (ds_read_b64_tr_b16) that form the V^T operand.
//
// A workgroup holds four such waves, each on its own unit, sharing nothing
// but the launch (one-wave workgroups left the dispatcher the bottleneck:
// 64-token windows ran 11% slower); two workgroups share a CU (256
// registers a wave, 2 x 6 KB of LDS a wave at d_v 80).  SGLang PR #41344,
// "Speed Tests and Profiling" ("Where fa4 loses" (b)), asks for a smaller
// query tile for short segments; this is it.
//
// The arithmetic on each 32-key tile is the four-wave kernel's per wave,
// step for step: the same tiles (they start at the segment's first key), the
// same QK^T accumulation order, fast-path test, slow path, lazy rescale and
// PV order, the same epilogue.  The output is therefore bit-identical to an
// unpacked launch of the four-wave kernel on the same call.
//
// Small launches of longer segments (Params::key_split = 4) use the same
// code with the four waves of a workgroup on one 64-row block instead, each
// walking a quarter of its key tiles; their (max, sum, accumulator) states
// are merged through LDS before wave 0's epilogue.  That is the same softmax
// summed in another order: within rounding of the four-wave kernel, not
// bit-identical to it.
#include "attn_common.h"
#include "wide_tile.h"

namespace va {
namespace narrow {
constexpr int kBN = 32;      // keys per tile
constexpr int kStages = 2;   // tile t: K in register set t % 2, V in LDS stage t % 2
constexpr int kWaves = 4;    // waves (independent work units) per workgroup
template <int DQK, int DV>
struct Cfg : TileGeom<DQK, DV, kBN> {
  static constexpr int QB = 2;         // 32-row query blocks of the wave
  static constexpr int RPW = 32 * QB;  // query rows per wave (one work unit)
  static constexpr int V_PAD = Cfg::CPR_V - Cfg::V_REAL;
  static_assert(2 * Cfg::KC + Cfg::V_WL < 64, "vmcnt range");
  static_assert(Cfg::CPR_V != 12 || v_swizzle<12>(1) == 0, "pad chunks sit at fixed positions");
};
}  // namespace narrow

template <int DQK, int DV, RowSum SUM>
__global__ __launch_bounds__(64 * narrow::kWaves, 2) void attn_fwd_short(Params p) {
  using namespace narrow;
  using C = Cfg<DQK, DV>;
  constexpr int QB = C::QB;
  constexpr bool SUM_BY_MFMA = SUM == RowSum::kMfma;
  static_assert(!SUM_BY_MFMA || C::V_PAD > 0, "the ones column needs a padded d_v");
  __shared__ __attribute__((aligned(4096))) char vs0[kWaves * C::V_TILE];
  __shared__ __attribute__((aligned(4096))) char vs1[kWaves * C::V_TILE];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  auto vst = [&](auto st) VA_INLINE -> lds_char* {  // this wave's stage st
    if constexpr (decltype(st)::value % 2 == 0) return (lds_char*)vs0 + wave * C::V_TILE;
    else return (lds_char*)vs1 + wave * C::V_TILE;
  };

  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31;
  const int g = lane >> 5;
  // This wave's work unit: workgroup w's wave v takes unit ((w >> 3) kWaves
  // + v) x 8 + (w & 7), on the XCD (w % 8) the unit's dealing intends.  On
  // small launches (Params::key_split) the four waves share unit w instead,
  // each with a quarter of its key tiles, and merge their partial results
  // through LDS before wave 0 writes them out; the early exits below are then
  // the whole workgroup's, so every wave meets the merge's barriers.
  const bool ksplit = p.key_split > 1;
  const int64_t unit =
      ksplit ? (int64_t)blockIdx.x : ((int64_t)(blockIdx.x >> 3) * kWaves + wave) * 8 + (blockIdx.x & 7);
  const BlockWork bw = block_work<kPackNone>(p, lane, C::RPW, unit);
  if (!bw.u.valid) return;
  const int h = bw.u.h;
  const int q0 = bw.q0, Lq = bw.lq, k0 = bw.k0, Lk = bw.lk;
  const int r0 = bw.u.qt * C::RPW;
  if (r0 >= Lq) return;
  const int r1 = min(r0 + C::RPW, Lq);
  const TileRange tr_unit = tile_range(Lq, Lk, r0, r1, p.causal, p.wl, p.wr, kBN);
  const TileRange tr = ksplit ? split_range(tr_unit, wave, kWaves) : tr_unit;  // this wave's tiles
  const int ntiles = tr.kt_end - tr.kt_begin;

  // ---- Q fragments (B operand of S^T = K Q^T): rows [r0, r1), zero past r1
  // and in the head-dim padding of d 72.
  bf16x8 qf[QB][C::KC];
  {
    const int64_t q_row_b = p.q_row * 2;
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.q + (int64_t)(q0 + r0) * p.q_row + (int64_t)h * p.q_head), (short)0,
        (int)(uint32_t)((r1 - r0) * q_row_b), kBufferFlags);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const uint32_t row_off = (uint32_t)((32 * qb + l32) * q_row_b);
#pragma unroll
      for (int c = 0; c < C::KC; ++c) {
        const int d = c * 16 + 8 * g;
        const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rq, d < DQK ? row_off + 2 * d : kOOB, 0, 0);
        qf[qb][c] = __builtin_bit_cast(bf16x8, x);
      }
    }
  }

  // ---- tile loads: K into registers, V into an LDS stage ---------------------
  // K: lane (l32, g) reads key l32 of the tile, head dims 16 c + 8 g .. + 7
  // (zero for the pad chunk of d 72), into register set t % 2.  V: wave-load
  // i covers V slots [64 i, 64 i + 64) of the tile (row-major, CPR_V chunks a
  // row, chunk index swizzled); lanes on padded chunks load nothing, lanes
  // past the slots read zeros into the stage's tail.  Issue order: Q, K 0,
  // V 0, K 1, V 1, then per tile j: K j + 2 (once tile j's scores are
  // final), V j + 2 (after PV j).
  const int hk = (int)fdiv((uint32_t)h, p.fd_group);  // the KV head query head h reads
  const int64_t k_row_b = p.k_row * 2, v_row_b = p.v_row * 2;
  uint32_t k_off[C::KC];
#pragma unroll
  for (int c = 0; c < C::KC; ++c)
    k_off[c] = 2 * c + g < C::K_REAL ? (uint32_t)(l32 * k_row_b + (16 * c + 8 * g) * 2) : kOOB;
  uint32_t v_off[C::V_WL];
  bool v_on[C::V_WL];
#pragma unroll
  for (int i = 0; i < C::V_WL; ++i) {
    const int sl = i * 64 + lane;
    const int row = sl / C::CPR_V;
    const int c = (sl % C::CPR_V) ^ v_swizzle<C::CPR_V>(row);
    v_on[i] = sl >= C::V_SLOTS || c < C::V_REAL;
    v_off[i] = (sl < C::V_SLOTS && c < C::V_REAL) ? (uint32_t)(row * v_row_b + c * 16) : kOOB;
  }
  const char* k_seg = (const char*)(p.k + (int64_t)k0 * p.k_row + (int64_t)hk * p.k_head);
  const char* v_seg = (const char*)(p.v + (int64_t)k0 * p.v_row + (int64_t)hk * p.v_head);
  bf16x8 kf[kStages][C::KC];
  auto tile_rows = [&](int t) VA_INLINE {  // keys of tile t (relative to kt_begin), clamped to [0, 32]
    return __builtin_amdgcn_readfirstlane(max(min(Lk - (tr.kt_begin + t) * kBN, kBN), 0));
  };
  auto issue_k = [&](auto st, int t) VA_INLINE {
    constexpr int S = decltype(st)::value;
    const int key = (tr.kt_begin + t) * kBN;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(k_seg + (int64_t)key * k_row_b), (short)0, (int)(tile_rows(t) * k_row_b), kBufferFlags);
#pragma unroll
    for (int c = 0; c < C::KC; ++c)
      kf[S][c] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, k_off[c], 0, 0));
  };
  auto issue_v = [&](auto st, int t) VA_INLINE {
    const int key = (tr.kt_begin + t) * kBN;
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(v_seg + (int64_t)key * v_row_b), (short)0, (int)(tile_rows(t) * v_row_b), kBufferFlags);
#pragma unroll
    for (int i = 0; i < C::V_WL; ++i)
      if (v_on[i]) dma16(rv, vst(st) + i * 1024, v_off[i]);
  };
  if (ntiles > 0) {
    issue_k(Int<0>{}, 0);
    issue_v(Int<0>{}, 0);
  }
  if (ntiles > 1) {
    issue_k(Int<1>{}, 1);
    issue_v(Int<1>{}, 1);
  }

  // ---- padded V chunks: zeros, or a one in column d_v (the row sum) ------------
  if constexpr (C::V_PAD > 0) {
    static_for<0, kStages>([&](auto st) VA_INLINE {
#pragma unroll
      for (int i = lane; i < kBN * C::V_PAD; i += 64) {
        const int row = i / C::V_PAD, c = C::V_REAL + i % C::V_PAD;
        const u32x4 val = {(SUM_BY_MFMA && c == C::V_REAL) ? 0x3F80u : 0u, 0u, 0u, 0u};  // bf16 1.0
        *(__attribute__((address_space(3))) u32x4*)(vst(st) + (row * C::CPR_V + c) * 16) = val;
      }
    });
  }
  // V^T operand reads: lane (G = l / 16, i = l % 16) of block vb.
  int v_rd[C::VB];
  {
    const int G = lane >> 4, i = lane & 15;
    const int vrow = 4 * g + (i >> 2);
    const int y = 2 * (G & 1) + ((i >> 1) & 1);
#pragma unroll
    for (int vb = 0; vb < C::VB; ++vb)
      v_rd[vb] = (vrow * C::CPR_V + ((4 * vb + y) ^ v_swizzle<C::CPR_V>(vrow))) * 16 + 8 * (i & 1);
  }

  // ---- running state ----------------------------------------------------------
  f32x16 acc[C::VB][QB];
#pragma unroll
  for (int vb = 0; vb < C::VB; ++vb)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[vb][qb][r] = 0.f;
  float m_run[QB], nm[QB], lim[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;  // running max of s * scale * log2(e)
    nm[qb] = 0.f;           // -m_run, or 0 while m_run is -inf
    lim[qb] = -FLT_MAX;     // m_run + kRescaleTau, or -FLT_MAX while m_run is -inf
    l_run[qb] = 0.f;        // fp32 row sum (unless SUM_BY_MFMA)
  }
  int row_lo[QB], row_hi[QB], first_j[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const RowBounds rb = row_bounds(r0 + 32 * qb + l32, Lq, Lk, p.causal, p.wl, p.wr);
    row_lo[qb] = (int)imin64(rb.lo, (int64_t)Lk);
    row_hi[qb] = (int)imax64(rb.hi, (int64_t)-1);
    // the tile holding the row's first visible key (relative), or -1
    first_j[qb] = row_lo[qb] <= row_hi[qb] ? row_lo[qb] / kBN - tr.kt_begin : -1;
  }
  const int full_begin = tr.full_begin - tr.kt_begin, full_end = tr.full_end - tr.kt_begin;
  bf16x8 pf[QB][2];  // probabilities: the PV B operand per (query block, 16-key half)

  // S^T of one tile: scores sbuf[qb][r] = key 8 (r / 4) + 4 g + r % 4, query l32.
  auto qk = [&](const bf16x8 (&kop)[C::KC], f32x16 (&s)[QB]) VA_INLINE {
    const f32x16 zero = {};
#pragma unroll
    for (int c = 0; c < C::KC; ++c)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[c], qf[qb][c], c == 0 ? zero : s[qb], 0, 0, 0);
  };
  // Boundary tiles only: scores of keys a row may not see become -inf.
  auto mask = [&](int j, f32x16 (&s)[QB]) VA_INLINE {
    if ((unsigned)(j - full_begin) >= (unsigned)(full_end - full_begin)) {
      const int key0 = (tr.kt_begin + j) * kBN;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int jj = key0 + 8 * (r >> 2) + 4 * g + (r & 3);
          s[qb][r] = (jj >= row_lo[qb] && jj <= row_hi[qb]) ? s[qb][r] : -INFINITY;
        }
    }
  };
  // Full online-softmax step (the slow path): row max, lazy-rescale
  // decision for the whole wave, p = exp2(s * scale * log2(e) - m), row sum,
  // bf16 pack.  Returns whether acc must be rescaled by alpha.
  auto softmax = [&](f32x16 (&s)[QB], float (&alpha)[QB]) VA_INLINE -> bool {
    float m_new[QB];
    bool need = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float m = fmaxf(fmaxf(s[qb][0], s[qb][1]), s[qb][2]);
#pragma unroll
      for (int r = 3; r < 15; r += 2) m = fmaxf(fmaxf(m, s[qb][r]), s[qb][r + 1]);
      m = fmaxf(m, s[qb][15]);
      m_new[qb] = fmaxf(m_run[qb], xhalf_max(m) * p.scale_log2);
      need |= m_new[qb] > m_run[qb] + kRescaleTau;
    }
    const bool move = __any(need);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float m_next = move ? m_new[qb] : m_run[qb];
      alpha[qb] = (m_next == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run[qb] - m_next);
      m_run[qb] = m_next;
      nm[qb] = (m_next == -INFINITY) ? 0.f : -m_next;
      lim[qb] = (m_next == -INFINITY) ? -FLT_MAX : m_next + kRescaleTau;
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float sum = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        u32x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 8 * t + 2 * e;
          const float x0 = __builtin_amdgcn_exp2f(fmaf(s[qb][r], p.scale_log2, nm[qb]));
          const float x1 = __builtin_amdgcn_exp2f(fmaf(s[qb][r + 1], p.scale_log2, nm[qb]));
          pk[e] = pack_bf16x2(x0, x1);
          if constexpr (SUM == RowSum::kF32) sum += x0 + x1;
        }
        pf[qb][t] = __builtin_bit_cast(bf16x8, pk);
      }
      if constexpr (!SUM_BY_MFMA) l_run[qb] = l_run[qb] * alpha[qb] + sum;
    }
    return move;
  };
  // The full softmax step with its rescale (the slow path).
  auto slow = [&](f32x16 (&s)[QB]) VA_INLINE {
    float alpha[QB];
    const bool move = softmax(s, alpha);
    if (move) {
      asm volatile("; lazy rescale" ::: "memory");
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int vb = 0; vb < C::VB; ++vb)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[vb][qb][r] *= alpha[qb];
    }
  };
  // One tile: scores, mask, the fast path or the slow path, then
  // O^T += V^T P^T.  The wave's first tile holds some row's first visible
  // key, so the fast path cannot hold there: it takes the full softmax at
  // once (FIRST), with no fast-path work to discard and no scores to
  // recompute.
  auto tile = [&](auto st, int j, auto first) VA_INLINE {
    constexpr int S = decltype(st)::value;
    f32x16 s[QB];
    qk(kf[S], s);
    mask(j, s);
    if constexpr (decltype(first)::value) {
      slow(s);
    } else {
      // The fast path: p = exp2(s * scale * log2(e) - m_run) in place, packed
      // to bf16 (and summed in pairs with the fp32 sum), valid when every p <=
      // 2^kRescaleTau and no row meets its first visible key: tested on the
      // raw row maxima with the ones-column sum, on the tile's row sums and the
      // rows' first tiles with the fp32 sum.
      bool bad = false;
      if constexpr (SUM_BY_MFMA) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          float m = fmaxf(fmaxf(s[qb][0], s[qb][1]), s[qb][2]);
#pragma unroll
          for (int r = 3; r < 15; r += 2) m = fmaxf(fmaxf(m, s[qb][r]), s[qb][r + 1]);
          m = fmaxf(m, s[qb][15]);
          bad |= m * p.scale_log2 > lim[qb];
        }
      } else {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) bad |= j == first_j[qb];
      }
      float sum[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          u32x4 pk;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 8 * t + 2 * e;
            s[qb][r] = __builtin_amdgcn_exp2f(fmaf(s[qb][r], p.scale_log2, nm[qb]));
            s[qb][r + 1] = __builtin_amdgcn_exp2f(fmaf(s[qb][r + 1], p.scale_log2, nm[qb]));
            pk[e] = pack_bf16x2(s[qb][r], s[qb][r + 1]);
            if constexpr (!SUM_BY_MFMA) {
              const float pair = s[qb][r] + s[qb][r + 1];
              sum[qb] = (t == 0 && e == 0) ? pair : sum[qb] + pair;
            }
          }
          pf[qb][t] = __builtin_bit_cast(bf16x8, pk);
        }
        if constexpr (!SUM_BY_MFMA) bad |= !(sum[qb] <= kSumLimit);
      }
      // Commit the row sums on one path; the slow path restores them.
      float l_prev[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        l_prev[qb] = l_run[qb];
        if constexpr (!SUM_BY_MFMA) l_run[qb] += sum[qb];
      }
      if (__any(bad)) {
        // Some row's max moved past m_run + kRescaleTau (or a row met its
        // first key): recompute the scores from K, still in registers, and take
        // the full softmax with the rescale.
        asm volatile("; softmax slow path" ::: "memory");
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) l_run[qb] = l_prev[qb];
        qk(kf[S], s);
        mask(j, s);
        slow(s);
      }
    }
    // K of tile j + 2 into this register set, then V of this tile landed:
    // only K j + 1, V j + 1 and K j + 2 (those that exist) may be in flight.
    if (j + 2 < ntiles) {
      issue_k(st, j + 2);
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * C::KC + C::V_WL) : "memory");
    } else if (j + 1 < ntiles) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(C::KC + C::V_WL) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    // O^T += V^T P^T: operand (t, vb) is V^T rows 32 vb .., keys 16 t ..
    const lds_char* vs = vst(st);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int vb = 0; vb < C::VB; ++vb) {
        const bf16x4 lo = lds_read_tr(vs, v_rd[vb] + (16 * t) * C::CPR_V * 16);
        const bf16x4 hi = lds_read_tr(vs, v_rd[vb] + (16 * t + 8) * C::CPR_V * 16);
        const bf16x8 vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          acc[vb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qb][t], acc[vb][qb], 0, 0, 0);
      }
  };

  // ---- main loop: tile j in set / stage j % 2 (tile 0 on its own, then
  // the loop unrolled by the stage count so each is named statically); V of
  // tile j + 2 is issued into the stage once PV j has read it.  (K j's
  // registers are waited for by the compiler at their first use.)
  if (ntiles > 0) {
    tile(Int<0>{}, 0, BoolTag<true>{});
    if (kStages < ntiles) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // stage 0's V^T reads are done
      issue_v(Int<0>{}, kStages);
    }
  }
  for (int j0 = 1; j0 < ntiles; j0 += kStages) {
    static_for<0, kStages>([&](auto u) VA_INLINE {
      constexpr int S = (decltype(u)::value + 1) % kStages;
      const int j = j0 + decltype(u)::value;
      if (j < ntiles) {
        tile(Int<S>{}, j, BoolTag<false>{});
        if (j + kStages < ntiles) {
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this stage's V^T reads are done
          issue_v(Int<S>{}, j + kStages);
        }
      }
    });
  }

  // With SUM_BY_MFMA the row sum sits in column d_v of the accumulator:
  // dv block VB - 1, register 4 * ((d_v % 32) / 8), lanes 0-31.
  constexpr int kSumReg = 4 * ((DV % 32) / 8);

  // ---- merge of the key-split waves (small launches) --------------------------
  // Wave w holds (m_w, l_w, acc_w) over its keys, with p = exp2(s c - m_w).
  // With M = max_w m_w and f_w = exp2(m_w - M) (0 for a wave that saw no
  // key), the unit's state is (M, sum_w f_w l_w, sum_w f_w acc_w).  The
  // stages are free once every wave has left its loop: the m and l of all
  // waves go through vs1 + 8 KB, then one d_v block of acc at a time through
  // vs0 (waves 1, 2) and vs1 (wave 3), 8 KB a wave, summed by wave 0.
  if (ksplit) {
    static_assert(kWaves == 4 && kWaves * C::V_TILE >= 16384, "merge layout: 2 x 8 KB in vs0, 8 + 4 KB in vs1");
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) float lds_f32;
    typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    lds_f32* ml = (lds_f32*)((lds_char*)vs1 + 8192);  // [wave][qb][m, l][lane]
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      ml[((wave * QB + qb) * 2 + 0) * 64 + lane] = m_run[qb];
      ml[((wave * QB + qb) * 2 + 1) * 64 + lane] = SUM_BY_MFMA ? 0.f : xhalf_sum(l_run[qb]);
    }
    lds_barrier();
    float f[QB], m_all[QB], l_all[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mw[kWaves];
#pragma unroll
      for (int w = 0; w < kWaves; ++w) mw[w] = ml[((w * QB + qb) * 2 + 0) * 64 + lane];
      m_all[qb] = fmaxf(fmaxf(mw[0], mw[1]), fmaxf(mw[2], mw[3]));
      l_all[qb] = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w)
        if (mw[w] != -INFINITY)
          l_all[qb] += ml[((w * QB + qb) * 2 + 1) * 64 + lane] * __builtin_amdgcn_exp2f(mw[w] - m_all[qb]);
      f[qb] = m_run[qb] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[qb] - m_all[qb]);
    }
    lds_f32x4* slot = (lds_f32x4*)(wave == 3 ? (lds_char*)vs1 : (lds_char*)vs0 + (wave == 2 ? 8192 : 0));
#pragma unroll
    for (int vb = 0; vb < C::VB; ++vb) {
      if (wave > 0) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const f32x16& a = acc[vb][qb];
            const f32x4 x = {a[4 * r4] * f[qb], a[4 * r4 + 1] * f[qb], a[4 * r4 + 2] * f[qb], a[4 * r4 + 3] * f[qb]};
            slot[(qb * 4 + r4) * 64 + lane] = x;
          }
      }
      lds_barrier();
      if (wave == 0) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int e = (qb * 4 + r4) * 64 + lane;
            const f32x4 x1 = ((lds_f32x4*)vs0)[e], x2 = ((lds_f32x4*)((lds_char*)vs0 + 8192))[e],
                        x3 = ((lds_f32x4*)vs1)[e];
#pragma unroll
            for (int t = 0; t < 4; ++t)
              acc[vb][qb][4 * r4 + t] = acc[vb][qb][4 * r4 + t] * f[qb] + ((x1[t] + x2[t]) + x3[t]);
          }
      }
      lds_barrier();
    }
    if (wave != 0) return;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      m_run[qb] = m_all[qb];
      l_run[qb] = g == 0 ? l_all[qb] : 0.f;  // the epilogue's xhalf_sum gives l_all
    }
  }

  // ---- epilogue (as the four-wave kernel's) -----------------------------------
  if (p.out_scale != nullptr) {
    const float os = 1.f / *p.out_scale;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float l = SUM_BY_MFMA ? from_lower_half(acc[C::VB - 1][qb][kSumReg]) : xhalf_sum(l_run[qb]);
      const int row = r0 + 32 * qb + l32;
      const float inv = l > 0.f ? os / l : 0.f;
      uint8_t* dst = (uint8_t*)p.o + (int64_t)(q0 + row) * p.o_row + (int64_t)h * p.o_head;
#pragma unroll
      for (int vb = 0; vb < C::VB; ++vb)
#pragma unroll
        for (int jp = 0; jp < 4; jp += 2) {
          const f32x16& a = acc[vb][qb];
          const uint32_t x = quant_e4m3x4(a[4 * jp], a[4 * jp + 1], a[4 * jp + 2], a[4 * jp + 3], inv);
          const uint32_t y = quant_e4m3x4(a[4 * jp + 4], a[4 * jp + 5], a[4 * jp + 6], a[4 * jp + 7], inv);
          const auto sw = __builtin_amdgcn_permlane32_swap(x, y, false, false);
          const int dv = vb * 32 + 8 * (jp + g);
          if (row < r1 && dv < DV) {
            const u32x2 o2 = {sw[0], sw[1]};
            *(u32x2*)(dst + dv) = o2;
          }
        }
      if (row < r1 && p.lse != nullptr && g == 0)
        p.lse[(int64_t)h * p.total_q + q0 + row] = l > 0.f ? (m_run[qb] + log2f(l)) * kLn2 : -INFINITY;
    }
    return;
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l = SUM_BY_MFMA ? from_lower_half(acc[C::VB - 1][qb][kSumReg]) : xhalf_sum(l_run[qb]);
    const int row = r0 + 32 * qb + l32;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    uint16_t* dst = p.o + (int64_t)(q0 + row) * p.o_row + (int64_t)h * p.o_head;
#pragma unroll
    for (int vb = 0; vb < C::VB; ++vb)
#pragma unroll
      for (int jp = 0; jp < 4; jp += 2) {
        const f32x16& a = acc[vb][qb];
        const uint32_t x0 = pack_bf16x2(a[4 * jp] * inv, a[4 * jp + 1] * inv);
        const uint32_t x1 = pack_bf16x2(a[4 * jp + 2] * inv, a[4 * jp + 3] * inv);
        const uint32_t y0 = pack_bf16x2(a[4 * jp + 4] * inv, a[4 * jp + 5] * inv);
        const uint32_t y1 = pack_bf16x2(a[4 * jp + 6] * inv, a[4 * jp + 7] * inv);
        const auto s0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
        const int dv = vb * 32 + 8 * (jp + g);
        if (row < r1 && dv < DV) {
          const u32x4 o4 = {s0[0], s1[0], s0[1], s1[1]};
          *(u32x4*)(dst + dv) = o4;
        }
      }
    if (row < r1 && p.lse != nullptr && g == 0)
      p.lse[(int64_t)h * p.total_q + q0 + row] = l > 0.f ? (m_run[qb] + log2f(l)) * kLn2 : -INFINITY;
  }
}

bool short_supported(int dqk, int dv) {
  return (dqk == 64 && dv == 64) || (dqk == 72 && dv == 72) || (dqk == 80 && dv == 80);
}

template <int DQK, int DV, RowSum SUM>
static Variant short_variant_of() {
  using C = narrow::Cfg<DQK, DV>;
  return {(const void*)&attn_fwd_short<DQK, DV, SUM>, narrow::kStages * narrow::kWaves * C::V_TILE, C::RPW,
          narrow::kBN, 64 * narrow::kWaves, "attn_fwd_short", 2, narrow::kWaves};
}

// `lse`: whether the caller asked for the LSE (d_v 72 / 80 without one sum
// the probabilities with the ones column, as the four-wave kernel does).
Variant short_variant(int dqk, int dv, bool lse) {
  (void)dv;
  constexpr RowSum F = RowSum::kF32, M = RowSum::kMfma;
  if (dqk == 64) return short_variant_of<64, 64, F>();
  if (dqk == 72) return lse ? short_variant_of<72, 72, F>() : short_variant_of<72, 72, M>();
  return lse ? short_variant_of<80, 80, F>() : short_variant_of<80, 80, M>();
}

Variant short_key_split_variant(int dqk, int dv, bool lse) {
  Variant v = short_variant(dqk, dv, lse);
  v.units_per_wg = 1;
  v.key_split = narrow::kWaves;
  return v;
}

}  // namespace va
