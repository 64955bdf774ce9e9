// Fused variable-length attention forward for AMD Instinct MI355X (gfx950).
//
// A workgroup owns a block of query rows of one (segment, head), 64 rows per
// wavefront, and walks the key tiles those rows can see (tile_schedule.h),
// 32 keys at a time:
//
//   HBM K/V tile --buffer_load ... lds (direct to LDS, out-of-range rows
//   read as zero)--> one of six LDS stages, issued four tiles ahead
//   --> S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (Q held in registers)
//   --> online softmax in registers (exp2 with a log2(e)-prescaled scale,
//       lazy rescale past a threshold)
//   --> O^T += V^T P^T on the same MFMA, V^T read with ds_read_b64_tr_b16
//   --> epilogue: O = acc / l in bf16, LSE = (m + log2 l) ln 2 in fp32.
//
// Scores are computed transposed (keys on the MFMA M axis, queries on N), so
// each lane holds one query column: the row max and row sum over the keys a
// lane holds are in-lane reductions with a single cross-lane step (lane l with
// lane l ^ 32).  The probability registers then serve directly as the B
// operand of the PV product, with the key order inside each 16-key group
// permuted identically on the V side.  Each LDS operand read feeds the MFMAs
// of a wave's two 32-row query blocks.
//
// Each wave software-pipelines its tiles: iteration j runs PV of tile j - 1
// and QK^T of tile j + 1 on the matrix cores, interleaved by hand with the
// softmax of tile j, whose exp does not wait for tile j's max (see
// fused_block in attn_fwd_wide).
//
// Variations on the same workgroup: grouped KV heads (query head h reads KV
// head h / (H / H_kv)); short segments packed four or two to a workgroup,
// one or two waves each, sharing the workgroup's key tiles (segments of at
// most 64 / 128 queries; at most 64 with head dims <= 80 go to the
// short-segment kernel of varlen_attn_short.hip instead); and split-KV,
// where a workgroup visits one run of its key tiles and writes an fp32
// partial that combine_splits (merge_states.hip) reduces.
//
// Where the pages describe FA4 on Blackwell (TMEM, tcgen05.ld.red row max,
// 2-CTA MMA) that design is prior art only; what carries over is the online
// softmax step with exp2 and a rescale threshold (SGLang PR #41344,
// "Modifications": softmax.py update_row_max, "fast exp2, rescale
// threshold") and masking only on the tiles that need it (same section: only
// unmasked steady-state tiles take the fast path).
#include <mutex>

#include "attn_common.h"
#include "wide_tile.h"

namespace va {

// ============================================================================
// The kernel: 4 waves x 64 query rows (BM = 256), 32-key tiles, six LDS
// stages.
//
// Each LDS operand read feeds two MFMAs (the wave's two 32-row query
// blocks), and each wave software-pipelines its own work: iteration j runs
// the PV product of tile j - 1 and QK^T of tile j + 1 on the matrix cores
// while the VALU computes the softmax of tile j.  Splitting the two among
// waves instead (one wave's softmax against another's MFMAs, ping-pong
// style) leaves the softmax to a single wave per SIMD, which issues VALU at
// roughly half the rate of two.
//
// The rescale of the accumulator, when the running max moves, is applied at
// the end of the iteration, after the PV MFMAs of tile j - 1 and before
// those of tile j, so the interleaved block has no branch.
//
// Each K/V stage is its own __shared__ object and the loop is unrolled by
// the stage count, so every LDS access names its stage statically: the
// compiler then tells LDS-DMA writes into one stage from transposing reads
// of another.  With one shared array it must assume they overlap and makes
// every V read wait for all DMA in flight (s_waitcnt vmcnt(0)).
// ============================================================================
namespace wide {
constexpr int kRowsPerWave = 64;     // query rows per wave (Cfg::RPW)
constexpr int kBN = 32;              // keys per tile
constexpr int kStages = 6;           // tile t lives in stage t % 6 (an even count: see the loop)
constexpr int kAhead = kStages - 2;  // iteration j issues tile j + 4
constexpr int kDepth = 3;            // LDS operands read ahead of their MFMA
// Four waves, 256-row blocks.  Head dims <= 80 fit a wave in 256 registers,
// so two workgroups share a CU (two waves per SIMD); 128 and 192/128 (whose
// 64-row accumulators, Q fragments and two score tiles need more) run one
// wave per SIMD.  256-row blocks measured faster than 512-row ones for
// every head dim: finer blocks balance ragged segment mixes better.
constexpr int kWaves = 4;
static_assert(kWaves == 4, "the packed set-up shifts wave indices by log2(4 / pack)");
template <int DQK, int DV>
struct Cfg : TileGeom<DQK, DV, kBN> {
  static constexpr int WAVES = kWaves;
  static constexpr int THREADS = 64 * WAVES;
  // Query rows per wave: QB blocks of 32, each a separate MFMA N block that
  // shares the wave's K and V operand reads.  Two for every head dim: head
  // dims <= 80 run two waves per SIMD, which leaves 256 registers a wave, and
  // a third block at 128 and 192/128 (one wave per SIMD) would need more
  // than the 512 a wave can have (the compiler spills hundreds).
  static constexpr int QB = 2;
  static constexpr int RPW = 32 * QB;
  static_assert(RPW == kRowsPerWave, "one row count per wave for every head dim");
  static constexpr int BM = RPW * WAVES;  // query rows per workgroup
  // Every wave issues NK K and NV V wave-loads per tile (zeros into a dummy
  // area where the tile has fewer), so LOADS per tile and wave is constant.
  static constexpr int NK = (Cfg::K_WL + WAVES - 1) / WAVES;
  static constexpr int NV = (Cfg::V_WL + WAVES - 1) / WAVES;
  static constexpr int LOADS = NK + NV;
  static constexpr int LDS_BYTES = kStages * (Cfg::K_TILE + Cfg::V_TILE) + 1024;
  // V chunks past the data (d_v 72, 80 padded to 96) are never loaded; they
  // are set once, and may hold a ones column (see attn_fwd_wide).
  static constexpr int V_PAD = Cfg::CPR_V - Cfg::V_REAL;
  static_assert(Cfg::CPR_V != 12 || v_swizzle<12>(1) == 0, "pad chunks sit at fixed positions");
};
}  // namespace wide




template <int DQK, int DV, RowSum SUM, int PK>
__global__ __launch_bounds__(64 * wide::kWaves, DQK <= 80 ? 2 : 1) void attn_fwd_wide(Params p) {
  using namespace wide;
  using C = Cfg<DQK, DV>;
  constexpr bool SUM_BY_MFMA = SUM == RowSum::kMfma;
  static_assert(!SUM_BY_MFMA || C::V_PAD > 0, "the ones column needs a padded d_v");
  static_assert(kStages == 6, "stage objects below");
  // The V stages are aligned more strictly than the K stages so the LDS
  // allocator places them first, below 64 KB: there a transposing read folds
  // its stage's address into the instruction's 16-bit offset instead of
  // building it with a VALU op.
  __shared__ __attribute__((aligned(1024))) char ks0[C::K_TILE];
  __shared__ __attribute__((aligned(1024))) char ks1[C::K_TILE];
  __shared__ __attribute__((aligned(1024))) char ks2[C::K_TILE];
  __shared__ __attribute__((aligned(1024))) char ks3[C::K_TILE];
  __shared__ __attribute__((aligned(1024))) char ks4[C::K_TILE];
  __shared__ __attribute__((aligned(1024))) char ks5[C::K_TILE];
  __shared__ __attribute__((aligned(4096))) char vs0[C::V_TILE];
  __shared__ __attribute__((aligned(4096))) char vs1[C::V_TILE];
  __shared__ __attribute__((aligned(4096))) char vs2[C::V_TILE];
  __shared__ __attribute__((aligned(4096))) char vs3[C::V_TILE];
  __shared__ __attribute__((aligned(4096))) char vs4[C::V_TILE];
  __shared__ __attribute__((aligned(4096))) char vs5[C::V_TILE];
  auto kst = [&](auto st) VA_INLINE -> lds_char* {
    constexpr int i = decltype(st)::value % kStages;
    if constexpr (i == 0) return (lds_char*)ks0;
    else if constexpr (i == 1) return (lds_char*)ks1;
    else if constexpr (i == 2) return (lds_char*)ks2;
    else if constexpr (i == 3) return (lds_char*)ks3;
    else if constexpr (i == 4) return (lds_char*)ks4;
    else return (lds_char*)ks5;
  };
  auto vst = [&](auto st) VA_INLINE -> lds_char* {
    constexpr int i = decltype(st)::value % kStages;
    if constexpr (i == 0) return (lds_char*)vs0;
    else if constexpr (i == 1) return (lds_char*)vs1;
    else if constexpr (i == 2) return (lds_char*)vs2;
    else if constexpr (i == 3) return (lds_char*)vs3;
    else if constexpr (i == 4) return (lds_char*)vs4;
    else return (lds_char*)vs5;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int g = lane >> 5;

  // Split-KV copy of the work units this workgroup belongs to (0 without split).
  const int split = (int)blockIdx.y;  // split-KV copy (0 without split)
  const BlockWork bw = block_work<PK>(p, lane, C::BM, (int64_t)blockIdx.x);
  if (!bw.u.valid) return;
  // Causal launches of the one-workgroup-per-CU head dims pair a segment's
  // q-tiles n_b - 1 - t and t in one workgroup (Params::pair_qt), so that
  // every workgroup runs as many key tiles: dispatched in order to the shader
  // engines in turn, workgroups of unequal length otherwise leave compute
  // units idle behind one headed for an engine whose units are all busy.
  // The longer q-tile runs first.  (Head dims <= 80 share a CU between two
  // workgroups, which absorbs that, and have no registers to spare for the
  // loop.)
  constexpr bool kPairs = DQK > 80 && PK == kPackNone;
  int qt_first = bw.u.qt, qt_second = -1;
  if (kPairs && p.pair_qt) {
    const int nb = (bw.lq + C::BM - 1) / C::BM, t = bw.u.qt;
    if (nb - 1 - t < t) return;
    qt_first = nb - 1 - t;
    qt_second = nb - 1 - t > t ? t : -1;
  }
  const int n_runs = kPairs && qt_second >= 0 ? 2 : 1;
#pragma clang loop unroll(disable)
  for (int rep = 0; rep < n_runs; ++rep) {
    if (rep > 0) lds_barrier();  // every wave is done reading the previous q-tile's stages
    int h = bw.u.h;
    const int qt = rep == 0 ? qt_first : qt_second;
    const int k0 = bw.k0, Lk = bw.lk;  // the workgroup's keys
    const int r0 = qt * C::BM;
    if (r0 >= bw.lq) continue;
    constexpr bool packed = PK == kPackSegments;
    // This wave's rows: rows [wrow0, r1) of a segment whose first query row is
    // q0 and whose Lq queries see its Lk keys, found at key wkoff of the
    // workgroup's keys.  One segment: rows r0 + 64 wave on, wkoff = 0.  Packed
    // short segments: wave w takes segment pack * group + w / (4 / pack), rows
    // 64 (w % (4 / pack)) on (a wave past the last segment has no rows).
    int q0 = bw.q0, Lq = bw.lq, wLk = Lk, wkoff = 0, wrow0 = r0 + wave * C::RPW;
    int r1 = min(r0 + C::BM, Lq);
    if constexpr (packed) {
      const int per = C::WAVES >> p.pack_shift;
      const int seg = (bw.u.b << p.pack_shift) + (wave >> (2 - p.pack_shift));
      wrow0 = (wave & (per - 1)) * C::RPW;
      q0 = Lq = wLk = wkoff = r1 = 0;
      if (seg < p.batch) {
        q0 = p.cu_q[seg];
        Lq = p.cu_q[seg + 1] - q0;
        wkoff = p.cu_k[seg] - k0;
        wLk = p.cu_k[seg + 1] - k0 - wkoff;
        r1 = Lq;
      }
    }
    // The key tiles this workgroup visits: all its rows see (packed: all of
    // its keys, every tile masked), or with split-KV the split-th of
    // num_splits runs of them (possibly empty).
    if constexpr (PK == kPackHeads) {
      // Query head h + wave / (4 / pack), rows 64 (wave % (4 / pack)) on, of the
      // one segment (r0 = 0): the workgroup's tiles are an unpacked unit's.
      const int per = C::WAVES >> p.pack_shift;
      h += wave >> (2 - p.pack_shift);
      wrow0 = (wave & (per - 1)) * C::RPW;
    }
    TileRange tr0;
    if constexpr (packed) {
      tr0.kt_begin = tr0.full_begin = tr0.full_end = 0;
      tr0.kt_end = (Lk + kBN - 1) / kBN;
    } else {
      tr0 = tile_range(Lq, Lk, r0, r1, p.causal, p.wl, p.wr, kBN);
    }
    // Split-KV with per-segment split counts: this segment's units take
    // min(max(count, 1), num_splits) runs; copies past that have no work.
    int n_splits = p.num_splits;
    if constexpr (PK != kPackSegments) {  // (a unit holds one segment; the host never packs segments then)
      if (p.splits_dyn != nullptr) {
        n_splits = min(max(p.splits_dyn[bw.u.b], 1), p.num_splits);
        if (split >= n_splits) continue;
      }
    }
    const TileRange tr = split_range(tr0, split, n_splits);
    const int ntiles = tr.kt_end - tr.kt_begin;
    // ---- Q fragments (B operand of S^T = K Q^T) -----------------------------
    // For head dims <= 80, buffer loads over this wave's rows [wrow0, r1):
    // rows past r1 (and the head-dim padding of d 72) read as zero, with no
    // branch per load.  (At 128 and 192 the compiler then allocates the main
    // loop's registers worse, measured 7% slower on MLA; those keep plain
    // loads under a row check.)
    bf16x8 qf[C::QB][C::KC];
    if constexpr (DQK > 80) {
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb) {
        const int row = wrow0 + 32 * qb + l32;
        const uint16_t* src = p.q + (int64_t)(q0 + row) * p.q_row + (int64_t)h * p.q_head;
#pragma unroll
        for (int c = 0; c < C::KC; ++c) {
          const int d = c * 16 + 8 * g;
          u32x4 x = {0u, 0u, 0u, 0u};
          if (row < r1) x = *(const u32x4*)(src + d);
          qf[qb][c] = __builtin_bit_cast(bf16x8, x);
        }
      }
    } else {
      const int64_t q_row_b = p.q_row * 2;
      const int vrows = __builtin_amdgcn_readfirstlane(max(min(r1 - wrow0, C::RPW), 0));
      const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(p.q + (int64_t)(q0 + wrow0) * p.q_row + (int64_t)h * p.q_head), (short)0,
          (int)(uint32_t)(vrows * q_row_b), kBufferFlags);
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb) {
        const uint32_t row_off = (uint32_t)((32 * qb + l32) * q_row_b);
#pragma unroll
        for (int c = 0; c < C::KC; ++c) {
          const int d = c * 16 + 8 * g;
          const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rq, d < DQK ? row_off + 2 * d : kOOB, 0, 0);
          qf[qb][c] = __builtin_bit_cast(bf16x8, x);
        }
      }
    }

    // ---- direct-to-LDS tile loads ---------------------------------------------
    // A tile is K_WL K wave-loads then V_WL V wave-loads, each 64 lanes x 16
    // bytes: K wave-load i covers K slots [64 i, 64 i + 64), likewise for V.
    // Wave w issues K wave-loads w + WAVES x (x < NK) and V wave-loads
    // w + WAVES x (x < NV) every tile; where such a wave-load does not exist
    // it reads zeros into a dummy area instead, so every wave issues LOADS
    // loads per tile and every wait below is a constant.  K pad chunks, chunk
    // 9 of a 72-wide row and slots past the tile read zeros; lanes on padded V
    // chunks load nothing.
    __shared__ __attribute__((aligned(1024))) char dummy[1024];
    const int64_t k_row_b = p.k_row * 2, v_row_b = p.v_row * 2;
    uint32_t k_off[C::NK], v_off[C::NV];
    bool v_on[C::NV];
#pragma unroll
    for (int x = 0; x < C::NK; ++x) {
      const int i = wave + C::WAVES * x;
      const int sl = i * 64 + lane;
      const int row = sl / C::KPITCH, c = sl % C::KPITCH;
      k_off[x] = (i < C::K_WL && sl < C::K_SLOTS && c < C::K_REAL) ? (uint32_t)(row * k_row_b + c * 16) : kOOB;
    }
#pragma unroll
    for (int x = 0; x < C::NV; ++x) {
      const int i = wave + C::WAVES * x;
      const int sl = i * 64 + lane;
      const int row = sl / C::CPR_V;
      const int c = (sl % C::CPR_V) ^ v_swizzle<C::CPR_V>(row);
      v_on[x] = i >= C::V_WL || sl >= C::V_SLOTS || c < C::V_REAL;
      v_off[x] = (i < C::V_WL && sl < C::V_SLOTS && c < C::V_REAL) ? (uint32_t)(row * v_row_b + c * 16) : kOOB;
    }
    // K/V rows of the next tile to issue, advanced one tile per issue; tiles
    // past the workgroup's last (tr.kt_end, which for a causal q-tile is its
    // diagonal, not the segment's end) get an empty range, so the prefetches
    // past it read zeros instead of keys no row sees.
    const int hk = (int)fdiv((uint32_t)h, p.fd_group);  // the KV head query head h reads
    const char* k_next =
        (const char*)(p.k + ((int64_t)k0 + (int64_t)tr.kt_begin * kBN) * p.k_row + (int64_t)hk * p.k_head);
    const char* v_next =
        (const char*)(p.v + ((int64_t)k0 + (int64_t)tr.kt_begin * kBN) * p.v_row + (int64_t)hk * p.v_head);
    int keys_next = min(Lk, tr.kt_end * kBN) - tr.kt_begin * kBN;
    auto issue = [&](auto st) VA_INLINE {  // this wave's loads of the next tile into stage st
      // (readfirstlane: the clamp compiles to a VALU med3, and a descriptor
      // the compiler cannot prove uniform costs a waterfall loop per load)
      const int rows = __builtin_amdgcn_readfirstlane(max(min(keys_next, kBN), 0));
      const __amdgpu_buffer_rsrc_t rk =
          __builtin_amdgcn_make_buffer_rsrc((void*)k_next, (short)0, (int)(rows * k_row_b), kBufferFlags);
      const __amdgpu_buffer_rsrc_t rv =
          __builtin_amdgcn_make_buffer_rsrc((void*)v_next, (short)0, (int)(rows * v_row_b), kBufferFlags);
#pragma unroll
      for (int x = 0; x < C::NK; ++x) {
        const int i = wave + C::WAVES * x;
        dma16(rk, i < C::K_WL ? kst(st) + i * 1024 : (lds_char*)dummy, k_off[x]);
      }
#pragma unroll
      for (int x = 0; x < C::NV; ++x) {
        const int i = wave + C::WAVES * x;
        if (v_on[x]) dma16(rv, i < C::V_WL ? vst(st) + i * 1024 : (lds_char*)dummy, v_off[x]);
      }
      k_next += kBN * k_row_b;
      v_next += kBN * v_row_b;
      keys_next -= kBN;
    };
    // Every iteration issues LOADS loads per wave, and loads complete in issue
    // order: "tile t landed" with the loads of n later tiles in flight is
    // s_waitcnt vmcnt(n LOADS).
    auto wait_landed = [&](auto later_tiles) VA_INLINE {
      constexpr int n = C::LOADS * decltype(later_tiles)::value;
      static_assert(n < 64, "vmcnt range");
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(n) : "memory");
    };

    // The Q and first tiles' loads go out before the rest of the set-up, which
    // then runs under their latency.
    if (ntiles > 0) static_for<0, kAhead>([&](auto t) VA_INLINE { issue(t); });  // tiles 0-3

    // Each wave's own key-tile range (its 64 rows see a sub-range of the
    // workgroup's).  Iteration w_end, whose tile none of the wave's rows sees
    // (masked to zero probabilities, so the running max and sum stay put and
    // the slow path cannot trigger), still runs for the PV of tile w_end - 1;
    // after it the wave only issues its share of the loads and meets the
    // barriers.  Its own unmasked sub-range spares it the mask on tiles all its
    // rows see.  Waves past the segment's last row compute nothing.
    int w_beg = 0, w_end = 0, w_full_begin = 0, w_full_end = 0;  // relative to tr.kt_begin
    if (wrow0 < r1) {
      const TileRange wt =
          tile_range(Lq, wLk, wrow0, min(wrow0 + C::RPW, r1), p.causal, p.wl, p.wr, kBN, wkoff);
      // (clamped to this workgroup's tiles, which with split-KV are a run of
      // the rows' tiles)
      w_beg = min(max(wt.kt_begin, tr.kt_begin), tr.kt_end) - tr.kt_begin;
      w_end = min(max(wt.kt_end, tr.kt_begin), tr.kt_end) - tr.kt_begin;
      w_full_begin = min(max(wt.full_begin, tr.kt_begin), tr.kt_end) - tr.kt_begin;
      w_full_end = min(max(wt.full_end, tr.kt_begin), tr.kt_end) - tr.kt_begin;
    }
    const bool active = w_end > w_beg;
    // A wave computes iterations w_beg - 1 .. w_end: before its first tile it
    // only issues its share of the loads and meets the barriers (with short
    // segments packed into one workgroup, or a left window, the later waves'
    // keys start later).  Iteration w_beg - 1 computes QK^T of tile w_beg
    // (with the PV of tile w_beg - 2 on the zero probabilities below, and
    // the softmax of the fully masked tile w_beg - 1, which changes nothing).
    const int w_first = w_beg > 0 ? w_beg - 1 : 0;


    // ---- padded V chunks: zeros, or a one in column d_v ------------------------
    if constexpr (C::V_PAD > 0) {
      static_for<0, kStages>([&](auto st) VA_INLINE {
        for (int i = tid; i < kBN * C::V_PAD; i += C::THREADS) {
          const int row = i / C::V_PAD, c = C::V_REAL + i % C::V_PAD;
          const u32x4 val = {(SUM_BY_MFMA && c == C::V_REAL) ? 0x3F80u : 0u, 0u, 0u, 0u};  // bf16 1.0
          *(__attribute__((address_space(3))) u32x4*)(vst(st) + (row * C::CPR_V + c) * 16) = val;
        }
      });
    }

    // ---- LDS operand reads ----------------------------------------------------
    const int k_rd = (l32 * C::KPITCH + g) * 16;  // K row l32, chunk 2c + g at + 32c
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
    f32x16 acc[C::VB][C::QB];
#pragma unroll
    for (int vb = 0; vb < C::VB; ++vb)
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[vb][qb][r] = 0.f;
    float m_run[C::QB], nm[C::QB], lim[C::QB], l_run[C::QB];
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) {
      m_run[qb] = -INFINITY;  // running max of s * scale * log2(e)
      nm[qb] = 0.f;           // -m_run, or 0 while m_run is -inf
      lim[qb] = -FLT_MAX;     // m_run + kRescaleTau, or -FLT_MAX while m_run is -inf
      l_run[qb] = 0.f;        // fp32 row sum (unless SUM_BY_MFMA)
    }
    int row_lo[C::QB], row_hi[C::QB];
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) {
      const RowBounds rb = row_bounds(wrow0 + 32 * qb + l32, Lq, wLk, p.causal, p.wl, p.wr);
      row_lo[qb] = wkoff + (int)imin64(rb.lo, (int64_t)wLk);
      row_hi[qb] = wkoff + (int)imax64(rb.hi, (int64_t)-1);
    }
    // Iteration (relative key tile) holding each row's first visible key, or
    // -1 for a row that sees none: there the fast path cannot run (see
    // fused_block).
    int first_j[C::QB];
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb)
      first_j[qb] = row_lo[qb] <= row_hi[qb] ? row_lo[qb] / kBN - tr.kt_begin : -1;
    // Scores of two tiles (the one in the softmax and the next, which QK^T is
    // writing): sbuf[t % 2][qb][r] = key 8 (r / 4) + 4 g + r % 4, query l32.
    f32x16 sbuf[2][C::QB];
    // Probabilities, the PV B operand per (qb, 16-key half); zero until a
    // wave's first computed tile, whose PV of the previous tile then adds
    // nothing.
    bf16x8 pf[C::QB][2];
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) pf[qb][0] = pf[qb][1] = bf16x8{};

    // QK^T of one tile on its own (tile 0 and the next, and the slow path):
    // KC K operands into sn, each LDS operand feeding both query blocks,
    // operands read kDepth ahead into a ring of registers.
    auto qk_only = [&](const lds_char* ks, f32x16 (&sn)[C::QB]) VA_INLINE {
      const f32x16 zero = {};
      bf16x8 ring[kDepth];
#pragma unroll
      for (int i = 0; i < kDepth && i < C::KC; ++i) ring[i] = lds_read_b128(ks, k_rd + 32 * i);
#pragma unroll
      for (int c = 0; c < C::KC; ++c) {
        const bf16x8 op = ring[c % kDepth];
        if (c + kDepth < C::KC) ring[c % kDepth] = lds_read_b128(ks, k_rd + 32 * (c + kDepth));
#pragma unroll
        for (int qb = 0; qb < C::QB; ++qb)
          sn[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, qf[qb][c], c == 0 ? zero : sn[qb], 0, 0, 0);
      }
    };
    // Boundary tiles only: scores of keys a row may not see become -inf.
    auto mask = [&](int j, f32x16 (&s)[C::QB]) VA_INLINE {
      const int kt = tr.kt_begin + j;
      if ((unsigned)(j - w_full_begin) >= (unsigned)(w_full_end - w_full_begin)) {  // j outside [begin, end)
        const int key0 = kt * kBN;
#pragma unroll
        for (int qb = 0; qb < C::QB; ++qb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int jj = key0 + 8 * (r >> 2) + 4 * g + (r & 3);
            s[qb][r] = (jj >= row_lo[qb] && jj <= row_hi[qb]) ? s[qb][r] : -INFINITY;
          }
      }
    };
    // Online softmax of one tile, branch-free: row max, the lazy-rescale
    // decision (the running max moves only when some row's max grew by more
    // than kRescaleTau, in log2 units; then every row of the wave moves),
    // p = exp2(s * scale * log2(e) - m), row sum, bf16 pack into pf.  Returns
    // whether acc must be rescaled, with alpha per query block.
    auto softmax = [&](f32x16 (&s)[C::QB], float (&alpha)[C::QB]) VA_INLINE -> bool {
      float m_new[C::QB];
      bool need = false;
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb) {
        float m = fmaxf(fmaxf(s[qb][0], s[qb][1]), s[qb][2]);
#pragma unroll
        for (int r = 3; r < 15; r += 2) m = fmaxf(fmaxf(m, s[qb][r]), s[qb][r + 1]);
        m = fmaxf(m, s[qb][15]);
        m_new[qb] = fmaxf(m_run[qb], xhalf_max(m) * p.scale_log2);
        need |= m_new[qb] > m_run[qb] + kRescaleTau;
      }
      const bool move = __any(need);
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb) {
        const float m_next = move ? m_new[qb] : m_run[qb];
        alpha[qb] = (m_next == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run[qb] - m_next);
        m_run[qb] = m_next;
        nm[qb] = (m_next == -INFINITY) ? 0.f : -m_next;
        lim[qb] = (m_next == -INFINITY) ? -FLT_MAX : m_next + kRescaleTau;
      }
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb) {
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
    // One iteration's MFMAs and fast-path softmax, interleaved by hand.
    //
    // The fast path needs nothing of this tile's max: p = exp2(s * scale *
    // log2(e) - m_run) with the running max as it stands, in place, packed to
    // bf16, and a check that this was valid: every p <= 2^kRescaleTau (the
    // tile's max exceeds m_run by at most kRescaleTau, so the lazy rescale
    // would not have moved the max either) and no row saw its first visible
    // key (while m_run is -inf, p is not relative to any max yet).  With a
    // row sum in registers (kF32) the first condition is read off the
    // tile's row sum (sum <= 2^kRescaleTau bounds every term), so no row max
    // is taken; with the ones-column sum (kMfma) the row max is taken on the
    // raw scores as before.  The row sums go to sum[], committed by the caller
    // only if the check passed.
    //
    // Its VALU work is 80 or 96 units in dependency order: (16 row-max steps,
    // 8 per query block, on the raw scores, kMfma only), 32 scale-and-shift
    // FMAs, 32 in-place exps, 16 packs (+ sums).  The MFMAs (PV of the
    // previous tile, then QK^T of the next, two per LDS operand) each get an
    // even share of the units, in
    // source order pinned by scheduling barriers: the compiler's own schedule
    // bunches the MFMAs, and an MFMA hides only a few VALU ops behind it.  The
    // packs, which overwrite the probabilities PV reads, all fall after the
    // last PV MFMA.
    auto fused_block = [&](const lds_char* vs, const lds_char* ks, f32x16 (&s)[C::QB], f32x16 (&sn)[C::QB],
                           float (&sum)[C::QB], int j) VA_INLINE -> bool {
      constexpr bool kMaxCheck = SUM_BY_MFMA;
      constexpr int QB = C::QB;
      constexpr int kPVOps = 2 * C::VB, kOps = kPVOps + C::KC, kSlots = QB * kOps;
      // The scale-and-shift FMAs run as units of their own, all before the
      // exps, rather than each with its exp (measured +1% on the ViT batch and
      // the MLA prefill, +0.4% on d 128, bit-identical).
      constexpr int kMaxU = 8 * QB, kFmaU = 16 * QB, kExpU = 16 * QB, kPackU = 8 * QB;  // units per kind
      constexpr int kUnits = (kMaxCheck ? kMaxU : 0) + kFmaU + kExpU + kPackU;
      static_assert((kUnits - kPackU) * kSlots / kUnits >= QB * kPVOps, "packs must follow the PV MFMAs");
      float m[QB];
      bool bad = false;
      if constexpr (!kMaxCheck)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) bad |= j == first_j[qb];
      u32x4 pk[QB][2];
      auto unit = [&](auto uu) VA_INLINE {
        constexpr int u = decltype(uu)::value + (kMaxCheck ? 0 : kMaxU);
        if constexpr (u < kMaxU) {  // row max, 8 steps per query block
          constexpr int qb = u / 8, st = u % 8;
          if constexpr (st == 0) {
            m[qb] = fmaxf(fmaxf(s[qb][0], s[qb][1]), s[qb][2]);
          } else if constexpr (st < 7) {
            m[qb] = fmaxf(fmaxf(m[qb], s[qb][2 * st + 1]), s[qb][2 * st + 2]);
          } else {
            m[qb] = fmaxf(m[qb], s[qb][15]);
            bad |= m[qb] * p.scale_log2 > lim[qb];
          }
        } else if constexpr (u < kMaxU + kFmaU) {  // s * scale - m_run, in place
          constexpr int qb = (u - kMaxU) / 16, r = (u - kMaxU) % 16;
          s[qb][r] = fmaf(s[qb][r], p.scale_log2, nm[qb]);
        } else if constexpr (u < kMaxU + kFmaU + kExpU) {  // p = exp2(s * scale - m_run), in place
          constexpr int qb = (u - kMaxU - kFmaU) / 16, r = (u - kMaxU - kFmaU) % 16;
          s[qb][r] = __builtin_amdgcn_exp2f(s[qb][r]);
        } else {  // bf16 pack (and row sum)
          constexpr int i = u - kMaxU - kFmaU - kExpU, qb = i / 8, t = (i / 4) % 2, e = i % 4, r = 8 * t + 2 * e;
          constexpr bool first = t == 0 && e == 0;
          pk[qb][t][e] = pack_bf16x2(s[qb][r], s[qb][r + 1]);
          if constexpr (SUM == RowSum::kF32) {
            const float pair = s[qb][r] + s[qb][r + 1];
            sum[qb] = first ? pair : sum[qb] + pair;
          }
          if constexpr (e == 3) pf[qb][t] = __builtin_bit_cast(bf16x8, pk[qb][t]);
          if constexpr (!kMaxCheck && t == 1 && e == 3) bad |= !(sum[qb] <= kSumLimit);
        }
      };
      auto load_op = [&](auto ii, bf16x8& dst) VA_INLINE {
        constexpr int i = decltype(ii)::value;
        if constexpr (i < kPVOps) {  // V^T operand (t, vb) of PV
          constexpr int t = i / C::VB, vb = i % C::VB;
          const bf16x4 lo = lds_read_tr(vs, v_rd[vb] + (16 * t) * C::CPR_V * 16);
          const bf16x4 hi = lds_read_tr(vs, v_rd[vb] + (16 * t + 8) * C::CPR_V * 16);
          dst = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        } else {  // K operand i - kPVOps of QK^T
          dst = lds_read_b128(ks, k_rd + 32 * (i - kPVOps));
        }
      };
      const f32x16 zero = {};
      bf16x8 ring[kDepth];
      static_for<0, kDepth>([&](auto ii) VA_INLINE { load_op(ii, ring[decltype(ii)::value]); });
      static_for<0, kOps>([&](auto oo) VA_INLINE {
        constexpr int i = decltype(oo)::value;
        const bf16x8 op = ring[i % kDepth];
        if constexpr (i + kDepth < kOps) load_op(Int<i + kDepth>{}, ring[i % kDepth]);
        static_for<0, QB>([&](auto qq) VA_INLINE {
          constexpr int qb = decltype(qq)::value, slot = QB * i + qb;
          if constexpr (i < kPVOps) {
            constexpr int t = i / C::VB, vb = i % C::VB;
            acc[vb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, pf[qb][t], acc[vb][qb], 0, 0, 0);
          } else {
            constexpr int c = i - kPVOps;
            sn[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, qf[qb][c], c == 0 ? zero : sn[qb], 0, 0, 0);
          }
          static_for<slot * kUnits / kSlots, (slot + 1) * kUnits / kSlots>(unit);
          __builtin_amdgcn_sched_barrier(0);
        });
      });
      return __any(bad);
    };
    // acc *= alpha, after the PV MFMAs of the previous tile (rare).
    auto rescale = [&](bool move, const float (&alpha)[C::QB]) VA_INLINE {
      if (move) {
        asm volatile("; lazy rescale" ::: "memory");  // keep the rare rescale a branch
#pragma unroll
        for (int qb = 0; qb < C::QB; ++qb)
#pragma unroll
          for (int vb = 0; vb < C::VB; ++vb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[vb][qb][r] *= alpha[qb];
      }
    };

    // ---- main loop ----------------------------------------------------------------
    // Iteration j: issue tile j + 4; MFMAs of PV(j - 1) and QK^T(j + 1) with
    // the softmax of tile j; rescale; wait for this wave's share of tile j + 2;
    // barrier.  Tile t sits in stage t % 6, which last held tile t - 6: its K
    // was last read in iteration t - 7, its V in iteration t - 5, both before
    // iteration t - 4 issues tile t.  Tile j + 2 (read by iteration j + 1's
    // QK^T) is waited for at the end of iteration j, three iterations after
    // its issue.  Every iteration issues, past the last tile too (zeros), so
    // the waits are constants; QK^T of tile ntiles in the last iteration reads
    // such zeros, already landed, and its result is never used.
    //
    // Iteration j's softmax reads sbuf[j % 2] and QK^T writes sbuf[(j + 1) % 2];
    // the loop is unrolled by the (even) stage count so both are static.
    // PV of one tile on its own (the workgroup's last tile).
    auto pv_tile = [&](const lds_char* vs) VA_INLINE {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int vb = 0; vb < C::VB; ++vb) {
          const bf16x4 lo = lds_read_tr(vs, v_rd[vb] + (16 * t) * C::CPR_V * 16);
          const bf16x4 hi = lds_read_tr(vs, v_rd[vb] + (16 * t + 8) * C::CPR_V * 16);
          const bf16x8 vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
          for (int qb = 0; qb < C::QB; ++qb)
            acc[vb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qb][t], acc[vb][qb], 0, 0, 0);
        }
    };
    if (ntiles > 0) {
      wait_landed(Int<kAhead - 1>{});  // tile 0 (tiles 0-3 were issued above)
      lds_barrier();
      if (active && w_beg == 0) qk_only(kst(Int<0>{}), sbuf[0]);  // QK^T(0)
      wait_landed(Int<kAhead - 2>{});  // tile 1
      lds_barrier();
      // iteration 0 (no PV before it)
      {
        issue(Int<kAhead % kStages>{});
        if (active && w_first == 0) {
          mask(0, sbuf[0]);
          qk_only(kst(Int<1>{}), sbuf[1]);
          float alpha[C::QB];
          const bool move = softmax(sbuf[0], alpha);
          rescale(move, alpha);
        }
        wait_landed(Int<kAhead - 2>{});  // tile 2
        lds_barrier();
      }
      for (int j0 = 1; j0 < ntiles; j0 += kStages) {  // tile j0 + u sits in stage (u + 1) % 6
        static_for<0, kStages>([&](auto u) VA_INLINE {
          constexpr int U = decltype(u)::value;
          const int j = j0 + U;
          if (U == 0 || j < ntiles) {
            issue(Int<(U + 1 + kAhead) % kStages>{});  // tile j + 4 (zeros past the last)
            if (active && j <= w_end && j >= w_first) {
              constexpr int cur = (U + 1) % 2;  // j % 2, j0 being odd
              mask(j, sbuf[cur]);
              float sum[C::QB];
              const bool slow = fused_block(vst(Int<U % kStages>{}), kst(Int<(U + 2) % kStages>{}), sbuf[cur],
                                            sbuf[cur ^ 1], sum, j);
              // The probabilities are only read in the next iteration and the
              // row sums only on the fast path; without these uses the compiler
              // sinks their computation past the branch below, out of the
              // interleave, where nothing hides it.
#pragma unroll
              for (int qb = 0; qb < C::QB; ++qb) {
                asm volatile("" ::"v"(pf[qb][0]), "v"(pf[qb][1]));
                if constexpr (!SUM_BY_MFMA) asm volatile("" ::"v"(sum[qb]));
              }
              // Commit the row sums on one path (the slow path restores them):
              // two paths merging into l_run cost the register allocator dearly.
              float l_prev[C::QB];
#pragma unroll
              for (int qb = 0; qb < C::QB; ++qb) {
                l_prev[qb] = l_run[qb];
                if constexpr (!SUM_BY_MFMA) l_run[qb] += sum[qb];
              }
              if (slow) {
                // Some row's max moved past m_run + kRescaleTau (or a row saw
                // its first key): recompute this tile's scores from K, still
                // in its stage, and take the full softmax with the rescale.
                asm volatile("; softmax slow path" ::: "memory");
#pragma unroll
                for (int qb = 0; qb < C::QB; ++qb) l_run[qb] = l_prev[qb];
                qk_only(kst(Int<(U + 1) % kStages>{}), sbuf[cur]);
                mask(j, sbuf[cur]);
                float alpha[C::QB];
                const bool move = softmax(sbuf[cur], alpha);
                rescale(move, alpha);
              }
            }
            wait_landed(Int<kAhead - 2>{});  // tile j + 2
            lds_barrier();
          }
        });
      }
      // The zero loads past the last tile must land before the workgroup's LDS
      // can be handed to the next workgroup.
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (active && w_end == ntiles) {  // PV of the last tile, its stage picked at run time (all DMA has landed)
        const int last = (ntiles - 1) % kStages;
        const lds_char* vs = vst(Int<0>{});
        static_for<1, kStages>([&](auto st) VA_INLINE {
          if (last == decltype(st)::value) vs = vst(st);
        });
        pv_tile(vs);
      }
    }

    // ---- epilogue ---------------------------------------------------------------
    // With SUM_BY_MFMA the row sum sits in column d_v of the accumulator:
    // dv block VB - 1, register 4 * ((d_v % 32) / 8), lanes 0-31.
    constexpr int kSumReg = 4 * ((DV % 32) / 8);
    if (p.num_splits > 1) {
      // Split-KV partial: O = acc / l in fp32 (lane (row, g) holds d_v 8 jj +
      // 4 g .. + 3 of each 32-wide block: one 16-byte store each) and the LSE of
      // this split's keys (-inf where a row saw none of them).
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb) {
        const float l = SUM_BY_MFMA ? from_lower_half(acc[C::VB - 1][qb][kSumReg]) : xhalf_sum(l_run[qb]);
        const int row = wrow0 + 32 * qb + l32;
        const float inv = l > 0.f ? 1.f / l : 0.f;
        float* dst = p.part_o + (((int64_t)split * p.total_q + q0 + row) * p.heads + h) * DV;
#pragma unroll
        for (int vb = 0; vb < C::VB; ++vb)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int dv = vb * 32 + 8 * jj + 4 * g;
            if (row < r1 && dv < DV) {
              const f32x16& a = acc[vb][qb];
              typedef float f32x4 __attribute__((ext_vector_type(4)));
              const f32x4 o4 = {a[4 * jj] * inv, a[4 * jj + 1] * inv, a[4 * jj + 2] * inv, a[4 * jj + 3] * inv};
              *(f32x4*)(dst + dv) = o4;
            }
          }
        if (row < r1 && g == 0)
          p.part_lse[((int64_t)split * p.heads + h) * p.total_q + q0 + row] =
              l > 0.f ? (m_run[qb] + log2f(l)) * kLn2 : -INFINITY;
      }
      continue;
    }
    // Lane (row, g) holds d_v 8 jj + 4 g .. + 3 of its row for jj = 0..3 of
    // each 32-wide block.  Swapping halves with lane row ^ 32 over a pair of
    // chunks (jj, jj + 1) leaves lane g with the 8 contiguous values of chunk
    // jj + g: one 16-byte store instead of two 8-byte ones per lane.
    // With an output scale (varlen_attn_fwd_quant_out) the same values leave as
    // e4m3 codes of O / out_scale, 8 bytes a lane.
    if (p.out_scale != nullptr) {
      const float os = 1.f / *p.out_scale;
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb) {
        const float l = SUM_BY_MFMA ? from_lower_half(acc[C::VB - 1][qb][kSumReg]) : xhalf_sum(l_run[qb]);
        const int row = wrow0 + 32 * qb + l32;
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
      continue;
    }
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) {
      const float l = SUM_BY_MFMA ? from_lower_half(acc[C::VB - 1][qb][kSumReg]) : xhalf_sum(l_run[qb]);
      const int row = wrow0 + 32 * qb + l32;
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
      if (row < r1) {
        if (p.lse != nullptr && g == 0) {
          const float lse = l > 0.f ? (m_run[qb] + log2f(l)) * kLn2 : -INFINITY;
          p.lse[(int64_t)h * p.total_q + q0 + row] = lse;
        }
      }
    }
  }
}

}  // namespace va

// ============================================================================
// Host side: validation, launch-shape choice and the C entry points.
// ============================================================================
namespace va {

// One kernel, one instantiation per head-dim pair (and, for d_v 72/80, per
// whether the LSE is returned): 4 waves x 64 query rows, 256-row blocks.
template <int DQK, int DV, RowSum SUM>
static Variant wide_variant(int mode) {
  using C = wide::Cfg<DQK, DV>;
  const void* fn = mode == kPackHeads      ? (const void*)&attn_fwd_wide<DQK, DV, SUM, kPackHeads>
                   : mode == kPackSegments ? (const void*)&attn_fwd_wide<DQK, DV, SUM, kPackSegments>
                                           : (const void*)&attn_fwd_wide<DQK, DV, SUM, kPackNone>;
  return {fn, C::LDS_BYTES, C::BM, wide::kBN, C::THREADS, "attn_fwd_wide", DQK <= 80 ? 2 : 1, 1};
}

static bool supported_dims(int dqk, int dv) {
  return (dqk == 64 && dv == 64) || (dqk == 72 && dv == 72) || (dqk == 80 && dv == 80) ||
         (dqk == 128 && dv == 128) || (dqk == 192 && dv == 128);
}

// How a launch fills its workgroups (tile_schedule.h, pack_mode); with
// per-segment split counts (split-KV with num_splits_dynamic) a workgroup
// must hold one segment, so short segments are not packed together then.
static int32_t launch_mode(int64_t max_seqlen_q, int64_t heads, int64_t heads_k, bool segment_packing = true) {
  const int32_t mode = pack_mode(max_seqlen_q, wide::kRowsPerWave, heads, heads_k);
  return (mode == kPackSegments && !segment_packing) ? (int32_t)kPackNone : mode;
}

// `lse`: whether the caller asked for the LSE (without one the row sum is
// taken over the bf16 probabilities, see RowSum; the launch shape is the same
// either way).  Short segments take a packed instantiation (launch_mode); the
// unpacked one carries none of its set-up.
static Variant variant_for(int dqk, int dv, int32_t pk, bool lse = true) {
  (void)dv;
  constexpr RowSum F = RowSum::kF32, M = RowSum::kMfma;
  if (dqk == 64) return wide_variant<64, 64, F>(pk);
  if (dqk == 72) return lse ? wide_variant<72, 72, F>(pk) : wide_variant<72, 72, M>(pk);
  if (dqk == 80) return lse ? wide_variant<80, 80, F>(pk) : wide_variant<80, 80, M>(pk);
  if (dqk == 128) return wide_variant<128, 128, F>(pk);
  return wide_variant<192, 128, F>(pk);
}

// The kernel and fill mode of a bf16 launch.  Segments of at most 64
// queries that would be packed four to a workgroup (no grouped query heads
// to pack instead) take the short-segment kernel, one wave per (segment,
// head), four such units a workgroup, when the head dims have it and the
// call is not split.  Launches of longer segments (unpacked, or up to 128
// queries packed two to a workgroup) whose 64-row blocks fit one round of
// that kernel on every XCD (the padded grid, whose eighth is an XCD's share,
// at most kKeySplitMaxUnits: two workgroups on each of an XCD's 32 CUs) take
// the short-segment kernel with a workgroup's four waves on one 64-row block,
// each walking a quarter of its key tiles (Params::key_split): a quarter of
// the key loop on the path that sets the time.  Past one round the four-wave
// kernel is faster (3 x 1024 queries x 16 heads: 25 against 30 us; 1 x 8192
// x 4 heads, whose 4 (segment, head) groups fill only 4 XCDs: 182 against
// 238 us).
struct LaunchChoice {
  Variant var;
  int32_t mode;
};
static constexpr int64_t kKeySplitMaxUnits = 8 * 2 * 32;  // 8 XCDs x one round of two workgroups on 32 CUs
static LaunchChoice choose_launch(int dqk, int dv, int64_t max_seqlen_q, int64_t heads, int64_t heads_k, bool lse,
                                  bool split, int64_t batch, bool segment_packing = true) {
  const int32_t mode = launch_mode(max_seqlen_q, heads, heads_k, segment_packing);
  if (!split && mode == kPackSegments && max_seqlen_q <= wide::kRowsPerWave && short_supported(dqk, dv))
    return {short_variant(dqk, dv, lse), (int32_t)kPackNone};
  const int64_t bm = wide::kRowsPerWave;  // the short kernel's rows a unit
  if (!split && (mode == kPackNone || mode == kPackSegments) && max_seqlen_q > wide::kRowsPerWave &&
      short_supported(dqk, dv) && grid_blocks(batch, heads, (max_seqlen_q + bm - 1) / bm) <= kKeySplitMaxUnits)
    return {short_key_split_variant(dqk, dv, lse), (int32_t)kPackNone};
  return {variant_for(dqk, dv, mode, lse), mode};
}


// Work units of a launch (padding included): (segment, head, q-tile); with
// short segments packed (pack_mode) (group of segments, head) or (segment,
// group of query heads).
// The head-group shift a launch deals with (head_group_shift): only where
// every segment is one q-tile (at most 256 queries, or short segments
// packed together), whose workgroups read each K/V line once.  Segments of
// several q-tiles already share K/V lines in L2 between their own q-tiles,
// and dealing four heads' q-tiles as one group leaves the XCDs unevenly
// loaded on ragged batches (ViT batch: 0.317 -> 0.387 ms); and none when
// query heads of a KV head share workgroups.
static int32_t launch_hs(int32_t dqk, int32_t dv, int32_t heads, int32_t heads_k, int32_t mode, bool fp8,
                         int64_t max_seqlen_q, const Variant& var, int64_t batch) {
  if (mode == kPackHeads || (mode == kPackNone && max_seqlen_q > var.block_m)) return 0;
  if (var.units_per_wg > 1) return short_head_group_shift(dqk, dv, heads, heads_k, batch, 2);  // one-wave units
  return head_group_shift(dqk, dv, heads, heads_k, fp8 ? 1 : 2);
}

// Workgroups launched for `units` work units (a multiple of 8): one each, or
// for a kernel whose workgroup holds u > 1 units (attn_fwd_short: one per
// wave), ceil(units / 8u) x 8 of them, workgroup w's wave v taking unit
// ((w >> 3) u + v) x 8 + (w & 7), so that every unit keeps its XCD (w % 8 =
// unit % 8) and each XCD's units stay in dispatch order.
static int64_t launch_workgroups(int64_t units, const Variant& var) {
  const int64_t u = var.units_per_wg;
  return u == 1 ? units : (units / 8 + u - 1) / u * 8;
}

static int64_t launch_units(int64_t batch, int64_t heads, int64_t max_seqlen_q, int block_m, int32_t mode,
                            int32_t hs, int32_t* n_qt_out, int32_t* pack_out, bool pair = false) {
  const int32_t pack = mode == kPackNone ? 1 : segments_per_block(max_seqlen_q, block_m / 4);
  const int64_t n_qt1 = pack > 1 ? 1 : (max_seqlen_q + block_m - 1) / block_m;
  const int64_t n_qt = pair ? (n_qt1 + 1) / 2 : n_qt1;  // q-tiles, or pairs of them
  if (n_qt_out) *n_qt_out = (int32_t)n_qt;
  if (pack_out) *pack_out = pack;
  if (mode == kPackHeads) return grid_blocks(batch, heads / pack, 1);
  return grid_blocks((batch + pack - 1) / pack, heads >> hs, n_qt << hs);
}

// Whether a launch pairs each segment's q-tiles n_b - 1 - t and t in one
// workgroup (Params::pair_qt): causal, several q-tiles, one segment a
// workgroup, unsplit, on the four-wave bf16 kernel at the head dims that run
// one workgroup per CU, whose work units then all see the same number of key
// tiles.  The dealing gives each XCD an equal share of the padded grid (its
// units / 8) for its 32 CUs.  Pairs pay where the unpaired units take at
// least two rounds of an XCD (in one round the longest q-tile sets the time
// either way) and the pairs fill their last round (at least 15/16 of it):
// otherwise half-empty rounds of double-length workgroups cost more than the
// unequal q-tiles lose to in-order dispatch.
static constexpr int64_t kCusPerXcd = 32;
static bool pair_q_tiles(bool causal, int32_t mode, const Variant& var, int64_t batch, int64_t heads,
                         int64_t max_seqlen_q, int32_t hs, bool split, bool fp8) {
  if (!causal || split || fp8 || mode != kPackNone || var.units_per_wg != 1 || var.per_cu != 1 ||
      max_seqlen_q <= var.block_m)
    return false;
  const int64_t solo = launch_units(batch, heads, max_seqlen_q, var.block_m, mode, hs, nullptr, nullptr) / 8;
  const int64_t pairs = launch_units(batch, heads, max_seqlen_q, var.block_m, mode, hs, nullptr, nullptr, true) / 8;
  const int64_t rounds = (pairs + kCusPerXcd - 1) / kCusPerXcd;
  return solo >= 2 * kCusPerXcd && 16 * pairs >= 15 * kCusPerXcd * rounds;
}

// Row strides above 2^24 elements would overflow the 32-bit offsets of the
// per-tile buffer loads (64 rows x stride x 2 bytes).
static constexpr int64_t kMaxRowStride = (int64_t)1 << 24;

// Strides are in elements of elem_bytes bytes; rows and heads must start on
// `align`-byte boundaries: 16 for every tensor the kernels read or write
// with 16-byte accesses, 8 for e4m3 outputs (written 8 bytes at a time, so
// a head of d_v 72 packed contiguously qualifies).
static int check_tensor(const va_tensor* t, bool need_data, int elem_bytes = 2, int align = 16) {
  if (t->row_stride <= 0 || t->head_stride <= 0 || t->row_stride > kMaxRowStride) return VA_ERR_STRIDE;
  const int64_t m = align - 1;
  if (((t->row_stride * elem_bytes) & m) != 0 || ((t->head_stride * elem_bytes) & m) != 0) return VA_ERR_ALIGN;
  if (need_data && t->data == nullptr) return VA_ERR_NULL;
  if (((uintptr_t)t->data & (uintptr_t)m) != 0) return VA_ERR_ALIGN;
  return VA_OK;
}

}  // namespace va

extern "C" const char* varlen_attn_status_string(int status) {
  switch (status) {
    case VA_OK: return "ok";
    case VA_ERR_NULL: return "a required pointer is NULL";
    case VA_ERR_SHAPE: return "tensor rows/heads/dims disagree (q heads must be a multiple of k/v heads) or a size is out of range";
    case VA_ERR_HEADDIM: return "unsupported (head_dim_qk, head_dim_v); supported: (64,64) (72,72) (80,80) (128,128) (192,128)";
    case VA_ERR_STRIDE: return "a row or head stride is not positive";
    case VA_ERR_ALIGN: return "a data pointer or stride is not a multiple of 16 bytes (lse: 4 bytes)";
    case VA_ERR_ARG: return "a scalar argument is out of range";
    case VA_ERR_LAUNCH: return "the HIP kernel launch failed";
    case VA_ERR_SCRATCH: return "the split-KV partials need more than the allocation-free entry point's scratch (varlen_attn_scratch_bytes)";
    default: return "unknown status";
  }
}

extern "C" int varlen_attn_tile_range(int32_t seqlen_q, int32_t seqlen_k, int32_t row_begin,
                                      int32_t row_end, int32_t causal, int32_t window_left,
                                      int32_t window_right, int32_t block_n, int32_t* kt_begin,
                                      int32_t* kt_end, int32_t* full_begin, int32_t* full_end) {
  if (!kt_begin || !kt_end || !full_begin || !full_end) return VA_ERR_NULL;
  if (seqlen_q < 0 || seqlen_k < 0 || row_begin < 0 || row_end <= row_begin || row_end > seqlen_q ||
      block_n <= 0 || (causal != 0 && causal != 1) || window_left < -1 || window_right < -1)
    return VA_ERR_ARG;
  const va::TileRange t =
      va::tile_range(seqlen_q, seqlen_k, row_begin, row_end, causal, window_left, window_right, block_n);
  *kt_begin = t.kt_begin;
  *kt_end = t.kt_end;
  *full_begin = t.full_begin;
  *full_end = t.full_end;
  return VA_OK;
}

extern "C" int varlen_attn_work_unit(int64_t block, int32_t batch, int32_t num_heads, int32_t num_heads_k,
                                     int32_t head_dim_qk, int32_t head_dim_v, const int32_t* seqlens_q,
                                     const int32_t* seqlens_k, int32_t causal, int32_t* segment,
                                     int32_t* head, int32_t* q_tile) {
  if (!segment || !head || !q_tile) return VA_ERR_NULL;
  if (!va::supported_dims(head_dim_qk, head_dim_v)) return VA_ERR_HEADDIM;
  if (batch <= 0 || num_heads <= 0 || (causal != 0 && causal != 1)) return VA_ERR_ARG;
  if (num_heads_k <= 0 || num_heads % num_heads_k != 0) return VA_ERR_ARG;
  if (!seqlens_q || !seqlens_k) return VA_ERR_NULL;
  int32_t max_q = 0;
  for (int32_t i = 0; i < batch; ++i) {
    if (seqlens_q[i] < 0 || seqlens_k[i] < 0) return VA_ERR_ARG;
    max_q = seqlens_q[i] > max_q ? seqlens_q[i] : max_q;
  }
  if (max_q <= 0) return VA_ERR_ARG;
  const va::LaunchChoice lc =
      va::choose_launch(head_dim_qk, head_dim_v, max_q, num_heads, num_heads_k, true, false, batch);
  const int32_t mode = lc.mode;
  const va::Variant var = lc.var;
  const int32_t hs = va::launch_hs(head_dim_qk, head_dim_v, num_heads, num_heads_k, mode, false, max_q, var, batch);
  const bool pair = va::pair_q_tiles(causal != 0, mode, var, batch, num_heads, max_q, hs, false, false);
  int32_t n_qt = 0, pack = 1;
  if (block < 0 || block >= va::launch_units(batch, num_heads, max_q, var.block_m, mode, hs, &n_qt, &pack, pair))
    return VA_ERR_ARG;
  if (mode == va::kPackHeads) {  // (segment, first query head of the group)
    const int32_t vheads = num_heads / pack;
    const va::WorkUnit u = va::decode_block((uint32_t)block, (uint32_t)batch, va::make_fastdiv((uint32_t)vheads),
                                            va::make_fastdiv(1u), 0u, causal);
    *segment = u.valid ? u.b : -1;
    *head = u.valid ? va::query_head(u.h, va::make_fastdiv((uint32_t)num_heads_k), vheads / num_heads_k) * pack : -1;
    *q_tile = u.valid ? 0 : -1;
    return VA_OK;
  }
  const int32_t groups = (batch + pack - 1) / pack;
  const va::WorkUnit u = pack == 1 && va::lpt_applies(batch, seqlens_q, seqlens_k)
                             ? va::decode_block_lpt(block, batch, num_heads, var.block_m, n_qt, causal,
                                                    seqlens_q, seqlens_k, hs, pair)
                             : va::decode_block((uint32_t)block, (uint32_t)groups,
                                                va::make_fastdiv((uint32_t)(num_heads >> hs)),
                                                va::make_fastdiv((uint32_t)(n_qt << hs)), (uint32_t)hs, causal);
  int32_t qt = u.qt;
  bool valid = u.valid;
  if (valid && pair) {  // pair t: q-tile n_b - 1 - t first (none past the segment's middle)
    const int32_t nb = (seqlens_q[u.b] + var.block_m - 1) / var.block_m;
    valid = nb - 1 - u.qt >= u.qt;
    qt = nb - 1 - u.qt;
  }
  *segment = valid ? u.b * pack : -1;
  *head = valid ? va::query_head(u.h, va::make_fastdiv((uint32_t)num_heads_k), num_heads / num_heads_k) : -1;
  *q_tile = valid ? qt : -1;
  return VA_OK;
}

extern "C" int varlen_attn_plan(int32_t head_dim_qk, int32_t head_dim_v, int32_t batch,
                                int32_t num_heads, int32_t num_heads_k, int32_t max_seqlen_q,
                                int32_t max_seqlen_k, int32_t causal, va_plan* plan) {
  (void)max_seqlen_k;
  if (!plan) return VA_ERR_NULL;
  if (!va::supported_dims(head_dim_qk, head_dim_v)) return VA_ERR_HEADDIM;
  if (batch < 0 || num_heads <= 0 || max_seqlen_q < 0) return VA_ERR_ARG;
  if (num_heads_k <= 0 || num_heads % num_heads_k != 0) return VA_ERR_ARG;
  const va::LaunchChoice lc =
      va::choose_launch(head_dim_qk, head_dim_v, max_seqlen_q, num_heads, num_heads_k, true, false, batch);
  const int32_t mode = lc.mode;
  const va::Variant var = lc.var;
  plan->block_m = var.block_m;
  plan->block_n = var.block_n;
  plan->threads = var.threads;
  plan->lds_bytes = var.lds_bytes;
  const int32_t hs = va::launch_hs(head_dim_qk, head_dim_v, num_heads, num_heads_k, mode, false, max_seqlen_q, var,
                                   batch);
  const bool pair = va::pair_q_tiles(causal != 0, mode, var, batch, num_heads, max_seqlen_q, hs, false, false);
  plan->units = va::launch_units(batch, num_heads, max_seqlen_q, var.block_m, mode, hs, nullptr,
                                 &plan->segments_per_block, pair);
  plan->grid = va::launch_workgroups(plan->units, var);
  plan->pack_mode = mode;
  plan->kernel = var.name;
  plan->pair_q_tiles = pair ? 1 : 0;
  plan->key_split = var.key_split;
  return VA_OK;
}

extern "C" int varlen_attn_plan_fp8(int32_t head_dim_qk, int32_t head_dim_v, int32_t batch,
                                    int32_t num_heads, int32_t num_heads_k, int32_t max_seqlen_q,
                                    int32_t max_seqlen_k, int32_t causal, va_plan* plan) {
  (void)max_seqlen_k;
  (void)causal;
  if (!plan) return VA_ERR_NULL;
  if (!va::fp8_supported_dims(head_dim_qk, head_dim_v)) return VA_ERR_HEADDIM;
  if (batch < 0 || num_heads <= 0 || max_seqlen_q < 0) return VA_ERR_ARG;
  if (num_heads_k <= 0 || num_heads % num_heads_k != 0) return VA_ERR_ARG;
  const int32_t mode = va::launch_mode(max_seqlen_q, num_heads, num_heads_k);
  const va::Variant var = va::fp8_variant(head_dim_qk, head_dim_v, mode);
  plan->block_m = var.block_m;
  plan->block_n = var.block_n;
  plan->threads = var.threads;
  plan->lds_bytes = var.lds_bytes;
  plan->units = va::launch_units(batch, num_heads, max_seqlen_q, var.block_m, mode,
                                 va::launch_hs(head_dim_qk, head_dim_v, num_heads, num_heads_k, mode, true,
                                               max_seqlen_q, var, batch),
                                 nullptr,
                                 &plan->segments_per_block);
  plan->grid = va::launch_workgroups(plan->units, var);
  plan->pack_mode = mode;
  plan->kernel = var.name;
  plan->pair_q_tiles = 0;
  plan->key_split = 1;
  return VA_OK;
}

namespace va {

// Validation shared by the entry points; fills the launch parameters.
// Returns VA_OK (and *launch = false when there is nothing to launch).
// fp8: Q, K, V hold e4m3 bytes (and out too when out_fp8).
static int prepare(const va_tensor* q, const va_tensor* k, const va_tensor* v, const int32_t* cu_seqlens_q,
                   const int32_t* cu_seqlens_k, int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                   float softmax_scale, int32_t causal, int32_t window_left, int32_t window_right,
                   const va_tensor* out, float* lse, Params& p, bool& launch, bool fp8 = false,
                   bool out_fp8 = false) {
  launch = false;
  if (!q || !k || !v || !out) return VA_ERR_NULL;
  if (batch < 0 || max_seqlen_q < 0 || max_seqlen_k < 0) return VA_ERR_ARG;
  if (!(softmax_scale > 0.f) || !isfinite(softmax_scale)) return VA_ERR_ARG;
  if (causal != 0 && causal != 1) return VA_ERR_ARG;
  if (window_left < -1 || window_right < -1) return VA_ERR_ARG;
  if (q->heads <= 0 || k->heads <= 0 || v->heads != k->heads || out->heads != q->heads ||
      q->heads % k->heads != 0)
    return VA_ERR_SHAPE;
  if (q->rows < 0 || k->rows < 0 || v->rows != k->rows || out->rows != q->rows) return VA_ERR_SHAPE;
  if (q->rows > INT32_MAX || k->rows > INT32_MAX) return VA_ERR_SHAPE;
  if (k->dim != q->dim || out->dim != v->dim) return VA_ERR_SHAPE;
  if (!(fp8 ? fp8_supported_dims(q->dim, v->dim) : supported_dims(q->dim, v->dim))) return VA_ERR_HEADDIM;
  const bool has_q = q->rows > 0, has_k = k->rows > 0;
  const int in_bytes = fp8 ? 1 : 2, out_bytes = out_fp8 ? 1 : 2;
  int st;
  if ((st = check_tensor(q, has_q, in_bytes)) != VA_OK) return st;
  if ((st = check_tensor(k, has_k, in_bytes)) != VA_OK) return st;
  if ((st = check_tensor(v, has_k, in_bytes)) != VA_OK) return st;
  if ((st = check_tensor(out, has_q, out_bytes, out_fp8 ? 8 : 16)) != VA_OK) return st;
  if (lse != nullptr && ((uintptr_t)lse & 3u) != 0) return VA_ERR_ALIGN;
  if (batch == 0 || max_seqlen_q == 0 || q->rows == 0) return VA_OK;
  if (!cu_seqlens_q || !cu_seqlens_k) return VA_ERR_NULL;

  p.q = (const uint16_t*)q->data;
  p.k = (const uint16_t*)k->data;
  p.v = (const uint16_t*)v->data;
  p.o = (uint16_t*)out->data;
  p.lse = lse;
  p.cu_q = cu_seqlens_q;
  p.cu_k = cu_seqlens_k;
  p.q_row = q->row_stride;
  p.q_head = q->head_stride;
  p.k_row = k->row_stride;
  p.k_head = k->head_stride;
  p.v_row = v->row_stride;
  p.v_head = v->head_stride;
  p.o_row = out->row_stride;
  p.o_head = out->head_stride;
  p.total_q = q->rows;
  p.batch = batch;
  p.heads = q->heads;
  p.heads_k = k->heads;
  p.causal = causal;
  p.wl = window_left;
  p.wr = window_right;
  p.scale_log2 = softmax_scale * 1.4426950408889634f;
  p.num_splits = 1;
  p.splits_dyn = nullptr;
  p.pair_qt = 0;
  p.key_split = 1;
  p.part_o = nullptr;
  p.part_lse = nullptr;
  p.q_descale = p.k_descale = p.v_descale = p.out_scale = nullptr;
  (void)max_seqlen_k;
  launch = true;
  return VA_OK;
}

// One launch of the attention kernel over num_splits copies of the work units.
static int launch_attention(Params& p, int32_t head_dim_qk, int32_t head_dim_v, int32_t max_seqlen_q,
                            bool fp32_row_sum, void* stream, bool fp8 = false) {
  int32_t mode = launch_mode(max_seqlen_q, p.heads, p.heads_k, p.splits_dyn == nullptr);
  Variant var;
  if (fp8) {
    var = fp8_variant(head_dim_qk, head_dim_v, mode);
  } else {
    const LaunchChoice lc = choose_launch(head_dim_qk, head_dim_v, max_seqlen_q, p.heads, p.heads_k, fp32_row_sum,
                                          p.num_splits > 1, p.batch, p.splits_dyn == nullptr);
    var = lc.var;
    mode = lc.mode;
  }
  const int32_t hs = launch_hs(head_dim_qk, head_dim_v, p.heads, p.heads_k, mode, fp8, max_seqlen_q, var, p.batch);
  const bool pair = pair_q_tiles(p.causal != 0, mode, var, p.batch, p.heads, max_seqlen_q, hs,
                                 p.num_splits > 1 || p.splits_dyn != nullptr, fp8);
  p.pair_qt = pair ? 1 : 0;
  p.key_split = var.key_split;
  const int64_t units = launch_units(p.batch, p.heads, max_seqlen_q, var.block_m, mode, hs, &p.n_qt, &p.pack, pair);
  if (units > INT32_MAX) return VA_ERR_SHAPE;
  p.n_units = (int32_t)units;
  // The work-unit decode's divisors (the kernel divides by multiplying).
  const int32_t dealt_heads = mode == kPackHeads ? p.heads / p.pack : p.heads;
  p.hg_shift = hs;
  p.fd_heads = make_fastdiv((uint32_t)(dealt_heads >> hs));
  p.fd_nqt = make_fastdiv((uint32_t)(p.n_qt << hs));
  p.fd_heads_k = make_fastdiv((uint32_t)p.heads_k);
  p.fd_group = make_fastdiv((uint32_t)(p.heads / p.heads_k));
  p.qh_group = dealt_heads / p.heads_k;
  p.n_dealt = mode == kPackSegments ? (p.batch + p.pack - 1) / p.pack : p.batch;
  p.pack_shift = p.pack == 4 ? 2 : (p.pack == 2 ? 1 : 0);
  // Workgroups along x, split-KV copies along y.
  void* args[] = {&p};
  const hipError_t err = hipLaunchKernel(var.fn, dim3((unsigned)launch_workgroups(units, var), (unsigned)p.num_splits),
                                         dim3(var.threads), args, 0, (hipStream_t)stream);
  return err == hipSuccess ? VA_OK : VA_ERR_LAUNCH;
}

}  // namespace va

extern "C" int varlen_attn_fwd(const va_tensor* q, const va_tensor* k, const va_tensor* v,
                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t batch,
                               int32_t max_seqlen_q, int32_t max_seqlen_k, float softmax_scale,
                               int32_t causal, int32_t window_left, int32_t window_right,
                               const va_tensor* out, float* lse, void* stream) {
  va::Params p;
  bool launch = false;
  const int st = va::prepare(q, k, v, cu_seqlens_q, cu_seqlens_k, batch, max_seqlen_q, max_seqlen_k, softmax_scale,
                             causal, window_left, window_right, out, lse, p, launch);
  if (st != VA_OK || !launch) return st;
  return va::launch_attention(p, q->dim, v->dim, max_seqlen_q, lse != nullptr, stream);
}

extern "C" int varlen_attn_fwd_quant_out(const va_tensor* q, const va_tensor* k, const va_tensor* v,
                                         const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t batch,
                                         int32_t max_seqlen_q, int32_t max_seqlen_k, float softmax_scale,
                                         int32_t causal, int32_t window_left, int32_t window_right,
                                         const va_tensor* out, const float* out_scale, float* lse, void* stream) {
  if (!out_scale) return VA_ERR_NULL;
  if (((uintptr_t)out_scale & 3u) != 0) return VA_ERR_ALIGN;
  va::Params p;
  bool launch = false;
  const int st = va::prepare(q, k, v, cu_seqlens_q, cu_seqlens_k, batch, max_seqlen_q, max_seqlen_k, softmax_scale,
                             causal, window_left, window_right, out, lse, p, launch, false, true);
  if (st != VA_OK || !launch) return st;
  p.out_scale = out_scale;
  return va::launch_attention(p, q->dim, v->dim, max_seqlen_q, lse != nullptr, stream);
}

namespace va {
constexpr int kMaxSplits = 128;
static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
}  // namespace va

extern "C" size_t varlen_attn_splitkv_workspace_bytes(int64_t total_q, int32_t num_heads, int32_t head_dim_v,
                                                      int32_t num_splits) {
  if (total_q <= 0 || num_heads <= 0 || head_dim_v <= 0 || num_splits <= 1) return 0;
  const size_t n = (size_t)num_splits * (size_t)total_q * (size_t)num_heads;
  return va::align256(n * (size_t)head_dim_v * sizeof(float)) + n * sizeof(float);
}

extern "C" int varlen_attn_num_splits(int32_t head_dim_qk, int32_t head_dim_v, int32_t batch, int32_t num_heads,
                                      int32_t num_heads_k, int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t fp8,
                                      int32_t* num_splits) {
  if (!num_splits) return VA_ERR_NULL;
  if (!(fp8 ? va::fp8_supported_dims(head_dim_qk, head_dim_v) : va::supported_dims(head_dim_qk, head_dim_v)))
    return VA_ERR_HEADDIM;
  if (batch < 0 || num_heads <= 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || (fp8 != 0 && fp8 != 1))
    return VA_ERR_ARG;
  if (num_heads_k <= 0 || num_heads % num_heads_k != 0) return VA_ERR_ARG;
  *num_splits = 1;
  if (batch == 0 || max_seqlen_q == 0 || max_seqlen_k == 0) return VA_OK;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return VA_OK;
  // The work units the launch has (padding included; packing and grouped
  // heads as the launch takes them) against the workgroups the device holds
  // at once; each split keeps at least 16 key tiles of the kernel's width.
  const int32_t mode = va::launch_mode(max_seqlen_q, num_heads, num_heads_k);
  const va::Variant var = fp8 ? va::fp8_variant(head_dim_qk, head_dim_v, mode)
                              : va::variant_for(head_dim_qk, head_dim_v, mode, true);
  const int64_t units =
      va::launch_units(batch, num_heads, max_seqlen_q, var.block_m, mode,
                       va::launch_hs(head_dim_qk, head_dim_v, num_heads, num_heads_k, mode, fp8 != 0, max_seqlen_q,
                                     var, batch),
                       nullptr, nullptr);
  const int64_t slots = (int64_t)cus * var.per_cu;
  const int64_t by_tiles = ((int64_t)max_seqlen_k + 16 * var.block_n - 1) / (16 * var.block_n);
  int64_t s = slots / units;
  s = s < by_tiles ? s : by_tiles;
  s = s < va::kMaxSplits ? s : va::kMaxSplits;
  *num_splits = (int32_t)(s > 1 ? s : 1);
  return VA_OK;
}

namespace va_merge {
int launch_combine(const float* part_o, const float* part_lse, int32_t num_splits, int64_t total_q, int32_t heads,
                   int32_t dim, const int32_t* cu_seqlens_q, int32_t batch, const va_tensor* out, float* lse,
                   void* stream, const float* out_scale, const int32_t* splits_dyn);
}

extern "C" int varlen_attn_fwd_splitkv(const va_tensor* q, const va_tensor* k, const va_tensor* v,
                                       const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t batch,
                                       int32_t max_seqlen_q, int32_t max_seqlen_k, float softmax_scale,
                                       int32_t causal, int32_t window_left, int32_t window_right,
                                       const va_tensor* out, float* lse, int32_t num_splits,
                                       const int32_t* num_splits_dynamic, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  if (num_splits < 1 || num_splits > va::kMaxSplits) return VA_ERR_ARG;
  if (((uintptr_t)num_splits_dynamic & 3u) != 0) return VA_ERR_ALIGN;
  va::Params p;
  bool launch = false;
  int st = va::prepare(q, k, v, cu_seqlens_q, cu_seqlens_k, batch, max_seqlen_q, max_seqlen_k, softmax_scale,
                       causal, window_left, window_right, out, lse, p, launch);
  if (st != VA_OK) return st;
  if (num_splits == 1) return launch ? va::launch_attention(p, q->dim, v->dim, max_seqlen_q, lse != nullptr, stream)
                                     : VA_OK;
  const size_t need = varlen_attn_splitkv_workspace_bytes(q->rows, q->heads, v->dim, num_splits);
  if (!launch) return VA_OK;
  if (!workspace) return VA_ERR_NULL;
  if (((uintptr_t)workspace & 255u) != 0) return VA_ERR_ALIGN;
  if (workspace_bytes < need) return VA_ERR_ARG;
  p.num_splits = num_splits;
  p.splits_dyn = num_splits_dynamic;
  p.part_o = (float*)workspace;
  p.part_lse = (float*)((char*)workspace +
                        va::align256((size_t)num_splits * (size_t)q->rows * (size_t)q->heads * (size_t)v->dim * 4));
  // The partials' LSEs need the fp32 row sum, whether or not an LSE is returned.
  if ((st = va::launch_attention(p, q->dim, v->dim, max_seqlen_q, true, stream)) != VA_OK) return st;
  return va_merge::launch_combine(p.part_o, p.part_lse, num_splits, q->rows, q->heads, v->dim, cu_seqlens_q, batch,
                                  out, lse, stream, nullptr, num_splits_dynamic);
}

// ----------------------------------------------------------------------------
// Split-KV without a caller workspace: the fp32 partials live in one
// file-scope device array per GPU, found once per device with
// hipGetSymbolAddress (in host code the array's name is only a stand-in for
// that address).  Calls on one GPU share the array, so calls that overlap on
// one GPU (concurrent streams, host threads) race; consecutive calls on one
// stream do not.  The kernels write every partial the combine reads, so
// nothing is cleared between calls.
// ----------------------------------------------------------------------------
namespace va {
static __device__ __align__(256) char scratch[VA_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mutex;
static void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once found

// The current device's copy of `scratch` (nullptr: no device, or the lookup
// failed).
static void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace va

extern "C" size_t varlen_attn_scratch_bytes(void) { return (size_t)VA_SCRATCH_BYTES; }

extern "C" int varlen_attn_fwd_splitkv_noalloc(const va_tensor* q, const va_tensor* k, const va_tensor* v,
                                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                               int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                               float softmax_scale, int32_t causal, int32_t window_left,
                                               int32_t window_right, const va_tensor* out, float* lse,
                                               int32_t num_splits, void* stream) {
  if (num_splits < 1 || num_splits > va::kMaxSplits) return VA_ERR_ARG;
  if (num_splits == 1)
    return varlen_attn_fwd_splitkv(q, k, v, cu_seqlens_q, cu_seqlens_k, batch, max_seqlen_q, max_seqlen_k,
                                   softmax_scale, causal, window_left, window_right, out, lse, 1, nullptr, nullptr,
                                   0, stream);
  // The argument checks first (they make no HIP call); then the size limit.
  va::Params p;
  bool launch = false;
  const int st = va::prepare(q, k, v, cu_seqlens_q, cu_seqlens_k, batch, max_seqlen_q, max_seqlen_k,
                             softmax_scale, causal, window_left, window_right, out, lse, p, launch);
  if (st != VA_OK || !launch) return st;
  const size_t need = varlen_attn_splitkv_workspace_bytes(q->rows, q->heads, v->dim, num_splits);
  if (need > (size_t)VA_SCRATCH_BYTES) return VA_ERR_SCRATCH;
  void* ws = va::scratch_address();
  if (ws == nullptr) return VA_ERR_LAUNCH;
  return varlen_attn_fwd_splitkv(q, k, v, cu_seqlens_q, cu_seqlens_k, batch, max_seqlen_q, max_seqlen_k,
                                 softmax_scale, causal, window_left, window_right, out, lse, num_splits, nullptr, ws,
                                 (size_t)VA_SCRATCH_BYTES, stream);
}

extern "C" int varlen_attn_fwd_fp8(const va_tensor* q, const va_tensor* k, const va_tensor* v,
                                   const float* q_descale, const float* k_descale, const float* v_descale,
                                   const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t batch,
                                   int32_t max_seqlen_q, int32_t max_seqlen_k, float softmax_scale, int32_t causal,
                                   int32_t window_left, int32_t window_right, const va_tensor* out,
                                   const float* out_scale, float* lse, int32_t num_splits,
                                   const int32_t* num_splits_dynamic, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  if (num_splits < 1 || num_splits > va::kMaxSplits) return VA_ERR_ARG;
  for (const float* d : {q_descale, k_descale, v_descale, out_scale})
    if (((uintptr_t)d & 3u) != 0) return VA_ERR_ALIGN;
  if (((uintptr_t)num_splits_dynamic & 3u) != 0) return VA_ERR_ALIGN;
  va::Params p;
  bool launch = false;
  int st = va::prepare(q, k, v, cu_seqlens_q, cu_seqlens_k, batch, max_seqlen_q, max_seqlen_k, softmax_scale,
                       causal, window_left, window_right, out, lse, p, launch, true, out_scale != nullptr);
  if (st != VA_OK || !launch) return st;
  p.q_descale = q_descale;
  p.k_descale = k_descale;
  p.v_descale = v_descale;
  p.out_scale = out_scale;
  if (num_splits == 1) return va::launch_attention(p, q->dim, v->dim, max_seqlen_q, true, stream, true);
  const size_t need = varlen_attn_splitkv_workspace_bytes(q->rows, q->heads, v->dim, num_splits);
  if (!workspace) return VA_ERR_NULL;
  if (((uintptr_t)workspace & 255u) != 0) return VA_ERR_ALIGN;
  if (workspace_bytes < need) return VA_ERR_ARG;
  p.num_splits = num_splits;
  p.splits_dyn = num_splits_dynamic;
  p.part_o = (float*)workspace;
  p.part_lse = (float*)((char*)workspace +
                        va::align256((size_t)num_splits * (size_t)q->rows * (size_t)q->heads * (size_t)v->dim * 4));
  if ((st = va::launch_attention(p, q->dim, v->dim, max_seqlen_q, true, stream, true)) != VA_OK) return st;
  return va_merge::launch_combine(p.part_o, p.part_lse, num_splits, q->rows, q->heads, v->dim, cu_seqlens_q, batch,
                                  out, lse, stream, out_scale, num_splits_dynamic);
}
