// Fused variable-length attention forward on fp8 e4m3 Q, K, V for AMD
// Instinct MI355X (gfx950).
//
// The same workgroup structure, tile schedule, staging and online softmax as
// attn_fwd_wide (varlen_attn_fwd.hip), with both products on
// v_mfma_f32_32x32x64_f8f6f4 (e4m3 x e4m3, fp32 accumulate), which runs at
// twice the bf16 MFMA rate:
//
//   S^T = K Q^T     32-key x 32-query blocks, 64 head dims per MFMA;
//   p = exp2(s * scale * log2(e) * q_descale * k_descale - m), rounded to
//       e4m3 for the PV product (p <= 2^kRescaleTau = 256 < 448, the
//       largest e4m3 value, so no p saturates);
//   O^T += V^T P^T  64 keys per MFMA, hence 64-key tiles;
//   O = acc * v_descale / l, l the fp32 sum of the unrounded p.  The fp8
//       MFMA sums its 64 products at less than fp32 precision (within
//       2^-15 of sum |q k| a score), which bounds the LSE error beyond the
//       fp32 arithmetic.
//
// The descales (one fp32 per segment and KV head) undo a per-block
// quantisation of the inputs: the scores see q_descale * k_descale folded
// into the softmax scale, O sees v_descale.  With an output scale the result
// leaves as e4m3 codes of O / out_scale, clamped to +-448 (a static
// per-tensor symmetric quantisation of the output).  The pages list fp8 e4m3
// with descales among the FA4 configurations checked for bit-exactness
// (SGLang PR #41344, "Accuracy Tests") and the fp8 static per-tensor
// output quantisation (vLLM MLA prefill docs, supports_quant_output /
// output_scale).
//
// Operand layouts, measured with in-bounds probes on gfx950:
// * 32x32x64 fp8 MFMA: lane l holds row (A) or column (B) l % 32 and 32 of
//   the 64 k values in its 8 registers, the same k for the same (l / 32,
//   byte) position in A and B.  Any placement of head dims (QK^T) or keys
//   (PV) on (l / 32, byte) positions that both operands share therefore gives
//   the product; the accumulator layout is that of the bf16 32x32 MFMA.
// * ds_read_b64_tr_b8: in each 16-lane group, lanes 2i and 2i + 1 give the
//   two 8-byte halves of row i of an 8 x 16-byte matrix, and lane j receives
//   byte j of the eight rows.
#include "attn_common.h"

namespace va {

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));

namespace fp8k {
constexpr int kRowsPerWave = 64;     // query rows per wave
constexpr int kBN = 64;              // keys per tile: the k extent of one PV MFMA
constexpr int kSB = kBN / 32;        // 32-key score blocks per tile
constexpr int kStages = 6;           // tile t lives in stage t % 6 (an even count: see the loop)
constexpr int kAhead = kStages - 2;  // iteration j issues tile j + 4
constexpr int kDepth = 3;            // LDS operands read ahead of their MFMA
constexpr int kWaves = 4;
static_assert(kWaves == 4, "the packed set-up shifts wave indices by log2(4 / pack)");

template <int DQK, int DV>
struct Cfg {
  static constexpr int WAVES = kWaves;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int QB = 2;  // 32-row query blocks per wave
  static constexpr int RPW = 32 * QB;
  static constexpr int BM = RPW * WAVES;
  static constexpr int KC = DQK / 64;  // 64-wide k-chunks of QK^T
  static constexpr int VB = DV / 32;   // 32-row d_v blocks of PV
  // K tile: kBN rows of DQK bytes = CPR_K 16-byte chunks plus one pad chunk,
  // so the rows an operand read touches hit distinct banks.
  static constexpr int CPR_K = DQK / 16;
  static constexpr int KPITCH = CPR_K + 1;
  // V tile: kBN rows of DV bytes, chunk index XOR-swizzled per row.
  static constexpr int CPR_V = DV / 16;
  static constexpr int K_SLOTS = kBN * KPITCH;
  static constexpr int V_SLOTS = kBN * CPR_V;
  static constexpr int K_WL = (K_SLOTS + 63) / 64;  // 64-lane x 16-byte wave-loads per tile
  static constexpr int V_WL = (V_SLOTS + 63) / 64;
  static constexpr int K_TILE = K_WL * 1024;
  static constexpr int V_TILE = V_WL * 1024;
  static constexpr int NK = (K_WL + WAVES - 1) / WAVES;
  static constexpr int NV = (V_WL + WAVES - 1) / WAVES;
  static constexpr int LOADS = NK + NV;
  static constexpr int LDS_BYTES = kStages * (K_TILE + V_TILE) + 1024;
  static_assert(DQK % 64 == 0 && DV % 32 == 0, "fp8 MFMA granularity");
  static_assert(CPR_V == 4 || CPR_V == 8, "V swizzle defined for 4 and 8 chunks");
  static_assert(RPW == kRowsPerWave, "one row count per wave");
};

// XOR applied to the chunk index of V row `row`.  A transposing read takes
// eight rows (keys b..b+3 and b+8..b+11, b a multiple of 4) times two
// adjacent chunks per 32 lanes; with this swizzle those 16 chunks fall on
// distinct 16-byte bank groups.
template <int CPR_V>
__host__ __device__ constexpr int v_swizzle(int row) {
  return CPR_V == 8 ? 2 * (((row >> 1) & 1) | (((row >> 3) & 1) << 1)) : 2 * ((row >> 3) & 1);
}
}  // namespace fp8k

__device__ __forceinline__ f32x16 mfma_e4m3(i32x8 a, i32x8 b, f32x16 c) {
  // Format codes 0 / 0: both operands e4m3; no block scales.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ i32x8 lds_read_2xb128(const lds_char* base, int byte_off) {
  const u32x4 lo = *(const __attribute__((address_space(3))) u32x4*)(base + byte_off);
  const u32x4 hi = *(const __attribute__((address_space(3))) u32x4*)(base + byte_off + 16);
  return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ i32x2 lds_read_tr8(const lds_char* base, int byte_off) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(base + byte_off));
}

// ============================================================================
// The kernel: 4 waves x 64 query rows (BM = 256), 64-key tiles, six LDS
// stages; see attn_fwd_wide for the pipeline, which is the same.
//
// Probabilities as the PV B operand: byte j of lane (query, g) is key
// 32 (j / 16) + 8 ((j / 4) % 4) + 4 g + j % 4 of the tile, which is where
// the score blocks' accumulator layout puts them (score block j / 16,
// register j % 16), so each register packs four consecutive scores.  The
// V^T A operand takes the same keys at the same positions: transposing read
// t of lane (d, g) covers bytes 8t..8t+7, i.e. keys 16 t + 8 (i / 4) + 4 g +
// i % 4 for rows i = 0..7.
// ============================================================================
template <int DQK, int DV, int PK>
__global__ __launch_bounds__(64 * fp8k::kWaves, 1) void attn_fwd_fp8(Params p) {
  using namespace fp8k;
  using C = Cfg<DQK, DV>;
  static_assert(kStages == 6, "stage objects below");
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

  const int split = (int)blockIdx.y;  // split-KV copy (0 without split)
  const BlockWork bw = block_work<PK>(p, lane, C::BM, (int64_t)blockIdx.x);
  if (!bw.u.valid) return;
  int h = bw.u.h;
  const int qt = bw.u.qt;
  const int k0 = bw.k0, Lk = bw.lk;
  const int r0 = qt * C::BM;
  if (r0 >= bw.lq) return;
  constexpr bool packed = PK == kPackSegments;
  // This wave's rows and segment (as in attn_fwd_wide).
  int q0 = bw.q0, Lq = bw.lq, wLk = Lk, wkoff = 0, wrow0 = r0 + wave * C::RPW;
  int r1 = min(r0 + C::BM, Lq);
  int wseg = bw.u.b;
  if constexpr (packed) {
    const int per = C::WAVES >> p.pack_shift;
    const int seg = (bw.u.b << p.pack_shift) + (wave >> (2 - p.pack_shift));
    wrow0 = (wave & (per - 1)) * C::RPW;
    q0 = Lq = wLk = wkoff = r1 = 0;
    wseg = seg;
    if (seg < p.batch) {
      q0 = p.cu_q[seg];
      Lq = p.cu_q[seg + 1] - q0;
      wkoff = p.cu_k[seg] - k0;
      wLk = p.cu_k[seg + 1] - k0 - wkoff;
      r1 = Lq;
    }
  }
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
  // Per-segment split counts, as in attn_fwd_wide.
  int n_splits = p.num_splits;
  if constexpr (PK != kPackSegments) {  // (a unit holds one segment; the host never packs segments then)
    if (p.splits_dyn != nullptr) {
      n_splits = min(max(p.splits_dyn[bw.u.b], 1), p.num_splits);
      if (split >= n_splits) return;
    }
  }
  const TileRange tr = split_range(tr0, split, n_splits);
  const int ntiles = tr.kt_end - tr.kt_begin;
  const int hk = (int)fdiv((uint32_t)h, p.fd_group);  // the KV head query head h reads

  // ---- Q fragments (B operand of S^T = K Q^T): lane (query, g) holds head
  // dims 64 c + 32 g .. + 31 of chunk c.
  // Buffer loads over this wave's rows [wrow0, r1): rows past r1 read as
  // zero, with no branch per load.
  i32x8 qf[C::QB][C::KC];
  {
    const int64_t q_row_b = p.q_row;  // one byte per element
    const int vrows = __builtin_amdgcn_readfirstlane(max(min(r1 - wrow0, C::RPW), 0));
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const uint8_t*)p.q + (int64_t)(q0 + wrow0) * p.q_row + (int64_t)h * p.q_head), (short)0,
        (int)(uint32_t)(vrows * q_row_b), kBufferFlags);
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) {
      const uint32_t row_off = (uint32_t)((32 * qb + l32) * q_row_b);
#pragma unroll
      for (int c = 0; c < C::KC; ++c) {
        const uint32_t off = row_off + 64 * c + 32 * g;
        const u32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
        const u32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(rq, off + 16, 0, 0);
        qf[qb][c] = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
  }

  // ---- direct-to-LDS tile loads (as in attn_fwd_wide; every V chunk holds
  // data) ----------------------------------------------------------------------
  __shared__ __attribute__((aligned(1024))) char dummy[1024];
  const int64_t k_row_b = p.k_row, v_row_b = p.v_row;  // one byte per element
  uint32_t k_off[C::NK], v_off[C::NV];
#pragma unroll
  for (int x = 0; x < C::NK; ++x) {
    const int i = wave + C::WAVES * x;
    const int sl = i * 64 + lane;
    const int row = sl / C::KPITCH, c = sl % C::KPITCH;
    k_off[x] = (i < C::K_WL && sl < C::K_SLOTS && c < C::CPR_K) ? (uint32_t)(row * k_row_b + c * 16) : kOOB;
  }
#pragma unroll
  for (int x = 0; x < C::NV; ++x) {
    const int i = wave + C::WAVES * x;
    const int sl = i * 64 + lane;
    const int row = sl / C::CPR_V;
    const int c = (sl % C::CPR_V) ^ v_swizzle<C::CPR_V>(row);
    v_off[x] = (i < C::V_WL && sl < C::V_SLOTS) ? (uint32_t)(row * v_row_b + c * 16) : kOOB;
  }
  const char* k_next =
      (const char*)p.k + ((int64_t)k0 + (int64_t)tr.kt_begin * kBN) * p.k_row + (int64_t)hk * p.k_head;
  const char* v_next =
      (const char*)p.v + ((int64_t)k0 + (int64_t)tr.kt_begin * kBN) * p.v_row + (int64_t)hk * p.v_head;
  // (prefetches past the workgroup's last tile, a causal q-tile's diagonal,
  // read zeros: an empty range)
  int keys_next = min(Lk, tr.kt_end * kBN) - tr.kt_begin * kBN;
  auto issue = [&](auto st) VA_INLINE {
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
      dma16(rv, i < C::V_WL ? vst(st) + i * 1024 : (lds_char*)dummy, v_off[x]);
    }
    k_next += kBN * k_row_b;
    v_next += kBN * v_row_b;
    keys_next -= kBN;
  };
  auto wait_landed = [&](auto later_tiles) VA_INLINE {
    constexpr int n = C::LOADS * decltype(later_tiles)::value;
    static_assert(n < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(n) : "memory");
  };

  if (ntiles > 0) static_for<0, kAhead>([&](auto t) VA_INLINE { issue(t); });  // tiles 0-3

  // Descales of this wave's segment and KV head (a wave past the last packed
  // segment has no rows and keeps 1).
  float sl2 = p.scale_log2, vsc = 1.f;
  if (wseg < p.batch) {
    const int64_t di = (int64_t)wseg * p.heads_k + hk;
    if (p.q_descale != nullptr) sl2 *= p.q_descale[di];
    if (p.k_descale != nullptr) sl2 *= p.k_descale[di];
    if (p.v_descale != nullptr) vsc = p.v_descale[di];
  }

  int w_beg = 0, w_end = 0, w_full_begin = 0, w_full_end = 0;  // relative to tr.kt_begin
  if (wrow0 < r1) {
    const TileRange wt =
        tile_range(Lq, wLk, wrow0, min(wrow0 + C::RPW, r1), p.causal, p.wl, p.wr, kBN, wkoff);
    w_beg = min(max(wt.kt_begin, tr.kt_begin), tr.kt_end) - tr.kt_begin;
    w_end = min(max(wt.kt_end, tr.kt_begin), tr.kt_end) - tr.kt_begin;
    w_full_begin = min(max(wt.full_begin, tr.kt_begin), tr.kt_end) - tr.kt_begin;
    w_full_end = min(max(wt.full_end, tr.kt_begin), tr.kt_end) - tr.kt_begin;
  }
  const bool active = w_end > w_beg;
  // As in attn_fwd_wide: a wave computes iterations w_beg - 1 .. w_end only.
  const int w_first = w_beg > 0 ? w_beg - 1 : 0;

  // ---- LDS operand reads ----------------------------------------------------
  // K operand (sb, c): row 32 sb + l32, chunks 4 c + 2 g and 4 c + 2 g + 1.
  const int k_rd = (l32 * C::KPITCH + 2 * g) * 16;
  // V^T operand vb, read t: lane (16 G1 + m, g) of a 16-lane group supplies
  // half m % 2 of row m / 2, i.e. key 16 t + vrow, chunk 2 vb + G1.
  int v_rd[C::VB];
  {
    const int i = (lane & 15) >> 1, G1 = (lane >> 4) & 1;
    const int vrow = 8 * (i >> 2) + 4 * g + (i & 3);
#pragma unroll
    for (int vb = 0; vb < C::VB; ++vb)
      v_rd[vb] = (vrow * C::CPR_V + ((2 * vb + G1) ^ v_swizzle<C::CPR_V>(vrow))) * 16 + 8 * (lane & 1);
  }
  constexpr int kVRead = 16 * C::CPR_V * 16;  // bytes between transposing reads t and t + 1

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
    m_run[qb] = -INFINITY;
    nm[qb] = 0.f;
    lim[qb] = -FLT_MAX;
    l_run[qb] = 0.f;
  }
  int row_lo[C::QB], row_hi[C::QB], first_j[C::QB];
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    const RowBounds rb = row_bounds(wrow0 + 32 * qb + l32, Lq, wLk, p.causal, p.wl, p.wr);
    row_lo[qb] = wkoff + (int)imin64(rb.lo, (int64_t)wLk);
    row_hi[qb] = wkoff + (int)imax64(rb.hi, (int64_t)-1);
    first_j[qb] = row_lo[qb] <= row_hi[qb] ? row_lo[qb] / kBN - tr.kt_begin : -1;
  }
  // Scores of two tiles: sbuf[t % 2][qb][sb][r] = key 32 sb + 8 (r / 4) +
  // 4 g + r % 4, query l32.
  f32x16 sbuf[2][C::QB][kSB];
  i32x8 pf[C::QB];  // probabilities, PV B operand; zero until a wave's first computed tile
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) pf[qb] = i32x8{};

  auto load_op = [&](int i, int pv_ops, const lds_char* vs, const lds_char* ks, i32x8& dst) VA_INLINE {
    if (i < pv_ops) {  // V^T operand vb = i
      const i32x2 t0 = lds_read_tr8(vs, v_rd[i]);
      const i32x2 t1 = lds_read_tr8(vs, v_rd[i] + kVRead);
      const i32x2 t2 = lds_read_tr8(vs, v_rd[i] + 2 * kVRead);
      const i32x2 t3 = lds_read_tr8(vs, v_rd[i] + 3 * kVRead);
      dst = (i32x8){t0[0], t0[1], t1[0], t1[1], t2[0], t2[1], t3[0], t3[1]};
    } else {  // K operand (sb, c)
      const int o = i - pv_ops, sb = o / C::KC, c = o % C::KC;
      dst = lds_read_2xb128(ks, k_rd + (32 * sb * C::KPITCH + 4 * c) * 16);
    }
  };
  // MFMAs of one iteration without the interleaved softmax: PV of the
  // previous tile (if kPV) then QK^T of a tile into sn.
  auto mfma_ops = [&](const lds_char* vs, const lds_char* ks, f32x16 (&sn)[C::QB][kSB], auto pv_tag) VA_INLINE {
    constexpr bool kPV = decltype(pv_tag)::value;
    constexpr int kPVOps = kPV ? C::VB : 0;
    constexpr int kOps = kPVOps + kSB * C::KC;
    const f32x16 zero = {};
    i32x8 ring[kDepth];
#pragma unroll
    for (int i = 0; i < kDepth && i < kOps; ++i) load_op(i, kPVOps, vs, ks, ring[i]);
#pragma unroll
    for (int i = 0; i < kOps; ++i) {
      const i32x8 op = ring[i % kDepth];
      if (i + kDepth < kOps) load_op(i + kDepth, kPVOps, vs, ks, ring[i % kDepth]);
      if (i < kPVOps) {
#pragma unroll
        for (int qb = 0; qb < C::QB; ++qb) acc[i][qb] = mfma_e4m3(op, pf[qb], acc[i][qb]);
      } else {
        const int o = i - kPVOps, sb = o / C::KC, c = o % C::KC;
#pragma unroll
        for (int qb = 0; qb < C::QB; ++qb) sn[qb][sb] = mfma_e4m3(op, qf[qb][c], c == 0 ? zero : sn[qb][sb]);
      }
    }
  };
  auto mask = [&](int j, f32x16 (&s)[C::QB][kSB]) VA_INLINE {
    const int kt = tr.kt_begin + j;
    if ((unsigned)(j - w_full_begin) >= (unsigned)(w_full_end - w_full_begin)) {
      const int key0 = kt * kBN;
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb)
#pragma unroll
        for (int sb = 0; sb < kSB; ++sb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int jj = key0 + 32 * sb + 8 * (r >> 2) + 4 * g + (r & 3);
            s[qb][sb][r] = (jj >= row_lo[qb] && jj <= row_hi[qb]) ? s[qb][sb][r] : -INFINITY;
          }
    }
  };
  // Full online-softmax step of one tile (first tile and slow path): row max,
  // lazy-rescale decision, p, e4m3 pack into pf, fp32 row sum.
  auto softmax = [&](f32x16 (&s)[C::QB][kSB], float (&alpha)[C::QB]) VA_INLINE -> bool {
    float m_new[C::QB];
    bool need = false;
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) {
      float m = -INFINITY;
#pragma unroll
      for (int sb = 0; sb < kSB; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) m = fmaxf(m, s[qb][sb][r]);
      m_new[qb] = fmaxf(m_run[qb], xhalf_max(m) * sl2);
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
      for (int sb = 0; sb < kSB; ++sb)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          float x[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[e] = __builtin_amdgcn_exp2f(fmaf(s[qb][sb][4 * w + e], sl2, nm[qb]));
            sum += x[e];
          }
          pf[qb][4 * sb + w] = (int)pack_e4m3x4(x[0], x[1], x[2], x[3], (uint32_t)pf[qb][4 * sb + w]);
        }
      l_run[qb] = l_run[qb] * alpha[qb] + sum;
    }
    return move;
  };
  // One iteration's MFMAs and fast-path softmax, interleaved by hand (see
  // attn_fwd_wide's fused_block; the check is the row-sum one).  VALU units:
  // 16 exps per (query block, score block), then one unit per pair of
  // probabilities: e4m3 pack and pair sum.
  auto fused_block = [&](const lds_char* vs, const lds_char* ks, f32x16 (&s)[C::QB][kSB],
                         f32x16 (&sn)[C::QB][kSB], float (&sum)[C::QB], int j) VA_INLINE -> bool {
    constexpr int QB = C::QB;
    constexpr int kPVOps = C::VB, kOps = kPVOps + kSB * C::KC, kSlots = QB * kOps;
    constexpr int kExpU = 16 * kSB * QB, kPackU = 8 * kSB * QB;
    constexpr int kUnits = kExpU + kPackU;
    static_assert((kUnits - kPackU) * kSlots / kUnits >= QB * kPVOps, "packs must follow the PV MFMAs");
    bool bad = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) bad |= j == first_j[qb];
    auto unit = [&](auto uu) VA_INLINE {
      constexpr int u = decltype(uu)::value;
      if constexpr (u < kExpU) {  // p = exp2(s * scale - m_run), in place
        constexpr int qb = u / (16 * kSB), sb = (u / 16) % kSB, r = u % 16;
        s[qb][sb][r] = __builtin_amdgcn_exp2f(fmaf(s[qb][sb][r], sl2, nm[qb]));
      } else {  // e4m3 pack of a pair (and its sum)
        constexpr int i = u - kExpU, qb = i / (8 * kSB), sb = (i / 8) % kSB, pr = i % 8, r = 2 * pr;
        constexpr int w = 4 * sb + pr / 2;
        constexpr bool hi = pr % 2 == 1, first = sb == 0 && pr == 0, last = sb == kSB - 1 && pr == 7;
        // (straight into the PV operand: every PV MFMA reading it has issued)
        // (the low half's pack keeps the old high bytes, which the high half's replaces)
        pf[qb][w] = (int)pack_e4m3x2<hi>(s[qb][sb][r], s[qb][sb][r + 1], (uint32_t)pf[qb][w]);
        const float pair = s[qb][sb][r] + s[qb][sb][r + 1];
        sum[qb] = first ? pair : sum[qb] + pair;
        if constexpr (last) bad |= !(sum[qb] <= kSumLimit);
      }
    };
    const f32x16 zero = {};
    i32x8 ring[kDepth];
#pragma unroll
    for (int i = 0; i < kDepth; ++i) load_op(i, kPVOps, vs, ks, ring[i]);
    static_for<0, kOps>([&](auto oo) VA_INLINE {
      constexpr int i = decltype(oo)::value;
      const i32x8 op = ring[i % kDepth];
      if constexpr (i + kDepth < kOps) load_op(i + kDepth, kPVOps, vs, ks, ring[i % kDepth]);
      static_for<0, QB>([&](auto qq) VA_INLINE {
        constexpr int qb = decltype(qq)::value, slot = QB * i + qb;
        if constexpr (i < kPVOps) {
          acc[i][qb] = mfma_e4m3(op, pf[qb], acc[i][qb]);
        } else {
          constexpr int o = i - kPVOps, sb = o / C::KC, c = o % C::KC;
          sn[qb][sb] = mfma_e4m3(op, qf[qb][c], c == 0 ? zero : sn[qb][sb]);
        }
        static_for<slot * kUnits / kSlots, (slot + 1) * kUnits / kSlots>(unit);
        __builtin_amdgcn_sched_barrier(0);
      });
    });
    return __any(bad);
  };
  auto qk_only = [&](const lds_char* ks, f32x16 (&sn)[C::QB][kSB]) VA_INLINE {
    mfma_ops(nullptr, ks, sn, BoolTag<false>{});
  };
  auto rescale = [&](bool move, const float (&alpha)[C::QB]) VA_INLINE {
    if (move) {
      asm volatile("; lazy rescale" ::: "memory");
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb)
#pragma unroll
        for (int vb = 0; vb < C::VB; ++vb)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[vb][qb][r] *= alpha[qb];
    }
  };
  auto pv_tile = [&](const lds_char* vs) VA_INLINE {
#pragma unroll
    for (int vb = 0; vb < C::VB; ++vb) {
      i32x8 op;
      load_op(vb, C::VB, vs, nullptr, op);
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb) acc[vb][qb] = mfma_e4m3(op, pf[qb], acc[vb][qb]);
    }
  };

  // ---- main loop (the schedule of attn_fwd_wide) ----------------------------------
  if (ntiles > 0) {
    wait_landed(Int<kAhead - 1>{});  // tile 0
    lds_barrier();
    if (active && w_beg == 0) mfma_ops(nullptr, kst(Int<0>{}), sbuf[0], BoolTag<false>{});  // QK^T(0)
    wait_landed(Int<kAhead - 2>{});  // tile 1
    lds_barrier();
    {
      issue(Int<kAhead % kStages>{});
      if (active && w_first == 0) {
        mask(0, sbuf[0]);
        mfma_ops(nullptr, kst(Int<1>{}), sbuf[1], BoolTag<false>{});
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
            constexpr int cur = (U + 1) % 2;
            mask(j, sbuf[cur]);
            float sum[C::QB];
            const bool slow = fused_block(vst(Int<U % kStages>{}), kst(Int<(U + 2) % kStages>{}), sbuf[cur],
                                          sbuf[cur ^ 1], sum, j);
#pragma unroll
            for (int qb = 0; qb < C::QB; ++qb) {
              // (one register per operand: the host pass rejects a 256-bit one
              // and would silently drop the kernel)
#pragma unroll
              for (int e = 0; e < 8; ++e) asm volatile("" ::"v"(pf[qb][e]));
              asm volatile("" ::"v"(sum[qb]));
            }
            float l_prev[C::QB];
#pragma unroll
            for (int qb = 0; qb < C::QB; ++qb) {
              l_prev[qb] = l_run[qb];
              l_run[qb] += sum[qb];
            }
            if (slow) {
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
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (active && w_end == ntiles) {  // PV of the last tile, its stage picked at run time
      const int last = (ntiles - 1) % kStages;
      const lds_char* vs = vst(Int<0>{});
      static_for<1, kStages>([&](auto st) VA_INLINE {
        if (last == decltype(st)::value) vs = vst(st);
      });
      pv_tile(vs);
    }
  }

  // ---- epilogue ---------------------------------------------------------------
  if (p.num_splits > 1) {  // fp32 partial O * v_descale / l and the split's LSE
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) {
      const float l = xhalf_sum(l_run[qb]);
      const int row = wrow0 + 32 * qb + l32;
      const float inv = l > 0.f ? vsc / l : 0.f;
      float* dst = p.part_o + (((int64_t)split * p.total_q + q0 + row) * p.heads + h) * DV;
#pragma unroll
      for (int vb = 0; vb < C::VB; ++vb)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int dv = vb * 32 + 8 * jj + 4 * g;
          if (row < r1) {
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
    return;
  }
  const bool out_e4m3 = p.out_scale != nullptr;
  const float osc = out_e4m3 ? vsc / *p.out_scale : vsc;
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    const float l = xhalf_sum(l_run[qb]);
    const int row = wrow0 + 32 * qb + l32;
    const float inv = l > 0.f ? osc / l : 0.f;
    // Lane (row, g) holds d_v 8 jj + 4 g .. + 3 of each 32-wide block; a
    // swap with lane row ^ 32 over chunks (jj, jj + 1) leaves lane g with the
    // 8 contiguous values of chunk jj + g (see attn_fwd_wide's epilogue).
    if (out_e4m3) {
      uint8_t* dst = (uint8_t*)p.o + (int64_t)(q0 + row) * p.o_row + (int64_t)h * p.o_head;
      auto q4 = [&](const f32x16& a, int r) VA_INLINE -> uint32_t {
        return quant_e4m3x4(a[r], a[r + 1], a[r + 2], a[r + 3], inv);
      };
#pragma unroll
      for (int vb = 0; vb < C::VB; ++vb)
#pragma unroll
        for (int jp = 0; jp < 4; jp += 2) {
          const uint32_t x = q4(acc[vb][qb], 4 * jp), y = q4(acc[vb][qb], 4 * jp + 4);
          const auto sw = __builtin_amdgcn_permlane32_swap(x, y, false, false);
          const int dv = vb * 32 + 8 * (jp + g);
          if (row < r1) {
            const u32x2 o2 = {sw[0], sw[1]};
            *(u32x2*)(dst + dv) = o2;
          }
        }
    } else {
      uint16_t* dst = (uint16_t*)p.o + (int64_t)(q0 + row) * p.o_row + (int64_t)h * p.o_head;
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
          if (row < r1) {
            const u32x4 o4 = {s0[0], s1[0], s0[1], s1[1]};
            *(u32x4*)(dst + dv) = o4;
          }
        }
    }
    if (row < r1 && p.lse != nullptr && g == 0)
      p.lse[(int64_t)h * p.total_q + q0 + row] = l > 0.f ? (m_run[qb] + log2f(l)) * kLn2 : -INFINITY;
  }
}

// ---- host side ----------------------------------------------------------------
bool fp8_supported_dims(int dqk, int dv) {
  return (dqk == 64 && dv == 64) || (dqk == 128 && dv == 128) || (dqk == 192 && dv == 128);
}

template <int DQK, int DV>
static Variant fp8_variant_t(int mode) {
  using C = fp8k::Cfg<DQK, DV>;
  const void* fn = mode == kPackHeads      ? (const void*)&attn_fwd_fp8<DQK, DV, kPackHeads>
                   : mode == kPackSegments ? (const void*)&attn_fwd_fp8<DQK, DV, kPackSegments>
                                           : (const void*)&attn_fwd_fp8<DQK, DV, kPackNone>;
  return {fn, C::LDS_BYTES, C::BM, fp8k::kBN, C::THREADS, "attn_fwd_fp8", 1, 1};
}

Variant fp8_variant(int dqk, int dv, int pack_mode) {
  (void)dv;
  if (dqk == 64) return fp8_variant_t<64, 64>(pack_mode);
  if (dqk == 128) return fp8_variant_t<128, 128>(pack_mode);
  return fp8_variant_t<192, 128>(pack_mode);
}

}  // namespace va
