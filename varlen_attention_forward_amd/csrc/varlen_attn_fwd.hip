// Fused variable-length attention forward for AMD Instinct MI355X (gfx950).
//
// One workgroup = 8 wavefronts (512 threads, two per SIMD) owns BM = 256
// query rows of one (segment, head); each wave owns 32 of them.  It walks
// the key tiles those rows can see (tile_schedule.h), BN = 64 keys at a time:
//
//   HBM K/V tile --buffer_load ... lds (direct to LDS, out-of-range rows
//   read as zero)--> LDS, double buffered
//   --> S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (Q held in registers)
//   --> online softmax in registers (exp2 with a log2(e)-prescaled scale,
//       lazy rescale past a threshold)
//   --> O^T += V^T P^T on the same MFMA, V^T read with ds_read_b64_tr_b16
//   --> epilogue: O = acc / l in bf16, LSE = (m + log2 l) ln 2 in fp32.
//
// Scores are computed transposed (keys on the MFMA M axis, queries on N), so
// each lane holds one query column: the row max and row sum over the keys a
// lane holds are in-lane reductions with a single cross-lane step (lane l with
// lane l ^ 32) per tile.  The probability registers then serve directly as
// the B operand of the PV product, with the key order inside each 16-key
// group permuted identically on the V side.
//
// The two waves on each SIMD run half a tile apart (ping-pong), so one
// wave's softmax overlaps the other's MFMAs; K/V tiles stream into LDS two
// phases ahead of use.
//
// Where the pages describe FA4 on Blackwell (TMEM, tcgen05.ld.red row max,
// 2-CTA MMA) that design is prior art only; what carries over is the online
// softmax step with exp2 and a rescale threshold (SGLang PR #41344,
// "Modifications": softmax.py update_row_max, "fast exp2, rescale
// threshold") and masking only on the tiles that need it (same section: only
// unmasked steady-state tiles take the fast path).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "tile_schedule.h"
#include "varlen_attn.h"

namespace va {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;        // query rows per workgroup
constexpr int kBN = 64;                 // keys per tile
constexpr float kRescaleTau = 8.0f;     // lazy rescale threshold, log2 units
constexpr float kLn2 = 0.6931471805599453f;
constexpr uint32_t kOOB = 0x80000000u;  // buffer offset past every range: reads 0
constexpr int kBufferFlags = 0x00020000;  // raw buffer, 32-bit data format

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const int32_t* cu_q;
  const int32_t* cu_k;
  int64_t q_row, q_head, k_row, k_head, v_row, v_head, o_row, o_head;  // elements
  int64_t total_q;
  int32_t batch, heads, n_qt;
  int32_t causal, wl, wr;
  float scale_log2;  // softmax_scale * log2(e)
};

template <int DQK, int DV>
struct Cfg {
  static constexpr int DQKP = (DQK + 15) / 16 * 16;  // MFMA K granularity (72 -> 80)
  static constexpr int DVP = (DV + 31) / 32 * 32;    // 32-row V^T MFMA blocks (72, 80 -> 96)
  static constexpr int KC = DQKP / 16;               // k-chunks of the QK^T product
  static constexpr int VB = DVP / 32;                // dv blocks of the PV product
  // K tile: 64 rows of DQKP bf16 = CPR_K 16-byte chunks, plus one pad chunk
  // per row so the 32 rows an MFMA operand read touches hit distinct banks.
  static constexpr int CPR_K = DQKP / 8;
  static constexpr int KPITCH = CPR_K + 1;           // chunks per K row in LDS
  static constexpr int K_REAL = DQK / 8;             // chunks holding data
  // V tile: 64 rows of DVP bf16, chunk index XOR-swizzled per row so the
  // four rows a transposing read touches hit distinct banks.
  static constexpr int CPR_V = DVP / 8;
  static constexpr int V_REAL = DV / 8;
  static constexpr int K_TILE = kBN * KPITCH * 16;   // bytes
  static constexpr int V_TILE = kBN * CPR_V * 16;
  static constexpr int LDS_BYTES = 2 * (K_TILE + V_TILE);
  static constexpr int K_LOADS = (KPITCH + kWaves - 1) / kWaves;  // wave-loads per wave
  static constexpr int V_LOADS = (CPR_V + kWaves - 1) / kWaves;
  static_assert(CPR_V == 8 || CPR_V == 12 || CPR_V == 16, "V swizzle defined for 8/12/16 chunks");
};

// XOR applied to the chunk index of V row `row` (see Cfg).
template <int CPR_V>
__host__ __device__ constexpr int v_swizzle(int row) {
  return CPR_V == 16 ? 4 * (row & 3) : (CPR_V == 8 ? 4 * ((row >> 1) & 1) : 0);
}

// 16-byte-per-lane load from a buffer straight into LDS: lane i's bytes land
// at dst + 16 i; offsets past the buffer's range read as zero.  (A plain
// device function: inside the kernel template the builtin trips the host pass.)
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, lds_char* dst, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)dst, 16, off, 0, 0, 0);
}

template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (__bf16)a;  // round to nearest even
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// Value of lane l ^ 32 (the other half of the wave), without an LDS trip.
__device__ __forceinline__ float other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  // lanes 0-31 find the upper half's values in r[1], lanes 32-63 the lower
  // half's in r[0]
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

__device__ __forceinline__ bf16x8 lds_read_b128(const lds_char* base, int byte_off) {
  return *(const __attribute__((address_space(3))) bf16x8*)(base + byte_off);
}

__device__ __forceinline__ bf16x4 lds_read_tr(const lds_char* base, int byte_off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(base + byte_off));
}

template <int DQK, int DV>
__global__ __launch_bounds__(kThreads) void varlen_attn_fwd_kernel(Params p) {
  using C = Cfg<DQK, DV>;
  __shared__ __attribute__((aligned(1024))) char lds_raw[C::LDS_BYTES];
  lds_char* lds = (lds_char*)lds_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  // ---- work unit (see decode_block in tile_schedule.h) -------------------
  const WorkUnit wu = decode_block(blockIdx.x, p.batch, p.heads, p.n_qt, p.causal);
  if (!wu.valid) return;
  const int b = wu.b, h = wu.h, qt = wu.qt;

  const int q0 = p.cu_q[b];
  const int Lq = p.cu_q[b + 1] - q0;
  const int k0 = p.cu_k[b];
  const int Lk = p.cu_k[b + 1] - k0;
  const int r0 = qt * kBM;
  if (r0 >= Lq) return;
  const int r1 = min(r0 + kBM, Lq);
  const TileRange tr = tile_range(Lq, Lk, r0, r1, p.causal, p.wl, p.wr, kBN);
  const int ntiles = tr.kt_end - tr.kt_begin;
  const int wrow0 = r0 + wave * 32;
  const int myrow = wrow0 + l32;

  // ---- Q fragments (B operand of S^T = K Q^T), kept in registers ---------
  bf16x8 qf[C::KC];
  {
    const uint16_t* src = p.q + (int64_t)(q0 + myrow) * p.q_row + (int64_t)h * p.q_head;
#pragma unroll
    for (int c = 0; c < C::KC; ++c) {
      const int d = c * 16 + 8 * g;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (myrow < r1 && d < DQK) x = *(const u32x4*)(src + d);
      qf[c] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // ---- per-lane offsets of the direct-to-LDS tile loads --------------------
  // K wave-load j covers LDS chunk slots [64 j, 64 j + 64) of the tile; slot
  // s holds row s / KPITCH, chunk s % KPITCH (the last chunk of a row is pad).
  const int64_t k_row_b = p.k_row * 2, v_row_b = p.v_row * 2;
  uint32_t koff[C::K_LOADS];
  bool kact[C::K_LOADS];
#pragma unroll
  for (int i = 0; i < C::K_LOADS; ++i) {
    const int s = (wave + kWaves * i) * 64 + lane;
    const int row = s / C::KPITCH, c = s % C::KPITCH;
    kact[i] = c < C::CPR_K;
    koff[i] = c < C::K_REAL ? (uint32_t)(row * k_row_b + c * 16) : kOOB;  // 72: chunk 9 -> zeros
  }
  uint32_t voff[C::V_LOADS];
  bool vact[C::V_LOADS];
#pragma unroll
  for (int i = 0; i < C::V_LOADS; ++i) {
    const int s = (wave + kWaves * i) * 64 + lane;
    const int row = s / C::CPR_V;
    const int c = (s % C::CPR_V) ^ v_swizzle<C::CPR_V>(row);
    vact[i] = c < C::V_REAL;  // padded dv chunks are never loaded
    voff[i] = (uint32_t)(row * v_row_b + c * 16);
  }
  const char* kseg = (const char*)(p.k + (int64_t)k0 * p.k_row + (int64_t)h * p.k_head);
  const char* vseg = (const char*)(p.v + (int64_t)k0 * p.v_row + (int64_t)h * p.v_head);

  auto kbuf = [&](int i) { return lds + (i & 1) * (C::K_TILE + C::V_TILE); };
  auto vbuf = [&](int i) { return lds + (i & 1) * (C::K_TILE + C::V_TILE) + C::K_TILE; };

  auto load_k = [&](int tile, lds_char* dst) {
    const int key0 = tile * kBN;
    const int rows = min(Lk - key0, kBN);
    __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kseg + key0 * k_row_b), (short)0, (int)(rows * k_row_b), kBufferFlags);
#pragma unroll
    for (int i = 0; i < C::K_LOADS; ++i) {
      const int wl = wave + kWaves * i;
      if (wl < C::KPITCH && kact[i])
        dma16(rs, dst + wl * 1024, koff[i]);
    }
  };
  auto load_v = [&](int tile, lds_char* dst) {
    const int key0 = tile * kBN;
    const int rows = min(Lk - key0, kBN);
    __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(vseg + key0 * v_row_b), (short)0, (int)(rows * v_row_b), kBufferFlags);
#pragma unroll
    for (int i = 0; i < C::V_LOADS; ++i) {
      const int wl = wave + kWaves * i;
      if (wl < C::CPR_V && vact[i])
        dma16(rs, dst + wl * 1024, voff[i]);
    }
  };

  // ---- per-lane LDS read offsets -------------------------------------------
  // K operand: row kb*32 + l32, chunk 2c + g  ->  k_rd + kb*32*KPITCH*16 + 32c
  const int k_rd = (l32 * C::KPITCH + g) * 16;
  // V^T operand via transposing reads: lane i of 16-lane group G supplies
  // row (4g + i/4) [+ 16t + 8h], dv 32vb + 16(G%2) + 4(i%4).
  int v_rd[C::VB];
  {
    const int G = lane >> 4, i = lane & 15;
    const int vrow = 4 * g + (i >> 2);
    const int y = 2 * (G & 1) + ((i >> 1) & 1);
#pragma unroll
    for (int vb = 0; vb < C::VB; ++vb)
      v_rd[vb] = (vrow * C::CPR_V + ((4 * vb + y) ^ v_swizzle<C::CPR_V>(vrow))) * 16 + 8 * (i & 1);
  }

  // ---- running state -------------------------------------------------------
  f32x16 acc[C::VB];
#pragma unroll
  for (int vb = 0; vb < C::VB; ++vb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[vb][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  int row_lo, row_hi;
  {
    const RowBounds rb = row_bounds(myrow, Lq, Lk, p.causal, p.wl, p.wr);
    row_lo = (int)imin64(rb.lo, (int64_t)Lk);  // clamp into int range
    row_hi = (int)imax64(rb.hi, (int64_t)-1);
  }

  // S^T = K Q^T for one tile: [64 keys = 2 x 32] x [32 queries].
  auto qk = [&](const lds_char* ks, f32x16 (&s)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
    for (int c = 0; c < C::KC; ++c) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kf = lds_read_b128(ks, k_rd + kb * 32 * C::KPITCH * 16 + 32 * c);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], s[kb], 0, 0, 0);
      }
    }
  };

  // O^T += V^T P^T: [dv] x [32 queries], 16 keys per MFMA.
  auto pv = [&](const lds_char* vs, const bf16x8 (&pf)[4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int vb = 0; vb < C::VB; ++vb) {
        const bf16x4 lo = lds_read_tr(vs, v_rd[vb] + (16 * t) * C::CPR_V * 16);
        const bf16x4 hi = lds_read_tr(vs, v_rd[vb] + (16 * t + 8) * C::CPR_V * 16);
        const bf16x8 vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        acc[vb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[t], acc[vb], 0, 0, 0);
      }
    }
  };

  // Online softmax of one tile of scores.  The lane holds query l32 and keys
  // key0 + 32 kb + 8 (r / 4) + 4 g + r % 4; it leaves the probabilities in
  // pf, packed to bf16 as the B operand of the PV product.
  auto softmax = [&](f32x16 (&s)[2], bf16x8 (&pf)[4], int key0, auto masked_tag) {
    constexpr bool kMasked = decltype(masked_tag)::value;
    if constexpr (kMasked) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = key0 + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
          s[kb][r] = (j >= row_lo && j <= row_hi) ? s[kb][r] : -INFINITY;
        }
    }
    float mx = fmaxf(s[0][0], s[1][0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(s[0][r], s[1][r]));
    mx = fmaxf(mx, other_half(mx));
    const float m_new = fmaxf(m_run, mx * p.scale_log2);
    if (__any(m_new > m_run + kRescaleTau)) {
      // Keeps the rescale a real branch: it is rare, and speculating it
      // would put 16 * VB multiplies on every tile.
      asm volatile("; lazy rescale" ::: "memory");
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int vb = 0; vb < C::VB; ++vb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[vb][r] *= alpha;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    float sum = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      u32x4 pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 8 * (t & 1) + 2 * e;
        const float x0 = __builtin_amdgcn_exp2f(fmaf(s[t >> 1][r], p.scale_log2, -m_use));
        const float x1 = __builtin_amdgcn_exp2f(fmaf(s[t >> 1][r + 1], p.scale_log2, -m_use));
        sum += x0 + x1;
        pk[e] = pack_bf16x2(x0, x1);
      }
      pf[t] = __builtin_bit_cast(bf16x8, pk);
    }
    l_run += sum;
  };

  // ---- ping-pong main loop -------------------------------------------------
  // Waves 0-3 (group 0) and 4-7 (group 1) put one wave of each group on
  // every SIMD.  Each wave alternates an MFMA phase (PV of the previous tile,
  // then QK^T of the current one) and a VALU phase (softmax of the current
  // tile).  Group 1 runs one phase behind group 0, and every phase ends at a
  // workgroup barrier, so in each slot one wave per SIMD is in its MFMA phase
  // while the other is in its softmax.
  //
  // Tile j (counted from kt_begin) has K in kbuf(j) and V in vbuf(j).  The
  // MFMA phase of tile j reads K_j and V_{j-1}; in slot 2j (the slot where
  // group 0 starts tile j) every wave issues its share of the loads of K_{j+1}
  // and V_j, and waits for them at the end of slot 2j + 1, so they are
  // visible from slot 2j + 2 on.  Those buffers last held K_{j-1} and
  // V_{j-2}, whose readers finished by slot 2j - 1.
  const int grp = wave >> 2;
  auto issue_loads = [&](int j) {  // K_{j+1} and V_j
    if (j + 1 < ntiles) load_k(tr.kt_begin + j + 1, kbuf(j + 1));
    if (j < ntiles) load_v(tr.kt_begin + j, vbuf(j));
  };
  auto wait_loads = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  if (ntiles > 0) {
    f32x16 s[2];
    bf16x8 pf[4];
    // One MFMA phase as a single stream of MFMAs: the PV product of the
    // previous tile (4 * VB MFMAs) then QK^T of this one (2 * KC).  Each MFMA's
    // LDS operand is read kDepth MFMAs ahead into a ring of registers, and
    // scheduling barriers keep that order, so every 32-cycle MFMA finds its
    // operand waiting instead of stalling on LDS latency.
    auto mfma_phase = [&](int j, auto pv_tag) {  // slot 2j + grp
      constexpr bool kPV = decltype(pv_tag)::value;
      constexpr int kPVOps = kPV ? 4 * C::VB : 0;
      constexpr int kOps = kPVOps + 2 * C::KC;
      constexpr int kDepth = 6;
      if (grp == 0) issue_loads(j);
      const lds_char* vs = vbuf(j - 1);
      const lds_char* ks = kbuf(j);
      auto load_op = [&](int i, bf16x8& dst) {
        if (i < kPVOps) {  // V^T operand of PV MFMA (t, vb)
          const int t = i / C::VB, vb = i % C::VB;
          const bf16x4 lo = lds_read_tr(vs, v_rd[vb] + (16 * t) * C::CPR_V * 16);
          const bf16x4 hi = lds_read_tr(vs, v_rd[vb] + (16 * t + 8) * C::CPR_V * 16);
          dst = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        } else {  // K operand of QK MFMA (c, kb)
          const int c = (i - kPVOps) / 2, kb = (i - kPVOps) % 2;
          dst = lds_read_b128(ks, k_rd + kb * 32 * C::KPITCH * 16 + 32 * c);
        }
      };
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
      bf16x8 ring[kDepth];
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int i = 0; i < kDepth && i < kOps; ++i) load_op(i, ring[i]);
#pragma unroll
      for (int i = 0; i < kOps; ++i) {
        if (i < kPVOps) {
          const int t = i / C::VB, vb = i % C::VB;
          acc[vb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[i % kDepth], pf[t], acc[vb], 0, 0, 0);
        } else {
          const int c = (i - kPVOps) / 2, kb = (i - kPVOps) % 2;
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[i % kDepth], qf[c], s[kb], 0, 0, 0);
        }
        if (i + kDepth < kOps) load_op(i + kDepth, ring[i % kDepth]);
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
      if (grp == 1) wait_loads();
      __syncthreads();
    };
    auto valu_phase = [&](int j, auto masked_tag) {  // slot 2j + 1 + grp
      if (grp == 1) issue_loads(j + 1);
      softmax(s, pf, (tr.kt_begin + j) * kBN, masked_tag);
      if (grp == 0) wait_loads();
      __syncthreads();
    };
    load_k(tr.kt_begin, kbuf(0));
    wait_loads();
    __syncthreads();
    if (grp == 1) {  // slot 0 for group 1: issue its loads of K_1, V_0
      issue_loads(0);
      __syncthreads();
    }
    // Tile 0, then tiles [1, a) masked, [a, b) unmasked, [b, ntiles) masked:
    // masked tiles only sit at the two ends of the visited range.
    mfma_phase(0, BoolTag<false>{});
    if (tr.kt_begin >= tr.full_begin && tr.kt_begin < tr.full_end)
      valu_phase(0, BoolTag<false>{});
    else
      valu_phase(0, BoolTag<true>{});
    const int a = min(max(tr.full_begin - tr.kt_begin, 1), ntiles);
    const int bnd = min(max(tr.full_end - tr.kt_begin, a), ntiles);
    int j = 1;
    for (; j < a; ++j) {
      mfma_phase(j, BoolTag<true>{});
      valu_phase(j, BoolTag<true>{});
    }
    for (; j < bnd; ++j) {
      mfma_phase(j, BoolTag<true>{});
      valu_phase(j, BoolTag<false>{});
    }
    for (; j < ntiles; ++j) {
      mfma_phase(j, BoolTag<true>{});
      valu_phase(j, BoolTag<true>{});
    }
    pv(vbuf(ntiles - 1), pf);
    if (grp == 0) __syncthreads();  // matches group 1's extra slot-0 barrier
  }

  // ---- epilogue ------------------------------------------------------------
  const float l = l_run + other_half(l_run);
  if (myrow < r1) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    uint16_t* dst = p.o + (int64_t)(q0 + myrow) * p.o_row + (int64_t)h * p.o_head;
#pragma unroll
    for (int vb = 0; vb < C::VB; ++vb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int dv = vb * 32 + 8 * j + 4 * g;
        if (dv < DV) {
          u32x2 o2;
          o2[0] = pack_bf16x2(acc[vb][4 * j] * inv, acc[vb][4 * j + 1] * inv);
          o2[1] = pack_bf16x2(acc[vb][4 * j + 2] * inv, acc[vb][4 * j + 3] * inv);
          *(u32x2*)(dst + dv) = o2;
        }
      }
    if (p.lse != nullptr && g == 0) {
      const float lse = l > 0.f ? (m_run + log2f(l)) * kLn2 : -INFINITY;
      p.lse[(int64_t)h * p.total_q + q0 + myrow] = lse;
    }
  }
}

}  // namespace va

// ============================================================================
// Host side: validation, launch-shape choice and the C entry points.
// ============================================================================
namespace va {

template <int DQK, int DV>
static const void* kernel_ptr() {
  return (const void*)&varlen_attn_fwd_kernel<DQK, DV>;
}

struct Variant {
  const void* fn;
  int lds_bytes;
};

static bool supported_dims(int dqk, int dv) {
  return (dqk == 64 && dv == 64) || (dqk == 72 && dv == 72) || (dqk == 80 && dv == 80) ||
         (dqk == 128 && dv == 128) || (dqk == 192 && dv == 128);
}

static Variant variant_for(int dqk, int dv) {
  if (dqk == 64) return {kernel_ptr<64, 64>(), Cfg<64, 64>::LDS_BYTES};
  if (dqk == 72) return {kernel_ptr<72, 72>(), Cfg<72, 72>::LDS_BYTES};
  if (dqk == 80) return {kernel_ptr<80, 80>(), Cfg<80, 80>::LDS_BYTES};
  if (dqk == 128) return {kernel_ptr<128, 128>(), Cfg<128, 128>::LDS_BYTES};
  return {kernel_ptr<192, 128>(), Cfg<192, 128>::LDS_BYTES};
}

static bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

// Row strides above 2^24 elements would overflow the 32-bit offsets of the
// per-tile buffer loads (64 rows x stride x 2 bytes).
static constexpr int64_t kMaxRowStride = (int64_t)1 << 24;

static int check_tensor(const va_tensor* t, bool need_data) {
  if (t->row_stride <= 0 || t->head_stride <= 0 || t->row_stride > kMaxRowStride) return VA_ERR_STRIDE;
  if ((t->row_stride & 7) != 0 || (t->head_stride & 7) != 0) return VA_ERR_ALIGN;
  if (need_data && t->data == nullptr) return VA_ERR_NULL;
  if (!aligned16(t->data)) return VA_ERR_ALIGN;
  return VA_OK;
}

}  // namespace va

extern "C" const char* varlen_attn_status_string(int status) {
  switch (status) {
    case VA_OK: return "ok";
    case VA_ERR_NULL: return "a required pointer is NULL";
    case VA_ERR_SHAPE: return "tensor rows/heads/dims disagree or a size is out of range";
    case VA_ERR_HEADDIM: return "unsupported (head_dim_qk, head_dim_v); supported: (64,64) (72,72) (80,80) (128,128) (192,128)";
    case VA_ERR_STRIDE: return "a row or head stride is not positive";
    case VA_ERR_ALIGN: return "a data pointer or stride is not a multiple of 16 bytes (lse: 4 bytes)";
    case VA_ERR_ARG: return "a scalar argument is out of range";
    case VA_ERR_LAUNCH: return "the HIP kernel launch failed";
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

extern "C" int varlen_attn_work_unit(int64_t block, int32_t batch, int32_t num_heads,
                                     int32_t max_seqlen_q, int32_t causal, int32_t* segment,
                                     int32_t* head, int32_t* q_tile) {
  if (!segment || !head || !q_tile) return VA_ERR_NULL;
  if (batch < 0 || num_heads <= 0 || max_seqlen_q <= 0 || (causal != 0 && causal != 1)) return VA_ERR_ARG;
  const int64_t n_qt = ((int64_t)max_seqlen_q + va::kBM - 1) / va::kBM;
  if (block < 0 || block >= va::grid_blocks(batch, num_heads, n_qt)) return VA_ERR_ARG;
  const va::WorkUnit u = va::decode_block(block, batch, num_heads, n_qt, causal);
  *segment = u.valid ? u.b : -1;
  *head = u.valid ? u.h : -1;
  *q_tile = u.valid ? u.qt : -1;
  return VA_OK;
}

extern "C" int varlen_attn_plan(int32_t head_dim_qk, int32_t head_dim_v, int32_t batch,
                                int32_t num_heads, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                int32_t causal, va_plan* plan) {
  (void)max_seqlen_k;
  (void)causal;
  if (!plan) return VA_ERR_NULL;
  if (!va::supported_dims(head_dim_qk, head_dim_v)) return VA_ERR_HEADDIM;
  if (batch < 0 || num_heads <= 0 || max_seqlen_q < 0) return VA_ERR_ARG;
  const va::Variant var = va::variant_for(head_dim_qk, head_dim_v);
  plan->block_m = va::kBM;
  plan->block_n = va::kBN;
  plan->threads = va::kThreads;
  plan->lds_bytes = var.lds_bytes;
  const int64_t n_qt = ((int64_t)max_seqlen_q + va::kBM - 1) / va::kBM;
  plan->grid = va::grid_blocks(batch, num_heads, n_qt);
  plan->kernel = "varlen_attn_fwd_kernel";
  return VA_OK;
}

extern "C" int varlen_attn_fwd(const va_tensor* q, const va_tensor* k, const va_tensor* v,
                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t batch,
                               int32_t max_seqlen_q, int32_t max_seqlen_k, float softmax_scale,
                               int32_t causal, int32_t window_left, int32_t window_right,
                               const va_tensor* out, float* lse, void* stream) {
  using namespace va;
  if (!q || !k || !v || !out) return VA_ERR_NULL;
  if (batch < 0 || max_seqlen_q < 0 || max_seqlen_k < 0) return VA_ERR_ARG;
  if (!(softmax_scale > 0.f) || !isfinite(softmax_scale)) return VA_ERR_ARG;
  if (causal != 0 && causal != 1) return VA_ERR_ARG;
  if (window_left < -1 || window_right < -1) return VA_ERR_ARG;
  if (q->heads <= 0 || k->heads != q->heads || v->heads != q->heads || out->heads != q->heads)
    return VA_ERR_SHAPE;
  if (q->rows < 0 || k->rows < 0 || v->rows != k->rows || out->rows != q->rows) return VA_ERR_SHAPE;
  if (q->rows > INT32_MAX || k->rows > INT32_MAX) return VA_ERR_SHAPE;
  if (k->dim != q->dim || out->dim != v->dim) return VA_ERR_SHAPE;
  if (!supported_dims(q->dim, v->dim)) return VA_ERR_HEADDIM;
  const bool has_q = q->rows > 0, has_k = k->rows > 0;
  int st;
  if ((st = check_tensor(q, has_q)) != VA_OK) return st;
  if ((st = check_tensor(k, has_k)) != VA_OK) return st;
  if ((st = check_tensor(v, has_k)) != VA_OK) return st;
  if ((st = check_tensor(out, has_q)) != VA_OK) return st;
  if (lse != nullptr && ((uintptr_t)lse & 3u) != 0) return VA_ERR_ALIGN;
  if (batch == 0 || max_seqlen_q == 0 || q->rows == 0) return VA_OK;
  if (!cu_seqlens_q || !cu_seqlens_k) return VA_ERR_NULL;

  const Variant var = variant_for(q->dim, v->dim);
  const int64_t n_qt = ((int64_t)max_seqlen_q + kBM - 1) / kBM;
  const int64_t grid = grid_blocks(batch, q->heads, n_qt);
  if (grid > INT32_MAX) return VA_ERR_SHAPE;

  Params p;
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
  p.n_qt = (int32_t)n_qt;
  p.causal = causal;
  p.wl = window_left;
  p.wr = window_right;
  p.scale_log2 = softmax_scale * 1.4426950408889634f;

  void* args[] = {&p};
  const hipError_t err = hipLaunchKernel(var.fn, dim3((unsigned)grid), dim3(kThreads), args, 0,
                                         (hipStream_t)stream);
  return err == hipSuccess ? VA_OK : VA_ERR_LAUNCH;
}
