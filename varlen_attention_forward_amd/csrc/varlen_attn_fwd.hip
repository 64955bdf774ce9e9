// Fused variable-length attention forward for AMD Instinct MI355X (gfx950).
//
// One workgroup = 4 wavefronts (256 threads) owns BM = 4 * NQB * 32 query
// rows of one (segment, head).  It walks the key tiles the rows can see
// (tile_schedule.h), BN = 64 keys at a time:
//
//   global K/V tile --(registers, prefetched one tile ahead)--> LDS (double
//   buffered; V written transposed) --> S^T = K Q^T on v_mfma_f32_32x32x16_bf16
//   --> online softmax (exp2, log2(e)-prescaled scale, lazy rescale)
//   --> O^T += V^T P^T on the same MFMA --> epilogue: O = acc / l in bf16,
//   LSE = (m + log2 l) ln 2 in fp32.
//
// Scores are computed transposed (keys on the MFMA M axis, queries on N), so
// each lane holds one query column: the row max and row sum over the keys a
// lane holds are plain in-lane reductions, and only one cross-lane step (lane
// l with lane l ^ 32) is needed per tile.  The same layout makes the
// probability registers usable directly as the B operand of the PV product
// once the key order inside each 16-key group is permuted the same way for V.
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
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBN = 64;                 // keys per tile
constexpr float kRescaleTau = 8.0f;     // lazy rescale threshold, log2 units
constexpr float kLn2 = 0.6931471805599453f;

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const int32_t* cu_q;
  const int32_t* cu_k;
  int64_t q_row, q_head, k_row, k_head, v_row, v_head, o_row, o_head;
  int64_t total_q;
  int32_t batch, heads, n_qt, num_blocks;
  int32_t causal, wl, wr;
  float scale_log2;  // softmax_scale * log2(e)
};

template <int DQK, int DV, int NQB>
struct Cfg {
  static constexpr int DQKP = (DQK + 15) / 16 * 16;  // MFMA K granularity
  static constexpr int DVP = (DV + 31) / 32 * 32;    // 32-row MFMA blocks of V^T
  static constexpr int KC = DQKP / 16;               // k-chunks of the QK^T product
  static constexpr int VB = DVP / 32;                // dv blocks of the PV product
  static constexpr int BM = kWaves * NQB * 32;
  static constexpr int K_PITCH = DQKP + 8;   // +16 B per row: conflict-free column reads
  static constexpr int VT_PITCH = kBN + 8;   // V^T rows: 64 keys + 16 B
  static constexpr int K_TILE = kBN * K_PITCH;
  static constexpr int VT_TILE = DVP * VT_PITCH;
  static constexpr int LDS_ELEMS = 2 * (K_TILE + VT_TILE);
  static constexpr int K_CHUNKS = kBN * (DQKP / 8);       // 16-byte chunks per K tile
  static constexpr int K_ITERS = (K_CHUNKS + kThreads - 1) / kThreads;
  static constexpr int V_UNITS = (kBN / 4) * (DV / 8);    // 4 keys x 8 dv per unit
  static constexpr int V_ITERS = (V_UNITS + kThreads - 1) / kThreads;
};

// Position of key kappa (0..63) inside a V^T row: bits 2 and 3 swapped, so
// the 8 keys one lane feeds to one PV MFMA are adjacent (see file comment).
__device__ __forceinline__ int vt_pos(int kappa) {
  return (kappa & ~12) | ((kappa & 4) << 1) | ((kappa & 8) >> 1);
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

template <int DQK, int DV, int NQB>
__global__ __launch_bounds__(kThreads) void varlen_attn_fwd_kernel(Params p) {
  using C = Cfg<DQK, DV, NQB>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  // ---- work unit: XCD-aware remap, then (segment, head, q-tile) ----------
  // Consecutive workgroup ids are dispatched round-robin over the 8 XCDs;
  // give each XCD a contiguous run of work ids so the q-tiles of one
  // (segment, head) share that XCD's L2 while they stream the same K/V.
  const int w = blockIdx.x;
  const int N = p.num_blocks;
  const int per = N >> 3, rem = N & 7;
  const int xcd = w & 7, slot = w >> 3;
  const int lin = xcd * per + (xcd < rem ? xcd : rem) + slot;
  const int qt_idx = lin % p.n_qt;
  const int rest = lin / p.n_qt;
  const int h = rest % p.heads;
  const int b = rest / p.heads;
  // Causal: the last q-tiles see the most keys; start them first.
  const int qt = p.causal ? (p.n_qt - 1 - qt_idx) : qt_idx;

  const int q0 = p.cu_q[b];
  const int Lq = p.cu_q[b + 1] - q0;
  const int k0 = p.cu_k[b];
  const int Lk = p.cu_k[b + 1] - k0;
  const int r0 = qt * C::BM;
  if (r0 >= Lq) return;
  const int r1 = min(r0 + C::BM, Lq);
  const TileRange tr = tile_range(Lq, Lk, r0, r1, p.causal, p.wl, p.wr, kBN);

  const int wrow0 = r0 + wave * NQB * 32;

  // ---- Q fragments (B operand of S^T = K Q^T), kept in registers ---------
  bf16x8 qf[NQB][C::KC];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int row = wrow0 + qb * 32 + l32;
    const uint16_t* src = p.q + (int64_t)(q0 + row) * p.q_row + (int64_t)h * p.q_head;
#pragma unroll
    for (int c = 0; c < C::KC; ++c) {
      const int d = c * 16 + 8 * g;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (row < r1 && d < DQK) x = *(const u32x4*)(src + d);
      qf[qb][c] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // Padded V^T rows [DV, DVP) only feed output rows that are never stored;
  // clear them once so the LDS holds no stale data.
  if constexpr (C::DVP > DV) {
    constexpr int kPad = (C::DVP - DV) * C::VT_PITCH;
    for (int i = tid; i < 2 * kPad; i += kThreads) {
      const int bsel = i / kPad;
      lds[bsel * (C::K_TILE + C::VT_TILE) + C::K_TILE + DV * C::VT_PITCH + i % kPad] = 0;
    }
  }

  const uint16_t* kbase = p.k + (int64_t)k0 * p.k_row + (int64_t)h * p.k_head;
  const uint16_t* vbase = p.v + (int64_t)k0 * p.v_row + (int64_t)h * p.v_head;

  u32x4 kreg[C::K_ITERS];
  u32x4 vreg[C::V_ITERS][4];

  auto load_tile = [&](int t) {
    const int key0 = t * kBN;
#pragma unroll
    for (int i = 0; i < C::K_ITERS; ++i) {
      const int c = tid + i * kThreads;
      const int row = c / (C::DQKP / 8);
      const int col = (c % (C::DQKP / 8)) * 8;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (c < C::K_CHUNKS && key0 + row < Lk && col < DQK)
        x = *(const u32x4*)(kbase + (int64_t)(key0 + row) * p.k_row + col);
      kreg[i] = x;
    }
#pragma unroll
    for (int i = 0; i < C::V_ITERS; ++i) {
      const int u = tid + i * kThreads;
      const int kg = u & 15;
      const int dc = u >> 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = key0 + 4 * kg + e;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (u < C::V_UNITS && key < Lk) x = *(const u32x4*)(vbase + (int64_t)key * p.v_row + dc * 8);
        vreg[i][e] = x;
      }
    }
  };

  auto store_tile = [&](int buf) {
    uint16_t* ks = lds + buf * (C::K_TILE + C::VT_TILE);
    uint16_t* vts = ks + C::K_TILE;
#pragma unroll
    for (int i = 0; i < C::K_ITERS; ++i) {
      const int c = tid + i * kThreads;
      if (c < C::K_CHUNKS) {
        const int row = c / (C::DQKP / 8);
        const int col = (c % (C::DQKP / 8)) * 8;
        *(u32x4*)(ks + row * C::K_PITCH + col) = kreg[i];
      }
    }
#pragma unroll
    for (int i = 0; i < C::V_ITERS; ++i) {
      const int u = tid + i * kThreads;
      if (u < C::V_UNITS) {
        const int kg = u & 15;
        const int dc = u >> 4;
        const int pos = vt_pos(4 * kg);
#pragma unroll
        for (int dw = 0; dw < 4; ++dw) {
          // dv = dc*8 + 2*dw (low halves) and dc*8 + 2*dw + 1 (high halves)
          const uint32_t a0 = vreg[i][0][dw], a1 = vreg[i][1][dw];
          const uint32_t a2 = vreg[i][2][dw], a3 = vreg[i][3][dw];
          u32x2 lo, hi;
          lo[0] = __builtin_amdgcn_perm(a1, a0, 0x05040100u);
          lo[1] = __builtin_amdgcn_perm(a3, a2, 0x05040100u);
          hi[0] = __builtin_amdgcn_perm(a1, a0, 0x07060302u);
          hi[1] = __builtin_amdgcn_perm(a3, a2, 0x07060302u);
          const int dv = dc * 8 + 2 * dw;
          *(u32x2*)(vts + dv * C::VT_PITCH + pos) = lo;
          *(u32x2*)(vts + (dv + 1) * C::VT_PITCH + pos) = hi;
        }
      }
    }
  };

  // ---- running state -------------------------------------------------------
  f32x16 acc[C::VB][NQB];
#pragma unroll
  for (int vb = 0; vb < C::VB; ++vb)
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[vb][qb][r] = 0.f;
  float m_run[NQB], l_run[NQB];
  int row_lo[NQB], row_hi[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
    const RowBounds rb = row_bounds(wrow0 + qb * 32 + l32, Lq, Lk, p.causal, p.wl, p.wr);
    // clamp into int range: lo in [0, Lk], hi in [-1, Lk - 1]
    row_lo[qb] = (int)imin64(rb.lo, (int64_t)Lk);
    row_hi[qb] = (int)imax64(rb.hi, (int64_t)-1);
  }

  auto process_tile = [&](const uint16_t* ks, const uint16_t* vts, int key0, auto masked_tag) {
    constexpr bool kMasked = decltype(masked_tag)::value;
    // S^T = K Q^T : [keys 64 = 2 x 32] x [queries NQB x 32]
    f32x16 s[2][NQB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][qb][r] = 0.f;
#pragma unroll
    for (int c = 0; c < C::KC; ++c) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kf = *(const bf16x8*)(ks + (kb * 32 + l32) * C::K_PITCH + c * 16 + 8 * g);
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
          s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][c], s[kb][qb], 0, 0, 0);
      }
    }

    // Lane holds, for query column l32 of block qb, keys
    //   key0 + 32*kb + 8*(r/4) + 4*g + (r%4),  r = 0..15.
    if constexpr (kMasked) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = key0 + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
            const bool vis = (j >= row_lo[qb]) && (j <= row_hi[qb]);
            s[kb][qb][r] = vis ? s[kb][qb][r] : -INFINITY;
          }
    }

    float m_new[NQB];
    bool need = false;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      float mx = s[0][qb][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][qb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      m_new[qb] = fmaxf(m_run[qb], mx * p.scale_log2);
      need |= m_new[qb] > m_run[qb] + kRescaleTau;
    }
    if (__any(need)) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const float alpha = (m_new[qb] == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run[qb] - m_new[qb]);
        m_run[qb] = m_new[qb];
        l_run[qb] *= alpha;
#pragma unroll
        for (int vb = 0; vb < C::VB; ++vb)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[vb][qb][r] *= alpha;
      }
    }

    // P = exp2(s * scale*log2e - m), packed to bf16 as the PV B operand.
    bf16x8 pf[NQB][4];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const float m_use = (m_run[qb] == -INFINITY) ? 0.f : m_run[qb];
      float sum = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        u32x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 8 * (t & 1) + 2 * e;
          const float x0 = __builtin_amdgcn_exp2f(fmaf(s[t >> 1][qb][r], p.scale_log2, -m_use));
          const float x1 = __builtin_amdgcn_exp2f(fmaf(s[t >> 1][qb][r + 1], p.scale_log2, -m_use));
          sum += x0 + x1;
          pk[e] = pack_bf16x2(x0, x1);
        }
        pf[qb][t] = __builtin_bit_cast(bf16x8, pk);
      }
      l_run[qb] += sum;
    }

    // O^T += V^T P^T : [dv] x [queries], K = 16 keys per MFMA
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int vb = 0; vb < C::VB; ++vb) {
        const bf16x8 vf = *(const bf16x8*)(vts + (vb * 32 + l32) * C::VT_PITCH + 16 * t + 8 * g);
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
          acc[vb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qb][t], acc[vb][qb], 0, 0, 0);
      }
    }
  };


  if (tr.kt_begin < tr.kt_end) {
    load_tile(tr.kt_begin);
    store_tile(0);
  }
  __syncthreads();
  for (int t = tr.kt_begin; t < tr.kt_end; ++t) {
    const int buf = (t - tr.kt_begin) & 1;
    const bool more = t + 1 < tr.kt_end;
    if (more) load_tile(t + 1);
    const uint16_t* ks = lds + buf * (C::K_TILE + C::VT_TILE);
    const uint16_t* vts = ks + C::K_TILE;
    if (t >= tr.full_begin && t < tr.full_end)
      process_tile(ks, vts, t * kBN, BoolTag<false>{});
    else
      process_tile(ks, vts, t * kBN, BoolTag<true>{});
    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue ------------------------------------------------------------
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const float l = l_run[qb] + __shfl_xor(l_run[qb], 32);
    const int row = wrow0 + qb * 32 + l32;
    if (row < r1) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
      uint16_t* dst = p.o + (int64_t)(q0 + row) * p.o_row + (int64_t)h * p.o_head;
#pragma unroll
      for (int vb = 0; vb < C::VB; ++vb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int dv = vb * 32 + 8 * j + 4 * g;
          if (dv < DV) {
            u32x2 o2;
            o2[0] = pack_bf16x2(acc[vb][qb][4 * j] * inv, acc[vb][qb][4 * j + 1] * inv);
            o2[1] = pack_bf16x2(acc[vb][qb][4 * j + 2] * inv, acc[vb][qb][4 * j + 3] * inv);
            *(u32x2*)(dst + dv) = o2;
          }
        }
      if (p.lse != nullptr && g == 0) {
        const float lse = l > 0.f ? (m_run[qb] + log2f(l)) * kLn2 : -INFINITY;
        p.lse[(int64_t)h * p.total_q + q0 + row] = lse;
      }
    }
  }
}

}  // namespace va

// ============================================================================
// Host side: validation, launch-shape choice and the C entry points.
// ============================================================================
namespace va {

template <int DQK, int DV, int NQB>
static const void* kernel_ptr() {
  return (const void*)&varlen_attn_fwd_kernel<DQK, DV, NQB>;
}

struct Variant {
  const void* fn;
  int block_m;
  int lds_bytes;
};

template <int DQK, int DV>
static Variant pick_nqb(int nqb) {
  (void)nqb;
  return {kernel_ptr<DQK, DV, 1>(), Cfg<DQK, DV, 1>::BM, Cfg<DQK, DV, 1>::LDS_ELEMS * 2};
}

static bool supported_dims(int dqk, int dv) {
  return (dqk == 64 && dv == 64) || (dqk == 72 && dv == 72) || (dqk == 80 && dv == 80) ||
         (dqk == 128 && dv == 128) || (dqk == 192 && dv == 128);
}

// Query rows per wave, in 32-row blocks.  One block per wave for now: two
// blocks halve the LDS reads per MFMA but do not fit the register file
// without spilling in this loop structure.
static int choose_nqb(int max_seqlen_q) {
  (void)max_seqlen_q;
  return 1;
}

static Variant variant_for(int dqk, int dv, int nqb) {
  if (dqk == 64) return pick_nqb<64, 64>(nqb);
  if (dqk == 72) return pick_nqb<72, 72>(nqb);
  if (dqk == 80) return pick_nqb<80, 80>(nqb);
  if (dqk == 128) return pick_nqb<128, 128>(nqb);
  return pick_nqb<192, 128>(nqb);
}

static bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

static int check_tensor(const va_tensor* t, bool need_data) {
  if (t->row_stride <= 0 || t->head_stride <= 0) return VA_ERR_STRIDE;
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

extern "C" int varlen_attn_plan(int32_t head_dim_qk, int32_t head_dim_v, int32_t batch,
                                int32_t num_heads, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                int32_t causal, va_plan* plan) {
  (void)max_seqlen_k;
  (void)causal;
  if (!plan) return VA_ERR_NULL;
  if (!va::supported_dims(head_dim_qk, head_dim_v)) return VA_ERR_HEADDIM;
  if (batch < 0 || num_heads <= 0 || max_seqlen_q < 0) return VA_ERR_ARG;
  const va::Variant var = va::variant_for(head_dim_qk, head_dim_v, va::choose_nqb(max_seqlen_q));
  plan->block_m = var.block_m;
  plan->block_n = va::kBN;
  plan->threads = va::kThreads;
  plan->lds_bytes = var.lds_bytes;
  const int64_t n_qt = ((int64_t)max_seqlen_q + var.block_m - 1) / var.block_m;
  plan->grid = n_qt * num_heads * (int64_t)batch;
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

  const Variant var = variant_for(q->dim, v->dim, choose_nqb(max_seqlen_q));
  const int64_t n_qt = ((int64_t)max_seqlen_q + var.block_m - 1) / var.block_m;
  const int64_t grid = n_qt * q->heads * (int64_t)batch;
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
  p.num_blocks = (int32_t)grid;
  p.causal = causal;
  p.wl = window_left;
  p.wr = window_right;
  p.scale_log2 = softmax_scale * 1.4426950408889634f;

  void* args[] = {&p};
  const hipError_t err = hipLaunchKernel(var.fn, dim3((unsigned)grid), dim3(kThreads), args, 0,
                                         (hipStream_t)stream);
  return err == hipSuccess ? VA_OK : VA_ERR_LAUNCH;
}
