// Device-side pieces shared by the attention kernels (bf16 and fp8 e4m3
// inputs): kernel parameters, the direct-to-LDS load, the workgroup barrier,
// the work-unit decode and cross-half lane reductions; plus the host-side
// description of a kernel instantiation.
#pragma once

#include <hip/hip_runtime.h>
#include <float.h>
#include <math.h>
#include <stdint.h>

#include "tile_schedule.h"
#include "varlen_attn.h"

// Kernel-local lambdas must inline: out-of-line copies would pass the
// register arrays they capture through scratch memory.
#define VA_INLINE __attribute__((always_inline))

namespace va {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr float kRescaleTau = 8.0f;     // lazy rescale threshold, log2 units
constexpr float kSumLimit = 256.0f;     // 2^kRescaleTau: a tile row sum this small bounds every p
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
  int32_t heads_k;  // KV heads; heads is a multiple of it
  // Split-KV: with num_splits > 1 the grid holds num_splits copies of the
  // n_units work units; copy s takes the s-th of num_splits equal runs of
  // each unit's key tiles and writes a normalised fp32 partial O and its
  // LSE instead of out / lse (combined by combine_splits).
  int32_t num_splits, n_units;
  // Optional per-segment split counts [batch] (device; null: num_splits for
  // every segment).  Only with launches of one segment per workgroup.
  const int32_t* splits_dyn;
  int32_t pack;  // segments, or query heads, per workgroup (segments_per_block): 1, 2 or 4
  int32_t pack_shift;  // log2(pack)
  // Work-unit decode, set up on the host: the head count the dealing runs
  // over (query heads, or groups of pack query heads of one KV head), the
  // q-tiles per (segment, head) group, the KV heads, and the query heads
  // per KV head, as FastDivs; the segment count the dealing runs over
  // (groups of pack segments when packed); the group size query_head takes.
  FastDiv fd_heads, fd_nqt, fd_heads_k, fd_group;
  int32_t n_dealt, qh_group;
  int32_t hg_shift;  // log2 of the heads dealt together (head_group_shift); fd_heads
                     // then counts head groups and fd_nqt workgroups per group
  // Causal q-tile pairing (attn_fwd_wide, unsplit, unpacked): a work unit's
  // q-tile index t stands for the pair of q-tiles n_b - 1 - t and t of its
  // segment (n_b = ceil(Lq / block_m)), so that every workgroup of a causal
  // launch has the same number of key tiles; n_qt then counts pairs.
  int32_t pair_qt;
  // attn_fwd_short on small launches: the waves of a workgroup that share one
  // work unit (64 query rows) and split its key tiles (1: a unit per wave).
  int32_t key_split;
  float* part_o;    // [num_splits, total_q, heads, d_v]
  float* part_lse;  // [num_splits, heads, total_q]
  int32_t causal, wl, wr;
  float scale_log2;  // softmax_scale * log2(e)
  // fp8 e4m3 inputs only: descales per (segment, KV head), [batch, heads_k]
  // fp32 each, null meaning 1; out_scale (one fp32) non-null when out holds
  // e4m3 codes of O / *out_scale instead of bf16.
  const float* q_descale;
  const float* k_descale;
  const float* v_descale;
  const float* out_scale;
};

// How the bf16 kernels form the row sum of the probabilities: an fp32 sum of
// the fp32 probabilities (kF32), or, for d_v 72 and 80 without an LSE, a
// column of ones in the padded V tile, which makes the PV product accumulate
// the sum of the bf16 probabilities it multiplies alongside O with no VALU
// work (kMfma).  O only needs the sum to normalise what the PV product
// accumulated, so the bf16 sum serves it; a bf16 sum can move the LSE by up
// to ln(1 + 2^-9), which is why an LSE keeps the fp32 sum.
enum class RowSum { kF32, kMfma };

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

template <int N>
struct Int {
  static constexpr int value = N;
};

// f(Int<I>{}), ..., f(Int<N - 1>{}) in order, unrolled.
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(Int<I>{});
    static_for<I + 1, N>(f);
  }
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (__bf16)a;  // round to nearest even
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}


// Workgroup barrier without __syncthreads()'s release/acquire fences.  With
// LDS-DMA in flight the release fence turns into s_waitcnt vmcnt(0), making
// every wave wait for the prefetch it has just issued; the kernels that use
// this wait for the loads a barrier must cover themselves.  LDS reads are
// drained first so no stage is overwritten under a read still in flight,
// and the empty asm statements keep the compiler from moving memory
// accesses across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// This workgroup's work unit (tile_schedule.h) and its segment's bounds:
// longest-first dealing when it applies, computed by every wave from
// cu_seqlens with one lane per segment (whose loads then also give the
// bounds); else dealing in packing order.
struct BlockWork {
  WorkUnit u;
  int q0, lq, k0, lk;  // the segment's first query / key row and lengths
};

template <int PK>
__device__ __forceinline__ BlockWork block_work(const Params& p, int lane, int block_m, int64_t w) {
  BlockWork r;
  if constexpr (PK == kPackHeads) {
    // (segment, group of pack query heads of one KV head): the group index
    // takes the place of the head in the dealing, and query_head keeps a KV
    // head's groups on one XCD; r.u.h is the group's first query head.
    r.u = decode_block((uint32_t)w, (uint32_t)p.n_dealt, p.fd_heads, p.fd_nqt, 0u, p.causal);
    r.u.h = query_head(r.u.h, p.fd_heads_k, p.qh_group) << p.pack_shift;
    if (r.u.valid) {
      r.q0 = p.cu_q[r.u.b];
      r.lq = p.cu_q[r.u.b + 1] - r.q0;
      r.k0 = p.cu_k[r.u.b];
      r.lk = p.cu_k[r.u.b + 1] - r.k0;
    }
    return r;
  }
  if constexpr (PK == kPackSegments) {  // a group of pack short segments: one unit per (group, head), in packing order
    r.u = decode_block((uint32_t)w, (uint32_t)p.n_dealt, p.fd_heads, p.fd_nqt, (uint32_t)p.hg_shift, p.causal);
    r.u.h = query_head(r.u.h, p.fd_heads_k, p.qh_group);
    if (r.u.valid) {
      const int first = r.u.b << p.pack_shift, last = min(first + p.pack, p.batch);
      r.q0 = p.cu_q[first];
      r.lq = p.cu_q[last] - r.q0;
      r.k0 = p.cu_k[first];
      r.lk = p.cu_k[last] - r.k0;
    }
    return r;
  }
  if (p.batch <= kLptMaxBatch) {
    int cq0 = 0, cq1 = 0, ck0 = 0, ck1 = -1;
    if (lane < p.batch) {
      cq0 = p.cu_q[lane];
      cq1 = p.cu_q[lane + 1];
      ck0 = p.cu_k[lane];
      ck1 = p.cu_k[lane + 1];
    }
    const int lq = cq1 - cq0, lk = ck1 - ck0;  // lk = -1 on lanes past the batch
    const int lq0 = __builtin_amdgcn_readfirstlane(lq), lk0 = __builtin_amdgcn_readfirstlane(lk);
    if (__ballot(lane < p.batch && (lq != lq0 || lk != lk0)) != 0) {
      const int x = (int)(w & 7);
      const int k = (int)snake_quads((uint32_t)(w >> 3), (uint32_t)p.n_units / 8u);
      int rank = 0;
      for (int j = 0; j < p.batch; ++j) {
        const int kj = __builtin_amdgcn_readlane(lk, j);
        rank += (kj > lk || (kj == lk && j < lane)) ? 1 : 0;
      }
      const int nqt1 = lane < p.batch ? (lq + block_m - 1) / block_m : 0;
      const int nqt = p.pair_qt ? (nqt1 + 1) >> 1 : nqt1;  // q-tiles, or pairs of them
      const int hgroups = p.heads >> p.hg_shift;
      const int h0 = xcd_first_head(rank, hgroups, x);
      const int n = xcd_head_count(h0, hgroups) * (nqt << p.hg_shift);
      int pre = 0;  // blocks of this XCD before this segment's
      for (int j = 0; j < p.batch; ++j)
        pre += __builtin_amdgcn_readlane(rank, j) < rank ? __builtin_amdgcn_readlane(n, j) : 0;
      const uint64_t hit = __ballot(lane < p.batch && k >= pre && k < pre + n);
      r.u.valid = hit != 0;
      r.u.b = r.u.h = r.u.qt = -1;
      if (hit != 0) {
        const int i = (int)__builtin_ctzll(hit);
        const int local = k - __builtin_amdgcn_readlane(pre, i);
        const int nq = __builtin_amdgcn_readlane(nqt, i);
        const int per = nq << p.hg_shift;
        const int grp = local / per, rem = local - grp * per, qi = rem >> p.hg_shift;
        r.u.b = i;
        r.u.h = query_head(((__builtin_amdgcn_readlane(h0, i) + 8 * grp) << p.hg_shift) + (rem & ((1 << p.hg_shift) - 1)),
                           p.fd_heads_k, p.qh_group);
        r.u.qt = p.causal ? nq - 1 - qi : qi;
      }
    } else {
      r.u = decode_block((uint32_t)w, (uint32_t)p.n_dealt, p.fd_heads, p.fd_nqt, (uint32_t)p.hg_shift, p.causal);
      r.u.h = query_head(r.u.h, p.fd_heads_k, p.qh_group);
    }
    if (r.u.valid) {
      const int b = __builtin_amdgcn_readfirstlane(r.u.b);
      r.q0 = __builtin_amdgcn_readlane(cq0, b);
      r.lq = __builtin_amdgcn_readlane(lq, b);
      r.k0 = __builtin_amdgcn_readlane(ck0, b);
      r.lk = __builtin_amdgcn_readlane(lk, b);
    }
    return r;
  }
  r.u = decode_block((uint32_t)w, (uint32_t)p.n_dealt, p.fd_heads, p.fd_nqt, (uint32_t)p.hg_shift, p.causal);
  r.u.h = query_head(r.u.h, p.fd_heads_k, p.qh_group);
  if (r.u.valid) {
    const int b = __builtin_amdgcn_readfirstlane(r.u.b);
    r.q0 = p.cu_q[b];
    r.lq = p.cu_q[b + 1] - r.q0;
    r.k0 = p.cu_k[b];
    r.lk = p.cu_k[b + 1] - r.k0;
  }
  return r;
}

__device__ __forceinline__ bf16x8 lds_read_b128(const lds_char* base, int byte_off) {
  return *(const __attribute__((address_space(3))) bf16x8*)(base + byte_off);
}

constexpr float kE4M3Max = 448.f;  // largest finite e4m3 value

// Two fp32 values to e4m3 (round to nearest even) in bytes 2 HI, 2 HI + 1 of
// `old`, the other two bytes kept.
template <bool HI>
__device__ __forceinline__ uint32_t pack_e4m3x2(float a, float b, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}
// Four fp32 values to e4m3 bytes 0-3.  The second pack replaces the two
// bytes the first one keeps, so `reg` (the destination's old value) only
// spares the compiler a zeroing move.
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d, uint32_t reg = 0u) {
  return pack_e4m3x2<true>(c, d, pack_e4m3x2<false>(a, b, reg));
}


// e4m3 codes of four values times `scale`, clamped to +-448 first (the
// static per-tensor output quantisation).
__device__ __forceinline__ uint32_t quant_e4m3x4(float a, float b, float c, float d, float scale) {
  auto q = [scale](float x) { return fminf(fmaxf(x * scale, -kE4M3Max), kE4M3Max); };
  return pack_e4m3x4(q(a), q(b), q(c), q(d));
}

// Cross-half (lane l and lane l ^ 32) max and sum: v_permlane32_swap
// leaves lane l's and lane l ^ 32's values in the two results.
__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Lane l ^ 32's value for lanes 32-63, the lane's own for lanes 0-31:
// broadcasts what lanes 0-31 hold to the whole wave.
__device__ __forceinline__ float from_lower_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]);
}

// One kernel instantiation and its launch shape.
struct Variant {
  const void* fn;
  int lds_bytes;
  int block_m;
  int block_n;
  int threads;
  const char* name;
  int per_cu;  // workgroups a compute unit holds at once (the launch bounds' minimum)
  int units_per_wg;  // work units a workgroup holds (its waves' own units; 1 but for attn_fwd_short)
  int key_split = 1;  // waves that split one unit's key tiles (attn_fwd_short on small launches: 4)
};

// The fp8 e4m3 kernel (varlen_attn_fwd_fp8.hip): whether it has an
// instantiation for (dqk, dv), and that instantiation.
bool fp8_supported_dims(int dqk, int dv);
Variant fp8_variant(int dqk, int dv, int pack_mode);
// The one-wave short-segment kernel (varlen_attn_short.hip): head dims it
// has, and its variant (lse: whether the call returns the LSE).
bool short_supported(int dqk, int dv);
Variant short_variant(int dqk, int dv, bool lse);
// The same kernel with a workgroup's four waves on one unit, each taking a
// quarter of its key tiles (launches too small to fill the CUs otherwise).
Variant short_key_split_variant(int dqk, int dv, bool lse);

}  // namespace va
