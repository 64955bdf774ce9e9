// Merge of two attention results over disjoint key sets of the same queries.
//
// A prefill that reads its context in chunks computes attention of the new
// queries over each context chunk (non-causal) and over the new tokens
// (causal), each call returning its normalised output and log-sum-exp, and
// then merges those token-major partials (vLLM docs page
// "vllm.v1.attention.backends.mla.prefill.flash_attn", FlashAttnPrefillBackend:
// `run_prefill_context_chunk`, `run_prefill_new_tokens`, and the remark in
// `_flash_attn_varlen_diff_headdims` that merge_attn_states needs token-major
// partials).  A split-KV forward ends with the same combine over its splits
// (same page, FA4SplitKVCombineKernel).
//
// For row i of head h, with parts (O_a, L_a) and (O_b, L_b) over key sets A
// and B, the result over A u B is, exactly,
//     L = ln(e^L_a + e^L_b),   O = e^(L_a - L) O_a + e^(L_b - L) O_b,
// because O_x = sum_{j in x} e^{s_j} v_j / e^{L_x}.  A part whose LSE is -inf
// saw no key and contributes nothing; both -inf gives O = 0, L = -inf, as the
// forward writes for a row with no visible key.
//
// The kernel is an elementwise pass bound by HBM: per (row, head) it reads
// two d_v-vectors of bf16 and two fp32 LSEs and writes one of each.  A group
// of G lanes (G the power of two >= d_v / 8, so a group never straddles a
// wave) owns one (row, head); lane c of the group moves the 16 bytes of
// columns 8c .. 8c + 7, so consecutive lanes touch consecutive bytes of a
// row.  The outputs are streamed with non-temporal loads and stores (each
// byte is touched once; measured 6.25 TB/s against 5.78 through the caches).
// Because a group's lanes read the LSEs in the same instruction before
// lane 0 writes the result, the output LSE may be the same array as an
// input's; the output O may be the same buffer as an input O.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "attn_common.h"  // quant_e4m3x4
#include "varlen_attn.h"

namespace va_merge {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct Params {
  const uint16_t* oa;
  const uint16_t* ob;
  uint16_t* o;
  const float* la;
  const float* lb;
  float* l;
  int64_t a_row, a_head, b_row, b_head, o_row, o_head;  // elements
  int64_t rows;
  int32_t heads;
  int32_t chunks;      // d_v / 8
  int32_t lane_shift;  // log2 of the lanes per (row, head)
};

__device__ __forceinline__ float lo_bf16(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }

// Two fp32 values rounded to bf16 (round to nearest even) in one word, a low.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

__global__ __launch_bounds__(256) void merge_states(Params p) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t pair = t >> p.lane_shift;
  const int c = (int)(t & ((1 << p.lane_shift) - 1));
  if (pair >= p.rows * p.heads) return;
  const int64_t i = pair / p.heads;
  const int h = (int)(pair - i * p.heads);
  const float la = p.la[(int64_t)h * p.rows + i];
  const float lb = p.lb[(int64_t)h * p.rows + i];
  const float m = fmaxf(la, lb);
  float wa = 0.f, wb = 0.f, lse = -INFINITY;
  if (m != -INFINITY) {
    const float ea = expf(la - m), eb = expf(lb - m);  // the larger one is exactly 1
    const float s = ea + eb;
    wa = ea / s;
    wb = eb / s;
    lse = m + logf(s);
  }
  if (c < p.chunks) {
    const u32x4 a = __builtin_nontemporal_load((const u32x4*)(p.oa + i * p.a_row + h * p.a_head + 8 * c));
    const u32x4 b = __builtin_nontemporal_load((const u32x4*)(p.ob + i * p.b_row + h * p.b_head + 8 * c));
    u32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // A part with weight 0 (no key, or negligible) is skipped, not scaled:
      // its O is never read into the sum.
      float x0 = 0.f, x1 = 0.f;
      if (wa > 0.f) {
        x0 += wa * lo_bf16(a[e]);
        x1 += wa * hi_bf16(a[e]);
      }
      if (wb > 0.f) {
        x0 += wb * lo_bf16(b[e]);
        x1 += wb * hi_bf16(b[e]);
      }
      r[e] = pack_bf16x2(x0, x1);
    }
    __builtin_nontemporal_store(r, (u32x4*)(p.o + i * p.o_row + h * p.o_head + 8 * c));
  }
  if (c == 0 && p.l != nullptr) p.l[(int64_t)h * p.rows + i] = lse;
}

// Combine of split-KV partials (varlen_attn_fwd_splitkv).  The attention
// kernel leaves, per split s, the normalised fp32 output O_s [S, rows, H, d]
// and its natural-log LSE L_s [S, H, rows] over the split's keys (-inf where
// a row saw none of them); the combine over the S disjoint key sets is the
// merge above taken S ways: L = m + ln sum_s e^(L_s - m) with m = max_s L_s,
// O = sum_s e^(L_s - L) O_s, out = bf16(O), or with an output scale the
// e4m3 codes of clamp(O / scale, +-448) (the fp8 call's static per-tensor
// output quantisation).  Only rows of some segment,
// [cu_seqlens_q[0], cu_seqlens_q[batch]), are written: the others were not
// computed and are left untouched, as the unsplit forward leaves them.  A
// group of G lanes (G the power of two >= d / 4) owns one (row, head); lane
// c reads the 16 bytes of columns 4c .. 4c + 3 of every split.
struct CombineParams {
  const float* part_o;
  const float* part_lse;
  uint16_t* o;
  float* l;
  const int32_t* cu_q;
  int64_t o_row, o_head;  // elements
  int64_t rows;
  int32_t heads, dim, splits, batch;
  int32_t lane_shift;
  const float* out_scale;  // null: bf16 out; else e4m3 out (o holds bytes)
  // Per-segment split counts [batch] (null: `splits` for every row): the
  // rows of segment b combine the first min(max(count, 1), splits) partials.
  const int32_t* splits_dyn;
};

__global__ __launch_bounds__(256) void combine_splits(CombineParams p) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t pair = t >> p.lane_shift;
  const int c = (int)(t & ((1 << p.lane_shift) - 1));
  if (pair >= p.rows * p.heads) return;
  const int64_t i = pair / p.heads;
  const int h = (int)(pair - i * p.heads);
  if (i < p.cu_q[0] || i >= p.cu_q[p.batch]) return;
  int splits = p.splits;
  if (p.splits_dyn != nullptr) {
    // the row's segment: the last b with cu_q[b] <= i (binary search)
    int lo = 0, hi = p.batch - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.cu_q[mid] <= i) lo = mid; else hi = mid - 1;
    }
    splits = min(max(p.splits_dyn[lo], 1), p.splits);
  }
  const int64_t plane = p.rows * p.heads;  // (row, head) pairs per split
  // Lane c of the group reads the LSE of split s0 + c, and the group's
  // lanes pass them round (__shfl within the group), so each LSE is loaded
  // once rather than by every lane in every pass.  The arithmetic is the
  // same in every lane and in split order: the max, then the sum of
  // exp(lse - max), then the weighted O; a split past the row's count
  // contributes an LSE of -inf, whose exp(-inf - max) = 0 leaves the sum as
  // it was.  The loops run to the launch's split count, the same for every
  // lane of the wave.  The partial O loads of eight splits are issued
  // before any is used.
  const int G = 1 << p.lane_shift;
  const float* lse_row = p.part_lse + (int64_t)h * p.rows + i;
  auto lse_chunk = [&](int s0) {  // this lane's LSE of split s0 + c
    return s0 + c < splits ? lse_row[(int64_t)(s0 + c) * plane] : -INFINITY;
  };
  float m = -INFINITY;
  for (int s0 = 0; s0 < p.splits; s0 += G) {
    const float mine = lse_chunk(s0);
    const int n = min(G, p.splits - s0);
    for (int k = 0; k < n; ++k) m = fmaxf(m, __shfl(mine, k, G));
  }
  float sum = 0.f;
  for (int s0 = 0; s0 < p.splits; s0 += G) {
    const float mine = lse_chunk(s0);
    const int n = min(G, p.splits - s0);
    for (int k = 0; k < n; ++k) {
      const float l = __shfl(mine, k, G);
      if (m != -INFINITY && s0 + k < splits) sum += expf(l - m);
    }
  }
  // (Every lane runs the loops, so each __shfl reads lanes that take part;
  // lanes past the head dim only skip the loads.)
  const bool cols = 4 * c < p.dim;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const float inv = m != -INFINITY ? 1.f / sum : 0.f;
  constexpr int kC = 8;
  for (int s0 = 0; s0 < p.splits; s0 += G) {
    const float mine = lse_chunk(s0);
    const int n = min(G, p.splits - s0);
    for (int k0 = 0; k0 < n; k0 += kC) {
      float w[kC];
      f32x4 x[kC];
#pragma unroll
      for (int k = 0; k < kC; ++k) {
        const float l = __shfl(mine, min(k0 + k, G - 1), G);
        w[k] = (m != -INFINITY && k0 + k < n && s0 + k0 + k < splits) ? expf(l - m) * inv : 0.f;
      }
      // A split with weight 0 (no key, or negligible) is skipped, not
      // scaled: its O is never read into the sum.
#pragma unroll
      for (int k = 0; k < kC; ++k) {
        x[k] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (cols && w[k] > 0.f)
          x[k] = __builtin_nontemporal_load(
              (const f32x4*)(p.part_o + ((int64_t)(s0 + k0 + k) * plane + i * p.heads + h) * p.dim + 4 * c));
      }
#pragma unroll
      for (int k = 0; k < kC; ++k)
        if (w[k] > 0.f) acc += w[k] * x[k];
    }
  }
  if (cols) {
    if (p.out_scale != nullptr) {
      const uint32_t code = va::quant_e4m3x4(acc[0], acc[1], acc[2], acc[3], 1.f / *p.out_scale);
      *(uint32_t*)((uint8_t*)p.o + i * p.o_row + h * p.o_head + 4 * c) = code;
    } else {
      const u32x2 r = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
      *(u32x2*)(p.o + i * p.o_row + h * p.o_head + 4 * c) = r;
    }
  }
  if (c == 0 && p.l != nullptr) p.l[(int64_t)h * p.rows + i] = m != -INFINITY ? m + logf(sum) : -INFINITY;
}

int launch_combine(const float* part_o, const float* part_lse, int32_t num_splits, int64_t total_q, int32_t heads,
                   int32_t dim, const int32_t* cu_seqlens_q, int32_t batch, const va_tensor* out, float* lse,
                   void* stream, const float* out_scale, const int32_t* splits_dyn) {
  CombineParams p;
  p.out_scale = out_scale;
  p.splits_dyn = splits_dyn;
  p.part_o = part_o;
  p.part_lse = part_lse;
  p.o = (uint16_t*)out->data;
  p.l = lse;
  p.cu_q = cu_seqlens_q;
  p.o_row = out->row_stride;
  p.o_head = out->head_stride;
  p.rows = total_q;
  p.heads = heads;
  p.dim = dim;
  p.splits = num_splits;
  p.batch = batch;
  int shift = 0;
  while ((1 << shift) < (dim + 3) / 4) ++shift;
  p.lane_shift = shift;
  const int64_t grid = ((total_q * heads << shift) + 255) / 256;
  if (grid > INT32_MAX) return VA_ERR_SHAPE;
  void* args[] = {&p};
  const hipError_t err =
      hipLaunchKernel((const void*)&combine_splits, dim3((unsigned)grid), dim3(256), args, 0, (hipStream_t)stream);
  return err == hipSuccess ? VA_OK : VA_ERR_LAUNCH;
}

// Per-segment split counts for split-KV, on the device from cu_seqlens_k:
// count_b = min(max(ceil(Lk_b / keys_per_split), 1), max_splits), so a
// segment gets one split per keys_per_split keys (short segments one).
__global__ __launch_bounds__(256) void splitkv_counts(const int32_t* cu_k, int32_t batch, int32_t max_splits,
                                                      int32_t keys_per_split, int32_t* counts) {
  const int b = (int)(blockIdx.x * 256 + threadIdx.x);
  if (b >= batch) return;
  const int64_t lk = (int64_t)cu_k[b + 1] - cu_k[b];
  const int64_t n = (lk + keys_per_split - 1) / keys_per_split;
  counts[b] = (int32_t)(n < 1 ? 1 : (n > max_splits ? max_splits : n));
}

static int check(const va_tensor* t, int64_t rows, int32_t heads, int32_t dim) {
  if (t->rows != rows || t->heads != heads || t->dim != dim) return VA_ERR_SHAPE;
  if (t->row_stride <= 0 || t->head_stride <= 0) return VA_ERR_STRIDE;
  if ((t->row_stride & 7) != 0 || (t->head_stride & 7) != 0) return VA_ERR_ALIGN;
  if (rows > 0 && t->data == nullptr) return VA_ERR_NULL;
  if (((uintptr_t)t->data & 15u) != 0) return VA_ERR_ALIGN;
  return VA_OK;
}

}  // namespace va_merge

extern "C" int varlen_attn_merge(const va_tensor* out_a, const float* lse_a, const va_tensor* out_b,
                                 const float* lse_b, const va_tensor* out, float* lse, void* stream) {
  using namespace va_merge;
  if (!out_a || !out_b || !out) return VA_ERR_NULL;
  const int64_t rows = out_a->rows;
  const int32_t heads = out_a->heads, dim = out_a->dim;
  if (rows < 0 || rows > INT32_MAX || heads <= 0) return VA_ERR_SHAPE;
  if (dim < 8 || dim > 256 || (dim & 7) != 0) return VA_ERR_SHAPE;
  int st;
  if ((st = check(out_a, rows, heads, dim)) != VA_OK) return st;
  if ((st = check(out_b, rows, heads, dim)) != VA_OK) return st;
  if ((st = check(out, rows, heads, dim)) != VA_OK) return st;
  if (rows == 0) return VA_OK;
  if (!lse_a || !lse_b) return VA_ERR_NULL;
  if (((uintptr_t)lse_a & 3u) || ((uintptr_t)lse_b & 3u) || ((uintptr_t)lse & 3u)) return VA_ERR_ALIGN;

  Params p;
  p.oa = (const uint16_t*)out_a->data;
  p.ob = (const uint16_t*)out_b->data;
  p.o = (uint16_t*)out->data;
  p.la = lse_a;
  p.lb = lse_b;
  p.l = lse;
  p.a_row = out_a->row_stride;
  p.a_head = out_a->head_stride;
  p.b_row = out_b->row_stride;
  p.b_head = out_b->head_stride;
  p.o_row = out->row_stride;
  p.o_head = out->head_stride;
  p.rows = rows;
  p.heads = heads;
  p.chunks = dim / 8;
  int shift = 0;
  while ((1 << shift) < p.chunks) ++shift;
  p.lane_shift = shift;
  const int64_t threads = rows * heads << shift;
  const int64_t grid = (threads + 255) / 256;
  if (grid > INT32_MAX) return VA_ERR_SHAPE;
  void* args[] = {&p};
  const hipError_t err =
      hipLaunchKernel((const void*)&merge_states, dim3((unsigned)grid), dim3(256), args, 0, (hipStream_t)stream);
  return err == hipSuccess ? VA_OK : VA_ERR_LAUNCH;
}

extern "C" int varlen_attn_splitkv_counts(const int32_t* cu_seqlens_k, int32_t batch, int32_t max_splits,
                                          int32_t keys_per_split, int32_t* num_splits_dynamic, void* stream) {
  if (batch < 0 || max_splits < 1 || max_splits > 128 || keys_per_split < 1) return VA_ERR_ARG;
  if (batch == 0) return VA_OK;
  if (!cu_seqlens_k || !num_splits_dynamic) return VA_ERR_NULL;
  if (((uintptr_t)cu_seqlens_k & 3u) != 0 || ((uintptr_t)num_splits_dynamic & 3u) != 0) return VA_ERR_ALIGN;
  void* args[] = {(void*)&cu_seqlens_k, &batch, &max_splits, &keys_per_split, &num_splits_dynamic};
  const hipError_t err = hipLaunchKernel((const void*)&va_merge::splitkv_counts, dim3((unsigned)((batch + 255) / 256)),
                                         dim3(256), args, 0, (hipStream_t)stream);
  return err == hipSuccess ? VA_OK : VA_ERR_LAUNCH;
}
