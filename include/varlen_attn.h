/*
 * varlen_attn.h -- C interface of the MI355X (gfx950) fused variable-length
 * attention forward pass.
 *
 * The operation.  For sequences packed back to back along the token axis and
 * delimited by prefix offsets cu_seqlens, for every segment b and head h:
 *
 *     O   = softmax(scale * Q K^T + mask) V          (bf16 out, fp32 math)
 *     LSE = ln sum_j exp(scale * q . k_j)            (fp32, per query row)
 *
 * This is the forward computed by FA4's flash_attn_varlen_func as the vLLM
 * MLA-prefill docs page ("vllm.v1.attention.backends.mla.prefill.flash_attn",
 * FA4MLAPrefillKernel.dispatch and FlashAttnPrefillBackend) calls it: packed
 * q/k/v of shape [total, heads, dim], cu_seqlens_q/k of shape [batch + 1],
 * max_seqlen_q/k, softmax_scale (default qk_head_dim^-0.5), causal,
 * window_size, an optional caller-provided out and an optional LSE.  The
 * same call serves ViT encoder attention (non-causal, no LSE, 16 heads,
 * head dims 64/72/80/128; SGLang PR #41344, "Speed Tests and Profiling")
 * and MLA prefill (causal, qk head dim 192 = 128 nope + 64 rope, v head dim
 * 128; vLLM docs page, FlashAttnPrefillBackend.supports_mla_dimensions).
 *
 * Masking (readings where the pages are silent):
 *   - query row i of a segment with Lq queries and Lk keys sits at key
 *     position p = i + Lk - Lq (bottom-right alignment, so chunked prefill
 *     with q < k lets the new queries see the whole context);
 *   - causal: key j is visible only if j <= p;
 *   - window (left, right): visible only if p - left <= j <= p + right,
 *     -1 meaning unbounded on that side; causal caps the right side at p;
 *   - a row that sees no key gets O = 0 and LSE = -inf.
 *
 * Execution.  Every call enqueues at most one kernel on `stream` and returns
 * without synchronising, allocating device memory, or reading cu_seqlens on
 * the host, so it may be recorded into a HIP graph.  The library keeps no
 * state and no pointer between calls; it is reentrant.
 *
 * Errors.  Arguments are validated on the host before any HIP call; a
 * failing check returns a negative VA_ERR_* code and nothing is launched.
 * VA_ERR_LAUNCH reports a failed kernel launch.  Nothing is printed and
 * nothing aborts.  varlen_attn_status_string() names every code.
 */
#ifndef VARLEN_ATTN_H
#define VARLEN_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VA_OK 0
#define VA_ERR_NULL (-1)    /* a required pointer is NULL */
#define VA_ERR_SHAPE (-2)   /* rows/heads disagree between tensors, or sizes out of range */
#define VA_ERR_HEADDIM (-3) /* (head_dim_qk, head_dim_v) is not a supported pair */
#define VA_ERR_STRIDE (-4)  /* a stride is not positive, or a row stride exceeds 2^24 elements */
#define VA_ERR_ALIGN (-5)   /* a pointer or stride breaks the 16-byte alignment rule */
#define VA_ERR_ARG (-6)     /* a scalar argument is out of range */
#define VA_ERR_LAUNCH (-7)  /* the HIP kernel launch failed */
#define VA_ERR_SCRATCH (-8) /* more scratch than varlen_attn_fwd_splitkv_noalloc holds */

/*
 * A packed bf16 tensor [rows, heads, dim] in device memory.  Element (t, h, c)
 * lives at data + t * row_stride + h * head_stride + c (strides in elements;
 * the last dimension is contiguous).  `data`, row_stride and head_stride must
 * be multiples of 16 bytes (8 elements).  Strided views are accepted, e.g. V
 * interleaved with the nope part of K as in MLA (vLLM docs page,
 * FA4MLAPrefillKernel.dispatch, v_stride = (H * (nope + v), nope + v, 1)).
 * The caller owns the memory.
 */
typedef struct va_tensor {
  void* data;
  int64_t rows;
  int32_t heads;
  int32_t dim;
  int64_t row_stride;
  int64_t head_stride;
} va_tensor;

/*
 * varlen_attn_fwd -- fused varlen attention forward.
 *
 *   q, k, v        bf16 [total_q, H, d_qk], [total_k, H_kv, d_qk], [total_k, H_kv, d_v]
 *   cu_seqlens_q   device int32 [batch + 1]: segment b owns q rows
 *                  [cu_seqlens_q[b], cu_seqlens_q[b + 1]); same for _k
 *   batch          number of segments (>= 0)
 *   max_seqlen_q   host upper bound on every segment's query count (>= 0);
 *                  sizes the grid only
 *   max_seqlen_k   host upper bound on every segment's key count (>= 0)
 *   softmax_scale  finite, > 0 (the Python layer defaults it to d_qk^-0.5)
 *   causal         0 or 1
 *   window_left,
 *   window_right   >= 0, or -1 for unbounded
 *   out            bf16 [total_q, H, d_v], written only on rows that belong
 *                  to a segment; other rows are left untouched
 *   lse            NULL (not computed) or device fp32 [H, total_q] contiguous:
 *                  lse[h * total_q + t]; rows outside every segment untouched
 *   stream         hipStream_t (NULL = the default stream)
 *
 * Supported (d_qk, d_v): (64,64), (72,72), (80,80), (128,128), (192,128).
 * Heads: out->heads == q->heads = H; k->heads == v->heads = H_kv, and H is a
 * multiple of H_kv (grouped KV heads; SGLang PR #41344, "Accuracy Tests",
 * lists GQA among the cases FA4 covers): query head h reads KV head
 * h / (H / H_kv), so consecutive query heads share a KV head (a reading: the
 * pages do not spell the grouping out; this is the usual one).  H_kv == H is
 * plain multi-head attention.
 *
 * Preconditions that are documented but not checked (checking would need a
 * device-to-host copy): cu_seqlens are non-decreasing and start at 0; every
 * segment's rows lie inside the tensors; every segment has at most
 * max_seqlen_q queries (rows past that bound are not computed); inputs are
 * finite; out and lse do not overlap the inputs.
 *
 * Returns VA_OK or a VA_ERR_* code.  batch == 0, max_seqlen_q == 0 or
 * total_q == 0 return VA_OK without launching.
 */
int varlen_attn_fwd(const va_tensor* q, const va_tensor* k, const va_tensor* v,
                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t batch,
                    int32_t max_seqlen_q, int32_t max_seqlen_k, float softmax_scale,
                    int32_t causal, int32_t window_left, int32_t window_right,
                    const va_tensor* out, float* lse, void* stream);

/*
 * varlen_attn_fwd_quant_out -- varlen_attn_fwd with the output quantised to
 * fp8 e4m3 under one static per-tensor scale: out = RNE(clamp(O / *out_scale,
 * -448, 448)) (the vLLM MLA-prefill docs page: supports_quant_output with
 * kFp8StaticTensorSym, the output_scale argument of
 * _flash_attn_varlen_diff_headdims; bf16 inputs as there).
 *
 *   out        e4m3 [total_q, H, d_v] (va_tensor with strides in bytes; data,
 *              row and head strides multiples of 8 bytes: the codes are
 *              written 8 bytes at a time)
 *   out_scale  device fp32 scalar > 0 (not checked), 4-byte aligned
 *   the rest   as for varlen_attn_fwd; the LSE is the same as there
 *
 * Returns what varlen_attn_fwd returns, and VA_ERR_NULL for a NULL
 * out_scale, VA_ERR_ALIGN for a misaligned one.
 */
int varlen_attn_fwd_quant_out(const va_tensor* q, const va_tensor* k, const va_tensor* v,
                              const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t batch,
                              int32_t max_seqlen_q, int32_t max_seqlen_k, float softmax_scale, int32_t causal,
                              int32_t window_left, int32_t window_right, const va_tensor* out,
                              const float* out_scale, float* lse, void* stream);

/*
 * varlen_attn_fwd_splitkv -- varlen_attn_fwd with each work unit's key tiles
 * split into num_splits runs computed by separate workgroups, then combined.
 * Split-KV prefill as the vLLM MLA-prefill docs page describes it (FA4's
 * `num_splits` argument in FA4MLAPrefillKernel.dispatch, and
 * FA4SplitKVCombineKernel: per-split fp32 partial outputs [num_splits,
 * total_q, H, d_v] and LSEs [num_splits, H, total_q] reduced by a combine
 * kernel).  It fills the GPU when a call has few query tiles per head but
 * long key ranges (a chunked prefill's context chunk, long K with short Q).
 *
 *   q .. lse, stream   as for varlen_attn_fwd (same checks, same results
 *                      up to rounding: each split's partial is exact
 *                      attention over its keys, and the combine is exact)
 *   num_splits         1 .. 128; 1 is exactly varlen_attn_fwd (workspace
 *                      unused, may be NULL)
 *   num_splits_dynamic NULL, or device int32 [batch], 4-byte aligned:
 *                      per-segment split counts, as FA4's scheduler
 *                      supplies its combine a num_splits_dynamic_ptr (vLLM
 *                      docs page, FA4SplitKVCombineKernel).  Segment b's
 *                      keys are then split into min(max(count_b, 1),
 *                      num_splits) runs and the combine reads that many
 *                      partials for its rows; num_splits only bounds them
 *                      (and sizes the grid and workspace).  The counts are
 *                      read on the device; varlen_attn_splitkv_counts fills
 *                      them from cu_seqlens_k.  With counts, short segments
 *                      are not packed several to a workgroup.
 *   workspace          device memory of at least
 *                      varlen_attn_splitkv_workspace_bytes(total_q, H, d_v,
 *                      num_splits) bytes, 256-byte aligned, owned by the
 *                      caller; its contents on entry do not matter.  Calls
 *                      that share a workspace must not overlap.
 *
 * Enqueues two kernels on `stream` (the split attention, then the combine)
 * and returns; no allocation, no synchronisation, graph-capturable.
 * Returns VA_OK, any varlen_attn_fwd error, VA_ERR_ARG for num_splits out of
 * range or a workspace below the size, VA_ERR_NULL for a NULL workspace,
 * VA_ERR_ALIGN for a misaligned workspace or num_splits_dynamic.
 */
int varlen_attn_fwd_splitkv(const va_tensor* q, const va_tensor* k, const va_tensor* v,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t batch,
                            int32_t max_seqlen_q, int32_t max_seqlen_k, float softmax_scale,
                            int32_t causal, int32_t window_left, int32_t window_right,
                            const va_tensor* out, float* lse, int32_t num_splits,
                            const int32_t* num_splits_dynamic, void* workspace, size_t workspace_bytes,
                            void* stream);

/* Bytes of the per-GPU scratch array of varlen_attn_fwd_splitkv_noalloc. */
#define VA_SCRATCH_BYTES (64u << 20)

/*
 * varlen_attn_fwd_splitkv_noalloc -- varlen_attn_fwd_splitkv for callers
 * that cannot allocate device memory or pass a workspace (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).
 * The split partials live in a fixed array of VA_SCRATCH_BYTES (64 MiB) in
 * device memory that the library holds on each GPU it runs on until the
 * process ends; the call itself allocates nothing.
 *
 *   arguments   as for varlen_attn_fwd_splitkv, without the workspace; the
 *               caller passes inputs and outputs as there
 *   num_splits  1 .. 128; 1 is exactly varlen_attn_fwd (no scratch used)
 *
 * The partials need varlen_attn_splitkv_workspace_bytes(total_q, H, d_v,
 * num_splits) bytes; a call needing more than VA_SCRATCH_BYTES returns
 * VA_ERR_SCRATCH and launches nothing.  All calls on one GPU share that
 * GPU's array: calls that overlap on one GPU (several streams or host
 * threads at once) race and give undefined results; calls in order on one
 * stream do not.  The array keeps the last call's contents; nothing needs
 * clearing (every partial the combine reads is written by the same call).
 * The first call on a device looks the array up there (a host call that
 * makes no allocation and no synchronisation).  Returns what
 * varlen_attn_fwd_splitkv returns, VA_ERR_SCRATCH, or VA_ERR_LAUNCH when no
 * device is current or the lookup fails.
 */
int varlen_attn_fwd_splitkv_noalloc(const va_tensor* q, const va_tensor* k, const va_tensor* v,
                                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t batch,
                                    int32_t max_seqlen_q, int32_t max_seqlen_k, float softmax_scale,
                                    int32_t causal, int32_t window_left, int32_t window_right,
                                    const va_tensor* out, float* lse, int32_t num_splits, void* stream);

/* VA_SCRATCH_BYTES, as the library was built with it.  Host only. */
size_t varlen_attn_scratch_bytes(void);

/*
 * varlen_attn_fwd_fp8 -- the forward on fp8 e4m3 inputs with descales, and
 * optionally an e4m3 output.  SGLang PR #41344 ("Accuracy Tests") lists fp8
 * e4m3 with descales among the FA4 configurations; the vLLM MLA-prefill docs
 * page has the fp8 static per-tensor symmetric output quantisation
 * (supports_quant_output with kFp8StaticTensorSym, the output_scale
 * argument).  What is computed (readings; the pages give no formula):
 *
 *     Q~ = Q * q_descale[b, hk], K~ = K * k_descale[b, hk],
 *     V~ = V * v_descale[b, hk]          (hk = the KV head of query head h)
 *     O, LSE = the forward above on Q~, K~, V~ (same masks and scale)
 *     out = O in bf16, or, with out_scale, e4m3(clamp(O / *out_scale,
 *           -448, 448)) rounded to nearest even
 *
 *   q, k, v        e4m3 bytes (OCP E4M3: bias 7, no infinities, 0x7F/0xFF
 *                  NaN, largest 448), [total, heads, dim] as va_tensor with
 *                  strides in bytes; rows and heads 16-byte aligned
 *   q_descale, k_descale, v_descale
 *                  device fp32 [batch, H_kv] contiguous (entry b * H_kv +
 *                  hk), or NULL for all ones; a per-tensor scale is the case
 *                  of equal entries; q and k descales > 0 (see below)
 *   out            bf16 [total_q, H, d_v], or e4m3 when out_scale is given
 *                  (then data and strides multiples of 8 bytes)
 *   out_scale      NULL, or a device fp32 scalar > 0 (not checked)
 *   num_splits, num_splits_dynamic, workspace, workspace_bytes
 *                  as for varlen_attn_fwd_splitkv (1 = no split; with
 *                  splits the combine kernel writes the e4m3 output)
 *   other arguments as for varlen_attn_fwd
 *
 * Supported (d_qk, d_v): (64,64), (128,128), (192,128).  The kernel rounds
 * the softmax probabilities to e4m3 for the PV product (each p <= 256, so
 * none saturates) and normalises by the fp32 sum of the unrounded ones: O
 * carries a relative rounding of up to 2^-4 per term.  The fp8 MFMA sums
 * its products at less than fp32 precision: each score may be off by up to
 * 2^-15 * scale * q_descale * k_descale * sum_i |q_i k_i|, and the LSE by
 * the largest such error of its row beyond the fp32 arithmetic.
 *
 * Precondition (documented, not checked: the descales live in device
 * memory): every q_descale and k_descale entry is finite and > 0.  The
 * kernel folds their product into the softmax scale before it takes the
 * row max of the raw scores, which is the max of the scaled scores only for
 * a positive factor.  v_descale entries are finite (any sign).  Returns VA_OK or a VA_ERR_* code as
 * varlen_attn_fwd_splitkv, and VA_ERR_ALIGN for a descale or out_scale
 * pointer not 4-byte aligned.
 */
int varlen_attn_fwd_fp8(const va_tensor* q, const va_tensor* k, const va_tensor* v,
                        const float* q_descale, const float* k_descale, const float* v_descale,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t batch,
                        int32_t max_seqlen_q, int32_t max_seqlen_k, float softmax_scale, int32_t causal,
                        int32_t window_left, int32_t window_right, const va_tensor* out,
                        const float* out_scale, float* lse, int32_t num_splits,
                        const int32_t* num_splits_dynamic, void* workspace, size_t workspace_bytes,
                        void* stream);

/* Workspace bytes varlen_attn_fwd_splitkv needs (0 for num_splits <= 1). Host only. */
size_t varlen_attn_splitkv_workspace_bytes(int64_t total_q, int32_t num_heads, int32_t head_dim_v,
                                           int32_t num_splits);

/*
 * A split count for these sizes: the device's concurrent workgroups over
 * the call's work units, at most 128 and at most one split per 16 key tiles
 * (FA4's automatic choice on the vLLM page caps splits the same way, at
 * num_SMs // total_m_blocks and 128); 1 when the units already fill the
 * device.  The units and tile width are those of the launch the call makes:
 * with num_heads_k KV heads (grouped heads and short segments change how
 * many workgroups a launch has) and, for fp8 = 1, varlen_attn_fwd_fp8's
 * kernel (64-key tiles, one workgroup per compute unit).  Queries the
 * current device's compute-unit count (a host call, no synchronisation).
 * Returns VA_OK, VA_ERR_NULL, VA_ERR_HEADDIM or VA_ERR_ARG.
 */
int varlen_attn_num_splits(int32_t head_dim_qk, int32_t head_dim_v, int32_t batch, int32_t num_heads,
                           int32_t num_heads_k, int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t fp8,
                           int32_t* num_splits);

/*
 * varlen_attn_splitkv_counts -- per-segment split counts on the device, for
 * varlen_attn_fwd_splitkv's num_splits_dynamic: count_b = min(max(ceil(Lk_b
 * / keys_per_split), 1), max_splits) with Lk_b = cu_seqlens_k[b + 1] -
 * cu_seqlens_k[b], so each split gets at least keys_per_split keys where
 * the segment has them (FA4's automatic choice keeps splits similarly
 * long).  Enqueues one small kernel on `stream` (no host read of
 * cu_seqlens, no allocation); `num_splits_dynamic` is device int32 [batch],
 * owned by the caller.  Returns VA_OK (batch == 0: nothing launched),
 * VA_ERR_ARG for batch < 0, max_splits outside 1 .. 128 or keys_per_split
 * < 1, VA_ERR_NULL, VA_ERR_ALIGN (pointers 4-byte aligned) or VA_ERR_LAUNCH.
 */
int varlen_attn_splitkv_counts(const int32_t* cu_seqlens_k, int32_t batch, int32_t max_splits,
                               int32_t keys_per_split, int32_t* num_splits_dynamic, void* stream);

/*
 * varlen_attn_merge -- merge two attention results over disjoint key sets of
 * the same queries.  A prefill that reads its context in chunks merges the
 * token-major partials of its per-chunk (non-causal) and new-token (causal)
 * calls this way, and a split-KV forward ends with the same combine (vLLM
 * docs page "vllm.v1.attention.backends.mla.prefill.flash_attn":
 * FlashAttnPrefillBackend, `run_prefill_context_chunk` and the
 * merge_attn_states remark in `_flash_attn_varlen_diff_headdims`;
 * FA4SplitKVCombineKernel).
 *
 *   out_a, out_b   bf16 [rows, H, d] normalised partial outputs, as
 *                  varlen_attn_fwd writes them
 *   lse_a, lse_b   fp32 [H, rows] contiguous, their natural-log LSEs
 *                  (-inf: the part saw no key for that row)
 *   out            bf16 [rows, H, d]; may be the same buffer as out_a or out_b
 *   lse            fp32 [H, rows] contiguous, or NULL; may be the same array
 *                  as lse_a or lse_b
 *   stream         hipStream_t
 *
 * For every row i and head h:  lse = ln(e^lse_a + e^lse_b) and
 * out = e^(lse_a - lse) out_a + e^(lse_b - lse) out_b, in fp32, out rounded
 * to bf16 (round to nearest even).  A part whose lse is -inf contributes
 * nothing; both -inf give out = 0 and lse = -inf.  Every row of the
 * descriptors is merged.  d: a multiple of 8 from 8 to 256, the same for the
 * three tensors, as are rows and heads; strides in elements, positive,
 * multiples of 8; data pointers 16-byte aligned, lse pointers 4-byte aligned.
 * The caller owns every buffer.  Enqueues one kernel on `stream` and
 * returns: no allocation, no synchronisation.  Returns VA_OK (rows == 0:
 * nothing launched), VA_ERR_NULL, VA_ERR_SHAPE, VA_ERR_STRIDE, VA_ERR_ALIGN
 * or VA_ERR_LAUNCH.
 */
int varlen_attn_merge(const va_tensor* out_a, const float* lse_a, const va_tensor* out_b,
                      const float* lse_b, const va_tensor* out, float* lse, void* stream);

/* Static, never-NULL description of a status code. */
const char* varlen_attn_status_string(int status);

/*
 * The kernel's tile schedule for one block of query rows, computed on the
 * host by the same function the kernel runs (exported for tests).
 *
 * Rows [row_begin, row_end) of a segment with seqlen_q queries and seqlen_k
 * keys (0 <= row_begin < row_end <= seqlen_q).  Key tiles are block_n keys
 * wide.  On return the block visits key tiles [*kt_begin, *kt_end); tiles in
 * [*full_begin, *full_end) need no mask (every valid row sees every key of
 * the tile); the other visited tiles are masked.  An empty visit range means
 * no row of the block sees any key.  Returns VA_OK or VA_ERR_ARG / VA_ERR_NULL.
 * Host only; makes no HIP call.
 */
int varlen_attn_tile_range(int32_t seqlen_q, int32_t seqlen_k, int32_t row_begin, int32_t row_end,
                           int32_t causal, int32_t window_left, int32_t window_right,
                           int32_t block_n, int32_t* kt_begin, int32_t* kt_end,
                           int32_t* full_begin, int32_t* full_end);

/*
 * The kernel's workgroup-to-work mapping, computed on the host (exported for
 * tests).  `seqlens_q` / `seqlens_k` are host arrays of `batch` per-segment
 * lengths (the differences of cu_seqlens_q / cu_seqlens_k); max_seqlen_q is
 * taken as their maximum.  For workgroup `block` of the grid varlen_attn_fwd
 * launches for these sizes, returns the segment, head and q-tile (block_m
 * query rows, see varlen_attn_plan) it owns, or -1 in all three for a
 * workgroup that exits at once.  For attn_fwd_short `block` is a one-wave
 * work unit (va_plan.units of them, four to a workgroup).  Segments of different lengths (at most 64
 * of them) are dealt longest key length first; otherwise in packing order;
 * either way every odd quad of each XCD's dispatch order is reversed.
 * When va_plan.pair_q_tiles is 1, the workgroup runs q-tile `q_tile` and
 * then q-tile n_b - 1 - q_tile of the same (segment, head) if that is
 * another one (n_b = ceil(seqlen_q / block_m)); q_tile is the later, longer
 * one.  Segments of at most 64 queries with head dims <= 80 (and no grouped query
 * heads to pack instead) run one wave per (segment, head) on the
 * short-segment kernel (va_plan.kernel "attn_fwd_short", block_m 64): q-tile
 * 0 of each, a segment's heads dealt to one XCD in groups of up to 16.  On
 * small launches of longer segments (va_plan.key_split 4) the same kernel
 * takes unit `block` per workgroup: q-tile `q_tile` of 64 rows, its key
 * tiles split over the workgroup's four waves.  When
 * short segments share workgroups (va_plan.segments_per_block P > 1, every
 * segment at most 128 queries), workgroup `block` owns segments
 * [segment, segment + P) (those that exist), their q-tile 0 (pack_mode 1),
 * or, when the KV-head group size num_heads / num_heads_k is a multiple of
 * P, query heads [head, head + P) of one segment, q-tile 0 (pack_mode 2).
 * With num_heads_k KV heads (num_heads a multiple of it) the query heads of
 * one KV head are dealt to the same XCD where the head counts allow.
 * Returns VA_OK, VA_ERR_NULL, VA_ERR_HEADDIM, or VA_ERR_ARG for a block
 * outside the grid, a negative length or all-empty queries.
 * Host only; makes no HIP call.
 */
int varlen_attn_work_unit(int64_t block, int32_t batch, int32_t num_heads, int32_t num_heads_k,
                          int32_t head_dim_qk, int32_t head_dim_v, const int32_t* seqlens_q,
                          const int32_t* seqlens_k, int32_t causal, int32_t* segment, int32_t* head,
                          int32_t* q_tile);

/* Launch shape varlen_attn_fwd would use (host only; makes no HIP call). */
typedef struct va_plan {
  int32_t block_m;       /* query rows per work unit (per workgroup, but for attn_fwd_short) */
  int32_t block_n;       /* keys per K/V tile */
  int32_t threads;       /* threads per workgroup */
  int32_t lds_bytes;     /* LDS per workgroup */
  int64_t grid;          /* workgroups launched (some exit at once on short segments) */
  const char* kernel;    /* kernel name: "attn_fwd_wide", or "attn_fwd_short" for segments of at most
                            64 queries with head dims <= 80, whose workgroups hold four independent
                            one-wave units (block_m 64 rows each): workgroup w's wave v takes unit
                            ((w >> 3) * 4 + v) * 8 + (w & 7) */
  int32_t segments_per_block; /* 1, or 2 / 4 slots per workgroup for short segments (max_seqlen_q
                                 <= 128 / <= 64), one or two waves each; see pack_mode */
  int32_t pack_mode;          /* 0: unpacked; 1: the slots take consecutive segments of one head;
                                 2: they take query heads of one KV head over one segment (grouped
                                 KV heads with a group size that is a multiple of the slot count:
                                 FA4's pack_gqa, SGLang PR #41344 "Accuracy Tests") */
  int64_t units;              /* work units (varlen_attn_work_unit's blocks), padding included:
                                 grid, or 4 per workgroup for attn_fwd_short */
  int32_t pair_q_tiles;       /* 1 when each work unit runs two q-tiles of one segment, n_b - 1 - t
                                 and then t (n_b = ceil(seqlen_q / block_m)), so that every unit
                                 of a causal launch sees the same number of key tiles: causal,
                                 max_seqlen_q > block_m, unpacked, attn_fwd_wide at
                                 head_dim_qk > 80, unsplit, where the unpaired units fill at least
                                 two rounds of each XCD's 32 CUs (the padded grid / 8) and the
                                 pairs at least 15/16 of their last round */
  int32_t key_split;          /* waves of a workgroup that share one work unit and split its key
                                 tiles: 4 for attn_fwd_short on launches of segments longer than
                                 64 queries (head dims <= 80, unsplit) whose 64-row blocks fit one
                                 round on every XCD: 8 x ceil(batch x num_heads / 8) x
                                 ceil(max_seqlen_q / 64) <= 512 (an XCD's eighth: two workgroups
                                 on each of its 32 CUs); one block a workgroup, the waves' partial
                                 results merged in LDS; else 1 */
} va_plan;

int varlen_attn_plan(int32_t head_dim_qk, int32_t head_dim_v, int32_t batch, int32_t num_heads,
                     int32_t num_heads_k, int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t causal,
                     va_plan* plan);

/* varlen_attn_plan for varlen_attn_fwd_fp8's kernel (supported pairs (64,64),
 * (128,128), (192,128); 64-key tiles).  Host only; same returns. */
int varlen_attn_plan_fp8(int32_t head_dim_qk, int32_t head_dim_v, int32_t batch, int32_t num_heads,
                         int32_t num_heads_k, int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t causal,
                         va_plan* plan);

#ifdef __cplusplus
}
#endif

#endif /* VARLEN_ATTN_H */
