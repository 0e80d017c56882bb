/*
 * attnq.h -- C ABI of the quantized flash-attention forward path for MI355X
 * (gfx950).  Library: paged_kv_amd/libattnq.so.
 *
 * The path computes  O = softmax(scale * Dequant(Q) Dequant(K)^T + mask) Dequant(V)
 * (the formula of the Ascend "KvQuantSparseFlashAttention" page, with
 * Dequant(x, s) = x * s) over varlen batches, paged KV caches, fp8-e4m3 inputs
 * with per-head descales, SageAttention-style per-block int8 Q/K and
 * MLA-absorb sparse decode.
 *
 * Conventions shared by every entry point
 *  - Every pointer is a DEVICE pointer owned by the caller.  The library
 *    never allocates, frees, copies to the host or synchronizes: each call
 *    only validates its host arguments and enqueues kernels on `stream`
 *    (0 = the null stream), in order, asynchronously.
 *  - Capture-safe (FlashInfer "[Refactor] Unify JIT/Customization/AOT
 *    mode": the decode/prefill plans take enable_cuda_graph; Ascend
 *    "KvQuantSparseFlashAttention", 约束说明: graph mode): the enqueued work is
 *    kernels only (scales and counters are cleared by fill kernels, not
 *    memsets), so a sequence of calls can be recorded into a HIP graph and
 *    replayed; a replay reads the input buffers as they are at that time.
 *  - Return value: ATTNQ_OK (0) or a negative attnq_status.  On a negative
 *    status nothing was enqueued and attnq_last_error() (thread-local) holds
 *    a message.
 *  - Host arguments are checked; device-side contents (cu_seqlens, page
 *    indices, ...) are preconditions.  Kernels clamp every index they read
 *    from device memory to the buffer bounds given on the host, so a broken
 *    precondition gives wrong values, never an out-of-bounds access.
 *  - Pointers must be 16-byte aligned (4-byte for int32/fp32 arrays).
 *  - batch (batch * s_q for the sparse MLA decode) is at most 65535, a
 *    grid dimension of the launches; larger values give ATTNQ_EUNSUPPORTED.
 *  - sm_scale (attention calls) is any finite value, zero and negative
 *    values included, or NaN for the default 1/sqrt(d_k) (aiter's
 *    softmax_scale=None; the Ascend scale_value): d_k = head_dim, and 576
 *    for the sparse MLA decode.  Infinities give ATTNQ_EINVAL.
 *  - Layouts are row-major, last index contiguous.  T = total tokens of a
 *    varlen batch; cu_seqlens are int32 prefix sums [B+1], cu[0] = 0,
 *    cu[B] = T (the FlashInfer qo_indptr / kv_indptr of a ragged batch).
 *  - 16-bit float data is bf16 or fp16 as named by an attnq_dtype; fp8 is
 *    OCP e4m3fn (bias 7, max 448, S.1111.111 = NaN).
 */
#ifndef ATTNQ_H
#define ATTNQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTNQ_ABI_VERSION 2

typedef enum {
  ATTNQ_OK = 0,
  ATTNQ_EINVAL = -1,       /* bad argument (null pointer, size, alignment) */
  ATTNQ_EUNSUPPORTED = -2, /* valid but not implemented (head_dim, dtype mix) */
  ATTNQ_EWORKSPACE = -3,   /* workspace smaller than the *_workspace_size() */
  ATTNQ_ELAUNCH = -4       /* the HIP runtime refused a launch */
} attnq_status;

typedef enum { ATTNQ_BF16 = 0, ATTNQ_FP16 = 1, ATTNQ_FP8E4M3 = 2, ATTNQ_INT8 = 3 } attnq_dtype;

typedef enum {
  ATTNQ_Q_FP8_PER_HEAD = 0,   /* fp8 e4m3fn codes, one fp32 descale per head */
  ATTNQ_Q_INT8_PER_BLOCK = 1, /* int8 codes, one fp32 scale per (seq, head, 128-token block) */
  ATTNQ_Q_NONE = 2,           /* unquantized 16-bit data */
  ATTNQ_Q_FP8_PER_HEAD_WIDE = 3, /* fp8 e4m3fn codes as above, each stored as its exact fp16 value */
  ATTNQ_Q_INT8_PER_BLOCK_RAW_Q = 4, /* attn_prefill_varlen only: 16-bit Q quantized inside the call as
                                       INT8_PER_BLOCK, int8 per-block K */
  ATTNQ_Q_FP8_PER_CHANNEL = 5,      /* V only: e4m3fn codes, one fp32 descale per (sequence, kv head,
                                       channel) */
  ATTNQ_Q_FP8_PER_CHANNEL_WIDE = 6, /* V only: the codes of FP8_PER_CHANNEL stored as their exact
                                       fp16 values */
  ATTNQ_Q_FP8_PER_HEAD_MFMA8 = 7    /* attn_prefill_varlen only: FP8_PER_HEAD Q/K with QK^T on the
                                       fp8 matrix instruction, whose 128-product sums carry a
                                       relative error up to ~2^-11.8 of sum |q_d k_d| */
} attnq_qmode;

int attnq_abi_version(void);
const char* attnq_last_error(void);

/*
 * attn_quant_qk -- the varlen "quant qk" step (PaddleNLP "Sage Attention
 * Support Varlen"; aiter "[Triton] FP8 with FA v3 API": fp8 q/k with their
 * descales).
 *   x        [total_tokens, num_heads, head_dim], x_dtype BF16 or FP16.
 *   codes    same shape, 1 byte per element: e4m3fn (FP8_PER_HEAD) or int8.
 *   scales   FP8_PER_HEAD:   fp32 [num_heads], descale = amax/448 (amax over
 *                            all rows and channels of the head; 1 if amax = 0).
 *            INT8_PER_BLOCK: fp32 [batch, num_heads, ceil(max_seqlen/block_tokens)],
 *                            scale = amax/127 over block j = rows
 *                            [cu[b] + j*bt, min(cu[b] + (j+1)*bt, cu[b+1])) (1 if
 *                            amax = 0; 0 for blocks past the sequence's end).
 *   Codes: v = x / scale (IEEE fp32 division); fp8: NaN -> 0x7F, |v| clamped to
 *   448, round to nearest even, sign kept; int8: rint(v) clamped to [-127, 127].
 *   cu_seqlens: required for INT8_PER_BLOCK, ignored (may be NULL) for FP8.
 *   amax_in: optional fp32 [num_heads] per-head amax of x (e.g. from
 *   attn_append_kv_rope); FP8_PER_HEAD then skips its reduction pass.
 *   block_tokens must be 128.  head_dim in {64, 128}.
 */
int attn_quant_qk(const void* x, int x_dtype, const int32_t* cu_seqlens, int batch,
                  int max_seqlen, int total_tokens, int num_heads, int head_dim, int mode,
                  int block_tokens, const float* amax_in, void* codes, float* scales,
                  hipStream_t stream);

/*
 * attn_quant_kv -- the Sage flow's two input passes in one launch: K int8 per
 * 128-token block (exactly attn_quant_qk with INT8_PER_BLOCK on k) and V to
 * the permuted V^T layout unchanged (exactly attn_quant_v_permute with mode
 * NONE on v); the two run side by side in one grid instead of one after the
 * other (PaddleNLP "Sage Attention Support Varlen": the varlen "quant qk" and
 * "quant_transpose_permute v" steps).
 *   k, v [total_tokens, num_kv_heads, head_dim] of `dtype` (BF16 or FP16).
 *   k_codes int8 same shape; k_scales fp32 [batch, num_kv_heads,
 *   ceil(max_seqlen/128)]; v_out [batch, num_kv_heads, head_dim,
 *   round_up(max_seqlen, 128)] 16-bit.  block_tokens must be 128.
 */
int attn_quant_kv(const void* k, const void* v, int dtype, const int32_t* cu_seqlens, int batch,
                  int max_seqlen, int total_tokens, int num_kv_heads, int head_dim, int block_tokens,
                  void* k_codes, float* k_scales, void* v_out, hipStream_t stream);

/*
 * attn_quant_v_permute -- the varlen "quant_transpose_permute v" step
 * (PaddleNLP "Sage Attention Support Varlen").
 *   v      [total_tokens, num_kv_heads, head_dim], BF16 or FP16.
 *   v_out  [batch, num_kv_heads, head_dim, S_pad], S_pad = round_up(max_seqlen, 128):
 *          v_out[b][h][d][32*G + pi(j)] = enc(v[cu[b] + 32*G + j][h][d]) for
 *          tokens 32*G + j < L_b, all-zero bytes past L_b, with
 *          pi(j) = 8*((j%16)/4) + 4*(j/16) + j%4 (the order in which the
 *          prefill kernel's PV operand reads a 32-token group).
 *   mode   FP8_PER_HEAD: enc = e4m3fn code as in attn_quant_qk, 1 byte/element,
 *          v_scales fp32 [num_kv_heads] receives the descales;
 *          FP8_PER_HEAD_WIDE: the same codes and descales, each code stored as
 *          its value in fp16 (exact for every finite e4m3fn code), 2 bytes/element:
 *          the prefill then stages V with no widening step (pass v_dtype FP16
 *          and the descales as v_scale);
 *          FP8_PER_CHANNEL / FP8_PER_CHANNEL_WIDE (SageAttention's fp8 V with a
 *          scale per channel; the pages give V descales per head only): as the
 *          two modes above, but v_scales is fp32 [batch, num_kv_heads, head_dim]
 *          (16-byte aligned for the prefill) and receives descale = amax/448
 *          with amax over the sequence's tokens in that channel (1 if amax = 0,
 *          so also for an empty sequence); amax_in must be NULL;
 *          NONE: enc = the unchanged 16-bit value, v_scales ignored.
 *   amax_in optional, as in attn_quant_qk.
 */
int attn_quant_v_permute(const void* v, int v_dtype, const int32_t* cu_seqlens, int batch,
                         int max_seqlen, int total_tokens, int num_kv_heads, int head_dim,
                         int mode, const float* amax_in, void* v_out, float* v_scales,
                         hipStream_t stream);

/*
 * attn_append_kv_rope -- RoPE + write of the new K/V into a paged 16-bit
 * cache (PaddleNLP "write kv cache BF16/FP16 with RoPE"; FlashInfer's paged
 * layout and rope_theta).
 *   q [total_tokens, num_q_heads, head_dim], k/v [total_tokens, num_kv_heads, head_dim],
 *   all of `dtype` (BF16 or FP16).  q and k are rotated IN PLACE; v is read.
 *   Token i of sequence b has position p = (kv_len_before ? kv_len_before[b] : 0) + i.
 *   rope_cos_sin fp32 [max_pos, head_dim/2, 2] = (cos, sin) of p*theta^(-2i/D),
 *   built by the caller.  Rotate-half: for i < D/2, in fp32 with each product
 *   and sum rounded separately,
 *     y[i] = x[i]*c - x[i+D/2]*s,   y[i+D/2] = x[i+D/2]*c + x[i]*s,
 *   then rounded to `dtype` (nearest even).
 *   k_cache / v_cache [num_pages, page_size, num_kv_heads, head_dim] (NHD):
 *   position p of sequence b goes to page kv_indices[kv_indptr[b] + p/page_size],
 *   slot p % page_size; rotated k and unrotated v are written, nothing else.
 *   amax_q/amax_k/amax_v: optional fp32 [heads] outputs, max |value| per head
 *   of the stored rotated q, rotated k and v (input for attn_quant_qk's amax_in).
 *   Tokens whose position is >= max_pos, or whose page index is outside
 *   [0, num_pages), are not written.
 */
int attn_append_kv_rope(void* q, void* k, const void* v, int dtype, const int32_t* cu_seqlens,
                        const int32_t* kv_len_before, int batch, int total_tokens,
                        int num_q_heads, int num_kv_heads, int head_dim,
                        const float* rope_cos_sin, int max_pos, void* k_cache, void* v_cache,
                        const int32_t* kv_indptr, const int32_t* kv_indices, int num_pages,
                        int page_size, float* amax_q, float* amax_k, float* amax_v,
                        hipStream_t stream);

/*
 * attn_prefill_varlen -- causal or full attention over a ragged batch
 * (FlashInfer BatchPrefillWithRaggedKVCacheRun; aiter flash_attn_func with fp8
 * q/k/v and descales; PaddleNLP Sage attention over a varlen batch).
 *   q [total_q, num_q_heads, head_dim] and k [total_k, num_kv_heads, head_dim]:
 *     qk_dtype FP8E4M3 with scale_mode FP8_PER_HEAD (q_scale [Hq], k_scale [Hkv]): QK^T
 *     is summed exactly (up to fp32 accumulation) from the codes' fp16 values; or
 *     FP8E4M3 with FP8_PER_HEAD_MFMA8: the same scales, QK^T on the fp8 matrix
 *     instruction (faster; each 128-term dot product may be off by ~2^-11.8 of
 *     sum_d |q_d k_d|, which moves large logits -- outlier-heavy rows -- by more
 *     than the output tolerance allows), or
 *     qk_dtype INT8 with scale_mode INT8_PER_BLOCK (q_scale [B, Hq, ceil(max_seqlen_q/128)],
 *     k_scale [B, Hkv, ceil(max_seqlen_k/128)], as written by attn_quant_qk): the
 *     integer dot products are exact and each tile's multiplier sm_scale * log2(e) *
 *     q scale * k block scale is carried to 22 significant bits (2^-23 relative, felt
 *     only by logits of ~1e4 and more), or
 *     qk_dtype BF16 / FP16 with scale_mode INT8_PER_BLOCK_RAW_Q: q is the unquantized
 *     16-bit tensor of that type and k the int8 codes with k_scale as above.  Each
 *     128-query block (counted from its sequence's start) is quantized inside the
 *     call to exactly the codes and scale attn_quant_qk INT8_PER_BLOCK produces, so
 *     the result equals quantize-then-attend; q_scale is then an optional OUTPUT
 *     [B, Hq, ceil(max_seqlen_q/128)] receiving the scale of every block that holds
 *     a query (other entries are left as they are).  The codes never reach memory.
 *   v_perm: attn_quant_v_permute's output for the keys, [B, Hkv, D, round_up(max_seqlen_k,128)];
 *     v_dtype FP8E4M3 (v_scale required) or FP16 (v_scale optional: when given,
 *     V = value * descale, as for the _WIDE modes).  v_scale_mode FP8_PER_HEAD:
 *     v_scale [Hkv], one descale per kv head; FP8_PER_CHANNEL: v_scale [B, Hkv, D]
 *     as written by attn_quant_v_permute's per-channel modes (required, 16-byte
 *     aligned), V[j][d] = value * v_scale[b][kv head][d], applied to the output
 *     column d after the PV product.  The padding
 *     past each sequence's keys must hold finite values (attn_quant_v_permute
 *     writes zeros there): it meets p = 0 in the PV product.
 *   logit(i, j) = sm_scale * Dequant(q_i) . Dequant(k_j); q head h reads kv head
 *   h / (Hq/Hkv).  causal: key j visible to query i iff j <= i + L_k - L_q
 *   (bottom-right aligned); a masked key contributes nothing whatever the
 *   sign of sm_scale or of the scales.  With cu_seqlens_q != cu_seqlens_k a
 *   sequence may have queries and no keys (its rows get o = 0, lse = -inf).
 *   o [total_q, num_q_heads, head_dim], o_dtype BF16 or FP16.
 *   lse optional fp32 [num_q_heads, total_q], natural log; rows with no visible
 *   key get o = 0 and lse = -inf.
 *   Supported: head_dim 64 or 128; either Q/K mode with either V type;
 *   max_seqlen_k * num_kv_heads * head_dim < 2^31 (tiles are addressed with
 *   32-bit offsets inside one sequence), else ATTNQ_EUNSUPPORTED.
 */
int attn_prefill_varlen(const void* q, const void* k, const void* v_perm, int qk_dtype,
                        int v_dtype, const float* q_scale, const float* k_scale,
                        const float* v_scale, int v_scale_mode, int scale_mode, const int32_t* cu_seqlens_q,
                        const int32_t* cu_seqlens_k, int batch, int max_seqlen_q,
                        int max_seqlen_k, int total_q, int total_k, int num_q_heads,
                        int num_kv_heads, int head_dim, float sm_scale, int causal, void* o,
                        int o_dtype, float* lse, hipStream_t stream);

/*
 * attn_smooth_quant_k -- SageAttention's smoothing of K before its int8
 * quantization (PaddleNLP "Sage Attention Support Varlen" and SageAttention:
 * subtracting a per-channel mean from K changes every logit of a query by
 * the same amount, so the softmax output is unchanged while the channel
 * offsets stop inflating the int8 block scales).
 *   k fp16 [total_tokens, num_kv_heads, head_dim], cu_seqlens [batch+1] (device).
 *   mean fp32 [batch, num_kv_heads, head_dim] (written): the mean of each channel
 *   over the sequence's tokens, fp32(fp64(S) / fp64(L)) with S the exact sum; 0
 *   for an empty sequence.
 *   codes int8 [total_tokens, num_kv_heads, head_dim] and scales fp32
 *   [batch, num_kv_heads, ceil(max_seqlen/128)]: attn_quant_qk's INT8_PER_BLOCK
 *   applied to k - mean (one fp32 subtraction per element).
 *   With these codes attn_prefill_varlen returns the same softmax output; its
 *   lse is that of the smoothed logits, i.e. lower by sm_scale * q . mean for
 *   each query.  block_tokens must be 128; head_dim in {64, 128}.
 */
int attn_smooth_quant_k(const void* k, const int32_t* cu_seqlens, int batch, int max_seqlen,
                        int total_tokens, int num_kv_heads, int head_dim, int block_tokens,
                        void* codes, float* scales, float* mean, hipStream_t stream);

/*
 * attn_gather_paged_kv -- reads a paged KV cache into the ragged contiguous
 * layout [total_k, num_kv_heads, head_dim], so that a prefill chunk can attend
 * to the tokens already in the cache (FlashInfer's prefill run against a paged
 * KV cache; the pages as FlashInfer and attn_append_kv_rope lay them out).
 *   cache [num_pages, page_size, num_kv_heads, head_dim] (NHD), elem_bytes 1
 *   (fp8 / int8 codes) or 2 (bf16 / fp16); the bytes are copied unchanged.
 *   kv_indptr [batch+1], kv_indices [kv_indptr[batch]], kv_last_page_len [batch]:
 *   sequence b holds kv_len[b] = (kv_indptr[b+1]-kv_indptr[b]-1)*page_size +
 *   kv_last_page_len[b] tokens (0 with no page); token i is slot i % page_size of
 *   page kv_indices[kv_indptr[b] + i / page_size].
 *   cu_seqlens_k [batch+1] (device): row cu_seqlens_k[b] + i of out receives token i,
 *   for i < cu_seqlens_k[b+1] - cu_seqlens_k[b]; rows past kv_len[b], and rows whose
 *   page index lies outside [0, num_pages), are zero-filled.  max_seqlen_k must be
 *   >= every cu_seqlens_k[b+1] - cu_seqlens_k[b] (rows beyond it are not written).
 *   out [cu_seqlens_k[batch], num_kv_heads, head_dim], caller-allocated.
 *   head_dim in {64, 128}.  All pointers are device pointers; nothing is allocated.
 */
int attn_gather_paged_kv(const void* cache, int elem_bytes, const int32_t* kv_indptr,
                         const int32_t* kv_indices, const int32_t* kv_last_page_len,
                         const int32_t* cu_seqlens_k, int batch, int max_seqlen_k, int num_pages,
                         int page_size, int num_kv_heads, int head_dim, void* out,
                         hipStream_t stream);

/*
 * attn_prefill_paged -- a prefill chunk attending to a paged fp8 KV cache,
 * the pages read inside the attention kernel (FlashInfer
 * BatchPrefillWithPagedKVCacheRun over paged_kv_indptr / paged_kv_indices /
 * paged_kv_last_page_len; aiter's flash_attn_with_kvcache with an fp8 cache,
 * a page table and descales).
 *   q fp8 e4m3fn codes [total_q, num_q_heads, head_dim] with q_scale fp32 [Hq]
 *     (attn_quant_qk FP8_PER_HEAD); scale_mode FP8_PER_HEAD (QK^T summed
 *     exactly, as in attn_prefill_varlen) or FP8_PER_HEAD_MFMA8.
 *   k_cache / v_cache fp8 e4m3fn [num_pages, page_size, num_kv_heads, head_dim]
 *     (NHD), k_scale / v_scale fp32 [Hkv]: the cache attn_decode_paged reads.
 *   kv_indptr [batch+1], kv_indices, kv_last_page_len [batch]: sequence b's
 *     keys are kv_len[b] = (kv_indptr[b+1]-kv_indptr[b]-1)*page_size +
 *     kv_last_page_len[b] tokens (0 without a page), token t in page
 *     kv_indices[kv_indptr[b] + t/page_size], slot t % page_size.  Page ids
 *     outside [0, num_pages) are clamped into it.  Slots past kv_len in the
 *     last page may hold anything (NaN codes included): they are not read
 *     into the result.
 *   cu_seqlens_q [batch+1]: the chunk's queries of sequence b, the last
 *     L_q of its kv_len positions (causal: query i sees key j iff
 *     j <= i + kv_len - L_q).
 *   max_seqlen_q, max_kv_len: host upper bounds of L_q and kv_len.
 *   logit, masking, sm_scale (NaN: 1/sqrt(head_dim)), o [total_q, Hq, D]
 *   (BF16 or FP16) and lse (optional fp32 [Hq, total_q]) as attn_prefill_varlen.
 *   Supported: head_dim 64 or 128, page_size a multiple of 16 in [16, 1024],
 *   num_pages * page_size * num_kv_heads * head_dim < 2^31 bytes, else
 *   ATTNQ_EUNSUPPORTED.
 */
int attn_prefill_paged(const void* q, const float* q_scale, int scale_mode, const void* k_cache,
                       const void* v_cache, const float* k_scale, const float* v_scale,
                       const int32_t* kv_indptr, const int32_t* kv_indices,
                       const int32_t* kv_last_page_len, const int32_t* cu_seqlens_q, int batch,
                       int num_pages, int page_size, int max_seqlen_q, int max_kv_len, int total_q,
                       int num_q_heads, int num_kv_heads, int head_dim, float sm_scale, int causal,
                       void* o, int o_dtype, float* lse, hipStream_t stream);

/*
 * attn_decode_paged -- one query token per sequence against a paged fp8 cache,
 * split over KV chunks and merged by log-sum-exp (FlashInfer
 * BatchDecodeWithPagedKVCachePlan/Run; aiter's paged fp8 flash_attn_with_kvcache).
 *   q bf16 [batch, num_q_heads, head_dim]; k_cache / v_cache fp8 e4m3fn
 *   [num_pages, page_size, num_kv_heads, head_dim] (NHD); k_scale / v_scale fp32 [Hkv].
 *   kv_indptr [batch+1], kv_indices [kv_indptr[batch]], kv_last_page_len [batch]:
 *   kv_len[b] = (kv_indptr[b+1]-kv_indptr[b]-1)*page_size + kv_last_page_len[b]
 *   (0 if the sequence has no page); token t lives in page
 *   kv_indices[kv_indptr[b] + t/page_size], slot t % page_size.
 *   max_kv_len: host upper bound of every kv_len (sizes the split).
 *   workspace: caller-owned device scratch of at least
 *   attn_decode_paged_workspace_size(...) bytes (partial O and lse).
 *   o bf16 [batch, num_q_heads, head_dim]; lse optional fp32 [batch, num_q_heads].
 *   Supported: head_dim 64 or 128, num_q_heads % num_kv_heads == 0, group <= 16,
 *   page_size a multiple of 16 and <= 1024.
 */
size_t attn_decode_paged_workspace_size(int batch, int num_q_heads, int head_dim, int max_kv_len,
                                        int page_size);
int attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                      const float* k_scale, const float* v_scale, const int32_t* kv_indptr,
                      const int32_t* kv_indices, const int32_t* kv_last_page_len, int batch,
                      int num_pages, int page_size, int num_q_heads, int num_kv_heads,
                      int head_dim, int max_kv_len, float sm_scale, void* workspace,
                      size_t workspace_bytes, void* o, float* lse, hipStream_t stream);

/*
 * attn_decode_paged_noalloc -- attn_decode_paged for callers that cannot
 * allocate device memory (code recorded under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the same arguments without the
 * workspace, the same kernels and results.  The split partials go to a fixed
 * scratch array inside the library (80 MiB per device, held from the first
 * call on a device until the process ends); no call allocates or frees
 * anything.  Sizes whose partials, attn_decode_paged_workspace_size(...),
 * exceed 80 MiB return ATTNQ_EWORKSPACE with a message (80 MiB holds
 * 64 sequences x 32 q heads of 32K-token caches at head_dim 128).  Every call
 * on one device shares that device's scratch: calls that may overlap on one
 * device (several streams or threads) race and must be serialized by the
 * caller.  Nothing in the scratch needs clearing between calls.
 */
int attn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const float* k_scale, const float* v_scale, const int32_t* kv_indptr,
                              const int32_t* kv_indices, const int32_t* kv_last_page_len, int batch,
                              int num_pages, int page_size, int num_q_heads, int num_kv_heads,
                              int head_dim, int max_kv_len, float sm_scale, void* o, float* lse,
                              hipStream_t stream);

/*
 * attn_sparse_mla_decode -- MLA-absorb sparse attention over int8 or fp8 cache
 * rows with per-token tile-128 scales (Ascend "KvQuantSparseFlashAttention":
 * attention_mode 2, quant_scale_repo_mode 1, tile_size 128, rope_head_dim 64,
 * PA_BSND paging, key/value FLOAT8_E4M3 or INT8, sparse_block_size,
 * sparse_mode 0 or 3).
 *   q bf16 [batch, s_q, num_heads, 576] = [q_nope 512 | q_rope 64].
 *   kv_cache uint8 [num_blocks, block_size, 1, 656]; each 656-byte row is
 *     512 nope codes (kv_dtype INT8: int8; FP8E4M3: e4m3fn) | 64 bf16 rope values |
 *     4 fp32 scales (scale t covers nope channels [128t, 128t+128)).
 *     K = [codes*scale | rope], V = codes*scale.
 *   block_table int32 [batch, max_blocks_per_seq]: token i of sequence b is row
 *     i % block_size of block block_table[b][i / block_size].
 *   kv_lens int32 [batch]; sparse_indices int32 [batch, s_q, 1, topk]: an entry
 *     e >= 0 names the sparse_block_size tokens [e*sbs, e*sbs + sbs) (tokens of a
 *     block share its selection; -1 padding after the valid entries); a named
 *     token is used iff it is below kv_lens[b] and, with sparse_mode 3 (the
 *     right-down causal mask), at most kv_lens[b] - s_q + s for query row s.
 *     Each used token is one softmax term (an entry given twice counts twice).
 *   sparse_block_size in {1, 2, 4, 8, 16} (so it divides block_size).
 *   o bf16 [batch, s_q, num_heads, 512]; lse optional fp32 [batch, s_q, num_heads];
 *   rows with no used token get o = 0 and lse = -inf.
 *   Tile scales: any value with |s| <= 2^100 (zero and negative included);
 *   the kernels round p * s to bf16 with p <= 2^14, which stays finite in
 *   that range.
 *   num_heads in {1,2,4,8,16,32,48,64,128}; block_size a multiple of 16, <= 1024;
 *   topk > 0.  workspace >= attn_sparse_mla_decode_workspace_size(...) bytes,
 *   256-byte aligned (0 is returned for invalid sizes).
 */
size_t attn_sparse_mla_decode_workspace_size(int batch, int s_q, int num_heads, int topk,
                                             int sparse_block_size);
int attn_sparse_mla_decode(const void* q, const void* kv_cache, int kv_dtype,
                           const int32_t* block_table, int max_blocks_per_seq,
                           const int32_t* kv_lens, const int32_t* sparse_indices, int topk,
                           int sparse_block_size, int sparse_mode, int batch, int s_q,
                           int num_heads, int num_blocks, int block_size, float sm_scale,
                           void* workspace, size_t workspace_bytes, void* o, float* lse,
                           hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* ATTNQ_H */
