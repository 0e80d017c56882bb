// C ABI of libattnq: host-side validation, launch geometry and status codes.
// No entry point allocates, frees, copies or synchronizes; each validates its
// host arguments first and only then enqueues kernels on the caller's stream.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/attnq.h"
#include "launch.h"
#include "gather.h"
#include "smooth.h"
#include "mla.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return ATTNQ_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

#define REQUIRE(cond, code, ...) \
  do {                           \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

#define REQUIRE_PTR(p, a) \
  do { \
    REQUIRE((p) != nullptr, ATTNQ_EINVAL, "%s must not be NULL", #p); \
    REQUIRE(aligned((p), (a)), ATTNQ_EINVAL, "%s must be %d-byte aligned", #p, (int)(a)); \
  } while (0)

#define REQUIRE_OPT_PTR(p, a) \
  do { \
    REQUIRE((p) == nullptr || aligned((p), (a)), ATTNQ_EINVAL, "%s must be %d-byte aligned", #p, (int)(a)); \
  } while (0)

#define LAUNCHED(x) \
  do { \
    if (!(x)) return fail(ATTNQ_ELAUNCH, "kernel launch failed: %s", hipGetErrorString(hipGetLastError())); \
  } while (0)

const float LOG2E = 1.4426950408889634f;

bool is16(int dt) { return dt == ATTNQ_BF16 || dt == ATTNQ_FP16; }

// sm_scale: any finite value, or NaN for the default 1/sqrt(d_k) (aiter's
// softmax_scale=None; the Ascend scale_value); infinities are rejected.
bool scale_ok(float s) { return std::isfinite(s) || std::isnan(s); }
float scale_or_default(float s, int d_k) { return std::isnan(s) ? (float)(1.0 / std::sqrt((double)d_k)) : s; }
int round_up(int x, int m) { return ((x + m - 1) / m) * m; }

}  // namespace

extern "C" {

int attnq_abi_version(void) { return ATTNQ_ABI_VERSION; }

const char* attnq_last_error(void) { return g_err.c_str(); }

// ---------------------------------------------------------------- attn_quant_qk
int attn_quant_qk(const void* x, int x_dtype, const int32_t* cu_seqlens, int batch, int max_seqlen,
                  int total_tokens, int num_heads, int head_dim, int mode, int block_tokens,
                  const float* amax_in, void* codes, float* scales, hipStream_t stream) {
  REQUIRE(is16(x_dtype), ATTNQ_EUNSUPPORTED, "x_dtype must be BF16 or FP16");
  REQUIRE(head_dim == 64 || head_dim == 128, ATTNQ_EUNSUPPORTED, "head_dim must be 64 or 128 (got %d)", head_dim);
  REQUIRE(num_heads > 0 && num_heads <= 1024, ATTNQ_EINVAL, "num_heads must be in [1, 1024] (got %d)", num_heads);
  REQUIRE(total_tokens >= 0, ATTNQ_EINVAL, "total_tokens must be >= 0");
  REQUIRE(mode == ATTNQ_Q_FP8_PER_HEAD || mode == ATTNQ_Q_INT8_PER_BLOCK, ATTNQ_EINVAL,
          "mode must be FP8_PER_HEAD or INT8_PER_BLOCK");
  REQUIRE_PTR(scales, 4);
  if (total_tokens > 0) {
    REQUIRE_PTR(x, 16);
    REQUIRE_PTR(codes, 16);
  }
  REQUIRE_OPT_PTR(amax_in, 4);
  const bool bf = x_dtype == ATTNQ_BF16;
  if (mode == ATTNQ_Q_FP8_PER_HEAD) {
    if (!amax_in) {
      LAUNCHED(attnq::launch_fill_u32(reinterpret_cast<uint32_t*>(scales), num_heads, 0u, stream));
      LAUNCHED(attnq::launch_amax(x, total_tokens, num_heads, head_dim, bf,
                                  reinterpret_cast<uint32_t*>(scales), stream));
    }
    LAUNCHED(attnq::launch_finalize_scale(amax_in, scales, num_heads, 448.0f, stream));
    LAUNCHED(attnq::launch_quant_fp8(x, (long)total_tokens * num_heads * head_dim, num_heads, head_dim,
                                     bf, scales, codes, stream));
    return ok();
  }
  REQUIRE(block_tokens == 128, ATTNQ_EUNSUPPORTED, "block_tokens must be 128 (got %d)", block_tokens);
  REQUIRE(batch >= 0, ATTNQ_EINVAL, "batch must be >= 0");
  REQUIRE(batch <= 65535, ATTNQ_EUNSUPPORTED, "batch must be <= 65535");
  REQUIRE(max_seqlen >= 0, ATTNQ_EINVAL, "max_seqlen must be >= 0");
  REQUIRE(amax_in == nullptr, ATTNQ_EINVAL, "amax_in applies to FP8_PER_HEAD only");
  REQUIRE_PTR(cu_seqlens, 4);
  const int nblk = (max_seqlen + block_tokens - 1) / block_tokens;
  LAUNCHED(attnq::launch_quant_int8_block(x, cu_seqlens, batch, num_heads, head_dim, block_tokens, nblk,
                                          bf, total_tokens, codes, scales, stream));
  return ok();
}

// ---------------------------------------------------------------- attn_quant_kv
int attn_quant_kv(const void* k, const void* v, int dtype, const int32_t* cu_seqlens, int batch,
                  int max_seqlen, int total_tokens, int num_kv_heads, int head_dim, int block_tokens,
                  void* k_codes, float* k_scales, void* v_out, hipStream_t stream) {
  REQUIRE(is16(dtype), ATTNQ_EUNSUPPORTED, "dtype must be BF16 or FP16");
  REQUIRE(head_dim == 64 || head_dim == 128, ATTNQ_EUNSUPPORTED, "head_dim must be 64 or 128 (got %d)", head_dim);
  REQUIRE(num_kv_heads > 0 && num_kv_heads <= 1024, ATTNQ_EINVAL, "num_kv_heads must be in [1, 1024]");
  REQUIRE(block_tokens == 128, ATTNQ_EUNSUPPORTED, "block_tokens must be 128 (got %d)", block_tokens);
  REQUIRE(batch >= 0 && max_seqlen >= 0 && total_tokens >= 0, ATTNQ_EINVAL, "sizes must be >= 0");
  REQUIRE(batch <= 65535, ATTNQ_EUNSUPPORTED, "batch must be <= 65535");
  if (batch == 0 || max_seqlen == 0) return ok();
  REQUIRE_PTR(cu_seqlens, 4);
  REQUIRE_PTR(k_scales, 4);
  REQUIRE_PTR(v_out, 16);
  if (total_tokens > 0) {
    REQUIRE_PTR(k, 16);
    REQUIRE_PTR(v, 16);
    REQUIRE_PTR(k_codes, 16);
  }
  const int nblk = (max_seqlen + 127) / 128;
  LAUNCHED(attnq::launch_quant_k_permute_v(k, v, cu_seqlens, batch, num_kv_heads, head_dim, nblk,
                                           round_up(max_seqlen, 128), dtype == ATTNQ_BF16, total_tokens,
                                           k_codes, k_scales, v_out, stream));
  return ok();
}

// ---------------------------------------------------------------- attn_quant_v_permute
int attn_quant_v_permute(const void* v, int v_dtype, const int32_t* cu_seqlens, int batch,
                         int max_seqlen, int total_tokens, int num_kv_heads, int head_dim,
                         int mode, const float* amax_in, void* v_out, float* v_scales,
                         hipStream_t stream) {
  REQUIRE(is16(v_dtype), ATTNQ_EUNSUPPORTED, "v_dtype must be BF16 or FP16");
  REQUIRE(head_dim == 64 || head_dim == 128, ATTNQ_EUNSUPPORTED, "head_dim must be 64 or 128 (got %d)", head_dim);
  REQUIRE(num_kv_heads > 0 && num_kv_heads <= 1024, ATTNQ_EINVAL, "num_kv_heads must be in [1, 1024]");
  REQUIRE(batch >= 0 && max_seqlen >= 0 && total_tokens >= 0, ATTNQ_EINVAL, "sizes must be >= 0");
  REQUIRE(batch <= 65535, ATTNQ_EUNSUPPORTED, "batch must be <= 65535");
  const bool chan = mode == ATTNQ_Q_FP8_PER_CHANNEL || mode == ATTNQ_Q_FP8_PER_CHANNEL_WIDE;
  REQUIRE(mode == ATTNQ_Q_FP8_PER_HEAD || mode == ATTNQ_Q_FP8_PER_HEAD_WIDE || mode == ATTNQ_Q_NONE || chan,
          ATTNQ_EINVAL, "mode must be FP8_PER_HEAD, FP8_PER_HEAD_WIDE, FP8_PER_CHANNEL, FP8_PER_CHANNEL_WIDE or NONE");
  REQUIRE(!chan || !amax_in, ATTNQ_EINVAL, "amax_in holds per-head maxima: not accepted with a per-channel mode");
  REQUIRE(!chan || (long)batch * num_kv_heads * head_dim < (1L << 31), ATTNQ_EUNSUPPORTED,
          "batch * num_kv_heads * head_dim must stay below 2^31");
  REQUIRE_PTR(cu_seqlens, 4);
  REQUIRE_OPT_PTR(amax_in, 4);
  const int s_pad = round_up(max_seqlen, 128);
  if (batch > 0 && s_pad > 0) REQUIRE_PTR(v_out, 16);
  if (total_tokens > 0) REQUIRE_PTR(v, 16);
  const bool bf = v_dtype == ATTNQ_BF16;
  if (chan) {
    if (batch == 0) return ok();
    REQUIRE_PTR(v_scales, 4);
    LAUNCHED(attnq::launch_v_permute_per_channel(v, cu_seqlens, batch, num_kv_heads, head_dim, s_pad, bf,
                                                 total_tokens, mode == ATTNQ_Q_FP8_PER_CHANNEL_WIDE,
                                                 v_scales, v_out, stream));
    return ok();
  }
  const bool wide = mode == ATTNQ_Q_FP8_PER_HEAD_WIDE;
  const bool fp8 = mode == ATTNQ_Q_FP8_PER_HEAD || wide;
  if (fp8) {
    REQUIRE_PTR(v_scales, 4);
    if (!amax_in) {
      LAUNCHED(attnq::launch_fill_u32(reinterpret_cast<uint32_t*>(v_scales), num_kv_heads, 0u, stream));
      LAUNCHED(attnq::launch_amax(v, total_tokens, num_kv_heads, head_dim, bf,
                                  reinterpret_cast<uint32_t*>(v_scales), stream));
    }
    LAUNCHED(attnq::launch_finalize_scale(amax_in, v_scales, num_kv_heads, 448.0f, stream));
  }
  LAUNCHED(attnq::launch_v_permute(v, cu_seqlens, batch, num_kv_heads, head_dim, s_pad, bf,
                                   total_tokens, fp8, wide, fp8 ? v_scales : nullptr, v_out, stream));
  return ok();
}

// ---------------------------------------------------------------- attn_append_kv_rope
int attn_append_kv_rope(void* q, void* k, const void* v, int dtype, const int32_t* cu_seqlens,
                        const int32_t* kv_len_before, int batch, int total_tokens,
                        int num_q_heads, int num_kv_heads, int head_dim,
                        const float* rope_cos_sin, int max_pos, void* k_cache, void* v_cache,
                        const int32_t* kv_indptr, const int32_t* kv_indices, int num_pages,
                        int page_size, float* amax_q, float* amax_k, float* amax_v,
                        hipStream_t stream) {
  REQUIRE(is16(dtype), ATTNQ_EUNSUPPORTED, "dtype must be BF16 or FP16");
  REQUIRE(head_dim == 64 || head_dim == 128, ATTNQ_EUNSUPPORTED, "head_dim must be 64 or 128 (got %d)", head_dim);
  REQUIRE(num_q_heads > 0 && num_kv_heads > 0, ATTNQ_EINVAL, "head counts must be positive");
  REQUIRE(attnq::rope_units_fit(num_q_heads, num_kv_heads, head_dim), ATTNQ_EUNSUPPORTED,
          "num_q_heads + 2*num_kv_heads too large for one token per workgroup");
  REQUIRE(batch >= 1 && total_tokens >= 0, ATTNQ_EINVAL, "batch must be >= 1, total_tokens >= 0");
  REQUIRE(page_size > 0 && page_size <= 1024, ATTNQ_EINVAL, "page_size must be in [1, 1024]");
  REQUIRE(num_pages > 0 && max_pos > 0, ATTNQ_EINVAL, "num_pages and max_pos must be positive");
  REQUIRE_PTR(cu_seqlens, 4);
  REQUIRE_PTR(kv_indptr, 4);
  REQUIRE_PTR(kv_indices, 4);
  REQUIRE_PTR(rope_cos_sin, 16);
  REQUIRE_PTR(k_cache, 16);
  REQUIRE_PTR(v_cache, 16);
  REQUIRE_OPT_PTR(kv_len_before, 4);
  REQUIRE_OPT_PTR(amax_q, 4);
  REQUIRE_OPT_PTR(amax_k, 4);
  REQUIRE_OPT_PTR(amax_v, 4);
  if (total_tokens > 0) {
    REQUIRE_PTR(q, 16);
    REQUIRE_PTR(k, 16);
    REQUIRE_PTR(v, 16);
  }
  if (amax_q) LAUNCHED(attnq::launch_fill_u32(reinterpret_cast<uint32_t*>(amax_q), num_q_heads, 0u, stream));
  if (amax_k) LAUNCHED(attnq::launch_fill_u32(reinterpret_cast<uint32_t*>(amax_k), num_kv_heads, 0u, stream));
  if (amax_v) LAUNCHED(attnq::launch_fill_u32(reinterpret_cast<uint32_t*>(amax_v), num_kv_heads, 0u, stream));
  LAUNCHED(attnq::launch_append_rope(q, k, v, dtype == ATTNQ_BF16, cu_seqlens, kv_len_before, batch,
                                     total_tokens, num_q_heads, num_kv_heads, head_dim, rope_cos_sin,
                                     max_pos, k_cache, v_cache, kv_indptr, kv_indices, num_pages,
                                     page_size, amax_q, amax_k, amax_v, stream));
  return ok();
}

// ---------------------------------------------------------------- attn_prefill_varlen
int attn_prefill_varlen(const void* q, const void* k, const void* v_perm, int qk_dtype,
                        int v_dtype, const float* q_scale, const float* k_scale,
                        const float* v_scale, int v_scale_mode, int scale_mode, const int32_t* cu_seqlens_q,
                        const int32_t* cu_seqlens_k, int batch, int max_seqlen_q,
                        int max_seqlen_k, int total_q, int total_k, int num_q_heads,
                        int num_kv_heads, int head_dim, float sm_scale, int causal, void* o,
                        int o_dtype, float* lse, hipStream_t stream) {
  REQUIRE(head_dim == 64 || head_dim == 128, ATTNQ_EUNSUPPORTED, "head_dim must be 64 or 128 (got %d)", head_dim);
  REQUIRE(num_q_heads > 0 && num_kv_heads > 0 && num_q_heads % num_kv_heads == 0, ATTNQ_EINVAL,
          "num_q_heads must be a positive multiple of num_kv_heads");
  const bool fp8_mma8 = qk_dtype == ATTNQ_FP8E4M3 && scale_mode == ATTNQ_Q_FP8_PER_HEAD_MFMA8;
  const bool fp8qk = (qk_dtype == ATTNQ_FP8E4M3 && scale_mode == ATTNQ_Q_FP8_PER_HEAD) || fp8_mma8;
  const bool i8qk = qk_dtype == ATTNQ_INT8 && scale_mode == ATTNQ_Q_INT8_PER_BLOCK;
  const bool rawq = is16(qk_dtype) && scale_mode == ATTNQ_Q_INT8_PER_BLOCK_RAW_Q;
  REQUIRE(fp8qk || i8qk || rawq, ATTNQ_EUNSUPPORTED,
          "supported Q/K: FP8E4M3 with FP8_PER_HEAD or FP8_PER_HEAD_MFMA8 scales, INT8 with "
          "INT8_PER_BLOCK scales, or BF16/FP16 Q with INT8_PER_BLOCK_RAW_Q");
  REQUIRE(!rawq || (long)num_q_heads * head_dim < (1L << 22), ATTNQ_EUNSUPPORTED,
          "INT8_PER_BLOCK_RAW_Q: num_q_heads * head_dim must stay below 2^22");
  REQUIRE(v_dtype == ATTNQ_FP8E4M3 || v_dtype == ATTNQ_FP16, ATTNQ_EUNSUPPORTED, "v_dtype must be FP8E4M3 or FP16");
  REQUIRE(is16(o_dtype), ATTNQ_EUNSUPPORTED, "o_dtype must be BF16 or FP16");
  REQUIRE(batch >= 0 && max_seqlen_q >= 0 && max_seqlen_k >= 0 && total_q >= 0 && total_k >= 0,
          ATTNQ_EINVAL, "sizes must be >= 0");
  REQUIRE(max_seqlen_q <= 65535 * 128, ATTNQ_EINVAL, "max_seqlen_q too large");
  // K and V^T tiles are addressed with 32-bit byte offsets from the start of
  // one (sequence, kv head)
  REQUIRE((long)max_seqlen_k * num_kv_heads * head_dim < (1L << 31) &&
              (long)round_up(max_seqlen_k, 128) * head_dim * 2 < (1L << 31),
          ATTNQ_EUNSUPPORTED, "one sequence's K (max_seqlen_k * num_kv_heads * head_dim bytes) must stay below 2 GiB");
  REQUIRE(scale_ok(sm_scale), ATTNQ_EINVAL, "sm_scale must be finite (or NaN for 1/sqrt(head_dim))");
  sm_scale = scale_or_default(sm_scale, head_dim);
  REQUIRE_PTR(cu_seqlens_q, 4);
  REQUIRE_PTR(cu_seqlens_k, 4);
  if (rawq) REQUIRE_OPT_PTR(q_scale, 4);  // an output in this mode
  else REQUIRE_PTR(q_scale, 4);
  REQUIRE_PTR(k_scale, 4);
  REQUIRE(v_scale_mode == ATTNQ_Q_FP8_PER_HEAD || v_scale_mode == ATTNQ_Q_FP8_PER_CHANNEL, ATTNQ_EINVAL,
          "v_scale_mode must be FP8_PER_HEAD or FP8_PER_CHANNEL");
  const bool v_chan = v_scale_mode == ATTNQ_Q_FP8_PER_CHANNEL;
  if (v_chan) REQUIRE_PTR(v_scale, 16);  // read as 4-float vectors
  else if (v_dtype == ATTNQ_FP8E4M3) REQUIRE_PTR(v_scale, 4);
  else REQUIRE_OPT_PTR(v_scale, 4);
  if (total_q > 0) {
    REQUIRE_PTR(q, 16);
    REQUIRE_PTR(o, 16);
  }
  if (total_k > 0) {
    REQUIRE_PTR(k, 16);
    REQUIRE_PTR(v_perm, 16);
  }
  REQUIRE_OPT_PTR(lse, 4);
  attnq::PrefillArgs a;
  a.q = q; a.k = k; a.v = v_perm;
  a.q_scale = q_scale; a.k_scale = k_scale; a.v_scale = v_scale;
  a.v_chan = v_chan ? 1 : 0;
  a.cu_q = cu_seqlens_q; a.cu_k = cu_seqlens_k;
  a.o = o; a.lse = lse;
  a.q_scale_out = rawq ? const_cast<float*>(q_scale) : nullptr;
  a.batch = batch; a.hq = num_q_heads; a.hkv = num_kv_heads;
  a.s_pad = round_up(max_seqlen_k, 128);
  a.nblk_q = (max_seqlen_q + 127) / 128;
  a.nblk_k = (max_seqlen_k + 127) / 128;
  a.total_q = total_q; a.total_k = total_k;
  a.causal = causal ? 1 : 0;
  a.max_q = max_seqlen_q;
  a.max_k = max_seqlen_k;
  a.sm_scale_log2 = sm_scale * LOG2E;
  if (total_q == 0) return ok();
  const int q_mode = fp8_mma8 ? attnq::PF_Q_FP8_MFMA8
                   : fp8qk ? attnq::PF_Q_FP8
                   : i8qk  ? attnq::PF_Q_I8
                   : qk_dtype == ATTNQ_BF16 ? attnq::PF_Q_RAW_BF16 : attnq::PF_Q_RAW_F16;
  LAUNCHED(attnq::launch_prefill(a, head_dim, q_mode, v_dtype == ATTNQ_FP8E4M3, o_dtype == ATTNQ_BF16,
                                 max_seqlen_q, stream));
  return ok();
}

// ---------------------------------------------------------------- attn_prefill_paged
int attn_prefill_paged(const void* q, const float* q_scale, int scale_mode, const void* k_cache,
                       const void* v_cache, const float* k_scale, const float* v_scale,
                       const int32_t* kv_indptr, const int32_t* kv_indices,
                       const int32_t* kv_last_page_len, const int32_t* cu_seqlens_q, int batch,
                       int num_pages, int page_size, int max_seqlen_q, int max_kv_len, int total_q,
                       int num_q_heads, int num_kv_heads, int head_dim, float sm_scale, int causal,
                       void* o, int o_dtype, float* lse, hipStream_t stream) {
  REQUIRE(head_dim == 64 || head_dim == 128, ATTNQ_EUNSUPPORTED, "head_dim must be 64 or 128 (got %d)", head_dim);
  REQUIRE(num_q_heads > 0 && num_kv_heads > 0 && num_q_heads % num_kv_heads == 0, ATTNQ_EINVAL,
          "num_q_heads must be a positive multiple of num_kv_heads");
  REQUIRE(scale_mode == ATTNQ_Q_FP8_PER_HEAD || scale_mode == ATTNQ_Q_FP8_PER_HEAD_MFMA8, ATTNQ_EUNSUPPORTED,
          "scale_mode must be FP8_PER_HEAD or FP8_PER_HEAD_MFMA8");
  REQUIRE(is16(o_dtype), ATTNQ_EUNSUPPORTED, "o_dtype must be BF16 or FP16");
  REQUIRE(page_size >= 16 && page_size <= 1024 && page_size % 16 == 0, ATTNQ_EINVAL,
          "page_size must be a multiple of 16 in [16, 1024] (got %d)", page_size);
  REQUIRE(batch >= 0 && max_seqlen_q >= 0 && max_kv_len >= 0 && total_q >= 0, ATTNQ_EINVAL, "sizes must be >= 0");
  REQUIRE(num_pages > 0, ATTNQ_EINVAL, "num_pages must be positive");
  REQUIRE(max_seqlen_q <= 65535 * 128, ATTNQ_EINVAL, "max_seqlen_q too large");
  // the cache is addressed with 32-bit byte offsets, lanes past a sequence's
  // last key with offset 2^31
  REQUIRE((long)num_pages * page_size * num_kv_heads * head_dim < (1L << 31), ATTNQ_EUNSUPPORTED,
          "the cache (num_pages * page_size * num_kv_heads * head_dim bytes) must stay below 2 GiB");
  REQUIRE(scale_ok(sm_scale), ATTNQ_EINVAL, "sm_scale must be finite (or NaN for 1/sqrt(head_dim))");
  sm_scale = scale_or_default(sm_scale, head_dim);
  if (batch == 0 || total_q == 0) return ok();
  REQUIRE_PTR(q, 16);
  REQUIRE_PTR(q_scale, 4);
  REQUIRE_PTR(k_cache, 16);
  REQUIRE_PTR(v_cache, 16);
  REQUIRE_PTR(k_scale, 4);
  REQUIRE_PTR(v_scale, 4);
  REQUIRE_PTR(kv_indptr, 4);
  REQUIRE_PTR(kv_indices, 4);
  REQUIRE_PTR(kv_last_page_len, 4);
  REQUIRE_PTR(cu_seqlens_q, 4);
  REQUIRE_PTR(o, 16);
  REQUIRE_OPT_PTR(lse, 4);
  attnq::PrefillArgs a;
  a.q = q; a.k = k_cache; a.v = v_cache;
  a.q_scale = q_scale; a.k_scale = k_scale; a.v_scale = v_scale;
  a.v_chan = 0;
  a.cu_q = cu_seqlens_q; a.cu_k = nullptr;
  a.kv_indptr = kv_indptr; a.kv_indices = kv_indices; a.kv_last = kv_last_page_len;
  a.page_size = page_size; a.num_pages = num_pages;
  a.o = o; a.lse = lse;
  a.q_scale_out = nullptr;
  a.batch = batch; a.hq = num_q_heads; a.hkv = num_kv_heads;
  a.s_pad = 0;
  a.nblk_q = (max_seqlen_q + 127) / 128;
  a.nblk_k = (max_kv_len + 127) / 128;
  a.total_q = total_q; a.total_k = 0;
  a.causal = causal ? 1 : 0;
  a.max_q = max_seqlen_q;
  a.max_k = max_kv_len;
  a.sm_scale_log2 = sm_scale * LOG2E;
  const int q_mode = scale_mode == ATTNQ_Q_FP8_PER_HEAD_MFMA8 ? attnq::PF_Q_FP8_MFMA8 : attnq::PF_Q_FP8;
  LAUNCHED(attnq::launch_prefill_paged(a, head_dim, q_mode, o_dtype == ATTNQ_BF16, max_seqlen_q, stream));
  return ok();
}

// ---------------------------------------------------------------- attn_smooth_quant_k
int attn_smooth_quant_k(const void* k, const int32_t* cu_seqlens, int batch, int max_seqlen,
                        int total_tokens, int num_kv_heads, int head_dim, int block_tokens,
                        void* codes, float* scales, float* mean, hipStream_t stream) {
  REQUIRE(head_dim == 64 || head_dim == 128, ATTNQ_EUNSUPPORTED, "head_dim must be 64 or 128 (got %d)", head_dim);
  REQUIRE(block_tokens == 128, ATTNQ_EUNSUPPORTED, "block_tokens must be 128 (got %d)", block_tokens);
  REQUIRE(batch >= 0 && max_seqlen >= 0 && total_tokens >= 0 && num_kv_heads > 0, ATTNQ_EINVAL,
          "batch, max_seqlen, total_tokens must be >= 0 and num_kv_heads > 0");
  REQUIRE(num_kv_heads <= 65535 && batch <= 65535, ATTNQ_EUNSUPPORTED, "num_kv_heads and batch must be <= 65535");
  if (batch == 0) return ok();
  REQUIRE_PTR(cu_seqlens, 4);
  REQUIRE_PTR(mean, 4);
  const int nblk = (max_seqlen + 127) / 128;
  if (nblk > 0) {
    REQUIRE_PTR(scales, 4);
    if (total_tokens > 0) {
      REQUIRE_PTR(k, 16);
      REQUIRE_PTR(codes, 16);
    }
  }
  LAUNCHED(attnq::launch_smooth_quant_int8_block(k, cu_seqlens, batch, num_kv_heads, head_dim, nblk,
                                                 total_tokens, codes, scales, mean, stream));
  return ok();
}

// ---------------------------------------------------------------- attn_gather_paged_kv
int attn_gather_paged_kv(const void* cache, int elem_bytes, const int32_t* kv_indptr,
                         const int32_t* kv_indices, const int32_t* kv_last_page_len,
                         const int32_t* cu_seqlens_k, int batch, int max_seqlen_k, int num_pages,
                         int page_size, int num_kv_heads, int head_dim, void* out,
                         hipStream_t stream) {
  REQUIRE(elem_bytes == 1 || elem_bytes == 2, ATTNQ_EINVAL, "elem_bytes must be 1 or 2 (got %d)", elem_bytes);
  REQUIRE(head_dim == 64 || head_dim == 128, ATTNQ_EUNSUPPORTED, "head_dim must be 64 or 128 (got %d)", head_dim);
  REQUIRE(num_kv_heads > 0 && num_pages > 0 && page_size > 0, ATTNQ_EINVAL,
          "num_kv_heads, num_pages and page_size must be positive");
  REQUIRE(batch >= 0 && max_seqlen_k >= 0, ATTNQ_EINVAL, "batch and max_seqlen_k must be >= 0");
  REQUIRE(batch <= 65535, ATTNQ_EUNSUPPORTED, "batch must be <= 65535");
  if (batch == 0 || max_seqlen_k == 0) return ok();
  REQUIRE((long)num_kv_heads * head_dim * elem_bytes < (1L << 20), ATTNQ_EUNSUPPORTED, "row too wide");
  REQUIRE_PTR(cache, 16);
  REQUIRE_PTR(kv_indptr, 4);
  REQUIRE_PTR(kv_indices, 4);
  REQUIRE_PTR(kv_last_page_len, 4);
  REQUIRE_PTR(cu_seqlens_k, 4);
  REQUIRE_PTR(out, 16);
  attnq::GatherArgs a;
  a.cache = static_cast<const uint8_t*>(cache);
  a.kv_indptr = kv_indptr; a.kv_indices = kv_indices; a.kv_last_page_len = kv_last_page_len;
  a.cu_k = cu_seqlens_k;
  a.out = static_cast<uint8_t*>(out);
  a.batch = batch; a.num_pages = num_pages; a.page_size = page_size;
  a.row_bytes = num_kv_heads * head_dim * elem_bytes;
  LAUNCHED(attnq::launch_gather_paged(a, max_seqlen_k, stream));
  return ok();
}

// ---------------------------------------------------------------- attn_decode_paged
size_t attn_decode_paged_workspace_size(int batch, int num_q_heads, int head_dim, int max_kv_len,
                                        int page_size) {
  if (batch <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_kv_len < 0) return 0;
  return attnq::decode_workspace_bytes(batch, num_q_heads, head_dim, max_kv_len, page_size);
}

}  // extern "C"

namespace {

// Scratch of attn_decode_paged_noalloc: the split partials live in this
// fixed device array instead of a caller workspace.  Each device holds its
// own copy for the life of the process; host code reaches it only through
// the address hipGetSymbolAddress returns on that device (the array's name
// is a host-side stand-in, not a device address).
constexpr size_t kNoAllocScratchBytes = size_t(80) << 20;
__device__ __align__(256) static uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, looked up once per device.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(ATTNQ_ELAUNCH, "no usable current device for the library scratch (device %d)", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(ATTNQ_ELAUNCH, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ATTNQ_OK;
}

// The host checks of the paged decode, shared by both of its entry points
// (everything but the workspace).
int decode_check(const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
                 const float* v_scale, const int32_t* kv_indptr, const int32_t* kv_indices,
                 const int32_t* kv_last_page_len, int batch, int num_pages, int page_size, int num_q_heads,
                 int num_kv_heads, int head_dim, int max_kv_len, float sm_scale, void* o, float* lse) {
  REQUIRE(head_dim == 64 || head_dim == 128, ATTNQ_EUNSUPPORTED, "head_dim must be 64 or 128 (got %d)", head_dim);
  REQUIRE(num_q_heads > 0 && num_kv_heads > 0 && num_q_heads % num_kv_heads == 0, ATTNQ_EINVAL,
          "num_q_heads must be a positive multiple of num_kv_heads");
  REQUIRE(num_q_heads / num_kv_heads <= 16, ATTNQ_EUNSUPPORTED, "at most 16 q heads per kv head");
  REQUIRE(page_size >= 16 && page_size <= 1024 && page_size % 16 == 0, ATTNQ_EINVAL,
          "page_size must be a multiple of 16 in [16, 1024] (got %d)", page_size);
  REQUIRE(batch >= 0 && max_kv_len >= 0, ATTNQ_EINVAL, "batch and max_kv_len must be >= 0");
  REQUIRE(batch <= 65535, ATTNQ_EUNSUPPORTED, "batch must be <= 65535");
  REQUIRE(num_pages > 0, ATTNQ_EINVAL, "num_pages must be positive");
  REQUIRE(scale_ok(sm_scale), ATTNQ_EINVAL, "sm_scale must be finite (or NaN for 1/sqrt(head_dim))");
  if (batch == 0) return ok();
  REQUIRE_PTR(q, 16);
  REQUIRE_PTR(k_cache, 16);
  REQUIRE_PTR(v_cache, 16);
  REQUIRE_PTR(k_scale, 4);
  REQUIRE_PTR(v_scale, 4);
  REQUIRE_PTR(kv_indptr, 4);
  REQUIRE_PTR(kv_indices, 4);
  REQUIRE_PTR(kv_last_page_len, 4);
  REQUIRE_PTR(o, 16);
  REQUIRE_OPT_PTR(lse, 4);
  return ok();
}

}  // namespace

extern "C" {

int attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                      const float* k_scale, const float* v_scale, const int32_t* kv_indptr,
                      const int32_t* kv_indices, const int32_t* kv_last_page_len, int batch,
                      int num_pages, int page_size, int num_q_heads, int num_kv_heads,
                      int head_dim, int max_kv_len, float sm_scale, void* workspace,
                      size_t workspace_bytes, void* o, float* lse, hipStream_t stream) {
  const int st = decode_check(q, k_cache, v_cache, k_scale, v_scale, kv_indptr, kv_indices, kv_last_page_len, batch,
                              num_pages, page_size, num_q_heads, num_kv_heads, head_dim, max_kv_len, sm_scale, o, lse);
  if (st != ATTNQ_OK || batch == 0) return st;
  sm_scale = scale_or_default(sm_scale, head_dim);
  REQUIRE_PTR(workspace, 256);
  const size_t need = attn_decode_paged_workspace_size(batch, num_q_heads, head_dim, max_kv_len, page_size);
  REQUIRE(workspace_bytes >= need, ATTNQ_EWORKSPACE, "workspace too small: %zu < %zu bytes",
          workspace_bytes, need);
  attnq::DecodeArgs a;
  a.q = q;
  a.k_cache = static_cast<const uint8_t*>(k_cache);
  a.v_cache = static_cast<const uint8_t*>(v_cache);
  a.k_scale = k_scale; a.v_scale = v_scale;
  a.kv_indptr = kv_indptr; a.kv_indices = kv_indices; a.kv_last = kv_last_page_len;
  a.o = o; a.lse = lse;
  a.batch = batch; a.num_pages = num_pages; a.page_size = page_size;
  a.hq = num_q_heads; a.hkv = num_kv_heads;
  a.n_chunks = attnq::decode_n_chunks(max_kv_len);
  a.chunk_pages = attnq::decode_chunk_pages(page_size);
  const size_t rows = (size_t)batch * num_q_heads * a.n_chunks;
  a.ws_o = static_cast<float*>(workspace);
  a.ws_lse = a.ws_o + rows * head_dim;
  a.sm_scale_log2 = sm_scale * LOG2E;
  LAUNCHED(attnq::launch_decode(a, head_dim, stream));
  return ok();
}

int attn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const float* k_scale, const float* v_scale, const int32_t* kv_indptr,
                              const int32_t* kv_indices, const int32_t* kv_last_page_len, int batch,
                              int num_pages, int page_size, int num_q_heads, int num_kv_heads,
                              int head_dim, int max_kv_len, float sm_scale, void* o, float* lse,
                              hipStream_t stream) {
  // arguments first: the scratch array is looked up only for a call that runs
  const int st = decode_check(q, k_cache, v_cache, k_scale, v_scale, kv_indptr, kv_indices, kv_last_page_len, batch,
                              num_pages, page_size, num_q_heads, num_kv_heads, head_dim, max_kv_len, sm_scale, o, lse);
  if (st != ATTNQ_OK || batch == 0) return st;
  // the partials need no clearing: the merge reads exactly the chunks the
  // split phase of this call writes
  const size_t need = attn_decode_paged_workspace_size(batch, num_q_heads, head_dim, max_kv_len, page_size);
  REQUIRE(need <= kNoAllocScratchBytes, ATTNQ_EWORKSPACE,
          "attn_decode_paged_noalloc: the split partials need %zu bytes, more than the library's fixed "
          "scratch of %zu bytes (use attn_decode_paged with a workspace)", need, kNoAllocScratchBytes);
  void* ws = nullptr;
  const int sst = scratch_address(&ws);
  if (sst != ATTNQ_OK) return sst;
  return attn_decode_paged(q, k_cache, v_cache, k_scale, v_scale, kv_indptr, kv_indices, kv_last_page_len,
                           batch, num_pages, page_size, num_q_heads, num_kv_heads, head_dim, max_kv_len,
                           sm_scale, ws, kNoAllocScratchBytes, o, lse, stream);
}

// ---------------------------------------------------------------- attn_sparse_mla_decode
static bool mla_sbs_ok(int sbs) { return sbs == 1 || sbs == 2 || sbs == 4 || sbs == 8 || sbs == 16; }

size_t attn_sparse_mla_decode_workspace_size(int batch, int s_q, int num_heads, int topk,
                                             int sparse_block_size) {
  if (batch <= 0 || s_q <= 0 || num_heads <= 0 || topk <= 0 || !mla_sbs_ok(sparse_block_size)) return 0;
  if ((long)topk * sparse_block_size > 0x7FFFFFFFL) return 0;
  return attnq::mla_workspace_bytes(batch, s_q, num_heads, topk * sparse_block_size);
}

int attn_sparse_mla_decode(const void* q, const void* kv_cache, int kv_dtype, const int32_t* block_table,
                           int max_blocks_per_seq, const int32_t* kv_lens,
                           const int32_t* sparse_indices, int topk, int sparse_block_size,
                           int sparse_mode, int batch, int s_q, int num_heads, int num_blocks,
                           int block_size, float sm_scale, void* workspace, size_t workspace_bytes,
                           void* o, float* lse, hipStream_t stream) {
  static const int kHeads[] = {1, 2, 4, 8, 16, 32, 48, 64, 128};
  bool heads_ok = false;
  for (int h : kHeads) heads_ok |= (h == num_heads);
  REQUIRE(heads_ok, ATTNQ_EUNSUPPORTED, "num_heads must be one of 1,2,4,8,16,32,48,64,128 (got %d)", num_heads);
  REQUIRE(topk > 0, ATTNQ_EINVAL, "topk must be > 0 (got %d)", topk);
  REQUIRE(kv_dtype == ATTNQ_INT8 || kv_dtype == ATTNQ_FP8E4M3, ATTNQ_EUNSUPPORTED,
          "kv_dtype must be INT8 or FP8E4M3 (got %d)", kv_dtype);
  REQUIRE(mla_sbs_ok(sparse_block_size), ATTNQ_EUNSUPPORTED,
          "sparse_block_size must be 1, 2, 4, 8 or 16 (got %d)", sparse_block_size);
  REQUIRE(sparse_mode == 0 || sparse_mode == 3, ATTNQ_EUNSUPPORTED, "sparse_mode must be 0 or 3 (got %d)",
          sparse_mode);
  REQUIRE((long)topk * sparse_block_size <= 0x7FFFFFFFL, ATTNQ_EINVAL, "topk * sparse_block_size too large");
  REQUIRE(block_size >= 16 && block_size <= 1024 && block_size % 16 == 0, ATTNQ_EINVAL,
          "block_size must be a multiple of 16 in [16, 1024] (got %d)", block_size);
  REQUIRE(batch >= 0 && s_q >= 0, ATTNQ_EINVAL, "batch and s_q must be >= 0");
  REQUIRE((long)batch * s_q <= 65535, ATTNQ_EUNSUPPORTED, "batch * s_q must be <= 65535");
  REQUIRE(num_blocks > 0 && max_blocks_per_seq > 0, ATTNQ_EINVAL, "num_blocks and max_blocks_per_seq must be positive");
  REQUIRE(scale_ok(sm_scale), ATTNQ_EINVAL, "sm_scale must be finite (or NaN for 1/sqrt(576))");
  sm_scale = scale_or_default(sm_scale, 576);  // d_k of K = [nope 512 | rope 64]
  if (batch == 0 || s_q == 0) return ok();
  REQUIRE_PTR(q, 16);
  REQUIRE_PTR(kv_cache, 16);
  REQUIRE_PTR(block_table, 4);
  REQUIRE_PTR(kv_lens, 4);
  REQUIRE_PTR(sparse_indices, 4);
  REQUIRE_PTR(o, 16);
  REQUIRE_OPT_PTR(lse, 4);
  REQUIRE_PTR(workspace, 256);
  const size_t need = attn_sparse_mla_decode_workspace_size(batch, s_q, num_heads, topk, sparse_block_size);
  REQUIRE(workspace_bytes >= need, ATTNQ_EWORKSPACE, "workspace too small: %zu < %zu bytes",
          workspace_bytes, need);
  attnq::MlaArgs a;
  a.q = q;
  a.cache = static_cast<const uint8_t*>(kv_cache);
  a.block_table = block_table; a.kv_lens = kv_lens; a.idx = sparse_indices;
  a.o = o; a.lse = lse;
  a.batch = batch; a.s_q = s_q; a.heads = num_heads; a.num_blocks = num_blocks;
  a.block_size = block_size; a.max_blocks = max_blocks_per_seq; a.topk = topk;
  a.n_split = attnq::mla_n_split(topk * sparse_block_size);
  const size_t rows = (size_t)batch * s_q * a.n_split * num_heads;
  a.ws_o = static_cast<uint16_t*>(workspace);
  a.ws_lse = reinterpret_cast<float*>(a.ws_o + rows * 512);
  a.sm_scale_log2 = sm_scale * LOG2E;
  const attnq::MlaMode m{kv_dtype == ATTNQ_FP8E4M3 ? 1 : 0, sparse_block_size, sparse_mode};
  LAUNCHED(attnq::launch_mla_mode(a, m, stream));
  return ok();
}

}  // extern "C"
