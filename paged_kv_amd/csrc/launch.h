// Internal launchers of libattnq: host functions that enqueue one kernel each.
// They assume validated arguments and return false if the launch failed.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attnq {

bool launch_fill_u32(uint32_t* p, int n, uint32_t v, hipStream_t s);
bool launch_amax(const void* x, int rows, int heads, int dim, bool is_bf16, uint32_t* amax_bits,
                 hipStream_t s);
bool launch_finalize_scale(const float* amax_in, float* scales, int heads, float qmax,
                           hipStream_t s);
bool launch_quant_fp8(const void* x, long elems, int heads, int dim, bool is_bf16,
                      const float* descale, void* codes, hipStream_t s);
bool launch_quant_int8_block(const void* x, const int32_t* cu, int batch, int heads, int dim,
                             int block_tokens, int nblk, bool is_bf16, int total_tokens,
                             void* codes, float* scales, hipStream_t s);
bool launch_v_permute(const void* v, const int32_t* cu, int batch, int heads, int dim, int s_pad,
                      bool is_bf16, int total_tokens, bool fp8, bool wide, const float* descale,
                      void* out, hipStream_t s);

bool rope_units_fit(int hq, int hkv, int dim);
bool launch_append_rope(void* q, void* k, const void* v, bool is_bf16, const int32_t* cu,
                        const int32_t* before, int batch, int total_tokens, int hq, int hkv,
                        int dim, const float* cs, int max_pos, void* k_cache, void* v_cache,
                        const int32_t* kv_indptr, const int32_t* kv_indices, int num_pages,
                        int page_size, float* amax_q, float* amax_k, float* amax_v,
                        hipStream_t s);

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;          // permuted V^T [B, Hkv, D, s_pad]
  const float* q_scale;
  const float* k_scale;
  const float* v_scale;   // [Hkv], or [B, Hkv, D] when v_chan
  const int32_t* cu_q;
  const int32_t* cu_k;
  void* o;
  float* lse;
  float* q_scale_out;     // 16-bit Q quantized in the kernel: block scales written here (nullable)
  int batch, hq, hkv, s_pad, nblk_q, nblk_k, total_q, total_k, causal, max_q, max_k;
  int tblk;               // query tiles per block of the workgroup order (set by launch_prefill)
  int v_chan;             // v_scale holds one descale per (sequence, kv head, channel)
  float sm_scale_log2;    // sm_scale * log2(e)
  // paged form: k and v are fp8 caches [num_pages, page_size, hkv, D], each
  // sequence's keys in the pages kv_indices[kv_indptr[b] .. kv_indptr[b+1])
  const int32_t* kv_indptr = nullptr;
  const int32_t* kv_indices = nullptr;
  const int32_t* kv_last = nullptr;
  int page_size = 0, num_pages = 0;
};
// Q/K forms of the prefill: fp8 codes with per-head descales (QK^T summed
// exactly: codes widened to fp16, f16 MFMA); the same with the fp8 MFMA
// (faster, its 128-product sums carry a relative error up to ~2^-11.8 of
// sum |q_d k_d|); int8 codes with per-block scales; or 16-bit Q (fp16 /
// bf16) that the kernel quantizes to int8 per 128-query block itself, with
// int8 per-block K
enum { PF_Q_FP8 = 0, PF_Q_I8 = 1, PF_Q_RAW_F16 = 2, PF_Q_RAW_BF16 = 3, PF_Q_FP8_MFMA8 = 4 };
// q_mode: one of PF_Q_*; v_fp8: fp8 V (else fp16 V)
bool launch_prefill(const PrefillArgs& a, int head_dim, int q_mode, bool v_fp8, bool o_bf16,
                    int max_seqlen_q, hipStream_t s);
// the same over fp8 K/V pages (PrefillArgs' paged fields; q_mode PF_Q_FP8 or
// PF_Q_FP8_MFMA8)
bool launch_prefill_paged(const PrefillArgs& a, int head_dim, int q_mode, bool o_bf16, int max_seqlen_q,
                          hipStream_t s);

struct DecodeArgs {
  const void* q;           // bf16 [B, Hq, D]
  const uint8_t* k_cache;  // fp8 [P, ps, Hkv, D]
  const uint8_t* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  const int32_t* kv_last;
  float* ws_o;             // [B, Hq, n_chunks, D]
  float* ws_lse;           // [B, Hq, n_chunks]
  void* o;
  float* lse;
  int batch, num_pages, page_size, hq, hkv, n_chunks, chunk_pages;
  float sm_scale_log2;
};
size_t decode_workspace_bytes(int batch, int hq, int head_dim, int max_kv_len, int page_size);
int decode_chunk_pages(int page_size);
int decode_n_chunks(int max_kv_len);
bool launch_decode(const DecodeArgs& a, int head_dim, hipStream_t s);  // head_dim 64 or 128

struct MlaArgs {
  const void* q;           // bf16 [B, Sq, H, 576]
  const uint8_t* cache;    // [NB, bs, 1, 656]
  const int32_t* block_table;
  const int32_t* kv_lens;
  const int32_t* idx;      // [B, Sq, 1, topk]
  uint16_t* ws_o;          // bf16 [B*Sq, n_split, H, 512]
  float* ws_lse;           // [B*Sq, n_split, H]
  void* o;
  float* lse;
  int batch, s_q, heads, num_blocks, block_size, max_blocks, topk, n_split;
  float sm_scale_log2;
};
size_t mla_workspace_bytes(int batch, int s_q, int heads, int topk);
int mla_n_split(int topk);
bool launch_mla(const MlaArgs& a, hipStream_t s);

}  // namespace attnq
