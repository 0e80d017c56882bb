/* Drives the host validation layer of libattnq.so through every entry
 * point, built with AddressSanitizer and UndefinedBehaviorSanitizer on the
 * host side.  Every call here fails validation (or has nothing to do), so
 * no kernel is launched and no GPU is needed.  The device pointers are
 * fake aligned addresses that validation never dereferences.  Exits 0 when
 * every status is the expected one; the sanitizers abort on any finding. */
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "attnq.h"

#define FAKE ((void*)(uintptr_t)(1u << 20))
#define FAKE_OFF(n) ((void*)((uintptr_t)(1u << 20) + (n)))

static int failures = 0;

static void expect(int got, int want, const char* needle, const char* what) {
  const char* msg = attnq_last_error();
  if (got != want || (needle && (!msg || !strstr(msg, needle)))) {
    printf("FAIL %s: status %d (want %d), message '%s'\n", what, got, want, msg ? msg : "(null)");
    ++failures;
  }
}

int main(void) {
  const float inf = INFINITY, nan = NAN;
  if (attnq_abi_version() != ATTNQ_ABI_VERSION) { printf("FAIL abi version\n"); return 1; }

  /* quantizers */
  expect(attn_quant_qk(FAKE, ATTNQ_BF16, FAKE, 1, 10, 10, 2, 96, ATTNQ_Q_FP8_PER_HEAD, 128, NULL, FAKE, FAKE, 0),
         ATTNQ_EUNSUPPORTED, "head_dim", "quant_qk head_dim");
  expect(attn_quant_qk(FAKE_OFF(2), ATTNQ_BF16, FAKE, 1, 10, 10, 2, 64, ATTNQ_Q_FP8_PER_HEAD, 128, NULL, FAKE, FAKE, 0),
         ATTNQ_EINVAL, "aligned", "quant_qk alignment");
  expect(attn_quant_qk(FAKE, ATTNQ_FP16, NULL, 1, 10, 10, 2, 64, ATTNQ_Q_INT8_PER_BLOCK, 128, NULL, FAKE, FAKE, 0),
         ATTNQ_EINVAL, "cu_seqlens", "quant_qk cu_seqlens");
  expect(attn_quant_kv(FAKE, FAKE, ATTNQ_FP16, FAKE, 2, 300, 400, 8, 128, 64, FAKE, FAKE, FAKE, 0),
         ATTNQ_EUNSUPPORTED, "block_tokens", "quant_kv block_tokens");
  expect(attn_quant_v_permute(FAKE, ATTNQ_FP16, FAKE, 2, 100, 150, 8, 96, ATTNQ_Q_NONE, NULL, FAKE, NULL, 0),
         ATTNQ_EUNSUPPORTED, "head_dim", "v_permute head_dim");
  expect(attn_smooth_quant_k(FAKE, FAKE, 1, 10, 10, 2, 128, 128, FAKE, FAKE, NULL, 0), ATTNQ_EINVAL, "mean",
         "smooth mean");
  expect(attn_smooth_quant_k(NULL, NULL, 0, 10, 10, 2, 128, 128, NULL, NULL, NULL, 0), ATTNQ_OK, NULL,
         "smooth nothing to do");

  /* prefill (ragged) */
  expect(attn_prefill_varlen(FAKE, FAKE, FAKE, ATTNQ_FP8E4M3, ATTNQ_FP16, FAKE, FAKE, FAKE, ATTNQ_Q_FP8_PER_HEAD,
                             ATTNQ_Q_FP8_PER_HEAD, FAKE, FAKE, 2, 100, 100, 150, 150, 32, 8, 128, inf, 1, FAKE,
                             ATTNQ_BF16, NULL, 0),
         ATTNQ_EINVAL, "sm_scale", "prefill inf scale");
  expect(attn_prefill_varlen(FAKE, FAKE, FAKE, ATTNQ_FP8E4M3, ATTNQ_FP16, FAKE, FAKE, FAKE, ATTNQ_Q_FP8_PER_HEAD,
                             ATTNQ_Q_FP8_PER_HEAD, NULL, FAKE, 2, 100, 100, 150, 150, 32, 8, 128, nan, 1, FAKE,
                             ATTNQ_BF16, NULL, 0),
         ATTNQ_EINVAL, "cu_seqlens_q", "prefill default scale, then cu_seqlens_q");
  expect(attn_prefill_varlen(FAKE, FAKE, FAKE, ATTNQ_FP8E4M3, ATTNQ_FP16, FAKE, FAKE, FAKE, ATTNQ_Q_FP8_PER_HEAD,
                             ATTNQ_Q_FP8_PER_HEAD, FAKE, FAKE, 2, 100, 1 << 21, 150, 150, 8, 8, 128, 0.1f, 1, FAKE,
                             ATTNQ_BF16, NULL, 0),
         ATTNQ_EUNSUPPORTED, "2 GiB", "prefill 32-bit offsets");

  /* prefill over fp8 pages */
  expect(attn_prefill_paged(FAKE, FAKE, ATTNQ_Q_FP8_PER_HEAD, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 64,
                            8, 100, 1000, 150, 32, 8, 128, 0.1f, 1, FAKE, ATTNQ_BF16, NULL, 0),
         ATTNQ_EINVAL, "page_size", "prefill_paged page_size");
  expect(attn_prefill_paged(FAKE, FAKE, ATTNQ_Q_FP8_PER_HEAD, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2,
                            1 << 14, 1024, 100, 1000, 150, 32, 8, 128, 0.1f, 1, FAKE, ATTNQ_BF16, NULL, 0),
         ATTNQ_EUNSUPPORTED, "2 GiB", "prefill_paged cache size");
  expect(attn_prefill_paged(FAKE, FAKE, ATTNQ_Q_FP8_PER_HEAD, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, FAKE, 2, 64,
                            16, 100, 1000, 150, 32, 8, 128, 0.1f, 1, FAKE, ATTNQ_BF16, NULL, 0),
         ATTNQ_EINVAL, "kv_indices", "prefill_paged kv_indices");

  /* paged decode and its workspace */
  size_t need = attn_decode_paged_workspace_size(2, 32, 128, 100, 16);
  if (need == 0) { printf("FAIL decode workspace size\n"); ++failures; }
  expect(attn_decode_paged(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 10, 16, 32, 8, 128, 100, 0.1f, FAKE,
                           need - 1, FAKE, NULL, 0),
         ATTNQ_EWORKSPACE, "workspace", "decode workspace");
  expect(attn_decode_paged(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 10, 8, 32, 8, 128, 100, 0.1f, FAKE,
                           need, FAKE, NULL, 0),
         ATTNQ_EINVAL, "page_size", "decode page_size");
  expect(attn_decode_paged_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 10, 16, 32, 8, 96, 100, 0.1f,
                                   FAKE, NULL, 0),
         ATTNQ_EUNSUPPORTED, "head_dim", "decode_noalloc head_dim");

  /* gather */
  expect(attn_gather_paged_kv(FAKE, 4, FAKE, FAKE, FAKE, FAKE, 2, 100, 64, 16, 8, 128, FAKE, 0), ATTNQ_EINVAL,
         "elem_bytes", "gather elem_bytes");

  /* append + RoPE */
  expect(attn_append_kv_rope(FAKE, FAKE, FAKE, ATTNQ_BF16, FAKE, FAKE, 2, 10, 8, 8, 96, FAKE, 100, FAKE, FAKE, FAKE,
                             FAKE, 10, 16, NULL, NULL, NULL, 0),
         ATTNQ_EUNSUPPORTED, "head_dim", "append head_dim");

  /* sparse MLA */
  expect(attn_sparse_mla_decode(FAKE, FAKE, ATTNQ_INT8, FAKE, 4, FAKE, FAKE, 8, 3, 0, 1, 1, 16, 8, 64, 0.04f, FAKE,
                                (size_t)1 << 30, FAKE, NULL, 0),
         ATTNQ_EUNSUPPORTED, "sparse_block_size", "mla sparse_block_size");
  expect(attn_sparse_mla_decode(FAKE, FAKE, ATTNQ_INT8, FAKE, 4, FAKE, FAKE, 8, 1, 0, 0, 1, 16, 8, 64, nan, FAKE,
                                (size_t)1 << 30, FAKE, NULL, 0),
         ATTNQ_OK, NULL, "mla nothing to do");

  if (failures) { printf("%d failures\n", failures); return 1; }
  printf("abi_sanitize: all statuses as expected\n");
  return 0;
}
