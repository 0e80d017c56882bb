// Gather of a paged KV cache into the ragged contiguous layout: the step that
// lets a prefill read the cache (FlashInfer's paged run mode, in which a
// prefill chunk attends to the tokens already held in pages).  Token i of
// sequence b lives in slot i % page_size of page kv_indices[kv_indptr[b] +
// i / page_size]; its whole row (all kv heads, one head_dim each) is copied to
// row cu_k[b] + i.  Rows past the sequence's cached length (when cu_k holds
// more rows for it) and rows whose page index is out of range are zero-filled.
#include "kcommon.h"
#include "gather.h"

namespace attnq {

constexpr int GATHER_THREADS = 256;
constexpr int GATHER_TOKENS = 16;  // tokens per workgroup

// One workgroup per (16-token block, sequence); each thread moves 16-byte
// pieces of the block's rows.
__global__ __launch_bounds__(GATHER_THREADS) void k_gather_paged(const GatherArgs a) {
  const int b = blockIdx.y;
  const int t0 = blockIdx.x * GATHER_TOKENS;
  const int dst0 = a.cu_k[b], n = a.cu_k[b + 1] - dst0;
  if (t0 >= n) return;
  const int p0 = a.kv_indptr[b], np = a.kv_indptr[b + 1] - p0;
  const int last = min(max(a.kv_last_page_len[b], 0), a.page_size);
  const int kv_len = np > 0 ? (np - 1) * a.page_size + last : 0;
  const int pieces = a.row_bytes / 16;
  const int ntok = min(GATHER_TOKENS, n - t0);
  for (int e = threadIdx.x; e < ntok * pieces; e += GATHER_THREADS) {
    const int i = t0 + e / pieces, c = e - (e / pieces) * pieces;
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (i < kv_len) {
      const int page = a.kv_indices[p0 + i / a.page_size];
      if (page >= 0 && page < a.num_pages)
        v = *reinterpret_cast<const u32x4*>(a.cache + ((long)page * a.page_size + i % a.page_size) * a.row_bytes + 16 * c);
    }
    *reinterpret_cast<u32x4*>(a.out + (long)(dst0 + i) * a.row_bytes + 16 * c) = v;
  }
}

bool launch_gather_paged(const GatherArgs& a, int max_seqlen_k, hipStream_t s) {
  if (a.batch <= 0 || max_seqlen_k <= 0) return true;
  const dim3 grid((max_seqlen_k + GATHER_TOKENS - 1) / GATHER_TOKENS, a.batch);
  hipLaunchKernelGGL(k_gather_paged, grid, dim3(GATHER_THREADS), 0, s, a);
  return hipGetLastError() == hipSuccess;
}

}  // namespace attnq
