// Launch interface of the paged-cache gather (gather.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attnq {

struct GatherArgs {
  const uint8_t* cache;        // [num_pages, page_size, row_bytes]
  const int32_t* kv_indptr;    // [batch + 1]
  const int32_t* kv_indices;   // [kv_indptr[batch]]
  const int32_t* kv_last_page_len;  // [batch]
  const int32_t* cu_k;         // [batch + 1], destination row offsets
  uint8_t* out;                // [cu_k[batch], row_bytes]
  int batch, num_pages, page_size, row_bytes;
};
bool launch_gather_paged(const GatherArgs& a, int max_seqlen_k, hipStream_t s);

}  // namespace attnq
