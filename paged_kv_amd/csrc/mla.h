// Launch interface of the sparse MLA variants (mla.hip): the cache row's nope
// code type, block-wise sparse selection and the right-down causal mask.
#pragma once
#include "launch.h"

namespace attnq {

struct MlaMode {
  int kv_fp8;             // nope codes are fp8 e4m3fn (else int8)
  int sparse_block_size;  // an index names this many consecutive tokens (power of 2)
  int sparse_mode;        // 0: every selected token; 3: token <= kv_len - s_q + s for query row s
};
// a.topk is the number of index entries per query row; the kernels walk
// a.topk * m.sparse_block_size token slots (a.n_split = mla_n_split of that)
bool launch_mla_mode(const MlaArgs& a, const MlaMode& m, hipStream_t s);

}  // namespace attnq
