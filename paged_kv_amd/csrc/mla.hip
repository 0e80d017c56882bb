// Sparse MLA-absorb decode (placeholder until the kernel lands).
#include "kcommon.h"
#include "launch.h"

namespace attnq {
size_t mla_workspace_bytes(int batch, int s_q, int heads, int topk) {
  (void)topk;
  return (size_t)batch * s_q * heads * 513 * sizeof(float) + 256;
}
int mla_n_split(int topk) { (void)topk; return 1; }
bool launch_mla(const MlaArgs& a, hipStream_t s) { (void)a; (void)s; return false; }
}  // namespace attnq
