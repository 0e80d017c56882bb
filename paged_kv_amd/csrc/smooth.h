// Launch interface of K smoothing before the int8 block quantization (quant.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attnq {

// mean [batch, heads, dim] fp32 (written), then int8 codes / block scales of
// x - mean, fp16 x only.
bool launch_smooth_quant_int8_block(const void* x, const int32_t* cu, int batch, int heads, int dim,
                                    int nblk, int total_tokens, void* codes, float* scales, float* mean,
                                    hipStream_t s);

}  // namespace attnq
