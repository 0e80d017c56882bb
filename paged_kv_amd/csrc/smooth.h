// Launch interface of the Sage-flow quantizers beyond launch.h (quant.hip): K
// smoothing before the int8 block quantization, fp8 V with per-channel
// descales, and K int8 blocks with the V permute in one launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attnq {

// mean [batch, heads, dim] fp32 (written), then int8 codes / block scales of
// x - mean, fp16 x only.
bool launch_smooth_quant_int8_block(const void* x, const int32_t* cu, int batch, int heads, int dim,
                                    int nblk, int total_tokens, void* codes, float* scales, float* mean,
                                    hipStream_t s);

// descale [batch, heads, dim] fp32 (written: amax over the sequence's tokens
// / 448, 1 where amax = 0), then V^T as launch_v_permute's fp8 mode with the
// per-channel descales (wide: each code's fp16 value).
bool launch_v_permute_per_channel(const void* v, const int32_t* cu, int batch, int heads, int dim,
                                  int s_pad, bool is_bf16, int total_tokens, bool wide,
                                  float* descale, void* out, hipStream_t s);

// k int8 per 128-token block (codes, scales [batch, heads, nblk]) and v -> V^T
// [batch, heads, dim, s_pad] unchanged 16-bit values, in one launch.
bool launch_quant_k_permute_v(const void* k, const void* v, const int32_t* cu, int batch, int heads, int dim,
                              int nblk, int s_pad, bool is_bf16, int total_tokens, void* codes, float* scales,
                              void* v_out, hipStream_t s);

}  // namespace attnq
