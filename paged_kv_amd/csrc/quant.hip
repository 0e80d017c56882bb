// Quantizers of the path: per-head fp8 (amax -> descale -> e4m3fn codes),
// per-128-token-block int8 (SageAttention style), and the transpose/permute
// of V into the token order read by the prefill kernel's PV operand.
//
// Sources: PaddleNLP "Sage Attention Support Varlen" (varlen quant qk and
// quant_transpose_permute v kernels); aiter "[Triton] FP8 with FA v3 API"
// (fp8 q/k/v with per-head descales).  Arithmetic: the codes are those of the
// correctly rounded fp32 quotient x / scale, so that they are bit-identical
// to a plain definition of the quantizer; the quotient is formed from one
// reciprocal per scale and a fused-multiply-add correction (quot_by_recip).
#include "kcommon.h"
#include "launch.h"
#include "smooth.h"

namespace attnq {

// ---------------------------------------------------------------- helpers
__global__ void k_fill_u32(uint32_t* p, int n, uint32_t v) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// Per-head max |x| of x [rows, heads, dim] (16-bit), accumulated as fp32 bit
// patterns with atomicMax (valid because the values are non-negative).
constexpr int AMAX_THREADS = 256;
constexpr int AMAX_ROWS_PER_BLOCK = 64;

// Rows of at most AMAX_THREADS * 8 chunks: every thread keeps fixed columns
// (so fixed heads) for all rows of the block -- NCOL columns c = t + 256k of
// each row, or, for rows narrower than the workgroup, column t % cpr of rows
// t / cpr, t / cpr + 256 / cpr, ... -- with one running max per column, the
// loads of 4 rows in flight at once, and one LDS atomic per column at the end.
template <int NCOL>
__global__ __launch_bounds__(AMAX_THREADS) void k_amax_per_head_cols(
    const uint16_t* __restrict__ x, int rows, int heads, int dim, int is_bf16,
    uint32_t* __restrict__ amax_bits) {
  __shared__ uint32_t s_max[1024];
  for (int i = threadIdx.x; i < heads; i += AMAX_THREADS) s_max[i] = 0u;
  __syncthreads();
  const int cpr = heads * dim / 8;  // 16-byte chunks per row
  const int row0 = blockIdx.x * AMAX_ROWS_PER_BLOCK;
  const int nrows = min(AMAX_ROWS_PER_BLOCK, rows - row0);
  const uint4* src = reinterpret_cast<const uint4*>(x) + (long)row0 * cpr;
  const int rstep = cpr >= AMAX_THREADS ? 1 : AMAX_THREADS / cpr;   // rows per pass
  const int rfirst = cpr >= AMAX_THREADS ? 0 : threadIdx.x / cpr;
  const int col0 = cpr >= AMAX_THREADS ? threadIdx.x : threadIdx.x % cpr;
  const bool live = rfirst < rstep;   // threads past the last whole row of a pass idle
  float m[NCOL];
#pragma unroll
  for (int k = 0; k < NCOL; ++k) m[k] = 0.0f;
  for (int r = rfirst; live && r < nrows; r += 4 * rstep) {
    uint4 v[4][NCOL];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int k = 0; k < NCOL; ++k) {
        const int rr = r + u * rstep, c = col0 + k * AMAX_THREADS;
        v[u][k] = rr < nrows && c < cpr ? src[(long)rr * cpr + c] : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int k = 0; k < NCOL; ++k) {
        const uint32_t w[4] = {v[u][k].x, v[u][k].y, v[u][k].z, v[u][k].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          m[k] = fmaxf(m[k], fabsf(h16_to_f32(w[e] & 0xffffu, is_bf16)));
          m[k] = fmaxf(m[k], fabsf(h16_to_f32(w[e] >> 16, is_bf16)));
        }
      }
  }
#pragma unroll
  for (int k = 0; k < NCOL; ++k) {
    const int c = col0 + k * AMAX_THREADS;
    if (live && c < cpr && m[k] != 0.0f) atomicMax(&s_max[c * 8 / dim], __float_as_uint(m[k]));
  }
  __syncthreads();
  for (int i = threadIdx.x; i < heads; i += AMAX_THREADS)
    if (s_max[i]) atomicMax(&amax_bits[i], s_max[i]);
}

// Any row width: a thread walks the block's chunks with a stride of the
// workgroup size, folding its max into LDS whenever the head changes.
__global__ __launch_bounds__(AMAX_THREADS) void k_amax_per_head(
    const uint16_t* __restrict__ x, int rows, int heads, int dim, int is_bf16,
    uint32_t* __restrict__ amax_bits) {
  __shared__ uint32_t s_max[1024];
  for (int i = threadIdx.x; i < heads; i += AMAX_THREADS) s_max[i] = 0u;
  __syncthreads();
  const int cpr = heads * dim / 8;  // 16-byte chunks per row
  const int row0 = blockIdx.x * AMAX_ROWS_PER_BLOCK;
  const int nrows = min(AMAX_ROWS_PER_BLOCK, rows - row0);
  const long n = (long)nrows * cpr;
  const uint4* src = reinterpret_cast<const uint4*>(x) + (long)row0 * cpr;
  float m = 0.0f;
  int cur = -1;
  for (long i = threadIdx.x; i < n; i += AMAX_THREADS) {
    int h = (int)(i % cpr) * 8 / dim;
    if (h != cur) {
      if (cur >= 0) atomicMax(&s_max[cur], __float_as_uint(m));
      cur = h;
      m = 0.0f;
    }
    uint4 v = src[i];
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      m = fmaxf(m, fabsf(h16_to_f32(w[e] & 0xffffu, is_bf16)));
      m = fmaxf(m, fabsf(h16_to_f32(w[e] >> 16, is_bf16)));
    }
  }
  if (cur >= 0) atomicMax(&s_max[cur], __float_as_uint(m));
  __syncthreads();
  for (int i = threadIdx.x; i < heads; i += AMAX_THREADS)
    if (s_max[i]) atomicMax(&amax_bits[i], s_max[i]);
}

// scale[h] = amax[h] / qmax (IEEE division), 1 where amax == 0.  `amax_in`
// (fp32 values) overrides the in-place accumulated bits when given.
__global__ void k_finalize_scale(const float* __restrict__ amax_in, float* scales, int heads,
                                 float qmax) {
  int h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h >= heads) return;
  float a = amax_in ? amax_in[h] : __uint_as_float(reinterpret_cast<uint32_t*>(scales)[h]);
  scales[h] = (a == 0.0f) ? 1.0f : a / qmax;
}

// codes = e4m3fn(x / descale[head]).  x is [rows, heads, dim]; a thread owns
// one 16-byte chunk column of the row (so one head, one descale and its
// reciprocal) for FP8_ROWS consecutive rows, whose loads are all in flight
// before the first is encoded.
constexpr int FP8_THREADS = 256;
constexpr int FP8_ROWS = 8;   // measured: 8 beats 16 (-6%) and 32

template <bool BF16, int CPRH>
__global__ __launch_bounds__(FP8_THREADS) void k_quant_fp8(const uint16_t* __restrict__ x, int rows, int heads,
                                                           const float* __restrict__ descale,
                                                           uint8_t* __restrict__ codes) {
  const int cr = heads * CPRH;  // 16-byte chunks per row
  const int cc = blockIdx.y * FP8_THREADS + threadIdx.x;
  if (cc >= cr) return;
  const float d = descale[cc / CPRH];
  const float r = 1.0f / d;
  const int r0 = blockIdx.x * FP8_ROWS;
  const int nr = min(FP8_ROWS, rows - r0);
  const u32x4* src = reinterpret_cast<const u32x4*>(x) + (long)r0 * cr + cc;
  u32x4 v[FP8_ROWS];
#pragma unroll
  for (int k = 0; k < FP8_ROWS; ++k) v[k] = src[(long)min(k, nr - 1) * cr];
  u32x2* dst = reinterpret_cast<u32x2*>(codes) + (long)r0 * cr + cc;
#pragma unroll
  for (int k = 0; k < FP8_ROWS; ++k) {
    if (k >= nr) continue;
    uint32_t c[8];
    if (d >= QUOT_MIN_SCALE) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        c[e] = e4m3fn_encode(quot_by_recip(h16_to_f32(e & 1 ? v[k][e >> 1] >> 16 : v[k][e >> 1] & 0xffffu, BF16), d, r));
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        c[e] = e4m3fn_encode(h16_to_f32(e & 1 ? v[k][e >> 1] >> 16 : v[k][e >> 1] & 0xffffu, BF16) / d);
    }
    dst[(long)k * cr] = u32x2{c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24),
                              c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24)};
  }
}

// ---------------------------------------------------------------- int8 per block
// One workgroup per (block j, head h, sequence b): the block's rows (at most
// 128) are loaded into registers in one go (rows past the sequence end
// re-read its last row and are left out of the max), reduced to amax, then
// encoded.
constexpr int I8_THREADS = 256;
constexpr int I8_BLOCK = 128;

// SMOOTH: the values quantized are x - mean[b][h][channel] (fp32, rounded
// once), the sequence's per-channel mean of K written by k_channel_mean.
// The work of one workgroup (block j, head h, sequence b).
template <bool BF16, int DIM, bool SMOOTH>
__device__ __forceinline__ void quant_int8_block_wg(
    int j, int h, int b, const uint16_t* __restrict__ x, const int32_t* __restrict__ cu, int heads,
    int nblk, int total_tokens, int8_t* __restrict__ codes, float* __restrict__ scales,
    const float* __restrict__ mean) {
  constexpr int CPR = DIM / 8;                          // 16-byte chunks per row
  constexpr int NCH = I8_BLOCK * CPR / I8_THREADS;      // chunks per thread
  const int s0 = clampi(cu[b], 0, total_tokens), s1 = clampi(cu[b + 1], s0, total_tokens);
  const int r0 = s0 + j * I8_BLOCK;
  float* sc_out = scales + ((long)b * heads + h) * nblk + j;
  if (r0 >= s1) {
    if (threadIdx.x == 0) *sc_out = 0.0f;
    return;
  }
  const int nrows = min(I8_BLOCK, s1 - r0);
  u32x4 v[NCH];
#pragma unroll
  for (int k = 0; k < NCH; ++k) {
    const int c = threadIdx.x + k * I8_THREADS;
    const int row = min(c / CPR, nrows - 1), col = (c % CPR) * 8;
    v[k] = *reinterpret_cast<const u32x4*>(x + ((long)(r0 + row) * heads + h) * DIM + col);
  }
  // this thread's channels' means (the same 8 channels for every chunk of a row)
  float mu[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if constexpr (SMOOTH) {
    static_assert(I8_THREADS % CPR == 0, "a thread keeps its channel column");
    const float* mp = mean + ((long)b * heads + h) * DIM + (threadIdx.x % CPR) * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) mu[e] = mp[e];
  }
  auto val = [&](int k, int e) -> float {
    const float xv = h16_to_f32(e & 1 ? v[k][e >> 1] >> 16 : v[k][e >> 1] & 0xffffu, BF16);
    if constexpr (SMOOTH) return xv - mu[e];
    else return xv;
  };
  float m = 0.0f;
#pragma unroll
  for (int k = 0; k < NCH; ++k) {
    if ((threadIdx.x + k * I8_THREADS) / CPR < nrows) {
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(val(k, e)));
    }
  }
  __shared__ float s_red[I8_THREADS / 64];
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = m;
  __syncthreads();
  float amax = s_red[0];
#pragma unroll
  for (int w = 1; w < I8_THREADS / 64; ++w) amax = fmaxf(amax, s_red[w]);
  const float scale = (amax == 0.0f) ? 1.0f : amax / 127.0f;
  if (threadIdx.x == 0) *sc_out = scale;
  const float rs = 1.0f / scale;
  auto encode_all = [&](auto fast_c) {
    constexpr bool FAST = decltype(fast_c)::value;
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int c = threadIdx.x + k * I8_THREADS;
      const int row = c / CPR, col = (c % CPR) * 8;
      if (row < nrows) {
        uint32_t q[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float xv = val(k, e);
          q[e] = (uint32_t)int8_encode(FAST ? quot_by_recip_i8(xv, scale, rs) : xv / scale) & 0xffu;
        }
        *reinterpret_cast<u32x2*>(codes + ((long)(r0 + row) * heads + h) * DIM + col) =
            u32x2{q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24), q[4] | (q[5] << 8) | (q[6] << 16) | (q[7] << 24)};
      }
    }
  };
  if (scale >= QUOT_MIN_SCALE) encode_all(std::true_type{});  // uniform
  else encode_all(std::false_type{});
}

template <bool BF16, int DIM, bool SMOOTH = false>
__global__ __launch_bounds__(I8_THREADS) void k_quant_int8_block(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ cu, int heads, int nblk,
    int total_tokens, int8_t* __restrict__ codes, float* __restrict__ scales,
    const float* __restrict__ mean = nullptr) {
  quant_int8_block_wg<BF16, DIM, SMOOTH>(blockIdx.x, blockIdx.y, blockIdx.z, x, cu, heads, nblk, total_tokens,
                                         codes, scales, mean);
}

// ---------------------------------------------------------------- per-channel mean of K
// mean[b][h][c] of fp16 x over the tokens of sequence b: the exact sum S of
// the values, then fp32(fp64(S) / fp64(L)) * 2^-24 with S in units of 2^-24;
// 0 for an empty sequence.  Every fp16 value is an integer number of 2^-24
// units below 2^40, so a thread's fp64 partial sum of at most MEAN_FLUSH of
// them stays below 2^53 units and is exact; partials are then added as int64
// (order-free).  MEAN_SPLIT workgroups per (head, sequence), each owning a
// contiguous share of the channels; thread (row group, 16-byte channel
// chunk); finite inputs.
constexpr int MEAN_THREADS = 1024;
constexpr int MEAN_FLUSH = 8192;  // a multiple of MEAN_BATCH
constexpr int MEAN_BATCH = 8;
constexpr int MEAN_SPLIT = 2;     // workgroups per (head, sequence), by channel

template <int DIM>
__global__ __launch_bounds__(MEAN_THREADS) void k_channel_mean(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ cu, int heads, int total_tokens,
    float* __restrict__ mean) {
  constexpr int CPR = DIM / 8 / MEAN_SPLIT, G = MEAN_THREADS / CPR;  // this workgroup's chunks per row, row groups
  static_assert(CPR >= 1 && 64 % CPR == 0, "a wave holds whole rows of chunk columns");
  const int h = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = blockIdx.z * CPR + threadIdx.x % CPR, g = threadIdx.x / CPR;
  const int s0 = clampi(cu[b], 0, total_tokens), s1 = clampi(cu[b + 1], s0, total_tokens);
  long long acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (long c0 = s0 + g; c0 < s1; c0 += (long)G * MEAN_FLUSH) {
    const long cend = min((long)s1, c0 + (long)G * MEAN_FLUSH);
    double part[8] = {0., 0., 0., 0., 0., 0., 0., 0.};
    // MEAN_BATCH rows per thread in flight before they are added
    for (long t = c0; t < cend; t += (long)G * MEAN_BATCH) {
      u32x4 v[MEAN_BATCH];
#pragma unroll
      for (int u = 0; u < MEAN_BATCH; ++u) {
        const long tu = t + (long)u * G;
        v[u] = tu < cend ? *reinterpret_cast<const u32x4*>(x + (tu * heads + h) * DIM + col * 8)
                         : u32x4{0u, 0u, 0u, 0u};  // +0 adds nothing
      }
#pragma unroll
      for (int u = 0; u < MEAN_BATCH; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          part[e] += (double)f16_to_f32(e & 1 ? v[u][e >> 1] >> 16 : v[u][e >> 1] & 0xffffu);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += (long long)(part[e] * 16777216.0);  // exact
  }
  // lanes lane, lane ^ CPR, lane ^ 2 CPR, ... of a wave hold the same channels
#pragma unroll
  for (int e = 0; e < 8; ++e)
    for (int off = CPR; off < 64; off <<= 1) acc[e] += __shfl_xor(acc[e], off, 64);
  __shared__ long long s_acc[MEAN_THREADS / 64][DIM];
  if (lane < CPR) {
#pragma unroll
    for (int e = 0; e < 8; ++e) s_acc[wave][col * 8 + e] = acc[e];
  }
  __syncthreads();
  for (int c = blockIdx.z * (DIM / MEAN_SPLIT) + threadIdx.x; c < (blockIdx.z + 1) * (DIM / MEAN_SPLIT);
       c += MEAN_THREADS) {
    long long tot = 0;
    for (int w = 0; w < MEAN_THREADS / 64; ++w) tot += s_acc[w][c];
    const int L = s1 - s0;
    const float m = L > 0 ? (float)((double)tot / (double)L) * 5.9604644775390625e-08f : 0.0f;  // * 2^-24
    mean[((long)b * heads + h) * DIM + c] = m;
  }
}

// ---------------------------------------------------------------- per-channel amax
// max |x| per (sequence, head, channel) as fp32 bit patterns (order-free: a
// non-negative float compares like its bits), folded into amax_bits
// [batch, heads, dim] with atomic max.  One workgroup per (CA_TOK tokens,
// head, sequence); thread (row group, 16-byte channel chunk).
constexpr int CA_THREADS = 256;
constexpr int CA_TOK = 256;

template <bool BF16, int DIM>
__global__ __launch_bounds__(CA_THREADS) void k_channel_amax(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ cu, int heads, int total_tokens,
    uint32_t* __restrict__ amax_bits) {
  constexpr int CPR = DIM / 8, G = CA_THREADS / CPR;
  const int h = blockIdx.y, b = blockIdx.z;
  const int s0 = clampi(cu[b], 0, total_tokens), s1 = clampi(cu[b + 1], s0, total_tokens);
  const int t0 = s0 + blockIdx.x * CA_TOK;
  if (t0 >= s1) return;
  const int t1 = min(t0 + CA_TOK, s1);
  const int col = threadIdx.x % CPR, g = threadIdx.x / CPR;
  uint32_t m[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll 4
  for (int t = t0 + g; t < t1; t += G) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(x + ((long)t * heads + h) * DIM + col * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float f = h16_to_f32(e & 1 ? v[e >> 1] >> 16 : v[e >> 1] & 0xffffu, BF16);
      m[e] = max(m[e], __float_as_uint(f) & 0x7fffffffu);
    }
  }
  __shared__ uint32_t s_m[G][DIM];
#pragma unroll
  for (int e = 0; e < 8; ++e) s_m[g][col * 8 + e] = m[e];
  __syncthreads();
  for (int c = threadIdx.x; c < DIM; c += CA_THREADS) {
    uint32_t r = s_m[0][c];
    for (int k = 1; k < G; ++k) r = max(r, s_m[k][c]);
    if (r) atomicMax(amax_bits + ((long)b * heads + h) * DIM + c, r);
  }
}

// ---------------------------------------------------------------- V transpose / permute
// V [T, H, D] -> V^T [B, H, D, S_pad].  One workgroup per (64-token tile,
// head, sequence).  Inside each 32-token group, stored position 8g + s holds
// token (s/4)*16 + 4g + s%4: lane group g of the PV operand then reads its 8
// tokens as one contiguous 8-element vector.
constexpr int VP_THREADS = 256;
constexpr int VP_TILE = 64;

// The work of one workgroup (64-token tile, head h, sequence b).
__device__ __forceinline__ void v_permute_wg(
    int tile, int h, int b, const uint16_t* __restrict__ v, const int32_t* __restrict__ cu, int heads,
    int dim, int s_pad, int is_bf16, int total_tokens, int fp8, int wide, const float* __restrict__ descale,
    void* __restrict__ out, int chan) {
  __shared__ uint16_t s_t[128][VP_TILE + 2];  // [d][token], padded rows
  const int t0 = tile * VP_TILE;
  const int s0 = clampi(cu[b], 0, total_tokens), s1 = clampi(cu[b + 1], s0, total_tokens);
  const int L = s1 - s0;
  const int cpr = dim / 8;
  for (int c = threadIdx.x; c < VP_TILE * cpr; c += VP_THREADS) {
    int tok = c / cpr, col = (c % cpr) * 8;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (t0 + tok < L)
      val = *reinterpret_cast<const uint4*>(v + ((long)(s0 + t0 + tok) * heads + h) * dim + col);
    uint32_t w[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s_t[col + 2 * e][tok] = (uint16_t)(w[e] & 0xffffu);
      s_t[col + 2 * e + 1][tok] = (uint16_t)(w[e] >> 16);
    }
  }
  __syncthreads();
  // chan: one descale per (sequence, head, channel), descale[b][h][d]
  const float ds_h = fp8 && !chan ? descale[h] : 1.0f;
  const float rds_h = 1.0f / ds_h;
  const long row_base = ((long)b * heads + h) * dim;
  for (int it = threadIdx.x; it < dim * (VP_TILE / 8); it += VP_THREADS) {
    int d = it / (VP_TILE / 8), p0 = (it % (VP_TILE / 8)) * 8;
    const float ds = chan ? descale[row_base + d] : ds_h;
    const float rds = chan ? 1.0f / ds : rds_h;
    const bool fast = ds >= QUOT_MIN_SCALE;
    int grp = p0 / 32, g = (p0 % 32) / 8;
    uint32_t e16[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) e16[s] = s_t[d][grp * 32 + (s / 4) * 16 + 4 * g + (s % 4)];
    long o = (row_base + d) * s_pad + t0 + p0;
    if (fp8) {
      uint32_t c[8];
      if (fast) {
#pragma unroll
        for (int s = 0; s < 8; ++s) c[s] = e4m3fn_encode(quot_by_recip(h16_to_f32(e16[s], is_bf16), ds, rds));
      } else {
#pragma unroll
        for (int s = 0; s < 8; ++s) c[s] = e4m3fn_encode(h16_to_f32(e16[s], is_bf16) / ds);
      }
      const uint32_t w0 = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
      const uint32_t w1 = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
      if (wide) {  // each code's value in fp16 (exact)
        u32x4 h;
        h[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false));
        h[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true));
        h[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false));
        h[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true));
        *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + o) = h;
      } else {
        *reinterpret_cast<uint2*>(static_cast<uint8_t*>(out) + o) = make_uint2(w0, w1);
      }
    } else {
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + o) =
          make_uint4(e16[0] | (e16[1] << 16), e16[2] | (e16[3] << 16), e16[4] | (e16[5] << 16),
                     e16[6] | (e16[7] << 16));
    }
  }
}

__global__ __launch_bounds__(VP_THREADS) void k_v_permute(
    const uint16_t* __restrict__ v, const int32_t* __restrict__ cu, int heads, int dim,
    int s_pad, int is_bf16, int total_tokens, int fp8, int wide, const float* __restrict__ descale,
    void* __restrict__ out, int chan = 0) {
  v_permute_wg(blockIdx.x, blockIdx.y, blockIdx.z, v, cu, heads, dim, s_pad, is_bf16, total_tokens, fp8, wide,
               descale, out, chan);
}

// ---------------------------------------------------------------- K int8 blocks + V^T in one launch
// The Sage flow's two input passes side by side: workgroups x < nblk quantize
// K block x (as k_quant_int8_block), the others permute V tile x - nblk (as
// k_v_permute with 16-bit V, no encoding).  Same outputs as the two launches.
static_assert(I8_THREADS == VP_THREADS, "one workgroup size for both bodies");

template <bool BF16, int DIM>
__global__ __launch_bounds__(I8_THREADS) void k_quant_k_permute_v(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, const int32_t* __restrict__ cu,
    int heads, int nblk, int s_pad, int total_tokens, int8_t* __restrict__ codes, float* __restrict__ scales,
    void* __restrict__ v_out) {
  if ((int)blockIdx.x < nblk)
    quant_int8_block_wg<BF16, DIM, false>(blockIdx.x, blockIdx.y, blockIdx.z, k, cu, heads, nblk, total_tokens,
                                          codes, scales, nullptr);
  else
    v_permute_wg(blockIdx.x - nblk, blockIdx.y, blockIdx.z, v, cu, heads, DIM, s_pad, BF16, total_tokens, 0, 0,
                 nullptr, v_out, 0);
}

// ---------------------------------------------------------------- launchers
static inline bool ok(hipError_t e) { return e == hipSuccess; }

bool launch_fill_u32(uint32_t* p, int n, uint32_t v, hipStream_t s) {
  if (n <= 0) return true;
  hipLaunchKernelGGL(k_fill_u32, dim3((n + 255) / 256), dim3(256), 0, s, p, n, v);
  return ok(hipGetLastError());
}

bool launch_amax(const void* x, int rows, int heads, int dim, bool is_bf16, uint32_t* amax_bits,
                 hipStream_t s) {
  if (rows <= 0) return true;
  int grid = (rows + AMAX_ROWS_PER_BLOCK - 1) / AMAX_ROWS_PER_BLOCK;
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  const int ncol = (heads * dim / 8 + AMAX_THREADS - 1) / AMAX_THREADS;
  if (ncol <= 1) hipLaunchKernelGGL(k_amax_per_head_cols<1>, dim3(grid), dim3(AMAX_THREADS), 0, s, xp, rows, heads, dim, (int)is_bf16, amax_bits);
  else if (ncol <= 2) hipLaunchKernelGGL(k_amax_per_head_cols<2>, dim3(grid), dim3(AMAX_THREADS), 0, s, xp, rows, heads, dim, (int)is_bf16, amax_bits);
  else if (ncol <= 4) hipLaunchKernelGGL(k_amax_per_head_cols<4>, dim3(grid), dim3(AMAX_THREADS), 0, s, xp, rows, heads, dim, (int)is_bf16, amax_bits);
  else if (ncol <= 8) hipLaunchKernelGGL(k_amax_per_head_cols<8>, dim3(grid), dim3(AMAX_THREADS), 0, s, xp, rows, heads, dim, (int)is_bf16, amax_bits);
  else hipLaunchKernelGGL(k_amax_per_head, dim3(grid), dim3(AMAX_THREADS), 0, s, xp, rows, heads, dim, (int)is_bf16, amax_bits);
  return ok(hipGetLastError());
}

bool launch_finalize_scale(const float* amax_in, float* scales, int heads, float qmax,
                           hipStream_t s) {
  hipLaunchKernelGGL(k_finalize_scale, dim3((heads + 255) / 256), dim3(256), 0, s, amax_in,
                     scales, heads, qmax);
  return ok(hipGetLastError());
}

bool launch_quant_fp8(const void* x, long elems, int heads, int dim, bool is_bf16,
                      const float* descale, void* codes, hipStream_t s) {
  const long rows = elems / ((long)heads * dim);
  if (rows <= 0) return true;
  const int cr = heads * dim / 8;
  const dim3 grid((unsigned)((rows + FP8_ROWS - 1) / FP8_ROWS), (unsigned)((cr + FP8_THREADS - 1) / FP8_THREADS));
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  uint8_t* cp = static_cast<uint8_t*>(codes);
  if (dim == 128) {
    if (is_bf16) hipLaunchKernelGGL((k_quant_fp8<true, 16>), grid, dim3(FP8_THREADS), 0, s, xp, (int)rows, heads, descale, cp);
    else hipLaunchKernelGGL((k_quant_fp8<false, 16>), grid, dim3(FP8_THREADS), 0, s, xp, (int)rows, heads, descale, cp);
  } else {
    if (is_bf16) hipLaunchKernelGGL((k_quant_fp8<true, 8>), grid, dim3(FP8_THREADS), 0, s, xp, (int)rows, heads, descale, cp);
    else hipLaunchKernelGGL((k_quant_fp8<false, 8>), grid, dim3(FP8_THREADS), 0, s, xp, (int)rows, heads, descale, cp);
  }
  return ok(hipGetLastError());
}

bool launch_quant_int8_block(const void* x, const int32_t* cu, int batch, int heads, int dim,
                             int block_tokens, int nblk, bool is_bf16, int total_tokens,
                             void* codes, float* scales, hipStream_t s) {
  if (batch <= 0 || nblk <= 0) return true;
  if (block_tokens != I8_BLOCK) return false;
  const dim3 grid(nblk, heads, batch);
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  int8_t* cp = static_cast<int8_t*>(codes);
  if (dim == 128) {
    if (is_bf16) hipLaunchKernelGGL((k_quant_int8_block<true, 128>), grid, dim3(I8_THREADS), 0, s, xp, cu, heads, nblk, total_tokens, cp, scales);
    else hipLaunchKernelGGL((k_quant_int8_block<false, 128>), grid, dim3(I8_THREADS), 0, s, xp, cu, heads, nblk, total_tokens, cp, scales);
  } else {
    if (is_bf16) hipLaunchKernelGGL((k_quant_int8_block<true, 64>), grid, dim3(I8_THREADS), 0, s, xp, cu, heads, nblk, total_tokens, cp, scales);
    else hipLaunchKernelGGL((k_quant_int8_block<false, 64>), grid, dim3(I8_THREADS), 0, s, xp, cu, heads, nblk, total_tokens, cp, scales);
  }
  return ok(hipGetLastError());
}

bool launch_v_permute(const void* v, const int32_t* cu, int batch, int heads, int dim, int s_pad,
                      bool is_bf16, int total_tokens, bool fp8, bool wide, const float* descale,
                      void* out, hipStream_t s) {
  if (batch <= 0 || s_pad <= 0) return true;
  hipLaunchKernelGGL(k_v_permute, dim3(s_pad / VP_TILE, heads, batch), dim3(VP_THREADS), 0, s,
                     static_cast<const uint16_t*>(v), cu, heads, dim, s_pad, (int)is_bf16,
                     total_tokens, (int)fp8, (int)wide, descale, out);
  return ok(hipGetLastError());
}

}  // namespace attnq

namespace attnq {

bool launch_smooth_quant_int8_block(const void* x, const int32_t* cu, int batch, int heads, int dim,
                                    int nblk, int total_tokens, void* codes, float* scales, float* mean,
                                    hipStream_t s) {
  if (batch <= 0) return true;
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  int8_t* cp = static_cast<int8_t*>(codes);
  if (dim == 128) hipLaunchKernelGGL((k_channel_mean<128>), dim3(heads, batch, MEAN_SPLIT), dim3(MEAN_THREADS), 0, s, xp, cu, heads, total_tokens, mean);
  else hipLaunchKernelGGL((k_channel_mean<64>), dim3(heads, batch, MEAN_SPLIT), dim3(MEAN_THREADS), 0, s, xp, cu, heads, total_tokens, mean);
  if (hipGetLastError() != hipSuccess) return false;
  if (nblk <= 0) return true;
  const dim3 grid(nblk, heads, batch);
  if (dim == 128) hipLaunchKernelGGL((k_quant_int8_block<false, 128, true>), grid, dim3(I8_THREADS), 0, s, xp, cu, heads, nblk, total_tokens, cp, scales, mean);
  else hipLaunchKernelGGL((k_quant_int8_block<false, 64, true>), grid, dim3(I8_THREADS), 0, s, xp, cu, heads, nblk, total_tokens, cp, scales, mean);
  return hipGetLastError() == hipSuccess;
}

bool launch_quant_k_permute_v(const void* k, const void* v, const int32_t* cu, int batch, int heads, int dim,
                              int nblk, int s_pad, bool is_bf16, int total_tokens, void* codes, float* scales,
                              void* v_out, hipStream_t s) {
  if (batch <= 0 || nblk <= 0) return true;
  const dim3 grid(nblk + s_pad / VP_TILE, heads, batch);
  const uint16_t* kp = static_cast<const uint16_t*>(k);
  const uint16_t* vp = static_cast<const uint16_t*>(v);
  int8_t* cp = static_cast<int8_t*>(codes);
  if (dim == 128) {
    if (is_bf16) hipLaunchKernelGGL((k_quant_k_permute_v<true, 128>), grid, dim3(I8_THREADS), 0, s, kp, vp, cu, heads, nblk, s_pad, total_tokens, cp, scales, v_out);
    else hipLaunchKernelGGL((k_quant_k_permute_v<false, 128>), grid, dim3(I8_THREADS), 0, s, kp, vp, cu, heads, nblk, s_pad, total_tokens, cp, scales, v_out);
  } else {
    if (is_bf16) hipLaunchKernelGGL((k_quant_k_permute_v<true, 64>), grid, dim3(I8_THREADS), 0, s, kp, vp, cu, heads, nblk, s_pad, total_tokens, cp, scales, v_out);
    else hipLaunchKernelGGL((k_quant_k_permute_v<false, 64>), grid, dim3(I8_THREADS), 0, s, kp, vp, cu, heads, nblk, s_pad, total_tokens, cp, scales, v_out);
  }
  return ok(hipGetLastError());
}

bool launch_v_permute_per_channel(const void* v, const int32_t* cu, int batch, int heads, int dim,
                                  int s_pad, bool is_bf16, int total_tokens, bool wide,
                                  float* descale, void* out, hipStream_t s) {
  if (batch <= 0) return true;
  const int n = batch * heads * dim;
  if (!launch_fill_u32(reinterpret_cast<uint32_t*>(descale), n, 0u, s)) return false;
  if (s_pad > 0 && total_tokens > 0) {
    const dim3 grid(s_pad / CA_TOK + (s_pad % CA_TOK != 0), heads, batch);
    const uint16_t* xp = static_cast<const uint16_t*>(v);
    uint32_t* ab = reinterpret_cast<uint32_t*>(descale);
    if (dim == 128) {
      if (is_bf16) hipLaunchKernelGGL((k_channel_amax<true, 128>), grid, dim3(CA_THREADS), 0, s, xp, cu, heads, total_tokens, ab);
      else hipLaunchKernelGGL((k_channel_amax<false, 128>), grid, dim3(CA_THREADS), 0, s, xp, cu, heads, total_tokens, ab);
    } else {
      if (is_bf16) hipLaunchKernelGGL((k_channel_amax<true, 64>), grid, dim3(CA_THREADS), 0, s, xp, cu, heads, total_tokens, ab);
      else hipLaunchKernelGGL((k_channel_amax<false, 64>), grid, dim3(CA_THREADS), 0, s, xp, cu, heads, total_tokens, ab);
    }
    if (!ok(hipGetLastError())) return false;
  }
  if (!launch_finalize_scale(nullptr, descale, n, 448.0f, s)) return false;
  if (s_pad <= 0) return true;
  hipLaunchKernelGGL(k_v_permute, dim3(s_pad / VP_TILE, heads, batch), dim3(VP_THREADS), 0, s,
                     static_cast<const uint16_t*>(v), cu, heads, dim, s_pad, (int)is_bf16,
                     total_tokens, 1, (int)wide, descale, out, 1);
  return ok(hipGetLastError());
}

}  // namespace attnq
