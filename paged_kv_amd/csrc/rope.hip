// RoPE (rotate-half) on the new Q/K of a varlen batch, in place, plus the
// write of rotated K and of V into a paged 16-bit cache (PaddleNLP "write kv
// cache BF16/FP16 with RoPE"; FlashInfer's paged_kv_indptr/indices layout).
// Optionally reduces the per-head max |value| of the stored Q, K, V so that
// the following per-head fp8 quantizers can skip their own reduction pass.
//
// The rotation is evaluated in fp32 with every product and every sum rounded
// on its own (no fused multiply-add), then rounded once to the 16-bit type.
#include "kcommon.h"
#include "launch.h"

#pragma clang fp contract(off)

namespace attnq {

constexpr int RP_THREADS = 256;
constexpr int RP_TOKENS = 2;       // tokens per workgroup (each walks its tokens one after another)
constexpr int RP_MAXK = 32;        // units per thread per token (<= 8192 units)
constexpr int RP_MAX_HEADS = 1024;
constexpr int RP_MAX_CU = 1024;    // cu_seqlens cached in LDS up to this many entries

__device__ __forceinline__ void rot4(const uint2& a, const uint2& b, const float* c, const float* s,
                                     bool is_bf16, uint2& ya, uint2& yb, float& m) {
#pragma clang fp contract(off)
  uint32_t wa[2] = {a.x, a.y}, wb[2] = {b.x, b.y};
  uint32_t oa[2], ob[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    uint32_t ra[2], rb[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      int i = 2 * p + e;
      float x1 = h16_to_f32((wa[p] >> (16 * e)) & 0xffffu, is_bf16);
      float x2 = h16_to_f32((wb[p] >> (16 * e)) & 0xffffu, is_bf16);
      float p1 = x1 * c[i];
      float p2 = x2 * s[i];
      float p3 = x2 * c[i];
      float p4 = x1 * s[i];
      float y1 = p1 - p2;
      float y2 = p3 + p4;
      ra[e] = f32_to_h16(y1, is_bf16);
      rb[e] = f32_to_h16(y2, is_bf16);
      m = fmaxf(m, fabsf(h16_to_f32(ra[e], is_bf16)));
      m = fmaxf(m, fabsf(h16_to_f32(rb[e], is_bf16)));
    }
    oa[p] = ra[0] | (ra[1] << 16);
    ob[p] = rb[0] | (rb[1] << 16);
  }
  ya = make_uint2(oa[0], oa[1]);
  yb = make_uint2(ob[0], ob[1]);
}

__device__ __forceinline__ float absmax4(const uint2& a, bool is_bf16, float m) {
  uint32_t w[2] = {a.x, a.y};
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    m = fmaxf(m, fabsf(h16_to_f32(w[p] & 0xffffu, is_bf16)));
    m = fmaxf(m, fabsf(h16_to_f32(w[p] >> 16, is_bf16)));
  }
  return m;
}

// Unit u of a token = (head, 4 consecutive rotation pairs).  head index space:
// [0, Hq) q heads, [Hq, Hq+Hkv) k heads, [Hq+Hkv, Hq+2Hkv) v heads.
__global__ __launch_bounds__(RP_THREADS) void k_append_rope(
    uint16_t* __restrict__ q, uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    int is_bf16, const int32_t* __restrict__ cu, const int32_t* __restrict__ before, int batch,
    int total_tokens, int hq, int hkv, int dim, const float* __restrict__ cs, int max_pos,
    uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache,
    const int32_t* __restrict__ kv_indptr, const int32_t* __restrict__ kv_indices, int num_pages,
    int page_size, uint32_t* __restrict__ amax_q, uint32_t* __restrict__ amax_k,
    uint32_t* __restrict__ amax_v) {
  __shared__ int32_t s_cu[RP_MAX_CU];
  __shared__ uint32_t s_max[RP_MAX_HEADS];
  const int heads = hq + 2 * hkv;
  const int half = dim / 2;
  const int upr = half / 4;             // units per head
  const int units = heads * upr;
  const bool cu_in_lds = batch + 1 <= RP_MAX_CU;
  if (cu_in_lds)
    for (int i = threadIdx.x; i <= batch; i += RP_THREADS) s_cu[i] = cu[i];
  for (int i = threadIdx.x; i < heads; i += RP_THREADS) s_max[i] = 0u;
  __syncthreads();
  const bool want_amax = amax_q != nullptr || amax_k != nullptr || amax_v != nullptr;
  float m[RP_MAXK];
#pragma unroll
  for (int j = 0; j < RP_MAXK; ++j) m[j] = 0.0f;

  const int tok0 = blockIdx.x * RP_TOKENS;
  for (int tt = 0; tt < RP_TOKENS; ++tt) {
    const int tok = tok0 + tt;
    if (tok >= total_tokens) break;
    // sequence of this token: last b with cu[b] <= tok
    int lo = 0, hi = batch - 1;
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      int c = cu_in_lds ? s_cu[mid] : cu[mid];
      if (c <= tok) lo = mid; else hi = mid - 1;
    }
    const int b = lo;
    const int start = cu_in_lds ? s_cu[b] : cu[b];
    const int pos = (before ? before[b] : 0) + (tok - start);
    const bool pos_ok = pos >= 0 && pos < max_pos;
    int page = -1;
    if (pos_ok) {
      const int pi = kv_indptr[b] + pos / page_size;
      if (pi >= kv_indptr[b] && pi < kv_indptr[b + 1]) {
        page = kv_indices[pi];
        if (page < 0 || page >= num_pages) page = -1;
      }
    }
    const int slot = pos_ok ? pos % page_size : 0;
#pragma unroll
    for (int j = 0; j < RP_MAXK; ++j) {
      const int u = threadIdx.x + j * RP_THREADS;
      if (u >= units) break;
      const int head = u / upr;
      const int i0 = (u % upr) * 4;
      if (head < hq + hkv) {
        if (!pos_ok) continue;
        const bool isq = head < hq;
        const int hh = isq ? head : head - hq;
        uint16_t* base = isq ? q + ((long)tok * hq + hh) * dim : k + ((long)tok * hkv + hh) * dim;
        const float4 c01 = *reinterpret_cast<const float4*>(cs + ((long)pos * half + i0) * 2);
        const float4 c23 = *reinterpret_cast<const float4*>(cs + ((long)pos * half + i0 + 2) * 2);
        const float c[4] = {c01.x, c01.z, c23.x, c23.z};
        const float s[4] = {c01.y, c01.w, c23.y, c23.w};
        uint2 a = *reinterpret_cast<const uint2*>(base + i0);
        uint2 bb = *reinterpret_cast<const uint2*>(base + i0 + half);
        uint2 ya, yb;
        rot4(a, bb, c, s, is_bf16, ya, yb, m[j]);
        *reinterpret_cast<uint2*>(base + i0) = ya;
        *reinterpret_cast<uint2*>(base + i0 + half) = yb;
        if (!isq && page >= 0) {
          uint16_t* dst = k_cache + (((long)page * page_size + slot) * hkv + hh) * dim;
          *reinterpret_cast<uint2*>(dst + i0) = ya;
          *reinterpret_cast<uint2*>(dst + i0 + half) = yb;
        }
      } else {
        const int hh = head - hq - hkv;
        const uint16_t* src = v + ((long)tok * hkv + hh) * dim;
        uint2 a = *reinterpret_cast<const uint2*>(src + i0);
        uint2 bb = *reinterpret_cast<const uint2*>(src + i0 + half);
        m[j] = absmax4(bb, is_bf16, absmax4(a, is_bf16, m[j]));
        if (page >= 0) {
          uint16_t* dst = v_cache + (((long)page * page_size + slot) * hkv + hh) * dim;
          *reinterpret_cast<uint2*>(dst + i0) = a;
          *reinterpret_cast<uint2*>(dst + i0 + half) = bb;
        }
      }
    }
  }
  if (!want_amax) return;
#pragma unroll
  for (int j = 0; j < RP_MAXK; ++j) {
    const int u = threadIdx.x + j * RP_THREADS;
    if (u < units) atomicMax(&s_max[u / upr], __float_as_uint(m[j]));
  }
  __syncthreads();
  for (int h = threadIdx.x; h < heads; h += RP_THREADS) {
    uint32_t val = s_max[h];
    uint32_t* dst = h < hq ? amax_q + h : (h < hq + hkv ? amax_k + (h - hq) : amax_v + (h - hq - hkv));
    bool have = h < hq ? amax_q != nullptr : (h < hq + hkv ? amax_k != nullptr : amax_v != nullptr);
    if (have && val) atomicMax(dst, val);
  }
}

bool launch_append_rope(void* q, void* k, const void* v, bool is_bf16, const int32_t* cu,
                        const int32_t* before, int batch, int total_tokens, int hq, int hkv,
                        int dim, const float* cs, int max_pos, void* k_cache, void* v_cache,
                        const int32_t* kv_indptr, const int32_t* kv_indices, int num_pages,
                        int page_size, float* amax_q, float* amax_k, float* amax_v,
                        hipStream_t s) {
  if (total_tokens <= 0) return true;
  int grid = (total_tokens + RP_TOKENS - 1) / RP_TOKENS;
  hipLaunchKernelGGL(k_append_rope, dim3(grid), dim3(RP_THREADS), 0, s,
                     static_cast<uint16_t*>(q), static_cast<uint16_t*>(k),
                     static_cast<const uint16_t*>(v), (int)is_bf16, cu, before, batch,
                     total_tokens, hq, hkv, dim, cs, max_pos, static_cast<uint16_t*>(k_cache),
                     static_cast<uint16_t*>(v_cache), kv_indptr, kv_indices, num_pages, page_size,
                     reinterpret_cast<uint32_t*>(amax_q), reinterpret_cast<uint32_t*>(amax_k),
                     reinterpret_cast<uint32_t*>(amax_v));
  return hipGetLastError() == hipSuccess;
}

bool rope_units_fit(int hq, int hkv, int dim) {
  int heads = hq + 2 * hkv;
  return heads <= RP_MAX_HEADS && heads * (dim / 8) <= RP_MAXK * RP_THREADS;
}

}  // namespace attnq
