// Paged fp8 decode with split-KV and log-sum-exp merge (FlashInfer's batch
// decode over paged_kv_indptr / paged_kv_indices / paged_kv_last_page_len;
// aiter's paged fp8 flash_attn_with_kvcache with per-head descales).
//
// Split phase: one workgroup (4 waves) per (sequence, chunk of DEC_CHUNK_TOKENS
// cached tokens); wave w handles kv heads w, w+4, ...  For each pair of
// 16-token page blocks:
//   K rows (NHD, one 128-byte row per token and kv head) are read straight
//   into the A operand of S^T = K Q^T (bf16 16x16x32 MFMA, fp8 -> bf16 exact);
//   the q heads of the group are the 16 columns (unused columns are zero);
//   V is widened to fp16 and written transposed into a per-wave LDS tile in
//   the token order of the P^T operand, then O^T += V^T P^T (fp16 MFMA).
// Each chunk writes its normalized partial O and its log2-sum-exp to the
// caller's workspace; the merge kernel combines the chunks of a sequence.
#include "kcommon.h"
#include "launch.h"

namespace attnq {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int DEC_THREADS = 256;
constexpr int DEC_D = 128;
constexpr int DEC_CHUNK_TOKENS = 512;
constexpr int DEC_VROW = 32 * 2 + 16;  // bytes per LDS V^T row: 32 tokens fp16 + pad
constexpr float DEC_LN2 = 0.69314718055994530942f;

struct PairRegs {
  uint4 k[2][2];  // [block][half]: 32 fp8 K bytes of token n, d in [32g, 32g+32)
  uint4 v[2][2];  // same for V
};

__global__ __launch_bounds__(DEC_THREADS, 2) void k_decode_split(const DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_v[4][DEC_D * DEC_VROW];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int chunk = blockIdx.x, b = blockIdx.y;
  const int p0 = a.kv_indptr[b], p1 = a.kv_indptr[b + 1];
  const int npg = p1 - p0;
  const int ps = a.page_size;
  const int kv_len = npg > 0 ? (npg - 1) * ps + clampi(a.kv_last[b], 0, ps) : 0;
  const int t_begin = chunk * DEC_CHUNK_TOKENS;
  if (t_begin >= kv_len) return;
  const int t_end = min(kv_len, t_begin + DEC_CHUNK_TOKENS);
  const int nblk = (t_end - t_begin + 15) / 16;  // 16-token blocks in this chunk
  const int G = a.hq / a.hkv;
  uint8_t* sv = s_v[wave];

  for (int hk = wave; hk < a.hkv; hk += 4) {
    // Q^T operand: lane (n, g) holds q head hk*G + n, d in [32g + 8j, 32g + 8j + 8) for MFMA j
    v8bf qop[4];
    {
      const bool have = n < G;
      const uint16_t* qp = static_cast<const uint16_t*>(a.q) + ((long)b * a.hq + hk * G + n) * DEC_D + 32 * g;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint4 w = have ? *reinterpret_cast<const uint4*>(qp + 8 * j) : make_uint4(0, 0, 0, 0);
        qop[j] = __builtin_bit_cast(v8bf, w);
      }
    }
    const float kfold = a.sm_scale_log2 * a.k_scale[hk];
    const float vsc = a.v_scale[hk];
    v4f oacc[DEC_D / 16];
#pragma unroll
    for (int db = 0; db < DEC_D / 16; ++db) oacc[db] = v4f{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    auto load_pair = [&](int pair, PairRegs& r) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int t = t_begin + (2 * pair + j) * 16 + n;  // token of this lane
        r.k[j][0] = r.k[j][1] = r.v[j][0] = r.v[j][1] = make_uint4(0, 0, 0, 0);
        if (t < t_end) {
          int page = a.kv_indices[p0 + t / ps];
          page = clampi(page, 0, a.num_pages - 1);
          const long off = (((long)page * ps + t % ps) * a.hkv + hk) * DEC_D + 32 * g;
          r.k[j][0] = *reinterpret_cast<const uint4*>(a.k_cache + off);
          r.k[j][1] = *reinterpret_cast<const uint4*>(a.k_cache + off + 16);
          r.v[j][0] = *reinterpret_cast<const uint4*>(a.v_cache + off);
          r.v[j][1] = *reinterpret_cast<const uint4*>(a.v_cache + off + 16);
        }
      }
    };

    const int npairs = (nblk + 1) / 2;
    PairRegs cur, nxt;
    load_pair(0, cur);
    for (int pair = 0; pair < npairs; ++pair) {
      if (pair + 1 < npairs) load_pair(pair + 1, nxt);
      // ---- S^T = K Q^T for the two 16-token blocks
      float s[2][4];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
        uint32_t w[8] = {cur.k[j][0].x, cur.k[j][0].y, cur.k[j][0].z, cur.k[j][0].w,
                         cur.k[j][1].x, cur.k[j][1].y, cur.k[j][1].z, cur.k[j][1].w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          // 8 fp8 codes (2 dwords) -> 8 bf16
          v2bf c0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 * m], 1.0f, false);
          v2bf c1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 * m], 1.0f, true);
          v2bf c2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 * m + 1], 1.0f, false);
          v2bf c3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 * m + 1], 1.0f, true);
          v8bf kop = v8bf{c0[0], c0[1], c1[0], c1[1], c2[0], c2[1], c3[0], c3[1]};
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[m], acc, 0, 0, 0);
        }
        // lane (n, g) holds S^T[token 4g + r of block j][q head n]
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = t_begin + (2 * pair + j) * 16 + 4 * g + r;
          s[j][r] = t < t_end ? acc[r] * kfold : -INFINITY;
        }
      }
      // ---- V^T staging: token n of block j -> LDS column pos = 8*(n/4) + 4j + n%4
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int t = t_begin + (2 * pair + j) * 16 + n;
        const bool valid = t < t_end;
        const int col = 8 * (n / 4) + 4 * j + (n % 4);
        uint32_t w[8] = {cur.v[j][0].x, cur.v[j][0].y, cur.v[j][0].z, cur.v[j][0].w,
                         cur.v[j][1].x, cur.v[j][1].y, cur.v[j][1].z, cur.v[j][1].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          v2h lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(valid ? w[e] : 0u, 1.0f, false);
          v2h hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(valid ? w[e] : 0u, 1.0f, true);
          const int d0 = 32 * g + 4 * e;
          _Float16* base = reinterpret_cast<_Float16*>(sv + col * 2);
          base[(d0 + 0) * (DEC_VROW / 2)] = lo[0];
          base[(d0 + 1) * (DEC_VROW / 2)] = lo[1];
          base[(d0 + 2) * (DEC_VROW / 2)] = hi[0];
          base[(d0 + 3) * (DEC_VROW / 2)] = hi[1];
        }
      }
      // ---- online softmax over the 32 tokens of this pair
      float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                       fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      m_run = m_new;
      v8h pk;
      float rs = 0.f;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __builtin_amdgcn_exp2f(s[j][r] - m_use);
          rs += p;
          pk[4 * j + r] = (_Float16)p;
        }
      l_run = l_run * alpha + rs;
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int db = 0; db < DEC_D / 16; ++db) {
        oacc[db] *= alpha;
        const uint4 vv = *reinterpret_cast<const uint4*>(sv + (db * 16 + n) * DEC_VROW + 16 * g);
        oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, vv), pk, oacc[db], 0, 0, 0);
      }
      __builtin_amdgcn_wave_barrier();
      if (pair + 1 < npairs) cur = nxt;
    }
    // ---- partial results: O_c = O / l (times the V descale, fp8 -> fp16 was exact),
    //      lse_c = m + log2(l) in log2 units
    float l = l_run;
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (n < G) {
      const int qh = hk * G + n;
      const long row = ((long)b * a.hq + qh) * a.n_chunks + chunk;
      const float inv = l > 0.f ? vsc / l : 0.f;
#pragma unroll
      for (int db = 0; db < DEC_D / 16; ++db) {
        float4 o4 = make_float4(oacc[db][0] * inv, oacc[db][1] * inv, oacc[db][2] * inv, oacc[db][3] * inv);
        *reinterpret_cast<float4*>(a.ws_o + row * DEC_D + db * 16 + 4 * g) = o4;
      }
      if (g == 0) a.ws_lse[row] = l > 0.f ? m_run + __log2f(l) : -INFINITY;
    }
  }
}

// Merge: O = sum_c 2^(lse_c - lse) O_c, lse = log2 sum_c 2^lse_c.  One
// 32-lane group per (sequence, q head), four d values per lane.
constexpr int MERGE_THREADS = 128;

__global__ __launch_bounds__(MERGE_THREADS) void k_decode_merge(const DecodeArgs a) {
  const int row = blockIdx.x * (MERGE_THREADS / 32) + threadIdx.x / 32;  // b * hq + qh
  if (row >= a.batch * a.hq) return;
  const int b = row / a.hq;
  const int d0 = (threadIdx.x % 32) * 4;
  const int p0 = a.kv_indptr[b], p1 = a.kv_indptr[b + 1];
  const int npg = p1 - p0;
  const int kv_len = npg > 0 ? (npg - 1) * a.page_size + clampi(a.kv_last[b], 0, a.page_size) : 0;
  const int nc = min(a.n_chunks, (kv_len + DEC_CHUNK_TOKENS - 1) / DEC_CHUNK_TOKENS);
  const long row0 = (long)row * a.n_chunks;
  float m = -INFINITY;
  for (int c = 0; c < nc; ++c) m = fmaxf(m, a.ws_lse[row0 + c]);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  float tot = 0.f;
  if (m != -INFINITY) {
    for (int c = 0; c < nc; ++c) {
      const float lc = a.ws_lse[row0 + c];
      if (lc == -INFINITY) continue;
      const float w = __builtin_amdgcn_exp2f(lc - m);
      tot += w;
      const float4 o4 = *reinterpret_cast<const float4*>(a.ws_o + (row0 + c) * DEC_D + d0);
      acc[0] += w * o4.x; acc[1] += w * o4.y; acc[2] += w * o4.z; acc[3] += w * o4.w;
    }
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  uint32_t w0 = f32_to_bf16(acc[0] * inv) | (f32_to_bf16(acc[1] * inv) << 16);
  uint32_t w1 = f32_to_bf16(acc[2] * inv) | (f32_to_bf16(acc[3] * inv) << 16);
  *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.o) + (long)row * DEC_D + d0) = make_uint2(w0, w1);
  if (a.lse && d0 == 0) a.lse[row] = tot > 0.f ? (m + __log2f(tot)) * DEC_LN2 : -INFINITY;
}

int decode_chunk_pages(int page_size) { return DEC_CHUNK_TOKENS / page_size; }

static int n_chunks_for(int max_kv_len) {
  return max_kv_len > 0 ? (max_kv_len + DEC_CHUNK_TOKENS - 1) / DEC_CHUNK_TOKENS : 1;
}

size_t decode_workspace_bytes(int batch, int hq, int head_dim, int max_kv_len, int page_size) {
  (void)page_size;
  const size_t rows = (size_t)batch * hq * n_chunks_for(max_kv_len);
  return rows * head_dim * sizeof(float) + rows * sizeof(float) + 256;
}

bool launch_decode(const DecodeArgs& a, hipStream_t s) {
  if (a.batch <= 0) return true;
  hipLaunchKernelGGL(k_decode_split, dim3(a.n_chunks, a.batch), dim3(DEC_THREADS), 0, s, a);
  if (hipGetLastError() != hipSuccess) return false;
  const int rows = a.batch * a.hq;
  hipLaunchKernelGGL(k_decode_merge, dim3((rows + MERGE_THREADS / 32 - 1) / (MERGE_THREADS / 32)),
                     dim3(MERGE_THREADS), 0, s, a);
  return hipGetLastError() == hipSuccess;
}

int decode_n_chunks(int max_kv_len) { return n_chunks_for(max_kv_len); }

}  // namespace attnq
