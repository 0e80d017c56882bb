// Varlen flash-attention prefill on quantized Q/K/V for gfx950.
//
// Computes O = softmax(sm_scale * Dequant(Q) Dequant(K)^T + causal mask) Dequant(V)
// (Ascend "KvQuantSparseFlashAttention" formula; FlashInfer's ragged batch
// prefill; aiter's fp8 flash_attn_func with q/k/v descales; PaddleNLP's Sage
// attention over a varlen batch with per-block int8 Q/K).
//
// Work split: one workgroup (4 waves) per (sequence, q head, 128-query tile);
// the grid's y index runs over query tiles from the end of the sequence
// (the tiles with the most visible keys start first).  Each wave owns 32
// queries and streams 64-key tiles staged in LDS (double-buffered).
//
// Per key tile and wave:
//   S^T = K Q^T          fp8 16x16x128 MFMA (or two int8 16x16x64), fp32/i32 acc;
//                        the codes' scales and sm_scale*log2(e) are folded into
//                        one multiplier per tile;
//   online softmax       row max across the 4 lanes that hold one query,
//                        exp2, lane-local partial row sums;
//   O^T += V^T P^T       fp16 16x16x32 MFMA; P is rounded to fp16, fp8 V codes
//                        are widened to fp16 (exactly, as value * 2^-8) when
//                        staged into LDS.
// Because S^T's accumulator layout (lane n of each 16-lane row holds query n,
// keys 4g..4g+3) is the B-operand layout of the PV product, P never leaves
// registers.  V^T arrives permuted (attn_quant_v_permute) so that the 8 keys a
// lane group needs for one PV step are one contiguous 16-byte LDS read.
#include "kcommon.h"
#include "launch.h"

namespace attnq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

constexpr int PF_THREADS = 256;
constexpr int PF_BM = 128;  // queries per workgroup (4 waves x 32)
constexpr int PF_BN = 64;   // keys per tile
constexpr float PF_LN2 = 0.69314718055994530942f;

template <int D>
struct PfLds {
  static constexpr int KROW = D + 16;            // bytes per staged K row
  static constexpr int VROW = PF_BN * 2 + 16;    // bytes per staged V^T row (fp16)
  static constexpr int KBYTES = PF_BN * KROW;
  static constexpr int VBYTES = D * VROW;
  static constexpr int STAGE = KBYTES + VBYTES;
};

template <int D, bool QK_I8, bool V_F8, bool O_BF16>
__global__ __launch_bounds__(PF_THREADS, 2) void k_prefill(const PrefillArgs a) {
  using L = PfLds<D>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int h = blockIdx.x % a.hq, b = blockIdx.x / a.hq;
  const int tile = gridDim.y - 1 - blockIdx.y;
  const int q0 = clampi(a.cu_q[b], 0, a.total_q), q1 = clampi(a.cu_q[b + 1], q0, a.total_q);
  const int k0 = clampi(a.cu_k[b], 0, a.total_k), k1 = clampi(a.cu_k[b + 1], k0, a.total_k);
  // lengths beyond the host-given maxima would address past the padded V^T
  // rows and the scale arrays: clamp (a broken precondition, not a fault)
  const int Lq = min(q1 - q0, a.max_q), Lk = min(k1 - k0, a.max_k);
  const int qs = tile * PF_BM;
  if (qs >= Lq) return;
  const int hk = h / (a.hq / a.hkv);
  const int off = Lk - Lq;  // bottom-right causal alignment
  int kend = Lk;
  if (a.causal) kend = min(Lk, qs + PF_BM + off);
  const int n_kt = kend > 0 ? (kend + PF_BN - 1) / PF_BN : 0;

  // ---- Q operand (B of S^T = K Q^T): lane (n, g) holds d in [g*D/4, (g+1)*D/4)
  constexpr int QB = D / 4;  // bytes per lane
  v8i qop[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = qs + wave * 32 + qb * 16 + n;
    qop[qb] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    if (row < Lq) {
      const uint8_t* src = static_cast<const uint8_t*>(a.q) + ((long)(q0 + row) * a.hq + h) * D + g * QB;
      uint4 x0 = *reinterpret_cast<const uint4*>(src);
      qop[qb][0] = x0.x; qop[qb][1] = x0.y; qop[qb][2] = x0.z; qop[qb][3] = x0.w;
      if constexpr (QB == 32) {
        uint4 x1 = *reinterpret_cast<const uint4*>(src + 16);
        qop[qb][4] = x1.x; qop[qb][5] = x1.y; qop[qb][6] = x1.z; qop[qb][7] = x1.w;
      }
    }
  }

  float q_sc = 1.0f;
  if constexpr (QK_I8) q_sc = a.q_scale[((long)b * a.hq + h) * a.nblk_q + tile];
  else q_sc = a.q_scale[h];
  const float k_sc_head = QK_I8 ? 0.0f : a.k_scale[hk];
  const float base_fold = a.sm_scale_log2 * q_sc;

  // ---- global -> register staging of one K tile and one V^T tile
  const uint8_t* kbase = static_cast<const uint8_t*>(a.k) + ((long)k0 * a.hkv + hk) * D;
  const long kstride = (long)a.hkv * D;
  constexpr int V_ELEM = V_F8 ? 1 : 2;
  const uint8_t* vbase = static_cast<const uint8_t*>(a.v) + ((long)b * a.hkv + hk) * D * (long)a.s_pad * V_ELEM;
  // K tile: PF_BN rows x D bytes -> D*PF_BN/16 uint4 chunks (2 per thread at D=128)
  constexpr int K_CHUNKS = PF_BN * D / 16 / PF_THREADS;
  // V tile: D rows x PF_BN elements -> D*PF_BN*V_ELEM/16 chunks
  constexpr int V_CHUNKS = D * PF_BN * V_ELEM / 16 / PF_THREADS;
  uint4 kreg[K_CHUNKS > 0 ? K_CHUNKS : 1];
  uint4 vreg[V_CHUNKS > 0 ? V_CHUNKS : 1];

  auto load_tile = [&](int kt) {
#pragma unroll
    for (int c = 0; c < K_CHUNKS; ++c) {
      const int idx = threadIdx.x + c * PF_THREADS;
      const int row = idx / (D / 16), col = (idx % (D / 16)) * 16;
      const int key = kt * PF_BN + row;
      kreg[c] = make_uint4(0, 0, 0, 0);
      if (key < Lk) kreg[c] = *reinterpret_cast<const uint4*>(kbase + key * kstride + col);
    }
#pragma unroll
    for (int c = 0; c < V_CHUNKS; ++c) {
      const int idx = threadIdx.x + c * PF_THREADS;
      constexpr int CPR = PF_BN * V_ELEM / 16;  // chunks per V^T row
      const int row = idx / CPR, col = (idx % CPR) * 16;
      vreg[c] = *reinterpret_cast<const uint4*>(vbase + ((long)row * a.s_pad + kt * PF_BN) * V_ELEM + col);
    }
  };
  auto store_tile = [&](uint8_t* st) {
    uint8_t* sk = st;
    uint8_t* sv = st + L::KBYTES;
#pragma unroll
    for (int c = 0; c < K_CHUNKS; ++c) {
      const int idx = threadIdx.x + c * PF_THREADS;
      const int row = idx / (D / 16), col = (idx % (D / 16)) * 16;
      *reinterpret_cast<uint4*>(sk + row * L::KROW + col) = kreg[c];
    }
#pragma unroll
    for (int c = 0; c < V_CHUNKS; ++c) {
      const int idx = threadIdx.x + c * PF_THREADS;
      constexpr int CPR = PF_BN * V_ELEM / 16;
      const int row = idx / CPR, colb = (idx % CPR) * 16;  // byte column in the global row
      if constexpr (V_F8) {
        // 16 fp8 codes -> 16 fp16 (value * 2^-8) -> 32 bytes
        uint32_t w[4] = {vreg[c].x, vreg[c].y, vreg[c].z, vreg[c].w};
        uint32_t o[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) e4m3x4_to_f16x4_scaled(w[e], o[2 * e], o[2 * e + 1]);
        uint8_t* dst = sv + row * L::VROW + colb * 2;
        *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<uint4*>(dst + 16) = make_uint4(o[4], o[5], o[6], o[7]);
      } else {
        *reinterpret_cast<uint4*>(sv + row * L::VROW + colb) = vreg[c];
      }
    }
  };

  // ---- accumulators
  v4f oacc[D / 16][2];
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) oacc[db][qb] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};

  if (n_kt > 0) load_tile(0);
  for (int kt = 0; kt < n_kt; ++kt) {
    uint8_t* st = smem + (kt & 1) * L::STAGE;
    store_tile(st);
    __syncthreads();
    if (kt + 1 < n_kt) load_tile(kt + 1);
    const uint8_t* sk = st;
    const uint8_t* sv = st + L::KBYTES;

    // ---- S^T = K Q^T
    float s[4][2][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const uint8_t* kp = sk + (kb * 16 + n) * L::KROW + g * QB;
      v8i kop;
      uint4 y0 = *reinterpret_cast<const uint4*>(kp);
      kop[0] = y0.x; kop[1] = y0.y; kop[2] = y0.z; kop[3] = y0.w;
      if constexpr (QB == 32) {
        uint4 y1 = *reinterpret_cast<const uint4*>(kp + 16);
        kop[4] = y1.x; kop[5] = y1.y; kop[6] = y1.z; kop[7] = y1.w;
      } else {
        kop[4] = 0; kop[5] = 0; kop[6] = 0; kop[7] = 0;
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        if constexpr (QK_I8) {
          v4i acc = v4i{0, 0, 0, 0};
          v4i a0 = v4i{kop[0], kop[1], kop[2], kop[3]};
          v4i b0 = v4i{qop[qb][0], qop[qb][1], qop[qb][2], qop[qb][3]};
          acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0, acc, 0, 0, 0);
          if constexpr (QB == 32) {
            v4i a1 = v4i{kop[4], kop[5], kop[6], kop[7]};
            v4i b1 = v4i{qop[qb][4], qop[qb][5], qop[qb][6], qop[qb][7]};
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1, acc, 0, 0, 0);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) s[kb][qb][r] = (float)acc[r];
        } else {
          v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
          acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kop, qop[qb], acc, 0, 0, 0, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) s[kb][qb][r] = acc[r];
        }
      }
    }

    // ---- scale, mask
    float fold;
    if constexpr (QK_I8)
      fold = base_fold * a.k_scale[((long)b * a.hkv + hk) * a.nblk_k + (kt * PF_BN) / 128];
    else
      fold = base_fold * k_sc_head;
    const int kfirst = kt * PF_BN;
    const int wq0 = qs + wave * 32;
    const bool need_mask = (kfirst + PF_BN > Lk) || (a.causal && kfirst + PF_BN - 1 > wq0 + off);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = s[kb][qb][r] * fold;
          if (need_mask) {
            const int key = kfirst + kb * 16 + 4 * g + r;
            const int qrow = wq0 + qb * 16 + n;
            const bool vis = key < Lk && (!a.causal || key <= qrow + off);
            v = vis ? v : -INFINITY;
          }
          s[kb][qb][r] = v;
        }

    // ---- online softmax
    v8h pk[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[kb][qb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run[qb], mx);
      const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_use);
      m_run[qb] = m_new;
      float rs = 0.f;
      float p[4][4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[kb][r] = __builtin_amdgcn_exp2f(s[kb][qb][r] - m_use);
          rs += p[kb][r];
        }
      l_run[qb] = l_run[qb] * alpha + rs;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) oacc[db][qb] *= alpha;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) pk[qb][ks][e] = (_Float16)p[2 * ks + e / 4][e % 4];
    }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const uint4 vv = *reinterpret_cast<const uint4*>(sv + (db * 16 + n) * L::VROW + (ks * 32 + 8 * g) * 2);
        v8h vop = __builtin_bit_cast(v8h, vv);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          oacc[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, pk[qb][ks], oacc[db][qb], 0, 0, 0);
      }
  }

  // ---- epilogue: O = O^T / l, lse = (m + log2 l) * ln 2
  const float vsc = V_F8 ? a.v_scale[hk] * 256.0f : 1.0f;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float l = l_run[qb];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int row = qs + wave * 32 + qb * 16 + n;
    if (row >= Lq) continue;
    const bool any = l > 0.0f;
    const float inv = any ? vsc / l : 0.0f;
    const long obase = ((long)(q0 + row) * a.hq + h) * D;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const int d0 = db * 16 + 4 * g;
      uint32_t w0 = f32_to_h16(oacc[db][qb][0] * inv, O_BF16) | (f32_to_h16(oacc[db][qb][1] * inv, O_BF16) << 16);
      uint32_t w1 = f32_to_h16(oacc[db][qb][2] * inv, O_BF16) | (f32_to_h16(oacc[db][qb][3] * inv, O_BF16) << 16);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.o) + obase + d0) = make_uint2(w0, w1);
    }
    if (a.lse && g == 0)
      a.lse[(long)h * a.total_q + q0 + row] = any ? (m_run[qb] + __log2f(l)) * PF_LN2 : -INFINITY;
  }
}

template <int D, bool I8, bool F8>
static bool launch_t(const PrefillArgs& a, bool o_bf16, int tiles, hipStream_t s) {
  dim3 grid((unsigned)(a.batch * a.hq), (unsigned)tiles);
  const size_t lds = 2 * PfLds<D>::STAGE;
  if (o_bf16)
    hipLaunchKernelGGL((k_prefill<D, I8, F8, true>), grid, dim3(PF_THREADS), lds, s, a);
  else
    hipLaunchKernelGGL((k_prefill<D, I8, F8, false>), grid, dim3(PF_THREADS), lds, s, a);
  return hipGetLastError() == hipSuccess;
}

bool launch_prefill(const PrefillArgs& a, int head_dim, bool qk_int8, bool v_fp8, bool o_bf16,
                    int max_seqlen_q, hipStream_t s) {
  const int tiles = (max_seqlen_q + PF_BM - 1) / PF_BM;
  if (tiles <= 0 || a.batch <= 0) return true;
  if (head_dim == 128) {
    if (qk_int8) return v_fp8 ? launch_t<128, true, true>(a, o_bf16, tiles, s) : launch_t<128, true, false>(a, o_bf16, tiles, s);
    return v_fp8 ? launch_t<128, false, true>(a, o_bf16, tiles, s) : launch_t<128, false, false>(a, o_bf16, tiles, s);
  }
  if (qk_int8) return v_fp8 ? launch_t<64, true, true>(a, o_bf16, tiles, s) : launch_t<64, true, false>(a, o_bf16, tiles, s);
  return v_fp8 ? launch_t<64, false, true>(a, o_bf16, tiles, s) : launch_t<64, false, false>(a, o_bf16, tiles, s);
}

}  // namespace attnq
