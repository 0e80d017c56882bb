// MLA-absorb sparse decode over int8 cache rows with per-token tile-128
// scales (Ascend "KvQuantSparseFlashAttention": attention_mode 2, combined
// quant-scale rows, PA_BSND paging through block_table, sparse_indices).
//
// Row format (656 bytes): 512 int8 nope codes | 64 bf16 rope | 4 fp32 scales
// (scale t covers nope channels [128t, 128t+128)).  K = [codes*scale | rope],
// V = codes*scale, logit = sm_scale * q . K.
//
// Split phase: one workgroup (4 waves, one per SIMD) per (query row, split of
// the index list, group of 64 heads).  Per 32-index step the workgroup gathers
// the 32 selected rows once,
// widens the int8 codes to fp16 (exact) into LDS twice -- token-major for the
// QK operand and channel-major (in the PV operand's token order) for the PV
// operand -- and each wave then serves 16 heads:
//   S^T = K Q^T    per 128-channel tile: fp16 16x16x32 MFMA, then the tile's
//                  scale per token in fp32; rope part: bf16 MFMA;
//   online softmax per head (exp2, lane-local partial sums);
//   O^T += codes^T (P * scale_t)^T   fp16 MFMA, one P operand per tile.
// Each split writes its normalized partial O and log2-sum-exp; the merge
// kernel combines the splits.
//
// The query's nope part is rounded to fp16 for the fp16 MFMA (exact for
// 2^-14 <= |q| <= 65504); everything else is exact up to fp32 accumulation.
#include "kcommon.h"
#include "launch.h"

namespace attnq {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int MLA_THREADS = 256;
constexpr int MLA_HB = 1;                        // 16-head blocks per wave
constexpr int MLA_WG_HEADS = 4 * 16 * MLA_HB;    // heads per workgroup
constexpr int MLA_STEP = 32;                     // indices per step
constexpr int MLA_NOPE = 512, MLA_ROPE = 64, MLA_ROW = 656;
constexpr int MLA_CPR = MLA_ROW / 16;            // 41 16-byte chunks per row
constexpr int MLA_RAW = (MLA_STEP * MLA_CPR + MLA_THREADS - 1) / MLA_THREADS;  // 6
constexpr int NAT_ROW = MLA_NOPE + 8;            // halfs per token-major row
constexpr int T_ROW = MLA_STEP + 8;              // halfs per channel-major row
constexpr int ROPE_ROW = MLA_ROPE + 8;           // bf16 per rope row
constexpr int MLA_MIN_TOKENS_PER_SPLIT = 256;
constexpr int MLA_TARGET_WG = 256;
constexpr float MLA_LN2 = 0.69314718055994530942f;

struct MlaLds {
  _Float16 nat[MLA_STEP * NAT_ROW];
  _Float16 tr[MLA_NOPE * T_ROW];
  uint16_t rope[MLA_STEP * ROPE_ROW];
  float scale[MLA_STEP * 4];
  int valid[MLA_STEP];
};

// stored position of token r (0..31) in the PV operand order: lane group g
// reads positions 8g..8g+7 = tokens 4g..4g+3 and 16+4g..16+4g+3
ATTNQ_DEV int pv_pos(int r) { return 8 * ((r & 15) >> 2) + 4 * (r >> 4) + (r & 3); }

// 4 int8 codes -> 4 fp16 values, exactly: 0x64XX is fp16 1024 + XX, and
// XX = code + 128 after flipping the sign bit.
ATTNQ_DEV void i8x4_to_f16x4(uint32_t w, uint32_t& lo, uint32_t& hi) {
  const uint32_t u = w ^ 0x80808080u;
  const uint32_t a = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
  const uint32_t b = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
  const v2h off = v2h{(_Float16)1152.0f, (_Float16)1152.0f};
  lo = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, a) - off);
  hi = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, b) - off);
}

__global__ __launch_bounds__(MLA_THREADS, 1) void k_mla_split(const MlaArgs a) {
  __shared__ __attribute__((aligned(16))) MlaLds L;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int split = blockIdx.x, row = blockIdx.y;  // row = b * s_q + s
  const int b = row / a.s_q;
  const int per = ((a.topk + a.n_split - 1) / a.n_split + MLA_STEP - 1) / MLA_STEP * MLA_STEP;
  const int e_begin = split * per;
  const int e_end = min(a.topk, e_begin + per);
  const int kv_len = a.kv_lens[b];
  const int* idx_row = a.idx + (long)row * a.topk;
  const int head0 = blockIdx.z * MLA_WG_HEADS;     // first head of this workgroup
  const bool wave_active = head0 + wave * 16 * MLA_HB < a.heads;

  // ---- query operands: nope as fp16 (B of the fp16 MFMA), rope as bf16
  v8h qn[MLA_HB][16];
  v8bf qr[MLA_HB][2];
#pragma unroll
  for (int hb = 0; hb < MLA_HB; ++hb) {
    const int head = head0 + (wave * MLA_HB + hb) * 16 + n;
    const bool have = head < a.heads;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + ((long)row * a.heads + head) * (MLA_NOPE + MLA_ROPE);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        uint4 w = have ? *reinterpret_cast<const uint4*>(qp + 128 * t + 32 * g + 8 * m) : make_uint4(0, 0, 0, 0);
        uint32_t ww[4] = {w.x, w.y, w.z, w.w};
        v8h h;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          h[2 * e] = (_Float16)bf16_to_f32(ww[e] & 0xffffu);
          h[2 * e + 1] = (_Float16)bf16_to_f32(ww[e] >> 16);
        }
        qn[hb][4 * t + m] = h;
      }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      uint4 w = have ? *reinterpret_cast<const uint4*>(qp + MLA_NOPE + 16 * g + 8 * m) : make_uint4(0, 0, 0, 0);
      qr[hb][m] = __builtin_bit_cast(v8bf, w);
    }
  }

  v4f oacc[MLA_HB][MLA_NOPE / 16];
#pragma unroll
  for (int hb = 0; hb < MLA_HB; ++hb)
#pragma unroll
    for (int db = 0; db < MLA_NOPE / 16; ++db) oacc[hb][db] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run[MLA_HB], l_run[MLA_HB];
#pragma unroll
  for (int hb = 0; hb < MLA_HB; ++hb) {
    m_run[hb] = -INFINITY;
    l_run[hb] = 0.f;
  }

  // ---- gather of one step's rows into registers
  uint4 raw[MLA_RAW];
  auto row_ptr = [&](int e, bool& valid) -> const uint8_t* {
    valid = false;
    if (e >= e_end) return nullptr;
    const int i = idx_row[e];
    if (i < 0 || i >= kv_len) return nullptr;
    const int bi = i / a.block_size;
    if (bi >= a.max_blocks) return nullptr;
    const int blk = a.block_table[(long)b * a.max_blocks + bi];
    if (blk < 0 || blk >= a.num_blocks) return nullptr;
    valid = true;
    return a.cache + ((long)blk * a.block_size + i % a.block_size) * MLA_ROW;
  };
  auto load_step = [&](int e0) {
#pragma unroll
    for (int k = 0; k < MLA_RAW; ++k) {
      const int c = threadIdx.x + k * MLA_THREADS;
      raw[k] = make_uint4(0, 0, 0, 0);
      if (c < MLA_STEP * MLA_CPR) {
        bool v;
        const uint8_t* p = row_ptr(e0 + c / MLA_CPR, v);
        if (v) raw[k] = *reinterpret_cast<const uint4*>(p + (c % MLA_CPR) * 16);
      }
    }
  };
  auto store_step = [&](int e0) {
#pragma unroll
    for (int k = 0; k < MLA_RAW; ++k) {
      const int c = threadIdx.x + k * MLA_THREADS;
      if (c >= MLA_STEP * MLA_CPR) continue;
      const int r = c / MLA_CPR, col = (c % MLA_CPR) * 16;
      const uint32_t w[4] = {raw[k].x, raw[k].y, raw[k].z, raw[k].w};
      if (col < MLA_NOPE) {
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) i8x4_to_f16x4(w[e], h[2 * e], h[2 * e + 1]);
        uint4* dn = reinterpret_cast<uint4*>(&L.nat[r * NAT_ROW + col]);
        dn[0] = make_uint4(h[0], h[1], h[2], h[3]);
        dn[1] = make_uint4(h[4], h[5], h[6], h[7]);
        const int pos = pv_pos(r);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          L.tr[(col + 2 * e) * T_ROW + pos] = __builtin_bit_cast(_Float16, (uint16_t)(h[e] & 0xffffu));
          L.tr[(col + 2 * e + 1) * T_ROW + pos] = __builtin_bit_cast(_Float16, (uint16_t)(h[e] >> 16));
        }
      } else if (col < MLA_NOPE + 2 * MLA_ROPE) {
        *reinterpret_cast<uint4*>(&L.rope[r * ROPE_ROW + (col - MLA_NOPE) / 2]) = raw[k];
      } else {
        *reinterpret_cast<uint4*>(&L.scale[r * 4]) = raw[k];
        bool v;
        row_ptr(e0 + r, v);
        L.valid[r] = v ? 1 : 0;
      }
    }
  };

  const int nsteps = e_end > e_begin ? (e_end - e_begin + MLA_STEP - 1) / MLA_STEP : 0;
  if (nsteps > 0) load_step(e_begin);
  for (int st = 0; st < nsteps; ++st) {
    const int e0 = e_begin + st * MLA_STEP;
    if (st > 0) __syncthreads();  // previous step's LDS reads are done
    store_step(e0);
    __syncthreads();
    if (st + 1 < nsteps) load_step(e0 + MLA_STEP);
    if (!wave_active) continue;

    // ---- S^T for the two 16-token blocks, lane (n, g): tokens 16j + 4g + r, head n
    float sv[MLA_HB][2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float sacc[MLA_HB][4];
      v4f racc[MLA_HB];
#pragma unroll
      for (int hb = 0; hb < MLA_HB; ++hb) {
        racc[hb] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 4; ++r) sacc[hb][r] = 0.f;
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        v4f acc[MLA_HB];
#pragma unroll
        for (int hb = 0; hb < MLA_HB; ++hb) acc[hb] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const v8h kop = *reinterpret_cast<const v8h*>(&L.nat[(16 * j + n) * NAT_ROW + 128 * t + 32 * g + 8 * m]);
#pragma unroll
          for (int hb = 0; hb < MLA_HB; ++hb)
            acc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qn[hb][4 * t + m], acc[hb], 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float sc = L.scale[(16 * j + 4 * g + r) * 4 + t];
#pragma unroll
          for (int hb = 0; hb < MLA_HB; ++hb) sacc[hb][r] += sc * acc[hb][r];
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const v8bf kop = *reinterpret_cast<const v8bf*>(&L.rope[(16 * j + n) * ROPE_ROW + 16 * g + 8 * m]);
#pragma unroll
        for (int hb = 0; hb < MLA_HB; ++hb)
          racc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qr[hb][m], racc[hb], 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool valid = L.valid[16 * j + 4 * g + r] != 0;
#pragma unroll
        for (int hb = 0; hb < MLA_HB; ++hb)
          sv[hb][j][r] = valid ? (sacc[hb][r] + racc[hb][r]) * a.sm_scale_log2 : -INFINITY;
      }
    }
    // ---- online softmax per head
    float p[MLA_HB][8];
    float alpha[MLA_HB];
#pragma unroll
    for (int hb = 0; hb < MLA_HB; ++hb) {
      float mx = -INFINITY;
#pragma unroll
      for (int sl = 0; sl < 8; ++sl) mx = fmaxf(mx, sv[hb][sl / 4][sl % 4]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run[hb], mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      alpha[hb] = __builtin_amdgcn_exp2f(m_run[hb] - m_use);
      m_run[hb] = m_new;
      float rs = 0.f;
#pragma unroll
      for (int sl = 0; sl < 8; ++sl) {
        p[hb][sl] = __builtin_amdgcn_exp2f(sv[hb][sl / 4][sl % 4] - m_use);
        rs += p[hb][sl];
      }
      l_run[hb] = l_run[hb] * alpha[hb] + rs;
    }
    // ---- O^T += codes^T (P * scale_t)^T, one P operand per 128-channel tile
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      v8h pk[MLA_HB];
#pragma unroll
      for (int sl = 0; sl < 8; ++sl) {
        const float sc = L.scale[((sl / 4) * 16 + 4 * g + (sl % 4)) * 4 + t];
#pragma unroll
        for (int hb = 0; hb < MLA_HB; ++hb) pk[hb][sl] = (_Float16)(p[hb][sl] * sc);
      }
#pragma unroll
      for (int dbt = 0; dbt < 8; ++dbt) {
        const int db = 8 * t + dbt;
        const v8h vop = *reinterpret_cast<const v8h*>(&L.tr[(16 * db + n) * T_ROW + 8 * g]);
#pragma unroll
        for (int hb = 0; hb < MLA_HB; ++hb) {
          oacc[hb][db] *= alpha[hb];
          oacc[hb][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, pk[hb], oacc[hb][db], 0, 0, 0);
        }
        // keep operand loads next to their MFMAs (bounded live ranges)
        if (dbt & 1) __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  if (!wave_active) return;
  // ---- partial result of this split
#pragma unroll
  for (int hb = 0; hb < MLA_HB; ++hb) {
    const int head = head0 + (wave * MLA_HB + hb) * 16 + n;
    float l = l_run[hb];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (head < a.heads) {
      const long prow = ((long)row * a.n_split + split) * a.heads + head;
      const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
      for (int db = 0; db < MLA_NOPE / 16; ++db) {
        float4 o4 = make_float4(oacc[hb][db][0] * inv, oacc[hb][db][1] * inv, oacc[hb][db][2] * inv,
                                oacc[hb][db][3] * inv);
        *reinterpret_cast<float4*>(a.ws_o + prow * MLA_NOPE + db * 16 + 4 * g) = o4;
      }
      if (g == 0) a.ws_lse[prow] = l > 0.f ? m_run[hb] + __log2f(l) : -INFINITY;
    }
  }
}

// Merge of the splits: one 128-thread workgroup per (query row, head).
__global__ __launch_bounds__(128) void k_mla_merge(const MlaArgs a) {
  const int rh = blockIdx.x;  // row * heads + head
  const int row = rh / a.heads, head = rh % a.heads;
  const int d0 = threadIdx.x * 4;
  float m = -INFINITY;
  for (int c = 0; c < a.n_split; ++c) m = fmaxf(m, a.ws_lse[((long)row * a.n_split + c) * a.heads + head]);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  float tot = 0.f;
  if (m != -INFINITY) {
    for (int c = 0; c < a.n_split; ++c) {
      const long prow = ((long)row * a.n_split + c) * a.heads + head;
      const float lc = a.ws_lse[prow];
      if (lc == -INFINITY) continue;
      const float w = __builtin_amdgcn_exp2f(lc - m);
      tot += w;
      const float4 o4 = *reinterpret_cast<const float4*>(a.ws_o + prow * MLA_NOPE + d0);
      acc[0] += w * o4.x; acc[1] += w * o4.y; acc[2] += w * o4.z; acc[3] += w * o4.w;
    }
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  uint32_t w0 = f32_to_bf16(acc[0] * inv) | (f32_to_bf16(acc[1] * inv) << 16);
  uint32_t w1 = f32_to_bf16(acc[2] * inv) | (f32_to_bf16(acc[3] * inv) << 16);
  *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.o) + (long)rh * MLA_NOPE + d0) = make_uint2(w0, w1);
  if (a.lse && threadIdx.x == 0) a.lse[rh] = tot > 0.f ? (m + __log2f(tot)) * MLA_LN2 : -INFINITY;
}

int mla_n_split(int topk) {
  // enough splits to fill the chip for small batches, never fewer than
  // MLA_MIN_TOKENS_PER_SPLIT indices per split
  int s = (topk + MLA_MIN_TOKENS_PER_SPLIT - 1) / MLA_MIN_TOKENS_PER_SPLIT;
  return s < 1 ? 1 : s;
}

size_t mla_workspace_bytes(int batch, int s_q, int heads, int topk) {
  const size_t rows = (size_t)batch * s_q * mla_n_split(topk) * heads;
  return rows * MLA_NOPE * sizeof(float) + rows * sizeof(float) + 256;
}

bool launch_mla(const MlaArgs& a, hipStream_t s) {
  const int rows = a.batch * a.s_q;
  if (rows <= 0) return true;
  const int hgroups = (a.heads + MLA_WG_HEADS - 1) / MLA_WG_HEADS;
  hipLaunchKernelGGL(k_mla_split, dim3(a.n_split, rows, hgroups), dim3(MLA_THREADS), 0, s, a);
  if (hipGetLastError() != hipSuccess) return false;
  hipLaunchKernelGGL(k_mla_merge, dim3(rows * a.heads), dim3(128), 0, s, a);
  return hipGetLastError() == hipSuccess;
}

}  // namespace attnq
