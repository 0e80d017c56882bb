// MLA-absorb sparse decode over int8 or fp8 cache rows with per-token
// tile-128 scales (Ascend "KvQuantSparseFlashAttention": attention_mode 2,
// combined quant-scale rows, PA_BSND paging through block_table,
// sparse_indices, sparse_block_size, sparse_mode 0 or 3).
//
// Row format (656 bytes): 512 nope codes (int8 or e4m3fn) | 64 bf16 rope |
// 4 fp32 scales (scale t covers nope channels [128t, 128t+128)).
// K = [codes*scale | rope], V = codes*scale, logit = sm_scale * q . K.
// An index entry e >= 0 names tokens [e*sbs, e*sbs + sbs); a token is used
// if it is below kv_len and, with sparse_mode 3, at most kv_len - s_q + s.
//
// Split phase: one workgroup (16 waves) per (query row, 512-index split,
// group of 64 heads).  The split's indices are resolved through block_table
// once, into LDS.  Per 32-index step the workgroup gathers the 32 selected
// rows and widens the codes to bf16 (exact for int8 and e4m3fn) into
// token-major LDS rows.  Four waves serve 16 heads, split by channel tile:
// each owns one 128-channel tile of QK and PV (the last one also the rope
// part) and the four exchange their partial scores through LDS once per
// step; the PV operand (channel-major) is read from the token-major rows
// with transposing LDS reads:
//   S^T = K Q^T    per 128-channel tile: bf16 16x16x32 MFMA on the exact
//                  codes and the bf16 query, then the tile's scale per token
//                  in fp32; rope part: bf16 MFMA;
//   softmax per head against a lagging reference max (exact rescale only
//   when a step's row sum leaves [0, 2^14]), lane-local partial sums;
//   O^T += codes^T (P * scale_t)^T   bf16 MFMA, one P operand per tile.
// P * scale_t is rounded to bf16, whose range is fp32's: with p <= 2^14 the
// operand stays finite for every tile scale up to 2^100 in magnitude.
// Each split writes its normalized partial O (bf16) and log2-sum-exp; the
// merge kernel combines the splits.
//
// Rounding: P * scale_t to bf16 for the PV product and the split partials
// of O to bf16; everything else is exact up to fp32 accumulation.
#include "kcommon.h"
#include "launch.h"
#include "mla.h"

namespace attnq {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));

constexpr int MLA_THREADS = 1024;                // 16 waves: 4 head blocks x 4 channel tiles
constexpr int MLA_WG_HEADS = 64;                 // 4 blocks x 16 heads
constexpr int MLA_STEP = 32;                     // indices per step
constexpr int MLA_NOPE = 512, MLA_ROPE = 64, MLA_ROW = 656;
constexpr int MLA_CPR = MLA_ROW / 16;            // 41 16-byte chunks per row
constexpr int MLA_RAW = (MLA_STEP * MLA_CPR + MLA_THREADS - 1) / MLA_THREADS;  // 2
constexpr int NAT_ROW = MLA_NOPE + 16;           // bf16 per token row: 1056 B, 8 banks apart
constexpr int ROPE_ROW = MLA_ROPE + 8;           // bf16 per rope row
constexpr int MLA_SPLIT_TOKENS = 512;            // indices per split (16 steps)
constexpr float MLA_LN2 = 0.69314718055994530942f;
// a step whose partial row sum stays at or below this keeps the lagging
// reference max (every p <= 2^14)
constexpr float MLA_TILE_SUM_MAX = 16384.0f;

struct MlaStage {
  uint16_t nat[MLA_STEP * NAT_ROW];  // bf16 codes
  uint16_t rope[MLA_STEP * ROPE_ROW];
  float scale[MLA_STEP * 4];
};
constexpr int MLA_NBUF = 2;  // staging buffers: step st computes, step st + 1 is staged
struct MlaLds {
  MlaStage buf[MLA_NBUF];
  v4f xs[4][2][4][64];            // partial scores [head block][16-token block][channel tile][lane]
  int row_idx[MLA_SPLIT_TOKENS];  // cache row of each selected index, -1 if unused
  float mask[MLA_SPLIT_TOKENS];   // 0 for a used slot, -inf otherwise (added to its logits)
};

typedef __fp16 lds_h4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef __attribute__((address_space(3))) lds_h4* lds_h4_ptr;

// Transposed LDS read (ds_read_b64_tr_b16): inside each 16-lane group, lane
// 4k + q names 4 consecutive 16-bit values of row k; lane n receives value n
// of the 4 rows (column n of the 4 x 16 block).
ATTNQ_DEV uint2 read_tr16(const uint16_t* p) {
  const lds_h4 v = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_h4_ptr)(p));
  return __builtin_bit_cast(uint2, v);
}

// 4 int8 codes -> 4 bf16 values, exactly (|code| <= 128 has at most 8
// significant bits): each byte converted to fp32, pairs rounded to bf16.
ATTNQ_DEV void i8x4_to_bf16x4(uint32_t w, uint32_t& lo, uint32_t& hi) {
  // code + 128 as unsigned bytes, each converted exactly to fp32, minus 128;
  // the upper halves of the fp32 values are the exact bf16 patterns
  const uint32_t u = w ^ 0x80808080u;
  const float f0 = (float)(u & 0xffu) - 128.0f, f1 = (float)((u >> 8) & 0xffu) - 128.0f;
  const float f2 = (float)((u >> 16) & 0xffu) - 128.0f, f3 = (float)(u >> 24) - 128.0f;
  lo = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
  hi = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
}

// 4 e4m3fn codes -> 4 bf16 values (every e4m3fn value is exact in bf16).
ATTNQ_DEV void f8x4_to_bf16x4(uint32_t w, uint32_t& lo, uint32_t& hi) {
  lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
}

template <bool KV_FP8>
__global__ __launch_bounds__(MLA_THREADS, 1) void k_mla_split(const MlaArgs a, const MlaMode md) {
  __shared__ __attribute__((aligned(16))) MlaLds L;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hb = wave & 3;  // 16-head block
  const int t = wave >> 2;  // 128-channel tile of QK and PV (t = 3 also owns rope)
  const int n = lane & 15, g = lane >> 4;
  const int split = blockIdx.x, row = blockIdx.y;  // row = b * s_q + s
  const int b = row / a.s_q;
  const int sbs = md.sparse_block_size;           // a power of 2
  const int ntok = a.topk * sbs;                  // token slots of the row
  const int e_begin = split * MLA_SPLIT_TOKENS;
  const int e_end = min(ntok, e_begin + MLA_SPLIT_TOKENS);
  const int head = blockIdx.z * MLA_WG_HEADS + hb * 16 + n;
  const bool wave_active = blockIdx.z * MLA_WG_HEADS + hb * 16 < a.heads;

  // ---- resolve this split's token slots to cache rows once.  Slot u is
  // token idx[u / sbs] * sbs + u % sbs; used below `lim`.
  {
    const int kv_len = a.kv_lens[b];
    const int s = row - b * a.s_q;
    const int lim = md.sparse_mode == 3 ? kv_len - a.s_q + s + 1 : kv_len;
    const int sh = __builtin_ctz((unsigned)sbs);
    const int* idx_row = a.idx + (long)row * a.topk;
    for (int e = threadIdx.x; e < MLA_SPLIT_TOKENS; e += MLA_THREADS) {
      int r = -1;
      const int u = e_begin + e;
      if (u < e_end) {
        const int ent = idx_row[u >> sh];
        const long i = ((long)ent << sh) + (u & (sbs - 1));
        if (ent >= 0 && i < lim && i / a.block_size < a.max_blocks) {
          const int blk = a.block_table[(long)b * a.max_blocks + (int)(i / a.block_size)];
          if (blk >= 0 && blk < a.num_blocks) r = blk * a.block_size + (int)(i % a.block_size);
        }
      }
      L.row_idx[e] = r;
      L.mask[e] = r >= 0 ? 0.0f : -INFINITY;
    }
  }

  // ---- query operands (bf16, as given) of this wave's nope tile and, for t = 3, rope
  v8bf qn[4];
  v8bf qr[2];
  {
    const bool have = head < a.heads;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + ((long)row * a.heads + head) * (MLA_NOPE + MLA_ROPE);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const u32x4 w = have ? *reinterpret_cast<const u32x4*>(qp + 128 * t + 32 * g + 8 * m) : u32x4{0u, 0u, 0u, 0u};
      qn[m] = __builtin_bit_cast(v8bf, w);
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const u32x4 w = (have && t == 3) ? *reinterpret_cast<const u32x4*>(qp + MLA_NOPE + 16 * g + 8 * m)
                                       : u32x4{0u, 0u, 0u, 0u};
      qr[m] = __builtin_bit_cast(v8bf, w);
    }
  }
  __syncthreads();  // row_idx visible

  v4f oacc[8];  // O^T for channels [128 t, 128 t + 128)
#pragma unroll
  for (int db = 0; db < 8; ++db) oacc[db] = v4f{0.f, 0.f, 0.f, 0.f};
  // reference max (log2 units); -inf until set so the first step's p are
  // inf/NaN and force the exact path
  float m_ref = -INFINITY, l_run = 0.f;

  // ---- staging: chunk c of a step = (row c % 32, 16-byte column c / 32).
  // The rows of step st + 1 are gathered into registers while step st computes.
  u32x4 raw[MLA_RAW];
  auto gather = [&](int st) {
    static_for<0, MLA_RAW>([&](auto ki) {
      constexpr int k = decltype(ki)::value;
      const int c = threadIdx.x + k * MLA_THREADS;
      raw[k] = u32x4{0u, 0u, 0u, 0u};
      if (c < MLA_STEP * MLA_CPR) {
        const int r = L.row_idx[st * MLA_STEP + (c % MLA_STEP)];
        if (r >= 0) raw[k] = *reinterpret_cast<const u32x4*>(a.cache + (long)r * MLA_ROW + (c / MLA_STEP) * 16);
      }
    });
  };
  auto stage = [&](MlaStage& B) {
    static_for<0, MLA_RAW>([&](auto ki) {
      constexpr int k = decltype(ki)::value;
      const int c = threadIdx.x + k * MLA_THREADS;
      if (c < MLA_STEP * MLA_CPR) {
        const int r = c % MLA_STEP, col = (c / MLA_STEP) * 16;
        if (col < MLA_NOPE) {
          uint32_t h[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if constexpr (KV_FP8) f8x4_to_bf16x4(raw[k][e], h[2 * e], h[2 * e + 1]);
            else i8x4_to_bf16x4(raw[k][e], h[2 * e], h[2 * e + 1]);
          }
          u32x4* dn = reinterpret_cast<u32x4*>(&B.nat[r * NAT_ROW + col]);
          dn[0] = u32x4{h[0], h[1], h[2], h[3]};
          dn[1] = u32x4{h[4], h[5], h[6], h[7]};
        } else if (col < MLA_NOPE + 2 * MLA_ROPE) {
          *reinterpret_cast<u32x4*>(&B.rope[r * ROPE_ROW + (col - MLA_NOPE) / 2]) = raw[k];
        } else {
          *reinterpret_cast<u32x4*>(&B.scale[r * 4]) = raw[k];  // zero for unused rows
        }
      }
    });
  };

  // Pipeline: step st computes on buffer st % 2.  Between the two barriers of
  // step st the workgroup stages step st + 1 (gathered into registers during
  // step st - 1) into the other buffer -- free because every wave finished
  // the PV of step st - 1 before the first barrier -- and gathers step st + 2.
  const int nsteps = e_end > e_begin ? (e_end - e_begin + MLA_STEP - 1) / MLA_STEP : 0;
  if (nsteps > 0) {
    gather(0);
    stage(L.buf[0]);
    if (nsteps > 1) gather(1);
    __syncthreads();
  }
  for (int st = 0; st < nsteps; ++st) {
    MlaStage& B = L.buf[st % MLA_NBUF];
    v4f (*xs)[2][4][64] = L.xs;
    // ---- partial S^T of this wave's tile, lane (n, g): tokens 16j + 4g + r, head n
    float sp[2][4];
    // this lane's tokens' scales of tile t (used by QK and by P)
    float sc[2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[j][r] = B.scale[(16 * j + 4 * g + r) * 4 + t];
    if (wave_active) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const v8bf kop = *reinterpret_cast<const v8bf*>(&B.nat[(16 * j + n) * NAT_ROW + 128 * t + 32 * g + 8 * m]);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qn[m], acc, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) sp[j][r] = sc[j][r] * acc[r];
        if (t == 3) {
          v4f racc = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            const v8bf kop = *reinterpret_cast<const v8bf*>(&B.rope[(16 * j + n) * ROPE_ROW + 16 * g + 8 * m]);
            racc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qr[m], racc, 0, 0, 0);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) sp[j][r] += racc[r];
        }
        xs[hb][j][t][lane] = v4f{sp[j][0], sp[j][1], sp[j][2], sp[j][3]};
      }
    }
    __syncthreads();  // scores exchanged; the PV of step st - 1 is done everywhere
    // stage step st + 1 (gathered during step st - 1), gather step st + 2
    if (st + 1 < nsteps) stage(L.buf[(st + 1) % MLA_NBUF]);
    if (st + 2 < nsteps) gather(st + 2);
    if (!wave_active) {
      __syncthreads();
      continue;
    }
    // logits of the lane's tokens 16j + 4g + r: the mask adds -inf to an
    // unused slot, whose staged row (codes, scales, rope) is all zeros, so
    // its score is 0 and the sum -inf for any sm_scale
    float s[2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const v4f tot = (xs[hb][j][0][lane] + xs[hb][j][1][lane]) + (xs[hb][j][2][lane] + xs[hb][j][3][lane]);
      const float* mk = &L.mask[st * MLA_STEP + 16 * j + 4 * g];
#pragma unroll
      for (int r = 0; r < 4; ++r) s[j][r] = __builtin_fmaf(tot[r], a.sm_scale_log2, mk[r]);
    }

    // ---- softmax against a lagging reference max (the four waves of a
    // head block compute identical values); exact path when a step would
    // leave fp16 range or no reference exists yet
    float p[8];
    float lt = 0.f;
#pragma unroll
    for (int sl = 0; sl < 8; sl += 2) {
      const float p0 = __builtin_amdgcn_exp2f(s[sl / 4][sl % 4] - m_ref);
      const float p1 = __builtin_amdgcn_exp2f(s[sl / 4][sl % 4 + 1] - m_ref);
      p[sl] = p0;
      p[sl + 1] = p1;
      lt += p0 + p1;
    }
    if (__ballot(!(lt <= MLA_TILE_SUM_MAX))) {
      float mx = -INFINITY;
#pragma unroll
      for (int sl = 0; sl < 8; ++sl) mx = fmaxf(mx, s[sl / 4][sl % 4]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_ref, mx);
      const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 8; ++db) oacc[db] *= alpha;
      const float mu = m_new == -INFINITY ? 0.0f : m_new;
      lt = 0.f;
#pragma unroll
      for (int sl = 0; sl < 8; sl += 2) {
        const float p0 = __builtin_amdgcn_exp2f(s[sl / 4][sl % 4] - mu);
        const float p1 = __builtin_amdgcn_exp2f(s[sl / 4][sl % 4 + 1] - mu);
        p[sl] = p0;
        p[sl + 1] = p1;
        lt += p0 + p1;
      }
    }
    l_run += lt;

    // ---- O^T += codes^T (P * scale_t)^T for this wave's tile.  Slot sl of
    // lane group g is token (sl / 4) * 16 + 4g + sl % 4; the codes^T operand
    // comes from the token-major rows through two transposed reads.
    v8bf pk;
#pragma unroll
    for (int sl = 0; sl < 8; sl += 2) {
      const v2bf pb = __builtin_convertvector(v2f{p[sl] * sc[sl / 4][sl % 4], p[sl + 1] * sc[sl / 4][sl % 4 + 1]}, v2bf);
      pk[sl] = pb[0];
      pk[sl + 1] = pb[1];
    }
    // address lane (g, 4k + q) names token (4g + k) (+16), channels 4q..4q+3 of the d-block
    const int tr_row = 4 * g + (n >> 2), tr_col = 4 * (n & 3);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int c0 = 128 * t + 16 * db + tr_col;
      const uint2 lo = read_tr16(&B.nat[tr_row * NAT_ROW + c0]);
      const uint2 hi = read_tr16(&B.nat[(16 + tr_row) * NAT_ROW + c0]);
      const v8bf vop = __builtin_bit_cast(v8bf, u32x4{lo.x, lo.y, hi.x, hi.y});
      oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pk, oacc[db], 0, 0, 0);
    }
    __syncthreads();  // step st + 1 staged; exchange buffer free again
  }
  if (!wave_active) return;
  // ---- partial result of this split: normalized O and log2-sum-exp
  float l = l_run;
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (head < a.heads) {
    const long prow = ((long)row * a.n_split + split) * a.heads + head;
    const float inv = l != 0.f ? 1.f / l : 0.f;  // a NaN sum stays NaN
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const v4f o4 = oacc[db] * inv;
      const uint32_t w0 = f32_to_bf16(o4[0]) | (f32_to_bf16(o4[1]) << 16);
      const uint32_t w1 = f32_to_bf16(o4[2]) | (f32_to_bf16(o4[3]) << 16);
      *reinterpret_cast<uint2*>(a.ws_o + prow * MLA_NOPE + 128 * t + db * 16 + 4 * g) = make_uint2(w0, w1);
    }
    if (g == 0 && t == 0) a.ws_lse[prow] = l != 0.f ? m_ref + __log2f(l) : -INFINITY;
  }
}

// Merge of the splits: one 128-thread workgroup per (query row, head).
__global__ __launch_bounds__(128) void k_mla_merge(const MlaArgs a) {
  const int rh = blockIdx.x;  // row * heads + head
  const int row = rh / a.heads, head = rh % a.heads;
  const int d0 = threadIdx.x * 4;
  // a NaN partial (a NaN value among the used tokens) makes the row NaN
  float m = -INFINITY;
  bool nan = false;
  for (int c = 0; c < a.n_split; ++c) {
    const float lc = a.ws_lse[((long)row * a.n_split + c) * a.heads + head];
    nan |= lc != lc;
    m = fmaxf(m, lc);
  }
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  float tot = 0.f;
  if (m != -INFINITY && !nan) {
    for (int c = 0; c < a.n_split; ++c) {
      const long prow = ((long)row * a.n_split + c) * a.heads + head;
      const float lc = a.ws_lse[prow];
      if (lc == -INFINITY) continue;
      const float w = __builtin_amdgcn_exp2f(lc - m);
      tot += w;
      const uint2 o2 = *reinterpret_cast<const uint2*>(a.ws_o + prow * MLA_NOPE + d0);
      acc[0] += w * bf16_to_f32(o2.x & 0xffffu); acc[1] += w * bf16_to_f32(o2.x >> 16);
      acc[2] += w * bf16_to_f32(o2.y & 0xffffu); acc[3] += w * bf16_to_f32(o2.y >> 16);
    }
  }
  const float inv = nan ? __builtin_nanf("") : tot > 0.f ? 1.f / tot : 0.f;
  uint32_t w0 = f32_to_bf16(acc[0] * inv) | (f32_to_bf16(acc[1] * inv) << 16);
  uint32_t w1 = f32_to_bf16(acc[2] * inv) | (f32_to_bf16(acc[3] * inv) << 16);
  *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.o) + (long)rh * MLA_NOPE + d0) = make_uint2(w0, w1);
  if (a.lse && threadIdx.x == 0)
    a.lse[rh] = nan ? __builtin_nanf("") : tot > 0.f ? (m + __log2f(tot)) * MLA_LN2 : -INFINITY;
}

int mla_n_split(int topk) { return (topk + MLA_SPLIT_TOKENS - 1) / MLA_SPLIT_TOKENS; }

size_t mla_workspace_bytes(int batch, int s_q, int heads, int topk) {
  const size_t rows = (size_t)batch * s_q * mla_n_split(topk) * heads;
  return rows * MLA_NOPE * sizeof(uint16_t) + rows * sizeof(float) + 256;
}

bool launch_mla_mode(const MlaArgs& a, const MlaMode& m, hipStream_t s) {
  const int rows = a.batch * a.s_q;
  if (rows <= 0) return true;
  const int hgroups = (a.heads + MLA_WG_HEADS - 1) / MLA_WG_HEADS;
  if (m.kv_fp8)
    hipLaunchKernelGGL((k_mla_split<true>), dim3(a.n_split, rows, hgroups), dim3(MLA_THREADS), 0, s, a, m);
  else
    hipLaunchKernelGGL((k_mla_split<false>), dim3(a.n_split, rows, hgroups), dim3(MLA_THREADS), 0, s, a, m);
  if (hipGetLastError() != hipSuccess) return false;
  hipLaunchKernelGGL(k_mla_merge, dim3(rows * a.heads), dim3(128), 0, s, a);
  return hipGetLastError() == hipSuccess;
}

bool launch_mla(const MlaArgs& a, hipStream_t s) { return launch_mla_mode(a, MlaMode{0, 1, 0}, s); }

}  // namespace attnq
