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
// once, into LDS (the block-table row itself is read into LDS beside the
// index loads when it holds at most 2048 entries).  Per 32-index step the
// workgroup gathers the 32 selected rows and widens the codes to bf16
// (exact for int8 and e4m3fn) into token-major LDS rows.  Four waves serve
// 16 heads, split by channel tile: each owns one 128-channel tile of QK and
// PV (the last one also the rope part):
//   S^T = K Q^T    per 128-channel tile: bf16 16x16x32 MFMA on the exact
//                  codes and the bf16 query, then the tile's scale per token
//                  in fp32; rope part: bf16 MFMA; the partial scores go to
//                  LDS;
//   softmax: wave t of a head block sums the four partials of heads
//                  4t..4t+3 (each score and each P is computed once), against
//                  a lagging reference max per head (exact rescale only when
//                  a lane's two p leave [0, 2^14]), and publishes P and the
//                  step's rescale factor of O per head;
//   O^T += codes^T (P * scale_t)^T   bf16 MFMA, one P operand per tile; the
//                  PV operand (channel-major) is read from the token-major
//                  rows with transposing LDS reads.
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
constexpr int ROPE_ROW = MLA_ROPE + 16;          // bf16 per rope row: 160 B
constexpr int MLA_SPLIT_TOKENS = 512;            // indices per split (16 steps)
constexpr int MLA_BT_LDS = 2048;                 // block-table rows up to this long are read into LDS
static_assert(MLA_THREADS >= MLA_SPLIT_TOKENS, "one slot per thread");
constexpr float MLA_LN2 = 0.69314718055994530942f;
// a step whose partial row sum stays at or below this keeps the lagging
// reference max (every p <= 2^14)
constexpr float MLA_TILE_SUM_MAX = 16384.0f;

struct MlaStage {
  uint16_t nat[MLA_STEP * NAT_ROW + 8];  // bf16 codes, row r at nat_row(r)
  uint16_t rope[MLA_STEP * ROPE_ROW + 8];  // row r at rope_row(r)
  float scale[4][MLA_STEP];          // [tile][token]
};
constexpr int MLA_NBUF = 2;  // staging buffers: step st computes, step st + 1 is staged
struct MlaLds {
  MlaStage buf[MLA_NBUF];
  float part[4][4][16 * MLA_STEP];  // partial scores [head block][channel tile][xsw(head, token)]
  float pex[4][16 * MLA_STEP];      // P [head block][xsw(head, token)]
  float alpha[4][16];             // this step's rescale of O per head (1 unless the reference moved)
  float lsum[4][16];              // row sums of the split per head
  int row_idx[MLA_SPLIT_TOKENS];  // cache row of each selected index, -1 if unused
  float mask[MLA_SPLIT_TOKENS];   // 0 for a used slot, -inf otherwise (added to its logits)
  int bt[MLA_BT_LDS];             // the sequence's block-table row, when it fits
};

// LDS passes (measured): a 16-byte read is served in four passes of 16
// lanes -- each half-wave split by the parity of lane bits 2..4 -- across 64
// four-byte banks, an 8-byte read (plain or transposed) in two passes of 32
// lanes across 64 banks, a 16-byte write in eight passes of 8 consecutive
// lanes across 32 banks and an 8-byte write in four passes of 16 lanes
// across 32 banks.  Every access below keeps each pass on distinct banks.
//
// Staged code rows are 1056 bytes (66 16-byte groups) apart and rows 16..31
// sit 16 bytes further on: the K-operand reads (16 rows x 2 adjacent 16-byte
// groups per pass) and the transposed reads (8 rows x 32 bytes per pass)
// spread over all banks, and a staging write pass covers rows 4a..4a+3 and
// 16+4a..16+4a+3 (stage_row), which land on 8 distinct 16-byte groups.
ATTNQ_DEV int nat_row(int r) { return r * NAT_ROW + 8 * (r >> 4); }
// Rope rows: 160 bytes (10 groups: twice an odd number, so 16 rows of a read
// pass fall on 8 distinct even groups per lane parity), rows 16..31 16 bytes on.
ATTNQ_DEV int rope_row(int r) { return r * ROPE_ROW + 8 * (r >> 4); }
// Token row of staging chunk c (c % 32 -> a permutation of the step's rows).
ATTNQ_DEV int stage_row(int c) { return (((c >> 2) & 1) << 4) | (((c >> 3) & 3) << 2) | (c & 3); }
// Offset of (head h, token k) in a 16-head x 32-token exchange array: rows of
// 32 floats whose 4-token groups are XOR-swizzled by h % 8, so the 16-byte
// writes of 8 heads x one token group, the 16-byte reads of 16 heads x two
// token groups and the 8-byte reads and writes of heads x 32 tokens each hit
// distinct banks.
ATTNQ_DEV int xsw(int h, int k) { return h * MLA_STEP + ((((k >> 2) ^ (h & 7)) << 2) | (k & 3)); }

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
// significant bits): each signed byte converted to fp32 (one instruction per
// byte with a sign-extending byte select), pairs packed by taking the upper
// halves, which are the exact bf16 patterns.
ATTNQ_DEV void i8x4_to_bf16x4(uint32_t w, uint32_t& lo, uint32_t& hi) {
  const float f0 = (float)(int8_t)(w), f1 = (float)(int8_t)(w >> 8);
  const float f2 = (float)(int8_t)(w >> 16), f3 = (float)((int32_t)w >> 24);
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
  const int t = wave >> 2;  // 128-channel tile of QK and PV (t = 3 also owns rope); softmax of heads 4t..4t+3
  const int n = lane & 15, g = lane >> 4;
  const int split = blockIdx.x, row = blockIdx.y;  // row = b * s_q + s
  const int b = row / a.s_q;
  const int sbs = md.sparse_block_size;           // a power of 2
  const int ntok = a.topk * sbs;                  // token slots of the row
  const int e_begin = split * MLA_SPLIT_TOKENS;
  const int e_end = min(ntok, e_begin + MLA_SPLIT_TOKENS);
  const int head = blockIdx.z * MLA_WG_HEADS + hb * 16 + n;
  const bool wave_active = blockIdx.z * MLA_WG_HEADS + hb * 16 < a.heads;
  // softmax lanes: head sh of the block (4t + lane / 16), tokens 2 (lane % 16) + {0, 1}
  const int sh = 4 * t + (lane >> 4), sk = 2 * (lane & 15);

  // ---- query operands (bf16, as given) of this wave's nope tile and, for t = 3, rope
  v8bf qn[4];
  v8bf qr[2];
  {
    const bool have = head < a.heads;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + ((long)row * a.heads + head) * (MLA_NOPE + MLA_ROPE);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const u32x4 w = have ? *reinterpret_cast<const u32x4*>(qp + 128 * t + 8 * g + 32 * m) : u32x4{0u, 0u, 0u, 0u};
      qn[m] = __builtin_bit_cast(v8bf, w);
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const u32x4 w = (have && t == 3) ? *reinterpret_cast<const u32x4*>(qp + MLA_NOPE + 8 * g + 32 * m)
                                       : u32x4{0u, 0u, 0u, 0u};
      qr[m] = __builtin_bit_cast(v8bf, w);
    }
  }
  // ---- resolve this split's token slots to cache rows once.  Slot u is
  // token idx[u / sbs] * sbs + u % sbs; used below `lim`.  The sequence's
  // block-table row is read into LDS beside the index loads when it fits,
  // so the lookup costs no second dependent round trip to memory.
  {
    const int kv_len = a.kv_lens[b];
    const int s = row - b * a.s_q;
    const int lim = md.sparse_mode == 3 ? kv_len - a.s_q + s + 1 : kv_len;
    const int sbl = __builtin_ctz((unsigned)sbs);
    const int* idx_row = a.idx + (long)row * a.topk;
    const int* bt_row = a.block_table + (long)b * a.max_blocks;
    const bool bt_lds = a.max_blocks <= MLA_BT_LDS;
    if (bt_lds)
      for (int i = threadIdx.x; i < a.max_blocks; i += MLA_THREADS) L.bt[i] = bt_row[i];
    const int e = threadIdx.x;  // one slot per thread (MLA_THREADS >= MLA_SPLIT_TOKENS)
    const int u = e_begin + e;
    const int ent = (e < MLA_SPLIT_TOKENS && u < e_end) ? idx_row[u >> sbl] : -1;
    __syncthreads();  // block-table row in LDS
    if (e < MLA_SPLIT_TOKENS) {
      int r = -1;
      const long i = ((long)ent << sbl) + (u & (sbs - 1));
      if (ent >= 0 && i < lim && i / a.block_size < a.max_blocks) {
        const int bi = (int)(i / a.block_size);
        const int blk = bt_lds ? L.bt[bi] : bt_row[bi];
        if (blk >= 0 && blk < a.num_blocks) r = blk * a.block_size + (int)(i % a.block_size);
      }
      L.row_idx[e] = r;
      L.mask[e] = r >= 0 ? 0.0f : -INFINITY;
    }
  }
  __syncthreads();  // row_idx visible

  v4f oacc[8];  // O^T for channels [128 t, 128 t + 128), head n
#pragma unroll
  for (int db = 0; db < 8; ++db) oacc[db] = v4f{0.f, 0.f, 0.f, 0.f};
  // reference max (log2 units) of head sh; -inf until set so the first
  // step's p are inf/NaN and force the exact path
  float m_ref = -INFINITY, l_run = 0.f;

  // ---- staging: chunk c of a step = (row stage_row(c), 16-byte column c / 32).
  // The rows of step st + 1 are gathered into registers while step st computes.
  u32x4 raw[MLA_RAW];
  auto gather = [&](int st) {
    int rr[MLA_RAW];
    static_for<0, MLA_RAW>([&](auto ki) {
      constexpr int k = decltype(ki)::value;
      const int c = threadIdx.x + k * MLA_THREADS;
      rr[k] = c < MLA_STEP * MLA_CPR ? L.row_idx[st * MLA_STEP + stage_row(c)] : -1;
    });
    static_for<0, MLA_RAW>([&](auto ki) {
      constexpr int k = decltype(ki)::value;
      const int c = threadIdx.x + k * MLA_THREADS;
      raw[k] = u32x4{0u, 0u, 0u, 0u};
      if (rr[k] >= 0) raw[k] = *reinterpret_cast<const u32x4*>(a.cache + (long)rr[k] * MLA_ROW + (c / MLA_STEP) * 16);
    });
  };
  auto stage = [&](MlaStage& B) {
    static_for<0, MLA_RAW>([&](auto ki) {
      constexpr int k = decltype(ki)::value;
      const int c = threadIdx.x + k * MLA_THREADS;
      if (c < MLA_STEP * MLA_CPR) {
        const int r = stage_row(c), col = (c / MLA_STEP) * 16;
        if (col < MLA_NOPE) {
          uint32_t h[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if constexpr (KV_FP8) f8x4_to_bf16x4(raw[k][e], h[2 * e], h[2 * e + 1]);
            else i8x4_to_bf16x4(raw[k][e], h[2 * e], h[2 * e + 1]);
          }
          u32x4* dn = reinterpret_cast<u32x4*>(&B.nat[nat_row(r) + col]);
          dn[0] = u32x4{h[0], h[1], h[2], h[3]};
          dn[1] = u32x4{h[4], h[5], h[6], h[7]};
        } else if (col < MLA_NOPE + 2 * MLA_ROPE) {
          *reinterpret_cast<u32x4*>(&B.rope[rope_row(r) + (col - MLA_NOPE) / 2]) = raw[k];
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u) B.scale[u][r] = __uint_as_float(raw[k][u]);  // zero for unused rows
        }
      }
    });
  };

  // Pipeline: step st computes on buffer st % 2.
  //   QK: each wave's partial S^T (its tile's codes times the tile scales,
  //   plus rope for t = 3) to LDS -> barrier -> softmax: wave t of a head
  //   block sums the four partials of heads 4t..4t+3 and computes their P
  //   and rescale factors (so each value is computed once), to LDS; the
  //   workgroup stages step st + 1 (gathered during step st - 1) into the
  //   other buffer -- free because every wave finished the PV of step
  //   st - 1 before the first barrier -- and gathers step st + 2 ->
  //   barrier -> PV: every wave rescales its O tile and adds P V.
  const int nsteps = e_end > e_begin ? (e_end - e_begin + MLA_STEP - 1) / MLA_STEP : 0;
  if (nsteps > 0) {
    gather(0);
    stage(L.buf[0]);
    if (nsteps > 1) gather(1);
    __syncthreads();
  }
  for (int st = 0; st < nsteps; ++st) {
    MlaStage& B = L.buf[st % MLA_NBUF];
    // this lane's tokens' scales of tile t: tokens 16j + 4g + r
    v4f sc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) sc[j] = *reinterpret_cast<const v4f*>(&B.scale[t][16 * j + 4 * g]);
    if (wave_active) {
      // ---- partial S^T of this wave's tile, lane (n, g): tokens 16j + 4g + r, head n
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const v8bf kop = *reinterpret_cast<const v8bf*>(&B.nat[nat_row(16 * j + n) + 128 * t + 8 * g + 32 * m]);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qn[m], acc, 0, 0, 0);
        }
        v4f sp = sc[j] * acc;
        if (t == 3) {
          v4f racc = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            const v8bf kop = *reinterpret_cast<const v8bf*>(&B.rope[rope_row(16 * j + n) + 8 * g + 32 * m]);
            racc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qr[m], racc, 0, 0, 0);
          }
          sp += racc;
        }
        *reinterpret_cast<v4f*>(&L.part[hb][t][xsw(n, 16 * j + 4 * g)]) = sp;
      }
    }
    __syncthreads();  // partial scores exchanged; the PV of step st - 1 is done everywhere
    if (wave_active) {
      // ---- logits of head sh, tokens sk, sk + 1: the mask adds -inf to an
      // unused slot, whose staged row (codes, scales, rope) is all zeros, so
      // its score is 0 and the sum -inf for any sm_scale
      v2f x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = *reinterpret_cast<const v2f*>(&L.part[hb][u][xsw(sh, sk)]);
      const v2f tot = (x[0] + x[1]) + (x[2] + x[3]);
      const v2f mk = *reinterpret_cast<const v2f*>(&L.mask[st * MLA_STEP + sk]);
      const float s0 = __builtin_fmaf(tot[0], a.sm_scale_log2, mk[0]);
      const float s1 = __builtin_fmaf(tot[1], a.sm_scale_log2, mk[1]);
      // ---- softmax against a lagging reference max; exact path when a step
      // would leave the bound or no reference exists yet
      float p0 = __builtin_amdgcn_exp2f(s0 - m_ref), p1 = __builtin_amdgcn_exp2f(s1 - m_ref);
      float lt = p0 + p1;
      float al = 1.0f;
      if (__ballot(!(lt <= MLA_TILE_SUM_MAX))) {
        float mx = fmaxf(s0, s1);
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
        const float m_new = fmaxf(m_ref, mx);
        al = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_ref - m_new);
        m_ref = m_new;
        l_run *= al;
        const float mu = m_new == -INFINITY ? 0.0f : m_new;
        p0 = __builtin_amdgcn_exp2f(s0 - mu);
        p1 = __builtin_amdgcn_exp2f(s1 - mu);
        lt = p0 + p1;
      }
      l_run += lt;
      *reinterpret_cast<v2f*>(&L.pex[hb][xsw(sh, sk)]) = v2f{p0, p1};
      if ((lane & 15) == 0) L.alpha[hb][sh] = al;
    }
    // stage step st + 1 (gathered during step st - 1), gather step st + 2
    if (st + 1 < nsteps) stage(L.buf[(st + 1) % MLA_NBUF]);
    if (st + 2 < nsteps) gather(st + 2);
    __syncthreads();  // P and rescale factors exchanged; step st + 1 staged
    if (!wave_active) continue;

    // ---- O^T += codes^T (P * scale_t)^T for this wave's tile.  Slot sl of
    // lane group g is token (sl / 4) * 16 + 4g + sl % 4; the codes^T operand
    // comes from the token-major rows through two transposed reads.
    const float al = L.alpha[hb][n];
    if (__ballot(al != 1.0f)) {
#pragma unroll
      for (int db = 0; db < 8; ++db) oacc[db] *= al;
    }
    v8bf pk;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const v4f pw = *reinterpret_cast<const v4f*>(&L.pex[hb][xsw(n, 16 * j + 4 * g)]) * sc[j];
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        const v2bf pb = __builtin_convertvector(v2f{pw[r], pw[r + 1]}, v2bf);
        pk[4 * j + r] = pb[0];
        pk[4 * j + r + 1] = pb[1];
      }
    }
    // address lane (g, 4k + q) names token (4g + k) (+16), channels 4q..4q+3 of the d-block
    const int tr_row = 4 * g + (n >> 2), tr_col = 4 * (n & 3);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int c0 = 128 * t + 16 * db + tr_col;
      const uint2 lo = read_tr16(&B.nat[nat_row(tr_row) + c0]);
      const uint2 hi = read_tr16(&B.nat[nat_row(16 + tr_row) + c0]);
      const v8bf vop = __builtin_bit_cast(v8bf, u32x4{lo.x, lo.y, hi.x, hi.y});
      oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pk, oacc[db], 0, 0, 0);
    }
  }
  // ---- partial result of this split: normalized O and log2-sum-exp
  if (wave_active) {
    float l = l_run;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) l += __shfl_xor(l, o, 64);
    if ((lane & 15) == 0) {
      L.lsum[hb][sh] = l;
      const int hs = blockIdx.z * MLA_WG_HEADS + hb * 16 + sh;
      if (hs < a.heads) a.ws_lse[((long)row * a.n_split + split) * a.heads + hs] = l != 0.f ? m_ref + __log2f(l) : -INFINITY;
    }
  }
  __syncthreads();  // row sums visible
  if (!wave_active || head >= a.heads) return;
  const float l = L.lsum[hb][n];
  const long prow = ((long)row * a.n_split + split) * a.heads + head;
  const float inv = l != 0.f ? 1.f / l : 0.f;  // a NaN sum stays NaN
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    const v4f o4 = oacc[db] * inv;
    const uint32_t w0 = f32_to_bf16(o4[0]) | (f32_to_bf16(o4[1]) << 16);
    const uint32_t w1 = f32_to_bf16(o4[2]) | (f32_to_bf16(o4[3]) << 16);
    *reinterpret_cast<uint2*>(a.ws_o + prow * MLA_NOPE + 128 * t + db * 16 + 4 * g) = make_uint2(w0, w1);
  }
}

// Merge of the splits: one 256-thread workgroup per (query row, 8 heads),
// 32 threads per head, 16 channels per thread.  The first four splits' lse
// and partials are loaded together, then the maximum is taken over all
// splits; a split whose lse is -inf (no used token with p > 0) is skipped.
constexpr int MRG_HEADS = 8;
constexpr int MRG_CHUNK = 4;
__global__ __launch_bounds__(256) void k_mla_merge(const MlaArgs a) {
  const int hgs = (a.heads + MRG_HEADS - 1) / MRG_HEADS;
  const int row = blockIdx.x / hgs;
  const int head = (blockIdx.x - row * hgs) * MRG_HEADS + (threadIdx.x >> 5);
  if (head >= a.heads) return;
  const int d0 = (threadIdx.x & 31) * 16;
  const long base = (long)row * a.n_split * a.heads + head;  // partial row of split c: base + c * heads
  float lc[MRG_CHUNK];
  u32x4 v[MRG_CHUNK][2];
  auto load_chunk = [&](int c0) {
#pragma unroll
    for (int k = 0; k < MRG_CHUNK; ++k) {
      const int c = c0 + k;
      lc[k] = -INFINITY;
      if (c < a.n_split) {
        const long prow = base + (long)c * a.heads;
        lc[k] = a.ws_lse[prow];
        const u32x4* src = reinterpret_cast<const u32x4*>(a.ws_o + prow * MLA_NOPE + d0);
        v[k][0] = src[0];
        v[k][1] = src[1];
      }
    }
  };
  load_chunk(0);
  // a NaN partial (a NaN value among the used tokens) makes the row NaN
  float m = -INFINITY;
  bool nan = false;
#pragma unroll
  for (int k = 0; k < MRG_CHUNK; ++k) {
    nan |= lc[k] != lc[k];
    m = fmaxf(m, lc[k]);
  }
  for (int c = MRG_CHUNK; c < a.n_split; ++c) {
    const float x = a.ws_lse[base + (long)c * a.heads];
    nan |= x != x;
    m = fmaxf(m, x);
  }
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  float tot = 0.f;
  if (m != -INFINITY && !nan) {
    for (int c0 = 0; c0 < a.n_split; c0 += MRG_CHUNK) {
      if (c0 > 0) load_chunk(c0);
#pragma unroll
      for (int k = 0; k < MRG_CHUNK; ++k) {
        if (lc[k] == -INFINITY) continue;
        const float w = __builtin_amdgcn_exp2f(lc[k] - m);
        tot += w;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t x = v[k][i >> 2][i & 3];
          acc[2 * i] += w * bf16_to_f32(x & 0xffffu);
          acc[2 * i + 1] += w * bf16_to_f32(x >> 16);
        }
      }
    }
  }
  const float inv = nan ? __builtin_nanf("") : tot > 0.f ? 1.f / tot : 0.f;
  u32x4 out[2];
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i >> 2][i & 3] = f32_to_bf16(acc[2 * i] * inv) | (f32_to_bf16(acc[2 * i + 1] * inv) << 16);
  u32x4* dst = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.o) + ((long)row * a.heads + head) * MLA_NOPE + d0);
  dst[0] = out[0];
  dst[1] = out[1];
  if (a.lse && (threadIdx.x & 31) == 0)
    a.lse[(long)row * a.heads + head] = nan ? __builtin_nanf("") : tot > 0.f ? (m + __log2f(tot)) * MLA_LN2 : -INFINITY;
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
  hipLaunchKernelGGL(k_mla_merge, dim3(rows * ((a.heads + MRG_HEADS - 1) / MRG_HEADS)), dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess;
}

bool launch_mla(const MlaArgs& a, hipStream_t s) { return launch_mla_mode(a, MlaMode{0, 1, 0}, s); }

}  // namespace attnq
