// Paged fp8 decode with split-KV and log-sum-exp merge (FlashInfer's batch
// decode over paged_kv_indptr / paged_kv_indices / paged_kv_last_page_len;
// aiter's paged fp8 flash_attn_with_kvcache with per-head descales).
//
// Split phase: one workgroup per (sequence, chunk of DEC_CHUNK_TOKENS cached
// tokens, group of 4 kv heads); each wave owns one kv head and runs its own
// pipeline (no workgroup barriers).  Per step of 32 tokens (two 16-token
// blocks, each inside one page since page sizes are multiples of 16):
//   K rows (NHD: 128 bytes per token and kv head) are loaded one step ahead
//   straight into the A operand of S^T = K Q^T (bf16 16x16x32 MFMA, fp8 ->
//   bf16 exact); the G q heads of the group are the MFMA columns;
//   V rows are copied one step ahead by direct loads into a per-wave LDS
//   stage (fp8, rows XOR-swizzled in 16-byte chunks) and read back with the
//   transposing 8-bit LDS read, which hands each lane the 8 tokens of one d
//   that the PV A operand needs; widened to fp16 (exact), O^T += V^T P^T.
//   Online softmax keeps a lagging reference max (rescale only when a score
//   exceeds it by more than 2^8).
// Each chunk writes its normalized partial O and its log2-sum-exp to the
// caller's workspace; the merge kernel combines the chunks of a sequence.
#include "kcommon.h"
#include "launch.h"

namespace attnq {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* dec_lds_t;

constexpr int DEC_THREADS = 256;
constexpr int DEC_CHUNK_TOKENS = 512;
constexpr int DEC_BLKS = DEC_CHUNK_TOKENS / 16;    // 16-token blocks per chunk (one table lane each)
static_assert(DEC_BLKS <= 64, "the block table lives in one VGPR");
constexpr int DEC_STEP = 32;                      // tokens per step
constexpr int DEC_VST = 2;                        // V stages per wave
constexpr float DEC_LN2 = 0.69314718055994530942f;
constexpr float DEC_REF_SLACK = 8.0f;             // log2 headroom before a rescale

// 16-byte chunk position of chunk c in V tile row t is c ^ dec_vsw<D>(t), so
// that the rows the transposed reads of one LDS pass name land in distinct
// bank groups.  An 8-byte (transposed) read is served in two passes of 32
// lanes across 64 four-byte banks (measured); the 32 lanes of a pass name 16
// rows (4g + r and 16 + 4g + r, r < 4, g in {0, 1} or {2, 3}) x 8 bytes of
// one chunk column.  D = 128 (rows 32 banks apart): the 8 rows of each row
// parity take the 8 chunk positions.  D = 64 (rows 16 banks apart): the 4
// rows of each row offset take the 4 chunk positions.
template <int D>
ATTNQ_DEV int dec_vsw(int t) {
  if constexpr (D == 128) return ((t >> 1) & 1) | (((t >> 2) & 1) << 1) | (((t >> 4) & 1) << 2);
  else return ((t >> 2) & 1) | (((t >> 4) & 1) << 1);
}

template <int N>
ATTNQ_DEV void dec_wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);  // vmcnt[3:0]; expcnt, lgkmcnt: no wait
}

template <int D>
__global__ __launch_bounds__(DEC_THREADS, 4) void k_decode_split(const DecodeArgs a) {
  constexpr int DEC_VTILE = DEC_STEP * D;           // bytes of one fp8 V stage
  constexpr int NM = D / 32;                        // QK MFMAs per 16-token block
  constexpr int KH = D / 64;                        // 64-byte halves of a K row
  constexpr int RPL = 1024 / D;                     // V rows per 1 KB direct load
  constexpr int CPR = D / 16;                       // 16-byte chunks per V row
  constexpr int NVL = DEC_STEP * D / 1024;          // V direct loads per step
  __shared__ __attribute__((aligned(16))) uint8_t s_v[4][DEC_VST][DEC_VTILE];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int chunk = blockIdx.x, b = blockIdx.y;
  const int hk = blockIdx.z * 4 + wave;
  if (hk >= a.hkv) return;
  const int p0 = a.kv_indptr[b], p1 = a.kv_indptr[b + 1];
  const int npg = p1 - p0;
  const int ps = a.page_size;
  const int kv_len = npg > 0 ? (npg - 1) * ps + clampi(a.kv_last[b], 0, ps) : 0;
  const int t_begin = chunk * DEC_CHUNK_TOKENS;
  if (t_begin >= kv_len) return;
  const int t_end = min(kv_len, t_begin + DEC_CHUNK_TOKENS);
  const int nblk = (t_end - t_begin + 15) / 16;        // 16-token blocks (<= DEC_BLKS)
  const int vb_last = t_end - (t_begin + 16 * (nblk - 1));  // valid tokens of the last block
  const int nsteps = (nblk + 1) / 2;
  const int G = a.hq / a.hkv;
  const long row_bytes = (long)a.hkv * D;              // bytes between consecutive slots of a page

  // byte offset of 16-token block i of the chunk (lane i; blocks past the
  // end repeat the last valid block so every address stays inside the cache)
  long boff;
  {
    const int i = min(lane, nblk - 1);
    const int tb = t_begin + 16 * i;
    const int page = clampi(a.kv_indices[p0 + tb / ps], 0, a.num_pages - 1);
    boff = ((long)page * ps + tb % ps) * row_bytes + (long)hk * D;
  }
  const uint32_t boff_lo = (uint32_t)boff, boff_hi = (uint32_t)(boff >> 32);
  auto blk_off = [&](int i) -> long {  // wave-uniform
    const uint32_t lo = __builtin_amdgcn_readlane(boff_lo, i), hi = __builtin_amdgcn_readlane(boff_hi, i);
    return (long)(((uint64_t)hi << 32) | lo);
  };
  auto blk_valid = [&](int i) { return i < nblk - 1 ? 16 : vb_last; };  // for i >= nblk - 1: the last block

  // Q^T operand: lane (n, g) holds q head hk*G + n, d in [64(m/2) + 16g + 8(m%2), +8)
  // for MFMA m (the K operand below uses the same d order)
  v8bf qop[NM];
  {
    const bool have = n < G;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + ((long)b * a.hq + hk * G + n) * D + 16 * g;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const u32x4 w = have ? *reinterpret_cast<const u32x4*>(qp + 64 * (m >> 1) + 8 * (m & 1)) : u32x4{0u, 0u, 0u, 0u};
      qop[m] = __builtin_bit_cast(v8bf, w);
    }
  }
  const float kfold = a.sm_scale_log2 * a.k_scale[hk];
  const float vsc = a.v_scale[hk];

  // K of one step: [block][half], bytes [16g, 16g+16) (and, for D = 128,
  // [64+16g, 64+16g+16)) of token n (clamped into the block): each load
  // reads 64 contiguous bytes per row
  struct KRegs { u32x4 k[2][KH]; };
  const uint32_t k_lane = (uint32_t)(n * row_bytes + 16 * g);
  auto load_k = [&](int st, KRegs& r) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int i = min(2 * st + j, DEC_BLKS - 1);
      const uint8_t* base = a.k_cache + blk_off(i);
      const int vb = blk_valid(i);
      const uint32_t off = vb == 16 ? k_lane : (uint32_t)(min(n, vb - 1) * row_bytes + 16 * g);
#pragma unroll
      for (int h = 0; h < KH; ++h) r.k[j][h] = *reinterpret_cast<const u32x4*>(base + off + 64 * h);
    }
  };
  // V of one step -> LDS stage: direct load i fills tile rows RPL*i .. RPL*i+RPL-1
  // (token rows of the step; 16 rows per 16-token block), lane L holds 16-byte
  // chunk L%CPR ^ swizzle of row RPL*i + L/CPR
  uint8_t* vst0 = s_v[wave][0];
  constexpr int LPB = 16 / RPL;                    // direct loads per 16-token block
  uint32_t v_lane[NVL];
#pragma unroll
  for (int i = 0; i < NVL; ++i)
    v_lane[i] = (uint32_t)(((i % LPB) * RPL + lane / CPR) * row_bytes +
                           (((lane % CPR) ^ dec_vsw<D>(RPL * i + lane / CPR)) << 4));
  auto load_v = [&](int st, int stage) {
#pragma unroll
    for (int i = 0; i < NVL; ++i) {
      const int bi = min(2 * st + i / LPB, DEC_BLKS - 1);
      const int vb = blk_valid(bi);
      uint32_t off = v_lane[i];
      if (vb < 16)  // rows past the end re-read the block's last valid token
        off = (uint32_t)(min((i % LPB) * RPL + lane / CPR, vb - 1) * row_bytes +
                         (((lane % CPR) ^ dec_vsw<D>(RPL * i + lane / CPR)) << 4));
      // descriptor over the 16 slots of this block (wave-uniform 64-bit base)
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(a.v_cache + blk_off(bi)), (short)0, (int)(16 * row_bytes), 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (dec_lds_t)(vst0 + stage * DEC_VTILE + i * 1024), 16, off, 0, 0, 0);
    }
  };

  // transposed-read row of this lane: k-slot 8g + e of the PV operand is token
  // 16*(e/4) + 4g + e%4 (the S^T accumulator order); lane k of a 16-lane group
  // supplies token slot e = k/2, bytes 8*(k%2) of the d chunk
  const int tr_row = 16 * ((n >> 1) >> 2) + 4 * g + ((n >> 1) & 3);
  const int tr_sw = dec_vsw<D>(tr_row);
  // LDS byte address (stage 0) of this lane's transposed read of d block db
  uint32_t tra[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
    tra[db] = (uint32_t)(uintptr_t)(dec_lds_t)(vst0 + tr_row * D + 8 * (n & 1) + ((db ^ tr_sw) << 4));

  v4f oacc[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) oacc[db] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY, l_run = 0.f;
  const v2h ones = v2h{(_Float16)1.0f, (_Float16)1.0f};

  // one step on K registers kc while step st+1 is fetched into kn.  In the
  // loop the fetch is unconditional (the last step of an even count re-reads
  // its own, cached, rows into registers the code after the loop may read),
  // so every loop step issues the same 2*KH + NVL loads and the wait below is
  // exact.  The step after the loop (LAST, odd counts) fetches nothing and
  // waits for every load: a K prefetch there would be dead, the compiler drops
  // dead loads, and a count that assumed them would let the previous step's
  // V loads into the stage it reads still be in flight.
  auto step = [&](auto stage_c, auto last_c, int st, const KRegs& kc, KRegs& kn) {
    constexpr int STAGE = decltype(stage_c)::value;  // == st % 2
    constexpr bool LAST = decltype(last_c)::value;
    const bool more = st + 1 < nsteps;
    if constexpr (!LAST) {
      const int nx = more ? st + 1 : st;
      load_k(nx, kn);
      load_v(nx, STAGE ^ 1);
    }
    // ---- S^T = K Q^T for the two 16-token blocks
    float s[2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const uint32_t w0 = kc.k[j][m >> 1][2 * (m & 1)], w1 = kc.k[j][m >> 1][2 * (m & 1) + 1];
        const v2bf c0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
        const v2bf c1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
        const v2bf c2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
        const v2bf c3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
        const v8bf kop = v8bf{c0[0], c0[1], c1[0], c1[1], c2[0], c2[1], c3[0], c3[1]};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[m], acc, 0, 0, 0);
      }
      // lane (n, g) holds S^T[token 16j + 4g + r of the step][q head n]
#pragma unroll
      for (int r = 0; r < 4; ++r) s[j][r] = acc[r] * kfold;
    }
    if (!more) {  // the last step may run past the chunk's end
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (t_begin + st * DEC_STEP + 16 * j + 4 * g + r >= t_end) s[j][r] = -INFINITY;
    }
    // ---- online softmax against a lagging reference max
    float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (__ballot(mx > m_ref + DEC_REF_SLACK)) {
      const float m_new = fmaxf(m_ref, mx);
      const float alpha = m_ref == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) oacc[db] *= alpha;
    }
    const float m_use = m_ref == -INFINITY ? 0.0f : m_ref;
    v8h pk;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        const v2h ph = __builtin_convertvector(
            (v4f{__builtin_amdgcn_exp2f(s[j][r] - m_use), __builtin_amdgcn_exp2f(s[j][r + 1] - m_use), 0.f, 0.f}).xy, v2h);
        pk[4 * j + r] = ph[0];
        pk[4 * j + r + 1] = ph[1];
        l_run = __builtin_amdgcn_fdot2(ph, ones, l_run, false);
      }
    // ---- O^T += V^T P^T; the step's V stage has landed (only step st+1's
    // KH*2 K loads and NVL V loads may still be in flight)
    if constexpr (LAST) dec_wait_vm<0>();
    else dec_wait_vm<2 * KH + NVL>();
    // the transposed reads as one block (the compiler would otherwise drain
    // every in-flight direct load before each of them)
    v2i raw[D / 16];
    if constexpr (D == 128) {
      asm volatile(
          "ds_read_b64_tr_b8 %0, %8 offset:%16\n\t"
          "ds_read_b64_tr_b8 %1, %9 offset:%16\n\t"
          "ds_read_b64_tr_b8 %2, %10 offset:%16\n\t"
          "ds_read_b64_tr_b8 %3, %11 offset:%16\n\t"
          "ds_read_b64_tr_b8 %4, %12 offset:%16\n\t"
          "ds_read_b64_tr_b8 %5, %13 offset:%16\n\t"
          "ds_read_b64_tr_b8 %6, %14 offset:%16\n\t"
          "ds_read_b64_tr_b8 %7, %15 offset:%16\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(raw[0]), "=&v"(raw[1]), "=&v"(raw[2]), "=&v"(raw[3]), "=&v"(raw[4]), "=&v"(raw[5]),
            "=&v"(raw[6]), "=&v"(raw[7])
          : "v"(tra[0]), "v"(tra[1]), "v"(tra[2]), "v"(tra[3]), "v"(tra[4]), "v"(tra[5]), "v"(tra[6]),
            "v"(tra[7]), "i"(STAGE * DEC_VTILE)
          : "memory");
    } else {
      asm volatile(
          "ds_read_b64_tr_b8 %0, %4 offset:%8\n\t"
          "ds_read_b64_tr_b8 %1, %5 offset:%8\n\t"
          "ds_read_b64_tr_b8 %2, %6 offset:%8\n\t"
          "ds_read_b64_tr_b8 %3, %7 offset:%8\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(raw[0]), "=&v"(raw[1]), "=&v"(raw[2]), "=&v"(raw[3])
          : "v"(tra[0]), "v"(tra[1]), "v"(tra[2]), "v"(tra[3]), "i"(STAGE * DEC_VTILE)
          : "memory");
    }
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const v2h h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((uint32_t)raw[db][0], 1.0f, false);
      const v2h h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((uint32_t)raw[db][0], 1.0f, true);
      const v2h h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((uint32_t)raw[db][1], 1.0f, false);
      const v2h h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((uint32_t)raw[db][1], 1.0f, true);
      const v8h vop = v8h{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
      oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, pk, oacc[db], 0, 0, 0);
    }
  };

  KRegs ka, kb;
  load_k(0, ka);
  load_v(0, 0);
  // two register sets, no copies; the loop body always runs both halves (a
  // conditional second half would let the compiler assume a prefetch into kb
  // still in flight at the top of the loop and wait for it there)
  int st = 0;
  for (; st + 1 < nsteps; st += 2) {
    step(std::integral_constant<int, 0>{}, std::false_type{}, st, ka, kb);
    step(std::integral_constant<int, 1>{}, std::false_type{}, st + 1, kb, ka);
  }
  if (st < nsteps) step(std::integral_constant<int, 0>{}, std::true_type{}, st, ka, kb);
  dec_wait_vm<0>();  // no direct load may outlive the workgroup's LDS
  // ---- partial results: O_c = O / l (times the V descale, fp8 -> fp16 was exact),
  //      lse_c = m + log2(l) in log2 units
  float l = l_run;
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (n < G) {
    const int qh = hk * G + n;
    const long row = ((long)b * a.hq + qh) * a.n_chunks + chunk;
    const float inv = l != 0.f ? vsc / l : 0.f;  // a NaN sum stays NaN
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
      *reinterpret_cast<v4f*>(a.ws_o + row * D + db * 16 + 4 * g) = oacc[db] * inv;
    if (g == 0) a.ws_lse[row] = l != 0.f ? m_ref + __log2f(l) : -INFINITY;
  }
}

// Merge: O = sum_c 2^(lse_c - lse) O_c, lse = log2 sum_c 2^lse_c.  One wave
// per (sequence, q head): lane c holds chunk c's lse (64 chunks per pass), the
// weights come from a wave max / sum, and each lane accumulates D/64 d values
// over the chunks with eight independent loads in flight.
constexpr int MERGE_THREADS = 256;

ATTNQ_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <int D>
__global__ __launch_bounds__(MERGE_THREADS) void k_decode_merge(const DecodeArgs a) {
  constexpr int VPL = D / 64;  // d values per lane
  typedef float vpl_t __attribute__((ext_vector_type(VPL)));
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * (MERGE_THREADS / 64) + (threadIdx.x >> 6);  // b * hq + qh
  if (row >= a.batch * a.hq) return;
  const int b = row / a.hq;
  const int p0 = a.kv_indptr[b], p1 = a.kv_indptr[b + 1];
  const int npg = p1 - p0;
  const int kv_len = npg > 0 ? (npg - 1) * a.page_size + clampi(a.kv_last[b], 0, a.page_size) : 0;
  const int nc = min(a.n_chunks, (kv_len + DEC_CHUNK_TOKENS - 1) / DEC_CHUNK_TOKENS);
  const long row0 = (long)row * a.n_chunks;
  // a NaN partial (a NaN value among the used tokens) makes the row NaN
  float m = -INFINITY;
  bool nan = false;
  for (int c0 = 0; c0 < nc; c0 += 64) {
    const float lc = c0 + lane < nc ? a.ws_lse[row0 + c0 + lane] : -INFINITY;
    nan |= __ballot(lc != lc) != 0;
    m = fmaxf(m, wave_max(lc));
  }
  float tot = 0.f;
  vpl_t acc = {};
  if (m != -INFINITY && !nan) {
    for (int c0 = 0; c0 < nc; c0 += 64) {
      const float lc = c0 + lane < nc ? a.ws_lse[row0 + c0 + lane] : -INFINITY;
      const float w = lc == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(lc - m);
      tot += wave_sum(w);
      const int cn = min(64, nc - c0);
      const float* op = a.ws_o + (row0 + c0) * D + VPL * lane;
      int c = 0;
      for (; c + 8 <= cn; c += 8) {
        vpl_t o8[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) o8[u] = *reinterpret_cast<const vpl_t*>(op + (long)(c + u) * D);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), c + u)) * o8[u];
      }
      for (; c < cn; ++c)
        acc += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), c)) *
               *reinterpret_cast<const vpl_t*>(op + (long)c * D);
    }
  }
  const float inv = nan ? __builtin_nanf("") : tot > 0.f ? 1.f / tot : 0.f;
  uint16_t* op = static_cast<uint16_t*>(a.o) + (long)row * D + VPL * lane;
  if constexpr (VPL == 2) {
    const v2bf ob = __builtin_convertvector(acc * inv, v2bf);
    *reinterpret_cast<uint32_t*>(op) = __builtin_bit_cast(uint32_t, ob);
  } else {
    const v2bf ob = __builtin_convertvector(v2f{acc[0] * inv, 0.f}, v2bf);
    *op = __builtin_bit_cast(uint16_t, ob[0]);
  }
  if (a.lse && lane == 0)
    a.lse[row] = nan ? __builtin_nanf("") : tot > 0.f ? (m + __log2f(tot)) * DEC_LN2 : -INFINITY;
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

template <int D>
static bool launch_decode_d(const DecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_decode_split<D>, dim3(a.n_chunks, a.batch, (a.hkv + 3) / 4), dim3(DEC_THREADS), 0, s, a);
  if (hipGetLastError() != hipSuccess) return false;
  const int rows = a.batch * a.hq;
  hipLaunchKernelGGL(k_decode_merge<D>, dim3((rows + MERGE_THREADS / 64 - 1) / (MERGE_THREADS / 64)),
                     dim3(MERGE_THREADS), 0, s, a);
  return hipGetLastError() == hipSuccess;
}

bool launch_decode(const DecodeArgs& a, int head_dim, hipStream_t s) {
  if (a.batch <= 0) return true;
  return head_dim == 128 ? launch_decode_d<128>(a, s) : launch_decode_d<64>(a, s);
}

int decode_n_chunks(int max_kv_len) { return n_chunks_for(max_kv_len); }

}  // namespace attnq
